"""The C ABI without a GPU: the library loads, exports what include/infllm2.h declares, and
every invalid argument is rejected on the host with the right status before anything is
enqueued (these calls never reach a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_long_semantic_amd as lib
from block_sparse_long_semantic_amd import _lib

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def so():
    return lib.load_library()


def test_library_exports_every_declared_symbol(so):
    assert len(lib.EXPORTED_SYMBOLS) == 14
    for name in lib.EXPORTED_SYMBOLS:
        assert hasattr(so, name), name
    assert lib.version() == 100


def test_header_and_binding_agree():
    with open(_lib._HEADER) as f:
        text = f.read()
    assert "INFLLM2_MAX_SEQS" not in text           # no cap on the number of sequences
    # struct field order of the binding matches the header
    fields = [f[0] for f in _lib._CParams._fields_]
    pos = [text.index(f"int32_t {n};") if n != "softmax_scale" else text.index("float softmax_scale;")
           for n in fields]
    assert pos == sorted(pos)
    body = text[text.index("typedef struct {\n  int32_t num_seqs;"):]
    body = body[:body.index("} infllm2_seqs;")]
    pos = [re.search(r"[ *]" + n + ";", body).start() for n, _ in _lib._CSeqs._fields_]
    assert pos == sorted(pos)


def test_status_strings(so):
    for st in range(7):
        assert so.infllm2_status_string(st)
    assert so.infllm2_status_string(99) == b"unknown status"


def params(**kw):
    base = dict(num_q_heads=32, num_kv_heads=2, head_dim=128, block_size=64, kernel_size=32,
                kernel_stride=16, topk=96, num_init_blocks=1, num_local_blocks=2,
                softmax_scale=0.0, dtype=lib.BF16)
    base.update(kw)
    return lib.Params(**base)


def seqs(**kw):
    base = dict(q_start=[0], q_len=[100], q_pos0=[0], kv_start=[0], kv_len=[100], kc_start=[0])
    base.update(kw)
    return lib.Seqs(**base)


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced: calls fail validation
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


def call_scores(so, p, s, q=FAKE, kern=FAKE, scores=FAKE, nb=2):
    cp, cs = p.c(), s.c()
    return so.infllm2_block_scores(ctypes.byref(cp), ctypes.byref(cs), q, kern, scores, nb, None)


def call_compress(so, p, s, k=FAKE, kern=FAKE, prev=None):
    cp, cs = p.c(), s.c()
    return so.infllm2_compress_kernels(ctypes.byref(cp), ctypes.byref(cs), k, prev, kern, None)


def call_attn(so, p, s, q=FAKE, idx=FAKE, out=FAKE):
    cp, cs = p.c(), s.c()
    return so.infllm2_sparse_attn_prefill(ctypes.byref(cp), ctypes.byref(cs), q, FAKE, FAKE, idx,
                                          out, None, None)


def last(so):
    return so.infllm2_last_error().decode()


@pytest.mark.parametrize("bad,status,text", [
    (dict(num_q_heads=33), SHAPE, "multiple"),
    (dict(num_kv_heads=0), SHAPE, "positive"),
    (dict(dtype=7), UNSUP, "dtype"),
    (dict(head_dim=100), UNSUP, "head_dim"),
    (dict(num_q_heads=64, num_kv_heads=2), UNSUP, "group"),
    (dict(kernel_size=40), SHAPE, "kernel_size"),
    (dict(block_size=72), SHAPE, "block_size"),
    (dict(topk=0), SHAPE, "topk"),
    (dict(num_local_blocks=0), SHAPE, "num_local_blocks"),
    (dict(topk=2, num_init_blocks=1, num_local_blocks=2), SHAPE, "forced"),
    (dict(softmax_scale=float("inf")), SHAPE, "softmax_scale"),
])
def test_bad_params_rejected(so, bad, status, text):
    assert call_scores(so, params(**bad), seqs()) == status
    assert text in last(so)


def test_bad_sequences_rejected(so):
    """The host bounds are checked; the device arrays only for presence (their contents are
    the kernels' to read, trusted)."""
    p = params()
    assert call_scores(so, p, seqs(max_q_len=101)) == SHAPE         # a query past every key
    assert "max_q_len" in last(so)
    assert call_scores(so, p, seqs(max_kv_len=-1, max_q_len=0)) == SHAPE
    assert call_scores(so, p, seqs(q_rows=-3)) == SHAPE and "bound" in last(so)
    empty = seqs()
    cs = empty.c()
    cs.num_seqs = 0
    cp = p.c()
    assert so.infllm2_block_scores(ctypes.byref(cp), ctypes.byref(cs), FAKE, FAKE, FAKE, 2,
                                   None) == SHAPE and "num_seqs" in last(so)
    cs = empty.c()
    cs.kv_len = None
    assert so.infllm2_block_scores(ctypes.byref(cp), ctypes.byref(cs), FAKE, FAKE, FAKE, 2,
                                   None) == NULL and "metadata" in last(so)
    # no limit on the number of sequences: 1000 pass the sequence checks and fail on nb_stride
    n = 1000
    many = lib.Seqs(np.arange(n), np.ones(n), np.zeros(n), np.arange(n) * 100, np.full(n, 100),
                    np.zeros(n))
    assert call_scores(so, p, many, nb=1) == SHAPE and "nb_stride" in last(so)
    assert so.infllm2_block_scores(ctypes.byref(cp), None, FAKE, FAKE, FAKE, 2, None) == NULL


def test_null_and_alignment(so):
    p, s = params(), seqs()
    assert call_scores(so, p, s, q=None) == NULL
    assert call_scores(so, p, s, scores=MISALIGNED) == ALIGN
    assert call_compress(so, p, s, kern=None) == NULL
    assert call_attn(so, p, s, idx=MISALIGNED) == ALIGN
    assert so.infllm2_block_scores(None, None, FAKE, FAKE, FAKE, 2, None) == NULL


def test_scores_stride_checked(so):
    p = params()
    # 100 tokens -> reachable blocks 0..1
    assert call_scores(so, p, seqs(), nb=1) == SHAPE and "nb_stride" in last(so)
    cp, cs = p.c(), seqs(q_len=[1], q_pos0=[2 ** 20 * 64 - 1], kv_len=[2 ** 20 * 64]).c()
    st = so.infllm2_topk_select(ctypes.byref(cp), ctypes.byref(cs), FAKE, 2 ** 20, FAKE, None)
    assert st == UNSUP and "4096" in last(so)


def test_decode_workspace(so):
    p = params()
    d = p.head_dim
    # two int32 counter arrays over the (row, KV head) pairs, each padded to 256 bytes, then
    # per (row, query head, split) the running max, denominator and d partial outputs (float32)
    al = lambda x: (x + 255) // 256 * 256
    counters = 2 * al(8 * p.num_kv_heads * 4)
    assert lib.decode_workspace_size(p, 8, 12) == 8 * 32 * 12 * (2 + d) * 4 + counters
    # automatic splits: one block per wave of 4 (96 / 4)
    assert lib.decode_workspace_size(p, 8, 0) == 8 * 32 * 24 * (2 + d) * 4 + counters
    cp, cs = p.c(), seqs(q_len=[1], q_pos0=[99]).c()
    st = so.infllm2_sparse_attn_decode(ctypes.byref(cp), ctypes.byref(cs), FAKE, FAKE, FAKE, FAKE,
                                       4, FAKE, 16, FAKE, None, None)
    assert st == WS and "workspace" in last(so)
    st = so.infllm2_sparse_attn_decode(ctypes.byref(cp), ctypes.byref(cs), FAKE, FAKE, FAKE, FAKE,
                                       97, FAKE, 1 << 30, FAKE, None, None)
    assert st == SHAPE


def test_decode_step_checks(so):
    """The single-launch decode step (bf16, d 128, G 16) checks every argument before anything
    is enqueued; each call below breaks exactly one of them."""
    p = params()
    s = seqs(q_len=[1], q_pos0=[99])
    cp, cs = p.c(), s.c()

    def call(ws=FAKE, ws_bytes=1 << 30, nb=2, scores=FAKE, splits=0):
        return so.infllm2_decode_step(ctypes.byref(cp), ctypes.byref(cs), FAKE, FAKE, FAKE, FAKE,
                                      None, scores, nb, FAKE, splits, ws, ws_bytes, FAKE, None,
                                      None)
    assert call(ws=None) == NULL and "workspace" in last(so)
    assert call(ws_bytes=16) == WS
    assert call(nb=1) == SHAPE and "nb_stride" in last(so)
    assert call(scores=MISALIGNED) == ALIGN
    assert call(splits=97) == SHAPE


def call_bwd(so, p, s, lse=FAKE, dq=FAKE, ws=FAKE, ws_bytes=1 << 30):
    cp, cs = p.c(), s.c()
    return so.infllm2_sparse_attn_backward(ctypes.byref(cp), ctypes.byref(cs), FAKE, FAKE, FAKE,
                                           FAKE, FAKE, lse, FAKE, dq, FAKE, FAKE, ws, ws_bytes,
                                           None)


def test_backward_workspace_and_checks(so):
    p, s = params(), seqs()
    # delta (rows x Hq float32), then per (row window, KV head, block) segment a count (and the
    # dK/dV work counter after them), two offset tables with a final total each, and the row list
    # (rows x Hkv x topk int32), each 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    n_seg = 1 * 2 * 2                   # one row window (100 rows), 2 KV heads, 100 keys -> 2 blocks
    want = al(100 * 32 * 4) + 3 * al((n_seg + 1) * 4) + al(100 * 2 * 96 * 4)
    assert lib.backward_workspace_size(p, s) == want
    assert call_bwd(so, p, s, ws_bytes=want - 1) == WS and "workspace" in last(so)
    assert call_bwd(so, p, s, lse=None) == NULL
    assert call_bwd(so, p, s, dq=MISALIGNED) == ALIGN
    for bad in (dict(dtype=lib.F32), dict(head_dim=96), dict(num_q_heads=8, num_kv_heads=2)):
        assert call_bwd(so, params(**bad), s) == UNSUP and "backward" in last(so)
        assert lib.backward_workspace_size(params(**bad), s) == 0
    far = seqs(q_len=[1], q_pos0=[2048 * 64], kv_len=[2048 * 64 + 1])
    assert call_bwd(so, p, far) == UNSUP


def test_sliding_window_checks(so):
    p, s = params(), seqs()
    cp, cs = p.c(), s.c()
    call = lambda w, q=FAKE, lse=None, pp=cp: so.infllm2_sliding_window_attn(
        ctypes.byref(pp), ctypes.byref(cs), w, q, FAKE, FAKE, FAKE, lse, None)
    assert call(0) == SHAPE and "window" in last(so)
    assert call(16, q=None) == NULL
    assert call(16, lse=MISALIGNED) == ALIGN
    cf = params(dtype=lib.F32).c()
    assert call(16, pp=cf) == UNSUP and "sliding-window" in last(so)


def test_last_error_is_thread_local(so):
    import threading
    call_scores(so, params(num_q_heads=33), seqs())
    seen = []
    t = threading.Thread(target=lambda: seen.append(last(so)))
    t.start(); t.join()
    assert seen == [""] and "multiple" in last(so)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setenv("INFLLM2_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load_library()
