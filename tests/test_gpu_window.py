"""Parity of the HIP sliding-window attention (infllm2_sliding_window_attn) with the oracle's
window_attention: every row of small cases, sampled rows at 128K.  Bounds as for the
block-sparse attention (tests/_compare.py): max-abs 2e-2 on O and 1e-3 on lse (bf16)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import infllm2_oracle as orc
from tests import _compare as cmp
from tests._gpu import dev, host, log, seqs_for

import block_sparse_long_semantic_amd as lib

pytestmark = pytest.mark.gpu


def run_window(wl, window):
    p = wl.params
    seqs = seqs_for(wl, p)
    q, k, v = dev(wl.q, p.dtype), dev(wl.k, p.dtype), dev(wl.v, p.dtype)
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    lse = torch.full((q.shape[0], p.num_q_heads), float("nan"), dtype=torch.float32,
                     device="cuda")
    lib.sliding_window_attn(p, seqs, window, q, k, v, out, lse)
    torch.cuda.synchronize()
    return host(out), host(lse)


def check_window(wl, out, lse, window, b, rows=None, label=""):
    p = wl.params
    sl_q, sl_k = wl.seq_slices(b)
    n = int(wl.q_len[b])
    if n == 0:
        return
    rows = np.arange(n) if rows is None else np.asarray(rows)
    pos = int(wl.q_pos0[b]) + rows
    O, L = orc.window_attention(wl.q[sl_q][rows], pos, wl.k[sl_k], wl.v[sl_k], window, p)
    g = int(wl.q_start[b]) + rows
    err, lerr = cmp.check_attention(out[g], lse[g], O, L, p.dtype)
    log(f"{label} seq {b}: rows {len(rows)} out-err {err:.3g} lse-err {lerr:.3g}")


@pytest.mark.parametrize("Hq,d", [(32, 128), (16, 128), (32, 64), (16, 64)])
@pytest.mark.parametrize("window", [1, 64, 100, 333])
def test_window_geometries_all_rows(Hq, d, window):
    """Each supported (head_dim, group) pair, windows shorter than, equal to and longer than a
    block; 700 tokens: a ragged last tile and block."""
    p = replace(synth.config_params("prefill32k"), num_q_heads=Hq, head_dim=d)
    wl = synth.make_prefill(f"win-{Hq}-{d}", p, [700], seed=71)
    log(f"case window Hq={Hq} d={d} W={window}")
    out, lse = run_window(wl, window)
    check_window(wl, out, lse, window, 0, label=f"win {Hq}/{d} W={window}")


def test_window_edge_sequences():
    p = synth.config_params("prefill32k")
    wl = synth.make_prefill("win-edge", p, [0, 1, 20, 64, 65, 700], seed=72)
    log("case window edge lengths")
    out, lse = run_window(wl, 100)
    for b in range(wl.num_seqs):
        check_window(wl, out, lse, 100, b, label="win edge")


def test_window_longer_than_sequence_is_causal_attention():
    """A window covering every earlier token is dense causal attention (torch SDPA, float64)."""
    p = synth.config_params("prefill32k")
    wl = synth.make_prefill("win-dense", p, [1100], seed=73)
    log("case window dense")
    out, lse = run_window(wl, 5000)
    G = p.group
    q = torch.from_numpy(wl.q.astype(np.float64)).transpose(0, 1)
    k = torch.from_numpy(wl.k.astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
    v = torch.from_numpy(wl.v.astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    refn = ref.transpose(0, 1).numpy()
    d = np.abs(out - refn)
    assert np.all(d <= cmp.out_tolerance(refn, "bf16")), float(d.max())
    check_window(wl, out, lse, 5000, 0, label="win dense")


def test_window_chunk_against_cache():
    """Queries for the last 700 tokens only (q_pos0 > 0); their windows reach into the cache."""
    p = synth.config_params("prefill32k")
    full = synth.make_prefill("win-chunk", p, [2600], seed=74)
    q0 = 1900
    wl = synth.Workload("win-chunk", p, full.q[q0:], full.k, full.v, np.array([0]),
                        np.array([700], np.int32), np.array([q0], np.int32), np.array([0]),
                        np.array([2600], np.int32))
    log("case window chunk")
    out, lse = run_window(wl, 500)
    check_window(wl, out, lse, 500, 0, label="win chunk")


def test_window_full_size_sampled():
    """The 128K layer with a 6144-token window (the keys a top-96 selection of 64-token blocks
    covers): sampled rows (start, every 1777th, the last rows)."""
    wl = synth.make("prefill128k")
    log("case window full 128K W=6144")
    out, lse = run_window(wl, 6144)
    L = int(wl.q_len[0])
    rows = np.array(sorted(set(range(0, 6200, 389)) | set(range(6200, L, 1777)) |
                           set(range(L - 3, L))))
    check_window(wl, out, lse, 6144, 0, rows=rows, label="win full")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
