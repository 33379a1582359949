"""Score mode 1 (per-head softmax over the visible kernels before the group sum) on the GPU:
scores within the float32 bound of tests/_compare.py (softmax_score_rel_bound), the top-k on
the GPU's own scores equal to the oracle's selection on them, indices equal to the oracle's up
to the 1e-3 tie band, and attention on the GPU's indices, as for score mode 0."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import infllm2_oracle as orc
from tests import _compare as cmp
from tests._gpu import dev, host, kc_starts, log, run_prefill_stages, seqs_for

import block_sparse_long_semantic_amd as lib

pytestmark = pytest.mark.gpu


def check_mode1(wl, res, b, rows=None, label=""):
    p = wl.params
    sl_q, sl_k = wl.seq_slices(b)
    q_seq, k_seq, v_seq = wl.q[sl_q], wl.k[sl_k], wl.v[sl_k]
    if q_seq.shape[0] == 0:
        return
    kc0, _ = kc_starts(wl.kv_len, p)
    C = orc.num_kernels(k_seq.shape[0], p.kernel_size, p.kernel_stride)
    kern = orc.compress_kernels(k_seq, p.kernel_size, p.kernel_stride, p.dtype)
    assert np.array_equal(res["kernels"][kc0[b]:kc0[b] + C], kern), f"{label}: kernels differ"
    rows = np.arange(q_seq.shape[0]) if rows is None else np.asarray(rows)
    ref = orc.run_sequence(q_seq, k_seq, v_seq, p, q_pos0=int(wl.q_pos0[b]), rows=rows,
                           kernels=kern, with_attention=False)
    grow = int(wl.q_start[b]) + rows
    NB = ref.scores.shape[2]
    gs = res["scores"][grow][:, :, :NB]
    rel = cmp.softmax_score_rel_bound(q_seq[rows], kern, ref.positions, p)
    worst = cmp.check_softmax_scores(gs, ref.scores, rel, ref.positions, p)
    gidx = res["idx"][grow]
    own_sel = orc.select_all(gs.astype(np.float64), ref.positions, p)
    assert np.array_equal(gidx, own_sel), f"{label}: top-k differs on the GPU's own scores"
    rep = cmp.check_indices(gidx, ref.idx, ref.scores, ref.positions, p)
    O, L = orc.sparse_attention(q_seq[rows].astype(np.float64), ref.positions, k_seq, v_seq,
                                gidx, p)
    err, lerr = cmp.check_attention(res["out"][grow], res["lse"][grow], O, L, p.dtype)
    log(f"{label} seq {b}: rows {len(rows)} score err/bound {worst:.3g} idx exact {rep.exact}/"
        f"{rep.rows} band {rep.band} out-err {err:.3g}")


def test_mode1_tiny_f32():
    """The generic float32 path (2 heads, d 64)."""
    wl = synth.make("tiny")
    wl.params = replace(wl.params, score_mode=1)
    log("case mode1 tiny f32")
    res = run_prefill_stages(wl)
    check_mode1(wl, res, 0, label="mode1 tiny")


@pytest.mark.parametrize("Hq,d", [(32, 128), (16, 128), (32, 64), (16, 64)])
def test_mode1_geometries_all_rows(Hq, d):
    """The matrix-core path for each (head_dim, group) pair; 1500 tokens, top-8."""
    p = replace(synth.config_params("prefill32k"), num_q_heads=Hq, head_dim=d, topk=8,
                score_mode=1)
    wl = synth.make_prefill(f"m1-{Hq}-{d}", p, [1500], seed=101, needles_per_seq=1)
    log(f"case mode1 Hq={Hq} d={d}")
    res = run_prefill_stages(wl)
    check_mode1(wl, res, 0, label=f"mode1 {Hq}/{d}")


def test_mode1_edge_and_packed():
    p = replace(synth.config_params("prefill32k"), topk=6, score_mode=1)
    wl = synth.make_prefill("m1-edge", p, [0, 1, 20, 31, 32, 64, 65, 700, 1300], seed=102)
    log("case mode1 edge lengths")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_mode1(wl, res, b, label="mode1 edge")


@pytest.mark.parametrize("n_rows", [1, 3, 40])
def test_mode1_few_rows_against_cache(n_rows):
    """Few query rows at the end of a 5000-token cache: the split path (fewer than 128 work
    items, so a workgroup divides the kernels over its waves); the other tests here take the
    path where every wave streams all kernels."""
    p = replace(synth.config_params("prefill32k"), topk=16, score_mode=1)
    full = synth.make_prefill("m1-few", p, [5000], seed=103, needles_per_seq=1)
    q0 = 5000 - n_rows
    wl = synth.Workload("m1-few", p, full.q[q0:], full.k, full.v, np.array([0]),
                        np.array([n_rows], np.int32), np.array([q0], np.int32), np.array([0]),
                        np.array([5000], np.int32))
    log(f"case mode1 few rows {n_rows}")
    res = run_prefill_stages(wl)
    check_mode1(wl, res, 0, label=f"mode1 few {n_rows}")


def test_mode1_full_size_sampled():
    """The 128K layer in score mode 1: sampled rows, and every needle query still finds its
    needle block."""
    wl = synth.make("prefill128k")
    wl.params = replace(wl.params, score_mode=1)
    log("case mode1 full 128K")
    res = run_prefill_stages(wl)
    for nd in wl.needles:
        rows = int(wl.q_start[nd.seq]) + nd.query_positions
        assert np.all(np.any(res["idx"][rows, nd.kv_head, :] == nd.block, axis=1))
    L = int(wl.q_len[0])
    rows = np.array(sorted(set(range(0, 6144, 509)) | set(range(6144, L, 4099)) |
                           set(range(L - 3, L)) |
                           {int(r) for nd in wl.needles[:4] for r in nd.query_positions[:2]}))
    check_mode1(wl, res, 0, rows=rows, label="mode1 full")


def test_mode1_decode_steps():
    """Two decode steps (infllm2_decode_step) in score mode 1: the step chains the separate
    calls for this mode; scores within the float32 bound, the top-k equal to the oracle's
    selection on the GPU's scores, attention on the GPU's indices."""
    p = replace(synth.config_params("decode128k"), score_mode=1)
    B, Lmax = 3, 6000
    wl = synth.make_decode("m1-dec", p, batch=B, max_len=Lmax, steps=2, seed=104,
                           kv_len0=[5990, 3000, 800])
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kern = torch.zeros((B * Ck, p.num_kv_heads, p.head_dim), dtype=k.dtype, device="cuda")
    bufs = lib.pipeline.decode_buffers(p, B, (Lmax + 63) // 64, 0, "cuda")
    for st in range(2):
        kv = wl.kv_len0.astype(np.int64) + st + 1
        seqs = lib.Seqs.decode(kv, Lmax, Ck)
        log(f"case mode1 decode step {st}")
        lib.decode_step(p, seqs, dev(wl.q_steps[st], p.dtype), k, v, kern, None, bufs)
        torch.cuda.synchronize()
        scores, idx = host(bufs["scores"]), host(bufs["idx"])
        out, lse = host(bufs["out"]), host(bufs["lse"])
        for b in range(B):
            L = int(kv[b])
            ks, vs = wl.k[b, :L], wl.v[b, :L]
            qr = wl.q_steps[st][b:b + 1]
            kern_ref = orc.compress_kernels(ks, p.kernel_size, p.kernel_stride, p.dtype)
            ref = orc.run_sequence(qr, ks, vs, p, q_pos0=L - 1, kernels=kern_ref,
                                   with_attention=False)
            NB = ref.scores.shape[2]
            gs = scores[b:b + 1, :, :NB]
            rel = cmp.softmax_score_rel_bound(qr, kern_ref, ref.positions, p)
            cmp.check_softmax_scores(gs, ref.scores, rel, ref.positions, p)
            gidx = idx[b:b + 1]
            assert np.array_equal(gidx, orc.select_all(gs.astype(np.float64), ref.positions, p))
            cmp.check_indices(gidx, ref.idx, ref.scores, ref.positions, p)
            O, Ls = orc.sparse_attention(qr.astype(np.float64), ref.positions, ks, vs, gidx, p)
            cmp.check_attention(out[b:b + 1], lse[b:b + 1], O, Ls, p.dtype)
