"""Parity of the HIP backward (dQ, dK, dV through infllm2_sparse_attn_backward) with the CPU
oracle, the block selection taken from the HIP forward and held fixed.

Small workloads are compared on every query row and every key; the 128K workload on sampled
query rows (dQ), on the keys of sampled blocks (dK, dV: every row that selected the block is
replayed in the oracle) and through two identities that hold for the whole tensors:
sum_j dV_j = sum over rows and heads of dO (the softmax weights of a row sum to one) and
sum_j dK_j = 0 (the dS of a row sum to zero).  Bounds are in tests/_compare.py.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import infllm2_oracle as orc
from tests import _compare as cmp
from tests._gpu import dev, host, log, run_prefill_stages, seqs_for

import block_sparse_long_semantic_amd as lib

pytestmark = pytest.mark.gpu


def run_backward(wl, res, dout, repeats=1):
    """Backward on the forward's own results; dq, dk, dv start as NaN so that every element
    the call must write is checked to be written."""
    p = wl.params
    seqs = seqs_for(wl, p)
    q, k, v = dev(wl.q, p.dtype), dev(wl.k, p.dtype), dev(wl.v, p.dtype)
    idx = torch.from_numpy(res["idx"]).to("cuda")
    out = dev(res["out"], p.dtype)
    lse = torch.from_numpy(res["lse"]).to("cuda")
    do = dev(dout, p.dtype)
    ws = torch.empty(lib.backward_workspace_size(p, seqs), dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(repeats):
        dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        dk = torch.full(k.shape, float("nan"), dtype=torch.float32, device="cuda")
        dv = torch.full(v.shape, float("nan"), dtype=torch.float32, device="cuda")
        lib.sparse_attn_backward(p, seqs, q, k, v, idx, out, lse, do, dq, dk, dv, ws)
        torch.cuda.synchronize()
        runs.append({"dq": host(dq), "dk": host(dk), "dv": host(dv)})
        del dq, dk, dv
    return runs if repeats > 1 else runs[0]


def check_backward_sequence(wl, res, dout, g, b, label):
    """Every row and key of sequence b against the oracle on the HIP path's indices."""
    p = wl.params
    sl_q, sl_k = wl.seq_slices(b)
    n = int(wl.q_len[b])
    if int(wl.kv_len[b]) == 0:
        return
    if n == 0:                          # no query: the keys' gradients are exactly zero
        assert np.all(g["dk"][sl_k] == 0) and np.all(g["dv"][sl_k] == 0), label
        return
    pos = int(wl.q_pos0[b]) + np.arange(n)
    args = (wl.q[sl_q], pos, wl.k[sl_k], wl.v[sl_k], res["idx"][sl_q], dout[sl_q], p)
    dQ, dK, dV = orc.sparse_attention_backward(*args)
    mq, mk, mv = cmp.backward_magnitudes(*args)
    rq = cmp.check_gradient(f"{label} dq", g["dq"][sl_q], dQ, mq)
    rk = cmp.check_gradient(f"{label} dk", g["dk"][sl_k], dK, mk)
    rv = cmp.check_gradient(f"{label} dv", g["dv"][sl_k], dV, mv)
    log(f"{label} seq {b}: rows {n} keys {int(wl.kv_len[b])} error/bound dq {rq:.3g} "
        f"dk {rk:.3g} dv {rv:.3g}")


def forward_and_backward(wl, seed, repeats=1):
    res = run_prefill_stages(wl)
    dout = synth.make_upstream_grad(wl.q.shape, seed, wl.params.dtype)
    return res, dout, run_backward(wl, res, dout, repeats)


# ------------------------------------------------------------------------- small, all rows

@pytest.mark.parametrize("Hq,Hkv,d", [(32, 2, 128), (16, 2, 128), (32, 2, 64), (16, 2, 64)])
def test_backward_geometries_all_rows(Hq, Hkv, d):
    """Each supported (head_dim, group) pair; 700 tokens = 11 blocks, a ragged last tile and
    block, top-4 so that rows attend few blocks."""
    p = replace(synth.config_params("prefill32k"), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                topk=4)
    wl = synth.make_prefill(f"bwd-{Hq}-{d}", p, [700], seed=51)
    log(f"case backward Hq={Hq} Hkv={Hkv} d={d}")
    res, dout, g = forward_and_backward(wl, seed=52)
    check_backward_sequence(wl, res, dout, g, 0, f"bwd {Hq}/{Hkv}/{d}")


def test_backward_8b_shape_sparse_and_dense():
    """MiniCPM4-8B head layout: 1100 tokens at top-8 (sparse) and at top-64 (every block, so
    the gradient is that of dense causal attention)."""
    base = synth.config_params("prefill32k")
    for topk in (8, 64):
        wl = synth.make_prefill("bwd-8b", replace(base, topk=topk), [1100], seed=53,
                                needles_per_seq=1)
        log(f"case backward 8b topk={topk}")
        res, dout, g = forward_and_backward(wl, seed=54)
        check_backward_sequence(wl, res, dout, g, 0, f"bwd 8b top{topk}")


def test_backward_edge_sequences():
    """Empty, single-token, shorter-than-a-window and one-block sequences packed together."""
    p = replace(synth.config_params("prefill32k"), topk=6)
    wl = synth.make_prefill("bwd-edge", p, [0, 1, 20, 31, 32, 64, 65, 700], seed=55)
    log("case backward edge lengths")
    res, dout, g = forward_and_backward(wl, seed=56)
    for b in range(wl.num_seqs):
        check_backward_sequence(wl, res, dout, g, b, "bwd edge")


def test_backward_varlen_packed():
    """The variable-length workload's layout (16 query heads, 2 KV heads, d = 64, heavy-tailed
    key norms), shrunk 32 times, top-8."""
    wl = synth.make("varlen", length_scale=1 / 32)
    wl.params = replace(wl.params, topk=8)
    log("case backward varlen/32")
    res, dout, g = forward_and_backward(wl, seed=57)
    for b in range(wl.num_seqs):
        check_backward_sequence(wl, res, dout, g, b, "bwd varlen/32")


def test_backward_chunk_against_cache():
    """Queries for the last 700 tokens only (q_pos0 > 0): keys before the chunk still receive
    gradients from the chunk's rows."""
    p = replace(synth.config_params("prefill32k"), topk=8)
    full = synth.make_prefill("bwd-chunk", p, [2600], seed=58, needles_per_seq=1)
    q0 = 1900
    wl = synth.Workload("bwd-chunk", p, full.q[q0:], full.k, full.v, np.array([0]),
                        np.array([700], np.int32), np.array([q0], np.int32), np.array([0]),
                        np.array([2600], np.int32))
    log("case backward chunk")
    res, dout, g = forward_and_backward(wl, seed=59)
    check_backward_sequence(wl, res, dout, g, 0, "bwd chunk")


def test_backward_repeat_calls():
    """The workspace needs no clearing between calls; dq is bit-identical, dk and dv (summed
    with atomics) agree to float32 rounding."""
    p = replace(synth.config_params("prefill32k"), topk=8)
    wl = synth.make_prefill("bwd-rep", p, [3000, 777], seed=60)
    log("case backward repeat")
    res, dout, runs = forward_and_backward(wl, seed=61, repeats=3)
    a = runs[0]
    for r in runs[1:]:
        assert np.array_equal(a["dq"], r["dq"])
        for n in ("dk", "dv"):
            scale = np.abs(a[n]).max()
            assert np.abs(a[n] - r[n]).max() <= 1e-5 * scale, n
    for b in range(wl.num_seqs):
        check_backward_sequence(wl, res, dout, a, b, "bwd repeat")


# ------------------------------------------------------------------------- full size

def test_backward_full_size_sampled():
    """The 128K workload: sampled rows, the keys of the last two blocks, whole-tensor sums."""
    wl = synth.make("prefill128k")
    p = wl.params
    log("case backward full prefill128k")
    res, dout, g = forward_and_backward(wl, seed=62)
    L = int(wl.q_len[0])
    pos = np.arange(L)
    # dQ on sampled rows
    dense = min(L, p.topk * p.block_size)
    rows = np.array(sorted(set(range(0, dense, 997)) | set(range(L - 3, L)) |
                           set(range(dense, L, 7919))))
    args = (wl.q[rows], pos[rows], wl.k, wl.v, res["idx"][rows], dout[rows], p)
    dQ, _, _ = orc.sparse_attention_backward(*args)
    mq, _, _ = cmp.backward_magnitudes(*args)
    rq = cmp.check_gradient("full dq", g["dq"][rows], dQ, mq)
    # dK, dV on the keys of the last two blocks: replay every row that selected them
    NB = (L + p.block_size - 1) // p.block_size
    for blk in (NB - 1, NB - 2):
        sel = np.any(res["idx"] == blk, axis=2).any(axis=1)
        r = np.nonzero(sel)[0]
        args = (wl.q[r], pos[r], wl.k, wl.v, res["idx"][r], dout[r], p)
        _, dK, dV = orc.sparse_attention_backward(*args)
        _, mk, mv = cmp.backward_magnitudes(*args)
        keys = slice(blk * p.block_size, min(L, (blk + 1) * p.block_size))
        rk = cmp.check_gradient(f"full dk block {blk}", g["dk"][keys], dK[keys], mk[keys])
        rv = cmp.check_gradient(f"full dv block {blk}", g["dv"][keys], dV[keys], mv[keys])
        log(f"full block {blk}: {len(r)} rows, error/bound dk {rk:.3g} dv {rv:.3g}")
    # whole-tensor identities per KV head
    G = p.group
    for kv in range(p.num_kv_heads):
        dsum = dout[:, kv * G:(kv + 1) * G, :].astype(np.float64)
        want = dsum.sum(axis=(0, 1))
        # each P_j is rounded to bf16 once (2^-9) and comes from the stored lse
        bound_v = 2.0 ** -8 * np.abs(dsum).sum(axis=(0, 1))
        got = g["dv"][:, kv, :].astype(np.float64).sum(axis=0)
        assert np.all(np.abs(got - want) <= bound_v), "sum of dV"
        # sum_j dS_j = 0 per (row, head); its rounding error is below 2^-8 sum_j E_j with
        # sum_j E_j <= 6 |dO|_1 max|v| (|dP_j|, |delta|, A and the dP term, each bounded by
        # |dO|_1 max|v| or twice it), hence |sum_j dK_j| <= 2^-8 scale sum 6 |dO|_1 vmax |q|
        vmax = float(np.abs(wl.v[:, kv, :]).max())
        l1 = np.abs(dsum).sum(axis=2)                                          # [L, G]
        qa = np.abs(wl.q[:, kv * G:(kv + 1) * G, :].astype(np.float64))
        bound_k = 2.0 ** -8 * p.scale * 6 * vmax * np.einsum("rh,rhd->d", l1, qa)
        gk = g["dk"][:, kv, :].astype(np.float64).sum(axis=0)
        assert np.all(np.abs(gk) <= bound_k), "sum of dK"
        log(f"full kv head {kv}: |sum dV - sum dO| / bound {np.abs(got - want).max() / bound_v.min():.3g}, "
            f"|sum dK| / bound {(np.abs(gk) / bound_k).max():.3g}")
    log(f"full dq rows {len(rows)} error/bound {rq:.3g}")
