"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names the pin it provides.  Library routines (numpy's sliding windows, torch's
scaled-dot-product attention), closed forms, a pure-Python brute force, and the one number
the pages print for this path (fewer than 5% of tokens attended at 128K, MiniCPM4-8B model
card, "Efficient Model Architecture") fix the oracle; nothing here compares the oracle with
itself.
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import brute
from oracle import infllm2_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_params(**kw):
    base = dict(num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=16, kernel_size=8,
                kernel_stride=4, topk=4, num_init_blocks=1, num_local_blocks=1, dtype="bf16")
    base.update(kw)
    return synth.Params(**base)


def to_nested(a):
    return [[[float(x) for x in row] for row in tok] for tok in a]


# ----------------------------------------------------------------------------- rounding

def test_storage_rounding_matches_exact_rational_rounding():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                        # exact ties between bf16 neighbours: 1 + (2j+1) * 2^-8
                        1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8,
                        -(1.0 + (2 * np.arange(64) + 1) * 2.0 ** -8), [0.0, -0.0]])
    got = orc.round_to_storage(x, "bf16")
    ref = np.array([brute.bf16_nearest(float(v)) for v in x])
    assert np.array_equal(got, ref)
    # ties go to the even neighbour: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    assert orc.round_to_storage(np.array([1 + 2 ** -8]), "bf16")[0] == 1.0
    assert orc.round_to_storage(np.array([1 + 3 * 2 ** -8]), "bf16")[0] == 1 + 2 ** -6


def test_storage_rounding_matches_torch_on_f32_values():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(20000) * 3).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_to_storage(x.astype(np.float64), "bf16"), ref)


# ----------------------------------------------------------------------------- kernels

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pooling_matches_numpy_window_mean(dtype):
    """P5: kernel c is the mean of keys s*c .. s*c+w-1 (numpy sliding windows)."""
    p = synth.config_params("tiny") if dtype == "f32" else synth.config_params("varlen")
    wl = synth.make_prefill("t", replace(p, dtype=dtype), [500], seed=11)
    K = wl.k.astype(np.float64)
    w, s = p.kernel_size, p.kernel_stride
    mean = np.lib.stride_tricks.sliding_window_view(K, w, axis=0)[::s].mean(axis=-1)
    ours = orc.exact_window_means(K, w, s, 0, orc.num_kernels(500, w, s), dtype)
    assert ours.shape == mean.shape == (orc.num_kernels(500, w, s),) + K.shape[1:]
    np.testing.assert_allclose(ours, mean, rtol=0, atol=1e-14)
    got = orc.compress_kernels(K, w, s, dtype)
    assert np.array_equal(got, orc.round_to_storage(ours, dtype))
    assert (500 - w) // s + 1 == got.shape[0]


def test_window_sum_certificate_falls_back_to_exact_sum():
    """Windows mixing magnitudes far apart must still give the exact mean."""
    K = np.zeros((32, 1, 1))
    K[0] = 2.0 ** 40
    K[1] = 2.0 ** -40
    K[2] = -(2.0 ** 40)
    m = orc.exact_window_means(K, 32, 16, 0, 1, "f32")
    assert m[0, 0, 0] == 2.0 ** -40 / 32


def test_window_mean_rounds_once_from_the_exact_value():
    """Rounding the exact mean, not a float64 approximation of it.  Window of w = 32 with keys
    1, 2^-8 and 2^-80 (all bf16 values) and zeros: the exact mean (1 + 2^-8 + 2^-80) / 32 lies
    just above the bf16 midpoint (1 + 2^-8) / 32 of its neighbours 2^-5 and (1 + 2^-7) 2^-5, so
    it rounds up, while its nearest float64 is the midpoint itself and would round to the even
    neighbour 2^-5.  Likewise for w = 6, where the division itself rounds: keys 4, 2, 2^-6,
    2^-7, 2^-58, 2^-59 have the exact mean 1 + 2^-8 + 2^-60 (just above a midpoint: up), and with
    the last two keys negated 1 + 2^-8 - 2^-60 (just below: down)."""
    K = np.zeros((32, 1, 1))
    K[0], K[1], K[2] = 1.0, 2.0 ** -8, 2.0 ** -80
    got = orc.compress_kernels(K, 32, 16, "bf16")
    assert got[0, 0, 0] == (1 + 2.0 ** -7) * 2.0 ** -5
    K6 = np.array([4.0, 2.0, 2.0 ** -6, 2.0 ** -7, 2.0 ** -58, 2.0 ** -59]).reshape(6, 1, 1)
    assert orc.compress_kernels(K6, 6, 6, "bf16")[0, 0, 0] == 1 + 2.0 ** -7
    K6[4:] *= -1
    assert orc.compress_kernels(K6, 6, 6, "bf16")[0, 0, 0] == 1.0
    # a mean that is exactly a midpoint still ties to even
    K6 = np.array([4.0, 2.0, 2.0 ** -6, 2.0 ** -7, 0.0, 0.0]).reshape(6, 1, 1)
    assert orc.compress_kernels(K6, 6, 6, "bf16")[0, 0, 0] == 1.0


def test_incremental_kernels_equal_full_compress():
    """P9: appending tokens one at a time creates exactly the kernels of the full pass."""
    p = synth.config_params("varlen")
    wl = synth.make_prefill("t", p, [301], seed=12, student_t_keys=True)
    K = wl.k.astype(np.float64)
    full = orc.compress_kernels(K, p.kernel_size, p.kernel_stride, p.dtype)
    parts = []
    for L in range(1, 302):
        lo, hi = orc.new_kernel_range(L - 1, L, p.kernel_size, p.kernel_stride)
        assert hi - lo in (0, 1)
        if hi > lo:
            assert p.kernel_stride * lo + p.kernel_size == L
            parts.append(orc.compress_kernels(K[:L], p.kernel_size, p.kernel_stride, p.dtype, lo, hi))
    assert np.array_equal(np.concatenate(parts), full)


# ----------------------------------------------------------------------------- geometry

def test_kernels_of_block_by_token_sets():
    for (B, w, s) in [(64, 32, 16), (16, 8, 4), (64, 64, 32), (32, 16, 16)]:
        C = 40
        for b in range(12):
            blk = set(range(B * b, B * (b + 1)))
            expect = [c for c in range(C) if set(range(s * c, s * c + w)) & blk]
            assert list(orc.kernels_of_block(b, B, w, s, C)) == expect
    # the measured geometry: kernels 4b-1 .. 4b+3
    assert list(orc.kernels_of_block(5, 64, 32, 16, 100)) == [19, 20, 21, 22, 23]


def test_presum_identity():
    """P10: sum_h q_h . k equals (sum_h q_h) . k to float64 rounding."""
    wl = synth.make("prefill32k", length_scale=1 / 64)
    p = wl.params
    K = wl.k.astype(np.float64)
    kern = orc.compress_kernels(K, p.kernel_size, p.kernel_stride, p.dtype)
    q = wl.q[:300].astype(np.float64)
    u = orc.kernel_scores(q, kern, p.num_kv_heads, p.scale)
    G = p.group
    for g in range(p.num_kv_heads):
        qs = q[:, g * G:(g + 1) * G, :].sum(axis=1)
        pre = p.scale * qs @ kern[:, g, :].T
        bound = p.scale * np.abs(q[:, g * G:(g + 1) * G, :]).sum(axis=1) @ np.abs(kern[:, g, :]).T
        assert np.all(np.abs(u[:, g, :] - pre) <= 1e-12 * bound)


# ----------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("case", [
    dict(p=small_params(), L=150, seed=21),
    dict(p=small_params(dtype="f32", topk=3, num_local_blocks=2, num_init_blocks=0), L=133, seed=22),
    dict(p=small_params(block_size=16, kernel_size=16, kernel_stride=8, topk=5,
                        num_init_blocks=2, num_local_blocks=1), L=170, seed=23),
])
def test_oracle_equals_brute_force(case):
    """P4: pure-Python loops with exact sums equal the numpy oracle."""
    p, L = case["p"], case["L"]
    wl = synth.make_prefill("b", p, [L], seed=case["seed"])
    res = orc.run_sequence(wl.q, wl.k, wl.v, p)
    kern, S, I, O, LSE = brute.run(to_nested(wl.q), to_nested(wl.k), to_nested(wl.v),
                                   p.num_kv_heads, p.block_size, p.kernel_size, p.kernel_stride,
                                   p.topk, p.num_init_blocks, p.num_local_blocks, p.dtype, p.scale)
    assert np.array_equal(res.kernels, np.array(kern))
    S = np.array(S)
    fin = np.isfinite(S)
    assert np.array_equal(fin, np.isfinite(res.scores))
    np.testing.assert_allclose(res.scores[fin], S[fin], rtol=1e-12, atol=1e-12)
    assert np.array_equal(res.idx, np.array(I, dtype=np.int32))
    np.testing.assert_allclose(res.out, np.array(O), rtol=0, atol=1e-12)
    np.testing.assert_allclose(res.lse, np.array(LSE), rtol=0, atol=1e-12)


def test_oracle_equals_brute_force_on_tiny_rows():
    """P4 on the measured tiny configuration (sampled rows, 64-token blocks)."""
    wl = synth.make("tiny")
    p = wl.params
    rows = [0, 30, 31, 63, 64, 200, 255, 256, 300, 447, 448, 511]
    res = orc.run_sequence(wl.q, wl.k, wl.v, p, rows=rows)
    kern, S, I, O, LSE = brute.run(to_nested(wl.q), to_nested(wl.k), to_nested(wl.v),
                                   p.num_kv_heads, p.block_size, p.kernel_size, p.kernel_stride,
                                   p.topk, p.num_init_blocks, p.num_local_blocks, p.dtype, p.scale,
                                   rows=rows)
    assert np.array_equal(res.kernels, np.array(kern))
    assert np.array_equal(res.idx, np.array(I, dtype=np.int32))
    np.testing.assert_allclose(res.out, np.array(O), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- selection

def test_dense_reduction_equals_causal_attention():
    """P1: with topk covering every block, the output is plain causal attention (torch SDPA in
    float64 and a textbook masked softmax)."""
    wl = synth.make("tiny")
    p = replace(wl.params, topk=8)
    res = orc.run_sequence(wl.q, wl.k, wl.v, p)
    q = torch.from_numpy(wl.q.astype(np.float64)).transpose(0, 1)     # [H, L, d]
    G = p.group
    k = torch.from_numpy(wl.k.astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
    v = torch.from_numpy(wl.v.astype(np.float64)).transpose(0, 1).repeat_interleave(G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    np.testing.assert_allclose(res.out, ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    # textbook: masked full matrix, log-sum-exp
    qn, kn, vn = wl.q.astype(np.float64), wl.k.astype(np.float64), wl.v.astype(np.float64)
    L = qn.shape[0]
    mask = np.tril(np.ones((L, L), bool))
    for h in range(p.num_q_heads):
        z = p.scale * qn[:, h] @ kn[:, h // G].T
        z = np.where(mask, z, -np.inf)
        lse = np.log(np.exp(z - z.max(1, keepdims=True)).sum(1)) + z.max(1)
        np.testing.assert_allclose(res.lse[:, h], lse, rtol=0, atol=1e-12)


def test_group_sharing_and_head_permutation():
    """P2: one block set per (token, KV head); permuting the heads inside a group leaves the
    selection unchanged and permutes the outputs."""
    wl = synth.make("varlen", length_scale=1 / 16)
    p = wl.params
    sl_q, sl_k = wl.seq_slices(2)
    q, k, v = wl.q[sl_q], wl.k[sl_k], wl.v[sl_k]
    rows = np.arange(0, q.shape[0], 7)
    base = orc.run_sequence(q, k, v, p, rows=rows)
    assert base.idx.shape == (len(rows), p.num_kv_heads, p.topk)
    G = p.group
    perm = np.concatenate([g * G + np.random.default_rng(g).permutation(G)
                           for g in range(p.num_kv_heads)])
    other = orc.run_sequence(q[:, perm], k, v, p, rows=rows)
    assert np.array_equal(base.idx, other.idx)
    np.testing.assert_allclose(other.out, base.out[:, perm], rtol=0, atol=1e-12)


def test_selection_invariants():
    """P11: forced blocks always selected; exactly topk blocks once more than topk are
    reachable; selection inside the reachable blocks, ascending, -1 padded."""
    wl = synth.make("prefill32k", length_scale=1 / 16)
    p = wl.params
    rows = np.concatenate([np.arange(0, 200), np.arange(200, wl.q.shape[0], 37)])
    res = orc.run_sequence(wl.q, wl.k, wl.v, p, rows=rows, with_attention=False)
    for r, pos in enumerate(res.positions):
        own = pos // p.block_size
        F = set(orc.forced_blocks(int(pos), p).tolist())
        for g in range(p.num_kv_heads):
            sel = res.idx[r, g]
            real = sel[sel >= 0]
            assert np.all(np.diff(real) > 0)
            assert np.all(sel[len(real):] == -1)
            assert np.all(real <= own)
            assert F <= set(real.tolist())
            assert len(real) == min(p.topk, own + 1)
            # every unselected non-forced block scores no higher than every chosen one
            if own + 1 > p.topk:
                chosen = [b for b in real if b not in F]
                rest = [b for b in range(own + 1) if b not in set(real.tolist())]
                if rest:
                    assert min(res.scores[r, g, chosen]) >= max(res.scores[r, g, rest])


def test_ties_go_to_lower_index():
    p = small_params(topk=3, num_init_blocks=1, num_local_blocks=1)
    pos = 16 * 9 + 3                    # own block 9; forced {0, 9}; one free slot
    S = np.full(10, 1.0)
    S[[4, 7]] = 2.0
    assert orc.select_blocks(S, pos, p).tolist() == [0, 4, 9]
    S[4] = -0.0; S[7] = 0.0; S[[1, 2, 3, 5, 6, 8]] = -1.0
    assert orc.select_blocks(S, pos, p).tolist() == [0, 4, 9]


def test_needles_are_selected():
    """P6: every planted (query, needle block) pair is selected."""
    for name, scale in [("prefill32k", 1 / 8), ("prefill128k", 1 / 32)]:
        wl = synth.make(name, length_scale=scale)
        p = wl.params
        assert wl.needles
        for nd in wl.needles:
            res = orc.run_sequence(wl.q, wl.k, wl.v, p, rows=nd.query_positions,
                                   with_attention=False)
            assert np.all(np.any(res.idx[:, nd.kv_head, :] == nd.block, axis=1)), (name, nd.block)


# ----------------------------------------------------------------------------- attention

def test_gather_equals_masked_dense():
    """P7: attention over gathered block tokens equals a dense softmax with the block mask."""
    wl = synth.make("tiny")
    p = wl.params
    res = orc.run_sequence(wl.q, wl.k, wl.v, p)
    q, k, v = (a.astype(np.float64) for a in (wl.q, wl.k, wl.v))
    L = q.shape[0]
    j = np.arange(L)
    for h in range(p.num_q_heads):
        g = h // p.group
        sel_mask = np.zeros((L, L), bool)
        for i in range(L):
            chosen = res.idx[i, g][res.idx[i, g] >= 0]
            sel_mask[i] = np.isin(j // p.block_size, chosen) & (j <= i)
        z = np.where(sel_mask, p.scale * q[:, h] @ k[:, g].T, -np.inf)
        e = np.exp(z - z.max(1, keepdims=True))
        out = (e / e.sum(1, keepdims=True)) @ v[:, g]
        np.testing.assert_allclose(res.out[:, h], out, rtol=0, atol=1e-12)


def test_lse_merge_identity():
    """P8 (oracle side): attention over disjoint key subsets merged by log-sum-exp equals the
    attention over their union."""
    rng = np.random.default_rng(9)
    z = rng.standard_normal((3, 500)) * 3
    v = rng.standard_normal((500, 5))
    parts = np.array_split(np.arange(500), 7)
    ms = np.array([z[:, pp].max(1) for pp in parts])
    ls = np.array([np.exp(z[:, pp] - z[:, pp].max(1, keepdims=True)).sum(1) for pp in parts])
    os_ = np.array([(np.exp(z[:, pp] - z[:, pp].max(1, keepdims=True)) @ v[pp]) / l[:, None]
                    for pp, l in zip(parts, ls)])
    out, lse = orc.lse_merge(ms, ls, os_)
    e = np.exp(z - z.max(1, keepdims=True))
    np.testing.assert_allclose(out, (e @ v) / e.sum(1, keepdims=True), atol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(1)), atol=1e-12)


# ----------------------------------------------------------------------------- sparsity

def test_attended_key_counts_closed_form():
    """P3: keys attended per query follow the closed form, on the oracle's own token sets."""
    wl = synth.make("tiny")
    p = wl.params
    res = orc.run_sequence(wl.q, wl.k, wl.v, p)
    for r, pos in enumerate(res.positions):
        n = len(orc.attended_keys(res.idx[r, 0], int(pos), wl.k.shape[0], p.block_size))
        assert n == orc.attended_key_count(int(pos), p)


def test_sparsity_matches_golden_and_page_claim():
    """P3 totals against hand-derived values, and the model card's '<5% of tokens at 128K'."""
    with open(os.path.join(GOLDEN, "sparsity.json")) as f:
        gold = json.load(f)
    for name, ent in gold["totals_per_head"].items():
        p = synth.config_params(name)
        lens = ent["seq_lens"]
        total = sum(orc.attended_key_count(i, p) for L in lens for i in range(L))
        assert total == ent["keys"], name
    p = synth.config_params("prefill128k")
    last = orc.attended_key_count(131071, p)
    assert last == gold["last_token_128k"]["keys"]
    assert last / 131072 < gold["last_token_128k"]["page_bound_fraction"]


# ----------------------------------------------------------------------------- backward

def _loss(q, k, v, idx, positions, dout, p):
    O, _ = orc.sparse_attention(q, positions, k, v, idx, p)
    return float((O * dout).sum())


def test_backward_matches_finite_differences():
    """Gradients of sum(O * dO) by central differences of the oracle's own forward, the
    selection held fixed (float64 inputs; sampled entries of Q, K and V)."""
    p = small_params(dtype="f32", topk=3, num_local_blocks=1, num_init_blocks=1)
    wl = synth.make_prefill("bwd", p, [70], seed=51)
    q, k, v = (a.astype(np.float64) for a in (wl.q, wl.k, wl.v))
    res = orc.run_sequence(wl.q, wl.k, wl.v, p, with_attention=False)
    idx, pos = res.idx, res.positions
    dout = np.random.default_rng(52).standard_normal(q.shape)
    dQ, dK, dV = orc.sparse_attention_backward(q, pos, k, v, idx, dout, p)
    rng = np.random.default_rng(53)
    eps = 1e-6
    for name, arr, grad in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        flat = rng.choice(arr.size, 40, replace=False)
        for f in flat:
            ix = np.unravel_index(f, arr.shape)
            saved = arr[ix]
            arr[ix] = saved + eps
            up = _loss(q, k, v, idx, pos, dout, p)
            arr[ix] = saved - eps
            dn = _loss(q, k, v, idx, pos, dout, p)
            arr[ix] = saved
            fd = (up - dn) / (2 * eps)
            assert abs(fd - grad[ix]) <= 1e-6 * (1 + abs(fd)), (name, ix, fd, grad[ix])


def test_backward_dense_reduction_equals_autograd():
    """With topk covering every block the gradients are those of plain causal attention
    (torch autograd through scaled_dot_product_attention, float64)."""
    wl = synth.make("tiny")
    p = replace(wl.params, topk=8)
    res = orc.run_sequence(wl.q, wl.k, wl.v, p, with_attention=False)
    q, k, v = (a.astype(np.float64) for a in (wl.q, wl.k, wl.v))
    dout = np.random.default_rng(54).standard_normal(q.shape)
    dQ, dK, dV = orc.sparse_attention_backward(q, res.positions, k, v, res.idx, dout, p)
    G = p.group
    tq = torch.from_numpy(q).transpose(0, 1).requires_grad_(True)          # [Hq, L, d]
    tk = torch.from_numpy(k).transpose(0, 1).requires_grad_(True)          # [Hkv, L, d]
    tv = torch.from_numpy(v).transpose(0, 1).requires_grad_(True)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, 0), tv.repeat_interleave(G, 0), is_causal=True)
    out.backward(torch.from_numpy(dout).transpose(0, 1))
    np.testing.assert_allclose(dQ, tq.grad.transpose(0, 1).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dK, tk.grad.transpose(0, 1).numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dV, tv.grad.transpose(0, 1).numpy(), rtol=0, atol=1e-10)


# ------------------------------------------------------------------------- sliding window

@pytest.mark.parametrize("window", [1, 5, 64, 100, 1000])
def test_window_attention_matches_banded_sdpa(window):
    """Sliding-window attention equals torch SDPA (float64) with an explicit band mask
    pos - window < j <= pos, for GQA heads; lse equals the band's log-sum-exp (torch)."""
    p = small_params(dtype="f32", num_q_heads=4, num_kv_heads=2)
    rng = np.random.default_rng(81)
    L = 150
    q = rng.standard_normal((L, 4, p.head_dim))
    k = rng.standard_normal((L, 2, p.head_dim))
    v = rng.standard_normal((L, 2, p.head_dim))
    rows = np.arange(L)
    O, lse = orc.window_attention(q, rows, k, v, window, p)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    band = (j <= i) & (j > i - window)
    qt = torch.from_numpy(q).transpose(0, 1)
    kt = torch.from_numpy(k).transpose(0, 1).repeat_interleave(2, 0)
    vt = torch.from_numpy(v).transpose(0, 1).repeat_interleave(2, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=band,
                                                           scale=p.scale)
    np.testing.assert_allclose(O, ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
    z = p.scale * torch.einsum("hid,hjd->hij", qt, kt).masked_fill(~band, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=2).transpose(0, 1).numpy(),
                               rtol=0, atol=1e-12)


def test_window_of_one_returns_own_value():
    """A window of one token: the output is that token's value and lse its own scaled logit."""
    p = small_params(dtype="f32")
    rng = np.random.default_rng(82)
    L = 40
    q = rng.standard_normal((L, p.num_q_heads, p.head_dim))
    k = rng.standard_normal((L, p.num_kv_heads, p.head_dim))
    v = rng.standard_normal((L, p.num_kv_heads, p.head_dim))
    O, lse = orc.window_attention(q, np.arange(L), k, v, 1, p)
    G = p.group
    for h in range(p.num_q_heads):
        np.testing.assert_array_equal(O[:, h], v[:, h // G])
        np.testing.assert_allclose(lse[:, h], p.scale * (q[:, h] * k[:, h // G]).sum(1),
                                   rtol=0, atol=1e-13)


def test_window_covering_the_past_is_sparse_attention_over_all_blocks():
    """A window at least as long as the sequence is plain causal attention, which is also what
    the block-sparse attention computes when every block is selected."""
    wl = synth.make("tiny")
    p = replace(wl.params, topk=8)
    pos = np.arange(512)
    idx = np.tile(np.arange(8, dtype=np.int32), (512, 1, 1))
    O1, L1 = orc.window_attention(wl.q, pos, wl.k, wl.v, 512, p)
    O2, L2 = orc.sparse_attention(wl.q, pos, wl.k, wl.v, idx, p)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)


# ------------------------------------------------------------------------- score mode 1

@pytest.mark.parametrize("case", [
    dict(p=small_params(score_mode=1), L=150, seed=91),
    dict(p=small_params(dtype="f32", topk=3, num_local_blocks=2, num_init_blocks=0,
                        score_mode=1), L=133, seed=92),
])
def test_softmax_scores_equal_brute_force(case):
    """P4 for score mode 1: the pure-Python statement (per-head exps over an fsum, explicit
    token sets) gives the same scores and selections."""
    p, L = case["p"], case["L"]
    wl = synth.make_prefill("b", p, [L], seed=case["seed"])
    res = orc.run_sequence(wl.q, wl.k, wl.v, p)
    kern, S, I, O, LSE = brute.run(to_nested(wl.q), to_nested(wl.k), to_nested(wl.v),
                                   p.num_kv_heads, p.block_size, p.kernel_size, p.kernel_stride,
                                   p.topk, p.num_init_blocks, p.num_local_blocks, p.dtype, p.scale,
                                   score_mode=1)
    S = np.array(S)
    fin = np.isfinite(S)
    assert np.array_equal(fin, np.isfinite(res.scores))
    np.testing.assert_allclose(res.scores[fin], S[fin], rtol=1e-12, atol=1e-14)
    assert np.array_equal(res.idx, np.array(I, dtype=np.int32))
    np.testing.assert_allclose(res.out, np.array(O), rtol=0, atol=1e-12)


def test_softmax_scores_against_scipy_softmax():
    """The per-head normalisation is scipy's softmax over the visible kernels; the group's
    probabilities sum to G per row; a row that sees exactly one kernel scores G on it."""
    from scipy.special import softmax
    p = small_params(score_mode=1)
    wl = synth.make_prefill("s", p, [90], seed=93)
    kern = orc.compress_kernels(wl.k, p.kernel_size, p.kernel_stride, p.dtype)
    pos = np.arange(90)
    u = orc.kernel_scores_softmax(wl.q, pos, kern, p)
    C = kern.shape[0]
    G = p.group
    for r in range(90):
        vis = [c for c in range(C) if p.kernel_stride * c + p.kernel_size - 1 <= r]
        for g in range(p.num_kv_heads):
            want = np.zeros(C)
            for h in range(g * G, (g + 1) * G):
                if vis:
                    z = p.scale * wl.q[r, h].astype(np.float64) @ kern[vis, g].astype(np.float64).T
                    want[vis] += softmax(z)
            np.testing.assert_allclose(u[r, g], want, rtol=1e-12, atol=1e-15)
            if vis:
                assert math.isclose(u[r, g].sum(), G, rel_tol=1e-12)
            if len(vis) == 1:
                assert math.isclose(u[r, g, vis[0]], G, rel_tol=1e-14)


def test_softmax_scores_without_kernels():
    """A sequence shorter than one kernel window has no kernels: every block score is -inf in
    both score modes (windows complete only; kernel visible only once its last token is seen)."""
    for mode in (0, 1):
        p = small_params(score_mode=mode)
        wl = synth.make_prefill("s", p, [p.kernel_size - 1], seed=94)
        res = orc.run_sequence(wl.q, wl.k, wl.v, p)
        assert res.kernels.shape[0] == 0
        assert np.all(np.isneginf(res.scores))
