"""Comparators between the HIP path's results and the oracle's (test infrastructure).

Parity rules:
  kernels     bit-exact
  scores      identical -inf pattern on reachable blocks; finite entries within
              2^-12 * scale * sum_h sum_d |q_h,d * kernel_d| of the block's largest kernel term
              (float32 accumulation over G*d <= 2048 terms plus the two-part bf16 query)
  indices     equal sets except swaps between blocks whose oracle scores differ by less than
              1e-3 relative; forced blocks always present; sizes equal
  attention   |O - O_oracle(on the HIP path's own indices)| <= 2e-2 (bf16) / 1e-4 (f32)
              elementwise, and for bf16 outputs of magnitude >= 4 one bf16 unit in the last
              place of the oracle's value (2^-5 there: the output format cannot hold such a
              value closer than half of it, and the probabilities enter the P V product as
              bf16 MFMA operands); |lse - lse_oracle| <= 1e-3 (bf16) / 1e-5 (f32)
  gradients   |g - g_oracle| <= 2^-7 * m elementwise, m the magnitude of the same sum taken
              over absolute values (backward_magnitudes); see there for the error budget
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from oracle import infllm2_oracle as orc

OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}
TIE_BAND = 1e-3
SCORE_REL = 2.0 ** -12


def score_bound(q_rows: np.ndarray, kernels: np.ndarray, positions: np.ndarray, p,
                num_blocks: int) -> np.ndarray:
    """scale * max over the block's kernels of sum_h sum_d |q_h,d * kernel_c,d|."""
    G = p.group
    C = kernels.shape[0]
    n = len(positions)
    out = np.zeros((n, p.num_kv_heads, num_blocks))
    for g in range(p.num_kv_heads):
        aq = np.abs(q_rows[:, g * G:(g + 1) * G, :].astype(np.float64)).sum(axis=1)  # [n, d]
        t = p.scale * aq @ np.abs(kernels[:, g, :].astype(np.float64)).T             # [n, C]
        for b in range(num_blocks):
            cs = orc.kernels_of_block(b, p.block_size, p.kernel_size, p.kernel_stride, C)
            if len(cs):
                out[:, g, b] = t[:, cs.start:cs.stop].max(axis=1)
    return out


def check_scores(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, positions, p):
    """Returns the largest |diff| / bound seen; raises AssertionError on a violation."""
    own = np.asarray(positions) // p.block_size
    worst = 0.0
    for r in range(len(own)):
        nb = int(own[r]) + 1
        g_s, r_s, bd = gpu[r, :, :nb], ref[r, :, :nb], bound[r, :, :nb]
        assert np.array_equal(np.isneginf(g_s), np.isneginf(r_s)), f"-inf pattern differs, row {r}"
        fin = np.isfinite(r_s)
        assert np.all(np.isfinite(g_s[fin])), f"non-finite GPU score, row {r}"
        d = np.abs(g_s[fin].astype(np.float64) - r_s[fin])
        lim = SCORE_REL * bd[fin] + 1e-30
        if d.size:
            worst = max(worst, float((d / lim).max()))
        assert np.all(d <= lim), f"score error beyond bound, row {r}: {(d / lim).max()}"
    return worst


@dataclass
class IndexReport:
    rows: int
    exact: int
    band: int


def check_indices(gpu_idx: np.ndarray, ref_idx: np.ndarray, ref_scores: np.ndarray,
                  positions, p) -> IndexReport:
    exact = band = 0
    n = len(positions)
    for r in range(n):
        pos = int(positions[r])
        F = set(orc.forced_blocks(pos, p).tolist())
        for g in range(p.num_kv_heads):
            a, o = gpu_idx[r, g], ref_idx[r, g]
            A = set(int(x) for x in a if x >= 0)
            O = set(int(x) for x in o if x >= 0)
            real = a[a >= 0]
            assert np.all(np.diff(real) > 0) and np.all(a[len(real):] == -1), f"bad layout row {r}"
            assert len(A) == len(O), f"row {r} g {g}: {len(A)} vs {len(O)} blocks"
            assert (F & set(range(pos // p.block_size + 1))) <= A, f"row {r}: forced block missing"
            if A == O:
                exact += 1
                continue
            S = ref_scores[r, g]
            for x in A - O:
                for y in O - A:
                    m = max(abs(S[x]), abs(S[y]))
                    assert abs(S[x] - S[y]) < TIE_BAND * m, (
                        f"row {r} g {g}: chose {x} ({S[x]}) over {y} ({S[y]})")
            band += 1
    return IndexReport(n * p.num_kv_heads, exact, band)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Unit in the last place of bfloat16 (8 significant bits) at magnitude |x|."""
    e = np.floor(np.log2(np.maximum(np.abs(x), np.finfo(np.float64).tiny)))
    return np.exp2(e - 7)


def out_tolerance(ref_out: np.ndarray, dtype: str) -> np.ndarray:
    """Elementwise output tolerance (see the module docstring)."""
    if dtype == "bf16":
        return np.maximum(OUT_TOL[dtype], bf16_ulp(ref_out))
    return np.full(ref_out.shape, OUT_TOL[dtype])


def check_attention(out: np.ndarray, lse: np.ndarray, ref_out: np.ndarray, ref_lse: np.ndarray,
                    dtype: str):
    d = np.abs(out.astype(np.float64) - ref_out)
    err = float(d.max()) if out.size else 0.0
    lerr = float(np.abs(lse.astype(np.float64) - ref_lse).max()) if lse.size else 0.0
    if out.size:
        tol = out_tolerance(ref_out, dtype)
        i = np.unravel_index(np.argmax(d - tol), d.shape)
        assert d[i] <= tol[i], (f"output error {d[i]} > {tol[i]} at {i} (oracle {ref_out[i]}, "
                                f"max-abs error {err})")
    assert lerr <= LSE_TOL[dtype], f"lse max-abs error {lerr} > {LSE_TOL[dtype]}"
    return err, lerr


BWD_REL = 2.0 ** -7


def backward_magnitudes(q_rows, positions, keys, values, idx, dout, p):
    """Elementwise error scales of the bf16 backward, from the oracle's own quantities.

    The HIP backward rounds dS (and P, for dV) to bf16 before its matrix products (relative
    2^-9 each) and forms delta = dO . O from the forward's output, whose error is at most
    2^-9 (|O_d| + sum_j P_j |v_j,d|) (bf16 P in the forward's P V product, then the bf16
    store).  With, per (row, head),
        A   = sum_d |dO_d| (|O_d| + sum_j P_j |v_j,d|)
        E_j = |dS_j| + P_j (A + sum_d |dO_d| |v_j,d|)
    the error of dS_j before rounding is below 2^-9 P_j A (delta) plus float32 terms (P from
    the stored lse, dP summed in float32: about 2^-20 E_j), and its rounding adds 2^-9 E_j:
    2^-8 E_j in all.  The budget 2^-7 leaves a factor 2 over that worst case, for
        m_dQ  = scale sum_j E_j |k_j|,   m_dK_j = scale sum E_j |q|,   m_dV_j = sum P_j |dO|."""
    n, Hq, d = q_rows.shape
    G = p.group
    kv_len = keys.shape[0]
    mq = np.zeros((n, Hq, d))
    mk = np.zeros((kv_len, p.num_kv_heads, d))
    mv = np.zeros((kv_len, p.num_kv_heads, d))
    for r in range(n):
        pos = int(positions[r])
        for g in range(p.num_kv_heads):
            J = orc.attended_keys(idx[r, g], pos, kv_len, p.block_size)
            kg = keys[J, g, :].astype(np.float64)
            vg = values[J, g, :].astype(np.float64)
            qh = q_rows[r, g * G:(g + 1) * G, :].astype(np.float64)
            do = dout[r, g * G:(g + 1) * G, :].astype(np.float64)
            z = p.scale * (qh @ kg.T)
            e = np.exp(z - z.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)                        # [G, |J|]
            O = P @ vg
            dS = P * (do @ vg.T - (do * O).sum(axis=1, keepdims=True))
            A = (np.abs(do) * (np.abs(O) + P @ np.abs(vg))).sum(axis=1, keepdims=True)
            E = np.abs(dS) + P * (A + np.abs(do) @ np.abs(vg).T)         # [G, |J|]
            mq[r, g * G:(g + 1) * G, :] = p.scale * (E @ np.abs(kg))
            mk[J, g, :] += p.scale * (E.T @ np.abs(qh))                  # J has no repeats
            mv[J, g, :] += P.T @ np.abs(do)
    return mq, mk, mv


def check_gradient(name: str, gpu: np.ndarray, ref: np.ndarray, mag: np.ndarray) -> float:
    """Returns max |gpu - ref| / (BWD_REL * mag); raises on a violation or a non-finite value."""
    gpu = np.asarray(gpu, dtype=np.float64)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    d = np.abs(gpu - ref)
    lim = BWD_REL * mag + 1e-30
    ratio = float((d / lim).max()) if d.size else 0.0
    bad = d > lim
    if bad.any():
        i = np.unravel_index(int(np.argmax(d / lim)), d.shape)
        raise AssertionError(f"{name}: error beyond bound at {i}: {gpu[i]} vs {ref[i]} "
                             f"(bound {lim[i]}, {int(bad.sum())} elements)")
    return ratio


def softmax_score_rel_bound(q_rows, kernels, positions, p) -> np.ndarray:
    """Relative error bound [n, Hkv] of score-mode-1 block scores computed in float32.

    Each probability is exp2(x - lse2) with x = log2(e) scale q . kernel: the float32 dot
    product of exact bf16 products errs by at most d 2^-24 sum |q k| (a = max of scale sum |q k|
    over the row's heads and visible kernels), lse2 adds the float32 sum of up to n_vis terms
    (n_vis 2^-24 relative) and that x's error again through the max; exp2, log2 and the group sum
    add a few float32 ulps.  So |dP / P| <= ln2 (2 log2(e) d 2^-24 a + n_vis 2^-24) + 2^-21, and
    the block score (a max of sums of such P) has the same relative bound."""
    positions = np.asarray(positions)
    n, Hq, d = q_rows.shape
    G = p.group
    C = kernels.shape[0]
    out = np.zeros((n, p.num_kv_heads))
    for r in range(n):
        nvis = 0 if positions[r] < p.kernel_size - 1 else min(
            C, (int(positions[r]) - p.kernel_size + 1) // p.kernel_stride + 1)
        if nvis == 0:
            continue
        for g in range(p.num_kv_heads):
            aq = np.abs(q_rows[r, g * G:(g + 1) * G, :].astype(np.float64))
            a = p.scale * (aq @ np.abs(kernels[:nvis, g, :].astype(np.float64)).T).max()
            out[r, g] = (math.log(2) * (2 * 1.4426950408889634 * d * 2.0 ** -24 * a
                                        + nvis * 2.0 ** -24) + 2.0 ** -21)
    return out


def check_softmax_scores(gpu, ref, rel, positions, p) -> float:
    """Identical -inf pattern on reachable blocks; |gpu - ref| <= rel[row, g] * ref elsewhere.
    Returns the largest error / bound."""
    own = np.asarray(positions) // p.block_size
    worst = 0.0
    for r in range(len(own)):
        nb = int(own[r]) + 1
        g_s, r_s = gpu[r, :, :nb].astype(np.float64), ref[r, :, :nb]
        assert np.array_equal(np.isneginf(g_s), np.isneginf(r_s)), f"-inf pattern differs, row {r}"
        fin = np.isfinite(r_s)
        lim = np.broadcast_to(rel[r][:, None], r_s.shape)[fin] * np.abs(r_s[fin]) + 1e-30
        d = np.abs(g_s[fin] - r_s[fin])
        if d.size:
            worst = max(worst, float((d / lim).max()))
        assert np.all(d <= lim), f"score error beyond bound, row {r}: {(d / lim).max()}"
    return worst
