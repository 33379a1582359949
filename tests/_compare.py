"""Comparators between the HIP path's results and the oracle's (test infrastructure).

Parity rules:
  kernels     bit-exact
  scores      identical -inf pattern on reachable blocks; finite entries within
              2^-12 * scale * sum_h sum_d |q_h,d * kernel_d| of the block's largest kernel term
              (float32 accumulation over G*d <= 2048 terms plus the two-part bf16 query)
  indices     equal sets except swaps between blocks whose oracle scores differ by less than
              1e-3 relative; forced blocks always present; sizes equal
  attention   max |O - O_oracle(on the HIP path's own indices)| <= 2e-2 (bf16) / 1e-4 (f32);
              |lse - lse_oracle| <= 1e-3 (bf16) / 1e-5 (f32)
"""
from __future__ import annotations

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


def check_attention(out: np.ndarray, lse: np.ndarray, ref_out: np.ndarray, ref_lse: np.ndarray,
                    dtype: str):
    err = float(np.abs(out.astype(np.float64) - ref_out).max()) if out.size else 0.0
    lerr = float(np.abs(lse.astype(np.float64) - ref_lse).max()) if lse.size else 0.0
    assert err <= OUT_TOL[dtype], f"output max-abs error {err} > {OUT_TOL[dtype]}"
    assert lerr <= LSE_TOL[dtype], f"lse max-abs error {lerr} > {LSE_TOL[dtype]}"
    return err, lerr
