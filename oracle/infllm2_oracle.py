"""Plain CPU oracle of InfLLM v2 block-sparse attention (float64 numpy).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or execute this
module: only the tests, the package smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library; it reads the same seeded inputs (module `synth`).

What it computes, in the order the method's description gives it (MiniCPM4 paper summary,
section 2.1.1 "overall framework" and 2.1.2 "dynamic context block selection"; the arXiv
abstract for the prefill and decode use):

  1. the key/value cache is cut into fixed-size blocks, and every query token attends to a
     few whole blocks only (section 2.1.1);
  2. each block is represented through fine-grained "semantic kernels" built from the keys
     (section 2.1.2) -- here the mean of `kernel_size` consecutive keys taken every
     `kernel_stride` tokens, rounded to the storage dtype;                  -> compress_kernels
  3. a relevance score between each query token and each block is computed from those
     kernels; the query heads of one GQA group share it (section 2.1.2) -- here the scaled dot
     product of every head of the group with each visible kernel, summed over the group's
     heads, then the maximum over the kernels that overlap the block;        -> block_scores
  4. the group's query heads share one set of highest-scoring blocks (section 2.1.2; the news
     article's "selects the relevant blocks per k" read as top-k), with the first
     `num_init_blocks` blocks and the `num_local_blocks` blocks ending at the query's own block
     always kept;                                                            -> select_blocks
  5. ordinary causal softmax attention over the tokens of the selected blocks only
     (section 2.1.3: each token attends only to its most relevant blocks), scale 1/sqrt(d)
     as in the skill page's textbook attention snippet.                      -> sparse_attention

  6. the gradients of that attention (the mechanism is trainable: model card, "Efficient Model
     Architecture"; arXiv abstract; paper summary section 2.1): with the selected blocks held
     fixed -- the selection is piecewise constant in Q and K, so its derivative is zero almost
     everywhere -- dQ, dK and dV of step 5 for an upstream gradient dO.     -> sparse_attention_backward
  3'. a second reading of step 3's relevance score (the other plain reading, selected by
     score_mode = 1): each head's scores are first normalised by a softmax over the kernels
     visible at the query's position, and the group sum is taken over those probabilities
     (section 2.1.2 names a relevance score without fixing its form).  -> kernel_scores_softmax
  7. sliding-window attention, the second attention workload the pages name (csdn summary,
     section 4.1.3: the speculative draft model uses it): causal softmax attention over the
     `window` most recent tokens, the query's own included.          -> window_attention

The pages give no formula, constant or worked example for steps 2-4.  Where they are silent
the oracle takes the plainest reading; every such reading is listed in the repository's
design notes and pinned by the tests in tests/test_oracle_*.py.  Functions are written for
clarity, not speed; large workloads are checked on sampled query rows.
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------------------
# storage rounding

def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of the storage format, ties to even.

    bf16 keeps 8 significant bits: write x = m * 2**e with m in [0.5, 1); the rounded value is
    round_half_even(m * 2**8) * 2**(e-8).  (Normal range only; inputs here are O(1).)
    f32 is IEEE single: numpy's cast rounds to nearest even.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0), e - 8)


def _significand_bits(dtype: str) -> int:
    return 24 if dtype == "f32" else 8


# ---------------------------------------------------------------------------------------
# step 2: semantic kernels

def num_kernels(length: int, kernel_size: int, kernel_stride: int) -> int:
    """Complete windows [s*c, s*c + w) inside a sequence of `length` tokens."""
    if length < kernel_size:
        return 0
    return (length - kernel_size) // kernel_stride + 1


def _storage_midpoint(x: float, dtype: str) -> bool:
    """Whether x lies exactly halfway between two neighbouring values of the storage format."""
    if x == 0.0 or not np.isfinite(x):
        return False
    m, e = np.frexp(x)
    t = m * 2.0 ** (_significand_bits(dtype) + 1)     # exact: a power-of-two scaling
    return float(t).is_integer() and int(t) % 2 == 1


def _toward(x: float, exact: Fraction, dtype: str) -> float:
    """x, the float64 nearest to `exact`, moved one float64 step toward `exact` when x is a
    storage midpoint that `exact` is not: rounding the result to the storage format then gives
    the rounding of `exact` itself, not of x (no double rounding)."""
    if _storage_midpoint(x, dtype) and Fraction(x) != exact:
        return float(np.nextafter(x, np.inf if exact > x else -np.inf))
    return x


def exact_window_means(keys: np.ndarray, kernel_size: int, kernel_stride: int,
                       c_lo: int, c_hi: int, dtype: str) -> np.ndarray:
    """Mean of keys[s*c : s*c+w] for c in [c_lo, c_hi), as the float64 nearest to the exact
    mean, except that a float64 landing exactly halfway between two storage values that the
    exact mean is not is moved one float64 step toward it (so that one rounding of the result
    to the storage format is the rounding of the exact mean).

    The window sum is taken with numpy in float64 and certified exact: every value is a
    multiple of 2**(e_min - p) (p = significand bits of the input format, e_min the smallest
    binary exponent in the window) and the sum of magnitudes is below 2**53 of that unit, so no
    partial sum can round.  Windows without the certificate are summed with Fractions.
    """
    w, s = kernel_size, kernel_stride
    rest = keys.shape[1:]
    n = c_hi - c_lo
    out = np.empty((max(n, 0),) + rest, dtype=np.float64)
    if n <= 0:
        return out
    p = _significand_bits(dtype)
    step = 512
    for a in range(c_lo, c_hi, step):
        b = min(c_hi, a + step)
        rows = s * np.arange(a, b)[:, None] + np.arange(w)[None, :]
        win = keys[rows]                                    # [nc, w, ...]
        sums = win.sum(axis=1)
        absum = np.abs(win).sum(axis=1)
        _, ex = np.frexp(np.where(win == 0.0, np.inf, win))
        ex = np.where(win == 0.0, 10_000, ex).min(axis=1)   # smallest exponent per window
        unit_ok = (absum == 0.0) | (np.log2(np.maximum(absum, 1e-300)) < 52 + ex - p)
        means = sums / w
        # a mean that lands on a storage midpoint: settle the side with the exact value (the
        # division by w may have rounded onto it)
        mant, _ = np.frexp(means)
        t = mant * 2.0 ** (_significand_bits(dtype) + 1)
        on_mid = unit_ok & (means != 0.0) & (t == np.floor(t)) & (np.mod(t, 2.0) == 1.0)
        for idx in np.argwhere(on_mid):
            key = tuple(int(x) for x in idx)
            means[key] = _toward(float(means[key]), Fraction(float(sums[key])) / w, dtype)
        if not np.all(unit_ok):
            bad = np.argwhere(~unit_ok)
            for idx in bad:
                c = int(idx[0]); rem = tuple(int(t) for t in idx[1:])
                vals = [Fraction(float(win[(c,) + (t,) + rem])) for t in range(w)]
                exact = sum(vals, Fraction(0)) / w
                means[(c,) + rem] = _toward(float(exact), exact, dtype)
        out[a - c_lo:b - c_lo] = means
    return out


def compress_kernels(keys: np.ndarray, kernel_size: int, kernel_stride: int, dtype: str,
                     c_lo: int = 0, c_hi: Optional[int] = None) -> np.ndarray:
    """Semantic kernels of one sequence's keys [L, Hkv, d] -> [c_hi - c_lo, Hkv, d].

    Kernel c is the mean of the keys of tokens s*c .. s*c+w-1, stored in the key dtype
    (rounded to nearest even).  Only complete windows exist.
    """
    L = keys.shape[0]
    C = num_kernels(L, kernel_size, kernel_stride)
    if c_hi is None:
        c_hi = C
    c_hi = min(c_hi, C)
    mean = exact_window_means(np.asarray(keys, np.float64), kernel_size, kernel_stride,
                              c_lo, c_hi, dtype)
    return round_to_storage(mean, dtype)


def new_kernel_range(prev_len: int, new_len: int, kernel_size: int, kernel_stride: int):
    """Kernels that become complete when a sequence grows from prev_len to new_len tokens:
    those c with prev_len < s*c + w <= new_len."""
    return (num_kernels(prev_len, kernel_size, kernel_stride),
            num_kernels(new_len, kernel_size, kernel_stride))


# ---------------------------------------------------------------------------------------
# step 3: query-block relevance

def kernel_visible(c: np.ndarray, pos: np.ndarray, kernel_size: int, kernel_stride: int):
    """A kernel may score a query only once its last token is at or before the query."""
    return kernel_stride * c + kernel_size - 1 <= pos


def kernels_of_block(b: int, block_size: int, kernel_size: int, kernel_stride: int, C: int):
    """Kernels whose window [s*c, s*c+w) overlaps block b's tokens [B*b, B*(b+1))."""
    B, w, s = block_size, kernel_size, kernel_stride
    lo = max(0, -((-(B * b - w + 1)) // s))     # smallest c with s*c + w > B*b
    hi = min(C, -((-(B * (b + 1))) // s))       # one past the largest c with s*c < B*(b+1)
    return range(lo, hi)


def kernel_scores(q_rows: np.ndarray, kernels: np.ndarray, num_kv_heads: int,
                  scale: float) -> np.ndarray:
    """u[n, g, c] = scale * sum over the heads h of group g of q[n, h] . kernel[c, g].

    Written literally: one dot product per head, then the sum over the group's heads.
    """
    n, Hq, d = q_rows.shape
    G = Hq // num_kv_heads
    C = kernels.shape[0]
    u = np.zeros((n, num_kv_heads, C), dtype=np.float64)
    for g in range(num_kv_heads):
        kg = kernels[:, g, :].astype(np.float64)                  # [C, d]
        for h in range(g * G, (g + 1) * G):
            u[:, g, :] += scale * (q_rows[:, h, :].astype(np.float64) @ kg.T)
    return u


def kernel_scores_softmax(q_rows: np.ndarray, positions: np.ndarray, kernels: np.ndarray,
                          p) -> np.ndarray:
    """Score mode 1: u[n, g, c] = sum over the heads h of group g of P_h[c], where P_h is the
    softmax, over the kernels visible at the query's position, of scale * q[n, h] . kernel[c, g]
    (0 for kernels not visible; a row that sees no kernel has u = 0 everywhere)."""
    n, Hq, d = q_rows.shape
    G = Hq // p.num_kv_heads
    C = kernels.shape[0]
    vis = kernel_visible(np.arange(C)[None, :], np.asarray(positions)[:, None], p.kernel_size,
                         p.kernel_stride)                                  # [n, C]
    u = np.zeros((n, p.num_kv_heads, C), dtype=np.float64)
    if C == 0:                     # shorter than one window: no kernel, every score is -inf
        return u
    for g in range(p.num_kv_heads):
        kg = kernels[:, g, :].astype(np.float64)
        for h in range(g * G, (g + 1) * G):
            z = p.scale * (q_rows[:, h, :].astype(np.float64) @ kg.T)        # [n, C]
            z = np.where(vis, z, NEG_INF)
            m = z.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(vis, np.exp(z - m), 0.0)
            den = e.sum(axis=1, keepdims=True)
            u[:, g, :] += np.divide(e, den, out=np.zeros_like(e), where=den > 0)
    return u


def block_scores(q_rows: np.ndarray, positions: np.ndarray, kernels: np.ndarray,
                 p, num_blocks: int) -> np.ndarray:
    """S[n, g, b] = max of u[n, g, c] over the kernels c that overlap block b and are visible
    at the query's position; -inf where no such kernel exists or b lies after the query's
    own block.  u is kernel_scores (score_mode 0) or kernel_scores_softmax (score_mode 1)."""
    positions = np.asarray(positions, dtype=np.int64)
    C = kernels.shape[0]
    if getattr(p, "score_mode", 0) == 1:
        u = kernel_scores_softmax(q_rows, positions, kernels, p)
    else:
        u = kernel_scores(q_rows, kernels, p.num_kv_heads, p.scale)
    vis = kernel_visible(np.arange(C)[None, :], positions[:, None], p.kernel_size, p.kernel_stride)
    u = np.where(vis[:, None, :], u, NEG_INF)
    S = np.full((len(positions), p.num_kv_heads, num_blocks), NEG_INF)
    for b in range(num_blocks):
        cs = kernels_of_block(b, p.block_size, p.kernel_size, p.kernel_stride, C)
        if len(cs):
            S[:, :, b] = u[:, :, cs.start:cs.stop].max(axis=2)
    own = positions // p.block_size
    after = np.arange(num_blocks)[None, :] > own[:, None]          # [n, NB]
    S[np.broadcast_to(after[:, None, :], S.shape)] = NEG_INF
    return S


# ---------------------------------------------------------------------------------------
# step 4: group-shared top-k with forced blocks

def forced_blocks(pos: int, p) -> np.ndarray:
    """Initial blocks 0..n_init-1 and the n_local blocks ending at the query's own block."""
    own = pos // p.block_size
    init = set(range(min(p.num_init_blocks, own + 1)))
    local = set(range(max(0, own - p.num_local_blocks + 1), own + 1))
    return np.array(sorted(init | local), dtype=np.int64)


def select_blocks(scores_row: np.ndarray, pos: int, p) -> np.ndarray:
    """Blocks one (query, KV head) attends to: ascending, padded with -1 to topk.

    All causally reachable blocks when there are at most topk of them; otherwise the forced
    blocks plus the best remaining ones by (score descending, block index ascending).
    """
    own = pos // p.block_size
    eligible = np.arange(own + 1)
    out = np.full(p.topk, -1, dtype=np.int32)
    if len(eligible) <= p.topk:
        out[:len(eligible)] = eligible
        return out
    forced = forced_blocks(pos, p)
    rest = np.setdiff1d(eligible, forced)
    sc = np.asarray(scores_row, dtype=np.float64)[rest]
    order = np.lexsort((rest, -sc))             # primary: -score, secondary: index
    chosen = rest[order[:p.topk - len(forced)]]
    sel = np.sort(np.concatenate([forced, chosen]))
    out[:len(sel)] = sel
    return out


def select_all(S: np.ndarray, positions: np.ndarray, p) -> np.ndarray:
    n = len(positions)
    idx = np.empty((n, p.num_kv_heads, p.topk), dtype=np.int32)
    for r in range(n):
        for g in range(p.num_kv_heads):
            idx[r, g] = select_blocks(S[r, g], int(positions[r]), p)
    return idx


# ---------------------------------------------------------------------------------------
# step 5: attention over the selected blocks

def attended_keys(sel: np.ndarray, pos: int, kv_len: int, block_size: int) -> np.ndarray:
    """Token positions of the selected blocks that are at or before the query."""
    toks = [np.arange(b * block_size, min((b + 1) * block_size, kv_len)) for b in sel if b >= 0]
    j = np.concatenate(toks) if toks else np.zeros(0, np.int64)
    return j[j <= pos]


def sparse_attention(q_rows: np.ndarray, positions: np.ndarray, keys: np.ndarray,
                     values: np.ndarray, idx: np.ndarray, p):
    """O[n, h] = softmax_j(scale * q[n,h] . k[j,g]) v[j,g] over the selected blocks' tokens,
    and lse[n, h] = log sum_j exp(scale * q . k_j) (natural log)."""
    n, Hq, d = q_rows.shape
    G = p.group
    kv_len = keys.shape[0]
    O = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    for r in range(n):
        pos = int(positions[r])
        for g in range(p.num_kv_heads):
            J = attended_keys(idx[r, g], pos, kv_len, p.block_size)
            qh = q_rows[r, g * G:(g + 1) * G, :].astype(np.float64)      # [G, d]
            z = p.scale * (qh @ keys[J, g, :].astype(np.float64).T)      # [G, |J|]
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            den = e.sum(axis=1, keepdims=True)
            O[r, g * G:(g + 1) * G, :] = (e / den) @ values[J, g, :].astype(np.float64)
            lse[r, g * G:(g + 1) * G] = (m + np.log(den))[:, 0]
    return O, lse


def sparse_attention_backward(q_rows: np.ndarray, positions: np.ndarray, keys: np.ndarray,
                              values: np.ndarray, idx: np.ndarray, dout: np.ndarray, p):
    """Gradients of sparse_attention for the upstream gradient dout [n, Hq, d], the block
    selection idx held fixed.  For each query row and head, with z_j = scale q . k_j over the
    attended tokens j, P = softmax(z), O = sum_j P_j v_j:
        dV_j += P_j dO,   dP_j = dO . v_j,   dz_j = P_j (dP_j - dO . O),
        dQ = scale sum_j dz_j k_j,   dK_j += scale dz_j q.
    Returns dQ [n, Hq, d] and dK, dV [kv_len, Hkv, d] (zero for tokens no row attends to)."""
    n, Hq, d = q_rows.shape
    G = p.group
    kv_len = keys.shape[0]
    dQ = np.zeros((n, Hq, d), dtype=np.float64)
    dK = np.zeros((kv_len, p.num_kv_heads, d), dtype=np.float64)
    dV = np.zeros((kv_len, p.num_kv_heads, d), dtype=np.float64)
    for r in range(n):
        pos = int(positions[r])
        for g in range(p.num_kv_heads):
            J = attended_keys(idx[r, g], pos, kv_len, p.block_size)
            kg = keys[J, g, :].astype(np.float64)                       # [|J|, d]
            vg = values[J, g, :].astype(np.float64)
            qh = q_rows[r, g * G:(g + 1) * G, :].astype(np.float64)     # [G, d]
            do = dout[r, g * G:(g + 1) * G, :].astype(np.float64)
            z = p.scale * (qh @ kg.T)                                   # [G, |J|]
            e = np.exp(z - z.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            O = P @ vg
            dP = do @ vg.T
            dz = P * (dP - (do * O).sum(axis=1, keepdims=True))
            dQ[r, g * G:(g + 1) * G, :] = p.scale * (dz @ kg)
            np.add.at(dK[:, g, :], J, p.scale * (dz.T @ qh))
            np.add.at(dV[:, g, :], J, P.T @ do)
    return dQ, dK, dV


def window_attention(q_rows: np.ndarray, positions: np.ndarray, keys: np.ndarray,
                     values: np.ndarray, window: int, p):
    """O[n, h] = softmax_j(scale * q[n,h] . k[j,g]) v[j,g] over the tokens pos - window < j <= pos
    (the last `window` tokens up to and including the query), and lse[n, h] (natural log)."""
    n, Hq, d = q_rows.shape
    G = p.group
    O = np.zeros((n, Hq, d), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    for r in range(n):
        pos = int(positions[r])
        J = np.arange(max(0, pos - window + 1), pos + 1)
        for g in range(p.num_kv_heads):
            qh = q_rows[r, g * G:(g + 1) * G, :].astype(np.float64)
            z = p.scale * (qh @ keys[J, g, :].astype(np.float64).T)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            den = e.sum(axis=1, keepdims=True)
            O[r, g * G:(g + 1) * G, :] = (e / den) @ values[J, g, :].astype(np.float64)
            lse[r, g * G:(g + 1) * G] = (m + np.log(den))[:, 0]
    return O, lse


# ---------------------------------------------------------------------------------------
# whole passes

@dataclass
class SeqResult:
    kernels: np.ndarray       # [C, Hkv, d]
    rows: np.ndarray          # query rows (within the sequence) evaluated
    positions: np.ndarray
    scores: np.ndarray        # [n, Hkv, NB]
    idx: np.ndarray           # [n, Hkv, topk]
    out: np.ndarray           # [n, Hq, d]
    lse: np.ndarray           # [n, Hq]


def num_blocks(length: int, block_size: int) -> int:
    return -(-length // block_size)


def run_sequence(q_seq: np.ndarray, k_seq: np.ndarray, v_seq: np.ndarray, p,
                 q_pos0: int = 0, rows: Optional[Sequence[int]] = None,
                 kernels: Optional[np.ndarray] = None, idx_override: Optional[np.ndarray] = None,
                 with_attention: bool = True) -> SeqResult:
    """One sequence: compress its keys, score and select blocks for the requested query rows
    (all by default), then attend.  `idx_override` replaces the selection (used to check the
    attention step on another implementation's block indices)."""
    L = k_seq.shape[0]
    if kernels is None:
        kernels = compress_kernels(k_seq, p.kernel_size, p.kernel_stride, p.dtype)
    rows = np.arange(q_seq.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    positions = q_pos0 + rows
    qr = np.asarray(q_seq[rows], dtype=np.float64)
    NB = num_blocks(L, p.block_size)
    S = block_scores(qr, positions, kernels, p, NB)
    idx = select_all(S, positions, p) if idx_override is None else idx_override
    if with_attention:
        O, lse = sparse_attention(qr, positions, k_seq, v_seq, idx, p)
    else:
        O = np.zeros(qr.shape); lse = np.zeros(qr.shape[:2])
    return SeqResult(kernels, rows, positions, S, idx, O, lse)


def attended_key_count(pos: int, p) -> int:
    """Closed form for the number of keys one query attends (any head): every reachable key
    while at most topk blocks are reachable; otherwise topk-1 full blocks plus the query's
    own partial block."""
    B = p.block_size
    own = pos // B
    if own + 1 <= p.topk:
        return pos + 1
    return (p.topk - 1) * B + (pos % B) + 1


def lse_merge(parts_m: np.ndarray, parts_l: np.ndarray, parts_o: np.ndarray):
    """Combine attention over disjoint key sets from per-part (max logit, sum of exp, normalised
    output): the standard log-sum-exp merge.  Returns (output, lse)."""
    m = parts_m.max(axis=0)
    wts = parts_l * np.exp(parts_m - m)
    den = wts.sum(axis=0)
    out = (wts[..., None] * parts_o).sum(axis=0) / den[..., None]
    return out, m + np.log(den)
