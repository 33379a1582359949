"""Brute-force second statement of the oracle, in pure Python.

TEST INFRASTRUCTURE ONLY (see oracle/infllm2_oracle.py).  This file re-derives every step
from the same description with scalar loops, exact sums (math.fsum / fractions) and
explicit token sets, sharing no code with either the numpy oracle or the HIP library.  It
is meant for tiny inputs; the tests compare it with the numpy oracle.

Steps (MiniCPM4 paper summary, sections 2.1.1-2.1.2): blocks of the KV cache; semantic
kernels as window means of keys; per-token relevance of each block through the kernels,
summed over a GQA group's heads; group-shared top-k with forced initial/local blocks;
softmax attention over the chosen blocks' tokens.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction
from typing import List


def bf16_nearest(x: float) -> float:
    """Nearest bfloat16 value to x (ties to even), from exact rational arithmetic."""
    if x == 0.0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = Fraction(abs(x))
    e = 0
    while a >= 2:
        a /= 2; e += 1
    while a < 1:
        a *= 2; e -= 1
    # a in [1, 2): 8 significant bits -> multiples of 1/128
    scaled = a * 128
    lo = math.floor(scaled)
    frac = scaled - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * float(Fraction(lo, 128) * Fraction(2) ** e)


def f32_nearest(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def to_storage(x: float, dtype: str) -> float:
    return bf16_nearest(x) if dtype == "bf16" else f32_nearest(x)


def kernels(keys, w: int, s: int, dtype: str):
    """keys: nested list [L][Hkv][d] -> [C][Hkv][d] window means rounded to storage."""
    L = len(keys)
    out = []
    c = 0
    while s * c + w <= L:
        row = []
        for g in range(len(keys[0])):
            row.append([to_storage(float(sum((Fraction(keys[s * c + t][g][e]) for t in range(w)),
                                             Fraction(0)) / w), dtype)
                        for e in range(len(keys[0][0]))])
        out.append(row)
        c += 1
    return out


def block_score(q_i, kern, g: int, G: int, pos: int, b: int, B: int, w: int, s: int,
                scale: float) -> float:
    """Max over kernels whose token window meets block b's tokens and ends at or before pos of
    scale * sum_h q_h . kernel; -inf if there is none."""
    block_tokens = set(range(B * b, B * (b + 1)))
    best = -math.inf
    for c in range(len(kern)):
        window = set(range(s * c, s * c + w))
        if not (window & block_tokens):
            continue
        if max(window) > pos:
            continue
        terms = [q_i[h][e] * kern[c][g][e] for h in range(g * G, (g + 1) * G)
                 for e in range(len(kern[c][g]))]
        best = max(best, scale * math.fsum(terms))
    return best


def block_score_softmax(q_i, kern, g: int, G: int, pos: int, b: int, B: int, w: int, s: int,
                        scale: float) -> float:
    """Score mode 1: each head's logits scale * q_h . kernel over the kernels whose window ends
    at or before pos are turned into probabilities (exp over the fsum of exps); the block's score
    is the max, over those kernels whose window meets block b, of the sum of the group's
    probabilities; -inf if there is none."""
    seen = [c for c in range(len(kern)) if s * c + w - 1 <= pos]
    block_tokens = set(range(B * b, B * (b + 1)))
    meets = [c for c in seen if set(range(s * c, s * c + w)) & block_tokens]
    if not meets:
        return -math.inf
    total = {c: 0.0 for c in meets}
    for h in range(g * G, (g + 1) * G):
        logits = {c: scale * math.fsum(q_i[h][e] * kern[c][g][e] for e in range(len(kern[c][g])))
                  for c in seen}
        top = max(logits.values())
        den = math.fsum(math.exp(z - top) for z in logits.values())
        for c in meets:
            total[c] += math.exp(logits[c] - top) / den
    return max(total.values())


def choose(scores: List[float], pos: int, B: int, k: int, n_init: int, n_local: int) -> List[int]:
    own = pos // B
    cand = list(range(own + 1))
    if len(cand) <= k:
        sel = cand
    else:
        forced = {b for b in cand if b < n_init or b > own - n_local}
        others = sorted((b for b in cand if b not in forced), key=lambda b: (-scores[b], b))
        sel = sorted(list(forced) + others[:k - len(forced)])
    return sel + [-1] * (k - len(sel))


def run(q, keys, values, Hkv: int, B: int, w: int, s: int, k: int, n_init: int, n_local: int,
        dtype: str, scale: float, rows=None, score_mode: int = 0):
    """q: [T][Hq][d] with query t at position t; keys/values: [T][Hkv][d].
    Returns (kernels, scores[t][g][b], idx[t][g], out[t][h][d], lse[t][h])."""
    T = len(keys)
    Hq = len(q[0]); G = Hq // Hkv; d = len(q[0][0])
    kern = kernels(keys, w, s, dtype)
    NB = -(-T // B)
    rows = range(len(q)) if rows is None else rows
    S_all, I_all, O_all, L_all = [], [], [], []
    for t in rows:
        S_t, I_t = [], []
        O_t = [[0.0] * d for _ in range(Hq)]
        L_t = [0.0] * Hq
        for g in range(Hkv):
            score = block_score_softmax if score_mode == 1 else block_score
            sc = [score(q[t], kern, g, G, t, b, B, w, s, scale) if b <= t // B else -math.inf
                  for b in range(NB)]
            sel = choose(sc, t, B, k, n_init, n_local)
            S_t.append(sc); I_t.append(sel)
            toks = [j for b in sel if b >= 0 for j in range(B * b, min(B * (b + 1), T)) if j <= t]
            for h in range(g * G, (g + 1) * G):
                logits = [scale * math.fsum(q[t][h][e] * keys[j][g][e] for e in range(d))
                          for j in toks]
                mx = max(logits)
                ex = [math.exp(z - mx) for z in logits]
                den = math.fsum(ex)
                for e in range(d):
                    O_t[h][e] = math.fsum(ex[n] * values[j][g][e] for n, j in enumerate(toks)) / den
                L_t[h] = mx + math.log(den)
        S_all.append(S_t); I_all.append(I_t); O_all.append(O_t); L_all.append(L_t)
    return kern, S_all, I_all, O_all, L_all
