"""Planted mistakes: each test swaps one oracle function for a plausibly wrong variant (a
dropped term, an off-by-one index, a transposed or wrong operand, a wrong sign, a wrong tie or
order rule) and checks that at least one pin of tests/test_oracle_pins.py then fails.  This is
what makes the pins worth trusting: a pin set that a mistake slips through pins nothing.

Everything runs on the CPU, on the oracle only.
"""
import numpy as np
import pytest

from oracle import infllm2_oracle as orc
from tests import test_oracle_pins as pins

ORIG = {name: getattr(orc, name) for name in (
    "round_to_storage", "exact_window_means", "compress_kernels", "kernel_visible",
    "kernels_of_block", "kernel_scores", "block_scores", "forced_blocks", "select_blocks",
    "attended_keys", "sparse_attention", "attended_key_count", "lse_merge",
    "sparse_attention_backward", "window_attention", "kernel_scores_softmax")}

# cheapest first; each entry is a pin from test_oracle_pins with its arguments bound
PINS = [
    ("rounding", pins.test_storage_rounding_matches_exact_rational_rounding),
    ("rounding_f32", pins.test_storage_rounding_matches_torch_on_f32_values),
    ("kernel_geometry", pins.test_kernels_of_block_by_token_sets),
    ("ties", pins.test_ties_go_to_lower_index),
    ("lse_merge", pins.test_lse_merge_identity),
    ("pooling_f32", lambda: pins.test_pooling_matches_numpy_window_mean("f32")),
    ("pooling_bf16", lambda: pins.test_pooling_matches_numpy_window_mean("bf16")),
    ("dense_reduction", pins.test_dense_reduction_equals_causal_attention),
    ("closed_form", pins.test_attended_key_counts_closed_form),
    ("golden_sparsity", pins.test_sparsity_matches_golden_and_page_claim),
    ("gather_vs_dense", pins.test_gather_equals_masked_dense),
    ("brute_force", lambda: pins.test_oracle_equals_brute_force(
        dict(p=pins.small_params(), L=150, seed=21))),
    ("brute_force_2", lambda: pins.test_oracle_equals_brute_force(
        dict(p=pins.small_params(dtype="f32", topk=3, num_local_blocks=2, num_init_blocks=0),
             L=133, seed=22))),
    ("brute_force_tiny", pins.test_oracle_equals_brute_force_on_tiny_rows),
    ("selection_invariants", pins.test_selection_invariants),
    ("incremental", pins.test_incremental_kernels_equal_full_compress),
    ("presum", pins.test_presum_identity),
    ("backward_fd", pins.test_backward_matches_finite_differences),
    ("backward_autograd", pins.test_backward_dense_reduction_equals_autograd),
    ("window_one", pins.test_window_of_one_returns_own_value),
    ("softmax_scipy", pins.test_softmax_scores_against_scipy_softmax),
    ("softmax_brute", lambda: pins.test_softmax_scores_equal_brute_force(
        dict(p=pins.small_params(score_mode=1), L=150, seed=91))),
    ("window_sdpa", lambda: pins.test_window_attention_matches_banded_sdpa(64)),
]


def first_failing_pin():
    for name, pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:           # an assertion, or the mutated code breaking a shape
            return name
    return None


# ----------------------------------------------------------------------------- mutations

def m_round_truncates(x, dtype):
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return ORIG["round_to_storage"](x, dtype)
    m, e = np.frexp(x)
    return np.ldexp(np.trunc(m * 256.0), e - 8)


def m_window_divisor(keys, w, s, c_lo, c_hi, dtype):
    return ORIG["exact_window_means"](keys, w, s, c_lo, c_hi, dtype) * w / (w - 1)


def m_window_shifted(keys, w, s, c_lo, c_hi, dtype):
    return ORIG["exact_window_means"](np.roll(keys, -1, axis=0), w, s, c_lo, c_hi, dtype)


def m_visible_leaks(c, pos, w, s):
    return s * c + w - 2 <= pos            # a kernel ending one token after the query counts


def m_visible_strict(c, pos, w, s):
    return s * c + w <= pos


def m_block_contained(b, B, w, s, C):
    lo = max(0, -((-(B * b)) // s))           # only kernels inside the block
    hi = min(C, (B * (b + 1) - w) // s + 1)
    return range(lo, max(lo, hi))


def m_scores_drop_head(q_rows, kernels, Hkv, scale):
    n, Hq, d = q_rows.shape
    G = Hq // Hkv
    u = np.zeros((n, Hkv, kernels.shape[0]))
    for g in range(Hkv):
        for h in range(g * G, (g + 1) * G - 1):
            u[:, g, :] += scale * (q_rows[:, h, :] @ kernels[:, g, :].T)
    return u


def m_scores_wrong_group(q_rows, kernels, Hkv, scale):
    u = ORIG["kernel_scores"](q_rows, kernels, Hkv, scale)
    return u[:, ::-1, :].copy() if Hkv > 1 else -u


def m_scores_no_scale(q_rows, kernels, Hkv, scale):
    return ORIG["kernel_scores"](q_rows, kernels, Hkv, 1.0)


def m_block_sum(q_rows, positions, kernels, p, NB):
    S = ORIG["block_scores"](q_rows, positions, kernels, p, NB)
    # replace the max-pool by the sum of the overlapping visible kernels
    C = kernels.shape[0]
    u = orc.kernel_scores(q_rows, kernels, p.num_kv_heads, p.scale)
    vis = orc.kernel_visible(np.arange(C)[None, :], np.asarray(positions)[:, None],
                             p.kernel_size, p.kernel_stride)
    u = np.where(vis[:, None, :], u, 0.0)
    for b in range(NB):
        cs = orc.kernels_of_block(b, p.block_size, p.kernel_size, p.kernel_stride, C)
        if len(cs):
            S[:, :, b] = np.where(np.isfinite(S[:, :, b]), u[:, :, cs.start:cs.stop].sum(2),
                                  S[:, :, b])
    return S


def m_forced_no_local(pos, p):
    own = pos // p.block_size
    return np.array(sorted(set(range(min(p.num_init_blocks, own + 1))) | {own}), dtype=np.int64)


def m_select_ties_high(scores_row, pos, p):
    own = pos // p.block_size
    out = np.full(p.topk, -1, dtype=np.int32)
    if own + 1 <= p.topk:
        out[:own + 1] = np.arange(own + 1)
        return out
    forced = orc.forced_blocks(pos, p)
    rest = np.setdiff1d(np.arange(own + 1), forced)
    sc = np.asarray(scores_row, dtype=np.float64)[rest]
    chosen = rest[np.lexsort((-rest, -sc))[:p.topk - len(forced)]]
    sel = np.sort(np.concatenate([forced, chosen]))
    out[:len(sel)] = sel
    return out


def m_select_descending(scores_row, pos, p):
    out = ORIG["select_blocks"](scores_row, pos, p)
    n = int((out >= 0).sum())
    out[:n] = out[:n][::-1]
    return out


def m_select_lowest(scores_row, pos, p):
    return ORIG["select_blocks"](-np.asarray(scores_row, dtype=np.float64), pos, p)


def m_keys_no_causal(sel, pos, kv_len, B):
    toks = [np.arange(b * B, min((b + 1) * B, kv_len)) for b in sel if b >= 0]
    return np.concatenate(toks) if toks else np.zeros(0, np.int64)


def _attention(q_rows, positions, keys, values, idx, p, variant):
    n, Hq, d = q_rows.shape
    G = p.group
    O = np.zeros((n, Hq, d))
    lse = np.zeros((n, Hq))
    for r in range(n):
        for g in range(p.num_kv_heads):
            J = orc.attended_keys(idx[r, g], int(positions[r]), keys.shape[0], p.block_size)
            qh = q_rows[r, g * G:(g + 1) * G, :]
            scale = 1.0 if variant == "no_scale" else p.scale
            z = scale * (qh @ keys[J, g, :].T)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z + m) if variant == "sign" else np.exp(z - m)
            den = e.sum(axis=1, keepdims=True)
            vals = keys if variant == "k_for_v" else values
            O[r, g * G:(g + 1) * G, :] = (e / den) @ vals[J, g, :]
            log = np.log2 if variant == "log2" else np.log
            lse[r, g * G:(g + 1) * G] = (m + log(den))[:, 0]
    return O, lse


def m_count_off_by_one(pos, p):
    B = p.block_size
    own = pos // B
    return pos + 1 if own + 1 <= p.topk else p.topk * B + (pos % B) + 1 - B + 1


def m_merge_no_exp(pm, pl, po):
    m = pm.max(axis=0)
    wts = pl * (pm - m + 1.0)
    den = wts.sum(axis=0)
    return (wts[..., None] * po).sum(axis=0) / den[..., None], m + np.log(den)


def _backward(q_rows, positions, keys, values, idx, dout, p, variant):
    dQ, dK, dV = ORIG["sparse_attention_backward"](q_rows, positions, keys, values, idx, dout, p)
    if variant == "no_delta":        # dz = P dP (the dO . O term dropped)
        n, Hq, d = q_rows.shape
        G = p.group
        dQ = np.zeros_like(dQ); dK = np.zeros_like(dK)
        for r in range(n):
            for g in range(p.num_kv_heads):
                J = orc.attended_keys(idx[r, g], int(positions[r]), keys.shape[0], p.block_size)
                qh = q_rows[r, g * G:(g + 1) * G, :]
                z = p.scale * (qh @ keys[J, g, :].T)
                P = np.exp(z - z.max(1, keepdims=True)); P /= P.sum(1, keepdims=True)
                dz = P * (dout[r, g * G:(g + 1) * G, :] @ values[J, g, :].T)
                dQ[r, g * G:(g + 1) * G, :] = p.scale * dz @ keys[J, g, :]
                np.add.at(dK[:, g, :], J, p.scale * dz.T @ qh)
    elif variant == "dk_unscaled":
        dK = dK / p.scale
    elif variant == "dv_transposed_heads":
        dV = dV[:, ::-1, :].copy() if p.num_kv_heads > 1 else -dV
    return dQ, dK, dV


def m_window(q_rows, positions, keys, values, window, p, variant):
    n, Hq, d = q_rows.shape
    G = p.group
    O = np.zeros((n, Hq, d))
    lse = np.zeros((n, Hq))
    for r in range(n):
        pos = int(positions[r])
        lo = max(0, pos - window) if variant == "one_more" else max(0, pos - window + 1)
        hi = pos if variant == "no_self" else pos + 1
        J = np.arange(lo, max(hi, lo + 1))
        for g in range(p.num_kv_heads):
            z = p.scale * (q_rows[r, g * G:(g + 1) * G, :] @ keys[J, g, :].T)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            den = e.sum(axis=1, keepdims=True)
            O[r, g * G:(g + 1) * G, :] = (e / den) @ values[J, g, :]
            lse[r, g * G:(g + 1) * G] = (m + np.log(den))[:, 0]
    return O, lse


def m_softmax(q_rows, positions, kernels, p, variant):
    n, Hq, d = q_rows.shape
    G = Hq // p.num_kv_heads
    C = kernels.shape[0]
    vis = orc.kernel_visible(np.arange(C)[None, :], np.asarray(positions)[:, None],
                             p.kernel_size, p.kernel_stride)
    if variant == "all_kernels":
        vis = np.ones_like(vis)
    u = np.zeros((n, p.num_kv_heads, C))
    for g in range(p.num_kv_heads):
        z = np.stack([p.scale * (q_rows[:, h, :] @ kernels[:, g, :].T)
                      for h in range(g * G, (g + 1) * G)])                  # [G, n, C]
        z = np.where(vis[None], z, -np.inf)
        if variant == "group_softmax":                 # one softmax over heads and kernels
            m = z.max(axis=(0, 2), keepdims=True)
            e = np.where(vis[None], np.exp(z - np.where(np.isfinite(m), m, 0)), 0)
            den = e.sum(axis=(0, 2), keepdims=True)
            u[:, g, :] = (G * e / np.where(den > 0, den, 1)).sum(axis=0)
        else:
            m = z.max(axis=2, keepdims=True)
            e = np.where(vis[None], np.exp(z - np.where(np.isfinite(m), m, 0)), 0)
            den = e.sum(axis=2, keepdims=True)
            u[:, g, :] = (e / np.where(den > 0, den, 1)).sum(axis=0)
    return u


MUTATIONS = {
    "rounding truncates": ("round_to_storage", m_round_truncates),
    "window mean divides by w-1": ("exact_window_means", m_window_divisor),
    "window starts one token late": ("exact_window_means", m_window_shifted),
    "kernel visible one token early": ("kernel_visible", m_visible_leaks),
    "kernel visible one token late": ("kernel_visible", m_visible_strict),
    "block takes contained kernels only": ("kernels_of_block", m_block_contained),
    "group sum drops a head": ("kernel_scores", m_scores_drop_head),
    "query group paired with wrong KV head": ("kernel_scores", m_scores_wrong_group),
    "score scale dropped": ("kernel_scores", m_scores_no_scale),
    "block score sums instead of max": ("block_scores", m_block_sum),
    "local blocks not forced": ("forced_blocks", m_forced_no_local),
    "ties to the higher index": ("select_blocks", m_select_ties_high),
    "selection written descending": ("select_blocks", m_select_descending),
    "lowest scores selected": ("select_blocks", m_select_lowest),
    "causal mask inside own block dropped": ("attended_keys", m_keys_no_causal),
    "softmax max-shift with wrong sign": (
        "sparse_attention", lambda *a: _attention(*a, variant="sign")),
    "keys used as values": ("sparse_attention", lambda *a: _attention(*a, variant="k_for_v")),
    "attention scale dropped": ("sparse_attention", lambda *a: _attention(*a, variant="no_scale")),
    "lse in log2": ("sparse_attention", lambda *a: _attention(*a, variant="log2")),
    "closed-form count off by one": ("attended_key_count", m_count_off_by_one),
    "lse merge without exp": ("lse_merge", m_merge_no_exp),
    "backward drops the dO . O term": (
        "sparse_attention_backward", lambda *a: _backward(*a, variant="no_delta")),
    "backward dK without the scale": (
        "sparse_attention_backward", lambda *a: _backward(*a, variant="dk_unscaled")),
    "backward dV on the wrong KV head": (
        "sparse_attention_backward", lambda *a: _backward(*a, variant="dv_transposed_heads")),
    "softmax over invisible kernels too": (
        "kernel_scores_softmax", lambda *a: m_softmax(*a, variant="all_kernels")),
    "one softmax across the group's heads": (
        "kernel_scores_softmax", lambda *a: m_softmax(*a, variant="group_softmax")),
    "window one token too long": ("window_attention", lambda *a: m_window(*a, variant="one_more")),
    "window leaves out the query's own token": (
        "window_attention", lambda *a: m_window(*a, variant="no_self")),
}


def test_unmutated_oracle_passes_every_pin():
    assert first_failing_pin() is None


@pytest.mark.parametrize("label", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(label, monkeypatch):
    name, fn = MUTATIONS[label]
    monkeypatch.setattr(orc, name, fn)
    assert first_failing_pin() is not None, f"no pin catches: {label}"
