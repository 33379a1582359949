"""The top-k selection alone, on synthetic score rows written straight into the scores buffer:
rows that reach 100 to 4096 blocks (up to a 256K-token sequence), rows around the all-blocks limit,
and score distributions that stress the selection (heavy ties, a single value, both signs with
+-0, a wide exponent range, -inf entries).  The indices must equal the oracle's selection
exactly."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import synth
from oracle import infllm2_oracle as orc
from tests._gpu import host, log

import block_sparse_long_semantic_amd as lib

pytestmark = pytest.mark.gpu


def score_rows(kind: str, shape, rng) -> np.ndarray:
    if kind == "normal":
        s = rng.normal(0.0, 1.0, shape)
    elif kind == "ties":                       # a quarter-step grid: long runs of equal scores
        s = np.round(rng.normal(0.0, 1.0, shape) * 4.0) / 4.0
    elif kind == "one-value":
        s = np.full(shape, 1.5)
    elif kind == "signs":                      # few values, -0 and +0 among them
        s = rng.choice([-1.0, -0.0, 0.0, 2.0, 3.0], shape)
    elif kind == "wide":                       # exponents over 60 decades
        s = rng.normal(0.0, 1.0, shape) * 10.0 ** rng.integers(-30, 30, shape)
    elif kind == "neg-inf":
        s = rng.normal(0.0, 1.0, shape)
        s[rng.random(shape) < 0.3] = -np.inf
    else:
        raise ValueError(kind)
    return s.astype(np.float32)


@pytest.mark.parametrize("kind", ["normal", "ties", "one-value", "signs", "wide", "neg-inf"])
@pytest.mark.parametrize("kv_len", [6400, 16384, 65536, 131072, 262144])
def test_topk_on_given_scores(kind, kv_len):
    p = synth.config_params("prefill128k")
    H = p.num_kv_heads
    # sequence 0: its last 600 positions (100 to 4096 reachable blocks: 1 to 64 keys per lane of
    # the one-wave selection); sequence 1: positions whose reachable block counts run from 93 to
    # 99 across topk = 96
    seqs = lib.Seqs(q_start=[0, 600], q_len=[600, 400], q_pos0=[kv_len - 600, 5900],
                    kv_start=[0, kv_len], kv_len=[kv_len, 6300], kc_start=[0, 0])
    pos = np.concatenate([kv_len - 600 + np.arange(600), 5900 + np.arange(400)])
    nb = kv_len // p.block_size
    assert len(pos) * H > 1024                # the one-wave-per-row selection, not the wide one
    kinds = ["normal", "ties", "one-value", "signs", "wide", "neg-inf"]
    rng = np.random.default_rng(500 + 10 * kinds.index(kind) + kv_len // 6400)
    S = score_rows(kind, (len(pos), H, nb), rng)
    log(f"case topk on given scores {kind} kv_len={kv_len}")
    scores = torch.from_numpy(S).cuda()
    idx = torch.full((len(pos), H, p.topk), -7, dtype=torch.int32, device="cuda")
    lib.topk_select(p, seqs, scores, idx)
    got = host(idx)
    want = orc.select_all(S, pos, p)
    bad = np.nonzero(np.any(got != want, axis=2))
    assert bad[0].size == 0, f"{kind}: rows {bad[0][:5]} heads {bad[1][:5]} differ"


@pytest.mark.parametrize("kind", ["normal", "ties", "one-value", "signs", "wide", "neg-inf"])
@pytest.mark.parametrize("kv_len", [6400, 65536, 262144])
def test_topk_few_rows_on_given_scores(kind, kv_len):
    """At most 1024 (row, KV head) pairs: the workgroup-wide form of the selection."""
    p = synth.config_params("prefill128k")
    H = p.num_kv_heads
    seqs = lib.Seqs(q_start=[0, 200], q_len=[200, 100], q_pos0=[kv_len - 200, 5950],
                    kv_start=[0, kv_len], kv_len=[kv_len, 6050], kc_start=[0, 0])
    pos = np.concatenate([kv_len - 200 + np.arange(200), 5950 + np.arange(100)])
    nb = kv_len // p.block_size
    assert len(pos) * H <= 1024
    kinds = ["normal", "ties", "one-value", "signs", "wide", "neg-inf"]
    rng = np.random.default_rng(700 + 10 * kinds.index(kind) + kv_len // 6400)
    S = score_rows(kind, (len(pos), H, nb), rng)
    log(f"case topk few rows on given scores {kind} kv_len={kv_len}")
    scores = torch.from_numpy(S).cuda()
    idx = torch.full((len(pos), H, p.topk), -7, dtype=torch.int32, device="cuda")
    lib.topk_select(p, seqs, scores, idx)
    got = host(idx)
    want = orc.select_all(S, pos, p)
    bad = np.nonzero(np.any(got != want, axis=2))
    assert bad[0].size == 0, f"{kind}: rows {bad[0][:5]} heads {bad[1][:5]} differ"


@pytest.mark.parametrize("kind", ["normal", "ties", "one-value", "signs", "wide", "neg-inf"])
@pytest.mark.parametrize("topk", [256, 1024])
@pytest.mark.parametrize("form", ["many-rows", "few-rows"])
def test_topk_large_k_on_given_scores(kind, topk, form):
    """top-k beyond 128 non-forced blocks: the one-wave form then starts its first radix pass at
    the smallest key instead of the lanes' lower bound.  Rows at the end of a 128K sequence and
    rows whose reachable block counts cross topk; both forms of the selection."""
    p = replace(synth.config_params("prefill128k"), topk=topk)
    H = p.num_kv_heads
    kv_len = 131072
    lim = topk * p.block_size
    n0, n1 = (600, 400) if form == "many-rows" else (200, 100)
    seqs = lib.Seqs(q_start=[0, n0], q_len=[n0, n1], q_pos0=[kv_len - n0, lim - n1 // 2],
                    kv_start=[0, kv_len], kv_len=[kv_len, lim + n1], kc_start=[0, 0])
    pos = np.concatenate([kv_len - n0 + np.arange(n0), lim - n1 // 2 + np.arange(n1)])
    nb = kv_len // p.block_size
    assert (len(pos) * H > 1024) == (form == "many-rows")
    kinds = ["normal", "ties", "one-value", "signs", "wide", "neg-inf"]
    rng = np.random.default_rng(900 + 10 * kinds.index(kind) + topk // 256 + 5 * (form == "few-rows"))
    S = score_rows(kind, (len(pos), H, nb), rng)
    log(f"case topk k={topk} {form} {kind}")
    scores = torch.from_numpy(S).cuda()
    idx = torch.full((len(pos), H, p.topk), -7, dtype=torch.int32, device="cuda")
    lib.topk_select(p, seqs, scores, idx)
    got = host(idx)
    want = orc.select_all(S, pos, p)
    bad = np.nonzero(np.any(got != want, axis=2))
    assert bad[0].size == 0, f"{kind}: rows {bad[0][:5]} heads {bad[1][:5]} differ"
