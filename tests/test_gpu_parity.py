"""Parity of the HIP path (through the C ABI) with the CPU oracle, on seeded inputs.

Small workloads are compared on every query row; the measured full-size workloads on sampled
rows (dense region, needle rows, the last rows, a stride).  Rules are in tests/_compare.py.
"""
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


def check_sequence(wl, res, b, rows=None, label=""):
    """Compare one sequence of a prefill run with the oracle on the given rows (all if None)."""
    p = wl.params
    sl_q, sl_k = wl.seq_slices(b)
    q_seq, k_seq, v_seq = wl.q[sl_q], wl.k[sl_k], wl.v[sl_k]
    if q_seq.shape[0] == 0:
        return
    kc0, _ = kc_starts(wl.kv_len, p)
    C = orc.num_kernels(k_seq.shape[0], p.kernel_size, p.kernel_stride)
    kern_ref = orc.compress_kernels(k_seq, p.kernel_size, p.kernel_stride, p.dtype)
    kern_gpu = res["kernels"][kc0[b]:kc0[b] + C]
    ndiff = int(np.sum(kern_gpu != kern_ref))
    assert ndiff == 0, f"{label}: {ndiff} kernel elements differ"
    rows = np.arange(q_seq.shape[0]) if rows is None else np.asarray(rows)
    q0 = int(wl.q_pos0[b])
    ref = orc.run_sequence(q_seq, k_seq, v_seq, p, q_pos0=q0, rows=rows, kernels=kern_ref,
                           with_attention=False)
    grow = int(wl.q_start[b]) + rows
    NB = ref.scores.shape[2]
    gs = res["scores"][grow][:, :, :NB]
    bound = cmp.score_bound(q_seq[rows].astype(np.float64), kern_ref, ref.positions, p, NB)
    worst = cmp.check_scores(gs, ref.scores, bound, ref.positions, p)
    # selection kernel alone: the oracle's selection applied to the GPU's own scores
    gidx = res["idx"][grow]
    own_sel = orc.select_all(gs.astype(np.float64), ref.positions, p)
    assert np.array_equal(gidx, own_sel), f"{label}: top-k differs on the GPU's own scores"
    rep = cmp.check_indices(gidx, ref.idx, ref.scores, ref.positions, p)
    # attention on the GPU's indices
    O, L = orc.sparse_attention(q_seq[rows].astype(np.float64), ref.positions, k_seq, v_seq,
                                gidx, p)
    err, lerr = cmp.check_attention(res["out"][grow], res["lse"][grow], O, L, p.dtype)
    log(f"{label} seq {b}: rows {len(rows)} score-ratio {worst:.3g} idx exact {rep.exact}/"
        f"{rep.rows} band {rep.band} out-err {err:.3g} lse-err {lerr:.3g}")


# ------------------------------------------------------------------------- small, all rows

def test_tiny_f32_all_rows():
    wl = synth.make("tiny")
    log("case tiny f32")
    res = run_prefill_stages(wl)
    check_sequence(wl, res, 0, label="tiny")


def test_tiny_dense_reduction():
    """topk >= number of blocks: the HIP output equals dense causal attention."""
    wl = synth.make("tiny")
    wl.params = replace(wl.params, topk=8)
    log("case tiny dense")
    res = run_prefill_stages(wl)
    q = torch.from_numpy(wl.q.astype(np.float64)).transpose(0, 1)
    k = torch.from_numpy(wl.k.astype(np.float64)).transpose(0, 1).repeat_interleave(2, 0)
    v = torch.from_numpy(wl.v.astype(np.float64)).transpose(0, 1).repeat_interleave(2, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    assert np.abs(res["out"] - ref.transpose(0, 1).numpy()).max() < 1e-4


@pytest.mark.parametrize("L", [3000, 1100])
def test_8b_shape_ragged_all_rows(L):
    """MiniCPM4-8B head layout, a length that is neither a multiple of 64 nor 16, needles."""
    p = synth.config_params("prefill32k")
    wl = synth.make_prefill("8b-ragged", p, [L], seed=31, needles_per_seq=2)
    log(f"case 8b ragged L={L}")
    res = run_prefill_stages(wl)
    check_sequence(wl, res, 0, label=f"8b L={L}")
    for nd in wl.needles:
        hit = np.any(res["idx"][nd.query_positions, nd.kv_head, :] == nd.block, axis=1)
        assert hit.all(), f"needle block {nd.block} missed"


def test_24_token_tiles_ragged_all_rows():
    """24-token tiles (3 tokens per wave) in packed sequences whose last tiles hold 17, 22, 17
    and 8 tokens, spanning 2, 2, 2 and 3 groups of 32 tiles: the launch schedule's levels 0 and 1
    hold every sequence, level 2 only the last; every row."""
    p = synth.config_params("prefill32k")
    wl = synth.make_prefill("tiles-24", p, [1001, 1030, 977, 2000], seed=35)
    log("case 24-token tiles, ragged")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label="24-token tiles")


def test_varlen_packed_small_all_rows():
    wl = synth.make("varlen", length_scale=1 / 16)
    log("case varlen 1/16")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label="varlen/16")


def test_edge_sequences():
    """Empty, single-token, shorter-than-a-window and one-block sequences packed together."""
    p = synth.config_params("prefill32k")
    wl = synth.make_prefill("edge", p, [0, 1, 20, 31, 32, 64, 65, 700], seed=33)
    log("case edge lengths")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label="edge")


@pytest.mark.parametrize("d", [64, 128])
def test_edge_sequences_group8(d):
    """Groups of 8 heads run 64-token (head_dim 64) or 32-token (128) tiles in which two tokens'
    heads share each matrix-core column group: sequences whose last tile is ragged at every
    parity (a lone token in its pair, a pair split by the sequence end) or full, packed
    together; every row."""
    p = replace(synth.config_params("varlen"), head_dim=d)
    wl = synth.make_prefill("edge-g8", p, [0, 1, 2, 17, 31, 32, 33, 47, 63, 64, 65, 127, 130, 700],
                            seed=34)
    log(f"case edge lengths, group 8, d {d}")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label=f"edge g8 d{d}")


def test_sixty_four_sequences_packed():
    """The largest sequence table (64 packed sequences) with seeded lengths from 0 to 1500,
    among them empty, single-token and shorter-than-a-window ones: every row of every sequence."""
    p = synth.config_params("prefill32k")
    rng = np.random.default_rng(48)
    lens = [int(x) for x in rng.integers(0, 1500, 64)]
    lens[:4] = [0, 1, 31, 64]
    wl = synth.make_prefill("sixty-four", p, lens, seed=48)
    log("case 64 packed sequences")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label="64 seqs")


def test_hundred_sequences_packed():
    """No cap on the sequence table: 100 packed sequences with seeded lengths from 0 to 1200
    (empty, single-token and shorter-than-a-window ones among them), every row of every
    sequence."""
    p = synth.config_params("prefill32k")
    rng = np.random.default_rng(52)
    lens = [int(x) for x in rng.integers(0, 1200, 100)]
    lens[:4] = [0, 1, 31, 64]
    wl = synth.make_prefill("hundred", p, lens, seed=52)
    log("case 100 packed sequences")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label="100 seqs")


def test_chunked_prefill_against_cache():
    """Queries for the last tokens only (q_pos0 > 0) attend to the whole cached sequence."""
    p = synth.config_params("prefill32k")
    full = synth.make_prefill("chunk", p, [2600], seed=34, needles_per_seq=1)
    q0 = 1900
    wl = synth.Workload("chunk", p, full.q[q0:], full.k, full.v, np.array([0]),
                        np.array([700], np.int32), np.array([q0], np.int32), np.array([0]),
                        np.array([2600], np.int32))
    log("case chunked prefill")
    res = run_prefill_stages(wl)
    check_sequence(wl, res, 0, label="chunk")


def test_prefill_tied_scores():
    """Every key equal, so every candidate block of a row scores the same (a single key value in
    the selection): besides the forced blocks the lowest block indices win."""
    p = synth.config_params("prefill32k")
    wl = synth.make_prefill("ties", p, [9000], seed=47)
    wl.k[:] = wl.k[:1]
    log("case prefill ties")
    res = run_prefill_stages(wl)
    rows = np.array(sorted(set(range(0, 9000, 97)) | set(range(8930, 9000))))
    check_sequence(wl, res, 0, rows=rows, label="ties")
    n_plain = p.topk - p.num_init_blocks - p.num_local_blocks
    for r in rows:
        own = int(r) // p.block_size
        if own + 1 <= p.topk:
            continue
        for h in range(p.num_kv_heads):
            chosen = res["idx"][r, h]
            assert np.array_equal(chosen[:p.num_init_blocks + n_plain],
                                  np.arange(p.num_init_blocks + n_plain))
            assert chosen[-2] == own - 1 and chosen[-1] == own


@pytest.mark.parametrize("name,lens", [("prefill32k", [20000, 13001, 77]),
                                       ("varlen", [16421, 9000, 30])])
def test_mfma_scores_ragged_tiles(name, lens):
    """Enough 64-row tiles for the matrix-core scoring path, with lengths that leave ragged last
    tiles (and a tiny sequence beside them); rows sampled across the tiles and every tail row."""
    p = synth.config_params(name)
    wl = synth.make_prefill("mfma-ragged", p, lens, seed=35, needles_per_seq=1)
    assert sum((L + 63) // 64 for L in lens) * p.num_kv_heads >= 512
    log(f"case mfma scores ragged {name} {lens}")
    res = run_prefill_stages(wl)
    for b, L in enumerate(lens):
        rows = sorted(set(range(0, L, 211)) | set(range(max(0, L - 70), L)))
        check_sequence(wl, res, b, rows=np.array(rows), label=f"mfma-ragged {name} seq {b}")


def test_compress_exactness_condition_wide_exponents():
    """Keys spread over 2^-60 .. 2^60 in some windows: a window's float64 sum is exact when its
    nonzero keys differ in binary exponent by at most 40 (8 significant bits each, at most 32
    terms), and the kernel then equals the exactly rounded mean bit for bit; other windows may
    round once more, and stay within one bf16 unit of the exact result."""
    p = synth.config_params("prefill32k")
    L = 4096
    rng = np.random.default_rng(71)
    k = rng.standard_normal((L, p.num_kv_heads, p.head_dim)).astype(np.float64)
    e = rng.integers(-15, 16, k.shape)
    wide = (np.arange(L) // 512) % 2 == 1
    e[wide] = rng.integers(-60, 61, (int(wide.sum()), p.num_kv_heads, p.head_dim))
    k = synth.round_to_bf16((k * 2.0 ** e).astype(np.float32))
    C = orc.num_kernels(L, p.kernel_size, p.kernel_stride)
    seqs = lib.Seqs([0], [0], [0], [0], [L], [0])
    kd = dev(k, "bf16")
    kern = torch.zeros((C, p.num_kv_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    log("case compress wide exponents")
    lib.compress_kernels(p, seqs, kd, kern)
    torch.cuda.synchronize()
    got = host(kern)
    ref = orc.compress_kernels(k, p.kernel_size, p.kernel_stride, p.dtype)
    ex = np.frexp(k.astype(np.float64))[1].astype(np.int64)
    big = np.where(k != 0, ex, np.iinfo(np.int64).min)
    small = np.where(k != 0, ex, np.iinfo(np.int64).max)
    exact_ok = np.zeros(got.shape, bool)
    for c in range(C):
        sl = slice(p.kernel_stride * c, p.kernel_stride * c + p.kernel_size)
        hi, lo = big[sl].max(axis=0), small[sl].min(axis=0)
        exact_ok[c] = (hi == np.iinfo(np.int64).min) | (hi - lo <= 40)
    assert np.array_equal(got[exact_ok], ref[exact_ok]), "kernel differs where the sum is exact"
    gb = got.view(np.uint32) >> 16
    rb = ref.astype(np.float32).view(np.uint32) >> 16
    diff = np.abs(gb.astype(np.int64) - rb.astype(np.int64))
    same_sign = np.sign(got) == np.sign(ref)
    assert np.all((diff <= 1) & (same_sign | (diff == 0)) | (got == ref)), "beyond one bf16 unit"
    log(f"compress wide: {int(exact_ok.sum())} exact-condition entries, "
        f"{int((~exact_ok).sum())} others, {int((diff[~exact_ok] > 0).sum())} of them off by one unit")


def test_results_are_deterministic():
    wl = synth.make("varlen", length_scale=1 / 32)
    a = run_prefill_stages(wl)
    b = run_prefill_stages(wl)
    for name in ("kernels", "idx", "out", "lse"):
        assert np.array_equal(a[name], b[name]), name


# ------------------------------------------------------------------------- decode

def check_decode_seq(p, ks, vs, q_rows, gk, scores, idx, out, lse, label):
    """One sequence of a decode step against the oracle: q_rows [n, Hq, d] are its new tokens
    (positions L-n .. L-1 of its L cached tokens); the other arguments are the GPU's kernels
    and the rows' scores, indices, outputs and LSE."""
    L = ks.shape[0]
    n = q_rows.shape[0]
    kern_ref = orc.compress_kernels(ks, p.kernel_size, p.kernel_stride, p.dtype)
    assert np.array_equal(gk[:kern_ref.shape[0]], kern_ref), f"{label}: kernels differ"
    ref = orc.run_sequence(q_rows, ks, vs, p, q_pos0=L - n, kernels=kern_ref,
                           with_attention=False)
    NB = ref.scores.shape[2]
    gs = scores[:, :, :NB]
    bound = cmp.score_bound(q_rows.astype(np.float64), kern_ref, ref.positions, p, NB)
    cmp.check_scores(gs, ref.scores, bound, ref.positions, p)
    assert np.array_equal(idx, orc.select_all(gs.astype(np.float64), ref.positions, p)), \
        f"{label}: top-k differs on the GPU's own scores"
    cmp.check_indices(idx, ref.idx, ref.scores, ref.positions, p)
    O, Ls = orc.sparse_attention(q_rows.astype(np.float64), ref.positions, ks, vs, idx, p)
    cmp.check_attention(out, lse, O, Ls, p.dtype)


def run_decode(wl, steps, num_splits=0, check=True, label="decode", step_fn=None):
    step_fn = step_fn or lib.decode_step
    p = wl.params
    B, Lmax = wl.batch, wl.max_len
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kern = torch.zeros((B * max(Ck, 1), p.num_kv_heads, p.head_dim), dtype=k.dtype, device="cuda")
    kv0 = wl.kv_len0.astype(np.int64)
    # prefill the kernel cache to the starting lengths (not timed here)
    s0 = lib.Seqs.decode(np.maximum(kv0, 1), Lmax, max(Ck, 1))
    lib.compress_kernels(p, lib.Seqs(s0.q_start, np.zeros(B), np.zeros(B), s0.kv_start, kv0,
                                     s0.kc_start), k, kern)
    nb = (Lmax + p.block_size - 1) // p.block_size
    bufs = lib.pipeline.decode_buffers(p, B, nb, num_splits, "cuda")
    outs = []
    prev = kv0.copy()
    for st in range(steps):
        kv = kv0 + st + 1
        seqs = lib.Seqs.decode(kv, Lmax, max(Ck, 1))
        q = dev(wl.q_steps[st], p.dtype)
        step_fn(p, seqs, q, k, v, kern, prev.astype(np.int32), bufs)
        torch.cuda.synchronize()
        prev = kv.copy()
        outs.append({n: host(bufs[n]) for n in ("scores", "idx", "out", "lse")})
        if check:
            for b in range(B):
                L = int(kv[b])
                o = outs[-1]
                check_decode_seq(p, wl.k[b, :L], wl.v[b, :L], wl.q_steps[st][b:b + 1],
                                 host(kern[b * Ck:(b + 1) * Ck]), o["scores"][b:b + 1],
                                 o["idx"][b:b + 1], o["out"][b:b + 1], o["lse"][b:b + 1],
                                 f"{label} seq {b} step {st}")
    return outs


def test_decode_small_ragged_lengths():
    p = synth.config_params("decode128k")
    wl = synth.make_decode("dec-small", p, batch=5, max_len=3000, steps=6, seed=41,
                           kv_len0=[2990, 2000, 1500, 700, 100])
    log("case decode small")
    run_decode(wl, 6)


def test_decode_sixty_four_sequences():
    """A decoding batch at the largest sequence table: 64 caches of seeded lengths (among them
    1 token and less than one kernel window), two steps."""
    p = synth.config_params("decode128k")
    rng = np.random.default_rng(49)
    kv0 = [int(x) for x in rng.integers(1, 5990, 64)]
    kv0[:3] = [1, 20, 63]
    wl = synth.make_decode("dec-64", p, batch=64, max_len=6000, steps=2, seed=49, kv_len0=kv0)
    log("case decode 64 sequences")
    run_decode(wl, 2)


def test_decode_hundred_sequences():
    """A decoding batch of 100 caches (seeded lengths from 1 token), two steps."""
    p = synth.config_params("decode128k")
    rng = np.random.default_rng(53)
    kv0 = [int(x) for x in rng.integers(1, 3990, 100)]
    kv0[:3] = [1, 20, 63]
    wl = synth.make_decode("dec-100", p, batch=100, max_len=4000, steps=2, seed=53, kv_len0=kv0)
    log("case decode 100 sequences")
    run_decode(wl, 2)


def test_decode_step_graph_replayed_with_device_metadata():
    """One decode step captured once in a HIP graph and replayed for three consecutive steps:
    between replays only the device copies of the lengths, positions, previous lengths and the
    new queries are rewritten.  Every replay equals the eagerly run step (indices and scores bit
    for bit, outputs to float32 rounding) and is checked against the oracle."""
    p = synth.config_params("decode128k")
    B, Lmax, steps = 3, 4096, 3
    wl = synth.make_decode("dec-graph", p, batch=B, max_len=Lmax, steps=steps, seed=54,
                           kv_len0=[4000, 3000, 2000])
    eager = run_decode(wl, steps, check=False, label="graph eager")
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kern = torch.zeros((B * Ck, p.num_kv_heads, p.head_dim), dtype=k.dtype, device="cuda")
    kv0 = wl.kv_len0.astype(np.int64)
    s0 = lib.Seqs.decode(kv0, Lmax, Ck)
    lib.compress_kernels(p, lib.Seqs(s0.q_start, np.zeros(B), np.zeros(B), s0.kv_start, kv0,
                                     s0.kc_start), k, kern)
    cuda = lambda a, dt: torch.tensor(np.asarray(a), dtype=dt, device="cuda")
    q_start, q_len = cuda(np.arange(B), torch.int64), cuda(np.ones(B), torch.int32)
    kv_start, kc_start = cuda(np.arange(B) * Lmax, torch.int64), cuda(np.arange(B) * Ck, torch.int64)
    kv_len, q_pos0, prev = (cuda(kv0 + 1, torch.int32), cuda(kv0, torch.int32),
                            cuda(kv0, torch.int32))
    seqs = lib.Seqs.on_device(q_start, q_len, q_pos0, kv_start, kv_len, kc_start, max_q_len=1,
                              max_kv_len=Lmax, q_rows=B)
    q = dev(wl.q_steps[0], p.dtype)
    bufs = lib.pipeline.decode_buffers(p, B, Lmax // p.block_size, 0, "cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.decode_step(p, seqs, q, k, v, kern, prev, bufs)
    torch.cuda.synchronize()
    for st in range(steps):
        kv = kv0 + st + 1
        kv_len.copy_(cuda(kv, torch.int32))
        q_pos0.copy_(cuda(kv - 1, torch.int32))
        prev.copy_(cuda(kv - 1, torch.int32))
        q.copy_(dev(wl.q_steps[st], p.dtype))
        torch.cuda.synchronize()
        log(f"case decode graph replay step {st}")
        graph.replay()
        torch.cuda.synchronize()
        got = {n: host(bufs[n]) for n in ("scores", "idx", "out", "lse")}
        assert np.array_equal(got["idx"], eager[st]["idx"]), f"replay {st}: indices differ"
        for r in range(B):
            nb = int(kv[r] - 1) // p.block_size + 1
            assert np.array_equal(got["scores"][r, :, :nb], eager[st]["scores"][r, :, :nb])
        assert np.abs(got["out"] - eager[st]["out"]).max() <= 1e-2
        assert np.abs(got["lse"] - eager[st]["lse"]).max() <= 1e-4
        for b in range(B):
            L = int(kv[b])
            check_decode_seq(p, wl.k[b, :L], wl.v[b, :L], wl.q_steps[st][b:b + 1],
                             host(kern[b * Ck:(b + 1) * Ck]), got["scores"][b:b + 1],
                             got["idx"][b:b + 1], got["out"][b:b + 1], got["lse"][b:b + 1],
                             f"graph step {st} seq {b}")
    assert int(torch.count_nonzero(bufs["workspace"].view(torch.int32)[:decode_counters_bytes(B, p) // 4])) == 0


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_decode_split_invariance(splits):
    p = synth.config_params("decode128k")
    wl = synth.make_decode("dec-split", p, batch=3, max_len=8192, steps=2, seed=42,
                           kv_len0=[8000, 6000, 3000])
    log(f"case decode splits={splits}")
    base = run_decode(wl, 2, num_splits=1, check=False)
    other = run_decode(wl, 2, num_splits=splits, check=(splits == 3))
    for a, b in zip(base, other):
        assert np.array_equal(a["idx"], b["idx"])
        assert np.abs(a["out"] - b["out"]).max() <= 1e-2
        assert np.abs(a["lse"] - b["lse"]).max() <= 1e-4


@pytest.mark.parametrize("Hq,d", [(32, 128), (16, 128), (32, 64), (16, 64)])
def test_decode_step_geometries(Hq, d):
    """The decode step's kernels for each (head_dim, group) pair (G = Hq / 2), checked against
    the oracle; ragged cache lengths, two steps."""
    p = replace(synth.config_params("decode128k"), num_q_heads=Hq, head_dim=d)
    wl = synth.make_decode(f"dec-geo-{Hq}-{d}", p, batch=3, max_len=9000, steps=2, seed=51,
                           kv_len0=[8990, 5000, 700])
    log(f"case decode step Hq={Hq} d={d}")
    run_decode(wl, 2, label=f"geo {Hq}/{d}")


def test_decode_f32_tiny_shape():
    p = synth.config_params("tiny")
    wl = synth.make_decode("dec-f32", p, batch=2, max_len=512, steps=3, seed=43,
                           kv_len0=[500, 300])
    log("case decode f32")
    run_decode(wl, 3, num_splits=2)


# ------------------------------------------------------------------------- full sizes

def whole_tiles(L, n_windows=8, needle_rows=()):
    """Every row of n_windows windows of 192 consecutive rows aligned to 192 (whole tiles of 16,
    24, 32 or 64 query rows): spread over the sequence, the last window, and one holding a needle
    query (when there is one)."""
    W = 192
    last = max(0, (L - 1) // W)
    starts = {int(x) for x in np.linspace(0, last, n_windows - 1).round()} | {last}
    if len(needle_rows):
        starts.add(int(needle_rows[0]) // W)
    rows = set()
    for st in starts:
        rows |= set(range(st * W, min(L, st * W + W)))
    return rows


def sample_rows(wl, b, extra=(), tiles=False):
    p = wl.params
    L = int(wl.q_len[b])
    dense = min(L, p.topk * p.block_size)
    rows = set(range(0, dense, 97)) | set(range(max(0, L - 5), L)) | set(range(dense, L, 1777))
    rows |= {r for r in extra if 0 <= r < L}
    if tiles:
        rows |= whole_tiles(L, needle_rows=[r for r in extra if 0 <= r < L])
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["prefill32k", "varlen", "prefill128k"])
def test_full_size_prefill_sampled(name):
    wl = synth.make(name)
    log(f"case full {name}")
    res = run_prefill_stages(wl)
    # every needle query selects its needle, on all rows (not only sampled)
    for nd in wl.needles:
        rows = int(wl.q_start[nd.seq]) + nd.query_positions
        assert np.all(np.any(res["idx"][rows, nd.kv_head, :] == nd.block, axis=1))
    for b in range(wl.num_seqs):
        extra = [int(r) for nd in wl.needles if nd.seq == b for r in nd.query_positions[:4]]
        check_sequence(wl, res, b, rows=sample_rows(wl, b, extra, tiles=True),
                       label=f"full {name}")
    # sparsity: selected-token fraction per row follows the configured top-k
    p = wl.params
    nsel = (res["idx"] >= 0).sum(axis=2)
    for b in range(wl.num_seqs):
        pos = np.arange(int(wl.q_len[b]))
        expect = np.minimum(pos // p.block_size + 1, p.topk)
        rows = int(wl.q_start[b]) + pos
        assert np.all(nsel[rows] == expect[:, None])


def test_full_size_chunk_sampled():
    """Chunked prefill at the measured size: the last 16K tokens of the 128K sequence as queries
    (q_pos0 = 112K) against the whole cache; sampled rows, and every needle query in the chunk
    finds its needle."""
    full = synth.make("prefill128k")
    p = full.params
    L, C = 131072, 16384
    wl = synth.Workload("chunk16k", p, full.q[L - C:], full.k, full.v, np.array([0]),
                        np.array([C], np.int32), np.array([L - C], np.int32), np.array([0]),
                        np.array([L], np.int32))
    log("case full chunk 16K of 128K")
    res = run_prefill_stages(wl)
    for nd in full.needles:
        qp = nd.query_positions[nd.query_positions >= L - C] - (L - C)
        if len(qp):
            assert np.all(np.any(res["idx"][qp, nd.kv_head, :] == nd.block, axis=1))
    rows = np.array(sorted(set(range(0, C, 997)) | set(range(C - 3, C))))
    check_sequence(wl, res, 0, rows=rows, label="full chunk")


def test_full_size_decode():
    wl = synth.make("decode128k", steps=2)
    log("case full decode128k")
    run_decode(wl, 2, label="full decode")


def test_decode_fused_call_matches_staged_calls():
    """infllm2_decode_step (scores and top-k in one launch, then the attention) against the four
    separate calls: both checked against the oracle, scores and indices identical, outputs
    equal to float32 rounding (the step may split the blocks over other workgroup shapes)."""
    p = synth.config_params("decode128k")
    wl = synth.make_decode("dec-fused", p, batch=4, max_len=4096, steps=2, seed=44,
                           kv_len0=[4000, 2500, 1000, 64])
    log("case decode fused vs staged")
    fused = run_decode(wl, 2, label="step")
    staged = run_decode(wl, 2, step_fn=lib.pipeline.decode_step_staged, label="staged")
    for st, (a, b) in enumerate(zip(fused, staged)):
        assert np.array_equal(a["idx"], b["idx"])
        for r in range(wl.batch):   # scores past the query's own block are left unwritten
            nb = (int(wl.kv_len0[r]) + st) // p.block_size + 1
            assert np.array_equal(a["scores"][r, :, :nb], b["scores"][r, :, :nb])
        assert np.abs(a["out"] - b["out"]).max() <= 1e-2
        assert np.abs(a["lse"] - b["lse"]).max() <= 1e-4


def test_decode_forced_blocks_only():
    """top-k equal to the forced blocks (1 first + 2 local): nothing is left to choose once a
    row sees more than 3 blocks."""
    p = replace(synth.config_params("decode128k"), topk=3)
    wl = synth.make_decode("dec-forced", p, batch=3, max_len=3000, steps=2, seed=45,
                           kv_len0=[2990, 900, 100])
    log("case decode forced only")
    run_decode(wl, 2)


def test_decode_tied_scores():
    """Every key equal, so every kernel and every block score ties: the lowest block indices
    win, and attention over equal keys is the mean of the selected values."""
    p = synth.config_params("decode128k")
    wl = synth.make_decode("dec-ties", p, batch=2, max_len=8192, steps=2, seed=46,
                           kv_len0=[8000, 7000])
    wl.k[:] = wl.k[:, :1]
    log("case decode ties")
    outs = run_decode(wl, 2)
    for st, o in enumerate(outs):
        for b in range(wl.batch):
            own = (int(wl.kv_len0[b]) + st) // p.block_size
            chosen = o["idx"][b, 0]
            assert chosen[0] == 0 and chosen[-2] == own - 1 and chosen[-1] == own
            assert np.array_equal(chosen[1:-2], np.arange(1, p.topk - 2))


def test_decode_several_rows_per_sequence():
    """Three new tokens per sequence in one step (positions L-3 .. L-1), each row with its own
    scores, selection and attention; one sequence with a single row."""
    p = synth.config_params("decode128k")
    lens, nq, Lmax = [3000, 2100, 700], [3, 3, 1], 3072
    B = len(lens)
    wl = synth.make_decode("dec-rows", p, batch=B, max_len=Lmax, steps=1, seed=47)
    rng = np.random.default_rng(48)
    qs = [synth.make_upstream_grad((n, p.num_q_heads, p.head_dim), int(rng.integers(1 << 30)))
          for n in nq]
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kern = torch.zeros((B * Ck, p.num_kv_heads, p.head_dim), dtype=k.dtype, device="cuda")
    q_start = np.concatenate([[0], np.cumsum(nq)[:-1]])
    seqs = lib.Seqs(q_start, nq, np.array(lens) - np.array(nq), np.arange(B) * Lmax, lens,
                    np.arange(B) * Ck)
    bufs = lib.pipeline.decode_buffers(p, sum(nq), (Lmax + 63) // 64, 0, "cuda")
    log("case decode several rows")
    lib.decode_step(p, seqs, dev(np.concatenate(qs), p.dtype), k, v, kern, None, bufs)
    torch.cuda.synchronize()
    res = {n: host(bufs[n]) for n in ("scores", "idx", "out", "lse")}
    for b in range(B):
        r = slice(int(q_start[b]), int(q_start[b]) + nq[b])
        check_decode_seq(p, wl.k[b, :lens[b]], wl.v[b, :lens[b]], qs[b],
                         host(kern[b * Ck:(b + 1) * Ck]), res["scores"][r], res["idx"][r],
                         res["out"][r], res["lse"][r], f"rows seq {b}")


def test_decode_step_compresses_kernels_past_the_queries():
    """The decode step stores every kernel completed since prev_kv_len, also those past its query
    rows' positions: a cache that runs past the last query (rows at 2000 of 3000 tokens, at 9000
    of 20000), prev_kv_len from 0 (every kernel new) to past the queries, and two rows of one
    sequence; the kernel rows never written are poisoned with NaN."""
    p = synth.config_params("decode128k")
    lens, prev, pos0, nq, Lmax = [3000, 3000, 3000, 20000], [0, 2500, 1500, 8000], \
        [2000, 2000, 1999, 9000], [1, 1, 2, 1], 20000
    B = len(lens)
    wl = synth.make_decode("dec-past", p, batch=B, max_len=Lmax, steps=1, seed=51)
    rng = np.random.default_rng(52)
    qs = [synth.make_upstream_grad((n, p.num_q_heads, p.head_dim), int(rng.integers(1 << 30)))
          for n in nq]
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kern = torch.full((B * Ck, p.num_kv_heads, p.head_dim), float("nan"), dtype=k.dtype,
                      device="cuda")
    kc = np.arange(B) * Ck
    lib.compress_kernels(p, lib.Seqs(np.arange(B), np.zeros(B), np.zeros(B), np.arange(B) * Lmax,
                                     prev, kc), k, kern)
    q_start = np.concatenate([[0], np.cumsum(nq)[:-1]])
    seqs = lib.Seqs(q_start, nq, pos0, np.arange(B) * Lmax, lens, kc)
    bufs = lib.pipeline.decode_buffers(p, sum(nq), Lmax // 64 + 1, 0, "cuda")
    log("case decode step, cache past the queries")
    lib.decode_step(p, seqs, dev(np.concatenate(qs), p.dtype), k, v, kern,
                    np.array(prev, dtype=np.int32), bufs)
    torch.cuda.synchronize()
    res = {n: host(bufs[n]) for n in ("scores", "idx", "out", "lse")}
    gk_all = host(kern)
    for b in range(B):
        L = lens[b]
        ks, vs = wl.k[b, :L], wl.v[b, :L]
        kern_ref = orc.compress_kernels(ks, p.kernel_size, p.kernel_stride, p.dtype)
        gk = gk_all[kc[b]:kc[b] + kern_ref.shape[0]]
        assert np.array_equal(gk, kern_ref), f"seq {b}: kernels differ"
        r = slice(int(q_start[b]), int(q_start[b]) + nq[b])
        ref = orc.run_sequence(qs[b], ks, vs, p, q_pos0=pos0[b], kernels=kern_ref,
                               with_attention=False)
        nbq = int(ref.positions[-1]) // p.block_size + 1
        gs = res["scores"][r][:, :, :nbq]
        bound = cmp.score_bound(qs[b].astype(np.float64), kern_ref, ref.positions, p, nbq)
        cmp.check_scores(gs, ref.scores[:, :, :nbq], bound, ref.positions, p)
        assert np.array_equal(res["idx"][r], orc.select_all(gs.astype(np.float64), ref.positions, p))
        cmp.check_indices(res["idx"][r], ref.idx, ref.scores[:, :, :nbq], ref.positions, p)
        O, Ls = orc.sparse_attention(qs[b].astype(np.float64), ref.positions, ks, vs,
                                     res["idx"][r], p)
        cmp.check_attention(res["out"][r], res["lse"][r], O, Ls, p.dtype)


def test_decode_longest_cache():
    """A 262144-token cache: 4096 blocks, the most a selection takes."""
    p = synth.config_params("decode128k")
    wl = synth.make_decode("dec-256k", p, batch=1, max_len=262144, steps=1, seed=49)
    log("case decode 256K")
    run_decode(wl, 1, label="256K decode")


def decode_counters_bytes(rows, p):
    al = lambda x: (x + 255) // 256 * 256
    return 2 * al(rows * p.num_kv_heads * 4)


def test_decode_leaves_workspace_counters_zero():
    """Each decode step zeroes the workspace counters it used (score chunks, attention splits),
    so consecutive steps share one workspace; every step checked against the oracle."""
    p = synth.config_params("decode128k")
    B, Lmax = 3, 4096
    wl = synth.make_decode("dec-ws", p, batch=B, max_len=Lmax, steps=3, seed=50,
                           kv_len0=[4000, 3000, 2000])
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kern = torch.zeros((B * Ck, p.num_kv_heads, p.head_dim), dtype=k.dtype, device="cuda")
    bufs = lib.pipeline.decode_buffers(p, B, Lmax // 64, 0, "cuda")
    n_cnt = decode_counters_bytes(B, p) // 4
    for st in range(3):
        kv = wl.kv_len0.astype(np.int64) + st + 1
        seqs = lib.Seqs.decode(kv, Lmax, Ck)
        log(f"case decode workspace step {st}")
        lib.decode_step(p, seqs, dev(wl.q_steps[st], p.dtype), k, v, kern, None, bufs)
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(bufs["workspace"].view(torch.int32)[:n_cnt])) == 0
        for b in range(B):
            L = int(kv[b])
            check_decode_seq(p, wl.k[b, :L], wl.v[b, :L], wl.q_steps[st][b:b + 1],
                             host(kern[b * Ck:(b + 1) * Ck]), host(bufs["scores"])[b:b + 1],
                             host(bufs["idx"])[b:b + 1], host(bufs["out"])[b:b + 1],
                             host(bufs["lse"])[b:b + 1], f"ws step {st} seq {b}")
