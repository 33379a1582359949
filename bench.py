"""Benchmark of the InfLLM v2 hot path on one MI355X.

A step is one pass of the whole prefill path over the 128K-token MiniCPM4-8B-shaped layer
(32 query heads / 2 KV heads, head_dim 128, bf16, block 64, kernels 32/16, top-96 with 1
initial + 2 local blocks): compress_kernels -> block_scores -> topk_select ->
sparse_attn_prefill, inputs resident in HBM.  `value` is prefill tokens/s of that pass.
The line also carries the decode measurement (batch 8 x 128K cache, one token each, 16
consecutive steps with incremental kernel updates), a chunked prefill (the last 16K tokens
against a 112K cache), block scores in score mode 1, sliding-window attention (window 6144),
the backward of the attention on the same layer (dQ, dK, dV for a seeded upstream gradient, the
forward's selection held fixed), the roofline of the dominant kernel (from HIP events on the
launch stream) and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload prefill128k|prefill32k|varlen]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tokens/s @128K + decode µs/token; % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
def _group_bound(lens, rows: int, gs: int, hkv: int) -> int:
    """The library's host bound on the groups of gs consecutive tiles of `rows` tokens (one XCD's
    share of a round; it sees the metadata's bounds only: sequences, longest query run, total
    rows)."""
    n_seq, max_q, T = len(lens), max(lens), sum(lens)
    per_seq = -(-(-(-max_q // rows)) // gs)
    return min(n_seq * per_seq, -(-T // (rows * gs)) + n_seq) * hkv


def tile_tokens(p) -> int:
    """Query tokens per prefill attention work item, chosen as the library chooses: when a group
    has 8 query heads (two tokens' heads share the 16 columns of each matrix-core tile), 64 at
    head_dim 64 and 32 at 128; else 24 (3 per wave)."""
    if p.num_q_heads // p.num_kv_heads == 8:
        return 64 if p.head_dim == 64 else 32
    return 24


ROUNDS_PER_LAUNCH = 3     # the library's tile-schedule rounds per attention launch
WINDOW = 6144             # sliding-window leg: 96 blocks x 64 tokens
CHUNK = 16384             # chunked-prefill leg: the last 16K tokens against a 112K cache
SPIN_CYCLES = 24_000_000  # GPU spin before the timed decode steps (about 10 ms at 2.4 GHz)
SPIN_SECONDS = 0.008      # enqueueing must finish well inside the spin
ATTN_SOURCES = ["block_sparse_long_semantic_amd/csrc/attn_tile.hip",
                "block_sparse_long_semantic_amd/csrc/internal.h"]
BWD_SOURCES = ["block_sparse_long_semantic_amd/csrc/attn_bwd.hip",
               "block_sparse_long_semantic_amd/csrc/internal.h"]
def _attn_form(kernel: str, bwd: str, win: str) -> bool:
    """True for an attn_tile instance whose gradient and window flags (its 6th and 7th
    template arguments) are the given ones."""
    if not kernel.startswith("attn_tile<"):
        return False
    args = [a.strip() for a in kernel[kernel.index("<") + 1:kernel.rindex(">")].split(",")]
    return len(args) >= 7 and args[5] == bwd and args[6] == win


# kernels whose HBM traffic the committed counter summary records: role -> (name test, sources)
TRAFFIC_ROLES = {
    "prefill_attention": (lambda k: _attn_form(k, "false", "false"), ATTN_SOURCES),
    "backward_dq": (lambda k: _attn_form(k, "true", "false"), ATTN_SOURCES),
    "window_attention": (lambda k: _attn_form(k, "false", "true"), ATTN_SOURCES),
    "backward_dkv": (lambda k: k.startswith("bwd_dkv"), BWD_SOURCES),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attended_keys_total(seq_lens, block, topk):
    """Keys attended per query head summed over all query tokens (valid keys only)."""
    tot = 0
    for L in seq_lens:
        i = np.arange(L, dtype=np.int64)
        dense = (i // block) + 1 <= topk
        tot += int(np.where(dense, i + 1, (topk - 1) * block + (i % block) + 1).sum())
    return tot


def run_prefill(args, torch, pkg, synth, workload=None, keep=True):
    workload = workload or args.workload
    wl = synth.make(workload)
    p = wl.params
    lens = [int(x) for x in wl.q_len]
    log(f"workload {workload}: seqs {lens}, inputs drawn")
    seqs = pkg.Seqs.packed_prefill(lens)
    dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
    q = torch.from_numpy(wl.q).cuda().to(dt)
    k = torch.from_numpy(wl.k).cuda().to(dt)
    v = torch.from_numpy(wl.v).cuda().to(dt)
    kc_rows = sum(pkg.num_kernels(L, p.kernel_size, p.kernel_stride) for L in lens)
    bufs = pkg.pipeline.prefill_buffers(p, seqs, q, kc_rows)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        pkg.compress_kernels(p, seqs, k, bufs["kernels"], stream=stream)
        if ev: ev[1].record(stream)
        pkg.block_scores(p, seqs, q, bufs["kernels"], bufs["scores"], stream=stream)
        if ev: ev[2].record(stream)
        pkg.topk_select(p, seqs, bufs["scores"], bufs["idx"], stream=stream)
        if ev: ev[3].record(stream)
        pkg.sparse_attn_prefill(p, seqs, q, k, v, bufs["idx"], bufs["out"], bufs["lse"],
                                stream=stream)
        if ev: ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    names = ["compress", "scores", "topk", "attention"]
    stage = {n: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
             for i, n in enumerate(names)}
    T = sum(lens)
    ms_step = wall * 1e3 / args.steps
    keys = attended_keys_total(lens, p.block_size, p.topk)
    flops = 4.0 * p.head_dim * p.num_q_heads * keys
    tflops = flops / (stage["attention"] * 1e-3) / 1e12
    d, Hq, Hkv = p.head_dim, p.num_q_heads, p.num_kv_heads
    C = kc_rows
    causal_blocks = sum(int(((np.arange(L) // p.block_size) + 1).sum()) for L in lens)
    bytes_scores = T * Hq * d * 2 + C * Hkv * d * 2 + causal_blocks * Hkv * 4
    bytes_topk = causal_blocks * Hkv * 4 + T * Hkv * p.topk * 4
    bytes_compress = T * Hkv * d * 2 + C * Hkv * d * 2
    # the attention call schedules its tiles in rounds of one workgroup per compute unit, 8
    # groups of CUs / 8 tiles each, ROUNDS_PER_LAUNCH rounds per launch; the rounds cover the
    # library's host bound on the groups (it sees only the metadata's bounds: sequences,
    # longest query run, total rows), not the exact count
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    TT = tile_tokens(p)
    launches = -(-_group_bound(lens, TT, max(1, cus // 8), Hkv) // (8 * ROUNDS_PER_LAUNCH))
    result = dict(
        workload=workload, tokens=T, seq_lens=lens, p=p, ms_step=ms_step, stage=stage,
        flops=flops, tflops=tflops, keys=keys, launches=launches,
        stage_gbs={"compress": bytes_compress / (stage["compress"] * 1e-3) / 1e9,
                   "scores": bytes_scores / (stage["scores"] * 1e-3) / 1e9,
                   "topk": bytes_topk / (stage["topk"] * 1e-3) / 1e9},
        wl=wl, kernels_gpu=bufs["kernels"],
        gather=gather_bound(p, bufs["idx"].cpu().numpy(), lens, flops, stage["attention"], TT))
    if not keep or (args.no_backward and args.no_window and args.no_score_mode1 and args.no_chunk):
        del q, k, v, bufs
    else:
        result["device"] = dict(q=q, k=k, v=v, seqs=seqs, idx=bufs["idx"], out=bufs["out"],
                                lse=bufs["lse"], scores=bufs["scores"])
        del bufs
    return result


def run_chunk(args, torch, pkg, pre):
    """Chunked prefill: the last CHUNK tokens of the 128K sequence arrive as a chunk against a
    cache holding the earlier ones (q_pos0 > 0): incremental kernels, scores, top-k and
    attention for the chunk's rows, timed per stage like the full prefill."""
    p, dv_ = pre["p"], pre["device"]
    L = pre["seq_lens"][0]
    C = min(CHUNK, L)
    q = dv_["q"][L - C:]
    k, v = dv_["k"], dv_["v"]
    seqs = pkg.Seqs(np.array([0]), np.array([C]), np.array([L - C]), np.array([0]), np.array([L]),
                    np.array([0]))
    prev = torch.tensor([L - C], dtype=torch.int32, device="cuda")
    nb = (L - 1) // p.block_size + 1
    dt = q.dtype
    scores = torch.empty((C, p.num_kv_heads, nb), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, p.num_kv_heads, p.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((C, p.num_q_heads), dtype=torch.float32, device="cuda")
    kern = pre["kernels_gpu"]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev: ev[0].record(stream)
        pkg.compress_kernels(p, seqs, k, kern, prev_kv_len=prev, stream=stream)
        if ev: ev[1].record(stream)
        pkg.block_scores(p, seqs, q, kern, scores, stream=stream)
        if ev: ev[2].record(stream)
        pkg.topk_select(p, seqs, scores, idx, stream=stream)
        if ev: ev[3].record(stream)
        pkg.sparse_attn_prefill(p, seqs, q, k, v, idx, out, lse, stream=stream)
        if ev: ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        step(evs[st])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    names = ["compress", "scores", "topk", "attention"]
    stage = {n: float(np.mean([evs[st][i].elapsed_time(evs[st][i + 1]) for st in range(args.steps)]))
             for i, n in enumerate(names)}
    i = np.arange(L - C, L, dtype=np.int64)
    keys = int(np.where((i // p.block_size) + 1 <= p.topk, i + 1,
                        (p.topk - 1) * p.block_size + (i % p.block_size) + 1).sum())
    flops = 4.0 * p.head_dim * p.num_q_heads * keys
    tflops = flops / (stage["attention"] * 1e-3) / 1e12
    del scores, idx, out, lse
    return dict(chunk_tokens=C, cache_tokens=L - C, ms_per_chunk=wall * 1e3,
                tokens_per_s=C / wall, stages_ms=stage,
                roofline={"kernel": "attn_tile (sparse_attn_prefill, q_pos0 > 0)", "bound": "mfma",
                          "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": tflops / PEAK_BF16_TFLOPS, "flops_per_call": flops})


def prefill_leg(args, torch, pkg, synth, workload):
    """Another prefill configuration, timed like the headline one (whole step of the four calls
    and its attention with the roofline against the bf16 peak); a parity-tested config, reported
    beside the headline workload."""
    r = run_prefill(args, torch, pkg, synth, workload=workload, keep=False)
    st = r["stage"]
    out = {"workload": workload, "seq_lens": r["seq_lens"], "ms_per_step": r["ms_step"],
           "tokens_per_s": r["tokens"] / (r["ms_step"] * 1e-3), "stages_ms": st,
           "stages_gbs": r["stage_gbs"],
           "attention_tokens_per_s": r["tokens"] / (st["attention"] * 1e-3),
           "roofline": {"kernel": "attn_tile (sparse_attn_prefill)", "bound": "mfma",
                        "achieved": r["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": r["tflops"] / PEAK_BF16_TFLOPS, "traffic": None,
                        "flops_per_call": r["flops"], "launches_per_call": r["launches"],
                        "avg_launch_us": st["attention"] * 1e3 / r["launches"],
                        "gather": r["gather"]}}
    tr = measured_traffic(workload)
    if tr is not None:
        out["roofline"]["traffic"] = tr["fetch_bytes_per_call"] + tr["write_bytes_per_call"]
    del r
    torch.cuda.empty_cache()
    return out


def gather_bound(p, idx, seq_lens, flops, ms_attention, TT):
    """The prefill attention's gather: K/V bytes of every (token, KV head)'s selected blocks
    (idx: host array [rows, Hkv, topk] of one packed prefill) against the bytes the tile kernel
    stages (each tile loads the union of its tokens' selected blocks once), the reuse factor and
    the staging rate achieved."""
    block_bytes = 2 * p.block_size * p.head_dim * 2                 # K and V, bf16
    selected = int((idx >= 0).sum()) * block_bytes
    staged_blocks = 0
    start = 0
    for L in seq_lens:
        sel = idx[start:start + L]
        start += L
        pad = (-L) % TT
        if pad:
            sel = np.concatenate([sel, np.full((pad,) + sel.shape[1:], -1, sel.dtype)])
        t = np.sort(sel.reshape(-1, TT, sel.shape[1], sel.shape[2]).transpose(0, 2, 1, 3)
                    .reshape(-1, TT * sel.shape[2]), axis=1)
        new = np.ones(t.shape, bool)
        new[:, 1:] = t[:, 1:] != t[:, :-1]
        staged_blocks += int((new & (t >= 0)).sum())
    staged = staged_blocks * block_bytes
    rate = staged / (ms_attention * 1e-3)
    return {"selected_bytes": selected, "staged_bytes": staged,
            "reuse_tokens_per_staged_block": selected / staged,
            "flop_per_staged_byte": flops / staged,
            "staging_rate_gbs": rate / 1e9,
            "staging_bytes_per_clk_per_cu": rate / 256 / 2.4e9,
            "note": f"{TT}-token tiles; each tile stages the union of its tokens' selected "
                    "blocks (K and V) from L2 into LDS once"}


def run_score_mode1(args, torch, pkg, pre):
    """Block scores in score mode 1 (per-head softmax over the visible kernels before the group
    sum) on the same layer and kernels; algorithmic work = the per-head products once."""
    from dataclasses import replace
    p = replace(pkg.Params.from_any(pre["p"]), score_mode=1)
    dv_ = pre["device"]
    stream = torch.cuda.current_stream()

    def call():
        pkg.block_scores(p, dv_["seqs"], dv_["q"], pre["kernels_gpu"], dv_["scores"], stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        ev[s][0].record(stream)
        call()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    vis = 0
    for L in pre["seq_lens"]:
        i = np.arange(L, dtype=np.int64)
        C = 0 if L < p.kernel_size else (L - p.kernel_size) // p.kernel_stride + 1
        vis += int(np.clip((i - p.kernel_size + 1) // p.kernel_stride + 1, 0, C).sum())
    flops = 2.0 * p.head_dim * p.num_q_heads * vis
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(ms_per_call=ms, visible_kernels=vis, flops_per_call=flops,
                note="two passes over the kernels (lse, then probabilities); flops count the "
                     "per-head products once",
                roofline={"kernel": "scores_softmax_mfma", "bound": "mfma", "achieved": tflops,
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": tflops / PEAK_BF16_TFLOPS})


def run_window(args, torch, pkg, pre):
    """Sliding-window attention over the same 128K layer (window WINDOW tokens: the keys a
    top-96 selection of 64-token blocks covers), timed like the sparse attention call."""
    p, dv_ = pre["p"], pre["device"]
    q, k, v, seqs = dv_["q"], dv_["k"], dv_["v"], dv_["seqs"]
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], p.num_q_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        pkg.sliding_window_attn(p, seqs, WINDOW, q, k, v, out, lse, stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        ev[s][0].record(stream)
        call()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    keys = sum(int(np.minimum(np.arange(L) + 1, WINDOW).sum()) for L in pre["seq_lens"])
    flops = 4.0 * p.head_dim * p.num_q_heads * keys
    tflops = flops / (ms * 1e-3) / 1e12
    del out, lse
    return dict(window=WINDOW, ms_per_call=ms, tokens_per_s=pre["tokens"] / (ms * 1e-3),
                keys_per_head=keys, flops_per_call=flops,
                roofline={"kernel": "attn_tile (window form)", "bound": "mfma", "achieved": tflops,
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": tflops / PEAK_BF16_TFLOPS,
                          "traffic": measured_traffic(pre["workload"], "window_attention")})


def run_backward(args, torch, pkg, synth, pre):
    """Backward of the attention call on the prefill workload: dout seeded, dq/dk/dv float32."""
    p, dv_ = pre["p"], pre.pop("device")
    q, k, v, seqs = dv_["q"], dv_["k"], dv_["v"], dv_["seqs"]
    dout = torch.from_numpy(synth.make_upstream_grad(tuple(q.shape), 62)).cuda().to(q.dtype)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dvv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(pkg.backward_workspace_size(p, seqs), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        pkg.sparse_attn_backward(p, seqs, q, k, v, dv_["idx"], dv_["out"], dv_["lse"], dout, dq,
                                 dk, dvv, ws, stream=stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        ev[s][0].record(stream)
        call()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    # algorithmic work: the five products of an attention backward (S recomputed, dP, dV, dQ,
    # dK), 2 d flops per (query head, attended key) each
    flops = 10.0 * p.head_dim * p.num_q_heads * pre["keys"]
    tflops = flops / (ms * 1e-3) / 1e12
    # (row, KV head, selected block) pairs; the dK/dV kernel stages, per pair, the row's q and
    # dout for the group's G heads (bf16) and their lse and delta (float32)
    lens = pre["seq_lens"]
    pairs = p.num_kv_heads * sum(int(np.minimum(np.arange(L) // p.block_size + 1, p.topk).sum())
                                 for L in lens)
    G = p.num_q_heads // p.num_kv_heads
    staged = pairs * G * (2 * p.head_dim * 2 + 2 * 4)
    out = dict(ms_per_call=ms, tokens_per_s=pre["tokens"] / (ms * 1e-3),
               flops_per_call=flops, tflops=tflops, frac_of_bf16_peak=tflops / PEAK_BF16_TFLOPS,
               workspace_bytes=int(ws.numel()),
               note="one infllm2_sparse_attn_backward call (zero-fill, delta and reverse index, "
                    "dQ kernel, dK/dV kernel); per-kernel times in the committed profile",
               kernels={
                   "dq": {"kernel": "attn_tile (gradient form)",
                          "flops_per_call": 6.0 * p.head_dim * p.num_q_heads * pre["keys"],
                          "traffic": measured_traffic(pre["workload"], "backward_dq")},
                   "dkv": {"kernel": "bwd_dkv", "pairs": pairs, "staged_bytes_per_call": staged,
                           "flops_per_call": 8.0 * p.head_dim * p.num_q_heads * pre["keys"],
                           "traffic": measured_traffic(pre["workload"], "backward_dkv")}})
    # the oracle's backward on a bounded sample of rows (every row attends topk blocks)
    if not args.no_cpu_baseline:
        from oracle import infllm2_oracle as orc
        wl = pre["wl"]
        L = pre["seq_lens"][0]
        rows = np.linspace(p.topk * p.block_size, L - 1, 4096).astype(np.int64)
        idx = dv_["idx"][torch.from_numpy(rows).cuda()].cpu().numpy()
        do = dout[torch.from_numpy(rows).cuda()].float().cpu().numpy()
        done, t0 = 0, time.perf_counter()
        while done < len(rows) and time.perf_counter() - t0 < args.cpu_budget / 3:
            r = slice(done, done + 8)
            orc.sparse_attention_backward(wl.q[rows[r]], rows[r], wl.k, wl.v, idx[r], do[r], p)
            done += 8
        el = time.perf_counter() - t0
        out["cpu_oracle"] = {"rows_per_s": done / el, "rows": done, "seconds": el,
                             "cores": int(os.environ.get("OMP_NUM_THREADS", "1")),
                             "kind": "oracle (float64 numpy, one process)",
                             "sample": f"{done} rows spread over positions "
                                       f"{rows[0]}..{rows[min(done, len(rows)) - 1]}",
                             "speedup_gpu_over_oracle": (pre["tokens"] / (ms * 1e-3)) / (done / el)}
    del dq, dk, dvv, ws, dout
    return out


def copy_calibration(torch, mib: int):
    """A plain streaming kernel of known traffic (read mib MiB, write mib MiB), for scaling the
    FETCH_SIZE / WRITE_SIZE counters: out = -in over bf16 elements."""
    n = (mib << 20) // 2
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: {mib} MiB read + {mib} MiB written")
    del src, dst


def measured_peaks(torch):
    """Achievable rates of this GPU, reported beside the datasheet peaks for context: a streaming
    kernel (out = -in over 1 GiB of bf16: 2 GiB moved per call) and a large bf16 matrix product
    (8192^3, the vendor GEMM behind torch.mm), each timed with events on the current stream."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps
    n = (1 << 30) // 2
    src = torch.randn(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: torch.neg(src, out=dst), 10)
    del src, dst
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(m, m, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(m, m, dtype=torch.bfloat16, device="cuda")
    t_mm = timed(lambda: torch.mm(a, b, out=c), 10)
    del a, b, c
    return {"hbm_stream_gbs": 2.0 * (n * 2) / t_copy / 1e9,
            "bf16_gemm_tflops": 2.0 * m ** 3 / t_mm / 1e12,
            "note": "out = -in over 1 GiB bf16 (2 GiB moved per call); torch.mm of two "
                    "8192 x 8192 bf16 matrices; context for the datasheet peaks "
                    f"({PEAK_HBM_GBS:.0f} GB/s, {PEAK_BF16_TFLOPS:.0f} TFLOP/s), which the "
                    "roofline fractions use"}


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, role: str = "prefill_attention"):
    """HBM bytes per call of one kernel (TRAFFIC_ROLES) from the committed counter summary, or
    None when there is none for this workload or the kernel's source has changed since."""
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("bench-data: "):
                rec = json.loads(line[len("bench-data: "):])
                if rec.get("role") != role:
                    continue
                if rec.get("source_sha256") != source_digest(TRAFFIC_ROLES[role][1]):
                    return None
                return rec
    return None


def run_decode(args, torch, pkg, synth):
    wl = synth.make("decode128k", steps=args.decode_steps)
    p = wl.params
    B, Lmax = wl.batch, wl.max_len
    dt = torch.bfloat16
    Ck = pkg.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = torch.from_numpy(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim)).cuda().to(dt)
    v = torch.from_numpy(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim)).cuda().to(dt)
    qs = torch.from_numpy(wl.q_steps).cuda().to(dt)
    kern = torch.zeros((B * Ck, p.num_kv_heads, p.head_dim), dtype=dt, device="cuda")
    kv0 = wl.kv_len0.astype(np.int64)
    s0 = pkg.Seqs(np.arange(B), np.zeros(B), np.zeros(B), np.arange(B) * Lmax, kv0,
                  np.arange(B) * Ck)
    nb = (Lmax + p.block_size - 1) // p.block_size
    bufs = pkg.pipeline.decode_buffers(p, B, nb, args.decode_splits, "cuda")
    stream = torch.cuda.current_stream()
    seqs = [pkg.Seqs.decode(kv0 + st + 1, Lmax, Ck) for st in range(args.decode_steps)]
    prevs = [torch.tensor(kv0 + st, dtype=torch.int32, device="cuda")
             for st in range(args.decode_steps)]
    for sq in seqs:
        sq.c(k.device)                  # the metadata's device copies, made before any timing

    def all_steps(on=stream):
        for st in range(args.decode_steps):
            pkg.decode_step(p, seqs[st], qs[st], k, v, kern, prevs[st], bufs, stream=on)

    for _ in range(max(1, args.warmup)):
        pkg.compress_kernels(p, s0, k, kern, stream=stream)
        all_steps()
    # host-inclusive: every step's Python marshalling and launches, synchronised at the end
    pkg.compress_kernels(p, s0, k, kern, stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_steps()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # GPU time per step: the GPU spins (about 10 ms) while the host enqueues all steps, so two
    # events bracket the steps' device work back to back, not the binding's per-call host
    # overhead (an event between every two steps would add its own cost to each); 4 sweeps
    sweeps = []
    for _ in range(4):
        pkg.compress_kernels(p, s0, k, kern, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        t1 = time.perf_counter()
        ev[0].record(stream)
        all_steps()
        ev[1].record(stream)
        enqueue = time.perf_counter() - t1
        torch.cuda.synchronize()
        sweeps.append(ev[0].elapsed_time(ev[1]) * 1e3 / args.decode_steps)
    # the same steps as separate calls, events between the stages (breakdown; the second of two
    # passes is kept, each interval includes one event's own cost)
    for _ in range(2):
      pkg.compress_kernels(p, s0, k, kern, stream=stream)
      sev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.decode_steps)]
      torch.cuda.synchronize()
      torch.cuda._sleep(SPIN_CYCLES)
      for st in range(args.decode_steps):
        e = sev[st]
        e[0].record(stream)
        pkg.compress_kernels(p, seqs[st], k, kern, prev_kv_len=prevs[st], stream=stream)
        e[1].record(stream)
        pkg.block_scores(p, seqs[st], qs[st], kern, bufs["scores"], stream=stream)
        e[2].record(stream)
        pkg.topk_select(p, seqs[st], bufs["scores"], bufs["idx"], stream=stream)
        e[3].record(stream)
        pkg.sparse_attn_decode(p, seqs[st], qs[st], k, v, bufs["idx"], bufs["out"], bufs["lse"],
                               num_splits=bufs["num_splits"], workspace=bufs["workspace"],
                               stream=stream)
        e[4].record(stream)
      torch.cuda.synchronize()
    stage_us = {n: float(np.mean([sev[st][i].elapsed_time(sev[st][i + 1]) * 1e3
                                  for st in range(args.decode_steps)]))
                for i, n in enumerate(["compress", "scores", "topk", "attention"])}
    # the same steps captured once as a HIP graph (the metadata is read from device memory when
    # the kernels run) and replayed: host-inclusive wall time per step, launch and sync included
    graph_us = None
    if not args.no_decode_graph:
        graph = torch.cuda.CUDAGraph()
        pkg.compress_kernels(p, s0, k, kern, stream=stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            all_steps(on=None)
        graph.replay()
        torch.cuda.synchronize()
        reps = 20
        t2 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - t2) * 1e6 / (reps * args.decode_steps)
        del graph
    # bytes a step must move: the kernel cache read for scoring, the selected K/V blocks, q/out
    kv_len = kv0 + args.decode_steps
    C = np.array([pkg.num_kernels(int(L), p.kernel_size, p.kernel_stride) for L in kv_len])
    bytes_kern = int(C.sum()) * p.num_kv_heads * p.head_dim * 2
    keys = sum(min(int(L), (p.topk - 1) * p.block_size + (int(L) - 1) % p.block_size + 1)
               for L in kv_len)
    bytes_kv = keys * p.num_kv_heads * p.head_dim * 2 * 2
    bytes_q = B * p.num_q_heads * p.head_dim * 2 * 2
    total = bytes_kern + bytes_kv + bytes_q
    us = float(np.median(sweeps))
    out = dict(us_per_step=us, us_per_step_sweeps=[round(x, 2) for x in sweeps],
               us_per_step_wall=wall * 1e6 / args.decode_steps,
               host_enqueue_us_per_step=enqueue * 1e6 / args.decode_steps,
               us_per_step_graph_wall=graph_us,
               gpu_busy_while_enqueueing=bool(enqueue < SPIN_SECONDS), stages_us=stage_us,
               tokens_per_s=B / (us * 1e-6), batch=B, cache_len=int(Lmax),
               steps=args.decode_steps, bytes_per_step=total,
               roofline={"bound": "hbm", "achieved": total / (us * 1e-6) / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": total / (us * 1e-6) / 1e9 / PEAK_HBM_GBS})
    del k, v, kern, bufs
    return out


def cpu_baseline(pre, budget_s: float):
    """The float64 oracle on the host cores: kernel compression, then block scores and top-k
    for every query row of the sequence, then attention (on those indices) for rows spread
    evenly over it until `budget_s` seconds have passed."""
    import multiprocessing as mp
    from oracle import infllm2_oracle as orc
    wl = pre["wl"]
    p = wl.params
    # one GPU's share of the host: at most 16 processes, whatever the machine has
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    L = int(wl.q_len[0])
    sl_q, sl_k = wl.seq_slices(0)
    t0 = time.perf_counter()
    kern = orc.compress_kernels(wl.k[sl_k], p.kernel_size, p.kernel_stride, p.dtype)
    t_comp = time.perf_counter() - t0
    idx = mp.RawArray("i", L * p.num_kv_heads * p.topk)
    global _CPU_STATE
    _CPU_STATE = (wl.q[sl_q], wl.k[sl_k], wl.v[sl_k], p, kern, idx)
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_limit_threads) as pool:
        # every row's indices: chunk c holds rows c, c + n, c + 2n, ... (balanced over positions)
        n_idx = workers * 16
        t1 = time.perf_counter()
        covered = sum(pool.map(_cpu_index_rows, [np.arange(c, L, n_idx) for c in range(n_idx)]))
        t_idx = time.perf_counter() - t1
        # attention on the oracle's own indices for evenly spread rows, within the budget
        n_att = max(1, L // 8)
        t2 = time.perf_counter()
        done = 0
        for res in pool.imap_unordered(_cpu_attention_rows,
                                       (np.arange(c, L, n_att) for c in range(n_att))):
            done += res
            if time.perf_counter() - t2 > budget_s:
                break
        t_att = time.perf_counter() - t2
    per_row = t_att / max(done, 1)
    tok_s = L / (t_comp + t_idx + per_row * L)
    return {"value": tok_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(), "index_rows": int(covered), "attention_rows": int(done),
            "sample": f"{args_workload_name(pre)}: full kernel compression ({t_comp:.1f} s), block "
                      f"scores and top-k for all {covered} of {L} query rows ({t_idx:.1f} s), "
                      f"attention for {done} rows spread evenly over the sequence "
                      f"({t_att:.1f} s); {workers} single-threaded processes, float64 numpy; "
                      f"tokens/s = L / (compression + scores and top-k + L x mean attention "
                      f"time per row)"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def args_workload_name(pre):
    return pre["workload"]


_CPU_STATE = None


def _limit_threads():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_index_rows(rows):
    from oracle import infllm2_oracle as orc
    q, k, v, p, kern, idx = _CPU_STATE
    res = orc.run_sequence(q, k, v, p, rows=rows, kernels=kern, with_attention=False)
    out = np.frombuffer(idx, dtype=np.int32).reshape(-1, p.num_kv_heads, p.topk)
    out[rows] = res.idx
    return len(rows)


def _cpu_attention_rows(rows):
    from oracle import infllm2_oracle as orc
    q, k, v, p, kern, idx = _CPU_STATE
    sel = np.frombuffer(idx, dtype=np.int32).reshape(-1, p.num_kv_heads, p.topk)[rows]
    orc.sparse_attention(np.asarray(q[rows], dtype=np.float64), rows, k, v, sel, p)
    return len(rows)


def _short(name: str) -> str:
    name = name.replace("infllm2::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
    cut = name.find("(")
    head = name[:cut] if cut > 0 else name
    if head.startswith("void "):
        head = head[5:]
    return head[:90]


def _csv_rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def summarize_counters(dirs, kernels=("attn_tile", "attn_decode", "decode_scores", "scores_mfma",
                                      "scores_decode", "topk_kernel", "topk_wide", "compress_kernel")):
    """Per-kernel totals of every counter in one or more rocprofv3 --pmc runs (sums over the
    kernel's dispatches), one table per run, plus derived ratios where their counters are
    present.  GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the MFMA busy fraction is
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 4 SIMDs x compute units)."""
    cus = 256
    for directory in dirs:
        tot, disp = {}, {}
        for r in _csv_rows(directory, "counter_collection.csv"):
            k = _short(r["Kernel_Name"])
            if not any(k.startswith(n) for n in kernels):
                continue
            d = tot.setdefault(k, {})
            c = r["Counter_Name"]
            c = c[:-4] if c.endswith("_sum") else c
            d[c] = d.get(c, 0.0) + float(r["Counter_Value"])
            disp.setdefault(k, set()).add(r["Dispatch_Id"])
        names = sorted({c for d in tot.values() for c in d})
        print(f"run `{os.path.basename(os.path.normpath(directory))}`\n")
        print("| kernel | dispatches | " + " | ".join(names) + " |")
        print("|---|---:|" + "---:|" * len(names))
        for k, d in sorted(tot.items()):
            print(f"| `{k}` | {len(disp[k])} | " +
                  " | ".join(f"{d.get(c, 0.0):.4g}" for c in names) + " |")
        print()
        for k, d in sorted(tot.items()):
            parts = []
            g = d.get("GRBM_GUI_ACTIVE")
            if g and "SQ_VALU_MFMA_BUSY_CYCLES" in d:
                parts.append(f"MFMA busy {d['SQ_VALU_MFMA_BUSY_CYCLES'] / (g / 8 * 4 * cus):.3f}")
            if "SQ_LDS_BANK_CONFLICT" in d and d.get("SQ_LDS_IDX_ACTIVE"):
                parts.append(f"LDS bank-conflict cycles / LDS active {d['SQ_LDS_BANK_CONFLICT'] / d['SQ_LDS_IDX_ACTIVE']:.4f}")
            if "SQ_WAIT_INST_ANY" in d and d.get("SQ_WAVE_CYCLES"):
                parts.append(f"waiting / wave cycles {d['SQ_WAIT_INST_ANY'] / d['SQ_WAVE_CYCLES']:.3f}")
            if d.get("SQ_INSTS_MFMA") and "SQ_INSTS_LDS" in d:
                parts.append(f"LDS instructions per MFMA {d['SQ_INSTS_LDS'] / d['SQ_INSTS_MFMA']:.2f}")
            if d.get("SQ_INSTS_MFMA") and "SQ_INSTS_SALU" in d:
                parts.append(f"SALU instructions per MFMA {d['SQ_INSTS_SALU'] / d['SQ_INSTS_MFMA']:.2f}")
            # request sizes as the streaming copy kernel shows them on this GPU: 128-byte reads
            # (none of 32 bytes), 64-byte writes
            if "TCC_EA0_RDREQ_32B" in d and "TCC_EA0_RDREQ" in d:
                rd = (d["TCC_EA0_RDREQ"] - d["TCC_EA0_RDREQ_32B"]) * 128 + d["TCC_EA0_RDREQ_32B"] * 32
                parts.append(f"EA reads {d['TCC_EA0_RDREQ']:.4g} requests = {rd / 2**20:.1f} MiB at 128 B")
            if "TCC_EA0_WRREQ_64B" in d and "TCC_EA0_WRREQ" in d:
                wr = d["TCC_EA0_WRREQ_64B"] * 64 + (d["TCC_EA0_WRREQ"] - d["TCC_EA0_WRREQ_64B"]) * 32
                parts.append(f"EA writes {wr / 2**20:.1f} MiB at 64 B")
            if parts:
                print(f"- `{k}`: " + "; ".join(parts))
        print()


def summarize_profile(argv):
    """Markdown summary of rocprofv3 output (kernel statistics, or per-kernel HBM traffic from
    a FETCH_SIZE run and a WRITE_SIZE run scaled by the copy-calibration kernel)."""
    if argv[0] == "stats":
        rows = _csv_rows(argv[1], "kernel_stats.csv")
        print("| kernel | calls | total ms | avg us | min us | max us | % |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for r in rows[:20]:
            print(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} "
                  f"| {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} "
                  f"| {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
        return
    if argv[0] == "counters":
        summarize_counters(argv[1:])
        return
    if argv[0] != "traffic" or len(argv) != 5:
        raise SystemExit("usage: --summarize-profile traffic FETCH_DIR WRITE_DIR WORKLOAD MIB")
    fetch_dir, write_dir, workload, mib = argv[1], argv[2], argv[3], int(argv[4])
    per = {}
    for key, directory, counter in (("fetch", fetch_dir, "FETCH_SIZE"),
                                    ("write", write_dir, "WRITE_SIZE")):
        for r in _csv_rows(directory, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            k = _short(r["Kernel_Name"])
            d = per.setdefault(k, {"fetch": [], "write": []})
            d[key].append(float(r["Counter_Value"]) * 1024.0)      # counters are in KiB
    copy = [k for k in per if "neg_kernel" in k]
    if not copy:
        raise SystemExit("no copy-calibration kernel in the counter output")
    known = float(mib << 20)
    cf = per[copy[0]]
    f_fetch = known / cf["fetch"][-1]
    f_write = known / cf["write"][-1]
    print(f"copy calibration kernel `{copy[0]}`: {mib} MiB read and written; FETCH_SIZE read "
          f"{cf['fetch'][-1] / 2**20:.1f} MiB (factor {f_fetch:.4f}), WRITE_SIZE "
          f"{cf['write'][-1] / 2**20:.1f} MiB (factor {f_write:.4f})\n")
    print("| kernel | dispatches | FETCH MiB (scaled) | WRITE MiB (scaled) |")
    print("|---|---:|---:|---:|")
    for k, d in sorted(per.items(), key=lambda kv: -sum(kv[1]["fetch"])):
        print(f"| `{k}` | {len(d['fetch'])} | {sum(d['fetch']) * f_fetch / 2**20:.1f} "
              f"| {sum(d['write']) * f_write / 2**20:.1f} |")
    print()
    for role, (match, sources) in TRAFFIC_ROLES.items():
        found = [k for k in per if match(k)]
        if not found:
            continue
        d = per[found[0]]
        rec = {"role": role, "kernel": found[0], "workload": workload,
               "source_sha256": source_digest(sources),
               "fetch_bytes_per_call": sum(d["fetch"]) * f_fetch,
               "write_bytes_per_call": sum(d["write"]) * f_write,
               "dispatches_per_call": len(d["fetch"])}
        print("bench-data: " + json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill128k", choices=["prefill128k", "prefill32k", "varlen"])
    ap.add_argument("--decode-steps", type=int, default=16)
    ap.add_argument("--decode-splits", type=int, default=0)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-graph", action="store_true",
                    help="skip the decode leg's graph replay (counter runs)")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-window", action="store_true")
    ap.add_argument("--no-score-mode1", action="store_true")
    ap.add_argument("--no-chunk", action="store_true")
    ap.add_argument("--no-other-prefills", action="store_true",
                    help="skip the 32K and varlen prefill legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the streaming-copy and GEMM rate measurements")
    ap.add_argument("--cpu-budget", type=float, default=8.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a streaming copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-profile", nargs="+", metavar="ARG",
                    help="stats DIR | traffic FETCH_DIR WRITE_DIR WORKLOAD MIB | counters DIR...: "
                         "print a summary of rocprofv3 csv output and exit (the traffic runs must "
                         "time one step with no warmup and --copy-calibration MIB)")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_long_semantic_amd as pkg
    import synth
    torch.cuda.set_device(0)
    pre = run_prefill(args, torch, pkg, synth)
    p = pre["p"]
    st = pre["stage"]
    log(f"prefill stages ms: {st}")
    line = {
        "metric": METRIC,
        "value": pre["tokens"] / (pre["ms_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": pre["workload"], "seq_lens": pre["seq_lens"],
                   "num_q_heads": p.num_q_heads, "num_kv_heads": p.num_kv_heads,
                   "head_dim": p.head_dim, "block_size": p.block_size,
                   "kernel_size": p.kernel_size, "kernel_stride": p.kernel_stride,
                   "topk": p.topk, "init_blocks": p.num_init_blocks,
                   "local_blocks": p.num_local_blocks},
        "stages_ms": st,
        "stages_gbs": pre["stage_gbs"],
        "attention_tokens_per_s": pre["tokens"] / (st["attention"] * 1e-3),
        "roofline": {"kernel": "attn_tile (sparse_attn_prefill)", "bound": "mfma",
                     "achieved": pre["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": pre["tflops"] / PEAK_BF16_TFLOPS, "traffic": None,
                     "flops_per_call": pre["flops"], "keys_per_head": pre["keys"],
                     "launches_per_call": pre["launches"],
                     "avg_launch_us": st["attention"] * 1e3 / pre["launches"]},
    }
    line["roofline"]["gather"] = pre["gather"]
    tr = measured_traffic(pre["workload"])
    if tr is not None:
        line["roofline"]["traffic"] = tr["fetch_bytes_per_call"] + tr["write_bytes_per_call"]
        line["roofline"]["traffic_split"] = {"fetch": tr["fetch_bytes_per_call"],
                                             "write": tr["write_bytes_per_call"],
                                             "unit": "bytes per call"}
    if not args.no_other_prefills:
        for name in ("prefill32k", "varlen"):
            if name != pre["workload"]:
                line[name] = prefill_leg(args, torch, pkg, synth, name)
                log(f"{name}: {line[name]['ms_per_step']:.2f} ms per step, attention "
                    f"{line[name]['roofline']['frac']:.3f} of bf16 peak")
    if not args.no_chunk:
        line["chunk"] = run_chunk(args, torch, pkg, pre)
        log(f"chunk: {line['chunk']['ms_per_chunk']:.2f} ms per {line['chunk']['chunk_tokens']} tokens")
    if not args.no_score_mode1:
        line["score_mode1"] = run_score_mode1(args, torch, pkg, pre)
        log(f"score mode 1: {line['score_mode1']['ms_per_call']:.2f} ms/call")
    if not args.no_window:
        line["window"] = run_window(args, torch, pkg, pre)
        log(f"window: {line['window']['ms_per_call']:.2f} ms/call")
    if not args.no_backward:
        line["backward"] = run_backward(args, torch, pkg, synth, pre)
        log(f"backward: {line['backward']['ms_per_call']:.2f} ms/call")
    if not args.no_decode:
        line["decode"] = run_decode(args, torch, pkg, synth)
        log(f"decode: {line['decode']['us_per_step']:.1f} us/step")
    if not args.no_peaks:
        line["measured_peaks"] = measured_peaks(torch)
        mp = line["measured_peaks"]
        log(f"measured peaks: stream {mp['hbm_stream_gbs']:.0f} GB/s, bf16 GEMM "
            f"{mp['bf16_gemm_tflops']:.0f} TFLOP/s")
    if not args.no_cpu_baseline:
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline(pre, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
