"""Host-side logic of bench.py (no GPU): the prefill gather accounting, the refusal of more
than one GPU, and the rocprofv3 counter summary with its copy calibration."""
import json
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_gather_bound_counts_tile_unions():
    # 24-token tiles: 30 rows are a full tile and a ragged one of 6; 2 KV heads, top-4
    idx = np.full((30, 2, 4), -1, np.int32)
    idx[:24, 0, :] = [0, 1, 2, 3]          # 24 tokens share 4 blocks
    idx[:24, 1, :2] = [5, 6]               # 24 tokens share 2 blocks
    idx[3, 1, 2] = 9                       # one token adds a block of its own
    idx[20, 0, :1] = 8                     # rows 20 and 25 share block 8 across the tile edge:
    idx[25, 0, :1] = 8                     # staged once per tile, twice in all
    idx[24:, 1, :1] = 7                    # ragged tile: 6 tokens, 1 block
    p = types.SimpleNamespace(block_size=64, head_dim=128, num_q_heads=32, num_kv_heads=2)
    g = bench.gather_bound(p, idx, [30], 1e9, 2.0, 24)
    blk = 2 * 64 * 128 * 2
    selected = 23 * 4 + 1 * 4 + 24 * 2 + 1 + 1 + 6
    assert g["selected_bytes"] == selected * blk
    # tile 0: head 0 {0,1,2,3,8}, head 1 {5,6,9}; tile 1: head 0 {8}, head 1 {7}
    assert g["staged_bytes"] == (5 + 3 + 1 + 1) * blk
    assert abs(g["reuse_tokens_per_staged_block"] - selected / 10) < 1e-12
    assert abs(g["staging_rate_gbs"] - 10 * blk / 2e-3 / 1e9) < 1e-9


def test_gather_bound_packed_sequences_tile_separately():
    # two sequences of 16 rows each selecting the same block: tiles do not straddle sequences
    # (one 24-token tile each)
    idx = np.zeros((32, 1, 1), np.int32)
    p = types.SimpleNamespace(block_size=64, head_dim=64, num_q_heads=16, num_kv_heads=1)
    g = bench.gather_bound(p, idx, [16, 16], 1.0, 1.0, 24)
    assert g["staged_bytes"] == 2 * (2 * 64 * 64 * 2)


def test_gather_bound_uses_32_token_tiles_at_group_8():
    # groups of 8 heads run 32-token tiles: 40 rows are a full tile and a ragged one of 8
    idx = np.full((40, 1, 2), -1, np.int32)
    idx[:16, 0, 0] = 1                     # first half of tile 0
    idx[16:32, 0, 0] = 2                   # second half of tile 0
    idx[32:, 0, 0] = 1                     # the ragged tile
    p = types.SimpleNamespace(block_size=64, head_dim=128, num_q_heads=16, num_kv_heads=2)
    assert bench.tile_tokens(p) == 32
    assert bench.tile_tokens(types.SimpleNamespace(head_dim=64, num_q_heads=16, num_kv_heads=2)) == 64
    g = bench.gather_bound(p, idx, [40], 1.0, 1.0, 32)
    assert g["staged_bytes"] == 3 * (2 * 64 * 128 * 2)


def test_tile_tokens_at_groups_of_16():
    # groups of 16: 24-token tiles (3 per wave) at every length
    p = types.SimpleNamespace(num_q_heads=32, num_kv_heads=2, head_dim=128)
    assert bench.tile_tokens(p) == 24
    assert bench.tile_tokens(types.SimpleNamespace(num_q_heads=32, num_kv_heads=2, head_dim=64)) == 24


def test_launches_cover_the_group_bound():
    # rounds of 8 groups of 32 tiles, three rounds per launch: 128K at 24 tokens has 171 groups
    # per KV head (43 rounds, 15 launches); the varlen batch's bound is 72 groups (3 launches)
    assert bench._group_bound([131072], 24, 32, 2) == 342
    assert -(-bench._group_bound([131072], 24, 32, 2) // (8 * bench.ROUNDS_PER_LAUNCH)) == 15
    assert bench._group_bound([8192, 16384, 32768, 8192], 64, 32, 2) == 72


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_scales_by_copy_calibration(tmp_path, capsys):
    # FETCH_SIZE and WRITE_SIZE in KiB per dispatch; the copy kernel over 1 MiB reads 512 KiB
    # by the counter (factor 2) and writes 1024 KiB (factor 1)
    fwd_name = "void infllm2::(anonymous namespace)::attn_tile<128, 16, 4, 8, 2, false, false>(int)"
    rows = [(fwd_name, 1000.0, 10.0), (fwd_name, 500.0, 5.0),
            ("at::native::vectorized_elementwise_kernel<8, at::native::neg_kernel_cuda>(int)",
             512.0, 1024.0)]
    for d, counter, col in (("f", "FETCH_SIZE", 1), ("w", "WRITE_SIZE", 2)):
        os.makedirs(tmp_path / d)
        with open(tmp_path / d / "x_counter_collection.csv", "w") as f:
            f.write("Kernel_Name,Counter_Name,Counter_Value\n")
            for r in rows:
                f.write(f'"{r[0]}",{counter},{r[col]}\n')
    bench.summarize_profile(["traffic", str(tmp_path / "f"), str(tmp_path / "w"), "tiny", "1"])
    out = capsys.readouterr().out
    assert "factor 2.0000" in out and "factor 1.0000" in out
    line = [ln for ln in out.splitlines()
            if ln.startswith("| `attn_tile<128, 16, 4, 8, 2, false, false>` |")][0]
    cells = [c.strip() for c in line.split("|")]
    # MiB with one decimal: 1500 KiB x 2 fetched, 15 KiB written
    assert cells[2] == "2" and cells[3] == f"{1500.0 * 2 / 1024:.1f}" and cells[4] == f"{15.0 / 1024:.1f}"
    recs = [json.loads(ln[len("bench-data: "):]) for ln in out.splitlines()
            if ln.startswith("bench-data: ")]
    fwd = [r for r in recs if r["role"] == "prefill_attention"]
    assert fwd and fwd[0]["fetch_bytes_per_call"] == 1500.0 * 1024 * 2


def test_group_bound_covers_every_group():
    # the launches cover a host bound on the tile groups computed from the metadata's bounds only
    # (sequences, longest run, total rows); it must never fall below the true count, or tiles
    # would be skipped
    rng = np.random.default_rng(7)
    for _ in range(500):
        n = int(rng.integers(1, 40))
        lens = [int(x) for x in rng.integers(1, 5000, n)]
        rows, gs, hkv = int(rng.choice([16, 24, 32, 64])), int(rng.choice([1, 8, 32])), int(rng.integers(1, 5))
        actual = sum(-(-(-(-L // rows)) // gs) for L in lens) * hkv
        assert bench._group_bound(lens, rows, gs, hkv) >= actual
