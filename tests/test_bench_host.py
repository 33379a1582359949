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
    # sequence of 20 rows (a full 16-row tile and a ragged one of 4), 2 KV heads, top-4
    idx = np.full((20, 2, 4), -1, np.int32)
    idx[:16, 0, :] = [0, 1, 2, 3]          # 16 tokens share 4 blocks
    idx[:16, 1, :2] = [5, 6]               # 16 tokens share 2 blocks
    idx[3, 1, 2] = 9                       # one token adds a block of its own
    idx[16:, 0, :1] = 7                    # ragged tile: 4 tokens, 1 block
    p = types.SimpleNamespace(block_size=64, head_dim=128)
    g = bench.gather_bound(p, idx, [20], 1e9, 2.0)
    blk = 2 * 64 * 128 * 2
    assert g["selected_bytes"] == (16 * 4 + 16 * 2 + 1 + 4) * blk
    assert g["staged_bytes"] == (4 + 3 + 1) * blk
    assert abs(g["reuse_tokens_per_staged_block"] - 101 / 8) < 1e-12
    assert abs(g["staging_rate_gbs"] - 8 * blk / 2e-3 / 1e9) < 1e-9


def test_gather_bound_packed_sequences_tile_separately():
    # two sequences of 16 rows each selecting the same block: tiles do not straddle sequences
    idx = np.zeros((32, 1, 1), np.int32)
    p = types.SimpleNamespace(block_size=64, head_dim=64)
    g = bench.gather_bound(p, idx, [16, 16], 1.0, 1.0)
    assert g["staged_bytes"] == 2 * (2 * 64 * 64 * 2)


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
