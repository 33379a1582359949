"""The allocation-free decoding step (infllm2_decode_step_noalloc, its workspace a buffer the
library keeps in device memory) against the step with a caller-given workspace
(infllm2_decode_step): two calls in a row, the second on a smaller batch, each equal to the
workspace step (indices and scores bit for bit, outputs to float32 rounding) and checked against
the oracle; the library's buffer is left with its counters zero."""
import numpy as np
import pytest
import torch

import synth
from oracle import infllm2_oracle as orc
from tests._gpu import dev, host, log
from tests.test_gpu_parity import check_decode_seq

import block_sparse_long_semantic_amd as lib

pytestmark = pytest.mark.gpu


def one_call(p, B, Lmax, kv0, seed, label):
    wl = synth.make_decode(label, p, batch=B, max_len=Lmax, steps=1, seed=seed, kv_len0=kv0)
    Ck = orc.num_kernels(Lmax, p.kernel_size, p.kernel_stride)
    k = dev(wl.k.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    v = dev(wl.v.reshape(B * Lmax, p.num_kv_heads, p.head_dim), p.dtype)
    kv = wl.kv_len0.astype(np.int64) + 1
    seqs = lib.Seqs.decode(kv, Lmax, Ck)
    q = dev(wl.q_steps[0], p.dtype)
    nb = (Lmax + p.block_size - 1) // p.block_size
    res = {}
    for name in ("workspace", "noalloc"):
        kern = torch.zeros((B * Ck, p.num_kv_heads, p.head_dim), dtype=k.dtype, device="cuda")
        bufs = lib.pipeline.decode_buffers(p, B, nb, 0, "cuda")
        for key in ("scores", "out", "lse"):
            bufs[key].fill_(float("nan"))
        bufs["idx"].fill_(-7)
        log(f"case {label} {name}")
        if name == "workspace":
            lib.decode_step(p, seqs, q, k, v, kern, None, bufs)
        else:
            lib.decode_step_noalloc(p, seqs, q, k, v, kern, None, bufs["scores"], bufs["idx"],
                                    bufs["out"], bufs["lse"])
        torch.cuda.synchronize()
        res[name] = {n: host(bufs[n]) for n in ("scores", "idx", "out", "lse")}
        res[name]["kernels"] = host(kern)
    a, b = res["workspace"], res["noalloc"]
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["kernels"], b["kernels"])
    for r in range(B):
        nbr = int(kv[r] - 1) // p.block_size + 1
        assert np.array_equal(a["scores"][r, :, :nbr], b["scores"][r, :, :nbr])
    assert np.abs(a["out"] - b["out"]).max() <= 1e-2
    assert np.abs(a["lse"] - b["lse"]).max() <= 1e-4
    for r in range(B):
        L = int(kv[r])
        check_decode_seq(p, wl.k[r, :L], wl.v[r, :L], wl.q_steps[0][r:r + 1],
                         b["kernels"][r * Ck:(r + 1) * Ck], b["scores"][r:r + 1],
                         b["idx"][r:r + 1], b["out"][r:r + 1], b["lse"][r:r + 1],
                         f"{label} seq {r}")


def test_noalloc_step_equals_workspace_step_twice():
    p = synth.config_params("decode128k")
    one_call(p, 6, 8192, [8000, 6000, 4100, 2000, 700, 64], 71, "noalloc-first")
    one_call(p, 2, 3000, [2990, 1500], 72, "noalloc-second")


def test_noalloc_step_rejects_oversized_workspace():
    p = synth.config_params("decode128k")
    B, Lmax = 700, 128
    seqs = lib.Seqs.decode(np.full(B, 100), Lmax, 5)
    k = torch.zeros((B * Lmax, p.num_kv_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    kern = torch.zeros((B * 5, p.num_kv_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((B, p.num_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    bufs = lib.pipeline.decode_buffers(p, B, 2, 0, "cuda")
    with pytest.raises(lib.InfLLM2Error) as e:
        lib.decode_step_noalloc(p, seqs, q, k, k, kern, None, bufs["scores"], bufs["idx"],
                                bufs["out"], bufs["lse"])
    assert e.value.status == 5 and "static buffer" in str(e.value)
