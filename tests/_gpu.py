"""Helpers for the GPU tests: move seeded workloads to the device and run the HIP path
through the C ABI (via the thin binding), returning host arrays."""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import block_sparse_long_semantic_amd as lib
from block_sparse_long_semantic_amd.pipeline import num_kernels, reachable_blocks


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def kc_starts(kv_len: Sequence[int], p) -> np.ndarray:
    nk = [num_kernels(int(L), p.kernel_size, p.kernel_stride) for L in kv_len]
    return np.concatenate([[0], np.cumsum(nk)[:-1]]).astype(np.int64), int(sum(nk))


def seqs_for(wl, p) -> lib.Seqs:
    kc, _ = kc_starts(wl.kv_len, p)
    return lib.Seqs(wl.q_start, wl.q_len, wl.q_pos0, wl.kv_start, wl.kv_len, kc)


def run_prefill_stages(wl, seqs: Optional[lib.Seqs] = None, q_rows: Optional[np.ndarray] = None
                       ) -> Dict[str, np.ndarray]:
    """Run the four prefill calls on the workload (optionally with other query metadata)."""
    p = wl.params
    seqs = seqs if seqs is not None else seqs_for(wl, p)
    q = dev(wl.q if q_rows is None else q_rows, p.dtype)
    k = dev(wl.k, p.dtype)
    v = dev(wl.v, p.dtype)
    _, kc_total = kc_starts(seqs.kv_len, p)
    bufs = lib.pipeline.prefill_buffers(p, seqs, q, kc_total)
    lib.prefill(p, seqs, q, k, v, bufs=bufs)
    torch.cuda.synchronize()
    res = {name: host(t) for name, t in bufs.items()}
    del q, k, v, bufs
    return res
