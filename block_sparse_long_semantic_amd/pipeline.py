"""Whole passes of the hot path: the library's five calls chained on one stream.

prefill:     compress_kernels -> block_scores -> topk_select -> sparse_attn_prefill
decode_step: compress_kernels (incremental) -> block_scores -> topk_select
             -> sparse_attn_decode
Buffers are torch tensors; pass `bufs` from a previous call to reuse them.  The sequence
metadata reaches the library as device arrays (Seqs copies them once per device).
"""
from __future__ import annotations

from typing import Dict, Optional

from ._lib import (BF16, Params, Seqs, block_scores, compress_kernels, decode_step_fused,
                   decode_workspace_size, sparse_attn_decode, sparse_attn_prefill, topk_select)


def num_kernels(length: int, kernel_size: int, kernel_stride: int) -> int:
    return 0 if length < kernel_size else (length - kernel_size) // kernel_stride + 1


def _dtype(p: Params):
    import torch
    return torch.bfloat16 if p.dtype == BF16 else torch.float32


def reachable_blocks(p: Params, seqs: Seqs) -> int:
    """Blocks a query of these sequences may reach: the library's bound ceil(max_kv_len / B),
    the score buffers' least row stride."""
    return (seqs.max_kv_len + p.block_size - 1) // p.block_size


def prefill_buffers(params, seqs: Seqs, q, kv_rows_kernels: int) -> Dict[str, object]:
    import torch
    p = Params.from_any(params)
    dev = q.device
    rows = q.shape[0]
    nb = max(1, reachable_blocks(p, seqs))
    return dict(
        kernels=torch.empty((max(1, kv_rows_kernels), p.num_kv_heads, p.head_dim),
                            dtype=_dtype(p), device=dev),
        scores=torch.empty((rows, p.num_kv_heads, nb), dtype=torch.float32, device=dev),
        idx=torch.empty((rows, p.num_kv_heads, p.topk), dtype=torch.int32, device=dev),
        out=torch.empty_like(q),
        lse=torch.empty((rows, p.num_q_heads), dtype=torch.float32, device=dev),
    )


def prefill(params, seqs: Seqs, q, k, v, bufs: Optional[Dict[str, object]] = None,
            stream=None) -> Dict[str, object]:
    p = Params.from_any(params)
    if seqs.kc_start is None:
        raise ValueError("seqs.kc_start is required")
    if bufs is None:
        kc_rows = int(max(int(seqs.kc_start[b]) + num_kernels(int(seqs.kv_len[b]), p.kernel_size,
                                                               p.kernel_stride)
                          for b in range(seqs.num_seqs)))
        bufs = prefill_buffers(p, seqs, q, kc_rows)
    compress_kernels(p, seqs, k, bufs["kernels"], stream=stream)
    block_scores(p, seqs, q, bufs["kernels"], bufs["scores"], stream=stream)
    topk_select(p, seqs, bufs["scores"], bufs["idx"], stream=stream)
    sparse_attn_prefill(p, seqs, q, k, v, bufs["idx"], bufs["out"], bufs["lse"], stream=stream)
    return bufs


def decode_buffers(params, batch: int, num_blocks: int, num_splits: int, device):
    import torch
    p = Params.from_any(params)
    ws = decode_workspace_size(p, batch, num_splits)
    return dict(
        scores=torch.empty((batch, p.num_kv_heads, num_blocks), dtype=torch.float32,
                           device=device),
        idx=torch.empty((batch, p.num_kv_heads, p.topk), dtype=torch.int32, device=device),
        out=torch.empty((batch, p.num_q_heads, p.head_dim), dtype=_dtype(p), device=device),
        lse=torch.empty((batch, p.num_q_heads), dtype=torch.float32, device=device),
        # partials + completion counters; must start zero-filled (calls leave it zeroed)
        workspace=torch.zeros((max(1, ws // 4),), dtype=torch.float32, device=device),
        num_splits=num_splits,
    )


def decode_step(params, seqs: Seqs, q, k_cache, v_cache, kernels_cache, prev_kv_len,
                bufs: Dict[str, object], stream=None) -> Dict[str, object]:
    """One decode step for a batch: q [batch, Hq, d]; caches [batch*max_len, Hkv, d] (padded);
    kernels_cache [batch*max_kernels, Hkv, d]; seqs from Seqs.decode(kv_len, ...), where kv_len
    already counts the new token.  prev_kv_len: lengths when kernels_cache was last updated."""
    decode_step_fused(params, seqs, q, k_cache, v_cache, kernels_cache, prev_kv_len,
                      bufs["scores"], bufs["idx"], bufs["out"], bufs["lse"], bufs["workspace"],
                      num_splits=bufs["num_splits"], stream=stream)
    return bufs


def decode_step_staged(params, seqs: Seqs, q, k_cache, v_cache, kernels_cache, prev_kv_len,
                       bufs: Dict[str, object], stream=None) -> Dict[str, object]:
    """The same step as four separate library calls."""
    p = Params.from_any(params)
    compress_kernels(p, seqs, k_cache, kernels_cache, prev_kv_len=prev_kv_len, stream=stream)
    block_scores(p, seqs, q, kernels_cache, bufs["scores"], stream=stream)
    topk_select(p, seqs, bufs["scores"], bufs["idx"], stream=stream)
    sparse_attn_decode(p, seqs, q, k_cache, v_cache, bufs["idx"], bufs["out"], bufs["lse"],
                       num_splits=bufs["num_splits"], workspace=bufs["workspace"], stream=stream)
    return bufs
