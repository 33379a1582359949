"""Seeded synthetic workloads for the InfLLM v2 block-sparse attention hot path.

This module only draws inputs: queries, keys, values, sequence metadata and planted
"needle" structure.  It holds none of the method's arithmetic (no pooling, scoring,
selection or attention), so both the CPU oracle and the GPU path may use it.

Workloads follow the shapes of the MiniCPM4 InfLLM v2 description (MiniCPM4 paper summary,
section 2.1; MiniCPM4-8B model card, "Efficient Model Architecture"): a MiniCPM4-8B-shaped
layer (32 query heads sharing 2 KV heads, head_dim 128), 64-token KV blocks, semantic
kernels of 32 tokens at stride 16.  The pages do not list these constants; they are the
configuration this library is measured on.

Values are drawn as float32 normals with numpy's PCG64 generator and, for bf16 workloads,
rounded to the nearest bf16 value (ties to even) so that the oracle (which reads them as
float64) and the GPU (which reads them as bf16) consume identical numbers.  Arrays are kept
as float32 holding bf16-representable values.

Needles stand in for a needle-in-a-haystack benchmark (the paper summary's long-context
evaluation, section 5.3): some KV blocks get keys aligned with a random unit direction and a
random subset of later queries in the same GQA group gets that direction added, so those
queries should select those blocks.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Params", "Workload", "DecodeWorkload", "Needle", "round_to_bf16", "make",
    "make_prefill", "make_decode", "CONFIG_NAMES", "config_params", "make_upstream_grad",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    u = x.view(np.uint32)                       # finite values: u + bias stays below 2^32
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    u += bias
    u &= np.uint32(0xFFFF0000)
    return x


@dataclass(frozen=True)
class Params:
    """Shape and method constants of one attention layer."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int = 64
    kernel_size: int = 32
    kernel_stride: int = 16
    topk: int = 96
    num_init_blocks: int = 1
    num_local_blocks: int = 2
    dtype: str = "bf16"          # "bf16" or "f32"
    softmax_scale: float = 0.0   # <= 0 means 1/sqrt(head_dim)
    score_mode: int = 0          # 0: group sum of scaled dot products; 1: of per-head softmaxes

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)


@dataclass
class Needle:
    seq: int
    kv_head: int
    block: int
    query_positions: np.ndarray   # positions (within the sequence) that got the direction


@dataclass
class Workload:
    """A packed (variable-length) prefill batch.

    q: [T, Hq, d], k/v: [Tkv, Hkv, d] float32 arrays (bf16-representable for bf16).
    Sequence b owns query rows [q_start[b], q_start[b]+q_len[b]) at positions
    q_pos0[b] + j, and key rows [kv_start[b], kv_start[b]+kv_len[b]).
    """
    name: str
    params: Params
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_start: np.ndarray
    q_len: np.ndarray
    q_pos0: np.ndarray
    kv_start: np.ndarray
    kv_len: np.ndarray
    needles: List[Needle] = field(default_factory=list)

    @property
    def num_seqs(self) -> int:
        return int(len(self.q_len))

    def seq_slices(self, b: int) -> Tuple[slice, slice]:
        qs = int(self.q_start[b]); ks = int(self.kv_start[b])
        return slice(qs, qs + int(self.q_len[b])), slice(ks, ks + int(self.kv_len[b]))


@dataclass
class DecodeWorkload:
    """A batch of sequences decoding against a padded KV cache.

    k/v: [batch, Lmax, Hkv, d]; q_steps: [steps, batch, Hq, d].  At step t every sequence b
    holds kv_len0[b] + t + 1 tokens (the new token's K/V is already in the cache) and
    queries at position kv_len0[b] + t.
    """
    name: str
    params: Params
    k: np.ndarray
    v: np.ndarray
    q_steps: np.ndarray
    kv_len0: np.ndarray

    @property
    def batch(self) -> int:
        return int(self.k.shape[0])

    @property
    def max_len(self) -> int:
        return int(self.k.shape[1])


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _plant_needles(rng, p: Params, q, k, q_start, kv_start, lens, n_needles: int,
                   queries_per_needle: int = 64) -> List[Needle]:
    """Give some KV blocks keys along a random unit direction u (sqrt(d)*u + 0.25*noise) and add
    4*u to every head of the owning group at random later query positions."""
    needles: List[Needle] = []
    if n_needles <= 0:
        return needles
    B, d, G = p.block_size, p.head_dim, p.group
    for b_seq, L in enumerate(lens):
        nb = -(-int(L) // B)
        hi = nb - 8
        if hi <= 1:
            continue
        blocks = rng.choice(np.arange(1, hi), size=min(n_needles, hi - 1), replace=False)
        for blk in blocks:
            for g in range(p.num_kv_heads):
                u = rng.standard_normal(d).astype(np.float64)
                u /= np.linalg.norm(u)
                noise = rng.standard_normal((B, d)).astype(np.float64)
                t0 = int(kv_start[b_seq]) + int(blk) * B
                k[t0:t0 + B, g, :] = (math.sqrt(d) * u[None, :] + 0.25 * noise).astype(np.float32)
                lo = B * (int(blk) + p.num_local_blocks + 1)
                npos = min(queries_per_needle, int(L) - lo)
                if npos <= 0:
                    continue
                pos = np.sort(rng.choice(np.arange(lo, int(L)), size=npos, replace=False))
                rows = int(q_start[b_seq]) + pos
                q[rows, g * G:(g + 1) * G, :] += (4.0 * u).astype(np.float32)[None, None, :]
                needles.append(Needle(b_seq, g, int(blk), pos))
    return needles


def make_prefill(name: str, params: Params, seq_lens: Sequence[int], seed: int,
                 needles_per_seq: int = 0, student_t_keys: bool = False) -> Workload:
    """Packed causal prefill: every sequence's queries are its own tokens (q_pos0 = 0)."""
    p = params
    lens = np.asarray(seq_lens, dtype=np.int64)
    T = int(lens.sum())
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rng = np.random.default_rng(seed)
    q = _normal(rng, (T, p.num_q_heads, p.head_dim))
    k = _normal(rng, (T, p.num_kv_heads, p.head_dim))
    v = _normal(rng, (T, p.num_kv_heads, p.head_dim))
    if student_t_keys:
        tau = rng.standard_t(3.0, size=(T, p.num_kv_heads)).astype(np.float32)
        k *= np.abs(tau)[:, :, None]
    needles = _plant_needles(rng, p, q, k, starts, starts, lens, needles_per_seq)
    return Workload(
        name=name, params=p,
        q=_finish(q, p.dtype), k=_finish(k, p.dtype), v=_finish(v, p.dtype),
        q_start=starts.copy(), q_len=lens.astype(np.int32), q_pos0=np.zeros(len(lens), np.int32),
        kv_start=starts.copy(), kv_len=lens.astype(np.int32), needles=needles)


def make_decode(name: str, params: Params, batch: int, max_len: int, steps: int, seed: int,
                kv_len0: Optional[Sequence[int]] = None) -> DecodeWorkload:
    """Decode batch: caches of max_len tokens (all drawn), `steps` new query tokens each."""
    p = params
    rng = np.random.default_rng(seed)
    q = _normal(rng, (steps, batch, p.num_q_heads, p.head_dim))
    k = _normal(rng, (batch, max_len, p.num_kv_heads, p.head_dim))
    v = _normal(rng, (batch, max_len, p.num_kv_heads, p.head_dim))
    if kv_len0 is None:
        kv_len0 = [max_len - steps] * batch
    kv_len0 = np.asarray(kv_len0, dtype=np.int32)
    if np.any(kv_len0 + steps > max_len) or np.any(kv_len0 < 0):
        raise ValueError("decode steps run past the cache")
    return DecodeWorkload(name=name, params=p, k=_finish(k, p.dtype), v=_finish(v, p.dtype),
                          q_steps=_finish(q, p.dtype), kv_len0=kv_len0)


def make_upstream_grad(shape, seed: int, dtype: str = "bf16") -> np.ndarray:
    """Upstream gradient of the attention output for backward tests and benchmarks: standard
    normals (the scale of dO does not matter to the backward's relative accuracy)."""
    rng = np.random.default_rng(seed)
    return _finish(_normal(rng, tuple(shape)), dtype)


# ---------------------------------------------------------------------------------------
# Named workloads.  Seeds: tiny 0, 32K 1, 128K 2, decode 3, varlen 4.

CONFIG_NAMES = ("tiny", "prefill32k", "prefill128k", "decode128k", "varlen")

_8B = dict(num_q_heads=32, num_kv_heads=2, head_dim=128, block_size=64, kernel_size=32,
           kernel_stride=16, num_init_blocks=1, num_local_blocks=2, dtype="bf16")


def config_params(name: str) -> Params:
    if name == "tiny":
        return Params(num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=64, kernel_size=32,
                      kernel_stride=16, topk=4, num_init_blocks=1, num_local_blocks=1, dtype="f32")
    if name == "prefill32k":
        return Params(topk=64, **_8B)
    if name in ("prefill128k", "decode128k"):
        return Params(topk=96, **_8B)
    if name == "varlen":
        return Params(num_q_heads=16, num_kv_heads=2, head_dim=64, block_size=64, kernel_size=32,
                      kernel_stride=16, topk=32, num_init_blocks=1, num_local_blocks=2, dtype="bf16")
    raise KeyError(name)


def make(name: str, seed: Optional[int] = None, length_scale: float = 1.0, steps: int = 16):
    """Build a named workload.  `length_scale` < 1 shrinks every sequence (same recipe) so the
    oracle can check it in seconds; needles scale with it."""
    p = config_params(name)

    def scaled(L: int) -> int:
        return max(1, int(round(L * length_scale)))

    if name == "tiny":
        return make_prefill(name, p, [scaled(512)], 0 if seed is None else seed)
    if name == "prefill32k":
        L = scaled(32768)
        return make_prefill(name, p, [L], 1 if seed is None else seed,
                            needles_per_seq=max(1, int(round(8 * length_scale))))
    if name == "prefill128k":
        L = scaled(131072)
        return make_prefill(name, p, [L], 2 if seed is None else seed,
                            needles_per_seq=max(1, int(round(32 * length_scale))))
    if name == "decode128k":
        L = scaled(131072)
        return make_decode(name, p, batch=8, max_len=L, steps=steps, seed=3 if seed is None else seed)
    if name == "varlen":
        lens = [scaled(x) for x in (8192, 16384, 32768, 8192)]
        return make_prefill(name, p, lens, 4 if seed is None else seed, student_t_keys=True)
    raise KeyError(name)
