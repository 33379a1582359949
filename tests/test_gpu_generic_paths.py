"""Parity of the kernels that only shapes outside the measured ones reach, against the oracle:

* bf16 layers whose geometry the matrix-core kernels do not take (group sizes other than 8 and
  16, head_dim 96, blocks of 32 or 128 tokens with their own kernel windows): the float32
  generic score and attention kernels on bf16 data, in prefill and in the decode step (which
  then chains the separate calls);
* a bf16 prefill whose queries reach more than 2048 blocks (positions past 131072): the tile
  kernel's union bitmap stops at 2048 blocks, so these rows go to the per-row matrix-core
  kernel; every row of the chunk is checked.
Rules are those of tests/_compare.py (kernels exact, scores within the float32 bound, indices
exact or inside the tie band, attention on the GPU's own indices)."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle import infllm2_oracle as orc
from tests._gpu import log, run_prefill_stages
from tests.test_gpu_parity import check_sequence, run_decode

pytestmark = pytest.mark.gpu

GENERIC = [
    # (Hq, Hkv, d, B, w, s)
    (8, 2, 96, 64, 32, 16),     # group 4, head_dim 96: generic attention, generic scores
    (32, 2, 128, 32, 16, 8),    # the 8B heads with 32-token blocks: generic scores and attention
    (4, 4, 64, 128, 64, 32),    # one head per group, 128-token blocks
    (24, 2, 128, 64, 32, 16),   # group 12: matrix-core scores, generic attention
]


def generic_params(Hq, Hkv, d, B, w, s):
    return replace(synth.config_params("prefill32k"), num_q_heads=Hq, num_kv_heads=Hkv,
                   head_dim=d, block_size=B, kernel_size=w, kernel_stride=s, topk=12)


@pytest.mark.parametrize("geo", GENERIC, ids=lambda g: "-".join(map(str, g)))
def test_bf16_generic_geometry_prefill_all_rows(geo):
    p = generic_params(*geo)
    lens = [1500, 77, 900]
    wl = synth.make_prefill("generic", p, lens, seed=61, needles_per_seq=1)
    log(f"case bf16 generic prefill {geo}")
    res = run_prefill_stages(wl)
    for b in range(wl.num_seqs):
        check_sequence(wl, res, b, label=f"generic {geo}")


@pytest.mark.parametrize("geo", GENERIC[:3], ids=lambda g: "-".join(map(str, g)))
def test_bf16_generic_geometry_decode(geo):
    """The decode step on a geometry its fused kernels do not take: the separate calls are
    chained (generic scores, the selection, split generic attention and the merge)."""
    p = generic_params(*geo)
    wl = synth.make_decode("generic-dec", p, batch=3, max_len=2600, steps=2, seed=62,
                           kv_len0=[2590, 1300, 90])
    log(f"case bf16 generic decode {geo}")
    run_decode(wl, 2, label=f"generic decode {geo}")


def test_bf16_prefill_beyond_2048_blocks_all_rows():
    """64 query rows at positions 139936 .. 139999 of a 140000-token sequence (2188 reachable
    blocks): every row, scores, indices and attention."""
    p = synth.config_params("prefill128k")
    L, n = 140000, 64
    full = synth.make_prefill("past2048", p, [L], seed=63, needles_per_seq=2)
    wl = synth.Workload("past2048", p, full.q[L - n:], full.k, full.v, np.array([0]),
                        np.array([n], np.int32), np.array([L - n], np.int32), np.array([0]),
                        np.array([L], np.int32))
    assert (L - 1) // p.block_size + 1 > 2048
    log("case bf16 prefill past 2048 blocks")
    res = run_prefill_stages(wl)
    check_sequence(wl, res, 0, label="past 2048 blocks")
    for nd in full.needles:
        qp = nd.query_positions[nd.query_positions >= L - n] - (L - n)
        if len(qp):
            assert np.all(np.any(res["idx"][qp, nd.kv_head, :] == nd.block, axis=1))
