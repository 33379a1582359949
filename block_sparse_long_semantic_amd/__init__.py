"""InfLLM v2 block-sparse attention on MI355X (gfx950): thin Python binding of libinfllm2.

Every compute step runs in the HIP library; this package only marshals arguments (device
pointers of torch tensors, the current HIP stream, the sequence metadata's device copy).  Importing
it loads the shared library and fails loudly if it has not been built
(`python -m block_sparse_long_semantic_amd.build`).
"""
from ._lib import (  # noqa: F401
    F32, BF16, InfLLM2Error, Params, Seqs, library_path, load_library,
    compress_kernels, block_scores, topk_select, sparse_attn_prefill,
    decode_workspace_size, sparse_attn_decode, decode_step_fused, version, EXPORTED_SYMBOLS,
    backward_workspace_size, sparse_attn_backward, sliding_window_attn, decode_step_noalloc,
)
from .pipeline import prefill, decode_step, num_kernels  # noqa: F401
