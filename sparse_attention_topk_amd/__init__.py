"""Python binding of libdsa (the MI355X DSA indexer + top-k + sparse-MLA
library).  Argument marshalling only: every step of the path runs in the HIP
kernels behind the C ABI in include/dsa.h; PyTorch supplies device memory
and the current HIP stream.

The library is loaded from this directory (libdsa.so, built by
``python -m sparse_attention_topk_amd.build``).  There is no fallback: if the
library is missing or cannot be loaded, using any entry point raises.  The
checked build libdsa_debug.so (same kernels, plus metadata validation and
output canaries around every call) is selected with DSA_LIBRARY=debug or
``use_library("debug")``; ``debug_faults()`` reads what it found.
"""

from ._binding import (  # noqa: F401
    DSA_F32, DSA_BF16, DSA_FP8_E4M3, DSA_LAYER_FULL, DSA_LAYER_SHARED,
    DSAError, Batch, library_path, load_library, exported_symbols,
    dsa_indexer_cache_write, dsa_indexer_topk, dsa_indexer_topk_workspace_size,
    dsa_indexer_topk_workspace_min,
    dsa_indexer_topk_noalloc, dsa_rotate_quantize, dsa_indexer_topk_fp8q,
    dsa_indexer_prologue,
    sparse_mla_attn, sparse_mla_attn_workspace_size,
    dsa_resolve_indexer_sources, indexshare_forward,
    indexshare_forward_workspace_size, dsa_fp8_decode_check, dsa_last_error,
    Layer, StackDims, use_library, debug_faults,
    DSA_FAULT_SEQ_LENS, DSA_FAULT_CU_Q, DSA_FAULT_BLOCK_TABLE, DSA_FAULT_SLOT_MAPPING,
    DSA_FAULT_TOPK_INPUT, DSA_FAULT_TOPK_OUTPUT, DSA_FAULT_UNWRITTEN)
