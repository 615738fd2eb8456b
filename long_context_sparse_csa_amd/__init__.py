"""MI355X (gfx950) HIP implementation of the compressed-sparse-attention hot path.

The compute lives in ``libcsa.so`` (C ABI in ``include/csa.h``); ``binding`` marshals PyTorch
tensors into it.  There is no fallback: without the built library every entry point raises.
"""
from .binding import (  # noqa: F401
    CSA_BF16, CSA_F32, CSA_FP4_E2M1, CSA_FP8_E4M3FN, CSA_KV_BF16, CSA_KV_F32, CSA_KV_FP8NOPE_BF16ROPE, CsaError,
    PagedIdx, PagedKV, csa_compress_index_keys, csa_compress_kv, csa_debug_violations, csa_decode, csa_decode_multi, csa_decode_noalloc, csa_decode_multi_workspace_bytes, csa_decode_workspace_bytes,
    csa_hca_decode, csa_hca_decode_workspace_bytes,
    csa_hca_prefill, csa_hca_prefill_workspace_bytes, csa_indexer_logits, csa_last_hip_error, csa_prefill,
    csa_prefill_workspace_bytes, csa_profile_collect, csa_profile_enable, csa_profile_reset, csa_sparse_attn,
    csa_sparse_attn_workspace_bytes, csa_status_string, csa_topk, csa_topk_workspace_bytes, lib, paged_idx,
    paged_kv,
)
from .layout import pack_index_keys, unpack_index_keys  # noqa: F401
