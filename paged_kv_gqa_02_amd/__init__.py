"""MI355X-native paged GQA decode and speculative-verify attention.

The work runs in ``libpaged_attn.so`` (HIP kernels for gfx950 behind the C ABI
declared in ``include/paged_attn.h``); ``binding`` marshals torch tensors into
it.  Importing this package fails if the library has not been built.
"""
from .binding import (  # noqa: F401
    PA_BF16, PA_F32, PA_FP8_E4M3, HipEvent, PagedAttnError, Pool, declared_symbols,
    paged_attn_append_kv, paged_attn_rejection_sample, paged_attn_rejection_sample_workspace_bytes,
    paged_attn_create_pool, paged_attn_decode, paged_attn_destroy_pool, paged_attn_plan,
    paged_attn_pool_bytes, paged_attn_validate, paged_attn_verify, paged_attn_verify_noalloc, paged_attn_verify_timed, paged_attn_verify_tree,
    paged_attn_workspace_bytes, workspace_for,
)
