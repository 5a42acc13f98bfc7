"""pkv — FP8 (OCP E4M3) paged KV cache and single-token decode attention on
AMD MI355X (gfx950).

The computation lives in libpkv.so (hand-written HIP kernels behind the C ABI
of include/pkv.h); this package is its Python binding, with the same entry
point names. torch supplies device memory and the stream, nothing else.

Method: "Smaller, faster, safer: running Kimi and GLM at scale" — sections
"Quantizing the KV cache" (e4m3 cache, converted on read by the attention
kernel) and "Protecting a shared KV cache" (per-page tags checked against
each request's recorded mapping in a separate pass before decode; mismatches
abort the request).
"""
from ._binding import (EXPORTS, LIB_PATH, PKV_EHIP, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_KV_BF16,
                       PKV_KV_E4M3, PKV_OK, Cache, PkvCacheStruct, PkvError, pkv_append,
                       pkv_combine, pkv_decode_attn, pkv_decode_attn_drafts,
                       pkv_decode_attn_static, STATIC_SCRATCH_BYTES, pkv_int4_linear,
                       pkv_int4_linear_workspace, int4_workspace,
                       pkv_fill_u32, pkv_read_u32, pkv_requantize_pages, pkv_scales_from_amax,
                       pkv_step_combine, pkv_step_decode, pkv_step_launches, pkv_strerror,
                       pkv_suggest_split, pkv_verify, pkv_verify_append, pkv_version)
from .step import DecodeStep, allocate_cache

__all__ = ["EXPORTS", "LIB_PATH", "PKV_EHIP", "PKV_EINVAL", "PKV_EUNSUPPORTED", "PKV_KV_BF16",
           "PKV_KV_E4M3", "PKV_OK", "Cache", "PkvCacheStruct", "PkvError", "pkv_append",
           "pkv_combine", "pkv_decode_attn", "pkv_decode_attn_drafts",
           "pkv_decode_attn_static", "STATIC_SCRATCH_BYTES", "pkv_int4_linear",
           "pkv_int4_linear_workspace", "int4_workspace",
           "pkv_fill_u32", "pkv_read_u32", "pkv_requantize_pages", "pkv_scales_from_amax",
           "pkv_step_combine", "pkv_step_decode", "pkv_step_launches", "pkv_strerror",
           "pkv_suggest_split", "pkv_verify", "pkv_verify_append", "pkv_version", "DecodeStep",
           "allocate_cache"]
