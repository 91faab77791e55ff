"""MI355X-native MLA decoding over a 64-token paged KV cache.

    md = get_mla_metadata(cache_seqlens, s_q * h_q // h_kv, h_kv)   # once per step
    out, lse = mla_decode_kvcache(q, kcache, block_table, cache_seqlens,
                                  causal=..., indices=..., metadata=md)   # per layer

The work runs in hand-written gfx950 HIP kernels in libmla.so (C ABI in
include/mla.h); this package only marshals torch tensors into that ABI.
"""
from .api import (  # noqa: F401
    MlaMetadata,
    get_mla_metadata,
    mla_decode_kvcache,
    make_args,
    workspace_bytes,
    default_softmax_scale,
    refresh_mla_metadata,
    DecodeCall,
    validate_inputs,
    append_kv,
)
from ._lib import MlaError, LIB_PATH, load as load_library  # noqa: F401
