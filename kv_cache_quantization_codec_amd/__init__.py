"""KIVI grouped KV-cache codec for AMD MI355X (gfx950).

The codec runs in hand-written HIP kernels behind the C ABI of ``libkivi``
(declared in ``include/kivi.h``); this package is the thin Python binding
over it.
"""

from .binding import (  # noqa: E402,F401
    ATTENTION_SCRATCH_BYTES,
    AttnCache,
    Config,
    KiviError,
    Stream,
    alloc_keys,
    alloc_layers,
    alloc_values,
    kivi_append_flush,
    kivi_attention_workspace_bytes,
    kivi_boundary_layers,
    kivi_decode_attention,
    kivi_decode_attention_noalloc,
    kivi_decode_k,
    kivi_decode_k_layers,
    kivi_decode_v,
    kivi_decode_v_layers,
    kivi_encode_k,
    kivi_encode_k_layers,
    kivi_encode_v,
    kivi_encode_v_layers,
    kivi_fp8_decode,
    kivi_fp8_encode,
    kivi_k_code_words,
    kivi_k_stat_elems,
    kivi_ring_elems,
    kivi_stream_image_bytes,
    kivi_stream_offload,
    kivi_stream_prefill,
    kivi_stream_restore,
    kivi_v_code_words,
    kivi_v_stat_elems,
)
