"""MI355X-native shared-KV cross-attention (YOCO Cross-Decoder hot path).

The compute lives in the HIP library ``lib/libyoco_xattn.so`` (C ABI in
``include/yoco_xattn.h``); this package is its thin Python binding. Nothing
here falls back to another implementation: calls raise if the library is
missing or rejects its arguments.
"""
from .xattn import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    SharedKV,
    YocoError,
    alloc_prefill_workspace,
    alloc_workspace,
    decode_splits,
    gret_decode,
    gret_prefill,
    gret_workspace_size,
    kv_append,
    kv_append_ring,
    kv_project_append,
    kv_project_pack,
    load_library,
    make_dims,
    workspace_size,
    xattn_decode,
    xattn_decode_noalloc,
    NOALLOC_SCRATCH_BYTES,
    xattn_decode_window,
    xattn_prefill,
    xattn_prefill_window,
)
