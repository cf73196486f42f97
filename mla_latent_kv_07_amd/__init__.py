"""MI355X (gfx950) MLA latent-KV decode and cache insert.

The compute lives in ``libmla.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/mla.h``).  This package is a thin ctypes binding with the
same entry-point names; torch is used only for device memory and streams.
"""
from ._lib import (  # noqa: F401
    FP8_ROW_BYTES,
    MLAError,
    abi_version,
    cache_insert,
    debug_checks,
    decode,
    decode_noalloc,
    decode_step,
    decode_workspace_bytes,
    dsa_decode,
    dsa_select,
    dsa_workspace_bytes,
    lib_path,
    load,
    noalloc_scratch_bytes,
    prefill,
    prefill_workspace_bytes,
    profile_collect,
    profile_collect_calls,
    profile_enable,
    status_string,
)
