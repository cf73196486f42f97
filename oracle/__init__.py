"""CPU oracle for MLA latent-KV decode and cache insert (test infrastructure).

This package is a plain, slow, float64 reference used only by the tests, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``.  The
product path (the HIP library and its Python binding) never imports it.

Parity status of each function is stated in ``oracle/mla_oracle.py``.
"""
from . import dsa, fp8  # noqa: F401
from .mla_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    rmsnorm_bf16,
    rope_pairs_f64,
    rope_bf16,
    rotate_q,
    cache_insert,
    decode_expanded,
    decode_absorbed,
)
