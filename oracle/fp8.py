"""Float64 CPU oracle for the FP8 latent cache (cache insert with FP8
quantisation, and decode over the FP8 cache).  TEST INFRASTRUCTURE ONLY:
imported by ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg, never by the product path.

Sources (pages, with their own section headings):

* [V32]  "DeepSeek-V3.2-Exp unboxing", section "初步研读": the model code
  notes that deployment keeps the KV cache in FP8 and simulates it by casting
  the latent to FP8 and back; the sparse-attention indexer next to it keeps
  FP8 keys with one scale per cached token (``k_scale_cache`` [B, T, 1]).
* [V4]   the vLLM DeepSeek-V4 MoE notes (section 一): "KV quant" fused into
  the cache-insert kernel, and UE8M0 (power-of-two) block scales.
* [V2L]  "DeepSeek-V2-Lite 模型结构详解" §五: the cache entry is the 512-wide
  latent followed by the 64-wide rope part.

Readings (each is listed in the design doc; the pages fix no format):

* element format: FP8 E4M3 in its "FN" form (1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite
  value 448; subnormals down to 2**-9), rounding to nearest, ties to even;
* only the latent is quantised (the code casts ``kv``, the normalised latent;
  k_pe stays in the activation type, bf16);
* one power-of-two scale per token (the indexer's per-token key scale, with
  the UE8M0 scale form): the smallest 2**e with max|x| * 2**-e <= 448, e
  clamped to [-126, 127], e = 0 for an all-zero latent; stored as the byte
  e + 127;
* cache row of 656 bytes: 512 codes, the 64 rope values as bf16 (128
  bytes, little endian), the scale byte, 15 zero bytes (rows stay 16-byte
  aligned); a page is 64 rows.

Every function here is pinned by ``tests/test_fp8_oracle.py`` (torch's
independent float8_e4m3fn conversion over every bf16 input and every code,
properties the format fixes, and an end-to-end identity with the bf16
oracle); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .mla_oracle import (bf16_bits_to_f64, cache_insert, decode_expanded, f64_to_bf16_bits,
                         rmsnorm_bf16, rope_bf16)

FP8_ROW_BYTES = 656           # bytes per cached token
FP8_MAX = 448.0               # largest finite E4M3 value
_ROPE_OFF = 512               # rope bytes start here (after 512 codes)
_SCALE_OFF = 640              # scale byte


# --------------------------------------------------------------------------
# E4M3 (FN) element format
# --------------------------------------------------------------------------


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code (uint8) as float64, from the format fields:
    exponent field 0 -> subnormal m * 2**-9; otherwise (1 + m/8) * 2**(E - 7);
    S.1111.111 -> NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    out[(e == 15) & ((c & 7) == 7)] = np.nan
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float64 values to E4M3 codes (nearest, ties to even).

    The representable magnitudes form a ladder with a fixed quantum per binade
    (2**-9 in the subnormal range and the first normal binade, 2**(E-10) in
    binade E >= 1 of the exponent field); a value rounds to the nearest rung,
    a tie goes to the rung with an even code.  Above 448 the next rung would
    be 480, which the FN form spends on NaN: values beyond the 448/480
    midpoint (464) become NaN, 464 itself rounds to 448 (even).  NaN in, NaN
    (0x7F with the sign) out.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        return _e4m3_encode(x)


def _e4m3_encode(x: np.ndarray) -> np.ndarray:
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8)
    a = np.abs(x)
    # quantum of the binade holding a: binade of the value with exponent
    # field E covers [2**(E-7), 2**(E-6)); below 2**-6 the quantum is 2**-9
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a = f * 2**ex, f in [0.5, 1)
    quantum = np.where(a >= 2.0 ** -6, np.exp2(ex - 4.0), 2.0 ** -9)
    q = np.rint(a / quantum) * quantum                # half to even in units of the quantum
    # a value may round up into the next binade: still exact there
    code = np.zeros(a.shape, dtype=np.int64)
    sub = q < 2.0 ** -6
    code[sub] = np.rint(q[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    fq, eq = np.frexp(np.where(nrm & np.isfinite(q), q, 1.0))  # q = fq * 2**eq
    efield = eq - 1 + 7
    mant = np.rint((fq * 2.0 - 1.0) * 8.0).astype(np.int64)
    code[nrm] = (efield[nrm] << 3) | mant[nrm]
    over = a > 464.0
    bad = over | np.isnan(x) | (code > 0x7E)
    code[bad] = 0x7F
    code[(a == 464.0)] = 0x7E
    return (code.astype(np.uint8) | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# Per-token power-of-two scale and the row format
# --------------------------------------------------------------------------


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax * 2**-e <= 448, clamped to [-126, 127]
    (0 where amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / FP8_MAX)).astype(np.int64)
    # log2 rounding can be off by one next to a power of two: settle exactly
    e = np.where(safe * np.exp2(-(e - 1.0)) <= FP8_MAX, e - 1, e)
    e = np.where(safe * np.exp2(-e.astype(np.float64)) > FP8_MAX, e + 1, e)
    e = np.clip(e, -126, 127)
    return np.where(amax > 0, e, 0)


def quantize_latent(lat_bits: np.ndarray):
    """bf16 latent rows [..., 512] -> (codes uint8 [..., 512], scale byte uint8 [...])."""
    x = bf16_bits_to_f64(lat_bits)
    e = scale_exponent(np.max(np.abs(x), axis=-1))
    codes = e4m3_encode(x * np.exp2(-e.astype(np.float64))[..., None])
    return codes, (e + 127).astype(np.uint8)


def dequantize_latent(codes: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """codes [..., 512], scale bytes [...] -> float64 latent values."""
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    return e4m3_decode(codes) * np.exp2(e.astype(np.float64))[..., None]


def pack_rows(codes: np.ndarray, rope_bits: np.ndarray, scale_bytes: np.ndarray) -> np.ndarray:
    """Assemble 656-byte cache rows from codes [..., 512], rope bf16 bits
    [..., 64] and scale bytes [...]."""
    lead = codes.shape[:-1]
    rows = np.zeros(lead + (FP8_ROW_BYTES,), dtype=np.uint8)
    rows[..., :_ROPE_OFF] = codes
    rope_le = np.ascontiguousarray(np.asarray(rope_bits, dtype=np.uint16).astype("<u2"))
    rows[..., _ROPE_OFF:_SCALE_OFF] = rope_le.view(np.uint8).reshape(lead + (128,))
    rows[..., _SCALE_OFF] = scale_bytes
    return rows


def unpack_rows(rows: np.ndarray):
    """Inverse of pack_rows: (codes, rope bf16 bits, scale bytes)."""
    rows = np.asarray(rows, dtype=np.uint8)
    lead = rows.shape[:-1]
    codes = rows[..., :_ROPE_OFF]
    rope = np.ascontiguousarray(rows[..., _ROPE_OFF:_SCALE_OFF]).view("<u2").reshape(lead + (64,))
    return codes, rope.astype(np.uint16), rows[..., _SCALE_OFF]


def quantize_cache(cache_bits: np.ndarray) -> np.ndarray:
    """A bf16 cache [N, page, 576] in the FP8 row format [N, page, 656]."""
    codes, scale = quantize_latent(cache_bits[..., :512])
    return pack_rows(codes, cache_bits[..., 512:], scale)


def dequantize_cache(cache_u8: np.ndarray) -> np.ndarray:
    """FP8 cache rows [N, page, 656] -> float64 entries [N, page, 576]."""
    codes, rope, scale = unpack_rows(cache_u8)
    return np.concatenate([dequantize_latent(codes, scale), bf16_bits_to_f64(rope)], axis=-1)


# --------------------------------------------------------------------------
# Insert and decode over the FP8 cache
# --------------------------------------------------------------------------


def cache_insert_fp8(cache_u8: np.ndarray, kv_a_bits: np.ndarray, w_bits: np.ndarray,
                     block_table: np.ndarray, seq_lens: np.ndarray, q_len: int,
                     eps: float, rope_base: float) -> np.ndarray:
    """Return a copy of the FP8 cache with the q_len new tokens written.

    The new entries are those of the bf16 insert ([V2L] §四 RMSNorm with the
    weight, RoPE on k_pe, see ``cache_insert``), then the latent is quantised
    ([V32] cast to FP8; [V4] KV quant inside the insert) with its per-token
    scale, and the row is packed.
    """
    out = np.array(cache_u8, dtype=np.uint8, copy=True)
    page = out.shape[1]
    bsz = kv_a_bits.shape[0]
    for b in range(bsz):
        start = int(seq_lens[b]) - q_len
        pos = np.arange(start, start + q_len)
        lat = rmsnorm_bf16(kv_a_bits[b, :, :512], w_bits, eps)
        pe = rope_bf16(kv_a_bits[b, :, 512:], pos, rope_base)
        codes, scale = quantize_latent(lat)
        rows = pack_rows(codes, pe, scale)
        for i, p in enumerate(pos):
            out[int(block_table[b, p // page]), p % page] = rows[i]
    return out


def decode_expanded_fp8(q_bits, kv_b_bits, cache_u8, block_table, seq_lens, q_len, *,
                        batches=None, **kw):
    """MLA decode over the FP8 cache: the expanded-form oracle
    (``decode_expanded``) on the dequantised entries (codes times the token's
    scale, exact in float64; rope bf16 widened exactly).

    Only the pages of the requested sequences are dequantised (the same
    entries, gathered into a smaller cache through a renumbered block table),
    so sampled checks at full size stay cheap."""
    bsz = q_bits.shape[0]
    batches = list(range(bsz)) if batches is None else list(batches)
    page = cache_u8.shape[1]
    need = [np.asarray(block_table[b, :(int(seq_lens[b]) + page - 1) // page], dtype=np.int64)
            for b in batches]
    used = np.unique(np.concatenate(need)) if need else np.zeros(0, dtype=np.int64)
    compact = dequantize_cache(cache_u8[used])
    bt = np.zeros((bsz, max(1, block_table.shape[1])), dtype=np.int64)
    for b, blocks in zip(batches, need):
        bt[b, :len(blocks)] = np.searchsorted(used, blocks)
    return decode_expanded(q_bits, kv_b_bits, compact, bt, seq_lens, q_len, batches=batches,
                           **kw)


__all__ = ["FP8_ROW_BYTES", "FP8_MAX", "e4m3_decode", "e4m3_encode", "scale_exponent",
           "quantize_latent", "dequantize_latent", "pack_rows", "unpack_rows",
           "quantize_cache", "dequantize_cache", "cache_insert_fp8", "decode_expanded_fp8",
           "cache_insert"]
