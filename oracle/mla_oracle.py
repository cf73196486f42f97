"""Float64 CPU oracle for MLA decode over a paged latent cache, and for the
cache-insert step.  TEST INFRASTRUCTURE ONLY: imported by ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg, never by the
product path.

Sources (pages, with their own section headings):

* [V3-src]  "深度解读DeepSeek：源码解读 DeepSeek-V3" (source walk-through of
  DeepSeek-V3 inference/model.py): section "MLA", its listing of
  ``MLA.forward``, the subsections "(a) Naive实现" (expanded MHA form) and
  "(b) 优化实现" (absorbed form), and the ``Transformer`` constructor
  (``freqs_cis`` buffer).
* [V2L]     "DeepSeek-V2-Lite 模型结构详解": section "四、RMSNorm" (row rule
  and the "精度" float32 rule) and section "五、MLA" (the 576-number cache
  entry, the two absorption identities in "最关键的一问：解压的代价去哪了",
  the 128+64 split in "为什么 Q/K 是 192 维而 V 只有 128 维").
* [TAGS]    the "DeepSeek" tag page: the excerpt on the 1/sqrt(d_k) scale and
  the excerpt on MLA under decode context parallelism (decode = one latent
  head of width ~576).
* [V32]     "DeepSeek-V3.2-Exp unboxing": section "初步研读", the forward
  listing (``-inf`` mask built with ``triu_(1)``).

Data conventions.  bf16 tensors are numpy ``uint16`` arrays holding the bf16
bit patterns; they are widened to float64 exactly.  Dimensions are arguments,
so the same code runs at the real sizes (latent 512, rope 64, nope 128, v 128)
and at tiny sizes for brute-force checks.

Readings where the pages are silent (each is listed in the design doc):

* softmax scale = 1/sqrt(qk_nope + qk_rope) (= 1/sqrt(192)) in both forms;
* RoPE rotates interleaved pairs (2j, 2j+1) as complex numbers, frequency
  base**(-2j/rope), angle = position * frequency, position = 0-based cache
  index; k_pe is rotated; q_pe arrives already rotated for the decode, and
  the fused step (``rotate_q``) rotates it at its own token's position;
* RMSNorm: eps inside the square root, two bf16 roundings (normalised value,
  then weight * value);
* cache entry = latent (first) then rope part, one paged tensor
  [num_blocks, page, latent + rope];
* decode causal rule: new query i of a sequence of (post-insert) length L sees
  cache positions t <= L - q_len + i.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, identities stated on the pages, brute force, library
routines); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bf16 <-> float64
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the upper half of a float32 with the lower 16 bits zero.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even).

    Written from the definition of the format: 8 significant bits for normal
    numbers (1 implicit + 7 stored), a fixed quantum of 2**-133 below the
    smallest normal 2**-126, overflow to infinity above the largest finite
    value.  The rounding happens once, directly from float64.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    ax = np.abs(x)
    normal = ax >= 2.0 ** -126
    m, e = np.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    # normal range: keep 8 significant bits of m
    q = np.rint(m * 256.0)  # numpy rint rounds half to even
    out[normal] = np.ldexp(q, e - 8)[normal]
    sub = ~normal
    out[sub] = (np.rint(x * 2.0 ** 133) * 2.0 ** -133)[sub]
    # overflow: the largest finite bf16 is (2 - 2**-7) * 2**127
    big = np.abs(out) > (2.0 - 2.0 ** -7) * 2.0 ** 127
    out[big] = np.copysign(np.inf, x[big])
    nan = np.isnan(x)
    f32 = out.astype(np.float32)  # exact: every value above is a bf16 value
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[nan] = np.uint16(0x7FC0)
    return bits


# --------------------------------------------------------------------------
# Insert step: RMSNorm on the latent, RoPE on k_pe, paged write
# --------------------------------------------------------------------------


def rmsnorm_bf16(x_bits: np.ndarray, w_bits: np.ndarray, eps: float) -> np.ndarray:
    """kv_a RMSNorm of bf16 rows, returning bf16 bits.

    [V2L] §四 RMSNorm: each row (last dimension) independently,
    rms = sqrt(sum(x^2)/D + eps), out = x / rms * weight; the "精度" paragraph
    computes the normalisation in a wider type, converts the normalised row
    back to the activation type, then multiplies by the weight (the product of
    two bf16 values, rounded to bf16).  Here the wide type is float64.
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    n = x / np.sqrt(ms + eps)
    n_b = bf16_bits_to_f64(f64_to_bf16_bits(n))
    return f64_to_bf16_bits(w * n_b)


def rope_pairs_f64(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate interleaved pairs of the last dimension by position (float64).

    [V3-src] ``freqs_cis`` is a complex table (one unit complex number per
    position and pair) and ``apply_rotary_emb`` multiplies each pair, read as
    (real, imaginary), by it.  Pair j of a width-R vector turns by the angle
    pos * base**(-2j/R).  ``pos`` broadcasts against ``x[..., 0]``.
    """
    x = np.asarray(x, dtype=np.float64)
    r = x.shape[-1]
    j = np.arange(r // 2, dtype=np.float64)
    freq = base ** (-2.0 * j / r)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    c, s = np.cos(ang), np.sin(ang)
    re, im = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = re * c - im * s
    out[..., 1::2] = re * s + im * c
    return out


def rope_bf16(x_bits: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """RoPE on bf16 input, one rounding of the rotated value back to bf16."""
    return f64_to_bf16_bits(rope_pairs_f64(bf16_bits_to_f64(x_bits), pos, base))


def rotate_q(q_bits: np.ndarray, seq_lens: np.ndarray, q_len: int, rope_base: float,
             nope: int) -> np.ndarray:
    """q [B, q_len, H, nope + rope] (uint16 bf16 bits) with every head's rope
    part rotated, one rounding to bf16; the nope part is returned unchanged.

    [V3-src] the query branch of ``MLA.forward`` applies ``apply_rotary_emb``
    to q_pe with the same ``freqs_cis`` rows as k_pe, those of the current
    positions start_pos ..: new query i of a sequence whose post-insert length
    is L sits at position L - q_len + i, the position its own k_pe is cached
    at.
    """
    out = np.array(q_bits, dtype=np.uint16, copy=True)
    for b in range(q_bits.shape[0]):
        pos = int(seq_lens[b]) - q_len + np.arange(q_len)
        out[b, :, :, nope:] = rope_bf16(q_bits[b, :, :, nope:], pos[:, None], rope_base)
    return out


def cache_insert(cache_bits: np.ndarray, kv_a_bits: np.ndarray, w_bits: np.ndarray,
                 block_table: np.ndarray, seq_lens: np.ndarray, q_len: int,
                 eps: float, rope_base: float, latent: int) -> np.ndarray:
    """Return a copy of the paged cache with the q_len new tokens written.

    cache_bits : uint16 [num_blocks, page, latent + rope]
    kv_a_bits  : uint16 [B, q_len, latent + rope]   (kv_a projection output)
    block_table: int    [B, max_blocks] physical block of each logical block
    seq_lens   : int    [B] cache length after the insert

    [V3-src] absorbed branch: the latent part goes to the cache through
    ``kv_norm`` and k_pe through ``apply_rotary_emb``, at positions
    start_pos .. start_pos + seqlen - 1; here start_pos = seq_lens - q_len.
    [V2L] §五: latent 512 then k_pe 64 form one 576-number entry.
    The page of position p is block_table[b, p // page], slot p % page.
    """
    out = np.array(cache_bits, dtype=np.uint16, copy=True)
    page = out.shape[1]
    bsz = kv_a_bits.shape[0]
    for b in range(bsz):
        start = int(seq_lens[b]) - q_len
        pos = np.arange(start, start + q_len)
        lat = rmsnorm_bf16(kv_a_bits[b, :, :latent], w_bits, eps)
        pe = rope_bf16(kv_a_bits[b, :, latent:], pos, rope_base)
        for i, p in enumerate(pos):
            blk = int(block_table[b, p // page])
            out[blk, p % page, :latent] = lat[i]
            out[blk, p % page, latent:] = pe[i]
    return out


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------


def _gather_sequence(cache: np.ndarray, block_table: np.ndarray, b: int, length: int):
    """Rows 0..length-1 of sequence b, through its block table (float64).

    ``cache`` holds bf16 bit patterns (uint16), or values already widened to
    float64 (the dequantised FP8 cache), which pass through unchanged."""
    page = cache.shape[1]
    t = np.arange(length)
    blocks = block_table[b, t // page].astype(np.int64)
    rows = cache[blocks, t % page, :]
    return rows if rows.dtype == np.float64 else bf16_bits_to_f64(rows)


def _visible(length: int, q_len: int) -> np.ndarray:
    """Mask [q_len, length]: new query i sees positions t <= length - q_len + i.

    [V32] 初步研读 forward listing: the mask is -inf above the diagonal of the
    block of new tokens (triu(1)); shifted to the cache offset length - q_len.
    """
    t = np.arange(length)[None, :]
    i = np.arange(q_len)[:, None]
    return t <= (length - q_len + i)


def decode_expanded(q_bits: np.ndarray, kv_b_bits: np.ndarray, cache_bits: np.ndarray,
                    block_table: np.ndarray, seq_lens: np.ndarray, q_len: int, *,
                    latent: int = 512, rope: int = 64, nope: int = 128, v_dim: int = 128,
                    softmax_scale: float | None = None, batches=None, heads=None,
                    chunk: int = 4096, return_probs: bool = False):
    """MLA decode in the non-absorbed (expanded multi-head) form, float64.

    q_bits     : uint16 [B, q_len, H, nope + rope], q_pe already rotated
    kv_b_bits  : uint16 [H * (nope + v_dim), latent] (kv_b_proj weight)
    cache_bits : uint16 [num_blocks, page, latent + rope] (or float64 values)
    Returns float64 [len(batches), q_len, len(heads), v_dim].

    [V3-src] "(a) Naive实现": kv_b_proj applied to the normalised latent gives
    per head [k_nope | v] (the weight viewed as [H, nope + v_dim, latent], rows
    0..nope-1 of each head produce k_nope, the rest produce v); the key is
    k_nope followed by the shared k_pe; scores = q . k * softmax_scale; the
    mask is added; softmax over cache positions; output = sum_t p_t v_t.
    [TAGS] the scale is 1/sqrt(d_k) with d_k = nope + rope.
    The key/value expansion runs over chunks of at most ``chunk`` positions
    (the listing's einsum over t, split only to bound memory).
    """
    q_all = bf16_bits_to_f64(q_bits)
    bsz, _, n_heads, qk = q_all.shape
    assert qk == nope + rope
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(nope + rope)
    w = bf16_bits_to_f64(kv_b_bits).reshape(n_heads, nope + v_dim, latent)
    batches = list(range(bsz)) if batches is None else list(batches)
    heads = list(range(n_heads)) if heads is None else list(heads)
    w_uk = w[heads, :nope, :]            # [h, nope, latent]
    w_uv = w[heads, nope:, :]            # [h, v_dim, latent]
    out = np.zeros((len(batches), q_len, len(heads), v_dim))
    probs = []
    for bi, b in enumerate(batches):
        length = int(seq_lens[b])
        rows = _gather_sequence(cache_bits, block_table, b, length)
        c, r = rows[:, :latent], rows[:, latent:latent + rope]
        q = q_all[b][:, heads, :]        # [q_len, h, nope + rope]
        scores = np.empty((q_len, len(heads), length))
        q_h = np.ascontiguousarray(q.transpose(1, 2, 0))                  # [h, nope+rope, i]
        for t0 in range(0, length, chunk):
            t1 = min(length, t0 + chunk)
            k_nope = np.matmul(c[None, t0:t1], w_uk.transpose(0, 2, 1))  # [h, t, nope]
            k = np.concatenate(
                [k_nope, np.broadcast_to(r[t0:t1][None], (len(heads), t1 - t0, rope))],
                axis=-1)                                                  # [h, t, nope+rope]
            scores[:, :, t0:t1] = np.matmul(k, q_h).transpose(2, 0, 1) * softmax_scale
        vis = _visible(length, q_len)[:, None, :]
        scores = np.where(vis, scores, -np.inf)
        mx = scores.max(axis=-1, keepdims=True)
        e = np.exp(scores - mx)
        p = e / e.sum(axis=-1, keepdims=True)
        if return_probs:
            probs.append(p)
        acc = np.zeros((len(heads), q_len, v_dim))
        p_h = p.transpose(1, 0, 2)                                        # [h, i, t]
        for t0 in range(0, length, chunk):
            t1 = min(length, t0 + chunk)
            v = np.matmul(c[None, t0:t1], w_uv.transpose(0, 2, 1))      # [h, t, v_dim]
            acc += np.matmul(p_h[:, :, t0:t1], v)                        # [h, i, v_dim]
        out[bi] = acc.transpose(1, 0, 2)
    if return_probs:
        return out, probs
    return out


def decode_absorbed(q_bits: np.ndarray, kv_b_bits: np.ndarray, cache_bits: np.ndarray,
                    block_table: np.ndarray, seq_lens: np.ndarray, q_len: int, *,
                    latent: int = 512, rope: int = 64, nope: int = 128, v_dim: int = 128,
                    softmax_scale: float | None = None, batches=None, heads=None):
    """MLA decode in the absorbed form, float64 (a cross-check of the
    expanded form, not the parity reference).

    [V3-src] "(b) 优化实现": q_nope is multiplied into latent space by the
    first nope rows of each head's kv_b block; scores are q_lat . c_t plus
    q_pe . k_pe_t, times the scale; after the softmax, the latent rows are
    summed with the weights and the result is multiplied by the last v_dim
    rows of each head's block.  [V2L] §五 states the two identities that make
    this equal to the expanded form.
    """
    q_all = bf16_bits_to_f64(q_bits)
    bsz, _, n_heads, _ = q_all.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(nope + rope)
    w = bf16_bits_to_f64(kv_b_bits).reshape(n_heads, nope + v_dim, latent)
    batches = list(range(bsz)) if batches is None else list(batches)
    heads = list(range(n_heads)) if heads is None else list(heads)
    w_uk = w[heads, :nope, :]
    w_uv = w[heads, nope:, :]
    out = np.zeros((len(batches), q_len, len(heads), v_dim))
    for bi, b in enumerate(batches):
        length = int(seq_lens[b])
        rows = _gather_sequence(cache_bits, block_table, b, length)
        c, r = rows[:, :latent], rows[:, latent:latent + rope]
        q = q_all[b][:, heads, :]
        q_lat = np.einsum("ihd,hdc->ihc", q[..., :nope], w_uk)
        scores = (np.einsum("ihc,tc->iht", q_lat, c)
                  + np.einsum("ihr,tr->iht", q[..., nope:], r)) * softmax_scale
        scores = np.where(_visible(length, q_len)[:, None, :], scores, -np.inf)
        mx = scores.max(axis=-1, keepdims=True)
        e = np.exp(scores - mx)
        p = e / e.sum(axis=-1, keepdims=True)
        o_lat = np.einsum("iht,tc->ihc", p, c)
        out[bi] = np.einsum("ihc,hdc->ihd", o_lat, w_uv)
    return out
