// Per-token cache insert, shared by the insert kernels and the fused step
// (insert + query preparation in one launch).
//
// Follows "DeepSeek-V2-Lite 模型结构详解" §四 RMSNorm (row rule; the 精度
// paragraph's wide accumulation, conversion of the normalised row back to the
// activation type, then multiplication by the weight) and "深度解读DeepSeek：
// 源码解读 DeepSeek-V3", section MLA (absorbed branch: kv_norm on the latent
// and apply_rotary_emb on k_pe, both cached at positions start_pos ..).
//
// One wavefront per new token.  Work per token is 1152 bytes in and out, so
// precision is spent freely: the reduction, the normalisation and the
// rotation run in double and round once to bf16.
#pragma once

#include <cmath>

#include "mla_common.h"

namespace mla {

struct InsertArgs {
  const uint16_t* kv_a;       // [B * q_len, 576] bf16: latent then k_pe (not rotated)
  const uint16_t* rms_w;      // [512] bf16
  double eps;
  double rope_base;
  const int32_t* block_table;
  int bt_stride;
  const int32_t* seq_lens;    // after the insert
  int q_len;
  void* cache;                // bf16 [.., 64, 576] or FP8 rows [.., 64, 656]
  double freq[kRope / 2];     // base^(-2j/64), set on the host by with_rope_freq
};

// The arguments with the rotary frequencies filled in, computed once on the
// host in double (the same expression the angle needs, so the kernels spend no
// pow per lane).
inline InsertArgs with_rope_freq(InsertArgs a) {
  for (int j = 0; j < kRope / 2; ++j) a.freq[j] = std::pow(a.rope_base, -2.0 * j / (double)kRope);
  return a;
}

// double -> bf16, rounded to nearest even, in integer arithmetic on the
// double's bits u: adding 2^44 - 1 plus the lowest kept bit and dropping the
// 45 low bits rounds the 52-bit mantissa to bf16's 7 (a carry moves into the
// exponent, and past the largest exponent gives infinity), then the exponent
// is rebiased from 1023 to 127.  That covers every result that is a normal
// bf16 or an overflow to infinity (biased exponent 897 .. 1150) and
// magnitudes below 2^-134, which round to a signed zero (exponent 0 .. 888).
// `covered` is false for the rest (bf16's subnormal band 889 .. 896, and
// 1151 .. 2047: beyond bf16's range, inf, NaN), whose value this does not
// give.  Host and device code, so that it can be checked on the CPU.
__host__ __device__ inline uint16_t f64_bits_to_bf16(uint64_t u, bool& covered) {
  const uint32_t e = (uint32_t)(u >> 52) & 0x7ffu;
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint32_t t = (uint32_t)((u + 0x00000fffffffffffull + ((u >> 45) & 1u)) >> 45);
  covered = e <= 888u || e - 897u <= 1150u - 897u;
  // (a mask, not a select: the zero case costs no branch around the rest)
  const uint32_t keep = 0u - (uint32_t)(e > 888u);
  return (uint16_t)(sign | (((t & 0x3ffffu) - (896u << 7)) & keep));
}

// f64_to_bf16's value without its emulated round-toward-zero conversion: the
// integer rounding above, and f64_to_bf16 only when some lane of the
// wavefront has an input it does not cover.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
  bool covered;
  uint16_t r = f64_bits_to_bf16((uint64_t)__double_as_longlong(d), covered);
  if (__builtin_amdgcn_ballot_w64(!covered) != 0) {
    if (!covered) r = f64_to_bf16(d);
  }
  return r;
}

// RoPE of one interleaved pair (re, im) = elements (2j, 2j+1) of a 64-wide
// rotary part at position pos ("深度解读DeepSeek：源码解读 DeepSeek-V3",
// section MLA, apply_rotary_emb with the complex freqs_cis of the Transformer
// constructor): angle pos * base^(-2j/64), rotation in double, each result
// rounded once to bf16.  Returns the rotated pair packed as (re | im << 16).
// (rope_angle: the cosine and sine of pair j's angle, freq = base^(-2j/64)
// from InsertArgs::freq; rotate_pair: the rotation of one packed pair by
// them.)
__device__ __forceinline__ void rope_angle(int pos, double freq, double& c, double& s) {
#pragma clang fp contract(off)
  const double ang = (double)pos * freq;
  sincos(ang, &s, &c);
}

__device__ __forceinline__ uint32_t rotate_pair(uint32_t pair, double c, double s) {
#pragma clang fp contract(off)
  const double re = (double)bf16_to_f32((uint16_t)(pair & 0xffffu));
  const double im = (double)bf16_to_f32((uint16_t)(pair >> 16));
  const uint16_t o_re = f64_to_bf16_rne(re * c - im * s);
  const uint16_t o_im = f64_to_bf16_rne(re * s + im * c);
  return (uint32_t)o_re | ((uint32_t)o_im << 16);
}


// The RMSNorm of the token's latent, 8 consecutive values per lane, as the
// bf16 cache values (widened to float, exactly).
__device__ __forceinline__ void rmsnorm_lane(const InsertArgs& a, const uint16_t* src, int lane,
                                             float (&y)[8]) {
#pragma clang fp contract(off)
  const u16x8 xv = *reinterpret_cast<const u16x8*>(src + lane * 8);
  const u16x8 wv = *reinterpret_cast<const u16x8*>(a.rms_w + lane * 8);
  double x[8];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (double)bf16_to_f32(xv[j]);
    ss += x[j] * x[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double denom = sqrt(ss / (double)kLatent + a.eps);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float nb = bf16_to_f32(f64_to_bf16_rne(x[j] / denom));  // normalised row in bf16
    y[j] = bf16_to_f32(f32_to_bf16(bf16_to_f32(wv[j]) * nb));  // exact product, one rounding
  }
}

// Position of token `token` (= b * q_len + i) in its sequence.
__device__ __forceinline__ int token_pos(const InsertArgs& a, int token) {
  const int b = token / a.q_len;
  return a.seq_lens[b] - a.q_len + (token - b * a.q_len);
}

// Insert token `token` (= b * q_len + i, at position pos) into the bf16
// cache; the calling wavefront's 64 lanes do it together.  (c, s): the
// rotation of pair lane % 32 at pos (rope_angle).
__device__ __forceinline__ void insert_token_bf16(const InsertArgs& a, int token, int lane,
                                                  int pos, double c, double s) {
  const int b = token / a.q_len;
  const int64_t blk = a.block_table[(int64_t)b * a.bt_stride + pos / kPage];
  uint16_t* dst = static_cast<uint16_t*>(a.cache) + (blk * kPage + pos % kPage) * (int64_t)kEntry;
  const uint16_t* src = a.kv_a + (int64_t)token * kEntry;
  float y[8];
  rmsnorm_lane(a, src, lane, y);
  u16x8 yv;
#pragma unroll
  for (int j = 0; j < 8; ++j) yv[j] = (uint16_t)(__float_as_uint(y[j]) >> 16);  // y holds bf16 values
  *reinterpret_cast<u16x8*>(dst + lane * 8) = yv;
  // k_pe: lane j < 32 rotates pair (2j, 2j+1)
  if (lane < kRope / 2) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(src + kLatent + 2 * lane);
    *reinterpret_cast<uint32_t*>(dst + kLatent + 2 * lane) = rotate_pair(pair, c, s);
  }
}

// FP8 cache insert: the same normalised latent and rotated k_pe as the bf16
// insert, then the latent is stored as E4M3 codes with one power-of-two scale
// per token (the KV quantisation inside the insert of the vLLM DeepSeek-V4
// notes, section 一; the FP8 cache of "DeepSeek-V3.2-Exp unboxing", 初步研读).
// Scale: the smallest 2^e with max|y| * 2^-e <= 448 (E4M3's largest finite
// value), e in [-126, 127], e = 0 for an all-zero row; codes round to nearest
// even (the gfx950 conversion, which only overflows above 464, a value the
// scale rules out).  Row: codes, rope (bf16), scale byte e + 127, zeros.
__device__ __forceinline__ void insert_token_fp8(const InsertArgs& a, int token, int lane,
                                                 int pos, double c, double s) {
  const int b = token / a.q_len;
  const int64_t blk = a.block_table[(int64_t)b * a.bt_stride + pos / kPage];
  uint8_t* dst =
      static_cast<uint8_t*>(a.cache) + (blk * kPage + pos % kPage) * (int64_t)kFp8EntryBytes;
  const uint16_t* src = a.kv_a + (int64_t)token * kEntry;
  float y[8];
  rmsnorm_lane(a, src, lane, y);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(y[j]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  // amax = f * 2^E with f in [0.5, 1); 448 = 0.875 * 2^9
  int e = 0;
  if (amax > 0.f) {
    int E;
    const float f = frexpf(amax, &E);
    e = f <= 0.875f ? E - 9 : E - 8;
    e = e < -126 ? -126 : (e > 127 ? 127 : e);
  }
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(y[0], -e), ldexpf(y[1], -e), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(y[2], -e), ldexpf(y[3], -e), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(y[4], -e), ldexpf(y[5], -e), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(y[6], -e), ldexpf(y[7], -e), hi, true);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u32x2*>(dst + lane * 8) = u32x2{lo, hi};
  // k_pe: lane j < 32 rotates pair (2j, 2j+1)
  if (lane < kRope / 2) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(src + kLatent + 2 * lane);
    *reinterpret_cast<uint32_t*>(dst + kFp8RopeOff + 4 * lane) = rotate_pair(pair, c, s);
  }
  // scale byte and zero padding: the row's last 16 bytes
  if (lane == 0)
    *reinterpret_cast<u32x4*>(dst + kFp8ScaleOff) = u32x4{(uint32_t)(e + 127), 0u, 0u, 0u};
}

}  // namespace mla
