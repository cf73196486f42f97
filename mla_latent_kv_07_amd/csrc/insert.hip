// Fused cache insert: kv_a RMSNorm on the 512-wide latent, RoPE on the 64-wide
// k_pe, and the write of the 576-number entry into its page slot.
//
// Follows "DeepSeek-V2-Lite 模型结构详解" §四 RMSNorm (row rule; the 精度
// paragraph's wide accumulation, conversion of the normalised row back to the
// activation type, then multiplication by the weight) and "深度解读DeepSeek：
// 源码解读 DeepSeek-V3", section MLA (absorbed branch: kv_norm on the latent
// and apply_rotary_emb on k_pe, both cached at positions start_pos ..).
//
// One wavefront per new token.  Work per token is 1152 bytes in and out, so
// the kernel is bound by launch latency; precision is spent freely: the
// reduction, the normalisation and the rotation run in double and round once
// to bf16.
#include "mla_common.h"

namespace mla {

__global__ __launch_bounds__(64) void insert_kernel(
    const uint16_t* __restrict__ kv_a, const uint16_t* __restrict__ rms_w, double eps,
    double rope_base, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ seq_lens, int q_len, uint16_t* __restrict__ cache) {
#pragma clang fp contract(off)
  const int token = blockIdx.x;  // b * q_len + i
  const int b = token / q_len;
  const int i = token - b * q_len;
  const int lane = threadIdx.x;
  const int pos = seq_lens[b] - q_len + i;
  const int64_t blk = block_table[(int64_t)b * bt_stride + pos / kPage];
  uint16_t* dst = cache + (blk * kPage + pos % kPage) * (int64_t)kEntry;
  const uint16_t* src = kv_a + (int64_t)token * kEntry;

  // ---- latent: 8 consecutive values per lane -------------------------------
  u16x8 xv = *reinterpret_cast<const u16x8*>(src + lane * 8);
  u16x8 wv = *reinterpret_cast<const u16x8*>(rms_w + lane * 8);
  double x[8];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (double)bf16_to_f32(xv[j]);
    ss += x[j] * x[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double denom = sqrt(ss / (double)kLatent + eps);
  u16x8 yv;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float nb = bf16_to_f32(f64_to_bf16(x[j] / denom));  // normalised row in bf16
    yv[j] = f32_to_bf16(bf16_to_f32(wv[j]) * nb);               // exact product, one rounding
  }
  *reinterpret_cast<u16x8*>(dst + lane * 8) = yv;

  // ---- k_pe: lane j < 32 rotates pair (2j, 2j+1) ----------------------------
  if (lane < kRope / 2) {
    const int j = lane;
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(src + kLatent + 2 * j);
    const double re = (double)bf16_to_f32((uint16_t)(pair & 0xffffu));
    const double im = (double)bf16_to_f32((uint16_t)(pair >> 16));
    const double freq = pow(rope_base, -2.0 * (double)j / (double)kRope);
    const double ang = (double)pos * freq;
    double s, c;
    sincos(ang, &s, &c);
    const uint16_t o_re = f64_to_bf16(re * c - im * s);
    const uint16_t o_im = f64_to_bf16(re * s + im * c);
    *reinterpret_cast<uint32_t*>(dst + kLatent + 2 * j) = (uint32_t)o_re | ((uint32_t)o_im << 16);
  }
}

// FP8 cache insert: the same normalised latent and rotated k_pe as
// insert_kernel, then the latent is stored as E4M3 codes with one
// power-of-two scale per token (the KV quantisation inside the insert of the
// vLLM DeepSeek-V4 notes, section 一; the FP8 cache of "DeepSeek-V3.2-Exp
// unboxing", 初步研读).  Scale: the smallest 2^e with max|y| * 2^-e <= 448
// (E4M3's largest finite value), e in [-126, 127], e = 0 for an all-zero row;
// codes round to nearest even (the gfx950 conversion, which only overflows
// above 464, a value the scale rules out).  Row: codes, rope (bf16), scale
// byte e + 127, zeros.
__global__ __launch_bounds__(64) void insert_fp8_kernel(
    const uint16_t* __restrict__ kv_a, const uint16_t* __restrict__ rms_w, double eps,
    double rope_base, const int32_t* __restrict__ block_table, int bt_stride,
    const int32_t* __restrict__ seq_lens, int q_len, uint8_t* __restrict__ cache) {
#pragma clang fp contract(off)
  const int token = blockIdx.x;  // b * q_len + i
  const int b = token / q_len;
  const int i = token - b * q_len;
  const int lane = threadIdx.x;
  const int pos = seq_lens[b] - q_len + i;
  const int64_t blk = block_table[(int64_t)b * bt_stride + pos / kPage];
  uint8_t* dst = cache + (blk * kPage + pos % kPage) * (int64_t)kFp8EntryBytes;
  const uint16_t* src = kv_a + (int64_t)token * kEntry;

  // ---- latent: RMSNorm exactly as insert_kernel, 8 values per lane ---------
  u16x8 xv = *reinterpret_cast<const u16x8*>(src + lane * 8);
  u16x8 wv = *reinterpret_cast<const u16x8*>(rms_w + lane * 8);
  double x[8];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (double)bf16_to_f32(xv[j]);
    ss += x[j] * x[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  const double denom = sqrt(ss / (double)kLatent + eps);
  float y[8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float nb = bf16_to_f32(f64_to_bf16(x[j] / denom));
    y[j] = bf16_to_f32(f32_to_bf16(bf16_to_f32(wv[j]) * nb));  // the bf16 cache value
    amax = fmaxf(amax, fabsf(y[j]));
  }
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

  // ---- k_pe: lane j < 32 rotates pair (2j, 2j+1), as insert_kernel --------
  if (lane < kRope / 2) {
    const int j = lane;
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(src + kLatent + 2 * j);
    const double re = (double)bf16_to_f32((uint16_t)(pair & 0xffffu));
    const double im = (double)bf16_to_f32((uint16_t)(pair >> 16));
    const double freq = pow(rope_base, -2.0 * (double)j / (double)kRope);
    const double ang = (double)pos * freq;
    double s, c;
    sincos(ang, &s, &c);
    const uint16_t o_re = f64_to_bf16(re * c - im * s);
    const uint16_t o_im = f64_to_bf16(re * s + im * c);
    *reinterpret_cast<uint32_t*>(dst + kFp8RopeOff + 4 * j) =
        (uint32_t)o_re | ((uint32_t)o_im << 16);
  }
  // ---- scale byte and zero padding: the row's last 16 bytes ----------------
  if (lane == 0)
    *reinterpret_cast<u32x4*>(dst + kFp8ScaleOff) = u32x4{(uint32_t)(e + 127), 0u, 0u, 0u};
}

hipError_t launch_insert(const uint16_t* kv_a, const uint16_t* rms_w, float eps, float rope_base,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int batch, int q_len, uint16_t* cache, hipStream_t stream) {
  hipLaunchKernelGGL(insert_kernel, dim3(batch * q_len), dim3(64), 0, stream, kv_a, rms_w,
                     (double)eps, (double)rope_base, block_table, bt_stride, seq_lens, q_len,
                     cache);
  return hipGetLastError();
}

hipError_t launch_insert_fp8(const uint16_t* kv_a, const uint16_t* rms_w, float eps,
                             float rope_base, const int32_t* block_table, int bt_stride,
                             const int32_t* seq_lens, int batch, int q_len, uint8_t* cache,
                             hipStream_t stream) {
  hipLaunchKernelGGL(insert_fp8_kernel, dim3(batch * q_len), dim3(64), 0, stream, kv_a, rms_w,
                     (double)eps, (double)rope_base, block_table, bt_stride, seq_lens, q_len,
                     cache);
  return hipGetLastError();
}

}  // namespace mla
