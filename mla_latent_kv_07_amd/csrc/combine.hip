// Merge of the split-KV partial results and the per-head output projection.
//
// Merge: the softmax over all positions of a sequence equals the per-item
// softmaxes weighted by exp2(lse_item - max lse) / sum (the log-sum-exp form
// of the softmax in the MLA forward pass; the tag page's excerpt on decode
// context parallelism describes the same merge across GPUs).
// Projection: "深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA, "(b)
// 优化实现", last einsum: out[h] = o_lat[h] W_UV[h]^T with W_UV[h] the last
// 128 rows of head h's kv_b block; "DeepSeek-V2-Lite 模型结构详解" §五 gives
// the identity that moves W_UV behind the weighted sum.
//
// One workgroup per (head, 64 query rows).  The merged latent rows are
// rounded to bf16 into LDS, then D^T = W_UV o_lat^T runs on the bf16 MFMA
// 16x16x32 with W_UV streamed from global memory (each head's 128 KB block is
// read once per workgroup).
#include "mla_common.h"

namespace mla {

constexpr int kCombRows = 64;                 // query rows per workgroup
constexpr int kCombRowBytes = kLatent * 2 + 16;  // padded LDS row (bank spread)

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      PlanView plan,
                                                      const uint16_t* __restrict__ kv_b,
                                                      int heads, int q_len, int batch,
                                                      uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char olat[kCombRows * kCombRowBytes];
  const int h = blockIdx.x;
  const int row_base = blockIdx.y * kCombRows;  // first (b, i) row of this workgroup
  const int total_rows = batch * q_len;
  const int rows_per_seq = heads * q_len;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;

  // ---- merge: wave w handles rows w*16 .. w*16+15, lane covers 8 columns ----
  for (int rr = 0; rr < kCombRows / 4; ++rr) {
    const int lr = wave * (kCombRows / 4) + rr;
    const int bi = row_base + lr;
    u16x8 packed;
    if (bi < total_rows) {
      const int b = bi / q_len;
      const int i = bi - b * q_len;
      const int srow = i * heads + h;
      const int s0 = plan.seq_start[b];
      const int ns = plan.seq_count[b];
      float mx = -INFINITY;
      for (int s = 0; s < ns; ++s)
        mx = fmaxf(mx, lse_part[(int64_t)(s0 + s) * rows_per_seq + srow]);
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      float wsum = 0.f;
      for (int s = 0; s < ns; ++s) {
        const int64_t r = (int64_t)(s0 + s) * rows_per_seq + srow;
        const float lse = lse_part[r];
        const float w = lse == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lse - mx);
        wsum += w;
        const f32x4* src = reinterpret_cast<const f32x4*>(o_part + r * kLatent + lane * 8);
        const f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] += w * v0[j];
          acc[4 + j] += w * v1[j];
        }
      }
      const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) packed[j] = f32_to_bf16(acc[j] * inv);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) packed[j] = 0;
    }
    *reinterpret_cast<u16x8*>(olat + lr * kCombRowBytes + lane * 16) = packed;
  }
  __syncthreads();

  // ---- projection: wave w computes d in [32w, 32w+32) for all 64 rows -------
  const int n = lane & 15;
  const int g = lane >> 4;
  f32x4 acc[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wuv = kv_b + ((int64_t)h * (kNope + kVdim) + kNope) * kLatent;
#pragma unroll 4
  for (int ks = 0; ks < kLatent / 32; ++ks) {
    bf16x8 av[2], bv[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      av[mt] = *reinterpret_cast<const bf16x8*>(wuv + (int64_t)(wave * 32 + mt * 16 + n) * kLatent +
                                                32 * ks + 8 * g);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      bv[nt] = *reinterpret_cast<const bf16x8*>(olat + (nt * 16 + n) * kCombRowBytes +
                                                (32 * ks + 8 * g) * 2);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
  }
  // D^T[d][row]: lane holds d = 16mt + 4g + i of row n of tile nt
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int bi = row_base + nt * 16 + n;
    if (bi >= total_rows) continue;
    uint16_t* dst = out + ((int64_t)bi * heads + h) * kVdim + wave * 32;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      u16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(acc[mt][nt][i]);
      *reinterpret_cast<u16x4*>(dst + mt * 16 + 4 * g) = v;
    }
  }
}

hipError_t launch_combine(const float* o_part, const float* lse_part, PlanView plan,
                          const uint16_t* kv_b, int heads, int q_len, int batch, uint16_t* out,
                          hipStream_t stream) {
  const int rows = batch * q_len;
  dim3 grid(heads, (rows + kCombRows - 1) / kCombRows);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, o_part, lse_part, plan, kv_b,
                     heads, q_len, batch, out);
  return hipGetLastError();
}

}  // namespace mla
