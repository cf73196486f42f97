// Query absorption: q_abs[row, h] = c * [ q_nope[row, h] W_UK[h]  |  q_pe[row, h] ]
// with c = softmax_scale * log2(e), so that the decode kernel's scores come
// out of the matrix cores already in log2 units.
//
// "深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA, "(b) 优化实现", first
// einsum (bshd,hdc->bshc): q_nope times the first 128 rows of head h's kv_b
// block; "DeepSeek-V2-Lite 模型结构详解" §五 gives the identity
// q . (W_k c) = (W_k^T q) . c that moves W_UK to the query side.
//
// The same launch also makes the split plan (plan.h) in its first workgroup
// (dispatched first), so the planner's latency hides under the absorption.
//
// One workgroup per (head, 128 latent columns); W_UK[h][:, cols] (32 KB) is
// staged in LDS and read as the MFMA A operand with the gfx950 transposing
// LDS read (the contraction index d is W_UK's row index).  The query rows are
// the B operand, straight from global memory.  Result rows are written with
// 8-byte stores (4 consecutive latent columns per lane).
#include "mla_common.h"
#include "plan.h"

namespace mla {

constexpr int kQaCols = 128;                 // latent columns per workgroup
constexpr int kQaStride = kQaCols * 2 + 32;  // padded LDS row of W_UK (bytes)

constexpr int kPrepSmem = kNope * kQaStride > kPlanSmemBytes ? kNope * kQaStride : kPlanSmemBytes;
static_assert(kPlanThreads == 256, "the plan runs on one 256-thread workgroup");

// Block 0: the split plan (independent work, hidden under the absorption).
// Blocks 1 .. 4H: absorption of head (b-1)/4, latent columns ((b-1)%4)*128 .. +128.
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ kv_b, int heads,
                                                   int rows, float q_scale,
                                                   uint16_t* __restrict__ q_abs, PlanArgs pa) {
  __shared__ __attribute__((aligned(16))) char smem[kPrepSmem];
  if (blockIdx.x == 0) {
    plan_block(pa, (MLA_LDS char*)smem);
    return;
  }
  MLA_LDS char* w_lds = (MLA_LDS char*)smem;
  const int h = (blockIdx.x - 1) / (kLatent / kQaCols);
  const int nc = (blockIdx.x - 1) % (kLatent / kQaCols);  // column chunk
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;

  // Every global load that does not depend on another goes out first: the
  // query rows of the first RT row tiles (B operands), then W_UK.
  constexpr int RT = 4;  // 16-row tiles per round: all their query loads before any MFMA
  auto load_q = [&](int rt0, bf16x8 (&bq)[RT][4]) {
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int rr = min((rt0 + u) * 16 + n, rows - 1);  // rows past the end: never stored
      const int64_t row = (int64_t)rr * heads + h;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        bq[u][ks] = *reinterpret_cast<const bf16x8*>(q + row * kQk + 32 * ks + 8 * g);
    }
  };
  bf16x8 bq[RT][4];
  load_q(0, bq);

  // stage W_UK[h][d][nc*128 .. +128] for d < 128
  const uint16_t* wuk = kv_b + (int64_t)h * (kNope + kVdim) * kLatent + nc * kQaCols;
  constexpr int kStage = (kNope * kQaCols / 8) / 256;
  u16x8 wst[kStage];
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int p = k * 256 + tid;
    wst[k] = *reinterpret_cast<const u16x8*>(wuk + (int64_t)(p >> 4) * kLatent + (p & 15) * 8);
  }
#pragma unroll
  for (int k = 0; k < kStage; ++k) {
    const int p = k * 256 + tid;
    *reinterpret_cast<MLA_LDS u16x8*>(w_lds + (p >> 4) * kQaStride + (p & 15) * 16) = wst[k];
  }
  // q_pe times the scale (done once per head, by column chunk 0)
  if (nc == 0) {
    for (int p = tid; p < rows * 8; p += 256) {
      const int r = p >> 3;
      const int j = p & 7;
      const int64_t row = (int64_t)r * heads + h;
      const u16x8 v = *reinterpret_cast<const u16x8*>(q + row * kQk + kNope + j * 8);
      u16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = f32_to_bf16(bf16_to_f32(v[e]) * q_scale);
      *reinterpret_cast<u16x8*>(q_abs + row * kEntry + kLatent + j * 8) = o;
    }
  }
  __syncthreads();

  // A operands: W_UK^T tiles for this wave's 32 columns, all 4 k-steps of 32 d
  const int s16 = lane & 15;
  const int r = s16 >> 2;
  const int qq = s16 & 3;
  bf16x8 aw[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = wave * 32 + mt * 16 + 4 * qq;
      const int d0 = 32 * ks + 8 * g + r;
      const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (MLA_LDS bf16x4*)(w_lds + d0 * kQaStride + c0 * 2));
      const bf16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (MLA_LDS bf16x4*)(w_lds + (d0 + 4) * kQaStride + c0 * 2));
      aw[mt][ks] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  for (int rt0 = 0; rt0 * 16 < rows; rt0 += RT) {
    if (rt0 > 0) load_q(rt0, bq);
#pragma unroll
    for (int u = 0; u < RT; ++u) {
      const int rr = (rt0 + u) * 16 + n;
      const int64_t row = (int64_t)rr * heads + h;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[mt][ks], bq[u][ks], acc, 0, 0, 0);
        if (rr < rows) {
          u16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(acc[i] * q_scale);
          *reinterpret_cast<u16x4*>(q_abs + row * kEntry + nc * kQaCols + wave * 32 + mt * 16 +
                                    4 * g) = v;
        }
      }
    }
  }
}

hipError_t launch_prep(const uint16_t* q, const uint16_t* kv_b, int heads, int rows,
                       float q_scale, uint16_t* q_abs, const int32_t* seq_lens, int batch,
                       int max_pages,
                       int slots, int max_items, int splits_hint, float item_cost_pages,
                       PlanView plan, hipStream_t stream) {
  PlanArgs pa{seq_lens, batch, max_pages, slots, max_items, splits_hint, item_cost_pages, plan};
  hipLaunchKernelGGL(prep_kernel, dim3(heads * (kLatent / kQaCols) + 1), dim3(256), 0, stream, q,
                     kv_b, heads, rows, q_scale, q_abs, pa);
  return hipGetLastError();
}

}  // namespace mla
