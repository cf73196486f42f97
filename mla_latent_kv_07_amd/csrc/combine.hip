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
// The split partials arrive as bf16 rows.  One workgroup per (head, 32 query
// rows).  The merged latent rows are rounded to bf16 into LDS, then
// D^T = W_UV o_lat^T runs on the bf16 MFMA 16x16x32.  The kernel is a chain
// of dependent memory round trips, so each step issues everything it can at
// once: W_UV (this wavefront's 32 output rows, all of K) is loaded into
// registers at entry, and the partial rows of the first KB splits go out
// together with the log-sum-exps they are weighted by.
#include "mla_common.h"

namespace mla {

constexpr int kCombRows = 32;                 // query rows per workgroup
constexpr int kCombRowBytes = kLatent * 2 + 16;  // padded LDS row (bank spread)

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ o_part,
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
  const int n = lane & 15;
  const int g = lane >> 4;

  // ---- W_UV rows of this wavefront's outputs d in [32w, 32w+32), all of K --
  // (A operand of D^T = W_UV o_lat^T; independent of the merge, so loaded
  // first and in flight during it)
  const uint16_t* wuv = kv_b + ((int64_t)h * (kNope + kVdim) + kNope) * kLatent;
  bf16x8 aw[kLatent / 32][2];
#pragma unroll
  for (int ks = 0; ks < kLatent / 32; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      aw[ks][mt] = *reinterpret_cast<const bf16x8*>(
          wuv + (int64_t)(wave * 32 + mt * 16 + n) * kLatent + 32 * ks + 8 * g);

  // ---- merge: wave w handles rows w*8 .. w*8+7 together; lane covers 8 columns
  // The split weights are lane-parallel (lane s <-> split s, 64 splits per
  // pass); the bf16 partial rows are loaded KB splits at a time with
  // independent loads before any is used.
  {
    constexpr int R = kCombRows / 4;
    constexpr int KB = 4;
    int s0[R], ns[R];
    int64_t srow[R];
    bool live[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int bi = row_base + wave * R + u;
      live[u] = bi < total_rows;
      const int b = live[u] ? bi / q_len : 0;
      const int i = live[u] ? bi - b * q_len : 0;
      srow[u] = i * heads + h;
      s0[u] = plan.seq_start[b];
      const int cnt = plan.seq_count[b];
      ns[u] = live[u] ? cnt : 0;  // 0: every weight is 0
    }
    // Loads never sit in a branch: a split index past the row's last split is
    // clamped to that split (its weight there is 0), and a row past the end
    // reads split 0 of sequence 0 (its result is never stored).
    auto split_of = [&](int u, int s) { return s0[u] + min(s, max(ns[u] - 1, 0)); };
    auto part_row = [&](int u, int s) -> u16x8 {
      const int64_t r = (int64_t)split_of(u, s) * rows_per_seq + srow[u];
      return *reinterpret_cast<const u16x8*>(o_part + r * kLatent + lane * 8);
    };
    auto lse_of = [&](int u, int s) -> float {
      const float v = lse_part[(int64_t)split_of(u, s) * rows_per_seq + srow[u]];
      return s < ns[u] ? v : -INFINITY;
    };
    // first pass: the lse of split `lane` and the partial rows of splits 0..KB-1
    float lse0[R];
    u16x8 v0[R][KB];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      lse0[u] = lse_of(u, lane);
#pragma unroll
      for (int k = 0; k < KB; ++k) v0[u][k] = part_row(u, k);
    }
    int nmax = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) nmax = max(nmax, ns[u]);
    // (KB is a multiple of 4 and divides 64: a batch never straddles two
    // 64-split blocks of weights)
    // max log2-sum-exp over all splits of each row
    float mx[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      mx[u] = lse0[u];
      for (int s = lane + 64; s < ns[u]; s += 64) mx[u] = fmaxf(mx[u], lse_of(u, s));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], o, 64));
    }
    float macc[R][8];
    float wsum[R];
    // weights of splits 0..63 (lane s <-> split s)
    float w_l[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
      w_l[u] = lse0[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lse0[u] - mx[u]);
    auto accumulate = [&](const u16x8 (&v)[R][KB], int s, bool first) {
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const float w = __shfl(w_l[u], (s + k) & 63, 64);  // 0 beyond ns (lse -inf)
          wsum[u] = (first && k == 0) ? w : wsum[u] + w;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            macc[u][e] = (first && k == 0) ? w * bf16_to_f32(v[u][k][e])
                                           : macc[u][e] + w * bf16_to_f32(v[u][k][e]);
        }
    };
    accumulate(v0, 0, true);
    for (int s = KB; s < nmax; s += KB) {
      if ((s & 63) == 0) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const float lse = lse_of(u, s + lane);
          w_l[u] = lse == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lse - mx[u]);
        }
      }
      u16x8 v[R][KB];
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int k = 0; k < KB; ++k)
          v[u][k] = part_row(u, s + k);
      accumulate(v, s, false);
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const float inv = wsum[u] > 0.f ? 1.f / wsum[u] : 0.f;
      u16x8 packed;
#pragma unroll
      for (int e = 0; e < 8; ++e) packed[e] = live[u] ? f32_to_bf16(macc[u][e] * inv) : 0;
      *reinterpret_cast<u16x8*>(olat + (wave * R + u) * kCombRowBytes + lane * 16) = packed;
    }
  }
  __syncthreads();

  // ---- projection: wave w computes d in [32w, 32w+32) for all 32 rows -------
  constexpr int NT = kCombRows / 16;
  f32x4 acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kLatent / 32; ++ks) {
    bf16x8 bv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      bv[nt] = *reinterpret_cast<const bf16x8*>(olat + (nt * 16 + n) * kCombRowBytes +
                                                (32 * ks + 8 * g) * 2);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[ks][mt], bv[nt], acc[mt][nt], 0,
                                                              0, 0);
  }
  // D^T[d][row]: lane holds d = 16mt + 4g + i of row n of tile nt
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
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

hipError_t launch_combine(const uint16_t* o_part, const float* lse_part, PlanView plan,
                          const uint16_t* kv_b, int heads, int q_len, int batch, uint16_t* out,
                          hipStream_t stream) {
  const int rows = batch * q_len;
  dim3 grid(heads, (rows + kCombRows - 1) / kCombRows);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, o_part, lse_part, plan, kv_b,
                     heads, q_len, batch, out);
  return hipGetLastError();
}

}  // namespace mla
