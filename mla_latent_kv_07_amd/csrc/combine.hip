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

constexpr int kCombRowBytes = kLatent * 2 + 16;  // padded LDS row (bank spread)

// RB query rows per workgroup; SP wavefronts share each row, each merging
// every SP-th split of it (SP = 1: every wavefront owns RB/4 rows and all
// their splits; SP = 4: all four wavefronts take the same RB rows and a
// quarter of the splits each, for few rows with many splits).  Every
// wavefront weighs its splits by exp2(lse - M) with M the row's maximum over
// ALL splits, so the SP partial sums of a row simply add (through LDS).
//
// LATE: W_UV is loaded only after the merge, so that its 128 registers are
// not held through it and two workgroups fit on a CU (launch bounds of two
// waves per SIMD): for launches of several workgroups per CU, where one
// workgroup's merge hides the other's W_UV round trip.
template <int RB, int SP, bool LATE = false>
__global__ __launch_bounds__(256, LATE ? 2 : 1) void combine_kernel(
    const uint16_t* __restrict__ o_part, const float* __restrict__ lse_part, PlanView plan,
    const uint16_t* __restrict__ kv_b, int heads, int q_len, int batch,
    uint16_t* __restrict__ out) {
  constexpr int R = RB * SP / 4;  // rows per wavefront
  static_assert(R * 4 == RB * SP && RB % R == 0, "four wavefronts: RB / R row groups x SP");
  constexpr int kPartBytes = SP > 1 ? 4 * R * kLatent * 4 : 16;  // fp32 partial sums
  __shared__ __attribute__((aligned(16))) char olat[(RB < 16 ? 16 : RB) * kCombRowBytes];
  __shared__ __attribute__((aligned(16))) char part[kPartBytes];
  __shared__ float psum[4 * R];
  const int h = blockIdx.x;
  const int row_base = blockIdx.y * RB;  // first (b, i) row of this workgroup
  const int total_rows = batch * q_len;
  const int rows_per_seq = heads * q_len;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int row_off = (wave / SP) * R;  // first row of this wavefront in the block
  const int ws = wave % SP;             // first split of this wavefront

  // W_UV rows of this wavefront's outputs d in [32w, 32w+32), all of K (the
  // A operand of D^T = W_UV o_lat^T), loaded into registers early so that
  // they are in flight during the merge.  Loads complete in order, so where
  // they go matters: with SP = 1 (one merge pass for the V3 shapes) right
  // after the plan entries, overlapping that round trip; with SP > 1 (several
  // passes) after the first pass's partial rows, which the merge needs first.
  const uint16_t* wuv = kv_b + ((int64_t)h * (kNope + kVdim) + kNope) * kLatent;
  bf16x8 aw[kLatent / 32][2];
  auto load_wuv = [&]() {
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        aw[ks][mt] = *reinterpret_cast<const bf16x8*>(
            wuv + (int64_t)(wave * 32 + mt * 16 + n) * kLatent + 32 * ks + 8 * g);
  };
  constexpr bool kWuvFirst = SP == 1 && !LATE;

  // ---- merge: lane covers 8 columns of each of the wavefront's R rows ------
  // The split weights are lane-parallel (lane s <-> split s, 64 splits per
  // pass); the bf16 partial rows are loaded KB splits at a time with
  // independent loads before any is used.
  {
    constexpr int KB = 4;
    int s0[R], ns[R];
    int64_t srow[R];
    bool live[R];
    // The plan entries of the R rows, lane u <-> row u, in two vector loads,
    // read (the empty asm pins the wait for them) after any loads that can go
    // out before them: waiting for the entries waits for nothing else.
    static_assert(R <= 64, "one lane per row");
    const int lrow = row_base + row_off + min(lane, R - 1);
    const int lb = lrow < total_rows ? lrow / q_len : 0;
    const int li = lrow < total_rows ? lrow - lb * q_len : 0;
    int p_start = plan.seq_start[lb];
    int p_count = plan.seq_count[lb];
    if constexpr (kWuvFirst) load_wuv();
    asm volatile("" : "+v"(p_start), "+v"(p_count) : : "memory");
#pragma unroll
    for (int u = 0; u < R; ++u) {
      live[u] = row_base + row_off + u < total_rows;
      srow[u] = __builtin_amdgcn_readlane(li, u) * heads + h;
      s0[u] = __builtin_amdgcn_readlane(p_start, u);
      ns[u] = live[u] ? __builtin_amdgcn_readlane(p_count, u) : 0;  // 0: every weight is 0
    }
    // Loads never sit in a branch: a split index past the row's last split is
    // clamped to that split (its weight there is 0), and a row past the end
    // reads split 0 of sequence 0 (its result is never stored).
    auto split_of = [&](int u, int s) { return s0[u] + min(s, max(ns[u] - 1, 0)); };
    auto part_row = [&](int u, int s) -> u16x8 {
      const int64_t r = (int64_t)split_of(u, s) * rows_per_seq + srow[u];
      return *reinterpret_cast<const u16x8*>(o_part + r * kLatent + lane * 8);
    };
    auto lse_raw = [&](int u, int s) -> float {
      return lse_part[(int64_t)split_of(u, s) * rows_per_seq + srow[u]];
    };
    auto lse_of = [&](int u, int s) -> float { return s < ns[u] ? lse_raw(u, s) : -INFINITY; };
    // this wavefront's k-th split is ws + SP k; the first pass: the partial
    // rows of this wavefront's first KB splits, then the lse of splits 0..63
    // (lane s); nothing waits before the last of them is issued.
    float lse0[R];
    u16x8 v0[R][KB];
#pragma unroll
    for (int u = 0; u < R; ++u)
#pragma unroll
      for (int k = 0; k < KB; ++k) v0[u][k] = part_row(u, ws + SP * k);
#pragma unroll
    for (int u = 0; u < R; ++u) lse0[u] = lse_raw(u, lane);
    if constexpr (!kWuvFirst && !LATE) {
      asm volatile("" : : : "memory");  // W_UV behind the first pass's loads
      load_wuv();
    }
    // the lse values are used (masked past the row's last split) only from
    // here on: no wait is scheduled between the loads above
#pragma unroll
    for (int u = 0; u < R; ++u) {
      asm volatile("" : "+v"(lse0[u]) : : "memory");
      lse0[u] = lane < ns[u] ? lse0[u] : -INFINITY;
    }
    int nmax = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) nmax = max(nmax, ns[u]);
    // max log2-sum-exp over all splits of each row (every wavefront: the same M)
    float mx[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      mx[u] = lse0[u];
      for (int s = lane + 64; s < ns[u]; s += 64) mx[u] = fmaxf(mx[u], lse_of(u, s));
    }
    // (the rows' reductions interleaved: one exchange latency per step for
    // all R rows)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int u = 0; u < R; ++u) mx[u] = fmaxf(mx[u], __shfl_xor(mx[u], o, 64));
    float macc[R][8];
    float wsum[R];
    // weights of splits 0..63 (lane s <-> split s)
    float w_l[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
      w_l[u] = lse0[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lse0[u] - mx[u]);
    // (KB SP is a multiple of 4 dividing 64: a batch never straddles two
    // 64-split blocks of weights)
    auto accumulate = [&](const u16x8 (&v)[R][KB], int s, bool first) {
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          // (the split index is uniform: a lane read, not an LDS permute)
          const float w = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l[u]), (s + SP * k) & 63));
          // (0 beyond ns: lse -inf)
          wsum[u] = (first && k == 0) ? w : wsum[u] + w;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            macc[u][e] = (first && k == 0) ? w * bf16_to_f32(v[u][k][e])
                                           : macc[u][e] + w * bf16_to_f32(v[u][k][e]);
        }
    };
    accumulate(v0, ws, true);
    for (int s = ws + SP * KB; s < nmax; s += SP * KB) {
      if ((s >> 6) != ((s - SP * KB) >> 6)) {
        // a new block of 64 splits: their weights, lane-parallel
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const float lse = lse_of(u, (s & ~63) + lane);
          w_l[u] = lse == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lse - mx[u]);
        }
      }
      u16x8 v[R][KB];
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int k = 0; k < KB; ++k) v[u][k] = part_row(u, s + SP * k);
      accumulate(v, s, false);
    }
    if constexpr (SP == 1) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const float inv = wsum[u] > 0.f ? 1.f / wsum[u] : 0.f;
        u16x8 packed;
#pragma unroll
        for (int e = 0; e < 8; ++e) packed[e] = live[u] ? f32_to_bf16(macc[u][e] * inv) : 0;
        *reinterpret_cast<u16x8*>(olat + (row_off + u) * kCombRowBytes + lane * 16) = packed;
      }
    } else {
      // the SP partial sums of each row: through LDS (wavefront w's row u
      // at w R + u), then wavefront w finishes block rows w, w + 4, ..
      float* pp = reinterpret_cast<float*>(part);
#pragma unroll
      for (int u = 0; u < R; ++u) {
#pragma unroll
        for (int e = 0; e < 8; e += 4)
          *reinterpret_cast<f32x4*>(pp + ((wave * R + u) * kLatent) + lane * 8 + e) =
              f32x4{macc[u][e], macc[u][e + 1], macc[u][e + 2], macc[u][e + 3]};
        if (lane == 0) psum[wave * R + u] = wsum[u];
      }
      __syncthreads();
      for (int r = wave; r < RB; r += 4) {
        const int w0 = (r / R) * SP;  // the wavefronts of row r's group
        const int u = r % R;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float ws_all = 0.f;
#pragma unroll
        for (int k = 0; k < SP; ++k) {
          ws_all += psum[(w0 + k) * R + u];
#pragma unroll
          for (int e = 0; e < 8; e += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(pp + (((w0 + k) * R + u) * kLatent) +
                                                            lane * 8 + e);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[e + c] += t[c];
          }
        }
        const float inv = ws_all > 0.f ? 1.f / ws_all : 0.f;
        const bool lv = row_base + r < total_rows;
        u16x8 packed;
#pragma unroll
        for (int e = 0; e < 8; ++e) packed[e] = lv ? f32_to_bf16(acc[e] * inv) : 0;
        *reinterpret_cast<u16x8*>(olat + r * kCombRowBytes + lane * 16) = packed;
      }
    }
  }
  if constexpr (RB < 16) {
    // rows RB .. 15 of the 16-row product tile are zero
    for (int u = RB + wave; u < 16; u += 4)
      *reinterpret_cast<u16x8*>(olat + u * kCombRowBytes + lane * 16) = u16x8{};
  }
  __syncthreads();

  if constexpr (LATE) load_wuv();

  // ---- projection: wave w computes d in [32w, 32w+32) for all rows --------
  constexpr int NT = (RB + 15) / 16;
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
    const int r = nt * 16 + n;
    const int bi = row_base + r;
    if (r >= RB || bi >= total_rows) continue;
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
                          int cus, hipStream_t stream) {
  const int rows = batch * q_len;
  // the largest row block that still gives every CU a workgroup: W_UV (128
  // KB per head) is read once per block, so fewer blocks read less; with two
  // or more workgroups per CU the late-W_UV form runs two on a CU at once
  if (heads * ((rows + 31) / 32) >= 2 * cus) {
    hipLaunchKernelGGL((combine_kernel<32, 1, true>), dim3(heads, (rows + 31) / 32), dim3(256), 0,
                       stream, o_part, lse_part, plan, kv_b, heads, q_len, batch, out);
  } else if (heads * ((rows + 31) / 32) >= cus) {
    hipLaunchKernelGGL((combine_kernel<32, 1>), dim3(heads, (rows + 31) / 32), dim3(256), 0,
                       stream, o_part, lse_part, plan, kv_b, heads, q_len, batch, out);
  } else if (heads * ((rows + 15) / 16) >= cus) {
    hipLaunchKernelGGL((combine_kernel<16, 2>), dim3(heads, (rows + 15) / 16), dim3(256), 0,
                       stream, o_part, lse_part, plan, kv_b, heads, q_len, batch, out);
  } else if (heads * ((rows + 7) / 8) >= cus) {
    hipLaunchKernelGGL((combine_kernel<8, 4>), dim3(heads, (rows + 7) / 8), dim3(256), 0, stream,
                       o_part, lse_part, plan, kv_b, heads, q_len, batch, out);
  } else {
    // few rows (a small batch): four-row blocks, so twice as many CUs share
    // the merge (each workgroup still reads its head's W_UV once)
    hipLaunchKernelGGL((combine_kernel<4, 4>), dim3(heads, (rows + 3) / 4), dim3(256), 0, stream,
                       o_part, lse_part, plan, kv_b, heads, q_len, batch, out);
  }
  return hipGetLastError();
}

}  // namespace mla
