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
// In the fused step (the insert and the query preparation in one launch, as
// the vLLM DeepSeek-V4 notes, section 一, fuse the query-side RoPE with the
// cache insert) the launch also writes the new tokens' cache entries
// (insert_dev.h, one wavefront per token), and the same wavefront rotates
// the token's q_pe of every head: the angles are those of the token's own
// k_pe, computed once per token.
//
// One workgroup per (head, 128 latent columns); W_UK[h][:, cols] (32 KB) is
// staged in LDS and read as the MFMA A operand with the gfx950 transposing
// LDS read (the contraction index d is W_UK's row index).  The query rows are
// the B operand, straight from global memory.  Result rows are written with
// 8-byte stores (4 consecutive latent columns per lane).
#include "insert_dev.h"
#include "mla_common.h"
#include "plan.h"

namespace mla {

constexpr int kQaCols = 128;                 // latent columns per workgroup
constexpr int kQaStride = kQaCols * 2 + 32;  // padded LDS row of W_UK (bytes)

constexpr int kPrepSmem = kNope * kQaStride > kPlanSmemBytes ? kNope * kQaStride : kPlanSmemBytes;
static_assert(kPlanThreads == 256, "the plan runs on one 256-thread workgroup");

// MODE 0: q_pe arrives rotated.  MODE 1 / 2: the fused step with the bf16 /
// FP8 cache: q_pe arrives unrotated, and the new tokens are inserted.
// Block 0: the split plan (independent work, hidden under the absorption).
// Blocks 1 .. n_ins (MODE > 0): one per new token, its insert and q_pe.
// Then 4H blocks: absorption of head k/4, latent columns (k%4)*128 .. +128.
// q_abs's rope part of query row `token`, for the heads of one of the
// kQpeWaves wavefronts that do it: q_pe rotated at the token's position (each
// head's 32 pairs rotated by the 32 angles of that position, see rope_angle),
// times q_scale, rounded to bf16.  Lane L of wavefront slot w handles pair
// L % 32 of heads 2w + L / 32 + 2 kQpeWaves u.  `heads` is even, so whether
// head 2w + 2 kQpeWaves u + L / 32 exists is the same for both halves of the
// wavefront: the per-head test is uniform (w is a scalar).  The pairs are
// loaded first (load_query_pe), so their latency is paid once.
constexpr int kQpeWaves = 3;
constexpr int kQpeBatch = (128 + 2 * kQpeWaves - 1) / (2 * kQpeWaves);
struct QueryPe {
  uint32_t pair[kQpeBatch];
};

__device__ __forceinline__ void load_query_pe(const uint16_t* __restrict__ q, int heads,
                                              int token, int lane, int w, QueryPe& qp) {
  const uint16_t* src =
      q + ((int64_t)token * heads + 2 * w + (lane >> 5)) * kQk + kNope + 2 * (lane & 31);
#pragma unroll
  for (int u = 0; u < kQpeBatch; ++u)
    if (2 * w + 2 * kQpeWaves * u < heads)
      qp.pair[u] = *reinterpret_cast<const uint32_t*>(src + u * 2 * kQpeWaves * kQk);
}

__device__ __forceinline__ void rotate_query_pe(const QueryPe& qp, int heads, float q_scale,
                                                uint16_t* __restrict__ q_abs, int token, int lane,
                                                int w, double c, double s) {
  uint16_t* dst =
      q_abs + ((int64_t)token * heads + 2 * w + (lane >> 5)) * kEntry + kLatent + 2 * (lane & 31);
#pragma unroll
  for (int u = 0; u < kQpeBatch; ++u) {
    if (2 * w + 2 * kQpeWaves * u < heads) {
      const uint32_t rot = rotate_pair(qp.pair[u], c, s);
      const uint32_t lo = f32_to_bf16(bf16_to_f32((uint16_t)(rot & 0xffffu)) * q_scale);
      const uint32_t hi = f32_to_bf16(bf16_to_f32((uint16_t)(rot >> 16)) * q_scale);
      *reinterpret_cast<uint32_t*>(dst + u * 2 * kQpeWaves * kEntry) = lo | (hi << 16);
    }
  }
}

// The absorption blocks start at the first multiple of 8 after the plan and
// insert blocks (the blocks in between return at once), and absorption block
// a = 8 s + x takes head x + 8 (s / 4), column chunk s % 4: the four chunks
// of a head then have the same block id modulo 8, i.e. run on the same XCD
// (blocks are dealt to the eight XCDs in turn), and read the head's query
// rows through one L2.
static_assert(kLatent / kQaCols == 4, "four column chunks per head");
__host__ __device__ constexpr int absorb_base(int n_ins) { return (1 + n_ins + 7) & ~7; }

template <int MODE>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ kv_b, int heads,
                                                   int rows, float q_scale,
                                                   uint16_t* __restrict__ q_abs, PlanArgs pa,
                                                   InsertArgs ia, int n_ins) {
  __shared__ __attribute__((aligned(16))) char smem[kPrepSmem];
  if (blockIdx.x == 0) {
    plan_block(pa, (MLA_LDS char*)smem);
    return;
  }
  if (MODE > 0 && (int)blockIdx.x <= n_ins) {
    // one workgroup per new token: wavefront 0 inserts the token, wavefronts
    // 1 .. kQpeWaves rotate its q_pe of every head (heads <= 128); each
    // computes the token's 32 angles, the same rotation for k_pe and q_pe
    static_assert(kQpeWaves + 1 == 4, "the insert workgroup is four wavefronts");
    const int token = blockIdx.x - 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    QueryPe qp;
    if (wave > 0) load_query_pe(q, heads, token, lane, wave - 1, qp);
    const int pos = token_pos(ia, token);
    double c, s;
    rope_angle(pos, ia.freq[lane & 31], c, s);
    if (wave == 0) {
      if (MODE == 1)
        insert_token_bf16(ia, token, lane, pos, c, s);
      else
        insert_token_fp8(ia, token, lane, pos, c, s);
    } else {
      rotate_query_pe(qp, heads, q_scale, q_abs, token, lane, wave - 1, c, s);
    }
    return;
  }
  MLA_LDS char* w_lds = (MLA_LDS char*)smem;
  const int base = absorb_base(MODE > 0 ? n_ins : 0);
  if ((int)blockIdx.x < base) return;
  const int ab = blockIdx.x - base;
  const int h = (ab & 7) + 8 * (ab >> 5);  // heads % 8 == 0
  const int nc = (ab >> 3) & 3;            // column chunk
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
  // q_pe times the scale (done once per head, by column chunk 0; in the
  // fused step the insert wavefronts write it, rotated)
  if (MODE == 0 && nc == 0) {
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
  hipLaunchKernelGGL(prep_kernel<0>, dim3(absorb_base(0) + heads * (kLatent / kQaCols)), dim3(256),
                     0, stream,
                     q, kv_b, heads, rows, q_scale, q_abs, pa, InsertArgs{}, 0);
  return hipGetLastError();
}

hipError_t launch_prep_step(bool fp8, const InsertArgs& ia, const uint16_t* q,
                            const uint16_t* kv_b, int heads, int rows, float q_scale,
                            uint16_t* q_abs, const int32_t* seq_lens, int batch, int max_pages,
                            int slots, int max_items, int splits_hint, float item_cost_pages,
                            PlanView plan, hipStream_t stream) {
  PlanArgs pa{seq_lens, batch, max_pages, slots, max_items, splits_hint, item_cost_pages, plan};
  const int n_ins = rows;  // one workgroup per new token
  const dim3 grid(absorb_base(n_ins) + heads * (kLatent / kQaCols));
  if (fp8)
    hipLaunchKernelGGL(prep_kernel<2>, grid, dim3(256), 0, stream, q, kv_b, heads, rows, q_scale,
                       q_abs, pa, ia, n_ins);
  else
    hipLaunchKernelGGL(prep_kernel<1>, grid, dim3(256), 0, stream, q, kv_b, heads, rows, q_scale,
                       q_abs, pa, ia, n_ins);
  return hipGetLastError();
}

}  // namespace mla
