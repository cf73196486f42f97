// Split-KV MLA decode over the paged latent cache (the hot loop).
//
// Absorbed form of "深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA,
// "(b) 优化实现": every head's absorbed query (q_nope W_UK, then q_pe) is
// scored against the single shared 576-wide cache entry of each position,
// the softmax runs over positions, and the weights sum the 512-wide latent
// part of the same entries.  "DeepSeek-V2-Lite 模型结构详解" §五 explains why
// this is the decode form (the cache is read once for all heads; the
// decompression never runs).
//
// gfx950 mapping
//   * One workgroup = one work item (a contiguous page range of one sequence)
//     x one group of up to 128 query rows (row = query index * H + head).
//     Each wavefront owns 16 rows.  All wavefronts share every cache chunk,
//     so the cache is read from HBM once per row group.
//   * Cache chunks (32 or 64 tokens, 36/72 KB) are copied HBM -> LDS by the
//     direct-to-LDS global loads, double buffered; one barrier per chunk.
//     In LDS the 16-byte pieces of each entry are XOR-swizzled by
//     (row / 2) mod 8 so both read patterns below are free of bank conflicts.
//   * Scores are computed transposed, S^T = K Q^T, with the bf16 MFMA
//     16x16x32: the cache tile is the A operand (16 positions x 8 features
//     per lane, one 16-byte LDS read), the query the B operand held in
//     registers for the whole launch.  The result leaves each lane with the
//     scores of ONE head for 4 positions per 16-position tile, which is
//     exactly the B-operand layout the P.V product needs: P never goes
//     through LDS, and the softmax needs only two cross-lane reductions.
//   * O^T = V^T P^T with the same MFMA; the V^T operand comes from LDS with
//     the gfx950 transposing read (ds_read_b64_tr_b16).  The fp32 output
//     accumulator of a lane belongs to one head, so the online-softmax
//     rescale is a per-lane scalar.
//   * Softmax statistics are fp32 in the log2 domain (scale * log2(e) folded
//     into one multiply), P is rounded to bf16 for the MFMA.
// Output per work item: normalised fp32 rows [rows, 512] and their log2-sum-
// exp, merged across items by the combine kernel.
#include "mla_common.h"

namespace mla {

struct DecodeArgs {
  const uint16_t* q_abs;     // [B * rows_per_seq, 576]
  const uint16_t* cache;     // [num_blocks, 64, 576]
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* o_part;             // [max_items, rows_per_seq, 512]
  float* lse_part;           // [max_items, rows_per_seq]
  PlanView plan;
  int bt_stride;
  int heads;
  int q_len;
  int rows_per_seq;
  int row_groups;
  float scale_log2;
};

template <int NW, int CHUNK>
struct DecodeShape {
  static constexpr int kThreads = NW * 64;
  static constexpr int kTiles = CHUNK / 16;                 // 16-position tiles per chunk
  static constexpr int kBufBytes = CHUNK * kEntryBytes;     // one LDS stage
  static constexpr int kPieces = CHUNK * kChunk16;          // 16-byte pieces per chunk
  static constexpr int kPerLane = (kPieces + NW * 64 - 1) / (NW * 64);  // DMA loads per lane
  static_assert(kPieces % 64 == 0, "whole wavefront-sized DMA instructions");
  static_assert(CHUNK == 32 || CHUNK == 64, "chunk of 32 or 64 positions");
};

// Issue the direct-to-LDS copy of one chunk: LDS piece P (16 bytes) holds
// global piece (P % 72) ^ swz(row) of entry row = P / 72.
template <int NW, int CHUNK>
__device__ __forceinline__ void load_chunk(MLA_LDS char* buf, const char* src, int wave,
                                           int lane) {
  using S = DecodeShape<NW, CHUNK>;
#pragma unroll
  for (int k = 0; k < S::kPerLane; ++k) {
    const int base = (k * NW + wave) * 64;  // first piece of this instruction (wave-uniform)
    if (S::kPieces % (NW * 64) != 0 && base >= S::kPieces) break;
    const int p = base + lane;
    const int row = p / kChunk16;
    const int col = p - row * kChunk16;
    const int gcol = col ^ ((row >> 1) & 7);
    const char* g = src + row * kEntryBytes + gcol * 16;
    __builtin_amdgcn_global_load_lds(g, buf + base * 16, 16, 0, 0);
  }
}

// One chunk of CHUNK positions starting at absolute position `t0`.
// MASK: some position in the chunk is beyond this wave's causal limit `tmax`
// (or beyond the sequence end `len`): scores there become -inf and the V
// operand rows beyond `len` are zeroed (their slots may hold anything).
template <int NW, int CHUNK, bool MASK>
__device__ __forceinline__ void compute_chunk(const MLA_LDS char* buf, const bf16x8 (&qreg)[18],
                                              f32x4 (&oacc)[32], float& m_run, float& l_run,
                                              int lane, int t0, int tmax, int len,
                                              float scale_log2) {
  using S = DecodeShape<NW, CHUNK>;
  constexpr int NT = S::kTiles;
  const int n = lane & 15;
  const int gq = lane >> 4;

  // ---- scores: S^T[tile] = K[tile] Q^T over 18 k-steps of 32 features ------
  // Software pipelined: the LDS reads of k-step ks + KPD are issued before the
  // MFMAs of k-step ks; scheduling barriers keep the compiler from hoisting
  // more reads (and spending more registers) than that.
  f32x4 sacc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    constexpr int KPD = NT >= 4 ? 1 : 2;  // k-steps of read-ahead
    const int x = gq ^ ((n >> 1) & 7);
    const int off_even = 16 * x;
    const int off_odd = 16 * (x ^ 4) - 64;
    const MLA_LDS char* rowp = buf + n * kEntryBytes;
    auto kload = [&](int ks, int t) -> bf16x8 {
      const int off = 64 * ks + ((ks & 1) ? off_odd : off_even);
      return *reinterpret_cast<const MLA_LDS bf16x8*>(rowp + t * 16 * kEntryBytes + off);
    };
    bf16x8 kb[KPD + 1][NT];
#pragma unroll
    for (int ks = 0; ks < KPD; ++ks)
#pragma unroll
      for (int t = 0; t < NT; ++t) kb[ks][t] = kload(ks, t);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + KPD < 18) {
#pragma unroll
        for (int t = 0; t < NT; ++t) kb[(ks + KPD) % (KPD + 1)][t] = kload(ks + KPD, t);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks % (KPD + 1)][t], qreg[ks],
                                                          sacc[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- online softmax (log2 domain), per head = per lane column -----------
  float mloc = -INFINITY;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = sacc[t][i] * scale_log2;
      if (MASK) {
        const int pos = t0 + 16 * t + 4 * gq + i;
        s = pos > tmax ? -INFINITY : s;
      }
      sacc[t][i] = s;
      mloc = fmaxf(mloc, s);
    }
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
  const float m_new = fmaxf(m_run, mloc);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
  float psum = 0.f;
  bf16x8 pk[NT / 2];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(sacc[t][i] - m_use);
      psum += p;
      pk[t >> 1][(t & 1) * 4 + i] = (__bf16)p;
    }
  }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
    for (int f = 0; f < 32; ++f) oacc[f] *= alpha;
  }

  // ---- O^T[f] += V^T[f] P^T, V^T read with the transposing LDS load --------
  {
    const int s16 = lane & 15;
    const int r = s16 >> 2;
    const int qq = s16 & 3;
    const int y = (qq >> 1) ^ ((2 * gq + (r >> 1)) & 7);
    const int half = (qq & 1) * 8;
    int troff[4];
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4) troff[f4] = 16 * ((2 * f4) ^ y) + half;
    const MLA_LDS char* rowp = buf + (4 * gq + r) * kEntryBytes;
    // step = (kk, f); the lane's 8 k-slots are positions
    // t0 + 32kk + 4gq + {0..3} and t0 + 32kk + 16 + 4gq + {0..3}
    constexpr int NSTEP = (NT / 2) * 32;
    constexpr int VPD = 3;  // steps of read-ahead
    auto vload = [&](int step) -> bf16x8 {
      const int kk = step >> 5;
      const int f = step & 31;
      const MLA_LDS char* p1 = rowp + (32 * kk) * kEntryBytes + 32 * (f & ~3) + troff[f & 3];
      const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p1);
      const bf16x4 a1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p1 + 16 * kEntryBytes));
      return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // MASK: zero the V elements of positions >= len (bit masks per k-step)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 vkeep[NT / 2];
    if (MASK) {
#pragma unroll
      for (int kk = 0; kk < NT / 2; ++kk) {
        const int pa = t0 + 32 * kk + 4 * gq;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int p0 = pa + (d >> 1) * 16 + (d & 1) * 2;
          vkeep[kk][d] = (p0 < len ? 0x0000ffffu : 0u) | (p0 + 1 < len ? 0xffff0000u : 0u);
        }
      }
    }
    bf16x8 vb[VPD + 1];
#pragma unroll
    for (int st = 0; st < VPD; ++st) vb[st] = vload(st);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      if (st + VPD < NSTEP) vb[(st + VPD) % (VPD + 1)] = vload(st + VPD);
      const int kk = st >> 5;
      const int f = st & 31;
      bf16x8 a = vb[st % (VPD + 1)];
      if (MASK) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        a = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, a) & vkeep[kk]);
      }
      oacc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[kk], oacc[f], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int NW, int CHUNK>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  using S = DecodeShape<NW, CHUNK>;
  __shared__ __attribute__((aligned(1024))) char lds0_raw[S::kBufBytes];
  __shared__ __attribute__((aligned(1024))) char lds1_raw[S::kBufBytes];
  MLA_LDS char* lds0 = (MLA_LDS char*)lds0_raw;
  MLA_LDS char* lds1 = (MLA_LDS char*)lds1_raw;

  // blockIdx -> (item, row group); the row groups of one item land on the
  // same XCD (block ids congruent mod 8) so their chunk reads share that L2.
  const int gid = blockIdx.x;
  const int xcd = gid & 7;
  const int slot = gid >> 3;
  const int item = (slot / a.row_groups) * 8 + xcd;
  const int rg = slot - (slot / a.row_groups) * a.row_groups;
  if (item >= a.plan.header[0]) return;

  const int b = a.plan.item_b[item];
  const int p0 = a.plan.item_p0[item];
  const int p1 = a.plan.item_p1[item];
  const int len = a.seq_lens[b];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int gq = lane >> 4;
  const int row0 = (rg * NW + wave) * 16;       // first row of this wave in the sequence
  const int qi = row0 / a.heads;                // query index shared by the 16 rows
  const int tmax = len - a.q_len + qi;          // last visible position

  // query rows stay in registers: lane holds features 32ks + 8gq .. +8 of row n
  bf16x8 qreg[18];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(
        a.q_abs + ((int64_t)b * a.rows_per_seq + row0 + n) * kEntry + 8 * gq);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = qp[4 * ks];
  }
  f32x4 oacc[32];
#pragma unroll
  for (int f = 0; f < 32; ++f) oacc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int tok_begin = p0 * kPage;
  const int tok_end = min(p1 * kPage, len);
  const int nchunks = (tok_end - tok_begin + CHUNK - 1) / CHUNK;
  const int32_t* bt = a.block_table + (int64_t)b * a.bt_stride;
  const char* cache = reinterpret_cast<const char*>(a.cache);
  auto chunk_src = [&](int j) -> const char* {
    const int t = tok_begin + j * CHUNK;
    const int64_t blk = bt[t / kPage];
    return cache + (blk * kPage + (t % kPage)) * (int64_t)kEntryBytes;
  };
  auto run = [&](const MLA_LDS char* buf, int j) {
    const int t0 = tok_begin + j * CHUNK;
    if (t0 + CHUNK - 1 > tmax)
      compute_chunk<NW, CHUNK, true>(buf, qreg, oacc, m_run, l_run, lane, t0, tmax, len,
                                     a.scale_log2);
    else
      compute_chunk<NW, CHUNK, false>(buf, qreg, oacc, m_run, l_run, lane, t0, tmax, len,
                                      a.scale_log2);
  };

  if (nchunks > 0) load_chunk<NW, CHUNK>(lds0, chunk_src(0), wave, lane);
  for (int j = 0; j < nchunks; j += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 < nchunks) load_chunk<NW, CHUNK>(lds1, chunk_src(j + 1), wave, lane);
    run(lds0, j);
    if (j + 1 >= nchunks) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 2 < nchunks) load_chunk<NW, CHUNK>(lds0, chunk_src(j + 2), wave, lane);
    run(lds1, j + 1);
  }

  // ---- finalise: normalised rows and log2-sum-exp ---------------------------
  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? m_run + __builtin_amdgcn_logf(l) : -INFINITY;
  const int64_t orow = (int64_t)item * a.rows_per_seq + row0 + n;
  float* op = a.o_part + orow * kLatent + 4 * gq;
#pragma unroll
  for (int f = 0; f < 32; ++f) *reinterpret_cast<f32x4*>(op + 16 * f) = oacc[f] * inv;
  if (gq == 0) a.lse_part[orow] = lse;
}

DecodeConfig decode_config(int rows_per_seq) {
  const int groups = rows_per_seq / 16;
  DecodeConfig c;
  if (groups % 4 == 0) {
    c.waves = 4;
    c.chunk = 64;
  } else if (groups % 2 == 0) {
    c.waves = 2;
    c.chunk = 32;
  } else {
    c.waves = 1;
    c.chunk = 32;
  }
  c.lds_bytes = 2 * c.chunk * kEntryBytes;
  c.wgs_per_cu = (160 * 1024) / c.lds_bytes;
  return c;
}

template <int NW, int CHUNK>
static hipError_t launch_t(int grid, const DecodeArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL((decode_kernel<NW, CHUNK>), dim3(grid), dim3(NW * 64), 0, stream, args);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeConfig& cfg, const uint16_t* q_abs, const uint16_t* cache,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int heads, int q_len, float scale_log2, PlanView plan, int max_items,
                         float* o_part, float* lse_part, hipStream_t stream) {
  DecodeArgs args;
  args.q_abs = q_abs;
  args.cache = cache;
  args.block_table = block_table;
  args.seq_lens = seq_lens;
  args.o_part = o_part;
  args.lse_part = lse_part;
  args.plan = plan;
  args.bt_stride = bt_stride;
  args.heads = heads;
  args.q_len = q_len;
  args.rows_per_seq = heads * q_len;
  args.row_groups = args.rows_per_seq / (16 * cfg.waves);
  args.scale_log2 = scale_log2;
  const int items8 = (max_items + 7) / 8;
  const int grid = items8 * 8 * args.row_groups;
  if (cfg.waves == 4) return launch_t<4, 64>(grid, args, stream);
  if (cfg.waves == 2) return launch_t<2, 32>(grid, args, stream);
  return launch_t<1, 32>(grid, args, stream);
}

}  // namespace mla
