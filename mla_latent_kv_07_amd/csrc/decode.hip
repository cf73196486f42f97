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
//     x one group of query rows (row = query index * H + head).  Each
//     wavefront owns NH groups of 16 rows; all wavefronts share every cache
//     chunk, which is read from HBM once per row group.
//   * Chunks of 32 positions (36 KB, half a page) are copied HBM -> LDS by
//     buffer loads straight to LDS into an NBUF-deep ring; one barrier per
//     chunk.  Every copy instruction moves 1 KB of contiguous cache bytes
//     (whole 128-byte lines): per-lane scattered copies run at about half the
//     HBM rate.  The chunk loop issues no other vector-memory instruction
//     (block table through scalar loads, no spills): vmcnt counts in order,
//     so any such load would make its consumer wait for every chunk in
//     flight.
//     In LDS, position r keeps its 1152-byte row; its 16-byte pieces are
//     permuted inside each aligned group of 8 by the 3-bit mask
//     swz(r) = 2*((r >> 1) & 3) XOR 7*((r >> 3) & 1).  The gfx950 LDS has
//     64 four-byte banks (256 bytes per clock).  A 16-byte read serves 16
//     lanes per clock: the lanes that agree in lane bit 5 and in the parity
//     of lane bits 2..4.  An 8-byte transposing read serves 32 lanes per
//     clock.  Rows start alternately at bank 0 and bank 32
//     (1152 = 4.5 * 256).  Under that map both read patterns below are free
//     of bank conflicts (checked by enumerating every lane's banks): 16 rows
//     x one 16-byte piece per score read, 8 rows x two adjacent 8-byte
//     halves per transposing read.
//   * Scores are computed transposed, S^T = K Q^T, with the bf16 MFMA
//     16x16x32: the cache tile is the A operand, the query the B operand
//     held in registers for the whole launch.  Each lane ends up with the
//     scores of ONE head for 4 positions per 16-position tile, exactly the
//     B-operand layout of O^T = V^T P^T, so P never goes through LDS.  V^T
//     comes from LDS through the transposing read (ds_read_b64_tr_b16).
//   * Per chunk a wavefront runs scores, softmax and P.V in that order
//     (scheduling barriers keep the phases apart, so no phase's registers
//     stay live across another).  The absorbed query (18 k-steps, 144 VGPRs)
//     and the 32 x 512 fp32 output tile (256 accumulation registers) stay in
//     registers for the whole item: one wavefront per SIMD.
//   * Online softmax in log2 units (the query arrives pre-multiplied by
//     softmax_scale * log2 e) with a fixed reference per row: the max of the
//     item's first chunk, the only chunk that needs a cross-lane reduction.
//     Later chunks compute p = 2^(s - ref) and check that each lane's chunk
//     sum stays <= 2^16, which bounds every p; the fp32 accumulators are never
//     rescaled.  If the check fails (never for well-scaled attention, but
//     possible), the workgroup restarts the item: one pass for the exact row
//     max, one pass with that max as the reference.
// Output per work item: normalised rows [rows, 512] rounded to bf16 and their
// log2-sum-exp, merged across items by the combine kernel.
#include <type_traits>

#include "mla_common.h"

namespace mla {

struct DecodeArgs {
  const uint16_t* q_abs;     // [B * rows_per_seq, 576]
  const void* cache;         // bf16 [num_blocks, 64, 576] or FP8 rows [num_blocks, 64, 656]
  const int32_t* seq_lens;
  uint16_t* o_part;          // [max_items, rows_per_seq, 512] bf16
  float* lse_part;           // [max_items, rows_per_seq]
  int* restart_flag;         // one int per workgroup (workgroup-local communication)
  PlanView plan;
  int bt_stride;
  int heads;
  int q_len;
  int rows_per_seq;
  int row_groups;
};

constexpr int kChunk = 32;                     // positions per LDS stage
constexpr int kBufBytes = kChunk * kEntryBytes;  // 36864
constexpr float kSlackPow = 65536.0f;          // 2^16: headroom above the reference max

// Encoding of "s_waitcnt vmcnt(n)" (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Copies of one chunk: 1 KB per wavefront-wide instruction.
//   bf16: the chunk's 36 KB is dealt to the wavefronts round robin (copy i of
//         wavefront w fills LDS bytes 1024 (i NW + w) ..); the chunk is read
//         by every wavefront, after a barrier.
//   FP8:  wavefront w copies rows w RW .. w RW + RW - 1 of the chunk (RW =
//         32 / NW) into a region of its own, the only rows it later expands,
//         so its own wait on the copies is all the expansion needs.
template <int NW, bool FP8>
struct Dma {
  static constexpr int kWaveBytes = (kChunk / NW) * kFp8EntryBytes;  // FP8 rows of a wavefront
  // copies per wavefront; when the count does not split evenly the last ones
  // are out of range (no memory access) and land in the slot's padding
  static constexpr int kPerWave = FP8 ? (kWaveBytes + 1023) / 1024 : (kBufBytes / 1024 + NW - 1) / NW;
  static constexpr int kSlotBytes = kPerWave * NW * 1024;
  static constexpr int kStride = FP8 ? 1024 : NW * 1024;      // LDS distance of a wavefront's copies
  static constexpr int kWaveBase = FP8 ? kPerWave * 1024 : 1024;  // LDS offset of wavefront w: w * this
};

// Piece permutation inside each aligned group of 8 pieces of row r.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 3) << 1) ^ (((r >> 3) & 1) * 7); }

// Per-lane source offsets of the wavefront's copies of one chunk.
// bf16: copy k = i NW + wave fills LDS pieces 64k .. 64k+63 (lane L -> piece
// Q = 64k + L, i.e. row Q / 72, slot Q % 72) from piece (Q % 72) ^ swz(row) of
// that row: the 64 lanes read the same contiguous 1 KB of the chunk, permuted
// within 128-byte lines.  The offsets are the same for every chunk (a chunk
// is 36 KB of contiguous cache: half a page), so they are computed once.
// FP8: copy i reads bytes 1024 i + 16 L of the wavefront's rows as they are
// (expanded into the bf16 layout later, by dequant_rows).
template <int NW, int KP, bool FP8>
__device__ __forceinline__ void dma_offsets(int wave, int lane, uint32_t (&off)[KP]) {
  using D = Dma<NW, FP8>;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if constexpr (FP8) {
      const int o = 1024 * i + 16 * lane;
      off[i] = o < D::kWaveBytes ? (uint32_t)(wave * D::kWaveBytes + o) : 0x80000000u;
    } else {
      const int k = i * NW + wave;
      const int q = 64 * k + lane;
      const int row = q / kChunk16;
      const int col = q - row * kChunk16;
      off[i] = k < kBufBytes / 1024 ? (uint32_t)(row * kEntryBytes + 16 * (col ^ swz(row)))
                                    : 0x80000000u;  // beyond any range
    }
  }
}

// Expand the wavefront's FP8 rows of a chunk (RW = 32 / NW rows of
// kFp8EntryBytes in its region of the ring slot `src`, see Dma) into the
// bf16 chunk layout the compute reads (1152-byte rows, 16-byte pieces
// permuted by swz): each group of 8 latent codes becomes 8 bf16 values times
// the row's power-of-two scale (exact: 4 significant bits), the rope part is
// copied.  Rows past the sequence end arrive as zeros and expand to zeros.
// Lane L expands code group L of every row (a contiguous 512-byte read per
// row across the wavefront).
template <int NW>
__device__ __forceinline__ void dequant_rows(const MLA_LDS char* src, MLA_LDS char* dst, int wave,
                                             int lane) {
  using D = Dma<NW, true>;
  constexpr int RW = kChunk / NW;
  // the per-lane offsets below are the same for every chunk: recompute them
  // here rather than let them stay live across the whole chunk loop
  asm volatile("" : "+v"(lane));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const MLA_LDS char* rows = src + wave * D::kWaveBase;
#pragma unroll
  for (int k = 0; k < RW; ++k) {
    const int r = wave * RW + k;  // row in the chunk
    const MLA_LDS char* row = rows + k * kFp8EntryBytes;
    const u32x2 codes = *reinterpret_cast<const MLA_LDS u32x2*>(row + 8 * lane);
    const uint32_t sb = *reinterpret_cast<const MLA_LDS unsigned char*>(row + kFp8ScaleOff);
    const float scale = __uint_as_float(sb << 23);  // 2^(sb - 127); only its exponent is used
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], scale, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[0], scale, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], scale, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes[1], scale, true);
    const bf16x8 v = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    *reinterpret_cast<MLA_LDS bf16x8*>(dst + r * kEntryBytes + 16 * (lane ^ swz(r))) = v;
  }
#pragma unroll
  for (int t = 0; t < (RW * 8 + 63) / 64; ++t) {  // rope: (row, 16-byte piece)
    const int task = t * 64 + lane;
    if (RW * 8 % 64 == 0 || task < RW * 8) {
      const int k = task >> 3;
      const int c = task & 7;
      const int r = wave * RW + k;
      const u32x4 v =
          *reinterpret_cast<const MLA_LDS u32x4*>(rows + k * kFp8EntryBytes + kFp8RopeOff + 16 * c);
      *reinterpret_cast<MLA_LDS u32x4*>(dst + r * kEntryBytes + 16 * ((64 + c) ^ swz(r))) = v;
    }
  }
}

// Buffer descriptor word 3 for gfx9-family raw buffer loads.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bits of the cache copies: non-temporal.  Every cache byte is
// read once per launch; the hint keeps the stream from displacing what the
// neighbouring kernels reuse from L2 and the last-level cache (the absorbed
// query, the partial rows, kv_b).
constexpr int kCopyPolicy = 2;

// Copy instructions I0 .. I1-1 of the wavefront's share of one chunk (at
// `src`, a wavefront-uniform address) into the LDS ring slot `buf`
// (wavefront-uniform; layout of the copies in D): buffer loads straight to
// LDS, with the chunk as the buffer (scalar descriptor) and a 32-bit per-lane
// offset.  The buffer range is `bytes`: lanes beyond it read no memory and
// write zeros to LDS (checked per dword).  A partial last chunk thus arrives
// zero-padded, and `bytes` = 0 gives an empty copy with the same instruction
// count.
// (WB, ST: Dma::kWaveBase, Dma::kStride)
template <int WB, int ST, int I0, int I1>
__device__ __forceinline__ void load_chunk(MLA_LDS char* buf, const char* src, int bytes,
                                           const uint32_t* off, int wave) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, bytes, kRsrcWord3);
#pragma unroll
  for (int i = I0; i < I1; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, buf + wave * WB + i * ST, 16, off[i], 0, 0,
                                             kCopyPolicy);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008;
constexpr int kSgVmemRead = 0x020;
constexpr int kSgDsRead = 0x100;

// One chunk's copy as a buffer (scalar descriptor) and its ring slot.
struct ChunkCopy {
  __amdgpu_buffer_rsrc_t rsrc;
  MLA_LDS char* dst;
};

// Copy instruction i of the wavefront's share of a chunk (see load_chunk).
// (WB, ST: Dma::kWaveBase, Dma::kStride)
template <int WB, int ST>
__device__ __forceinline__ void copy_piece(const ChunkCopy& c, const uint32_t* off, int i,
                                           int wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, c.dst + wave * WB + i * ST, 16, off[i], 0, 0,
                                           kCopyPolicy);
}

// Score k-step at which copy c of NC goes out: spread evenly over the first
// KS k-steps.
constexpr int copy_step(int c, int nc, int ks) { return c * ks / nc; }

// Schedule of k-steps KS .. KEND-1 of score_chunk: the step's copies, its
// MFMAs, then the LDS reads of a later step.
template <int NH, int NC, int KS, int KEND>
__device__ __forceinline__ void score_schedule() {
  if constexpr (KS < KEND) {
    constexpr int kNc = [] {
      int k = 0;
      for (int c = 0; c < NC; ++c) k += copy_step(c, NC, KEND) == KS;
      return k;
    }();
    if constexpr (kNc > 0) __builtin_amdgcn_sched_group_barrier(kSgVmemRead, kNc, 0);
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 2 * NH, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
    score_schedule<NH, NC, KS + 1, KEND>();
  }
}

// Scores of one chunk for the wavefront's NH row groups: sacc[h][t] holds
// S^T for positions 16t..16t+15.  The LDS reads of k-step ks + KPD are issued
// before the MFMAs of k-step ks.  NC > 0: the NC copy instructions of a later
// chunk (`cc`, into another slot) are spread over the k-steps: the LDS-DMA
// path takes roughly 15 cycles per 1 KB copy, and a wavefront that issues
// copies faster than that stalls, so they go out one at a time between
// MFMAs instead of all at once.
template <int NH, class D, int NC, int KPD = 4>
__device__ __forceinline__ void score_chunk(const MLA_LDS char* buf, int sbase_even,
                                            int sbase_odd, const bf16x8 (&qreg)[NH][18],
                                            f32x4 (&sacc)[NH][2], const ChunkCopy& cc,
                                            const uint32_t* off, int wave) {
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int t = 0; t < 2; ++t) sacc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane (row n, piece group gq) reads piece 4ks + gq of rows 16t + n:
  // byte (16t + n)*1152 + 16*((4ks + gq) ^ swz(n)) = base(ks parity) + 64ks + 18432t
  const MLA_LDS char* be = buf + sbase_even;
  const MLA_LDS char* bo = buf + sbase_odd;
  auto kload = [&](int ks, int t) -> bf16x8 {
    return *reinterpret_cast<const MLA_LDS bf16x8*>((ks & 1 ? bo : be) + 64 * ks +
                                                    16 * kEntryBytes * t);
  };
  bf16x8 kb[KPD + 1][2];
#pragma unroll
  for (int ks = 0; ks < KPD; ++ks)
#pragma unroll
    for (int t = 0; t < 2; ++t) kb[ks][t] = kload(ks, t);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    if (ks + KPD < 18) {
#pragma unroll
      for (int t = 0; t < 2; ++t) kb[(ks + KPD) % (KPD + 1)][t] = kload(ks + KPD, t);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (copy_step(c, NC, 18 - KPD) == ks) copy_piece<D::kWaveBase, D::kStride>(cc, off, c, wave);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const bf16x8 qb = qreg[h][ks];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        sacc[h][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks % (KPD + 1)][t], qb,
                                                             sacc[h][t], 0, 0, 0);
    }
  }
  // schedule: KPD k-steps of reads ahead, then per k-step its MFMAs and the
  // reads of k-step ks + KPD
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * KPD, 0);
  score_schedule<NH, NC, 0, 18 - KPD>();
  __builtin_amdgcn_sched_group_barrier(kSgMfma, 2 * NH * KPD, 0);
}

// Softmax of one chunk's scores (already scaled to log2 units: the query was
// pre-multiplied by softmax_scale * log2(e)) into bf16 probabilities pk[h],
// the B operand of the P.V product.
//   FIRST: the chunk sets each row's reference m_ref = its max (cross-lane
//          reduction over the 4 lanes of a head).  Later chunks reuse it.
//   MASK:  slots beyond the row's causal limit / the sequence end get p = 0
//          (lim[h]: the lane's slot 16t + i is visible iff 16t + i <= lim[h]).
// Returns true if some probability may exceed 2^kSlack (sum check, see the
// file header): the item must restart with an exact reference.
template <int NH, bool FIRST, bool MASK>
__device__ __forceinline__ bool softmax_chunk(f32x4 (&sacc)[NH][2], bf16x8 (&pk)[NH],
                                              float (&m_ref)[NH], float (&l_run)[NH],
                                              const int (&lim)[NH]) {
  bool restart = false;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (MASK) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sacc[h][t][i] = (16 * t + i > lim[h]) ? -INFINITY : sacc[h][t][i];
    }
    if (FIRST) {
      float mloc = fmaxf(fmaxf(fmaxf(sacc[h][0][0], sacc[h][0][1]), fmaxf(sacc[h][0][2], sacc[h][0][3])),
                         fmaxf(fmaxf(sacc[h][1][0], sacc[h][1][1]), fmaxf(sacc[h][1][2], sacc[h][1][3])));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      m_ref[h] = mloc;
    }
    const float m_use = m_ref[h] == -INFINITY ? 0.f : m_ref[h];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[h][t][i] - m_use);
        psum += p;
        pk[h][t * 4 + i] = (__bf16)p;
      }
    }
    l_run[h] += psum;
    // every p <= psum, so psum <= 2^kSlack bounds them all (NaN/inf fail too)
    if (!FIRST) restart |= !(psum <= kSlackPow);
  }
  return restart;
}


// P.V for the wavefront's slice of the latent features: for the FT = 32/NW
// feature tiles of the slice and all G = NW*NH row groups of the workgroup,
// O^T[g][f] += V^T[f] P^T[g].  pb[g] is the B operand of row group g.  V^T
// comes from the chunk through the transposing read; feature tile f of the
// slice sits at vbase[f & 3] + 128*(f >> 2) (vbase includes the slice).
template <int NW, int NH>
__device__ __forceinline__ void pv_slice(const MLA_LDS char* buf, const int (&vbase)[4],
                                         const bf16x8 (&pb)[NW * NH],
                                         f32x4 (&oacc)[NW * NH][32 / NW]) {
  constexpr int G = NW * NH;
  constexpr int FT = 32 / NW;
  bf16x8 vb[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    // one variable offset per read plus constants: the address stays a
    // short chain of offsets from the LDS array, short enough for the
    // compiler to keep track of which array it reads (and so of which copies
    // in flight it must wait for)
    const int o = vbase[f & 3] + 128 * (f >> 2);
    const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(buf + o));
    const bf16x4 a1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(buf + (o + 16 * kEntryBytes)));
    vb[f] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int g = 0; g < G; ++g)
      oacc[g][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[f], pb[g], oacc[g][f], 0, 0, 0);
  // schedule: VPD feature tiles of reads ahead, then one tile of reads per
  // tile of MFMAs (the reads of tile f + VPD overlap the MFMAs of tile f)
  constexpr int VPD = FT < 4 ? FT : 4;
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2 * VPD, 0);
#pragma unroll
  for (int f = 0; f < FT - VPD; ++f) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, G, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSgMfma, G * VPD, 0);
}

// The same product with the probabilities read from LDS one row group at a
// time (`pb_lds`, 1 KB B-operand tile per group): eight wavefronts cannot
// keep all groups' tiles in registers next to the query and accumulators.
template <int NW, int NH>
__device__ __forceinline__ void pv_slice_lds(const MLA_LDS char* buf, const int (&vbase)[4],
                                             const MLA_LDS char* pb_lds, int lane,
                                             f32x4 (&oacc)[NW * NH][32 / NW]) {
  constexpr int G = NW * NH;
  constexpr int FT = 32 / NW;
  bf16x8 vb[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    const int o = vbase[f & 3] + 128 * (f >> 2);
    const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(buf + o));
    const bf16x4 a1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(buf + (o + 16 * kEntryBytes)));
    vb[f] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bf16x8 pg = *reinterpret_cast<const MLA_LDS bf16x8*>(pb_lds + g * 1024 + lane * 16);
#pragma unroll
    for (int f = 0; f < FT; ++f)
      oacc[g][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[f], pg, oacc[g][f], 0, 0, 0);
  }
}

// Row max only (the first pass of a restart).
template <int NH>
__device__ __forceinline__ void max_chunk(const f32x4 (&sacc)[NH][2], float (&m)[NH],
                                          const int (&lim)[NH]) {
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mloc = fmaxf(mloc, (16 * t + i > lim[h]) ? -INFINITY : sacc[h][t][i]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    m[h] = fmaxf(m[h], mloc);
  }
}

template <int S>
using Slot = std::integral_constant<int, S>;

// Encoding of "s_waitcnt lgkmcnt(0)" (vmcnt and expcnt left unconstrained).
constexpr int kLgkm0 = 0xc07f;

// Workgroup barrier of the chunk ring: this wavefront's LDS accesses have
// completed, then s_barrier.  Written as asm with a memory clobber, so the
// compiler moves no memory access across it; unlike __syncthreads it adds no
// wait on the copies in flight (their completion is waited for explicitly).
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  asm volatile("s_barrier" ::: "memory");
}

// FP8: the cache holds FP8 rows; each chunk lands in the ring in that form
// and every wavefront expands its own rows of it into a bf16 staging chunk
// while the chunk before it is multiplied (double-buffered staging).
template <int NW, int NH, bool FP8>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a,
                                                         const int32_t* __restrict__ block_table) {
  constexpr int G = NW * NH;   // 16-row groups of the workgroup
  constexpr int FT = 32 / NW;  // feature tiles of a wavefront's P.V slice
  constexpr int kRowBytes = FP8 ? kFp8EntryBytes : kEntryBytes;  // cache bytes per position
  using D = Dma<NW, FP8>;
  // The ring: NS chunk slots (bf16: 4, or 3 of 40 KB with eight wavefronts;
  // FP8: 3 next to the two staging chunks), each its own array.  Chunk j lives in slot j % NS, and the chunk
  // loop is unrolled by NS so that every access names its slot at compile
  // time: the compiler then knows that the copies in flight (into the other
  // slots) never alias the slot being read and adds no wait of its own on
  // them.
  constexpr int NS = (FP8 || NW == 8) ? 3 : 4;
  // score read-ahead in k-steps (eight wavefronts: two, for registers)
  constexpr int kKpd = NW == 8 ? 2 : 4;
  __shared__ __attribute__((aligned(1024))) char ring0[D::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[D::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[D::kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring3[NS == 4 ? D::kSlotBytes : 16];
  // FP8: chunks j (read by the compute) and j + 1 (being expanded), bf16 layout
  __shared__ __attribute__((aligned(1024))) char stage[FP8 ? 2 * kBufBytes : 16];
  // probabilities of the chunk, one 1 KB B-operand tile per row group
  __shared__ __attribute__((aligned(1024))) char pbuf[G * 1024];
  // row sums at the end
  __shared__ float lbuf[G * 16];
  auto ring = [&](auto slot_c) -> MLA_LDS char* {
    constexpr int S = decltype(slot_c)::value;
    if constexpr (S == 0) return (MLA_LDS char*)ring0;
    else if constexpr (S == 1) return (MLA_LDS char*)ring1;
    else if constexpr (S == 2) return (MLA_LDS char*)ring2;
    else return (MLA_LDS char*)ring3;
  };
  // FP8: the staging chunk of chunk j.  The offset is made opaque so that
  // every access stays a plain offset from `stage` (not a select or phi of
  // two pointers): the compiler then still tells it apart from the ring
  // slots the copies in flight write, and adds no wait on them.
  auto stage_of = [&](int j) -> MLA_LDS char* {
    int off = (j & 1) * kBufBytes;
    asm volatile("" : "+s"(off));
    return (MLA_LDS char*)stage + off;
  };
  MLA_LDS char* pb_lds = (MLA_LDS char*)pbuf;

  // blockIdx -> (item, row group).  Workgroups are dispatched to the eight
  // XCDs round-robin (block id mod 8); XCD x takes a contiguous range of the
  // item list, which is in sequence order, so the items of one sequence (and
  // the row groups of one item) share that XCD's L2: the sequence's absorbed
  // query rows come from HBM once.
  const int gid = blockIdx.x;
  const int xcd = gid & 7;
  const int gslot = gid >> 3;
  const int n_items = a.plan.header[0];
  const int per_xcd = (n_items + 7) >> 3;
  const int local = gslot / a.row_groups;
  const int rg = gslot - local * a.row_groups;
  const int item = xcd * per_xcd + local;
  if (local >= per_xcd || item >= n_items) return;

  const int b = a.plan.item_b[item];
  const int p0 = a.plan.item_p0[item];
  const int p1 = a.plan.item_p1[item];
  const int len = a.seq_lens[b];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keep it scalar
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int gq = lane >> 4;
  const int rows0 = rg * G * 16;          // first row of the workgroup in the sequence
  const int row0 = rows0 + wave * 16 * NH;  // first scored row of this wavefront
  int tmax[NH];                           // last visible position per scored row group
  int tmax_min = 0x7fffffff;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    tmax[h] = len - a.q_len + (row0 + 16 * h) / a.heads;
    tmax_min = min(tmax_min, tmax[h]);
  }

  // per-lane LDS bases of the two read patterns (see the layout above)
  const int xs = gq ^ swz(n);
  const int sbase_even = n * kEntryBytes + 16 * xs;
  const int sbase_odd = n * kEntryBytes + 16 * (xs ^ 4) - 64;
  int vbase[4];
  {
    // transposing read: 16-lane group gq, lane 4r + qq supplies row 4gq + r,
    // features 16f + 4qq .. +3 = piece 2f + (qq >> 1), half qq & 1
    const int r4 = (lane & 15) >> 2;
    const int qq = lane & 3;
    const int row = 4 * gq + r4;
    const int y = (qq >> 1) ^ swz(row);
    // this wavefront's feature slice: tiles wave*FT .. +FT (FT is a multiple
    // of 4), folded into the bases (kept as one value each: see pv_slice)
    const int slice_off = 32 * wave * FT;
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4) {
      vbase[f4] = row * kEntryBytes + 16 * ((2 * f4) ^ y) + 8 * (qq & 1) + slice_off;
      asm volatile("" : "+v"(vbase[f4]));
    }
  }

  // the absorbed query rows, in registers for the whole item: lane holds
  // features 32ks + 8gq .. +8 of row n (the B operand of k-step ks)
  bf16x8 qreg[NH][18];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(
        a.q_abs + ((int64_t)b * a.rows_per_seq + row0 + 16 * h + n) * kEntry + 8 * gq);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[h][ks] = qp[4 * ks];
  }
  // O^T of the workgroup's rows, this wavefront's feature slice
  f32x4 oacc[G][FT];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int f = 0; f < FT; ++f) oacc[g][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[NH], l_run[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m_ref[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  // restart flag of this workgroup: written by any wavefront, read by all
  // after a barrier, which orders it within the workgroup
  int* flag = a.restart_flag + blockIdx.x;
  if (threadIdx.x == 0) __atomic_store_n(flag, 0, __ATOMIC_RELAXED);

  const int tok_begin = p0 * kPage;
  const int tok_end = min(p1 * kPage, len);
  const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;
  // chunks from jm on reach past the causal limit of some scored row (or the
  // sequence end) and take the masked softmax
  const int jm = (tmax_min - tok_begin + 1) / kChunk;
  const int32_t* bt = block_table + (int64_t)b * a.bt_stride;  // scalar loads (restrict)
  const char* cache = reinterpret_cast<const char*>(a.cache);
  constexpr int kPer = D::kPerWave;
  uint32_t doff[kPer];
  dma_offsets<NW, kPer, FP8>(wave, lane, doff);
  // Every interval issues exactly one chunk's copies (empty ones past the
  // item's end), so "chunk j has landed" is always the same count of copies
  // pending: one wait count for every chunk, which the compiler can follow
  // and so adds no conservative full drain of its own.
  // The last chunk of the sequence may end inside the chunk: its copy reads
  // only the valid rows, the others arrive as zeros (never the NaN sentinels
  // or stale data of the slots beyond the sequence end).
  auto chunk_src = [&](int j, int& bytes) -> const char* {
    const bool real = j < nchunks;
    const int t = tok_begin + (real ? j : 0) * kChunk;
    const int64_t blk = bt[t / kPage];
    bytes = real ? min(tok_end - t, kChunk) * kRowBytes : 0;
    return cache + (blk * kPage + (t % kPage)) * (int64_t)kRowBytes;
  };
  auto chunk_copy = [&](auto slot_c, int j) -> ChunkCopy {
    int bytes;
    const char* src = chunk_src(j, bytes);
    return ChunkCopy{
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, bytes, kRsrcWord3),
        ring(slot_c)};
  };
  // all copy instructions of chunk j into its slot
  auto issue = [&](auto slot_c, int j) {
    int bytes;
    const char* src = chunk_src(j, bytes);
    load_chunk<D::kWaveBase, D::kStride, 0, kPer>(ring(slot_c), src, bytes, doff, wave);
  };
  // visibility limit of chunk j for this lane, relative to its slot 16t + i
  auto chunk_limits = [&](int j, int (&lim)[NH]) {
    const int t0 = tok_begin + j * kChunk;
#pragma unroll
    for (int h = 0; h < NH; ++h) lim[h] = tmax[h] - t0 - 4 * gq;
  };
  // One chunk (bf16 layout at `buf`): scores and softmax of this wavefront's
  // rows, the probabilities to LDS, a barrier, then the P.V of all the
  // workgroup's rows for this wavefront's feature slice.  Returns the restart
  // verdict of its rows.  (NC > 0: the copies of `cc` go out during the score
  // phase; DQ: the wavefront's FP8 rows at `dq_src` are expanded into `dq_dst`
  // during the P.V phase.)
  auto compute = [&](const MLA_LDS char* buf, auto first_c, auto nc_c, auto dq_c, int j,
                     const ChunkCopy& cc, const MLA_LDS char* dq_src,
                     MLA_LDS char* dq_dst) __attribute__((always_inline)) -> bool {
    constexpr bool kFirst = decltype(first_c)::value;
    int lim[NH];
    chunk_limits(j, lim);
    f32x4 sacc[NH][2];
    // the phases stay in order: moving the next phase's LDS reads up would
    // keep their registers live across this one
    // wavefront priority: raised for the two matrix phases (the P.V one
    // from the probability writes and the barrier before it) and lowered for
    // the softmax, so that of the two wavefronts sharing a SIMD the one in a
    // matrix phase issues first and the other's softmax fills its gaps
    // (same-process A/Bs at the V3 shape: 142.7 -> 137.9 us per launch, then
    // 141.5 -> 138.1 us for raising it before the barrier)
    __builtin_amdgcn_s_setprio(1);
    score_chunk<NH, D, decltype(nc_c)::value, kKpd>(buf, sbase_even, sbase_odd, qreg, sacc, cc, doff,
                                              wave);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    bf16x8 pk[NH];
    bool need;
    if (j >= jm)
      need = softmax_chunk<NH, kFirst, true>(sacc, pk, m_ref, l_run, lim);
    else
      need = softmax_chunk<NH, kFirst, false>(sacc, pk, m_ref, l_run, lim);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h = 0; h < NH; ++h)
      *reinterpret_cast<MLA_LDS bf16x8*>(pb_lds + (wave * NH + h) * 1024 + lane * 16) = pk[h];
    ring_barrier();
    if constexpr (NW == 8) {
      pv_slice_lds<NW, NH>(buf, vbase, pb_lds, lane, oacc);
    } else {
      bf16x8 pb[G];
#pragma unroll
      for (int g = 0; g < G; ++g)
        pb[g] = *reinterpret_cast<const MLA_LDS bf16x8*>(pb_lds + g * 1024 + lane * 16);
      __builtin_amdgcn_sched_barrier(0);
      pv_slice<NW, NH>(buf, vbase, pb, oacc);
    }
    if constexpr (decltype(dq_c)::value) {
      // the rows to expand have landed once at most the copies of the two
      // chunks after them are pending
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPer));
      dequant_rows<NW>(dq_src, dq_dst, wave, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    return need;
  };

  // ---- main pass: reference = the first chunk's max per row ----------------
  // bf16: while chunk j is computed, chunks j+1 and j+2 are in flight and
  // chunk j+3 goes into chunk j-1's slot once every wavefront is past chunk
  // j-1; its copies run inside the score phase of chunk j.
  // FP8: chunk j was expanded into its staging chunk during the P.V of chunk
  // j-1; chunk j+3 goes into chunk j's ring slot (this wavefront expanded its
  // rows of it already), and chunk j+1 is expanded during the P.V of chunk j.
  // The chunks run in groups of NS; a group may reach past the item's end,
  // and such steps still pass the barrier and issue their (empty) copies but
  // skip the compute.  No vector memory instruction sits in a conditional,
  // so on every path the compiler sees the same copies pending.
  // (a wavefront that needs a restart keeps going with a useless result;
  // the verdict is taken once, after the pass)
  using T = std::true_type;
  using F = std::false_type;
  using NoCopy = std::integral_constant<int, 0>;
  using AllCopies = std::integral_constant<int, kPer>;
  bool need_restart = false;
  auto interval = [&](auto slot_c, auto first_c, int j) __attribute__((always_inline)) {
    constexpr int S = decltype(slot_c)::value;
    if constexpr (FP8) {
      // every wavefront's rows of chunk j are in its staging chunk, and every
      // wavefront is past chunk j-1 (whose staging chunk takes chunk j+1)
      ring_barrier();
      const ChunkCopy cc = chunk_copy(slot_c, j + 3);
      if (j < nchunks) {
        need_restart |= compute(stage_of(j), first_c, AllCopies{}, T{}, j, cc,
                                ring(Slot<(S + 1) % NS>{}), stage_of(j + 1));
      } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) copy_piece<D::kWaveBase, D::kStride>(cc, doff, i, wave);
      }
    } else {
      // chunk j has landed once at most the copies of chunks j+1 .. j+NS-2
      // are pending
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * kPer));
      ring_barrier();
      // chunk j+NS-1 goes into chunk j-1's slot: every wavefront is past it
      const ChunkCopy cc = chunk_copy(Slot<(S + NS - 1) % NS>{}, j + NS - 1);
      if (j < nchunks) {
        need_restart |= compute(ring(slot_c), first_c, AllCopies{}, F{}, j, cc, nullptr, nullptr);
      } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) copy_piece<D::kWaveBase, D::kStride>(cc, doff, i, wave);
      }
    }
  };
  // (an item always has at least one chunk)
  issue(Slot<0>{}, 0);
  issue(Slot<1>{}, 1);
  if constexpr (FP8 || NS == 4) issue(Slot<2>{}, 2);
  if constexpr (FP8) {
    dequant_rows<NW>(ring(Slot<0>{}), stage_of(0), wave, lane);
    interval(Slot<0>{}, T{}, 0);
    for (int j = 1; j < nchunks; j += 3) {
      interval(Slot<1>{}, F{}, j);
      interval(Slot<2>{}, F{}, j + 1);
      interval(Slot<0>{}, F{}, j + 2);
    }
  } else if constexpr (NS == 3) {
    interval(Slot<0>{}, T{}, 0);
    for (int j = 1; j < nchunks; j += 3) {
      interval(Slot<1>{}, F{}, j);
      interval(Slot<2>{}, F{}, j + 1);
      interval(Slot<0>{}, F{}, j + 2);
    }
  } else {
    interval(Slot<0>{}, T{}, 0);
    for (int j = 1; j < nchunks; j += 4) {
      interval(Slot<1>{}, F{}, j);
      interval(Slot<2>{}, F{}, j + 1);
      interval(Slot<3>{}, F{}, j + 2);
      interval(Slot<0>{}, F{}, j + 3);
    }
  }
  // every wavefront's verdict, then one decision for the workgroup
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(need_restart) != 0 && lane == 0)
    __atomic_store_n(flag, 1, __ATOMIC_RELAXED);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  const bool restart = __atomic_load_n(flag, __ATOMIC_RELAXED) != 0;

  // ---- restart (rare): exact row max, then a pass with it as the reference --
  // one chunk at a time through slot 0 (FP8: expanded into staging chunk 0)
  if (restart) {
    auto fetch = [&](int j) -> const MLA_LDS char* {
      issue(Slot<0>{}, j);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      if constexpr (FP8) {
        dequant_rows<NW>(ring(Slot<0>{}), stage_of(0), wave, lane);
        __syncthreads();
        return stage_of(0);
      } else {
        __syncthreads();
        return ring(Slot<0>{});
      }
    };
    float m_exact[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) m_exact[h] = -INFINITY;
    for (int j = 0; j < nchunks; ++j) {
      const MLA_LDS char* buf = fetch(j);
      int lim[NH];
      chunk_limits(j, lim);
      f32x4 sacc[NH][2];
      score_chunk<NH, D, 0, kKpd>(buf, sbase_even, sbase_odd, qreg, sacc, ChunkCopy{}, doff, wave);
      max_chunk<NH>(sacc, m_exact, lim);
      __syncthreads();
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      m_ref[h] = m_exact[h];
      l_run[h] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int f = 0; f < FT; ++f) oacc[g][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < nchunks; ++j) {
      const MLA_LDS char* buf = fetch(j);
      compute(buf, F{}, NoCopy{}, F{}, j, ChunkCopy{}, nullptr, nullptr);
      __syncthreads();
    }
  }

  // ---- finalise: normalised rows and log2-sum-exp ---------------------------
  // each wavefront's row sums to LDS; every wavefront normalises its slice
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float l = l_run[h];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float lse = l > 0.f ? m_ref[h] + __builtin_amdgcn_logf(l) : -INFINITY;
    if (gq == 0) {
      lbuf[(wave * NH + h) * 16 + n] = l;
      a.lse_part[(int64_t)item * a.rows_per_seq + row0 + 16 * h + n] = lse;
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = lbuf[g * 16 + n];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = (int64_t)item * a.rows_per_seq + rows0 + 16 * g + n;
    uint16_t* op = a.o_part + orow * kLatent + 16 * wave * FT + 4 * gq;
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      u16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(oacc[g][f][i] * inv);
      *reinterpret_cast<u16x4*>(op + 16 * f) = v;
    }
  }
}

DecodeConfig decode_config(int rows_per_seq) {
  const int groups = rows_per_seq / 16;
  DecodeConfig c;
  c.chunk = kChunk;
  c.nbuf = 4;
  if (groups % 8 == 0) {
    // eight wavefronts of one row group each: two per SIMD, so one's LDS
    // waits and softmax overlap the other's matrix work
    c.waves = 8;
    c.heads_per_wave = 1;
    c.nbuf = 3;
  } else if (groups % 4 == 0) {
    c.waves = 2;
    c.heads_per_wave = 2;
  } else if (groups % 2 == 0) {
    c.waves = 1;
    c.heads_per_wave = 2;
  } else {
    c.waves = 1;
    c.heads_per_wave = 1;
  }
  c.lds_bytes = c.nbuf * kBufBytes + c.waves * c.heads_per_wave * (1024 + 64);
  c.wgs_per_cu = 1;  // the ring fills the LDS
  return c;
}

template <int NW, int NH>
static hipError_t launch_t(int grid, bool fp8, const DecodeArgs& args,
                          const int32_t* block_table, hipStream_t stream) {
  if constexpr (NW == 8) {
    // no FP8 build of the eight-wavefront kernel (launch_decode routes FP8
    // caches to the four-wavefront one)
    if (fp8) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_kernel<NW, NH, false>), dim3(grid), dim3(NW * 64), 0, stream,
                       args, block_table);
  } else if (fp8) {
    hipLaunchKernelGGL((decode_kernel<NW, NH, true>), dim3(grid), dim3(NW * 64), 0, stream, args,
                       block_table);
  } else {
    hipLaunchKernelGGL((decode_kernel<NW, NH, false>), dim3(grid), dim3(NW * 64), 0, stream,
                       args, block_table);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeConfig& cfg, bool fp8, const uint16_t* q_abs, const void* cache,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int heads, int q_len, PlanView plan, int max_items,
                         uint16_t* o_part, float* lse_part,
                         int* restart_flags, hipStream_t stream) {
  DecodeArgs args;
  args.restart_flag = restart_flags;
  args.q_abs = q_abs;
  args.cache = cache;
  args.seq_lens = seq_lens;
  args.o_part = o_part;
  args.lse_part = lse_part;
  args.plan = plan;
  args.bt_stride = bt_stride;
  args.heads = heads;
  args.q_len = q_len;
  args.rows_per_seq = heads * q_len;
  args.row_groups = args.rows_per_seq / (16 * cfg.waves * cfg.heads_per_wave);
  const int items8 = (max_items + 7) / 8;
  const int grid = items8 * 8 * args.row_groups;
  // (the FP8 cache runs the four-wavefront kernel: same rows per workgroup,
  // so the same workspace layout)
  if (cfg.waves == 8)
    return fp8 ? launch_t<4, 2>(grid, fp8, args, block_table, stream)
               : launch_t<8, 1>(grid, fp8, args, block_table, stream);
  if (cfg.waves == 4) return launch_t<4, 2>(grid, fp8, args, block_table, stream);
  if (cfg.waves == 2) return launch_t<2, 2>(grid, fp8, args, block_table, stream);
  if (cfg.heads_per_wave == 2) return launch_t<1, 2>(grid, fp8, args, block_table, stream);
  return launch_t<1, 1>(grid, fp8, args, block_table, stream);
}

}  // namespace mla
