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
  // Rows in place (the sparse decode): slot list of cache row indices, one
  // per kept position (rank), `slot_stride` apart per sequence; the cache is
  // then one buffer of `cache_bytes` bytes.  nullptr: paged through the block
  // table.
  const int32_t* slots;
  int slot_stride;
  uint32_t cache_bytes;
};

constexpr int kChunk = 32;                     // positions per LDS stage
constexpr int kBufBytes = kChunk * kEntryBytes;  // 36864
constexpr float kSlackPow = 65536.0f;          // 2^16: headroom above the reference max

// Encoding of "s_waitcnt vmcnt(N)" (expcnt and lgkmcnt left unconstrained).
// The count has 6 bits: N above 63 is a compile error.
template <int N>
constexpr int vmcnt_imm() {
  static_assert(N >= 0 && N <= 63, "vmcnt has 6 bits");
  return (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
}

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

// A partial row's four values (an MFMA output tile's lane) times `inv`,
// rounded to bf16 (nearest even) by the hardware conversion, two values per
// instruction.
__device__ __forceinline__ u16x4 scaled_bf16x4(f32x4 x, float inv) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t b = {(__bf16)(x[0] * inv), (__bf16)(x[1] * inv), (__bf16)(x[2] * inv),
                      (__bf16)(x[3] * inv)};
  return __builtin_bit_cast(u16x4, b);
}

// Partial rows staged in LDS, to be stored as whole rows.  A tile's 8-byte
// writes are served 16 lanes at a time (one column unit of 16 rows) over 32
// four-byte banks.  Rows are kStageStride apart, 4 dwords past a multiple of
// 32 banks, so rows n and n + 8 of a group of 16 would meet; rows 8..15 of
// every group therefore hold their 8-byte units in swapped pairs (unit u at
// u ^ 1), and the 16 lanes cover the 32 banks once.  stage_swap(r): whether
// staged row r is swapped; stage_read: a lane's 16 bytes (units 2l, 2l + 1)
// of staged row r, in order.
constexpr int kStageStride = kLatent * 2 + 16;
__device__ __forceinline__ int stage_swap(int r) { return (r >> 3) & 1; }
__device__ __forceinline__ u16x8 stage_read(const MLA_LDS char* rows, int r, int lane) {
  const u16x8 v = *reinterpret_cast<const MLA_LDS u16x8*>(rows + r * kStageStride + 16 * lane);
  return stage_swap(r) ? __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3) : v;
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
  uint32_t srow;  // rows in place: lane r holds row r's byte offset in the cache
};

// Rows in place: the slot list of a work item is staged in LDS (at most
// kSlotCap positions: 16 KB beside the 144 KB ring), and a row past the end
// gets an offset beyond any cache buffer, so its copies write zeros.
constexpr int kSlotCap = 4096;
constexpr uint32_t kSlotOob = 0xF0000000u;
constexpr uint32_t kSlotMaxCacheBytes = 0xE0000000u;

// Rows in place, four wavefronts: wavefront w copies rows 8w .. 8w+7 of the
// chunk (9 KB of the slot: copies k = 9w + i, i = 0..8, each filling LDS
// pieces 64k .. 64k+63 as in the paged layout).  Copy i's lanes cover rows
// 8w + row_lo(i) and, from lane row_split(i) on, the next one: both are
// constants, so a copy's two row offsets are lane reads at fixed lanes of a
// register whose lane r holds row 8w + r's cache offset.
constexpr int kRowWaveBytes = 9 * 1024;
constexpr int row_lo(int i) { return (64 * i) / kChunk16; }
constexpr int row_split(int i) { return kChunk16 * (row_lo(i) + 1) - 64 * i; }
static_assert(8 * kEntryBytes == kRowWaveBytes, "a wavefront's nine copies are its eight rows");

// Per lane and copy i of the wavefront's nine: the piece within the row
// (offset / 16, 7 bits) and whether the lane is in the copy's second row (bit
// 7), three 8-bit fields a register: off[i / 3] bits 8 (i % 3) .. +7
// (off[3..8] are left unused).  No lane index stays live through the chunk
// loop.
__device__ __forceinline__ void dma_row_offsets(int wave, int lane, uint32_t (&off)[9]) {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int q = 64 * i + lane;  // piece within the wavefront's eight rows
    const int r = q / kChunk16;
    const int col = q - r * kChunk16;
    const uint32_t f = (uint32_t)((col ^ swz(8 * wave + r)) | (r > row_lo(i) ? 128 : 0));
    off[i / 3] = i % 3 == 0 ? f : off[i / 3] | (f << (8 * (i % 3)));
  }
}

template <int I>
__device__ __forceinline__ void row_piece(const ChunkCopy& c, const uint32_t* roff, int wave) {
  constexpr int lo = row_lo(I);
  constexpr int hi = lo + 1 < 8 ? lo + 1 : lo;
  const uint32_t s0 = __builtin_amdgcn_readlane(c.srow, lo);
  const uint32_t s1 = __builtin_amdgcn_readlane(c.srow, hi);
  const uint32_t f = __builtin_amdgcn_ubfe(roff[I / 3], 8 * (I % 3), 8);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, c.dst + wave * kRowWaveBytes + I * 1024, 16,
                                           (f & 128 ? s1 : s0) + 16 * (f & 127), 0, 0,
                                           kCopyPolicy);
}

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
  // (one wavefront: 36 copies per chunk, so only one chunk can be waited on
  // within vmcnt's 6 bits: three slots, two chunks in flight)
  constexpr int NS = (FP8 || NW == 8 || NW == 1) ? 3 : 4;
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
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<FP8 ? 2 * kPer : 0>());
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
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<(NS - 2) * kPer>());
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
    // chunk 0 has landed once at most the copies of chunks 1 and 2 are
    // pending.  The wait is explicit: left to the compiler, the 8-wavefront
    // build read the rows' scale bytes before the wait it inserted for the
    // codes (the scheduler moved the byte loads above it), so every item's
    // first chunk was expanded with stale scales.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * kPer>());
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
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(need_restart) != 0 && lane == 0)
    __atomic_store_n(flag, 1, __ATOMIC_RELAXED);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  __syncthreads();
  const bool restart = __atomic_load_n(flag, __ATOMIC_RELAXED) != 0;

  // ---- restart (rare): exact row max, then a pass with it as the reference --
  // one chunk at a time through slot 0 (FP8: expanded into staging chunk 0)
  if (restart) {
    auto fetch = [&](int j) -> const MLA_LDS char* {
      issue(Slot<0>{}, j);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
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
  if constexpr (FP8) {
    // the rows leave through LDS as whole 1 KB rows (a 16-byte piece per
    // lane) rather than as the tiles' 32-byte pieces of 16 rows: four row
    // groups (64 rows, see kStageStride) at a time in the staging buffer,
    // free here like the ring
    constexpr int kPassG = 4;
    static_assert(G % kPassG == 0 && kPassG * 16 * kStageStride <= 2 * kBufBytes,
                  "a pass's rows fit the staging buffer");
    MLA_LDS char* st = (MLA_LDS char*)stage;
    uint16_t* orows = a.o_part + ((int64_t)item * a.rows_per_seq + rows0) * kLatent;
#pragma unroll
    for (int p = 0; p < G / kPassG; ++p) {
#pragma unroll
      for (int g = p * kPassG; g < (p + 1) * kPassG; ++g) {
        const float l = lbuf[g * 16 + n];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const int sr = 16 * (g - p * kPassG) + n;  // staged row
        MLA_LDS char* dst = st + sr * kStageStride + 32 * wave * FT + 8 * (gq ^ stage_swap(sr));
#pragma unroll
        for (int f = 0; f < FT; ++f)
          *reinterpret_cast<MLA_LDS u16x4*>(dst + 32 * f) = scaled_bf16x4(oacc[g][f], inv);
      }
      __syncthreads();
#pragma unroll
      for (int r = wave; r < kPassG * 16; r += NW) {
        const u16x8 v = stage_read(st, r, lane);
        *reinterpret_cast<u16x8*>(orows + (int64_t)(p * kPassG * 16 + r) * kLatent + 8 * lane) = v;
      }
      if (p + 1 < G / kPassG) __syncthreads();  // the next pass overwrites the buffer
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float l = lbuf[g * 16 + n];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int64_t orow = (int64_t)item * a.rows_per_seq + rows0 + 16 * g + n;
      uint16_t* op = a.o_part + orow * kLatent + 16 * wave * FT + 4 * gq;
#pragma unroll
      for (int f = 0; f < FT; ++f)
        *reinterpret_cast<u16x4*>(op + 16 * f) = scaled_bf16x4(oacc[g][f], inv);
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined decode for 128 query rows per workgroup (H = 128 at q_len 1; one
// of the two row groups at q_len 2): four wavefronts, one per SIMD, each
// owning two groups of 16 rows and ALL 512 latent features of their outputs
// (O^T in 256 accumulation registers, the absorbed query in 144).  A row's
// probabilities therefore never leave the wavefront that computed them: no
// probability tiles go through LDS and the only barrier of a chunk is the one
// that hands out its ring slot.  The cost is that every wavefront reads the
// whole V^T of a chunk (32 KB) next to its whole K (36 KB): 68 KB of LDS
// reads per wavefront per 32 positions, one 1 KB read per two MFMAs.
//
// Software pipeline: while chunk j's P.V runs, the scores of chunk j+1 are
// taken (one fused stream of 18 score k-steps and 32 P.V feature tiles, with
// the LDS reads of each unit issued kFusedAhead units before its MFMAs), then
// the softmax of chunk j+1.  Chunk j lives in ring slot j % 4; at the top of
// interval j, chunk j+1 has landed and chunk j+3's copies go into the slot of
// chunk j-1, so two chunks are in flight while two are read.

// MFMAs with pinned register classes.  With 256 output accumulators per
// lane the kernel needs every AGPR for O; the compiler's own MFMA selection
// puts every accumulator (the scores' too) in AGPRs and then shuffles tiles
// between the two files.  Written as asm, the score tiles accumulate in
// VGPRs and the output tiles in AGPRs, with no copies.  The compiler does not
// know these are matrix instructions, so the one hazard it would miss is
// handled where it occurs: a vector instruction that reads an MFMA result
// (the softmax on the scores, the final read of O) must come at least eight
// wait states after it (mfma_drain below).  Their operands come from LDS or
// global loads (waited for by the compiler's counters) or, for P, from
// vector instructions many cycles earlier.
__device__ __forceinline__ void mfma_sc0(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_sc(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_o(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// 12 wait states after the last score MFMA, ordered before every read of the
// scores (they pass through this statement).
template <int NH>
__device__ __forceinline__ void mfma_drain(f32x4 (&sacc)[NH][2]) {
  static_assert(NH == 1 || NH == 2, "two or four score tiles");
  if constexpr (NH == 2)
    asm volatile("s_nop 7\n\ts_nop 3"
                 : "+v"(sacc[0][0]), "+v"(sacc[0][1]), "+v"(sacc[1][0]), "+v"(sacc[1][1]));
  else
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(sacc[0][0]), "+v"(sacc[0][1]));
}
// The same for the output tiles before they are read (after the chunk loop):
// the wait states first, then every tile passes through an (empty) statement
// ordered after them.
template <int NH, int FT>
__device__ __forceinline__ void mfma_drain_o(f32x4 (&oacc)[NH][FT]) {
  static_assert(FT % 8 == 0, "tiles pass through in eights");
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int f = 0; f < FT; f += 8)
      asm volatile(""
                   : "+a"(oacc[h][f]), "+a"(oacc[h][f + 1]), "+a"(oacc[h][f + 2]),
                     "+a"(oacc[h][f + 3]), "+a"(oacc[h][f + 4]), "+a"(oacc[h][f + 5]),
                     "+a"(oacc[h][f + 6]), "+a"(oacc[h][f + 7]));
}

// The probabilities pk as the B operand of the P.V MFMAs that follow in the
// same block (the restart pass): two wait states after the vector
// instructions that produced them, which the compiler may otherwise place
// right before the first MFMA.
template <int NH>
__device__ __forceinline__ void pin_pk(bf16x8 (&pk)[NH]) {
  if constexpr (NH == 2)
    asm volatile("s_nop 1" : "+v"(pk[0]), "+v"(pk[1]));
  else
    asm volatile("s_nop 1" : "+v"(pk[0]));
}

// Score k-step ks of the chunk at (be, bo) (see score_chunk) for NH row
// groups, the two 16-position tiles' K pieces already in kb.
template <int NH>
__device__ __forceinline__ void score_step(int ks, const bf16x8 (&kb)[2],
                                           const bf16x8 (&qreg)[NH][18], f32x4 (&sacc)[NH][2]) {
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (ks == 0)
        mfma_sc0(sacc[h][t], kb[t], qreg[h][ks]);
      else
        mfma_sc(sacc[h][t], kb[t], qreg[h][ks]);
    }
}

// Unit map of one fused interval: kFusedScore score k-steps spread over the
// first fused_span(FT) of its kFusedScore + FT units, the FT P.V feature tiles
// in the others.
constexpr int kFusedScore = 18;
constexpr int kFusedAhead = 6;  // LDS reads issued six units ahead
// The first fused_pre(FT) units are P.V units: they read only the chunk
// whose probabilities are known, so their LDS reads are issued at the end of
// the previous interval, before its barrier (their latency hides under it).
constexpr int fused_pre(int ft, int ah = kFusedAhead) { return ft - 6 < ah ? ft - 6 : ah; }
// Then the score k-steps: on every other unit of 36 (32 tiles), or on the
// units that leave six after the last k-step (fewer tiles).
constexpr int fused_span(int ft, int ah = kFusedAhead) {
  return ft == 32 ? 36 : kFusedScore + ft - fused_pre(ft, ah) - 6;
}
// After unit fused_mid(FT) (the last score k-step) the scores are complete:
// the softmax of the next chunk runs in pieces between the remaining units.
constexpr int fused_mid(int ft, int ah = kFusedAhead) {
  return fused_pre(ft, ah) + (kFusedScore - 1) * fused_span(ft, ah) / kFusedScore;
}
template <int FT, int AH = kFusedAhead>
struct FusedMap {
  static constexpr int kUnits = kFusedScore + FT;
  static_assert(fused_mid(FT, AH) + 6 <= kUnits, "softmax pieces fit after the last k-step");
  int kind[kUnits];  // 0: score k-step, 1: P.V feature tile
  int idx[kUnits];   // the k-step or the tile
  int copy[kUnits];  // copy instructions issued at this unit
  constexpr FusedMap(int ncopies) : kind(), idx(), copy() {
    int s = 0, p = 0;
    for (int u = 0; u < kUnits; ++u) {
      if (s < kFusedScore && u == fused_pre(FT, AH) + s * fused_span(FT, AH) / kFusedScore) {
        kind[u] = 0;
        idx[u] = s++;
      } else {
        kind[u] = 1;
        idx[u] = p++;
      }
      copy[u] = 0;
    }
    // one copy per unit, from unit 1 on (every other unit while they last)
    for (int c = 0; c < ncopies; ++c) copy[(1 + 2 * c) % kUnits] += 1;
  }
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Reads of fused unit v into rb: a score k-step's two K pieces from the
// chunk at (be, bo), or a P.V feature tile of V^T from the chunk at pv (tile f
// of the wavefront's slice at vbase[f & 3] + 128 (f >> 2); vbase holds the
// slice's offset).
template <int V, int FT, int AH = kFusedAhead>
__device__ __forceinline__ void fused_reads(bf16x8 (&rb)[2], const MLA_LDS char* be,
                                            const MLA_LDS char* bo, const MLA_LDS char* pv,
                                            const int (&vbase)[4]) {
  constexpr FusedMap<FT, AH> m(0);
  constexpr int i = m.idx[V];
  if constexpr (m.kind[V] == 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      rb[t] = *reinterpret_cast<const MLA_LDS bf16x8*>((i & 1 ? bo : be) + 64 * i +
                                                       16 * kEntryBytes * t);
  } else {
    const int o = vbase[i & 3] + 128 * (i >> 2);
    const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pv + o));
    const bf16x4 a1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pv + (o + 16 * kEntryBytes)));
    rb[0] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// P.V of chunk j (slot `pv`, probabilities pk) fused with the scores of
// chunk j+1 (slot `sc`, into sacc), the copies of `cc` issued along the way.
// Every matrix instruction is an ordered asm statement, so the stream runs in
// the order written: per unit its copies, the LDS reads of the unit
// kFusedAhead later, then its MFMAs; after the last score k-step, mid(unit)
// runs between the units (the next chunk's softmax, see the kernel).
// The LDS reads of the first fused_pre(FT) units (P.V tiles of the chunk at
// pv), issued ahead of the interval.
template <int FT, int AH = kFusedAhead>
__device__ __forceinline__ void fused_prefetch(bf16x8 (&rb)[AH + 1][2],
                                               const MLA_LDS char* pv, const int (&vbase)[4]) {
  static_for<0, fused_pre(FT, AH)>([&](auto v_c) __attribute__((always_inline)) {
    constexpr int v = decltype(v_c)::value;
    fused_reads<v, FT, AH>(rb[v % (AH + 1)], nullptr, nullptr, pv, vbase);
  });
}

// (rb: the read-ahead registers, the first fused_pre(FT) units' reads already
// issued by fused_prefetch)
template <int NH, int FT, int KPER, int WB, int ST, bool SLOT, int AH, class Mid>
__device__ __forceinline__ void fused_interval(const MLA_LDS char* pv, const int (&vbase)[4],
                                               const bf16x8 (&pk)[NH], f32x4 (&oacc)[NH][FT],
                                               const MLA_LDS char* sc, int sbase_even,
                                               int sbase_odd, const bf16x8 (&qreg)[NH][18],
                                               f32x4 (&sacc)[NH][2], const ChunkCopy& cc,
                                               const uint32_t* off, int wave,
                                               bf16x8 (&rb)[AH + 1][2], Mid&& mid) {
  using M = FusedMap<FT, AH>;
  constexpr M m(KPER);
  constexpr int U = M::kUnits;
  const MLA_LDS char* be = sc + sbase_even;
  const MLA_LDS char* bo = sc + sbase_odd;
  static_for<fused_pre(FT, AH), AH>([&](auto v_c) __attribute__((always_inline)) {
    constexpr int v = decltype(v_c)::value;
    fused_reads<v, FT, AH>(rb[v % (AH + 1)], be, bo, pv, vbase);
  });
  static_for<0, U>([&](auto u_c) __attribute__((always_inline)) {
    constexpr int u = decltype(u_c)::value;
    constexpr int r = u % (AH + 1);
    constexpr int i = m.idx[u];
    constexpr int c0 = [] {
      constexpr M mm(KPER);
      int c = 0;
      for (int k = 0; k < u; ++k) c += mm.copy[k];
      return c;
    }();
    if constexpr (SLOT) {
      static_assert(KPER == 9, "nine copies a wavefront");
      static_for<0, m.copy[u]>([&](auto c_c) __attribute__((always_inline)) {
        row_piece<c0 + decltype(c_c)::value>(cc, off, wave);
      });
    } else {
#pragma unroll
      for (int c = 0; c < m.copy[u]; ++c) copy_piece<WB, ST>(cc, off, c0 + c, wave);
    }
    if constexpr (u + AH < U)
      fused_reads<u + AH, FT, AH>(rb[(u + AH) % (AH + 1)], be, bo, pv,
                                       vbase);
    if constexpr (m.kind[u] == 0) {
      score_step<NH>(i, rb[r], qreg, sacc);
    } else {
#pragma unroll
      for (int h = 0; h < NH; ++h) mfma_o(oacc[h][i], rb[r][0], pk[h]);
    }
    if constexpr (u >= fused_mid(FT, AH)) {
      // the next chunk's softmax in pieces between the remaining P.V units
      __builtin_amdgcn_sched_barrier(0);
      mid(u_c);
      __builtin_amdgcn_sched_barrier(0);
    }
  });
}

// One piece of the masked softmax of a chunk (see softmax_chunk): row group
// H, positions 16T .. 16T+15 of this lane's four: p = 2^(s - ref) (0 past the
// causal limit), summed into psum[H], rounded into pk[H][4T .. 4T+3].
template <int NH, int H, int T>
__device__ __forceinline__ void softmax_piece(const f32x4 (&sacc)[NH][2], bf16x8 (&pk)[NH],
                                              const float (&m_ref)[NH], float (&psum)[NH],
                                              const int (&lim)[NH]) {
  const float m_use = m_ref[H] == -INFINITY ? 0.f : m_ref[H];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sv = (16 * T + i > lim[H]) ? -INFINITY : sacc[H][T][i];
    const float p = __builtin_amdgcn_exp2f(sv - m_use);
    psum[H] = (T == 0 && i == 0) ? p : psum[H] + p;
    pk[H][T * 4 + i] = (__bf16)p;
  }
}

// Scores of one chunk alone (the first chunk of an item, and the restart
// passes), with the same asm MFMAs: reads of k-step ks + 3 issued before the
// MFMAs of k-step ks.
template <int NH>
__device__ __forceinline__ void score_only(const MLA_LDS char* buf, int sbase_even, int sbase_odd,
                                           const bf16x8 (&qreg)[NH][18], f32x4 (&sacc)[NH][2]) {
  const MLA_LDS char* be = buf + sbase_even;
  const MLA_LDS char* bo = buf + sbase_odd;
  constexpr int A = 3;
  bf16x8 kb[A + 1][2];
  auto kload = [&](int ks, bf16x8 (&dst)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      dst[t] = *reinterpret_cast<const MLA_LDS bf16x8*>((ks & 1 ? bo : be) + 64 * ks +
                                                        16 * kEntryBytes * t);
  };
#pragma unroll
  for (int ks = 0; ks < A; ++ks) kload(ks, kb[ks]);
#pragma unroll
  for (int ks = 0; ks < 18; ++ks) {
    if (ks + A < 18) kload(ks + A, kb[(ks + A) % (A + 1)]);
    score_step<NH>(ks, kb[ks % (A + 1)], qreg, sacc);
  }
}

// P.V of one chunk alone (the last chunk of an item, and the restart pass).
template <int NH, int FT>
__device__ __forceinline__ void pv_only(const MLA_LDS char* buf, const int (&vbase)[4],
                                        const bf16x8 (&pk)[NH], f32x4 (&oacc)[NH][FT]) {
  constexpr int A = 3;
  bf16x8 vb[A + 1];
  auto vload = [&](int f, bf16x8& dst) {
    const int o = vbase[f & 3] + 128 * (f >> 2);
    const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(buf + o));
    const bf16x4 a1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(buf + (o + 16 * kEntryBytes)));
    dst = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
#pragma unroll
  for (int f = 0; f < A; ++f) vload(f, vb[f]);
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    if (f + A < FT) vload(f + A, vb[(f + A) % (A + 1)]);
#pragma unroll
    for (int h = 0; h < NH; ++h) mfma_o(oacc[h][f], vb[f % (A + 1)], pk[h]);
  }
}

// FS = 1: four wavefronts of NH row groups each (4 NH 16 rows), every
// wavefront accumulating all 512 features of its rows.  FS = 2 or 4: FS
// wavefronts share the same NH row groups (each scores them, so each has the
// probabilities) and take 32 / FS feature tiles each; the workgroup covers
// (4 / FS) NH 16 rows.
// SLOT: the rows of each chunk are scattered cache rows named by a slot list
// (the kept rows of the sparse decode, read in place).
template <int NH, int FS, bool SLOT = false>
__global__ __launch_bounds__(256, 1) void decode_pipe_kernel(DecodeArgs a,
                                                             const int32_t* __restrict__ block_table) {
  constexpr int NW = 4;
  constexpr int NS = 4;
  using D = Dma<NW, false>;
  constexpr int kPer = D::kPerWave;
  // LDS read-ahead of the fused intervals, in units (the in-place form's
  // copy addressing takes the registers of one unit)
  constexpr int AH = SLOT ? kFusedAhead - 1 : kFusedAhead;
  static_assert(D::kSlotBytes == kBufBytes, "the chunk's copies fill the slot exactly");
  static_assert(NS * kBufBytes <= 160 * 1024, "the ring fits in LDS");
  static_assert(2 * kPer <= 63, "copies in flight within the 6-bit vmcnt");
  __shared__ __attribute__((aligned(1024))) char ring0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char ring3[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint32_t slot_lds[SLOT ? kSlotCap : 1];
  static_assert(!SLOT || NS * kBufBytes + 4 * kSlotCap <= 160 * 1024, "slot list beside the ring");
  auto ring = [&](auto slot_c) -> MLA_LDS char* {
    constexpr int S = decltype(slot_c)::value % NS;
    if constexpr (S == 0) return (MLA_LDS char*)ring0;
    else if constexpr (S == 1) return (MLA_LDS char*)ring1;
    else if constexpr (S == 2) return (MLA_LDS char*)ring2;
    else return (MLA_LDS char*)ring3;
  };

  // blockIdx -> (item, row group): as decode_kernel (items of one XCD form a
  // contiguous range of the item list)
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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int gq = lane >> 4;
  constexpr int FT = 32 / FS;                 // feature tiles of a wavefront
  constexpr int kRowsWg = (NW / FS) * NH * 16;  // rows of the workgroup
  const int fslice = wave % FS;               // this wavefront's feature slice
  const int row0 = rg * kRowsWg + (wave / FS) * 16 * NH;  // first row of this wavefront
  int tmax[NH];
  int tmax_min = 0x7fffffff;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    tmax[h] = len - a.q_len + (row0 + 16 * h) / a.heads;
    tmax_min = min(tmax_min, tmax[h]);
  }
  const int xs = gq ^ swz(n);
  const int sbase_even = n * kEntryBytes + 16 * xs;
  const int sbase_odd = n * kEntryBytes + 16 * (xs ^ 4) - 64;
  int vbase[4];
  {
    const int r4 = (lane & 15) >> 2;
    const int qq = lane & 3;
    const int row = 4 * gq + r4;
    const int y = (qq >> 1) ^ swz(row);
#pragma unroll
    for (int f4 = 0; f4 < 4; ++f4) {
      vbase[f4] = row * kEntryBytes + 16 * ((2 * f4) ^ y) + 8 * (qq & 1) + 32 * FT * fslice;
      asm volatile("" : "+v"(vbase[f4]));
    }
  }
  // The item's block ids in registers, lane L of btv[k] holding page
  // p0 + 64 k + L's: a chunk's block is then a lane read, not a scalar load
  // (whose wait, lgkmcnt(0), would also wait for every LDS read in flight).
  // Items of more than 256 pages read the table with scalar loads.  Loaded
  // before the query rows: loads complete in order, so the first copies
  // (which need the block ids) then wait for these few loads only.
  const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
  constexpr int kBtRegs = 4;
  const int npages = p1 - p0;
  const bool bt_regs = !SLOT && npages <= 64 * kBtRegs;
  int btv[kBtRegs];
#pragma unroll
  for (int k = 0; k < kBtRegs; ++k)
    btv[k] = (bt_regs && 64 * k + lane < npages) ? bt[p0 + 64 * k + lane] : 0;
  // rows in place: the item's slot list into LDS (4 bytes a lane, a
  // wavefront-uniform number of copies; lanes past the item's end write
  // zeros), waited for after the query loads are issued
  const int slot_n = min(p1 * kPage, len) - p0 * kPage;
  if constexpr (SLOT) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(a.slots + (int64_t)b * a.slot_stride + p0 * kPage), (short)0,
        4 * slot_n, kRsrcWord3);
    for (int c = wave; 64 * c < slot_n; c += 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MLA_LDS char*)slot_lds + 256 * c, 4,
                                               4 * lane + 256 * c, 0, 0, 0);
  }
  bf16x8 qreg[NH][18];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(
        a.q_abs + ((int64_t)b * a.rows_per_seq + row0 + 16 * h + n) * kEntry + 8 * gq);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[h][ks] = qp[4 * ks];
  }
  // (kept in registers: an indexed form of these would be moved to LDS;
  // pinned only now, so that the wait for them comes after the query loads
  // are issued)
  if constexpr (!SLOT) {
#pragma unroll
    for (int k = 0; k < kBtRegs; ++k) asm volatile("" : "+v"(btv[k]));
  }
  f32x4 oacc[NH][FT];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int f = 0; f < FT; ++f) oacc[h][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[NH], l_run[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m_ref[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  int* flag = a.restart_flag + blockIdx.x;
  if (threadIdx.x == 0) __atomic_store_n(flag, 0, __ATOMIC_RELAXED);

  const int tok_begin = p0 * kPage;
  const int tok_end = min(p1 * kPage, len);
  const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;
  const int jm = (tmax_min - tok_begin + 1) / kChunk;
  const char* cache = reinterpret_cast<const char*>(a.cache);
  uint32_t doff[kPer];
  if constexpr (SLOT) {
    static_assert(kPer == 9, "nine copies a wavefront");
    dma_row_offsets(wave, lane, doff);
  } else {
    dma_offsets<NW, kPer, false>(wave, lane, doff);
  }
  const __amdgpu_buffer_rsrc_t cache_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(cache), (short)0,
                                        SLOT ? (int)a.cache_bytes : 0, kRsrcWord3);
  auto chunk_copy = [&](auto slot_c, int j) -> ChunkCopy {
    if constexpr (SLOT) {
      // lane r (r < 8; the others repeat them): row 8 wave + r of chunk j,
      // from the staged slot list
      // (the lane index recomputed here: held through the chunk loop for
      // the restart pass it would take a register)
      int lane_r = threadIdx.x & 7;
      asm volatile("" : "+v"(lane_r));
      const int r = kChunk * j + 8 * wave + lane_r;
      const uint32_t sv = slot_lds[min(r, kSlotCap - 1)];
      return ChunkCopy{cache_rsrc, ring(slot_c),
                       r < slot_n ? sv * (uint32_t)kEntryBytes : kSlotOob};
    }
    const bool real = j < nchunks;
    const int lp = real ? (j >> 1) : 0;  // page of the item (two chunks a page)
    int64_t blk;
    if (bt_regs) {
      // one lane read per register, then a scalar select
      int b = __builtin_amdgcn_readlane(btv[0], lp & 63);
#pragma unroll
      for (int k = 1; k < kBtRegs; ++k) {
        const int bk = __builtin_amdgcn_readlane(btv[k], lp & 63);
        b = (lp >> 6) == k ? bk : b;
      }
      blk = b;
    } else {
      // (the scalar load is waited for here, on this path only)
      int b = bt[p0 + lp];
      asm volatile("" : "+s"(b));
      blk = b;
    }
    const int t = tok_begin + lp * kPage + (real ? (j & 1) * kChunk : 0);
    const int bytes = real ? min(tok_end - t, kChunk) * kEntryBytes : 0;
    const char* src = cache + (blk * kPage + (t % kPage)) * (int64_t)kEntryBytes;
    return ChunkCopy{
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, bytes, kRsrcWord3),
        ring(slot_c), 0u};
  };
  auto issue_all = [&](const ChunkCopy& cc) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if constexpr (!SLOT) copy_piece<D::kWaveBase, D::kStride>(cc, doff, i, wave);
    }
    if constexpr (SLOT)
      static_for<0, 9>([&](auto i_c) __attribute__((always_inline)) {
        row_piece<decltype(i_c)::value>(cc, doff, wave);
      });
  };
  // read-ahead registers of the fused intervals (see fused_prefetch)
  bf16x8 rb[AH + 1][2];
  auto chunk_limits = [&](int j, int (&lim)[NH]) {
    const int t0 = tok_begin + j * kChunk;
#pragma unroll
    for (int h = 0; h < NH; ++h) lim[h] = tmax[h] - t0 - 4 * gq;
  };
  bool need_restart = false;
  bf16x8 pk[NH];
  auto softmax = [&](f32x4 (&sacc)[NH][2], int j, auto first_c) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_c)::value;
    int lim[NH];
    chunk_limits(j, lim);
    if (j >= jm)
      need_restart |= softmax_chunk<NH, kFirst, true>(sacc, pk, m_ref, l_run, lim);
    else
      need_restart |= softmax_chunk<NH, kFirst, false>(sacc, pk, m_ref, l_run, lim);
  };

  using T = std::true_type;
  using F = std::false_type;
  // prologue: chunks 0..2 in flight; the scores and softmax of chunk 0
  if constexpr (SLOT) {
    // the slot list has landed once at most the query loads are pending;
    // the barrier makes every wavefront's part of it visible
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<NH * 18>());
    ring_barrier();
  }
  issue_all(chunk_copy(Slot<0>{}, 0));
  issue_all(chunk_copy(Slot<1>{}, 1));
  issue_all(chunk_copy(Slot<2>{}, 2));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * kPer>());
  ring_barrier();
  {
    f32x4 sacc[NH][2];
    score_only<NH>(ring(Slot<0>{}), sbase_even, sbase_odd, qreg, sacc);
    mfma_drain<NH>(sacc);
    softmax(sacc, 0, T{});
  }
  if (1 < nchunks) fused_prefetch<FT, AH>(rb, ring(Slot<0>{}), vbase);
  // interval j: P.V of chunk j (slot j % 4) with the scores of chunk j+1
  // (slot (j+1) % 4); chunk j+3 goes into slot (j+3) % 4, chunk j-1's.
  auto interval = [&](auto s_c, int j) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    // chunk j+1 has landed once at most chunk j+2's copies are pending; the
    // barrier also tells that every wavefront is done with chunk j-1.  (No
    // LDS-read wait before it: every read of chunk j-1 has been consumed,
    // and the reads in flight, this interval's prefetch, are of chunk j.)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<kPer>());
    asm volatile("s_barrier" ::: "memory");
    const ChunkCopy cc = chunk_copy(Slot<S + 3>{}, j + 3);
    if (j + 1 < nchunks) {
      f32x4 sacc[NH][2];
      bf16x8 pk_next[NH];
      float psum[NH];
      int lim[NH];
      chunk_limits(j + 1, lim);
      fused_interval<NH, FT, kPer, D::kWaveBase, D::kStride, SLOT, AH>(
          ring(Slot<S>{}), vbase, pk, oacc, ring(Slot<S + 1>{}), sbase_even, sbase_odd, qreg,
          sacc, cc, doff, wave, rb, [&](auto u_c) __attribute__((always_inline)) {
            // after the last score unit: the wait states, then one piece per
            // P.V unit (the mask is applied to every chunk: no branch splits
            // the interval, and only chunks at the causal limit change)
            constexpr int k = decltype(u_c)::value - fused_mid(FT, AH);
            if constexpr (k == 0) mfma_drain<NH>(sacc);
            if constexpr (k >= 1 && k <= 2 * NH)
              softmax_piece<NH, (k - 1) / 2, (k - 1) % 2>(sacc, pk_next, m_ref, psum, lim);
            if constexpr (k == 2 * NH + 1) {
#pragma unroll
              for (int h = 0; h < NH; ++h) {
                l_run[h] += psum[h];
                // every p <= psum: psum <= 2^16 bounds them all (NaN/inf fail too)
                need_restart |= !(psum[h] <= kSlackPow);
              }
            }
          });
#pragma unroll
      for (int h = 0; h < NH; ++h) pk[h] = pk_next[h];
      // the next interval's first P.V reads (chunk j+1), before its barrier
      if (j + 2 < nchunks) fused_prefetch<FT, AH>(rb, ring(Slot<S + 1>{}), vbase);
    } else if (j < nchunks) {
      issue_all(cc);
      pv_only<NH, FT>(ring(Slot<S>{}), vbase, pk, oacc);
    } else {
      issue_all(cc);
    }
  };
  for (int j = 0; j < nchunks; j += 4) {
    interval(Slot<0>{}, j);
    interval(Slot<1>{}, j + 1);
    interval(Slot<2>{}, j + 2);
    interval(Slot<3>{}, j + 3);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(need_restart) != 0 && lane == 0)
    __atomic_store_n(flag, 1, __ATOMIC_RELAXED);
  __syncthreads();
  const bool restart = __atomic_load_n(flag, __ATOMIC_RELAXED) != 0;

  // ---- restart (rare): exact row max, then a pass with it as the reference --
  if (restart) {
    auto fetch = [&](int j) -> const MLA_LDS char* {
      issue_all(chunk_copy(Slot<0>{}, j));
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      __syncthreads();
      return ring(Slot<0>{});
    };
    float m_exact[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) m_exact[h] = -INFINITY;
    for (int j = 0; j < nchunks; ++j) {
      const MLA_LDS char* buf = fetch(j);
      int lim[NH];
      chunk_limits(j, lim);
      f32x4 sacc[NH][2];
      score_only<NH>(buf, sbase_even, sbase_odd, qreg, sacc);
      mfma_drain<NH>(sacc);
      max_chunk<NH>(sacc, m_exact, lim);
      __syncthreads();
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      m_ref[h] = m_exact[h];
      l_run[h] = 0.f;
    }
    // Zeroed with no statement that reads the old tiles, so they are dead on
    // this path (passing them through mfma_drain_o first kept them alive
    // across the exact-max pass, and the compiler spilled them on every
    // item).  The wait states the drain provided are not needed here: the
    // last matrix instruction that wrote them is a whole pass (and its
    // barriers) behind, and the first that reads them a fetch and a softmax
    // ahead.
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int f = 0; f < FT; ++f) oacc[h][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < nchunks; ++j) {
      const MLA_LDS char* buf = fetch(j);
      f32x4 sacc[NH][2];
      score_only<NH>(buf, sbase_even, sbase_odd, qreg, sacc);
      mfma_drain<NH>(sacc);
      softmax(sacc, j, F{});
      pin_pk<NH>(pk);
      pv_only<NH, FT>(buf, vbase, pk, oacc);
      __syncthreads();
    }
  }
  mfma_drain_o<NH, FT>(oacc);

  // ---- finalise: each wavefront normalises its own rows; the workgroup's
  // rows then leave through LDS as whole 1 KB rows (a 16-byte piece per lane)
  // rather than as the MFMA tiles' 32-byte pieces of 16 rows.  The ring is
  // free here: every copy has landed and every wavefront is past its reads.
  // Staged row r sits in ring slot r / 32 as its row r % 32 (see
  // kStageStride).
  static_assert(32 * kStageStride <= kBufBytes && kRowsWg <= 32 * NS, "staged rows fit the ring");
  auto out_slot = [&](int r32) -> MLA_LDS char* {
    return r32 == 0 ? ring(Slot<0>{})
                    : r32 == 1 ? ring(Slot<1>{}) : r32 == 2 ? ring(Slot<2>{}) : ring(Slot<3>{});
  };
  const int wrow0 = (wave / FS) * 16 * NH;  // this wavefront's first row in the workgroup
  // the lane indices again, from a value the compiler cannot move above the
  // chunk loop (addresses derived from them would stay live through it)
  int lane_f = threadIdx.x & 63;
  asm volatile("" : "+v"(lane_f));
  const int n_f = lane_f & 15;
  const int gq_f = lane_f >> 4;
  // every row's sum and log-sum-exp first, then the tiles one by one
  float inv[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float l = l_run[h];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float lse = l > 0.f ? m_ref[h] + __builtin_amdgcn_logf(l) : -INFINITY;
    // (the FS wavefronts of a row group hold the same sums)
    if (gq_f == 0 && fslice == 0)
      a.lse_part[(int64_t)item * a.rows_per_seq + row0 + 16 * h + n_f] = lse;
    inv[h] = l > 0.f ? 1.f / l : 0.f;
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int r = wrow0 + 16 * h;
    const int sr = (r & 31) + n_f;  // row within the slot
    MLA_LDS char* dst =
        out_slot(r >> 5) + sr * kStageStride + 32 * FT * fslice + 8 * (gq_f ^ stage_swap(sr));
    // (each tile written as soon as it is converted: batching the writes
    // would hold all converted tiles in registers at once)
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      *reinterpret_cast<MLA_LDS u16x4*>(dst + 32 * f) = scaled_bf16x4(oacc[h][f], inv[h]);
      asm volatile("" : : : "memory");
    }
  }
  __syncthreads();
  uint16_t* orows = a.o_part + ((int64_t)item * a.rows_per_seq + rg * kRowsWg) * kLatent;
#pragma unroll 8
  for (int r = wave; r < kRowsWg; r += 4) {
    const u16x8 v = stage_read(out_slot(r >> 5), r & 31, lane_f);
    *reinterpret_cast<u16x8*>(orows + (int64_t)r * kLatent + 8 * lane_f) = v;
  }
}

// ---------------------------------------------------------------------------
// Pipelined decode over the FP8 cache: the kernel above with each chunk kept
// in LDS as its FP8 rows (656 bytes: 512 E4M3 codes, the 64 bf16 RoPE values,
// the scale byte and zero padding).  The ring slot of a chunk is 21 KB
// instead of 36.
//
// Scores on the FP8 matrix cores.  The latent part of S^T = K Q^T takes the
// codes as they are, as the A operand of the block-scaled MFMA 16x16x128
// (E4M3 x E4M3, fp32 accumulation; two 16-byte LDS reads give a lane its 32
// codes).  The absorbed query (bf16) is carried as two E4M3 terms per value:
// with S = the row's power-of-two scale (largest with max |q| S <= 448),
// hi = q S rounded to E4M3 and lo = (q S - hi) 16 rounded to E4M3.  A bf16
// value has eight significant bits, hi keeps the top four and the remainder
// needs at most four, so hi + lo / 16 is q S exactly (unless lo falls below
// the E4M3 normal range: parts below 2^-6 of the row's largest value).  Each
// k-step runs the hi MFMA with unit scales and the lo MFMA with a B scale of
// 2^-4 into the same accumulator, so the latent scores cost two FP8 MFMAs per
// 128 dimensions (the matrix time of four bf16 16x16x32 k-steps).  After the
// last latent k-step each score is multiplied by its token's scale times
// 1 / S, and the two bf16 RoPE k-steps add the RoPE part.
// P.V keeps the bf16 MFMA: its operand V^T comes from the codes through the
// transposing byte read (ds_read_b64_tr_b8, one per 16 features x 32
// positions) and four conversions to bf16, and the weights are p times the
// token's scale (bf16(p 2^e) = bf16(p) 2^e), so the codes need no scale.
//
// Position order.  Score tile t, row 4g + i (g = 0..3, i = 0..3) is chunk
// position 8g + 4t + i.  A lane's four scores of tile t are then positions
// 8gq + 4t + i, its eight scores of the chunk positions 8gq .. 8gq+7: exactly
// the eight positions its P.V operand holds (P.V index k = chunk position).
// The transposing read supplies them from eight rows: lane L addresses row
// L >> 1, half L & 1 of a 16-byte feature group, and receives feature L & 15
// of rows 8 (L >> 4) .. 8 (L >> 4) + 7.
// Latent dimensions.  In k-step k (0..3) lane (n, gq = 2 g1 + g0) holds the
// codes of the 16-byte units 8k + 4 g0 + g1 and 8k + 4 g0 + g1 + 2 of its row
// (32 dimensions), the query terms of the same dimensions in the same byte
// order (the contraction is a sum over dimensions: any order both operands
// share gives the same products).  RoPE k-step 16 + r reads unit 32 + 4 g0 +
// 2 r + g1 (bf16).  Rows are 656 bytes apart, i.e. 144 bytes (nine 16-byte
// units) apart modulo the 256-byte bank window; with this order every read
// pattern of the kernel is free of bank conflicts (each lane's banks
// enumerated).
// Scales.  The chunk's 32 scale bytes come with the chunk: one 4-byte-per-
// lane copy puts their dwords in a 128-byte array after the rows.
// Hazards.  The P.V operands are converted by vector instructions and feed
// asm MFMAs, which the compiler does not see as matrix instructions: each is
// produced one unit before its MFMAs and pinned there (an ordered empty asm
// statement), so the previous unit's MFMAs stand between them (two wait
// states are required; with one row group per wavefront the pin adds an
// s_nop).  Vector instructions read FP8 MFMA results only after 16 wait
// states (mfma_drain_f8).

constexpr int kF8ChunkBytes = kChunk * kFp8EntryBytes;  // 20992
constexpr int kF8Whole = 20;                            // whole 1 KB copies of a chunk
constexpr int kF8Tail = kF8Whole * 1024;                // 20480: the last 512 bytes after it
constexpr int kF8ScaleLds = kF8ChunkBytes;              // 32 scale dwords after the rows
constexpr int kF8SlotBytes = kF8ScaleLds + 512;         // 21504
constexpr int kF8Per = 6;                               // copy instructions per wavefront
constexpr int kF8Ahead = 5;                             // LDS reads issued five units ahead
constexpr int kE8m0One = 127;                           // MFMA block scale 2^0
constexpr int kE8m0Lo = 127 - 4;                        // 2^-4: the lo query term

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_gnu_t __attribute__((vector_size(8)));

// ds_read_b64_tr_b8 at p (see the position order for the lane layout).
__device__ __forceinline__ u32x2_t ds_read_tr8(const MLA_LDS char* p) {
  const i32x2_gnu_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2_gnu_t*)p);
  return u32x2_t{(uint32_t)r[0], (uint32_t)r[1]};
}

// Source offsets of a wavefront's copies of one chunk (four wavefronts).
// Copies 0..4: 1 KB each, copy i of wavefront w fills chunk bytes
// 1024 (4i + w) ..; copy 5 moves 4 bytes per lane: the chunk's last 512 bytes
// (wavefronts 0 and 1), the scale dwords of the 32 rows (wavefront 2, lanes
// 0..31), nothing (wavefront 3).  Its LDS destination is kF8Tail + 256 w: the
// tail lands in place and the scales at kF8ScaleLds.
__device__ __forceinline__ void dma_offsets_f8(int wave, int lane, uint32_t (&off)[kF8Per]) {
#pragma unroll
  for (int i = 0; i < kF8Per - 1; ++i) off[i] = (uint32_t)(1024 * (4 * i + wave) + 16 * lane);
  uint32_t o5 = 0x80000000u;  // beyond any range: no memory access, zeros to LDS
  if (wave < 2) o5 = (uint32_t)(kF8Tail + 256 * wave + 4 * lane);
  if (wave == 2 && lane < kChunk) o5 = (uint32_t)(lane * kFp8EntryBytes + kFp8ScaleOff);
  off[kF8Per - 1] = o5;
}

// Copy instruction I (0..5) of the wavefront's share of an FP8 chunk.
template <int I>
__device__ __forceinline__ void copy_piece_f8(const ChunkCopy& c, const uint32_t* off, int wave) {
  if constexpr (I < kF8Per - 1)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, c.dst + wave * 1024 + I * 4096, 16, off[I], 0,
                                             0, kCopyPolicy);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, c.dst + kF8Tail + 256 * wave, 4, off[I], 0, 0,
                                             kCopyPolicy);
}

// Eight E4M3 codes (two dwords, code k in byte k) as eight bf16 values.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t d0, uint32_t d1) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// A token's scale 2^(s - 127) from its scale dword (s in the low byte).
__device__ __forceinline__ float f8_scale(uint32_t dw) { return __uint_as_float((dw & 0xffu) << 23); }

// The block-scaled FP8 MFMA (both operands E4M3; sa, sb: E8M0 scales, the same
// in every lane).  _0: with a zero accumulator.
__device__ __forceinline__ void mfma_f8_0(f32x4& acc, const u32x8_t& a, const u32x8_t& b, int sa,
                                          int sb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(acc)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void mfma_f8(f32x4& acc, const u32x8_t& a, const u32x8_t& b, int sa,
                                        int sb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(acc)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
// 16 wait states after the last FP8 score MFMA, ordered before every read of
// the scores.
template <int NH>
__device__ __forceinline__ void mfma_drain_f8(f32x4 (&sacc)[NH][2]) {
  static_assert(NH == 1 || NH == 2, "two or four score tiles");
  if constexpr (NH == 2)
    asm volatile("s_nop 7\n\ts_nop 7"
                 : "+v"(sacc[0][0]), "+v"(sacc[0][1]), "+v"(sacc[1][0]), "+v"(sacc[1][1]));
  else
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(sacc[0][0]), "+v"(sacc[0][1]));
}

// Per-lane LDS offsets inside a slot (see the position order above).
struct F8Lane {
  int k;  // score reads: row 8 (n >> 2) + (n & 3), unit 4 g0 + g1
  int v;  // transposing reads: row lane >> 1, half lane & 1, the wavefront's feature slice
  int s;  // scale reads: dwords 8 gq .. 8 gq + 7
};

// Offset (relative to F8Lane::k) of the first of latent k-step k's two reads
// of tile t (the second is 32 bytes further), and of RoPE k-step 16 + r.
constexpr int f8_kread(int k, int t) { return 4 * kFp8EntryBytes * t + 128 * k; }
constexpr int f8_rread(int r, int t) { return 4 * kFp8EntryBytes * t + kFp8RopeOff + 32 * r; }

// The query of a wavefront's NH row groups in the operand forms above.
template <int NH>
struct F8Query {
  u32x8_t hi[NH][4];   // latent k-steps: q S as E4M3
  u32x8_t lo[NH][4];   // (q S - hi) 16 as E4M3
  bf16x8 rope[NH][2];  // RoPE k-steps (bf16, as given)
  float inv_s[NH];     // 1 / S of the lane's row
};

// Split one row group's absorbed query (q: the lane's bf16 row of 576) into
// the operand forms: the lane's 128 latent values (units 8k + 4 g0 + g1 and
// + 2 for k = 0..3), the row scale S from the four lanes of the row.  Two
// passes over the values (the second reads them again from cache) keep the
// prologue's registers to those of the result.
template <int NH>
__device__ __forceinline__ void f8_split_query(const uint16_t* q, int g0, int g1, int h,
                                               F8Query<NH>& fq) {
  auto load = [&](int k, int j) -> u16x8 {  // 8 values: unit 8k + 4 g0 + g1 + 2 (j >> 1), half j & 1
    return *reinterpret_cast<const u16x8*>(q + 16 * (8 * k + 4 * g0 + g1 + 2 * (j >> 1)) +
                                           8 * (j & 1));
  };
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u16x8 v = load(k, j);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(__uint_as_float((uint32_t)v[e] << 16)));
    }
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  // S: the power of two at or below 448 / amax, kept within [2^-64, 2^64]
  // (an all-zero row gives 2^64 and zero codes)
  const float t = fminf(fmaxf(448.f / amax, 0x1p-64f), 0x1p64f);
  const float s = __uint_as_float(__float_as_uint(t) & 0xff800000u);
  fq.inv_s[h] = 1.f / s;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u16x8 v = load(k, j);
#pragma unroll
      for (int w = 0; w < 2; ++w) {  // dword 2j + w of the operand: values 4w .. 4w+3 of v
        uint32_t hw = 0, lw = 0;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float a = __uint_as_float((uint32_t)v[4 * w + 2 * p] << 16) * s;
          const float b = __uint_as_float((uint32_t)v[4 * w + 2 * p + 1] << 16) * s;
          const int hc = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
          const f32x2_t hv = __builtin_amdgcn_cvt_pk_f32_fp8(hc, false);
          const int lc =
              __builtin_amdgcn_cvt_pk_fp8_f32((a - hv[0]) * 16.f, (b - hv[1]) * 16.f, 0, false);
          hw |= ((uint32_t)hc & 0xffffu) << (16 * p);
          lw |= ((uint32_t)lc & 0xffffu) << (16 * p);
        }
        fq.hi[h][k][2 * j + w] = hw;
        fq.lo[h][k][2 * j + w] = lw;
      }
    }
  // (each term computed before this point; the kernel adds the wait states
  // before the first MFMA reads them)
#pragma unroll
  for (int k = 0; k < 4; ++k) asm volatile("" : "+v"(fq.hi[h][k]), "+v"(fq.lo[h][k]));
#pragma unroll
  for (int r = 0; r < 2; ++r)
    fq.rope[h][r] = *reinterpret_cast<const bf16x8*>(q + kLatent + 32 * g0 + 16 * r + 8 * g1);
}

// Unit map of one FP8 interval: LU latent score units (per k-step: one per
// tile with two row groups, both tiles in one with one, so that the hi and lo
// MFMAs of an accumulator are never adjacent), two RoPE units, FT P.V feature
// tiles; the score units spread over the interval as in FusedMap.
template <int NH>
constexpr int f8_lat_units() { return NH == 2 ? 8 : 4; }
template <int NH>
constexpr int f8_score_units() { return f8_lat_units<NH>() + 2; }
constexpr int f8_pre(int ft) { return ft - 6 < kF8Ahead ? ft - 6 : kF8Ahead; }
template <int NH, int FT>
constexpr int f8_span() { return f8_score_units<NH>() + FT - f8_pre(FT) - 6; }
template <int NH, int FT>
constexpr int f8_mid() {
  return f8_pre(FT) + (f8_score_units<NH>() - 1) * f8_span<NH, FT>() / f8_score_units<NH>();
}
template <int NH, int FT>
struct F8Map {
  static constexpr int kScore = f8_score_units<NH>();
  static constexpr int kUnits = kScore + FT;
  static_assert(f8_mid<NH, FT>() + 6 <= kUnits, "softmax pieces fit after the last k-step");
  static_assert(kUnits >= 2 * kF8Per, "the copies fit in the interval");
  int kind[kUnits];  // 0: latent score unit, 1: P.V feature tile, 2: RoPE k-step
  int idx[kUnits];   // latent unit, tile or RoPE k-step
  int copy[kUnits];  // copy instructions issued at this unit
  constexpr F8Map() : kind(), idx(), copy() {
    int s = 0, p = 0;
    for (int u = 0; u < kUnits; ++u) {
      if (s < kScore && u == f8_pre(FT) + s * f8_span<NH, FT>() / kScore) {
        kind[u] = s < f8_lat_units<NH>() ? 0 : 2;
        idx[u] = s < f8_lat_units<NH>() ? s : s - f8_lat_units<NH>();
        ++s;
      } else {
        kind[u] = 1;
        idx[u] = p++;
      }
      copy[u] = 0;
    }
    for (int c = 0; c < kF8Per; ++c) copy[1 + 2 * c] += 1;
  }
};

// LDS data of one interval's units (indexed by compile-time unit indices
// only, so every element is a register of its own, live from its read to its
// use): latent codes per k-step and tile, RoPE operands, V^T codes, the
// chunk's scale dwords.
template <int FT>
struct F8Raw {
  u32x8_t k[4][2];
  bf16x8 r[2][2];
  u32x2_t v[FT];
  u32x4_t s[2];
};

// The latent k-steps and tiles of latent unit i (one tile with two row groups,
// both tiles with one).
template <int NH>
constexpr int f8_lat_k(int i) { return NH == 2 ? i >> 1 : i; }
template <int NH>
constexpr int f8_lat_t0(int i) { return NH == 2 ? (i & 1) : 0; }
template <int NH>
constexpr int f8_lat_nt() { return NH == 2 ? 1 : 2; }

template <int NH>
__device__ __forceinline__ void f8_read_lat(u32x8_t& dst, const MLA_LDS char* p) {
  const u32x4_t a = *reinterpret_cast<const MLA_LDS u32x4_t*>(p);
  const u32x4_t b = *reinterpret_cast<const MLA_LDS u32x4_t*>(p + 32);
  dst = u32x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int NH, int FT, int V>
__device__ __forceinline__ void f8_reads(F8Raw<FT>& x, const MLA_LDS char* sc,
                                         const MLA_LDS char* pv, const F8Lane& ln) {
  constexpr F8Map<NH, FT> m;
  constexpr int i = m.idx[V];
  if constexpr (m.kind[V] == 0) {
    constexpr int k = f8_lat_k<NH>(i);
#pragma unroll
    for (int t = f8_lat_t0<NH>(i); t < f8_lat_t0<NH>(i) + f8_lat_nt<NH>(); ++t)
      f8_read_lat<NH>(x.k[k][t], sc + ln.k + f8_kread(k, t));
    if constexpr (i == f8_lat_units<NH>() - 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        x.s[t] = *reinterpret_cast<const MLA_LDS u32x4_t*>(sc + kF8ScaleLds + ln.s + 16 * t);
    }
  } else if constexpr (m.kind[V] == 2) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      x.r[i][t] = *reinterpret_cast<const MLA_LDS bf16x8*>(sc + ln.k + f8_rread(i, t));
  } else {
    x.v[i] = ds_read_tr8(pv + ln.v + 16 * i);
  }
}

// Two wait states with the operands of the MFMAs that follow in registers
// (inputs of this statement).  Where the output tiles leave accumulation
// registers free, the register allocator may keep an operand there and copy
// it back right before its asm MFMA; the copy, a vector instruction, then
// lands before these wait states.
// (plain overloads: the host pass rejects templates around these asm operands)
__device__ __forceinline__ void mfma_guard(const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1" ::"v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_guard(const bf16x8& a, const bf16x8& b, const bf16x8& c) {
  asm volatile("s_nop 1" ::"v"(a), "v"(b), "v"(c));
}
__device__ __forceinline__ void mfma_guard(const bf16x8& a, const bf16x8& b, const bf16x8& c,
                                           const bf16x8& d) {
  asm volatile("s_nop 1" ::"v"(a), "v"(b), "v"(c), "v"(d));
}
__device__ __forceinline__ void mfma_guard(const u32x8_t& a, const u32x8_t& b, const u32x8_t& c,
                                           const u32x8_t& d) {
  asm volatile("s_nop 1" ::"v"(a), "v"(b), "v"(c), "v"(d));
}
__device__ __forceinline__ void mfma_guard(const u32x8_t& a, const u32x8_t& b, const u32x8_t& c,
                                           const u32x8_t& d, const u32x8_t& e, const u32x8_t& f) {
  asm volatile("s_nop 1" ::"v"(a), "v"(b), "v"(c), "v"(d), "v"(e), "v"(f));
}

// The latent MFMAs of k-step k, tiles T0 .. T0 + NT - 1: every hi product
// before any lo product, so two MFMAs on one accumulator are never adjacent.
template <int NH, int K, int T0, int NT, bool GUARD>
__device__ __forceinline__ void f8_lat_mfma(f32x4 (&sacc)[NH][2], const u32x8_t (&a)[2],
                                            const F8Query<NH>& fq, int e_one, int e_lo) {
  if constexpr (GUARD) {
    if constexpr (NH == 2)
      mfma_guard(a[T0], a[T0 + NT - 1], fq.hi[0][K], fq.hi[1][K], fq.lo[0][K], fq.lo[1][K]);
    else
      mfma_guard(a[T0], a[T0 + NT - 1], fq.hi[0][K], fq.lo[0][K]);
  }
#pragma unroll
  for (int t = T0; t < T0 + NT; ++t)
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      if constexpr (K == 0)
        mfma_f8_0(sacc[h][t], a[t], fq.hi[h][K], e_one, e_one);
      else
        mfma_f8(sacc[h][t], a[t], fq.hi[h][K], e_one, e_one);
    }
#pragma unroll
  for (int t = T0; t < T0 + NT; ++t)
#pragma unroll
    for (int h = 0; h < NH; ++h) mfma_f8(sacc[h][t], a[t], fq.lo[h][K], e_one, e_lo);
}

// The latent scores times token scale / S (before the RoPE k-steps add their
// part): the wait states after the FP8 MFMAs, the products, two wait states
// before the next MFMA reads them.  scl receives the chunk's token scales.
template <int NH>
__device__ __forceinline__ void f8_scale_scores(f32x4 (&sacc)[NH][2], const u32x4_t (&s)[2],
                                                const float (&inv_s)[NH], float (&scl)[8]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) scl[4 * t + i] = f8_scale(s[t][i]);
  mfma_drain_f8<NH>(sacc);
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[h][t][i] *= scl[4 * t + i] * inv_s[h];
  if constexpr (NH == 2)
    asm volatile("s_nop 1"
                 : "+v"(sacc[0][0]), "+v"(sacc[0][1]), "+v"(sacc[1][0]), "+v"(sacc[1][1]));
  else
    asm volatile("s_nop 1" : "+v"(sacc[0][0]), "+v"(sacc[0][1]));
}

// The V^T reads of the first f8_pre(FT) units (P.V tiles of the chunk at
// pv), issued ahead of the interval.
template <int FT>
__device__ __forceinline__ void f8_prefetch(u32x2_t (&vpre)[f8_pre(FT)], const MLA_LDS char* pv,
                                            const F8Lane& ln) {
#pragma unroll
  for (int f = 0; f < f8_pre(FT); ++f) vpre[f] = ds_read_tr8(pv + ln.v + 16 * f);
}

// P.V of chunk j (slot pv, weights pk) fused with the scores of chunk j+1
// (slot sc, into sacc; its scales into scl), the copies of cc along the way:
// per unit its copies, the reads of the unit kF8Ahead later, the conversion
// of the next unit's V^T operand, then its MFMAs; after the last score unit,
// mid(unit) between the units.
template <int NH, int FT, bool GUARD, class Mid>
__device__ __forceinline__ void fused_interval_f8(const MLA_LDS char* pv, const bf16x8 (&pk)[NH],
                                                  f32x4 (&oacc)[NH][FT], const MLA_LDS char* sc,
                                                  const F8Lane& ln, const F8Query<NH>& fq,
                                                  int e_one, int e_lo, f32x4 (&sacc)[NH][2],
                                                  float (&scl)[8], const ChunkCopy& cc,
                                                  const uint32_t* off, int wave,
                                                  const u32x2_t (&vpre)[f8_pre(FT)], Mid&& mid) {
  using M = F8Map<NH, FT>;
  constexpr M m;
  constexpr int U = M::kUnits;
  static_assert(f8_pre(FT) <= kF8Ahead, "the prefetched units precede the read-ahead window");
  F8Raw<FT> x;
#pragma unroll
  for (int f = 0; f < f8_pre(FT); ++f) x.v[f] = vpre[f];
  static_for<f8_pre(FT), kF8Ahead>([&](auto v_c) __attribute__((always_inline)) {
    f8_reads<NH, FT, decltype(v_c)::value>(x, sc, pv, ln);
  });
  bf16x8 cv[U];
  cv[0] = fp8x8_to_bf16(x.v[0][0], x.v[0][1]);
  asm volatile("s_nop 1" : "+v"(cv[0]));
  static_for<0, U>([&](auto u_c) __attribute__((always_inline)) {
    constexpr int u = decltype(u_c)::value;
    constexpr int i = m.idx[u];
    constexpr int c0 = [] {
      constexpr M mm;
      int c = 0;
      for (int k = 0; k < u; ++k) c += mm.copy[k];
      return c;
    }();
    static_for<0, m.copy[u]>([&](auto c_c) __attribute__((always_inline)) {
      copy_piece_f8<c0 + decltype(c_c)::value>(cc, off, wave);
    });
    if constexpr (u + kF8Ahead < U) f8_reads<NH, FT, u + kF8Ahead>(x, sc, pv, ln);
    if constexpr (u + 1 < U && m.kind[u + 1] == 1) {
      constexpr int f = m.idx[u + 1];
      cv[u + 1] = fp8x8_to_bf16(x.v[f][0], x.v[f][1]);
      if constexpr (NH == 1) asm volatile("s_nop 1" : "+v"(cv[u + 1]));
      else asm volatile("" : "+v"(cv[u + 1]));
    }
    if constexpr (m.kind[u] == 0) {
      f8_lat_mfma<NH, f8_lat_k<NH>(i), f8_lat_t0<NH>(i), f8_lat_nt<NH>(), GUARD>(
          sacc, x.k[f8_lat_k<NH>(i)], fq, e_one, e_lo);
    } else if constexpr (m.kind[u] == 2) {
      if constexpr (i == 0) f8_scale_scores<NH>(sacc, x.s, fq.inv_s, scl);
      if constexpr (GUARD) {
        if constexpr (NH == 2)
          mfma_guard(x.r[i][0], x.r[i][1], fq.rope[0][i], fq.rope[1][i]);
        else
          mfma_guard(x.r[i][0], x.r[i][1], fq.rope[0][i]);
      }
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) mfma_sc(sacc[h][t], x.r[i][t], fq.rope[h][i]);
    } else {
      if constexpr (GUARD) {
        if constexpr (NH == 2)
          mfma_guard(cv[u], pk[0], pk[1]);
        else
          mfma_guard(cv[u], pk[0]);
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) mfma_o(oacc[h][i], cv[u], pk[h]);
    }
    if constexpr (u >= f8_mid<NH, FT>()) {
      __builtin_amdgcn_sched_barrier(0);
      mid(u_c);
      __builtin_amdgcn_sched_barrier(0);
    }
  });
}

// One piece of the FP8 chunk's masked softmax: row group H, tile T of the
// lane's positions (8 gq + 4T + i): p = 2^(s - ref) (0 past the causal limit:
// lim = the last visible position - 8 gq), summed into psum[H], and p times
// the token scale rounded into pk[H][4T + i].
template <int NH, int H, int T>
__device__ __forceinline__ void softmax_piece_f8(const f32x4 (&sacc)[NH][2], bf16x8 (&pk)[NH],
                                                 const float (&m_ref)[NH], float (&psum)[NH],
                                                 const int (&lim)[NH], const float (&scl)[8]) {
  const float m_use = m_ref[H] == -INFINITY ? 0.f : m_ref[H];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sv = (4 * T + i > lim[H]) ? -INFINITY : sacc[H][T][i];
    const float p = __builtin_amdgcn_exp2f(sv - m_use);
    psum[H] = (T == 0 && i == 0) ? p : psum[H] + p;
    pk[H][T * 4 + i] = (__bf16)(p * scl[4 * T + i]);
  }
}

// Softmax of a whole FP8 chunk (the first chunk of an item, and the restart
// pass): as softmax_chunk with the FP8 position order and weights.
template <int NH, bool FIRST>
__device__ __forceinline__ bool softmax_chunk_f8(const f32x4 (&sacc)[NH][2], bf16x8 (&pk)[NH],
                                                 float (&m_ref)[NH], float (&l_run)[NH],
                                                 const int (&lim)[NH], const float (&scl)[8]) {
  bool restart = false;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float sv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[k] = (k > lim[h]) ? -INFINITY : sacc[h][k >> 2][k & 3];
    if (FIRST) {
      float mloc = sv[0];
#pragma unroll
      for (int k = 1; k < 8; ++k) mloc = fmaxf(mloc, sv[k]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      m_ref[h] = mloc;
    }
    const float m_use = m_ref[h] == -INFINITY ? 0.f : m_ref[h];
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p = __builtin_amdgcn_exp2f(sv[k] - m_use);
      psum += p;
      pk[h][k] = (__bf16)(p * scl[k]);
    }
    l_run[h] += psum;
    if (!FIRST) restart |= !(psum <= kSlackPow);
  }
  return restart;
}

// Row max of an FP8 chunk's scores (the first pass of a restart).
template <int NH>
__device__ __forceinline__ void max_chunk_f8(const f32x4 (&sacc)[NH][2], float (&m)[NH],
                                             const int (&lim)[NH]) {
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float mloc = -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) mloc = fmaxf(mloc, (k > lim[h]) ? -INFINITY : sacc[h][k >> 2][k & 3]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    m[h] = fmaxf(m[h], mloc);
  }
}

// Scores of one FP8 chunk alone (the first chunk of an item, the restart
// passes), scaled, with the chunk's scales in scl.
template <int NH>
__device__ __forceinline__ void score_only_f8(const MLA_LDS char* buf, const F8Lane& ln,
                                              const F8Query<NH>& fq, int e_one, int e_lo,
                                              f32x4 (&sacc)[NH][2], float (&scl)[8]) {
  u32x8_t kr[4][2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int t = 0; t < 2; ++t) f8_read_lat<NH>(kr[k][t], buf + ln.k + f8_kread(k, t));
  static_for<0, 4>([&](auto k_c) __attribute__((always_inline)) {
    constexpr int k = decltype(k_c)::value;
    if constexpr (k + 2 < 4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) f8_read_lat<NH>(kr[k + 2][t], buf + ln.k + f8_kread(k + 2, t));
    }
    f8_lat_mfma<NH, k, 0, 2, true>(sacc, kr[k], fq, e_one, e_lo);
  });
  u32x4_t s[2];
  bf16x8 rr[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = *reinterpret_cast<const MLA_LDS u32x4_t*>(buf + kF8ScaleLds + ln.s + 16 * t);
#pragma unroll
    for (int r = 0; r < 2; ++r)
      rr[r][t] = *reinterpret_cast<const MLA_LDS bf16x8*>(buf + ln.k + f8_rread(r, t));
  }
  f8_scale_scores<NH>(sacc, s, fq.inv_s, scl);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if constexpr (NH == 2)
      mfma_guard(rr[r][0], rr[r][1], fq.rope[0][r], fq.rope[1][r]);
    else
      mfma_guard(rr[r][0], rr[r][1], fq.rope[0][r]);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int t = 0; t < 2; ++t) mfma_sc(sacc[h][t], rr[r][t], fq.rope[h][r]);
  }
}

// P.V of one FP8 chunk alone (the last chunk of an item, the restart pass).
template <int NH, int FT>
__device__ __forceinline__ void pv_only_f8(const MLA_LDS char* buf, const F8Lane& ln,
                                           const bf16x8 (&pk)[NH], f32x4 (&oacc)[NH][FT]) {
  constexpr int A = 4;
  u32x2_t vr[FT];
#pragma unroll
  for (int f = 0; f < A; ++f) vr[f] = ds_read_tr8(buf + ln.v + 16 * f);
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    if (f + A < FT) vr[f + A] = ds_read_tr8(buf + ln.v + 16 * (f + A));
    const bf16x8 c = fp8x8_to_bf16(vr[f][0], vr[f][1]);
    if constexpr (NH == 2)
      mfma_guard(c, pk[0], pk[1]);
    else
      mfma_guard(c, pk[0]);
#pragma unroll
    for (int h = 0; h < NH; ++h) mfma_o(oacc[h][f], c, pk[h]);
  }
}

// The pipelined kernel over FP8 rows (NH, FS as decode_pipe_kernel).
template <int NH, int FS>
__global__ __launch_bounds__(256, 1) void decode_pipe_f8_kernel(
    DecodeArgs a, const int32_t* __restrict__ block_table) {
  constexpr int NW = 4;
  constexpr int NS = 4;
  static_assert(kF8Per * NW * 1024 >= kF8ChunkBytes, "the copies cover the chunk");
  static_assert(kF8Tail + 512 == kF8ChunkBytes, "two 256-byte tail copies finish it");
  static_assert(NS * kF8SlotBytes <= 160 * 1024, "the ring fits in LDS");
  __shared__ __attribute__((aligned(1024))) char ring0[kF8SlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[kF8SlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[kF8SlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring3[kF8SlotBytes];
  auto ring = [&](auto slot_c) -> MLA_LDS char* {
    constexpr int S = decltype(slot_c)::value % NS;
    if constexpr (S == 0) return (MLA_LDS char*)ring0;
    else if constexpr (S == 1) return (MLA_LDS char*)ring1;
    else if constexpr (S == 2) return (MLA_LDS char*)ring2;
    else return (MLA_LDS char*)ring3;
  };

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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int gq = lane >> 4;
  const int g0 = gq & 1;
  const int g1 = gq >> 1;
  constexpr int FT = 32 / FS;
  constexpr int kRowsWg = (NW / FS) * NH * 16;
  // output tiles short of the 256 accumulation registers: guard the MFMAs
  constexpr bool kGuard = NH * FT * 4 < 256;
  const int fslice = wave % FS;
  const int row0 = rg * kRowsWg + (wave / FS) * 16 * NH;
  int tmax[NH];
  int tmax_min = 0x7fffffff;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    tmax[h] = len - a.q_len + (row0 + 16 * h) / a.heads;
    tmax_min = min(tmax_min, tmax[h]);
  }
  F8Lane ln;
  ln.k = kFp8EntryBytes * (8 * (n >> 2) + (n & 3)) + 16 * (4 * g0 + g1);
  ln.v = kFp8EntryBytes * (lane >> 1) + 8 * (lane & 1) + 16 * FT * fslice;
  ln.s = 32 * gq;
  asm volatile("" : "+v"(ln.k), "+v"(ln.v), "+v"(ln.s));
  // the absorbed query as FP8 terms (latent) and bf16 (RoPE); the MFMA block
  // scales in registers; then two wait states before any MFMA reads them
  int e_one = kE8m0One, e_lo = kE8m0Lo;
  asm volatile("" : "+v"(e_one), "+v"(e_lo));
  // the block ids first (as decode_pipe_kernel): the query split below waits
  // for its loads, and these then arrive with them rather than after
  const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
  constexpr int kBtRegs = 4;
  const int npages = p1 - p0;
  const bool bt_regs = npages <= 64 * kBtRegs;
  int btv[kBtRegs];
#pragma unroll
  for (int k = 0; k < kBtRegs; ++k)
    btv[k] = (bt_regs && 64 * k + lane < npages) ? bt[p0 + 64 * k + lane] : 0;
  F8Query<NH> fq;
#pragma unroll
  for (int h = 0; h < NH; ++h)
    f8_split_query<NH>(a.q_abs + ((int64_t)b * a.rows_per_seq + row0 + 16 * h + n) * kEntry, g0,
                       g1, h, fq);
  asm volatile("s_nop 1" ::: "memory");
#pragma unroll
  for (int k = 0; k < kBtRegs; ++k) asm volatile("" : "+v"(btv[k]));
  f32x4 oacc[NH][FT];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int f = 0; f < FT; ++f) oacc[h][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref[NH], l_run[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    m_ref[h] = -INFINITY;
    l_run[h] = 0.f;
  }
  int* flag = a.restart_flag + blockIdx.x;
  if (threadIdx.x == 0) __atomic_store_n(flag, 0, __ATOMIC_RELAXED);

  const int tok_begin = p0 * kPage;
  const int tok_end = min(p1 * kPage, len);
  const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;
  const int jm = (tmax_min - tok_begin + 1) / kChunk;
  const char* cache = reinterpret_cast<const char*>(a.cache);
  uint32_t doff[kF8Per];
  dma_offsets_f8(wave, lane, doff);
  auto chunk_copy = [&](auto slot_c, int j) -> ChunkCopy {
    const bool real = j < nchunks;
    const int lp = real ? (j >> 1) : 0;
    int64_t blk;
    if (bt_regs) {
      int bb = __builtin_amdgcn_readlane(btv[0], lp & 63);
#pragma unroll
      for (int k = 1; k < kBtRegs; ++k) {
        const int bk = __builtin_amdgcn_readlane(btv[k], lp & 63);
        bb = (lp >> 6) == k ? bk : bb;
      }
      blk = bb;
    } else {
      int bb = bt[p0 + lp];
      asm volatile("" : "+s"(bb));
      blk = bb;
    }
    const int t = tok_begin + lp * kPage + (real ? (j & 1) * kChunk : 0);
    const int bytes = real ? min(tok_end - t, kChunk) * kFp8EntryBytes : 0;
    const char* src = cache + (blk * kPage + (t % kPage)) * (int64_t)kFp8EntryBytes;
    return ChunkCopy{
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), (short)0, bytes, kRsrcWord3),
        ring(slot_c)};
  };
  auto issue_all = [&](const ChunkCopy& cc) {
    static_for<0, kF8Per>([&](auto i_c) __attribute__((always_inline)) {
      copy_piece_f8<decltype(i_c)::value>(cc, doff, wave);
    });
  };
  auto chunk_limits = [&](int j, int (&lim)[NH]) {
    const int t0 = tok_begin + j * kChunk;
#pragma unroll
    for (int h = 0; h < NH; ++h) lim[h] = tmax[h] - t0 - 8 * gq;
  };
  bool need_restart = false;
  bf16x8 pk[NH];
  u32x2_t vpre[f8_pre(FT)];

  issue_all(chunk_copy(Slot<0>{}, 0));
  issue_all(chunk_copy(Slot<1>{}, 1));
  issue_all(chunk_copy(Slot<2>{}, 2));
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<2 * kF8Per>());
  ring_barrier();
  {
    f32x4 sacc[NH][2];
    float scl[8];
    int lim[NH];
    chunk_limits(0, lim);
    score_only_f8<NH>(ring(Slot<0>{}), ln, fq, e_one, e_lo, sacc, scl);
    mfma_drain<NH>(sacc);
    softmax_chunk_f8<NH, true>(sacc, pk, m_ref, l_run, lim, scl);
  }
  if (1 < nchunks) f8_prefetch<FT>(vpre, ring(Slot<0>{}), ln);
  auto interval = [&](auto s_c, int j) __attribute__((always_inline)) {
    constexpr int S = decltype(s_c)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm<kF8Per>());
    asm volatile("s_barrier" ::: "memory");
    const ChunkCopy cc = chunk_copy(Slot<S + 3>{}, j + 3);
    if (j + 1 < nchunks) {
      f32x4 sacc[NH][2];
      float scl[8];
      bf16x8 pk_next[NH];
      float psum[NH];
      int lim[NH];
      chunk_limits(j + 1, lim);
      fused_interval_f8<NH, FT, kGuard>(
          ring(Slot<S>{}), pk, oacc, ring(Slot<S + 1>{}), ln, fq, e_one, e_lo, sacc, scl, cc, doff,
          wave, vpre, [&](auto u_c) __attribute__((always_inline)) {
            constexpr int k = decltype(u_c)::value - f8_mid<NH, FT>();
            if constexpr (k == 0) mfma_drain<NH>(sacc);
            if constexpr (k >= 1 && k <= 2 * NH)
              softmax_piece_f8<NH, (k - 1) / 2, (k - 1) % 2>(sacc, pk_next, m_ref, psum, lim, scl);
            if constexpr (k == 2 * NH + 1) {
#pragma unroll
              for (int h = 0; h < NH; ++h) {
                l_run[h] += psum[h];
                need_restart |= !(psum[h] <= kSlackPow);
              }
            }
          });
#pragma unroll
      for (int h = 0; h < NH; ++h) pk[h] = pk_next[h];
      if (j + 2 < nchunks) f8_prefetch<FT>(vpre, ring(Slot<S + 1>{}), ln);
    } else if (j < nchunks) {
      issue_all(cc);
      pv_only_f8<NH, FT>(ring(Slot<S>{}), ln, pk, oacc);
    } else {
      issue_all(cc);
    }
  };
  for (int j = 0; j < nchunks; j += 4) {
    interval(Slot<0>{}, j);
    interval(Slot<1>{}, j + 1);
    interval(Slot<2>{}, j + 2);
    interval(Slot<3>{}, j + 3);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(need_restart) != 0 && lane == 0)
    __atomic_store_n(flag, 1, __ATOMIC_RELAXED);
  __syncthreads();
  const bool restart = __atomic_load_n(flag, __ATOMIC_RELAXED) != 0;

  // ---- restart (rare): exact row max, then a pass with it as the reference --
  if (restart) {
    auto fetch = [&](int j) -> const MLA_LDS char* {
      issue_all(chunk_copy(Slot<0>{}, j));
      __builtin_amdgcn_s_waitcnt(vmcnt_imm<0>());
      __syncthreads();
      return ring(Slot<0>{});
    };
    float m_exact[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) m_exact[h] = -INFINITY;
    for (int j = 0; j < nchunks; ++j) {
      const MLA_LDS char* buf = fetch(j);
      int lim[NH];
      chunk_limits(j, lim);
      f32x4 sacc[NH][2];
      float scl[8];
      score_only_f8<NH>(buf, ln, fq, e_one, e_lo, sacc, scl);
      mfma_drain<NH>(sacc);
      max_chunk_f8<NH>(sacc, m_exact, lim);
      __syncthreads();
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      m_ref[h] = m_exact[h];
      l_run[h] = 0.f;
    }
    // (zeroed without reading the old tiles: see decode_pipe_kernel)
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int f = 0; f < FT; ++f) oacc[h][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < nchunks; ++j) {
      const MLA_LDS char* buf = fetch(j);
      int lim[NH];
      chunk_limits(j, lim);
      f32x4 sacc[NH][2];
      float scl[8];
      score_only_f8<NH>(buf, ln, fq, e_one, e_lo, sacc, scl);
      mfma_drain<NH>(sacc);
      softmax_chunk_f8<NH, false>(sacc, pk, m_ref, l_run, lim, scl);
      pin_pk<NH>(pk);
      pv_only_f8<NH, FT>(buf, ln, pk, oacc);
      __syncthreads();
    }
  }
  mfma_drain_o<NH, FT>(oacc);

  // ---- finalise (as decode_pipe_kernel): the rows leave through LDS as
  // whole 1 KB rows; 16 staged rows per 21 KB ring slot
  static_assert(16 * kStageStride <= kF8SlotBytes && kRowsWg <= 16 * NS, "staged rows fit the ring");
  auto out_slot = [&](int r16) -> MLA_LDS char* {
    return r16 == 0 ? ring(Slot<0>{})
                    : r16 == 1 ? ring(Slot<1>{}) : r16 == 2 ? ring(Slot<2>{}) : ring(Slot<3>{});
  };
  const int wrow0 = (wave / FS) * 16 * NH;
  int lane_f = threadIdx.x & 63;
  asm volatile("" : "+v"(lane_f));
  const int n_f = lane_f & 15;
  const int gq_f = lane_f >> 4;
  float inv[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float l = l_run[h];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float lse = l > 0.f ? m_ref[h] + __builtin_amdgcn_logf(l) : -INFINITY;
    if (gq_f == 0 && fslice == 0)
      a.lse_part[(int64_t)item * a.rows_per_seq + row0 + 16 * h + n_f] = lse;
    inv[h] = l > 0.f ? 1.f / l : 0.f;
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int r = wrow0 + 16 * h;
    MLA_LDS char* dst =
        out_slot(r >> 4) + n_f * kStageStride + 32 * FT * fslice + 8 * (gq_f ^ stage_swap(n_f));
#pragma unroll
    for (int f = 0; f < FT; ++f) {
      *reinterpret_cast<MLA_LDS u16x4*>(dst + 32 * f) = scaled_bf16x4(oacc[h][f], inv[h]);
      asm volatile("" : : : "memory");
    }
  }
  __syncthreads();
  uint16_t* orows = a.o_part + ((int64_t)item * a.rows_per_seq + rg * kRowsWg) * kLatent;
#pragma unroll 8
  for (int r = wave; r < kRowsWg; r += 4) {
    const u16x8 v = stage_read(out_slot(r >> 4), r & 15, lane_f);
    *reinterpret_cast<u16x8*>(orows + (int64_t)r * kLatent + 8 * lane_f) = v;
  }
}

DecodeConfig decode_config(int rows_per_seq) {
  const int groups = rows_per_seq / 16;
  DecodeConfig c;
  c.chunk = kChunk;
  c.nbuf = 4;
  // rows per workgroup 128, 64, 32 or 16: the pipelined kernel with four
  // wavefronts of their own rows (feature split 1), or pairs / quartets of
  // wavefronts sharing rows (split 2 / 4); the FP8 cache at 128 rows takes the
  // eight-wavefront kernel.  16 * waves * heads_per_wave is the row count the
  // launch and the split planner work with.
  if (groups % 8 == 0) {
    c.waves = 4;
    c.heads_per_wave = 2;
    c.pipe = 1;
  } else if (groups % 4 == 0) {
    c.waves = 2;
    c.heads_per_wave = 2;
    c.pipe = 2;
  } else if (groups % 2 == 0) {
    c.waves = 1;
    c.heads_per_wave = 2;
    c.pipe = 3;
  } else {
    c.waves = 1;
    c.heads_per_wave = 1;
    c.pipe = 4;
  }
  if (c.waves == 1) c.nbuf = 3;
  c.lds_bytes = c.nbuf * kBufBytes + c.waves * c.heads_per_wave * (1024 + 64);
  c.wgs_per_cu = 1;  // the ring fills the LDS
  return c;
}

hipError_t launch_decode(const DecodeConfig& cfg, bool fp8, const uint16_t* q_abs, const void* cache,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int heads, int q_len, PlanView plan, int max_items,
                         uint16_t* o_part, float* lse_part,
                         int* restart_flags, hipStream_t stream,
                         const int32_t* slots, int slot_stride, uint32_t cache_bytes) {
  DecodeArgs args;
  args.slots = slots;
  args.slot_stride = slot_stride;
  args.cache_bytes = cache_bytes;
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
  if (slots) {
    if (fp8 || cfg.pipe != 1 || cache_bytes > kSlotMaxCacheBytes) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_pipe_kernel<2, 1, true>), dim3(grid), dim3(256), 0, stream, args,
                       block_table);
    return hipGetLastError();
  }
  if (fp8) {
    // 128 rows per workgroup: the eight-wavefront kernel (expansion to bf16
    // in LDS); fewer rows: the pipelined kernel over the FP8 rows
    switch (cfg.pipe) {
      case 1:
        hipLaunchKernelGGL((decode_kernel<8, 1, true>), dim3(grid), dim3(512), 0, stream, args,
                           block_table);
        break;
      case 2:
        hipLaunchKernelGGL((decode_pipe_f8_kernel<2, 2>), dim3(grid), dim3(256), 0, stream, args,
                           block_table);
        break;
      case 3:
        hipLaunchKernelGGL((decode_pipe_f8_kernel<2, 4>), dim3(grid), dim3(256), 0, stream, args,
                           block_table);
        break;
      default:
        hipLaunchKernelGGL((decode_pipe_f8_kernel<1, 4>), dim3(grid), dim3(256), 0, stream, args,
                           block_table);
        break;
    }
    return hipGetLastError();
  }
  switch (cfg.pipe) {
    case 1:
      hipLaunchKernelGGL((decode_pipe_kernel<2, 1>), dim3(grid), dim3(256), 0, stream, args,
                         block_table);
      break;
    case 2:
      hipLaunchKernelGGL((decode_pipe_kernel<2, 2>), dim3(grid), dim3(256), 0, stream, args,
                         block_table);
      break;
    case 3:
      hipLaunchKernelGGL((decode_pipe_kernel<2, 4>), dim3(grid), dim3(256), 0, stream, args,
                         block_table);
      break;
    default:
      hipLaunchKernelGGL((decode_pipe_kernel<1, 4>), dim3(grid), dim3(256), 0, stream, args,
                         block_table);
      break;
  }
  return hipGetLastError();
}

int decode_slot_cap() { return kSlotCap; }
uint32_t decode_slot_cache_limit() { return kSlotMaxCacheBytes; }

}  // namespace mla
