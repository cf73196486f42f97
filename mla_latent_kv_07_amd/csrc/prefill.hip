// Prefill: MLA attention for many new tokens in the expanded multi-head form.
//
// "深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA, "(a) Naive实现":
// kv_b_proj applied to the cached latent gives every head its k_nope and v
// (the weight viewed as [H, 128 + 128, 512]); the key is k_nope followed by
// the shared k_pe; softmax(q k^T * scale) v.  The tag page's MLA excerpt and
// the vLLM DeepSeek-V4 notes name this form for prefill (many queries per
// sequence: the attention is compute-bound, and 192/128-wide heads cost less
// than the 576/512-wide absorbed ones); the decode path uses the absorbed
// form.  Both compute the same function; the causal rule is the decode rule,
// query i of a sequence of post-insert length L sees positions t <= L - S + i
// (S = q_len new tokens; "DeepSeek-V3.2-Exp unboxing", 初步研读, triu(1)).
//
// Two kernels:
//   expand_kernel       K = [c W_UK^T | k_pe], V = c W_UV^T for every head,
//                       into a workspace laid out for the attention kernel
//   prefill_attn_kernel causal attention of 256 query rows of one head over
//                       64-key blocks (online softmax), output bf16
//
// Workspace layout (bf16): Kx [B][H][Lpad][192], Vx [B][H][Lpad][128], rows
// t >= L hold zeros.  The 16-byte pieces of each row are permuted so that a
// straight copy of a 64-row block into LDS serves both matrix-core read
// patterns without bank conflicts (the gfx950 bank map: 64 four-byte banks; a
// 16-byte read serves the 16 lanes that agree in lane bit 5 and in the parity
// of lane bits 2..4; the 8-byte transposing read serves 32 consecutive
// lanes): piece p of K row t sits at (p & ~7) | ((p & 7) ^ (t & 6)), piece p
// of V row t at p ^ 2 (t & 7).
#include <type_traits>

#include "mla_common.h"

namespace mla {

constexpr int kKxRow = kQk * 2;    // 384 bytes per K row
constexpr int kVxRow = kVdim * 2;  // 256 bytes per V row
__device__ __forceinline__ int kx_piece(int p, int t) { return (p & ~7) | ((p & 7) ^ (t & 6)); }
__device__ __forceinline__ int vx_piece(int p, int t) { return p ^ ((t & 7) << 1); }

// Encoding of "s_waitcnt vmcnt(n)" (expcnt and lgkmcnt left unconstrained).
constexpr int pf_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kPfRsrcWord3 = 0x00020000;  // buffer descriptor word 3 (raw buffer)

// Workgroup barrier: this wavefront's LDS accesses completed, then s_barrier
// (no wait on the copies in flight; those are waited for explicitly).
__device__ __forceinline__ void pf_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kPfRsrcWord3);
}

// ============================================================================
// Expansion
// ============================================================================
// One workgroup per (sequence, span of 1024 positions, head): eight
// wavefronts, two per SIMD; wavefronts 0-3 make K (W_UK rows 32 w ..),
// 4-7 make V (W_UV rows 32 (w - 4) ..).  Each keeps its 32 weight rows (all
// 512 latent columns, 128 VGPRs) in registers as the MFMA A operand; the
// latent rows stream through LDS in chunks of 32 cache rows (36 KB, half a
// page) copied straight from the paged cache by buffer loads to LDS, three
// slots, two chunks in flight, with the decode kernel's row layout (1152-byte
// rows, pieces permuted by xswz) so the B-operand reads are conflict-free.
// D^T = W c^T leaves each lane 4 consecutive output columns of one position:
// 8-byte stores.  Wavefronts 0-3 also copy each row's k_pe into K's last 64
// columns.

constexpr int kXChunk = 32;
constexpr int kXChunkBytes = kXChunk * kEntryBytes;  // 36864
constexpr int kXWaves = 8;
constexpr int kXPer = (kXChunkBytes / 1024 + kXWaves - 1) / kXWaves;  // copies per wavefront: 5
constexpr int kXSlotBytes = kXPer * kXWaves * 1024;                   // 40 KB (4 KB padding)
constexpr int kXSpan = 1024;                                          // positions per workgroup

__device__ __forceinline__ int xswz(int r) { return (((r >> 1) & 3) << 1) ^ (((r >> 3) & 1) * 7); }

struct ExpandArgs {
  const uint16_t* cache;
  int bt_stride;
  const int32_t* seq_lens;
  const uint16_t* kv_b;
  int heads;
  int batch;
  int lpad;    // rows per (sequence, head) in Kx / Vx, a multiple of 64
  int n_span;  // spans of kXSpan positions per sequence
  uint16_t* kx;
  uint16_t* vx;
};

template <int S>
using XSlot = std::integral_constant<int, S>;

// (block_table: a restrict parameter of its own, so its entries come through
// scalar loads, which do not count against the copies in flight)
__global__ __launch_bounds__(kXWaves * 64) void expand_kernel(
    ExpandArgs a, const int32_t* __restrict__ block_table) {
  __shared__ __attribute__((aligned(1024))) char ring0[kXSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[kXSlotBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[kXSlotBytes];
  auto ring = [&](auto s) -> MLA_LDS char* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return (MLA_LDS char*)ring0;
    else if constexpr (S == 1) return (MLA_LDS char*)ring1;
    else return (MLA_LDS char*)ring2;
  };
  // block -> (head, sequence, span): each XCD (block id mod 8) takes a
  // contiguous range of the list (head-major: every XCD gets the same mix of
  // sequence lengths)
  const int total = a.heads * a.batch * a.n_span;
  const int per_xcd = (total + 7) >> 3;
  const int k = blockIdx.x >> 3;
  const int gidx = (blockIdx.x & 7) * per_xcd + k;
  if (k >= per_xcd || gidx >= total) return;
  const int h = gidx / (a.batch * a.n_span);
  const int rest = gidx - h * (a.batch * a.n_span);
  const int b = rest / a.n_span;
  const int span = rest - b * a.n_span;

  // (values the whole workgroup shares: kept scalar, so the copy descriptors
  // built from them need no per-lane loop)
  const int len = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
  const int t_begin = span * kXSpan;
  const int nchunks = (min(t_begin + kXSpan, a.lpad) - t_begin) / kXChunk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave >> 2;  // 0: K, 1: V
  const int wq = wave & 3;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int gq = lane >> 4;

  // weight rows of this wavefront: A operand of k-step ks, row tile mt
  const uint16_t* w = a.kv_b + ((int64_t)h * (kNope + kVdim) + part * kNope + 32 * wq) * kLatent;
  bf16x8 aw[kLatent / 32][2];
#pragma unroll
  for (int ks = 0; ks < kLatent / 32; ++ks)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      aw[ks][mt] = *reinterpret_cast<const bf16x8*>(w + (int64_t)(16 * mt + n) * kLatent +
                                                    32 * ks + 8 * gq);
  // copy offsets (the same for every chunk): copy k = 8 i + wave fills LDS
  // pieces 64 k + lane from piece (Q % 72) ^ xswz(row) of its row; copies
  // past the chunk's 36 read nothing and fill the slot's padding
  uint32_t doff[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int kc = kXWaves * i + wave;
    const int q = 64 * kc + lane;
    const int row = q / kChunk16;
    const int col = q - row * kChunk16;
    doff[i] = kc < kXChunkBytes / 1024 ? (uint32_t)(row * kEntryBytes + 16 * (col ^ xswz(row)))
                                       : 0x80000000u;
  }
  const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
  // chunk j (positions t_begin + 32 j ..): rows past the sequence end read
  // nothing and arrive as zeros; a chunk wholly past it (or past the span)
  // is an empty copy with the same instruction count
  auto issue = [&](auto s, int j) -> void {
    const int t = t_begin + j * kXChunk;
    const int valid =
        __builtin_amdgcn_readfirstlane((j < nchunks) ? min(max(len - t, 0), kXChunk) : 0);
    const uint16_t* src = a.cache;
    if (valid > 0) {
      const int blk = __builtin_amdgcn_readfirstlane(bt[t / kPage]);
      src = a.cache + ((int64_t)blk * kPage + (t % kPage)) * kEntry;
    }
    const __amdgpu_buffer_rsrc_t rs = pf_rsrc(src, valid * kEntryBytes);
#pragma unroll
    for (int i = 0; i < kXPer; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, ring(s) + (kXWaves * i + wave) * 1024, 16,
                                               doff[i], 0, 0, 2);
  };

  const int row_elems = part ? kVdim : kQk;
  uint16_t* dst_base = (part ? a.vx : a.kx) + ((int64_t)b * a.heads + h) * a.lpad * row_elems;
  const int xs = gq ^ xswz(n);
  const int sbase_even = n * kEntryBytes + 16 * xs;
  const int sbase_odd = n * kEntryBytes + 16 * (xs ^ 4) - 64;

  auto compute = [&](auto s, int j) -> void {
    const MLA_LDS char* buf = ring(s);
    f32x4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kLatent / 32; ++ks) {
      // row 16 tt + n, piece 4 ks + gq (the decode kernel's score read)
      bf16x8 bv[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        bv[tt] = *reinterpret_cast<const MLA_LDS bf16x8*>(buf + (ks & 1 ? sbase_odd : sbase_even) +
                                                          64 * ks + 16 * kEntryBytes * tt);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          acc[mt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[ks][mt], bv[tt], acc[mt][tt], 0,
                                                                0, 0);
    }
    // lane holds output columns 32 wq + 16 mt + 4 gq + i of position 16 tt + n
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = t_begin + j * kXChunk + 16 * tt + n;
      char* row = reinterpret_cast<char*>(dst_base + (int64_t)t * row_elems);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int d0 = 32 * wq + 16 * mt + 4 * gq;
        const int p = d0 >> 3;
        const int off = 16 * (part ? vx_piece(p, t) : kx_piece(p, t)) + 8 * ((d0 >> 2) & 1);
        u16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(acc[mt][tt][i]);
        *reinterpret_cast<u16x4*>(row + off) = v;
      }
    }
    if (part == 0) {
      // k_pe: chunk row r, rope piece c (LDS piece (64 + c) ^ xswz(r)) -> K piece 16 + c
      const int r = threadIdx.x >> 3;
      const int c = threadIdx.x & 7;
      const int t = t_begin + j * kXChunk + r;
      const u16x8 v = *reinterpret_cast<const MLA_LDS u16x8*>(buf + r * kEntryBytes +
                                                              16 * ((64 + c) ^ xswz(r)));
      *reinterpret_cast<u16x8*>(reinterpret_cast<char*>(dst_base + (int64_t)t * row_elems) +
                                16 * kx_piece(16 + c, t)) = v;
    }
  };
  // chunk j in slot j % 3; chunk j+2 goes into chunk j-1's slot once every
  // wavefront is past chunk j-1; chunk j has landed once at most chunk j+1's
  // copies are pending
  auto interval = [&](auto s, int j) __attribute__((always_inline)) -> void {
    constexpr int S = decltype(s)::value;
    __builtin_amdgcn_s_waitcnt(pf_vmcnt(kXPer));
    pf_barrier();
    issue(XSlot<(S + 2) % 3>{}, j + 2);
    if (j < nchunks) compute(s, j);
  };
  issue(XSlot<0>{}, 0);
  issue(XSlot<1>{}, 1);
  // the weight rows (loaded before the copies) have arrived once at most the
  // two chunks' copies are pending
  __builtin_amdgcn_s_waitcnt(pf_vmcnt(2 * kXPer));
  for (int j = 0; j < nchunks; j += 3) {
    interval(XSlot<0>{}, j);
    interval(XSlot<1>{}, j + 1);
    interval(XSlot<2>{}, j + 2);
  }
  __builtin_amdgcn_s_waitcnt(pf_vmcnt(0));
}

// ============================================================================
// Attention
// ============================================================================
// One workgroup per (256 query rows, head, sequence), the latest query rows
// (the most keys) first.  Eight wavefronts (two per SIMD, so one's softmax
// and LDS waits overlap the other's matrix work); wavefront w owns rows
// i0 + 32 w .. + 31 (2 tiles of 16): their queries stay in registers (48
// VGPRs) as the B operand of
// S^T = K Q^T (bf16 MFMA 16x16x32), which leaves each lane one row's scores
// in the B-operand layout of O^T = V^T P^T (the decode kernel's arrangement:
// P never leaves registers).  K and V blocks of 64 keys (24 + 16 KB) are
// copied into LDS by buffer loads to LDS, three stages, two blocks in flight
// while one is computed.  Workgroups of one (sequence, head) run on one XCD
// (its K and V stay in that XCD's L2).  Online softmax in log2 units with
// fp32 sums; a row's reference max is raised (a cross-lane max and a rescale
// of its output accumulators) only when a score exceeds it by more than 2^8.

constexpr int kPBlk = 64;
constexpr int kPRows = 256;
constexpr int kPWaves = 8;
constexpr int kPRt = kPRows / kPWaves / 16;  // 16-row tiles per wavefront: 2
constexpr int kKTile = kPBlk * kKxRow;  // 24576
constexpr int kVTile = kPBlk * kVxRow;  // 16384
constexpr int kPStage = kKTile + kVTile;

struct PrefillArgs {
  const uint16_t* kx;
  const uint16_t* vx;
  const uint16_t* q;       // [B, S, H, 192]
  uint16_t* out;           // [B, S, H, 128]
  const int32_t* seq_lens;
  int heads;
  int q_len;
  int lpad;
  int n_qblk;
  int batch;
  float scale_log2;        // softmax_scale * log2(e)
};

template <int S>
using PSlot = std::integral_constant<int, S>;
// a row's reference max is raised only when a score passes it by more than
// this (log2 units): probabilities stay <= 2^8
constexpr float kPRefSlack = 8.0f;
constexpr int kPCopies = kPStage / 1024 / kPWaves;  // copies per wavefront per block: 5

__global__ __launch_bounds__(kPWaves * 64) void prefill_attn_kernel(PrefillArgs a) {
  // three stages, each its own array: block kb in stage kb % 3, named at
  // compile time (the loop is unrolled by three), so the compiler sees that
  // the copies in flight never alias the stage being read
  __shared__ __attribute__((aligned(1024))) char st0[kPStage];
  __shared__ __attribute__((aligned(1024))) char st1[kPStage];
  __shared__ __attribute__((aligned(1024))) char st2[kPStage];
  auto stage = [&](auto s) -> MLA_LDS char* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return (MLA_LDS char*)st0;
    else if constexpr (S == 1) return (MLA_LDS char*)st1;
    else return (MLA_LDS char*)st2;
  };
  // block id -> (head, sequence, query block): each XCD (block id mod 8)
  // takes a contiguous range of the (head, sequence) list (head-major, so
  // every XCD gets the same mix of sequence lengths), all query blocks of
  // one pair in a row, the latest (most keys) first
  const int total = a.n_qblk * a.heads * a.batch;
  const int per_xcd = (total + 7) >> 3;
  const int local = blockIdx.x >> 3;
  const int gidx = (blockIdx.x & 7) * per_xcd + local;
  if (local >= per_xcd || gidx >= total) return;
  const int pair = gidx / a.n_qblk;
  const int qb = a.n_qblk - 1 - (gidx - pair * a.n_qblk);
  const int h = pair / a.batch;
  const int b = pair - h * a.batch;
  const int len = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);  // uniform: scalar
  const int P = len - a.q_len;  // cached positions before the new tokens
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int gq = lane >> 4;
  const int i0 = qb * kPRows;
  const int iw = i0 + 16 * kPRt * wave;  // first row of this wavefront

  // query rows (B operand): lane holds dims 32 ks + 8 gq .. of row iw + 16 rt + n
  bf16x8 qreg[kPRt][6];
#pragma unroll
  for (int rt = 0; rt < kPRt; ++rt) {
    const int i = min(iw + 16 * rt + n, a.q_len - 1);
    const uint16_t* qp = a.q + (((int64_t)b * a.q_len + i) * a.heads + h) * kQk + 8 * gq;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) qreg[rt][ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
  }

  // key blocks: the workgroup's last row sees keys <= P + that row
  const int max_blocks = a.lpad / kPBlk;
  auto blocks_for = [&](int last_row) {
    const int lim = P + last_row;
    return lim < 0 ? 0 : min(lim / kPBlk + 1, max_blocks);
  };
  const int nkb = blocks_for(min(i0 + kPRows - 1, a.q_len - 1));
  const int nkb_w = iw < a.q_len ? blocks_for(min(iw + 16 * kPRt - 1, a.q_len - 1)) : 0;

  const uint16_t* kbase = a.kx + ((int64_t)b * a.heads + h) * a.lpad * kQk;
  const uint16_t* vbase = a.vx + ((int64_t)b * a.heads + h) * a.lpad * kVdim;
  // block kb into a stage: wavefront w copies K pieces 3w .. 3w+2 and V
  // pieces 2w, 2w+1 (1 KB each); an empty copy past the last block
  auto issue = [&](auto s, int kb) -> void {
    const bool real = kb < nkb;
    const __amdgpu_buffer_rsrc_t rk =
        pf_rsrc(kbase + (int64_t)(real ? kb : 0) * kPBlk * kQk, real ? kKTile : 0);
    const __amdgpu_buffer_rsrc_t rv =
        pf_rsrc(vbase + (int64_t)(real ? kb : 0) * kPBlk * kVdim, real ? kVTile : 0);
    constexpr int kK = kKTile / 1024 / kPWaves;  // 3
    constexpr int kV = kVTile / 1024 / kPWaves;  // 2
#pragma unroll
    for (int i = 0; i < kK; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, stage(s) + (kK * wave + i) * 1024, 16,
                                               (kK * wave + i) * 1024 + 16 * lane, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kV; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, stage(s) + kKTile + (kV * wave + i) * 1024, 16,
                                               (kV * wave + i) * 1024 + 16 * lane, 0, 0, 0);
  };

  // per-lane LDS offsets: K (A operand of S^T): row 16 kt + n, piece 4 ks + gq
  // (the row's low bits are n's); V^T (transposing read): row 4 gq + r4 (+16,
  // +32 kk), pieces 2 dt + (qq >> 1), half qq & 1
  const int r4 = (lane & 15) >> 2;
  const int qq = lane & 3;
  const int vrow = 4 * gq + r4;
  // V^T read offsets of the 8 dim tiles for key rows vrow (+16, +32 kk add
  // constants: the piece permutation depends on the row's low 3 bits only).
  // Each is kept as one opaque value so that every read stays one variable
  // step from the stage array, which keeps the compiler aware of the array
  // it reads (and of which copies in flight it must wait for).
  int vofs[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    vofs[dt] = vrow * kVxRow + 16 * vx_piece(2 * dt + (qq >> 1), vrow) + 8 * (qq & 1);
    asm volatile("" : "+v"(vofs[dt]));
  }
  f32x4 o[8][kPRt];  // O^T tiles [dims dt][rows rt]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rt = 0; rt < kPRt; ++rt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[kPRt], l[kPRt];
#pragma unroll
  for (int rt = 0; rt < kPRt; ++rt) {
    m[rt] = -INFINITY;
    l[rt] = 0.f;
  }

  // One 64-key block in two halves of 32 keys (kk): S^T of the half, the
  // online softmax over it, then its P.V (the halves keep the score and
  // probability registers of only 32 keys live).
  auto compute = [&](auto s, int kb) __attribute__((always_inline)) -> void {
    const MLA_LDS char* K = stage(s);
    const MLA_LDS char* V = stage(s) + kKTile;
    // some key of the block lies beyond the limit of the wavefront's first row
    const bool mask = kPBlk * kb + kPBlk - 1 > P + iw;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      // ---- S^T = K Q^T: key tiles 2 kk, 2 kk + 1 x the row tiles
      f32x4 sc[2][kPRt];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int rt = 0; rt < kPRt; ++rt) sc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        bf16x8 ka[2];
        const int pz = kx_piece(4 * ks + gq, n);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          ka[u] = *reinterpret_cast<const MLA_LDS bf16x8*>(K + (32 * kk + 16 * u + n) * kKxRow +
                                                           16 * pz);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int rt = 0; rt < kPRt; ++rt)
            sc[u][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u], qreg[rt][ks], sc[u][rt], 0,
                                                                0, 0);
      }
      // ---- online softmax; lane: row iw + 16 rt + n, keys 32 kk + 16 u + 4 gq + j
      bf16x8 pb[kPRt];
#pragma unroll
      for (int rt = 0; rt < kPRt; ++rt) {
        // visible: 16 u + j <= lim
        const int lim = P + iw + 16 * rt + n - kPBlk * kb - 32 * kk - 4 * gq;
        float x[2][4];
        float lmax = -INFINITY;  // this lane's max over its 8 keys
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v = sc[u][rt][j] * a.scale_log2;
            if (mask && 16 * u + j > lim) v = -INFINITY;
            x[u][j] = v;
            lmax = fmaxf(lmax, v);
          }
        // The row's reference m[rt] is refreshed (row max across its 4 lanes,
        // accumulators rescaled) only when some score exceeds it by more than
        // 2^8; otherwise p = 2^(s - m) <= 2^8 (fp32 sums and bf16 products
        // keep their relative precision), and no cross-lane step is needed.
        if (__builtin_amdgcn_ballot_w64(lmax > m[rt] + kPRefSlack) != 0) {
          float mrow = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
          mrow = fmaxf(mrow, __shfl_xor(mrow, 32, 64));
          const float m_new = fmaxf(m[rt], mrow);
          const float alpha = m[rt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[rt] - m_new);
          l[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) o[dt][rt][j] *= alpha;
          m[rt] = m_new;
        }
        const float m_use = m[rt] == -INFINITY ? 0.f : m[rt];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = __builtin_amdgcn_exp2f(x[u][j] - m_use);
            psum += p;
            pb[rt][4 * u + j] = (__bf16)p;
          }
        l[rt] += psum;
      }
      // ---- O^T += V^T P^T over the 32 keys of the half
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const MLA_LDS char* vp = V + vofs[dt];
        const bf16x4 a0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(vp + 32 * kk * kVxRow));
        const bf16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (MLA_LDS bf16x4*)(vp + (32 * kk + 16) * kVxRow));
        const bf16x8 vb = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int rt = 0; rt < kPRt; ++rt)
          o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb[rt], o[dt][rt], 0, 0, 0);
      }
    }
  };
  // block kb in stage kb % 3: wait for its copies (block kb+1's may still be
  // in flight: every step issues one block's copies, an empty one past the
  // end, so that count is fixed), a barrier (every wavefront is past block
  // kb-1, whose stage takes block kb+2), issue block kb+2, compute block kb
  // (a wavefront whose rows see no key of it skips)
  auto step = [&](auto s, int kb) __attribute__((always_inline)) -> void {
    constexpr int S = decltype(s)::value;
    __builtin_amdgcn_s_waitcnt(pf_vmcnt(kPCopies));
    pf_barrier();
    issue(PSlot<(S + 2) % 3>{}, kb + 2);
    if (kb < nkb_w) compute(s, kb);
  };
  issue(PSlot<0>{}, 0);
  issue(PSlot<1>{}, 1);
  // the query rows (loaded before the copies) have arrived once at most the
  // two blocks' copies are pending
  __builtin_amdgcn_s_waitcnt(pf_vmcnt(2 * kPCopies));
  for (int kb = 0; kb < nkb; kb += 3) {
    step(PSlot<0>{}, kb);
    step(PSlot<1>{}, kb + 1);
    step(PSlot<2>{}, kb + 2);
  }
  __builtin_amdgcn_s_waitcnt(pf_vmcnt(0));

  // ---- normalise and store rows < q_len
#pragma unroll
  for (int rt = 0; rt < kPRt; ++rt) {
    float lt = l[rt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int i = iw + 16 * rt + n;
    if (i < a.q_len) {
      uint16_t* op = a.out + (((int64_t)b * a.q_len + i) * a.heads + h) * kVdim + 4 * gq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        u16x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = f32_to_bf16(o[dt][rt][j] * inv);
        *reinterpret_cast<u16x4*>(op + 16 * dt) = v;
      }
    }
  }
}

hipError_t launch_prefill(const uint16_t* q, const uint16_t* kv_b, const uint16_t* cache,
                          const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                          int batch, int heads, int q_len, int lpad, float scale_log2,
                          uint16_t* kx, uint16_t* vx, uint16_t* out, hipStream_t stream,
                          hipEvent_t mid) {
  ExpandArgs ea{cache, bt_stride, seq_lens, kv_b, heads, batch, lpad,
                (lpad + kXSpan - 1) / kXSpan, kx, vx};
  const int total = batch * ea.n_span * heads;
  hipLaunchKernelGGL(expand_kernel, dim3(8 * ((total + 7) / 8)), dim3(kXWaves * 64), 0, stream, ea,
                     block_table);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (mid) (void)hipEventRecord(mid, stream);
  PrefillArgs pa{kx, vx, q, out, seq_lens, heads, q_len, lpad, (q_len + kPRows - 1) / kPRows,
                 batch, scale_log2};
  const int blocks = pa.n_qblk * heads * batch;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(8 * ((blocks + 7) / 8)), dim3(kPWaves * 64), 0,
                     stream, pa);
  return hipGetLastError();
}

}  // namespace mla
