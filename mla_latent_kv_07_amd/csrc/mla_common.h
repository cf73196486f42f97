// Shared definitions of the gfx950 MLA kernels (device types, conversions,
// constants, launch-wrapper declarations).  Internal to libmla.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Fixed model dimensions (DeepSeek MLA: kv_lora_rank 512, qk_rope_head_dim 64,
// qk_nope_head_dim 128, v_head_dim 128) and the cache page of 64 tokens.
constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kEntry = kLatent + kRope;        // 576 numbers per cached token
constexpr int kEntryBytes = kEntry * 2;        // 1152 bytes in bf16
constexpr int kNope = 128;
constexpr int kVdim = 128;
constexpr int kQk = kNope + kRope;             // 192
constexpr int kPage = 64;
constexpr int kPageBytes = kPage * kEntryBytes;  // 73728
constexpr int kChunk16 = kEntryBytes / 16;     // 72 16-byte pieces per entry
// FP8 cache row: 512 E4M3 latent codes, the 64 rope values in bf16, one
// power-of-two scale byte (value 2^(byte - 127)), zero padding to 656 bytes.
constexpr int kFp8EntryBytes = 656;
constexpr int kFp8RopeOff = 512;
constexpr int kFp8ScaleOff = 640;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

#define MLA_LDS __attribute__((address_space(3)))

// ---- bf16 conversions (bit-level, round to nearest even) -------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  // NaN stays NaN (a select, not a branch: no exec-mask work per value)
  return (uint16_t)((u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : r);
}
// double -> bf16 with a single rounding: truncate to float, mark inexactness
// in the lowest bit (round-to-odd), then round the float to bf16.  Float keeps
// 16 more bits than bf16, so the odd bit cannot create a false tie.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  float f = __double2float_rz(d);
  uint32_t u = __float_as_uint(f);
  if ((double)f != d) u |= 1u;
  return f32_to_bf16(__uint_as_float(u));
}

// ---- split plan layout inside the workspace ---------------------------------
struct PlanView {
  int32_t* header;      // [0] = number of work items
  int32_t* item_b;      // [max_items] sequence of the item
  int32_t* item_p0;     // [max_items] first page (logical)
  int32_t* item_p1;     // [max_items] one past the last page
  int32_t* seq_start;   // [B] first item of each sequence
  int32_t* seq_count;   // [B] number of items of each sequence
};

// ---- launch wrappers (each returns hipGetLastError() of its launch) --------
hipError_t launch_insert(const uint16_t* kv_a, const uint16_t* rms_w, float eps, float rope_base,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int batch, int q_len, uint16_t* cache, hipStream_t stream);
hipError_t launch_insert_fp8(const uint16_t* kv_a, const uint16_t* rms_w, float eps,
                             float rope_base, const int32_t* block_table, int bt_stride,
                             const int32_t* seq_lens, int batch, int q_len, uint8_t* cache,
                             hipStream_t stream);

// query absorption and the split plan, in one launch
hipError_t launch_prep(const uint16_t* q, const uint16_t* kv_b, int heads, int rows,
                       float q_scale, uint16_t* q_abs, const int32_t* seq_lens, int batch,
                       int max_pages,
                       int slots, int max_items, int splits_hint, float item_cost_pages,
                       PlanView plan, hipStream_t stream);

// the fused step: the same, plus the insert of the new tokens (bf16 or FP8
// cache) and RoPE on q_pe (which arrives unrotated); qabsorb.hip
struct InsertArgs;
hipError_t launch_prep_step(bool fp8, const InsertArgs& ia, const uint16_t* q,
                            const uint16_t* kv_b, int heads, int rows, float q_scale,
                            uint16_t* q_abs, const int32_t* seq_lens, int batch, int max_pages,
                            int slots, int max_items, int splits_hint, float item_cost_pages,
                            PlanView plan, hipStream_t stream);

struct DecodeConfig {
  int waves;    // wavefronts per workgroup
  int heads_per_wave;  // 16-row groups per wavefront
  int chunk;    // tokens per LDS stage (32 or 64)
  int nbuf;     // LDS ring depth (chunks)
  int lds_bytes;
  int wgs_per_cu;
  int pipe = 0;  // pipelined kernel variant: 1..4 = 128, 64, 32, 16 rows per workgroup
};
DecodeConfig decode_config(int rows_per_seq);

// cache: bf16 rows [.., 64, 576], or FP8 rows [.., 64, 656] when fp8.
// slots != nullptr: rows in place (bf16, 128 rows per workgroup only): the
// positions of sequence b are cache rows slots[b * slot_stride + t] of a
// cache of cache_bytes bytes (below decode_slot_cache_limit()), the block
// table is not read, and an item spans at most decode_slot_cap() positions.
hipError_t launch_decode(const DecodeConfig& cfg, bool fp8, const uint16_t* q_abs, const void* cache,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int heads, int q_len, PlanView plan, int max_items,
                         uint16_t* o_part, float* lse_part,
                         int* restart_flags, hipStream_t stream,
                         const int32_t* slots = nullptr, int slot_stride = 0,
                         uint32_t cache_bytes = 0);
int decode_slot_cap();
uint32_t decode_slot_cache_limit();

// prefill in the expanded form (prefill.hip): expansion of K/V into kx/vx
// (bf16 [B][H][lpad][192] / [B][H][lpad][128]), then causal attention; `mid`
// (optional) is recorded between the two launches
hipError_t launch_prefill(const uint16_t* q, const uint16_t* kv_b, const uint16_t* cache,
                          const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                          int batch, int heads, int q_len, int lpad, float scale_log2,
                          uint16_t* kx, uint16_t* vx, uint16_t* out, hipStream_t stream,
                          hipEvent_t mid);

// sparse decode (dsa.hip): index scores [B][lpad] of the cached positions,
// top-k selection (kept positions ascending, -1 past the count; counts may be
// NULL) and the gather of the kept rows into kpages dense pages per sequence
// (bf16 or FP8 rows) with their identity block table [B][kpages]
hipError_t launch_index_scores(const uint8_t* index_q, const float* index_w, int index_heads,
                               const uint8_t* index_k, const float* index_k_scale,
                               const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                               int batch, int max_seq_len, float* scores, int lpad,
                               hipStream_t stream);
hipError_t launch_topk(const float* scores, int lpad, const int32_t* seq_lens, int max_seq_len,
                       int batch,
                       int top_k, int32_t* kept, int32_t* counts, hipStream_t stream);
hipError_t launch_gather(bool fp8, const void* cache, const int32_t* block_table, int bt_stride,
                         const int32_t* kept, int top_k, const int32_t* counts, int batch,
                         int kpages, void* dense, int32_t* dense_bt, hipStream_t stream);
// The kept rows' cache row indices (block * 64 + slot), for the decode that
// reads them in place: slots[b * kpages * 64 + j] for rank j < counts[b].
hipError_t launch_slots(const int32_t* block_table, int bt_stride, const int32_t* kept, int top_k,
                        const int32_t* counts, int batch, int kpages, int32_t* slots,
                        hipStream_t stream);

// The no-allocation entry point's device scratch (scratch.hip): its size and
// the address of the current device's copy.
constexpr size_t kScratchBytes = size_t(128) << 20;
hipError_t scratch_address(void** out);

// cus: compute units of the device (sizes the row blocks)
hipError_t launch_combine(const uint16_t* o_part, const float* lse_part, PlanView plan,
                          const uint16_t* kv_b, int heads, int q_len, int batch, uint16_t* out,
                          int cus, hipStream_t stream);

}  // namespace mla
