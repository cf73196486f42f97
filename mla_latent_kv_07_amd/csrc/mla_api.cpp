// libmla C ABI: argument validation, workspace layout and kernel sequencing.
// See include/mla.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "insert_dev.h"
#include "mla.h"
#include "mla_common.h"

namespace {

using namespace mla;

constexpr int kMaxQLen = 8;
constexpr int kMaxHint = 64;
constexpr int kMaxBatch = 1 << 16;
constexpr int kMaxSeqLen = 1 << 24;
constexpr int kMaxDevices = 64;
constexpr int kMaxInsert = 1 << 16;  // new tokens per sequence in one insert

int device_cus() {
  static std::once_flag once[kMaxDevices];
  static int cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(once[dev], [dev] {
    hipDeviceProp_t p;
    cus[dev] = (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0)
                   ? p.multiProcessorCount
                   : 256;
  });
  return cus[dev];
}

int check_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_NULL;
  if (d->kv_lora != kLatent || d->rope != kRope || d->qk_nope != kNope || d->v_dim != kVdim ||
      d->page != kPage)
    return MLA_ERR_UNSUPPORTED;
  if (d->heads < 16 || d->heads > 128 || d->heads % 16 != 0) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- debug checks of the device-side contract -------------------------------
// With MLA_DEBUG_CHECKS=1 in the environment (read once) or after
// mla_debug_checks(1), every entry point that takes a block table first
// copies the block table and the sequence lengths to the host (a synchronising
// copy on the call's stream) and checks them; a violation returns
// MLA_ERR_BOUNDS and nothing is enqueued.
std::atomic<int> g_debug{-1};

bool debug_checks() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("MLA_DEBUG_CHECKS");
    v = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    if (!g_debug.compare_exchange_strong(expected, v)) v = expected;
  }
  return v > 0;
}

// seq_lens[b] must lie in [lo, hi] and the block ids of the first
// ceil(seq_lens[b] / 64) logical blocks of sequence b (from logical block
// `first_page(len)` on) in [0, num_blocks).  Returns MLA_OK, MLA_ERR_BOUNDS, or
// MLA_ERR_HIP when the copies fail.
template <class FirstPage>
int check_tables(const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                 int32_t batch, int64_t lo, int64_t hi, int32_t num_blocks, hipStream_t s,
                 FirstPage first_page) {
  std::vector<int32_t> sl((size_t)batch), bt((size_t)batch * bt_stride);
  if (hipMemcpyAsync(sl.data(), seq_lens, sl.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MLA_ERR_HIP;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = sl[b];
    if (len < lo || len > hi) return MLA_ERR_BOUNDS;
    const int64_t pages = (len + kPage - 1) / kPage;
    if (pages > bt_stride) return MLA_ERR_BOUNDS;
    for (int64_t p = first_page(len); p < pages; ++p) {
      const int32_t blk = bt[(size_t)b * bt_stride + p];
      if (blk < 0 || blk >= num_blocks) return MLA_ERR_BOUNDS;
    }
  }
  return MLA_OK;
}

// every page of the sequence
int check_all_pages(const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                    int32_t batch, int64_t lo, int64_t hi, int32_t num_blocks, hipStream_t s) {
  return check_tables(block_table, bt_stride, seq_lens, batch, lo, hi, num_blocks, s,
                      [](int64_t) { return (int64_t)0; });
}

struct Layout {
  int max_items = 0;
  int slots = 0;
  DecodeConfig cfg{};
  size_t off_header = 0, off_item_b = 0, off_item_p0 = 0, off_item_p1 = 0, off_seq_start = 0,
         off_seq_count = 0, off_flags = 0, off_qabs = 0, off_opart = 0, off_lse = 0,
         total = 0;
};

// Workspace layout for one decode call (pure function of the sizes).
// item_cap > 0 bounds the number of work items the planner may choose (the
// no-allocation entry point sizes it to its scratch).
Layout make_layout(int heads, int batch, int q_len, int hint, int item_cap = 0) {
  Layout L;
  const int rows = heads * q_len;
  L.cfg = decode_config(rows);
  const int row_groups = rows / (16 * L.cfg.waves * L.cfg.heads_per_wave);
  L.slots = device_cus() * L.cfg.wgs_per_cu / row_groups;
  if (L.slots < 1) L.slots = 1;
  L.max_items = hint > 0 ? batch * hint : batch + 4 * L.slots;
  if (item_cap > 0 && item_cap < L.max_items) L.max_items = item_cap;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.off_header = take(64);
  L.off_item_b = take(4 * (size_t)L.max_items);
  L.off_item_p0 = take(4 * (size_t)L.max_items);
  L.off_item_p1 = take(4 * (size_t)L.max_items);
  L.off_seq_start = take(4 * (size_t)batch);
  L.off_seq_count = take(4 * (size_t)batch);
  L.off_flags = take(4 * ((size_t)L.max_items + 8) * row_groups);
  L.off_qabs = take((size_t)batch * rows * kEntry * 2);
  L.off_opart = take((size_t)L.max_items * rows * kLatent * 2);
  L.off_lse = take((size_t)L.max_items * rows * 4);
  L.total = off;
  return L;
}

// Benchmark stage timing (mla_profile_enable / mla_profile_collect).
struct Profile {
  std::vector<hipEvent_t> ev;  // kMarks per call
  int max_calls = 0;
  int used = 0;
};
Profile g_prof;
constexpr int kStages = 3;  // prep, decode, combine
constexpr int kMarks = kStages + 1;

void prof_mark(int call, int k, hipStream_t s) {
  if (call >= 0) hipEventRecord(g_prof.ev[call * kMarks + k], s);
}

}  // namespace

// The top-k launch (dsa.hip); slots != nullptr: also each kept position's
// cache row index (block * 64 + slot, through block_table) at
// slots[b * slot_stride + rank], for the decode that reads the kept rows in
// place.
namespace mla {
hipError_t launch_topk(const float* scores, int lpad, const int32_t* seq_lens, int max_seq_len,
                       int batch, int top_k, int32_t* kept, int32_t* counts, hipStream_t stream,
                       const int32_t* block_table, int bt_stride, int32_t* slots,
                       int slot_stride);
}  // namespace mla

extern "C" {

int mla_profile_enable(int32_t max_calls) {
  for (hipEvent_t e : g_prof.ev) hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.max_calls = 0;
  g_prof.used = 0;
  if (max_calls <= 0) return MLA_OK;
  if (max_calls > 100000) return MLA_ERR_SHAPE;
  g_prof.ev.resize((size_t)max_calls * kMarks);
  // timing-only events: no system-scope fence when recorded (a fence would
  // write back and invalidate the caches at every stage boundary, which adds
  // its own time to the stage and slows the next one)
  for (auto& e : g_prof.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return MLA_ERR_HIP;
  g_prof.max_calls = max_calls;
  return MLA_OK;
}

int mla_profile_collect(double* stage_ms, int32_t* calls) {
  if (!stage_ms || !calls) return MLA_ERR_NULL;
  for (int k = 0; k < kStages; ++k) stage_ms[k] = 0.0;
  for (int c = 0; c < g_prof.used; ++c) {
    if (hipEventSynchronize(g_prof.ev[c * kMarks + kStages]) != hipSuccess) return MLA_ERR_HIP;
    for (int k = 0; k < kStages; ++k) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_prof.ev[c * kMarks + k], g_prof.ev[c * kMarks + k + 1]) !=
          hipSuccess)
        return MLA_ERR_HIP;
      stage_ms[k] += ms;
    }
  }
  *calls = g_prof.used;
  g_prof.used = 0;
  return MLA_OK;
}

int mla_profile_collect_calls(double* stage_ms, int32_t max_calls, int32_t* calls) {
  if (!stage_ms || !calls) return MLA_ERR_NULL;
  if (max_calls < g_prof.used) return MLA_ERR_SHAPE;
  for (int c = 0; c < g_prof.used; ++c) {
    if (hipEventSynchronize(g_prof.ev[c * kMarks + kStages]) != hipSuccess) return MLA_ERR_HIP;
    for (int k = 0; k < kStages; ++k) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, g_prof.ev[c * kMarks + k], g_prof.ev[c * kMarks + k + 1]) !=
          hipSuccess)
        return MLA_ERR_HIP;
      stage_ms[c * kStages + k] = ms;
    }
  }
  *calls = g_prof.used;
  g_prof.used = 0;
  return MLA_OK;
}

int mla_abi_version(void) { return 1; }

int mla_debug_checks(int32_t enable) {
  const int prev = debug_checks() ? 1 : 0;
  if (enable >= 0) g_debug.store(enable ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions (need kv_lora 512, rope 64, qk_nope 128, v_dim 128, page 64, heads 16..128 in steps of 16)";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime error at kernel launch";
    case MLA_ERR_BOUNDS: return "block table or sequence lengths break the contract (debug checks)";
    case MLA_ERR_SCRATCH: return "the call needs more than the no-allocation scratch (mla_noalloc_scratch_bytes)";
    default: return "unknown status";
  }
}

namespace {

// The two cache formats share the argument checks of each entry point.
int cache_insert_any(bool fp8, const mla_dims* dims, const void* kv_a, const void* rms_w,
                     float eps, float rope_base, const int32_t* block_table, int32_t bt_stride,
                     const int32_t* seq_lens, int32_t batch, int32_t q_len, void* cache,
                     int32_t num_blocks, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || q_len < 1 || q_len > kMaxInsert || bt_stride < 1 ||
      num_blocks < 1 || (int64_t)batch * q_len > (int64_t)INT32_MAX)
    return MLA_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(rope_base) || rope_base <= 0.f)
    return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!kv_a || !rms_w || !block_table || !seq_lens || !cache) return MLA_ERR_NULL;
  if (debug_checks()) {
    // the pages that receive the new tokens
    st = check_tables(block_table, bt_stride, seq_lens, batch, q_len, (int64_t)bt_stride * kPage,
                      num_blocks, static_cast<hipStream_t>(stream),
                      [q_len](int64_t len) { return (len - q_len) / kPage; });
    if (st != MLA_OK) return st;
  }
  hipError_t e =
      fp8 ? launch_insert_fp8(static_cast<const uint16_t*>(kv_a),
                              static_cast<const uint16_t*>(rms_w), eps, rope_base, block_table,
                              bt_stride, seq_lens, batch, q_len, static_cast<uint8_t*>(cache),
                              static_cast<hipStream_t>(stream))
          : launch_insert(static_cast<const uint16_t*>(kv_a),
                          static_cast<const uint16_t*>(rms_w), eps, rope_base, block_table,
                          bt_stride, seq_lens, batch, q_len, static_cast<uint16_t*>(cache),
                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

int mla_cache_insert(const mla_dims* dims, const void* kv_a, const void* rms_w, float eps,
                     float rope_base, const int32_t* block_table, int32_t bt_stride,
                     const int32_t* seq_lens, int32_t batch, int32_t q_len, void* cache,
                     int32_t num_blocks, void* stream) {
  return cache_insert_any(false, dims, kv_a, rms_w, eps, rope_base, block_table, bt_stride,
                          seq_lens, batch, q_len, cache, num_blocks, stream);
}

int mla_cache_insert_fp8(const mla_dims* dims, const void* kv_a, const void* rms_w, float eps,
                         float rope_base, const int32_t* block_table, int32_t bt_stride,
                         const int32_t* seq_lens, int32_t batch, int32_t q_len, void* cache,
                         int32_t num_blocks, void* stream) {
  return cache_insert_any(true, dims, kv_a, rms_w, eps, rope_base, block_table, bt_stride,
                          seq_lens, batch, q_len, cache, num_blocks, stream);
}

size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t q_len,
                                  int32_t max_seq_len, int32_t num_splits_hint) {
  if (check_dims(dims) != MLA_OK) return 0;
  if (batch < 0 || batch > kMaxBatch || q_len < 1 || q_len > kMaxQLen || max_seq_len < q_len ||
      max_seq_len > kMaxSeqLen || num_splits_hint < 0 || num_splits_hint > kMaxHint)
    return 0;
  return make_layout(dims->heads, batch, q_len, num_splits_hint).total;
}


namespace {

// ins != nullptr: the fused step (insert of the new tokens and RoPE on q_pe
// in the query-preparation launch); ins->cache is `cache`.
int decode_any(bool fp8, const InsertArgs* ins, const mla_dims* dims, const void* q,
               const void* kv_b, const void* cache, int32_t num_blocks,
               const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
               int32_t batch, int32_t q_len, int32_t max_seq_len, float softmax_scale, void* out,
               void* workspace, size_t workspace_bytes, int32_t num_splits_hint, void* stream,
               int item_cap = 0, const int32_t* slots = nullptr) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || q_len < 1 || q_len > kMaxQLen || max_seq_len < q_len ||
      max_seq_len > kMaxSeqLen || num_blocks < 1 || num_splits_hint < 0 ||
      num_splits_hint > kMaxHint)
    return MLA_ERR_SHAPE;
  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  if (bt_stride < max_pages) return MLA_ERR_SHAPE;
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q || !kv_b || !cache || !block_table || !seq_lens || !out) return MLA_ERR_NULL;
  if (!workspace) return MLA_ERR_WORKSPACE;
  const int heads = dims->heads;
  const Layout L = make_layout(heads, batch, q_len, num_splits_hint, item_cap);
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  // (rows in place: the slot list comes from a checked block table)
  if (debug_checks() && !slots) {
    st = check_all_pages(block_table, bt_stride, seq_lens, batch, q_len, max_seq_len, num_blocks,
                         static_cast<hipStream_t>(stream));
    if (st != MLA_OK) return st;
  }

  char* ws = static_cast<char*>(workspace);
  PlanView plan;
  plan.header = reinterpret_cast<int32_t*>(ws + L.off_header);
  plan.item_b = reinterpret_cast<int32_t*>(ws + L.off_item_b);
  plan.item_p0 = reinterpret_cast<int32_t*>(ws + L.off_item_p0);
  plan.item_p1 = reinterpret_cast<int32_t*>(ws + L.off_item_p1);
  plan.seq_start = reinterpret_cast<int32_t*>(ws + L.off_seq_start);
  plan.seq_count = reinterpret_cast<int32_t*>(ws + L.off_seq_count);
  uint16_t* q_abs = reinterpret_cast<uint16_t*>(ws + L.off_qabs);
  uint16_t* o_part = reinterpret_cast<uint16_t*>(ws + L.off_opart);
  float* lse_part = reinterpret_cast<float*>(ws + L.off_lse);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rows = heads * q_len;
  // price of one item's fixed work in cache pages: its set-up (query rows,
  // plan entries: about four pages' time) plus its partial rows (bf16 write
  // + read)
  const float item_cost = 4.0f + (float)rows * kLatent * 2 * 2 / (float)kPageBytes;

  const int pc = g_prof.used < g_prof.max_calls ? g_prof.used++ : -1;
  prof_mark(pc, 0, s);
  // the absorbed query carries softmax_scale * log2(e): scores come out of the
  // matrix cores in log2 units
  const float q_scale = softmax_scale * 1.4426950408889634f;
  hipError_t e =
      ins ? launch_prep_step(fp8, *ins, static_cast<const uint16_t*>(q),
                             static_cast<const uint16_t*>(kv_b), heads, batch * q_len, q_scale,
                             q_abs, seq_lens, batch, max_pages, L.slots, L.max_items,
                             num_splits_hint, item_cost, plan, s)
          : launch_prep(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_b),
                        heads, batch * q_len, q_scale, q_abs, seq_lens, batch, max_pages,
                        L.slots, L.max_items, num_splits_hint, item_cost, plan, s);
  prof_mark(pc, 1, s);
  if (e == hipSuccess)
    e = launch_decode(L.cfg, fp8, q_abs, cache, block_table, bt_stride,
                      seq_lens, heads, q_len, plan,
                      L.max_items, o_part, lse_part,
                      reinterpret_cast<int*>(ws + L.off_flags), s, slots, bt_stride * kPage,
                      (uint32_t)((int64_t)num_blocks * kPageBytes));
  prof_mark(pc, 2, s);
  if (e == hipSuccess)
    e = launch_combine(o_part, lse_part, plan, static_cast<const uint16_t*>(kv_b), heads, q_len,
                       batch, static_cast<uint16_t*>(out), device_cus(), s);
  prof_mark(pc, 3, s);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

int mla_decode(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
               int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
               const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
               float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
               int32_t num_splits_hint, void* stream) {
  return decode_any(false, nullptr, dims, q, kv_b, cache, num_blocks, block_table, bt_stride,
                    seq_lens, batch, q_len, max_seq_len, softmax_scale, out, workspace,
                    workspace_bytes, num_splits_hint, stream);
}

int mla_decode_fp8(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                   int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
                   float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                   int32_t num_splits_hint, void* stream) {
  return decode_any(true, nullptr, dims, q, kv_b, cache, num_blocks, block_table, bt_stride,
                    seq_lens, batch, q_len, max_seq_len, softmax_scale, out, workspace,
                    workspace_bytes, num_splits_hint, stream);
}

size_t mla_noalloc_scratch_bytes(void) { return kScratchBytes; }

int mla_decode_noalloc(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t batch, int32_t q_len,
                       int32_t max_seq_len, float softmax_scale, void* out,
                       int32_t num_splits_hint, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || q_len < 1 || q_len > kMaxQLen || max_seq_len < q_len ||
      max_seq_len > kMaxSeqLen || num_splits_hint < 0 || num_splits_hint > kMaxHint)
    return MLA_ERR_SHAPE;
  if (batch == 0) return decode_any(false, nullptr, dims, q, kv_b, cache, num_blocks, block_table,
                                    bt_stride, seq_lens, batch, q_len, max_seq_len, softmax_scale,
                                    out, nullptr, 0, num_splits_hint, stream);
  // the workspace of mla_decode, with the item list capped so that it fits
  // the scratch: its size is linear in the item count
  const int heads = dims->heads;
  Layout L = make_layout(heads, batch, q_len, num_splits_hint);
  int cap = 0;
  if (L.total > kScratchBytes) {
    if (num_splits_hint > 0) return MLA_ERR_SCRATCH;  // the hint fixes the item count
    const Layout one = make_layout(heads, batch, q_len, 0, batch);
    const Layout two = make_layout(heads, batch, q_len, 0, batch + 1);
    if (one.total > kScratchBytes) return MLA_ERR_SCRATCH;
    const size_t per_item = two.total > one.total ? two.total - one.total : 1;
    cap = batch + (int)((kScratchBytes - one.total) / per_item);
    while (cap > batch && make_layout(heads, batch, q_len, 0, cap).total > kScratchBytes) --cap;
  }
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess || ws == nullptr) return MLA_ERR_HIP;
  return decode_any(false, nullptr, dims, q, kv_b, cache, num_blocks, block_table, bt_stride,
                    seq_lens, batch, q_len, max_seq_len, softmax_scale, out, ws, kScratchBytes,
                    num_splits_hint, stream, cap);
}

namespace {

int step_any(bool fp8, const mla_dims* dims, const void* q, const void* kv_a, const void* rms_w,
             float eps, float rope_base, const void* kv_b, void* cache, int32_t num_blocks,
             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
             int32_t batch, int32_t q_len, int32_t max_seq_len, float softmax_scale, void* out,
             void* workspace, size_t workspace_bytes, int32_t num_splits_hint, void* stream) {
  if (!std::isfinite(eps) || eps < 0.f || !std::isfinite(rope_base) || rope_base <= 0.f)
    return MLA_ERR_SHAPE;
  if (batch > 0 && (!kv_a || !rms_w)) return MLA_ERR_NULL;
  const InsertArgs ins = with_rope_freq(
      InsertArgs{static_cast<const uint16_t*>(kv_a), static_cast<const uint16_t*>(rms_w),
                 (double)eps, (double)rope_base, block_table, bt_stride, seq_lens, q_len, cache});
  return decode_any(fp8, &ins, dims, q, kv_b, cache, num_blocks, block_table, bt_stride,
                    seq_lens, batch, q_len, max_seq_len, softmax_scale, out, workspace,
                    workspace_bytes, num_splits_hint, stream);
}

}  // namespace

int mla_decode_step(const mla_dims* dims, const void* q, const void* kv_a, const void* rms_w,
                    float eps, float rope_base, const void* kv_b, void* cache, int32_t num_blocks,
                    const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                    int32_t batch, int32_t q_len, int32_t max_seq_len, float softmax_scale,
                    void* out, void* workspace, size_t workspace_bytes, int32_t num_splits_hint,
                    void* stream) {
  return step_any(false, dims, q, kv_a, rms_w, eps, rope_base, kv_b, cache, num_blocks,
                  block_table, bt_stride, seq_lens, batch, q_len, max_seq_len, softmax_scale, out,
                  workspace, workspace_bytes, num_splits_hint, stream);
}

int mla_decode_step_fp8(const mla_dims* dims, const void* q, const void* kv_a, const void* rms_w,
                        float eps, float rope_base, const void* kv_b, void* cache,
                        int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                        const int32_t* seq_lens, int32_t batch, int32_t q_len,
                        int32_t max_seq_len, float softmax_scale, void* out, void* workspace,
                        size_t workspace_bytes, int32_t num_splits_hint, void* stream) {
  return step_any(true, dims, q, kv_a, rms_w, eps, rope_base, kv_b, cache, num_blocks,
                  block_table, bt_stride, seq_lens, batch, q_len, max_seq_len, softmax_scale, out,
                  workspace, workspace_bytes, num_splits_hint, stream);
}

namespace {

// rows per (sequence, head) in the prefill workspace: max_seq_len rounded up
// to the 64-key block
int64_t prefill_lpad(int32_t max_seq_len) { return ((int64_t)max_seq_len + 63) / 64 * 64; }

}  // namespace

size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_seq_len) {
  if (check_dims(dims) != MLA_OK) return 0;
  if (batch < 0 || batch > kMaxBatch || max_seq_len < 1 || max_seq_len > kMaxSeqLen) return 0;
  return align256((size_t)batch * dims->heads * prefill_lpad(max_seq_len) * (kQk + kVdim) * 2) +
         256;
}

int mla_prefill(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
                float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxBatch || q_len < 1 || max_seq_len < q_len ||
      max_seq_len > kMaxSeqLen || num_blocks < 1)
    return MLA_ERR_SHAPE;
  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  if (bt_stride < max_pages) return MLA_ERR_SHAPE;
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  if (!q || !kv_b || !cache || !block_table || !seq_lens || !out) return MLA_ERR_NULL;
  const size_t need = mla_prefill_workspace_bytes(dims, batch, max_seq_len);
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (need == 0 || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (debug_checks()) {
    st = check_all_pages(block_table, bt_stride, seq_lens, batch, q_len, max_seq_len, num_blocks,
                         static_cast<hipStream_t>(stream));
    if (st != MLA_OK) return st;
  }
  const int heads = dims->heads;
  const int64_t lpad = prefill_lpad(max_seq_len);
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  uint16_t* kx = reinterpret_cast<uint16_t*>(ws);
  uint16_t* vx = kx + (size_t)batch * heads * lpad * kQk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int pc = g_prof.used < g_prof.max_calls ? g_prof.used++ : -1;
  prof_mark(pc, 0, s);
  hipError_t e = launch_prefill(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_b),
      static_cast<const uint16_t*>(cache), block_table, bt_stride, seq_lens, batch, heads, q_len,
      (int)lpad, softmax_scale * 1.4426950408889634f, kx, vx, static_cast<uint16_t*>(out), s,
      pc >= 0 ? g_prof.ev[pc * kMarks + 1] : nullptr);
  prof_mark(pc, 2, s);
  prof_mark(pc, 3, s);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

namespace {

constexpr int kMaxTopK = 1 << 16;
constexpr int kMaxIndexHeads = 1024;
constexpr int kMaxDsaBatch = 65535;  // the batch is a grid dimension of the selection launches

int64_t dsa_lpad(int32_t max_seq_len) { return ((int64_t)max_seq_len + 63) / 64 * 64; }
int dsa_kpages(int32_t max_seq_len, int32_t top_k) {
  const int ks = top_k < max_seq_len ? top_k : max_seq_len;
  return (ks + kPage - 1) / kPage;
}

struct DsaLayout {
  size_t off_scores = 0, off_kept = 0, off_counts = 0, off_dbt = 0, off_dense = 0, off_dec = 0,
         total = 0;
};

DsaLayout make_dsa_layout(int heads, int batch, int32_t max_seq_len, int32_t top_k, int hint) {
  DsaLayout L;
  const int kp = dsa_kpages(max_seq_len, top_k);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.off_scores = take((size_t)batch * dsa_lpad(max_seq_len) * 4);
  L.off_kept = take((size_t)batch * top_k * 4);
  L.off_counts = take((size_t)batch * 4);
  L.off_dbt = take((size_t)batch * kp * 4);
  L.off_dense = take((size_t)batch * kp * kPageBytes);
  L.off_dec = take(make_layout(heads, batch, 1, hint).total);
  L.total = off + 256;  // the workspace pointer is rounded up to 256 bytes
  return L;
}

int check_index(int32_t index_heads, const void* index_q, const float* index_w,
                const void* index_k, const float* index_k_scale, int32_t top_k) {
  if (index_heads < 1 || index_heads > kMaxIndexHeads || top_k < 1 || top_k > kMaxTopK)
    return MLA_ERR_SHAPE;
  if (!index_q || !index_w || !index_k || !index_k_scale) return MLA_ERR_NULL;
  return MLA_OK;
}

}  // namespace

int mla_dsa_select(int32_t index_heads, const void* index_q, const float* index_w,
                   const void* index_k, const float* index_k_scale, const int32_t* block_table,
                   int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                   int32_t max_seq_len, int32_t top_k, float* scores, int32_t scores_stride,
                   int32_t* indices, int32_t* counts, void* stream) {
  if (batch < 0 || batch > kMaxDsaBatch || max_seq_len < 1 || max_seq_len > kMaxSeqLen ||
      scores_stride < max_seq_len)
    return MLA_ERR_SHAPE;
  if (bt_stride < (max_seq_len + kPage - 1) / kPage) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  int st = check_index(index_heads, index_q, index_w, index_k, index_k_scale, top_k);
  if (st != MLA_OK) return st;
  if (!block_table || !seq_lens || !scores || !indices) return MLA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_checks()) {
    // (the index keys have no block count here: lengths and table width only)
    st = check_tables(block_table, bt_stride, seq_lens, batch, 1, max_seq_len, INT32_MAX, s,
                      [](int64_t) { return (int64_t)0; });
    if (st != MLA_OK) return st;
  }
  hipError_t e = launch_index_scores(static_cast<const uint8_t*>(index_q), index_w, index_heads,
                                     static_cast<const uint8_t*>(index_k), index_k_scale,
                                     block_table, bt_stride, seq_lens, batch, max_seq_len, scores,
                                     scores_stride, s);
  if (e == hipSuccess)
    e = launch_topk(scores, scores_stride, seq_lens, max_seq_len, batch, top_k, indices, counts, s,
                    nullptr, 0, nullptr, 0);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_dsa_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_seq_len,
                               int32_t top_k, int32_t num_splits_hint) {
  if (check_dims(dims) != MLA_OK) return 0;
  if (batch < 0 || batch > kMaxDsaBatch || max_seq_len < 1 || max_seq_len > kMaxSeqLen ||
      top_k < 1 || top_k > kMaxTopK || num_splits_hint < 0 || num_splits_hint > kMaxHint)
    return 0;
  return make_dsa_layout(dims->heads, batch, max_seq_len, top_k, num_splits_hint).total;
}

namespace {

// The two cache formats share the selection; the gather copies whole rows of
// either format and the decode reads them as it reads the paged cache.
int dsa_any(bool fp8, const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
            int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
            const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, int32_t index_heads,
            const void* index_q, const float* index_w, const void* index_k,
            const float* index_k_scale, int32_t top_k, float softmax_scale, void* out,
            int32_t* indices_out, void* workspace, size_t workspace_bytes,
            int32_t num_splits_hint, void* stream) {
  int st = check_dims(dims);
  if (st != MLA_OK) return st;
  if (batch < 0 || batch > kMaxDsaBatch || max_seq_len < 1 || max_seq_len > kMaxSeqLen ||
      num_blocks < 1 || num_splits_hint < 0 || num_splits_hint > kMaxHint)
    return MLA_ERR_SHAPE;
  if (bt_stride < (max_seq_len + kPage - 1) / kPage) return MLA_ERR_SHAPE;
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f) return MLA_ERR_SHAPE;
  if (batch == 0) return MLA_OK;
  st = check_index(index_heads, index_q, index_w, index_k, index_k_scale, top_k);
  if (st != MLA_OK) return st;
  if (!q || !kv_b || !cache || !block_table || !seq_lens || !out) return MLA_ERR_NULL;
  if (!workspace) return MLA_ERR_WORKSPACE;
  const DsaLayout L = make_dsa_layout(dims->heads, batch, max_seq_len, top_k, num_splits_hint);
  if (workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  if (debug_checks()) {
    st = check_all_pages(block_table, bt_stride, seq_lens, batch, 1, max_seq_len, num_blocks,
                         static_cast<hipStream_t>(stream));
    if (st != MLA_OK) return st;
  }
  char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~(uintptr_t)255);
  float* scores = reinterpret_cast<float*>(ws + L.off_scores);
  int32_t* kept = indices_out ? indices_out : reinterpret_cast<int32_t*>(ws + L.off_kept);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.off_counts);
  int32_t* dense_bt = reinterpret_cast<int32_t*>(ws + L.off_dbt);
  char* dense = ws + L.off_dense;  // bf16 or FP8 rows, 64 per page
  const int kp = dsa_kpages(max_seq_len, top_k);
  const int ks = top_k < max_seq_len ? top_k : max_seq_len;
  const int lpad = (int)dsa_lpad(max_seq_len);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // stage marks of the selection (index scores, top-k, gather); the decode
  // over the kept rows takes the next profile slot
  const int pc = g_prof.used < g_prof.max_calls ? g_prof.used++ : -1;
  prof_mark(pc, 0, s);
  hipError_t e = launch_index_scores(static_cast<const uint8_t*>(index_q), index_w, index_heads,
                                     static_cast<const uint8_t*>(index_k), index_k_scale,
                                     block_table, bt_stride, seq_lens, batch, max_seq_len, scores,
                                     lpad, s);
  prof_mark(pc, 1, s);
  // bf16 rows at 128 rows per workgroup are read in place (a slot list, no
  // copy, written by the top-k launch) when a work item's slot list fits the
  // decode kernel's LDS and the cache its 32-bit buffer offsets; otherwise
  // they are gathered into dense pages
  const bool in_place = !fp8 && decode_config(dims->heads).pipe == 1 &&
                        kp * kPage <= decode_slot_cap() &&
                        (int64_t)num_blocks * kPageBytes <= (int64_t)decode_slot_cache_limit();
  int32_t* slots = reinterpret_cast<int32_t*>(dense);  // batch x kp x 64 entries
  if (e == hipSuccess)
    e = launch_topk(scores, lpad, seq_lens, max_seq_len, batch, top_k, kept, counts, s,
                    in_place ? block_table : nullptr, bt_stride, in_place ? slots : nullptr,
                    kp * kPage);
  prof_mark(pc, 2, s);
  if (in_place) {
    // (the slot list came with the top-k launch)
    prof_mark(pc, 3, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
    return decode_any(false, nullptr, dims, q, kv_b, cache, num_blocks, slots, kp, counts, batch,
                      1, ks, softmax_scale, out, ws + L.off_dec,
                      make_layout(dims->heads, batch, 1, num_splits_hint).total, num_splits_hint,
                      stream, 0, slots);
  }
  if (e == hipSuccess)
    e = launch_gather(fp8, cache, block_table, bt_stride, kept, top_k, counts, batch, kp, dense,
                      dense_bt, s);
  prof_mark(pc, 3, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  return decode_any(fp8, nullptr, dims, q, kv_b, dense, batch * kp, dense_bt, kp, counts, batch,
                    1, ks, softmax_scale, out, ws + L.off_dec,
                    make_layout(dims->heads, batch, 1, num_splits_hint).total, num_splits_hint,
                    stream);
}

}  // namespace

int mla_dsa_decode(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                   int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                   int32_t index_heads, const void* index_q, const float* index_w,
                   const void* index_k, const float* index_k_scale, int32_t top_k,
                   float softmax_scale, void* out, int32_t* indices_out, void* workspace,
                   size_t workspace_bytes, int32_t num_splits_hint, void* stream) {
  return dsa_any(false, dims, q, kv_b, cache, num_blocks, block_table, bt_stride, seq_lens, batch,
                 max_seq_len, index_heads, index_q, index_w, index_k, index_k_scale, top_k,
                 softmax_scale, out, indices_out, workspace, workspace_bytes, num_splits_hint,
                 stream);
}

int mla_dsa_decode_fp8(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                       int32_t index_heads, const void* index_q, const float* index_w,
                       const void* index_k, const float* index_k_scale, int32_t top_k,
                       float softmax_scale, void* out, int32_t* indices_out, void* workspace,
                       size_t workspace_bytes, int32_t num_splits_hint, void* stream) {
  return dsa_any(true, dims, q, kv_b, cache, num_blocks, block_table, bt_stride, seq_lens, batch,
                 max_seq_len, index_heads, index_q, index_w, index_k, index_k_scale, top_k,
                 softmax_scale, out, indices_out, workspace, workspace_bytes, num_splits_hint,
                 stream);
}

}  // extern "C"
