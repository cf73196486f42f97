/*
 * mla.h — C ABI of libmla: DeepSeek Multi-head Latent Attention (MLA) decode
 * over a paged latent KV cache, and the fused cache-insert step, for AMD
 * Instinct MI355X (gfx950).
 *
 * Operations follow these pages (titles and sections as the pages give them):
 *   [V3-src] "深度解读DeepSeek：源码解读 DeepSeek-V3", section "MLA": the
 *            listing of MLA.forward and its subsections "(a) Naive实现" and
 *            "(b) 优化实现" (absorbed form: q_nope is multiplied by the first
 *            qk_nope rows of each head's kv_b block, scores are taken against
 *            the normalised latent plus the rope part, the softmax weights sum
 *            the latent rows, and the result is multiplied by the last v_dim
 *            rows of each head's block).
 *   [V2L]    "DeepSeek-V2-Lite 模型结构详解", §四 RMSNorm (row rule, float32
 *            arithmetic) and §五 MLA (one 576-number cache entry per token:
 *            512 latent + 64 rope; the two absorption identities).
 *   [TAGS]   the "DeepSeek" tag page: excerpt on the 1/sqrt(d_k) scale, and
 *            excerpt on MLA under decode context parallelism (decode runs as
 *            one shared latent head of width 576).
 *   [V32]    "DeepSeek-V3.2-Exp unboxing", section 初步研读: the FP8 index
 *            kernel that scores the cached tokens (its signature and the
 *            shapes observed in a run) and the top-k selection after it.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or retains them.  bf16 means IEEE
 *     bfloat16 bit patterns (uint16), all tensors are dense row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: they only enqueue kernels.  Arguments are validated on the
 *     host before anything is enqueued; a non-zero status means nothing ran.
 *   - Values stored in device arrays (block_table entries, seq_lens) are the
 *     caller's contract and are not checked: every used block id must lie in
 *     [0, num_blocks), and q_len <= seq_lens[b] <= max_seq_len.
 *   - Supported dimensions: kv_lora 512, rope 64, qk_nope 128, v_dim 128,
 *     page 64, heads a multiple of 16 in [16, 128]; q_len (new tokens per
 *     sequence) 1..8 for the decode entry points, 1..65536 for
 *     mla_cache_insert[_fp8], 1..max_seq_len for mla_prefill.
 *   - Thread safety: calls are re-entrant; two calls that share a workspace
 *     or an output buffer must be ordered by the caller (same stream).
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,         /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,        /* a size argument is out of range or inconsistent */
  MLA_ERR_UNSUPPORTED = 3,  /* dimensions this build does not implement */
  MLA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
  MLA_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
  MLA_ERR_BOUNDS = 6,       /* debug checks: a block id or length breaks the contract */
  MLA_ERR_SCRATCH = 7       /* mla_decode_noalloc: the call needs more than its scratch */
} mla_status;

/* Model dimensions ([V3-src] MLA: kv_lora_rank, qk_rope_head_dim,
 * qk_nope_head_dim, v_head_dim; `heads` = heads served by this call). */
typedef struct {
  int32_t heads;    /* H */
  int32_t kv_lora;  /* latent width, must be 512 */
  int32_t rope;     /* rope width, must be 64 */
  int32_t qk_nope;  /* must be 128 */
  int32_t v_dim;    /* must be 128 */
  int32_t page;     /* tokens per cache block, must be 64 */
} mla_dims;

/*
 * mla_cache_insert — write the q_len new tokens of each sequence into the
 * paged cache ([V3-src] absorbed branch: the latent goes through kv_norm and
 * k_pe through the rotary embedding before both are cached; [V2L] §五: the
 * entry is latent followed by k_pe).
 *
 *   kv_a        bf16 [B, q_len, 576]  kv_a projection output of the new tokens
 *   rms_w       bf16 [512]            kv_a RMSNorm weight
 *   eps         RMSNorm epsilon, added inside the square root ([V2L] §四)
 *   rope_base   RoPE frequency base; pair j of the 64-wide k_pe, taken as
 *               (real, imaginary) = elements (2j, 2j+1), turns by
 *               position * rope_base^(-2j/64)
 *   block_table int32 [B, bt_stride]  physical block of each logical block
 *   seq_lens    int32 [B]  cache length INCLUDING the new tokens; new token i
 *               of sequence b sits at position seq_lens[b] - q_len + i
 *   cache       bf16 [num_blocks, 64, 576], updated in place; only the
 *               B*q_len addressed entries are written
 *
 * Latent: per row, sum of squares in a wide type, n = x / sqrt(mean + eps)
 * rounded to bf16, then weight * n rounded to bf16 ([V2L] §四 precision
 * rule).  k_pe: rotated in double precision, rounded once to bf16.
 * B == 0 is a no-op returning MLA_OK.
 */
int mla_cache_insert(const mla_dims* dims, const void* kv_a, const void* rms_w,
                     float eps, float rope_base, const int32_t* block_table,
                     int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                     int32_t q_len, void* cache, int32_t num_blocks, void* stream);

/*
 * mla_decode_workspace_bytes — size in bytes of the device workspace
 * mla_decode needs for these sizes (split plan, absorbed queries, per-split
 * partial results).  `num_splits_hint` must match the value later passed to
 * mla_decode.  Returns 0 for unsupported arguments.
 */
size_t mla_decode_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t q_len,
                                  int32_t max_seq_len, int32_t num_splits_hint);

/*
 * mla_decode — absorbed MLA decode over the paged cache ([V3-src] "(b)
 * 优化实现"; [TAGS] decode as one latent head; [V2L] §五 identities).
 *
 *   q           bf16 [B, q_len, H, 192]: q_nope (128) then q_pe (64), q_pe
 *               already rotated to its position
 *   kv_b        bf16 [H*256, 512]: kv_b_proj weight; rows h*256 + [0,128)
 *               are head h's W_UK, rows h*256 + [128,256) its W_UV
 *   cache       bf16 [num_blocks, 64, 576] (latent 512 then rope 64)
 *   block_table int32 [B, bt_stride]; seq_lens int32 [B] (see insert)
 *   max_seq_len host-side bound on every seq_lens[b] (sizes the plan)
 *   softmax_scale  scale applied to q.k, normally 1/sqrt(qk_nope + rope)
 *               ([TAGS] 1/sqrt(d_k), d_k = 128 + 64)
 *   out         bf16 [B, q_len, H, 128]: per-head attention output before
 *               the output projection
 *   workspace   device buffer of at least mla_decode_workspace_bytes(...)
 *   num_splits_hint  0 = balanced automatic split of each sequence across
 *               the GPU; k > 0 = split every sequence into min(k, pages) parts
 *               (k <= 64)
 *
 * Causality: new query i of sequence b attends to positions
 * t <= seq_lens[b] - q_len + i (the triu(1) mask of the forward pass, moved
 * to the cache offset).  Cache slots at positions >= seq_lens[b] are never
 * used, whatever they hold.  Arithmetic: bf16 inputs, bf16 matrix-core
 * products with fp32 accumulation, fp32 softmax statistics, bf16 output.
 * B == 0 is a no-op returning MLA_OK.
 */
int mla_decode(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
               int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
               const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
               float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
               int32_t num_splits_hint, void* stream);

/*
 * mla_decode_noalloc — mla_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, allocation-free serving loops,
 * harnesses that forbid hipMalloc.  Same arguments as mla_decode minus the
 * workspace, same kernels and output.  The workspace is a file-scope device
 * array of the library (mla_noalloc_scratch_bytes() = 128 MiB), which every
 * GPU the library runs on holds from the library's load until the process
 * ends; its address on the current device is looked up once per device.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Every call on one GPU uses that GPU's one array: calls that
 * overlap on a GPU (other streams, other threads) race and must be ordered
 * by the caller; nothing in the array needs to start at zero.  When the
 * automatic split plan's worst case does not fit, the planner is limited to
 * fewer work items (at least one per sequence); a call that does not fit
 * even then (or with num_splits_hint > 0, whose item count is fixed) returns
 * MLA_ERR_SCRATCH with nothing enqueued.
 */
size_t mla_noalloc_scratch_bytes(void);
int mla_decode_noalloc(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t batch, int32_t q_len,
                       int32_t max_seq_len, float softmax_scale, void* out,
                       int32_t num_splits_hint, void* stream);

/*
 * FP8 latent cache ("DeepSeek-V3.2-Exp unboxing", 初步研读: the deployed KV
 * cache is FP8, and the indexer beside it keeps one scale per cached token;
 * the vLLM DeepSeek-V4 notes, section 一: KV quantisation fused into the
 * cache insert, UE8M0 power-of-two scales).  The pages fix no format; this
 * library's row is MLA_FP8_ROW_BYTES bytes per token:
 *   bytes [0, 512)    the 512 latent values as FP8 E4M3 ("FN": bias 7, no
 *                     infinities, 0x7F/0xFF NaN, largest finite 448) codes
 *   bytes [512, 640)  the 64 rope values, bf16, little endian
 *   byte  640         scale byte s: the latent value of code c is
 *                     e4m3(c) * 2^(s - 127)
 *   bytes [641, 656)  zero
 * A page is 64 such rows; cache = uint8 [num_blocks, 64, 656].
 *
 * mla_cache_insert_fp8 — as mla_cache_insert (same arguments, same
 * normalised latent and rotated k_pe), then per token the scale 2^e is the
 * smallest power of two with max|latent| * 2^-e <= 448 (e in [-126, 127];
 * e = 0 for an all-zero latent) and each latent value is stored as the E4M3
 * code of value * 2^-e, rounded to nearest even.  Writes whole 656-byte rows.
 *
 * mla_decode_fp8 — as mla_decode (same arguments and workspace size, same
 * output) over an FP8 cache: every cached latent value is taken as
 * e4m3(code) * 2^(s - 127), which is exact in bf16, so the arithmetic is that
 * of mla_decode on the dequantised cache.
 */
#define MLA_FP8_ROW_BYTES 656
int mla_cache_insert_fp8(const mla_dims* dims, const void* kv_a, const void* rms_w,
                         float eps, float rope_base, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                         int32_t q_len, void* cache, int32_t num_blocks, void* stream);
int mla_decode_fp8(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                   int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
                   float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                   int32_t num_splits_hint, void* stream);

/*
 * mla_decode_step / mla_decode_step_fp8 — one decoding step with the
 * query-side work fused into the insert (the vLLM DeepSeek-V4 notes, section
 * 一: RoPE of the query, KV quantisation and cache insert in one kernel;
 * "深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA: the new tokens'
 * entries are cached before attention and q_pe is rotated at the same
 * positions as k_pe).  Equivalent to
 *   mla_cache_insert[_fp8](dims, kv_a, rms_w, eps, rope_base, block_table,
 *                          bt_stride, seq_lens, batch, q_len, cache, ...)
 *   q' = q with each head's q_pe rotated at position seq_lens[b] - q_len + i
 *        (the rotation of the insert: interleaved pairs, angle
 *        position * rope_base^(-2j/64), computed in double, rounded once to
 *        bf16)
 *   mla_decode[_fp8](dims, q', kv_b, cache, ...)
 * with bit-identical cache contents and output, in three launches on
 * `stream` instead of four (the insert, the RoPE of q_pe, the query
 * absorption and the split plan share one launch).
 *   q      bf16 [B, q_len, H, 192], q_pe part NOT rotated; read only
 *   kv_a, rms_w, eps, rope_base: as mla_cache_insert
 *   cache  read and written (the q_len new rows of every sequence)
 *   every other argument, the workspace size and the errors: as mla_decode
 *   (the insert's arguments are checked as mla_cache_insert checks them).
 */
int mla_decode_step(const mla_dims* dims, const void* q, const void* kv_a, const void* rms_w,
                    float eps, float rope_base, const void* kv_b, void* cache,
                    int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                    const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
                    float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                    int32_t num_splits_hint, void* stream);
int mla_decode_step_fp8(const mla_dims* dims, const void* q, const void* kv_a,
                        const void* rms_w, float eps, float rope_base, const void* kv_b,
                        void* cache, int32_t num_blocks, const int32_t* block_table,
                        int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                        int32_t q_len, int32_t max_seq_len, float softmax_scale, void* out,
                        void* workspace, size_t workspace_bytes, int32_t num_splits_hint,
                        void* stream);

/*
 * Prefill: attention for many new tokens per sequence (a prompt, or a chunk
 * of one) in the expanded multi-head form ([V3-src] "(a) Naive实现":
 * kv_b_proj expands every cached latent into the head's k_nope and v, the
 * key is k_nope followed by the shared k_pe).  It computes the same function
 * as mla_decode (same arguments, same causal rule: new query i of sequence b
 * sees positions t <= seq_lens[b] - q_len + i, same scale), with no bound on
 * q_len beyond max_seq_len: the dense 192/128-wide heads suit the
 * compute-bound case, the absorbed 576/512-wide ones the memory-bound decode.
 * The new tokens' entries must already be in the cache (mla_cache_insert).
 *
 * mla_prefill_workspace_bytes — bytes of device workspace mla_prefill needs
 * for this batch and max_seq_len (the expanded keys and values of every
 * head: batch * H * roundup(max_seq_len, 64) * 640 bytes, plus alignment), or
 * 0 if the arguments are invalid.
 *
 * mla_prefill
 *   q, kv_b, cache, num_blocks, block_table, bt_stride, seq_lens,
 *   max_seq_len, softmax_scale, out: as mla_decode (q bf16 [B, q_len, H, 192]
 *   with q_pe rotated; out bf16 [B, q_len, H, 128]); bf16 cache only
 *   workspace   device memory, >= mla_prefill_workspace_bytes; overwritten
 * Arithmetic: the expanded keys and values are rounded to bf16; bf16
 * matrix-core products with fp32 accumulation, fp32 softmax statistics
 * (running max and sum per row), bf16 output.  Errors as mla_decode.  Two
 * launches on `stream`; with profiling enabled the stages are recorded as
 * (expansion, attention, empty).
 */
size_t mla_prefill_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_seq_len);
int mla_prefill(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                const int32_t* seq_lens, int32_t batch, int32_t q_len, int32_t max_seq_len,
                float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * Sparse decode (DeepSeek Sparse Attention; [V32] "DeepSeek-V3.2-Exp
 * unboxing", section 初步研读: once the cache is written, an FP8 index kernel
 * scores the cached tokens and only the highest-scoring ones enter the
 * attention).  One new token per sequence (q_len 1); its cache entry and its
 * index key must already be written, so seq_lens[b] >= 1.
 *
 * Index score of cached position n of sequence b (fp32 arithmetic):
 *   o[n] = (sum_h index_w[b,h] * index_q[b,h,:]) . index_k[slot(n),:]
 *          * index_k_scale[slot(n)]
 * with E4M3 (FN) values for index_q and index_k; slot(n) is the paged slot
 * of position n (block_table[b, n / 64] * 64 + n % 64), so the index keys
 * share the latent cache's pages.  The weighted query sum is taken first;
 * the pages' per-head form sum_h w_h (q_h . k_n) is the same number up to
 * fp32 rounding.  Top-k: the min(top_k, seq_lens[b]) largest scores, equal
 * scores (-0 and +0 included) taken lower position first, kept positions in
 * ascending order, -1 past the count.  NaN scores rank above every number.
 *
 * mla_dsa_select — index scores and top-k only.
 *   index_heads  Hi, 1..1024; index_q uint8 [B, Hi, 128]; index_w fp32 [B, Hi]
 *   index_k      uint8 [num_blocks, 64, 128]; index_k_scale fp32 [num_blocks, 64]
 *   block_table, bt_stride, seq_lens, max_seq_len: as mla_decode
 *   top_k        1..65536; batch at most 65535 (all three sparse entry points)
 *   scores       fp32 [B, scores_stride] (scores_stride >= max_seq_len), out:
 *                entries n < seq_lens[b] written, the rest untouched
 *   indices      int32 [B, top_k], out; counts int32 [B] (NULL allowed), out
 * Two launches on `stream`; no workspace.  Errors as mla_decode.
 *
 * mla_dsa_workspace_bytes — bytes of device workspace mla_dsa_decode and
 * mla_dsa_decode_fp8 need (scores, kept positions, room for the kept rows
 * gathered into dense pages: batch * ceil(min(top_k, max_seq_len) / 64) *
 * 73728 bytes, which also holds the kept rows' slot list when they are read
 * in place, and the decode workspace of q_len 1), or 0 if the arguments are
 * invalid.
 *
 * mla_dsa_decode / mla_dsa_decode_fp8 — selection as above, then the MLA
 * decode (as mla_decode / mla_decode_fp8, q_len 1) over the kept positions
 * only.
 *   q, kv_b, cache (bf16 rows, or the FP8 rows of mla_decode_fp8), num_blocks,
 *   block_table, bt_stride, seq_lens, max_seq_len, softmax_scale, out,
 *   num_splits_hint: as mla_decode
 *   index_*, top_k: as mla_dsa_select
 *   indices_out  int32 [B, top_k] or NULL: the kept positions
 *   workspace    device memory, >= mla_dsa_workspace_bytes; overwritten
 * Launches on `stream`: index scores, then top-k, which for mla_dsa_decode
 * at 128 heads (at most 4096 kept positions per sequence, a cache of at most
 * 3.5 GiB) also writes the kept rows' slot list so that the decode reads them
 * in place; otherwise (and for mla_dsa_decode_fp8) a gather of the kept rows
 * into dense pages follows; then the three decode launches.  With profiling
 * enabled a call takes two profile slots: (index scores, top-k, gather or
 * nothing), then (prep, decode, combine).
 */
int mla_dsa_select(int32_t index_heads, const void* index_q, const float* index_w,
                   const void* index_k, const float* index_k_scale, const int32_t* block_table,
                   int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                   int32_t max_seq_len, int32_t top_k, float* scores, int32_t scores_stride,
                   int32_t* indices, int32_t* counts, void* stream);
size_t mla_dsa_workspace_bytes(const mla_dims* dims, int32_t batch, int32_t max_seq_len,
                               int32_t top_k, int32_t num_splits_hint);
int mla_dsa_decode(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                   int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                   int32_t index_heads, const void* index_q, const float* index_w,
                   const void* index_k, const float* index_k_scale, int32_t top_k,
                   float softmax_scale, void* out, int32_t* indices_out, void* workspace,
                   size_t workspace_bytes, int32_t num_splits_hint, void* stream);
int mla_dsa_decode_fp8(const mla_dims* dims, const void* q, const void* kv_b, const void* cache,
                       int32_t num_blocks, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                       int32_t index_heads, const void* index_q, const float* index_w,
                       const void* index_k, const float* index_k_scale, int32_t top_k,
                       float softmax_scale, void* out, int32_t* indices_out, void* workspace,
                       size_t workspace_bytes, int32_t num_splits_hint, void* stream);

/*
 * mla_profile_enable / mla_profile_collect — stage timing for benchmarks.
 * While enabled (max_calls > 0), each mla_decode / mla_decode_fp8 /
 * mla_decode_step / mla_decode_step_fp8 call records
 * four HIP events
 * on its stream: before the prep kernel (query absorption + split plan),
 * before the split-KV decode kernel, before the merge + projection kernel, and
 * after it (for the step entry points the first stage also holds the
 * insert).  Events come from a pool of max_calls sets created here
 * (hipEventCreateWithFlags with hipEventDisableSystemFence: timing only, no
 * cache write-back at the stage boundaries; no device memory); calls beyond
 * the pool are not timed.
 * mla_profile_enable(0) releases the pool.  mla_profile_collect waits for the
 * recorded events and writes, per stage, the summed milliseconds over the
 * timed calls into stage_ms[3] (prep, decode, combine) and the call count into
 * *calls, then empties the pool for reuse.  mla_profile_collect_calls writes
 * each timed call's three stage times instead (stage_ms[3 * c + k] for call
 * c in order; MLA_ERR_SHAPE if more than max_calls calls were timed).  Each
 * recorded event adds a few microseconds to the stage it closes.  Not
 * thread-safe; for benchmarks only.
 */
int mla_profile_enable(int32_t max_calls);
int mla_profile_collect(double* stage_ms, int32_t* calls);
int mla_profile_collect_calls(double* stage_ms, int32_t max_calls, int32_t* calls);

/* Static, human-readable text for a status code (never NULL). */
const char* mla_status_string(int status);

/* ABI version of this header: 1. */
int mla_abi_version(void);

/*
 * mla_debug_checks — host-side checks of the device-side contract (block ids
 * in [0, num_blocks), lengths in [q_len, max_seq_len] and within the block
 * table's width): enable > 0 turns them on, 0 off, < 0 only queries.  Returns
 * the previous setting.  The initial setting is MLA_DEBUG_CHECKS from the
 * environment (unset or "0": off).  While on, every entry point that takes a
 * block table first copies it and seq_lens to the host on its stream and
 * waits for the copy (the call then synchronises); a violation returns
 * MLA_ERR_BOUNDS with nothing enqueued.  mla_cache_insert checks the blocks
 * that receive the new tokens, the decode, prefill and sparse entry points
 * every block of each sequence, mla_dsa_select the lengths and table width
 * (it has no block count).  For debugging: the copy costs a round trip.
 */
int mla_debug_checks(int32_t enable);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
