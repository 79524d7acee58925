/*
 * pa.h -- C ABI of the paged-attention library for MI355X (gfx950).
 *
 * Two device operations make up one step of attention over a paged KV cache:
 *
 *   pa_cache_write       scatter this step's new K/V rows into the block pool
 *                        through slot_mapping;
 *   pa_attention_varlen  causal softmax attention of packed query rows over
 *                        the pool, reached through per-request block tables.
 *
 * Sources, cited by page title and section:
 *   [Q67]  quant67, "【大模型基础设施工程】12：PagedAttention 与 Continuous
 *          Batching": §3.2 (KV cut into fixed-size blocks, logical->physical
 *          mapping through a block table), §3.3 (data structures, the worked
 *          address example, and the per-step order: compute the new token's
 *          K/V, append it to its block, then attend through the block table),
 *          §3.6 (the kernel walks block_table[seq][i] and accumulates an
 *          online softmax), §3.7 (16 tokens per block), §4.2 (chunked prefill
 *          mixes prompt chunks with decode rows), §8.3 (bytes per block count
 *          every KV head).
 *   [ICE]  ice-wocker, "推理优化与服务：从 PagedAttention 到分离式部署", latest
 *          developments: scheduled query tokens packed as [total_q, H, D]
 *          with cu_seqlens request boundaries, so one forward runs mixed
 *          prefill and decode.
 *
 * Conventions shared by every call (this library's reading of the pages):
 *   - Pools: K and V are separate device arrays [num_blocks, Hkv, 16, D],
 *     row-major.  One block id covers every KV head ([Q67] §8.3); each
 *     (block, head) tile of 16 x D elements is contiguous.
 *   - slot = physical_block * 16 + offset ([Q67] §3.3: token 18 of table
 *     [17, 42] lives in block 42 at offset 2, slot 674).
 *   - Request b owns packed query rows cu_seqlens[b] .. cu_seqlens[b+1]-1
 *     ([ICE]).  Its context length seq_lens[b] = L_b already counts those
 *     rows (new K/V are written before attention reads them, [Q67] §3.3).
 *     Row j (0-based within the request, n_b rows) is the token at position
 *     L_b - n_b + j and attends to keys 0 .. L_b - n_b + j (bottom-right
 *     causal alignment; a decode row sees all L_b keys).
 *   - GQA: query head h reads KV head h / G, G = num_q_heads / num_kv_heads.
 *   - q, out, the pools and the new rows share one element type (pa_dtype).
 *     Accumulation is fp32; bf16 results are rounded to nearest even.
 *
 * Pointers are DEVICE pointers unless marked host.  The device calls
 * allocate nothing and keep no state between calls; the caller owns every
 * buffer.  (The host block manager in pa_blocks.h is the one stateful part.)
 * Both hot calls only enqueue work on `stream` (a hipStream_t passed as
 * void*, NULL = the null stream) and return; they never synchronise, read
 * device memory from the host, or allocate, so they can be captured in a HIP
 * graph.  Buffers must stay alive until the stream's work completes.
 * Host-checkable preconditions are checked first; on failure a negative
 * status is returned and nothing is enqueued.  Device metadata (slots, block
 * ids, lengths) is trusted on the hot path; pa_validate_metadata checks it.
 * No C++ exception crosses this interface.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,         /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,        /* a size is out of range or inconsistent */
  PA_ERR_UNSUPPORTED = -3,  /* dtype / head_dim / group size / block size not built */
  PA_ERR_ALIGN = -4,        /* pointer or row stride not 16-byte aligned */
  PA_ERR_WORKSPACE = -5,    /* workspace missing or smaller than required */
  PA_ERR_LAUNCH = -6,       /* the HIP runtime rejected a kernel launch */
  PA_ERR_METADATA = -7,     /* pa_validate_metadata found a bad entry */
  PA_ERR_NO_BLOCKS = -8,    /* block manager: not enough free blocks; nothing changed */
  PA_ERR_STATE = -9,        /* block manager: unknown, existing or swapped-out sequence */
  PA_ERR_HOST_MEMORY = -10  /* block manager: host allocation failed */
} pa_status;

typedef enum {
  PA_F32 = 0,   /* IEEE fp32 */
  PA_BF16 = 1   /* bfloat16 */
} pa_dtype;

/* Host struct describing one pa_attention_varlen call. */
typedef struct {
  int32_t num_seqs;            /* B >= 0 */
  int64_t total_q;             /* packed query rows, = cu_seqlens_q[B] */
  int32_t num_q_heads;         /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;        /* Hkv */
  int32_t head_dim;            /* D: 64, 128 or 256 */
  int32_t block_size;          /* tokens per physical block: 16 (the pages' default), 8 or 32.
                                  The fast single-row decode kernel (bf16 or 8-bit pools)
                                  takes D = 64, 128 and 256 with Hq/Hkv a power of two up
                                  to 64, and at D = 128 also Hq/Hkv = 3, 5 to 7 and 9 to
                                  15, at all three block sizes; the MFMA prefill kernel
                                  takes the same shapes; every other shape runs on the
                                  generic split-K kernel (fp32, or bf16 at D = 64 and
                                  256, with Hq/Hkv up to 8 or 16), and the rest return
                                  PA_ERR_UNSUPPORTED. */
  int64_t num_blocks;          /* physical blocks in each pool */
  int32_t max_blocks_per_seq;  /* row length of block_tables */
  int32_t max_query_len;       /* host bound: >= every n_b */
  int32_t max_seq_len;         /* host bound: >= every L_b */
  int64_t q_row_stride;        /* elements between consecutive packed rows of q  (>= Hq*D) */
  int64_t o_row_stride;        /* elements between consecutive packed rows of out (>= Hq*D) */
  float scale;                 /* softmax scale, finite and > 0, usually 1/sqrt(D) */
  pa_dtype dtype;
  int32_t partition_size;      /* tokens per split-K context partition, a multiple of 16
                                  in [16, 8192].  Given explicitly, a request's result
                                  depends only on the request (bitwise the same in any
                                  batch).  0 = library default: 512, 1024 or 2048 chosen
                                  from num_seqs, num_kv_heads and max_seq_len (results may
                                  then differ in the last bits between batch shapes). */
  int32_t sliding_window;      /* 0: every row sees its whole causal context.  W > 0: row j
                                  of request b sees only the last W positions up to its own,
                                  keys max(0, p - W + 1) .. p with p = L_b - n_b + j ([Q67]
                                  §10.8 lists the sliding-window mask among the kernel
                                  variants; this is its reading).  Must be >= 0. */
  int32_t num_decode_rows;     /* host hint, >= 0: requests with exactly one query row (0 if none
                                  or unknown).  Scheduling only -- results are the same bits
                                  whatever it says.  When > 0 and the batch also has multi-row
                                  requests on the MFMA prefill kernel, the run overlaps the two
                                  kernels ([ICE]: one step packs decode and prefill rows; prefill is
                                  compute-bound, decode bandwidth-bound): the prefill kernel runs
                                  on a second stream of the library's (one per device, default
                                  priority), forked from and joined back to the caller's stream,
                                  so the call still completes in the caller's stream order.  A
                                  call captured into a graph records the fork and join; two
                                  captures that overlap on one device must not both use it. */
} pa_attn_params;

/*
 * pa_cache_write -- [Q67] §3.3: each new token's K and V are appended to the
 * block that holds its position.
 *
 * For every row i < num_tokens with slot_mapping[i] >= 0 and every KV head h:
 *   k_cache[s/16][h][s%16][:] = k_new[i*kv_row_stride + h*D + :]
 *   v_cache[s/16][h][s%16][:] = v_new[i*kv_row_stride + h*D + :]
 * with s = slot_mapping[i].  Rows with a negative slot are skipped.  The
 * copy is bit-exact.  Slots must be unique and < num_blocks*bs (not checked
 * here).  k_new/v_new: [num_tokens, Hkv, D] rows kv_row_stride elements
 * apart (>= Hkv*D).  k_cache, v_cache: [num_blocks, Hkv, bs, D] in place,
 * bs = block_size (the formulas above are written for 16; slot s names block
 * s / bs, offset s % bs).  num_tokens == 0 is a no-op.  Errors: NULL pointers
 * (when num_tokens > 0), non-positive sizes, block_size not in {8, 16, 32},
 * D not in {64, 128, 256}, unaligned pointers or stride.
 */
pa_status pa_cache_write(const void* k_new, const void* v_new, int64_t kv_row_stride,
                         void* k_cache, void* v_cache, const int64_t* slot_mapping,
                         int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                         void* stream);

/*
 * Bytes of device workspace pa_attention_varlen needs for these parameters
 * (0 when no request can span more than one context partition).  Returns
 * 0 as well for invalid parameters; pa_attention_varlen reports those.
 */
size_t pa_attention_workspace_size(const pa_attn_params* p);

/*
 * Context-partition length (tokens) pa_attention_varlen uses for these
 * parameters: p->partition_size when it is non-zero, else the library
 * default.  Returns 0 for invalid parameters.  A caller that needs results
 * independent of the batch shape can read the default here once and pass it
 * explicitly from then on.
 */
int32_t pa_attention_partition_size(const pa_attn_params* p);

/*
 * pa_attention_varlen -- [Q67] §3.6 and [ICE]: for every request b, row j,
 * query head h:
 *   s_t = scale * <q[row, h, :], K_b[t, h/G, :]>       for lo_j <= t <= L_b - n_b + j
 *   out[row, h, :] = sum_t softmax(s)_t * V_b[t, h/G, :]
 * with lo_j = 0, or max(0, L_b - n_b + j - W + 1) for a sliding window W > 0,
 * where K_b[t] = k_cache[block_tables[b][t/16]][h/G][t%16] (same for V) and
 * row = cu_seqlens_q[b] + j.
 *
 *   out           [total_q, Hq, D] rows o_row_stride elements apart (written)
 *   q             [total_q, Hq, D] rows q_row_stride elements apart
 *   k_cache/v_cache  pools as above (read only)
 *   cu_seqlens_q  int32 [B+1], [0] = 0, nondecreasing, [B] = total_q
 *   seq_lens      int32 [B], L_b >= n_b = cu[b+1]-cu[b]; n_b == 0 is allowed
 *   block_tables  int32 [B, max_blocks_per_seq]; entries at or past
 *                 ceil(L_b/16) are never read
 *   workspace     device scratch of >= pa_attention_workspace_size(p) bytes
 *                 (may be NULL when that size is 0); contents need no init
 *
 * Requests with one row run on the split-K decode kernels; in bf16, requests
 * with more rows run on the MFMA prefill kernel.  Results do not depend on
 * the other requests in the batch or on block placement.  `out` must not
 * alias q or the pools.
 */
pa_status pa_attention_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                              const int32_t* block_tables, const pa_attn_params* p,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_attention_plan / pa_attention_run -- pa_attention_varlen in two stages.
 * [Q67] §3.3: the scheduler builds the step's metadata (cu_seqlens, seq_lens,
 * block tables) once, and every layer's attention reads it.  The work lists
 * the kernels deal out depend only on cu_seqlens_q, seq_lens and *p, so
 * pa_attention_plan builds them once per step into the workspace and
 * pa_attention_run computes one layer from them, as often as there are
 * layers.  pa_attention_varlen(...) == pa_attention_plan(...) followed by
 * pa_attention_run(...), bit for bit.
 *
 * Preconditions of pa_attention_run (not checked on the device): the
 * workspace holds the lists of a pa_attention_plan (or pa_attention_varlen)
 * enqueued earlier with the same *p and the same cu_seqlens_q / seq_lens
 * contents, and nothing else wrote the workspace since; runs on one
 * workspace are serialised (same stream, or ordered by events), since each
 * run hands out the list's items from a counter in the workspace and leaves
 * it re-armed for the next run.  Arguments, layouts and host-side errors are
 * those of pa_attention_varlen; pa_attention_plan reads only cu_seqlens_q,
 * seq_lens, *p and the workspace.
 */
pa_status pa_attention_plan(const int32_t* cu_seqlens_q, const int32_t* seq_lens, const pa_attn_params* p,
                            void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_attention_run(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                           const int32_t* block_tables, const pa_attn_params* p,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * 8-bit KV cache (OCP FP8 E4M3).  [Q67] §8.8 and §10.3 name 8-bit KV caches
 * as the way to halve KV memory without fixing a format; the format taken is
 * OCP E4M3: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, subnormals
 * m * 2^-9, largest finite 448, S.1111.111 = NaN, no infinities.  Each pool
 * has one fp32 scale: a code c stands for decode(c) * scale.
 *
 * pa_cache_write_fp8 -- as pa_cache_write, but the new rows are bf16 and the
 * pools [num_blocks, Hkv, bs, D] hold one byte per element: each value x is
 * stored as the code nearest to x / scale (the fp32 quotient rounded to
 * nearest), ties to the even code, magnitudes of 448 and beyond saturated to
 * 448, NaN stored as 0x7F.  D in {64, 128, 256}; scales finite and > 0.
 * Errors as pa_cache_write.
 */
pa_status pa_cache_write_fp8(const void* k_new, const void* v_new, int64_t kv_row_stride,
                             void* k_cache, void* v_cache, const int64_t* slot_mapping,
                             int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int64_t num_blocks, float k_scale, float v_scale,
                             void* stream);

/*
 * pa_attention_varlen_fp8 -- as pa_attention_varlen with 8-bit pools: the
 * attention runs over K = decode(k_cache) * k_scale and V = decode(v_cache) *
 * v_scale.  q and out are bf16 (p->dtype == PA_BF16); D = 64, 128 or 256 with
 * Hq/Hkv a power of two up to 64, or at D = 128 also 3, 5 to 7 or 9 to 15;
 * block size 8, 16 or 32; other shapes return PA_ERR_UNSUPPORTED.  Requests with one row run on the split-K decode kernel,
 * requests with more rows (chunked prefill, [Q67] §4.2) on the MFMA kernel,
 * which widens the codes to bf16 as it stages them.  Scales finite and > 0.
 * The workspace is sized by pa_attention_workspace_size(p).
 */
pa_status pa_attention_varlen_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                  const int32_t* block_tables, const pa_attn_params* p,
                                  float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, void* stream);
/* The run stage of pa_attention_varlen_fp8 over lists from pa_attention_plan
 * (same contract as pa_attention_run). */
pa_status pa_attention_run_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                               const int32_t* block_tables, const pa_attn_params* p,
                               float k_scale, float v_scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * pa_attention_varlen_noalloc -- pa_attention_varlen for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, layouts, result and
 * host-side errors as pa_attention_varlen, without the workspace: the work
 * lists and split-K partials live in a static scratch of
 * PA_NOALLOC_SCRATCH_BYTES in the library's device memory, one copy per GPU,
 * held from the first call on that GPU until the process ends.  The call
 * uses the scratch of the current device (the stream must belong to it),
 * whose address it looks up on its first call there; it allocates nothing.
 * Parameters whose pa_attention_workspace_size exceeds
 * PA_NOALLOC_SCRATCH_BYTES return PA_ERR_WORKSPACE and enqueue nothing.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (other streams, other threads) race and give undefined results; calls
 * ordered on one stream are safe.  The scratch keeps the last call's
 * contents, and each call rewrites what it reads before reading it.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_attention_varlen_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                      const int32_t* block_tables, const pa_attn_params* p, void* stream);

/* Bits of the result word written by pa_validate_metadata. */
#define PA_BAD_CU_SEQLENS   1   /* cu[0] != 0, cu decreasing, or cu[B] != total_q */
#define PA_BAD_LENGTHS      2   /* n_b > L_b, L_b < 0, n_b > max_query_len or L_b > max_seq_len */
#define PA_BAD_TABLE_WIDTH  4   /* ceil(L_b/block_size) > max_blocks_per_seq */
#define PA_BAD_BLOCK_ID     8   /* a used block-table entry outside [0, num_blocks) */
#define PA_BAD_SLOT_RANGE  16   /* a slot >= num_blocks*block_size */
#define PA_BAD_SLOT_DUP    32   /* two rows share a non-negative slot */

/*
 * pa_validate_metadata -- debugging aid for the device-resident metadata
 * the hot calls trust.  Enqueues checks on `stream` and returns; when the
 * stream's work is done, *result (DEVICE, one int32 owned by the caller)
 * holds the OR of the PA_BAD_* bits of every failed check, 0 if all pass.
 * slot_mapping may be NULL (num_slots ignored); the duplicate-slot check is
 * quadratic in num_slots.  Host-side errors as for pa_attention_varlen.
 */
pa_status pa_validate_metadata(const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                               const int32_t* block_tables, const int64_t* slot_mapping,
                               int64_t num_slots, const pa_attn_params* p,
                               int32_t* result, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(pa_status s);

/* ABI version of this header: major*100 + minor (101: the 8-bit cache calls;
 * 102: block copies and the host block manager, pa_blocks.h; 200:
 * pa_attn_params.sliding_window; 201: block sizes 8 and 32, D = 256; 202:
 * 8-bit pools at block sizes 8 and 32; 203: pa_attention_plan / pa_attention_run;
 * 204: the fast decode kernel and 8-bit pools at D = 64 and 256, the MFMA
 * prefill kernel at D = 64 and 256; 205: the fast decode kernel and 8-bit
 * pools for Hq/Hkv above 8, and above 2 at D = 256; the MFMA prefill kernel
 * for Hq/Hkv above 8; 206: pa_attention_varlen_noalloc; 207: multi-row
 * requests on 8-bit pools; 208: pa_attn_params.num_decode_rows). */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
