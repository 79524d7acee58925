/*
 * pa_blocks.h -- block copies on the device and the host block manager.
 *
 * Sources, cited by page title and section:
 *   [Q67]  quant67, "【大模型基础设施工程】12：PagedAttention 与 Continuous
 *          Batching": §3.3 (a decode step appends to the last block if it has
 *          room, else takes a block from the free pool), §3.5 and §3.8
 *          (samples of one prompt share its blocks through reference counts;
 *          a sample that must write into a shared block copies it to a new
 *          block first -- copy-on-write), §3.9 and §6.1 (preemption by swap:
 *          a sequence's blocks go to host memory and come back later), §5.2
 *          (full blocks keyed by a hash of their tokens and of the previous
 *          block's key; a hit shares the block and adds a reference; blocks
 *          nobody references are evicted least recently used first).
 *   [LPNH] lpnh.cn, "大模型推理架构演进：从 PagedAttention 到 Prefill-Decode
 *          分离的深度解析", §二 2.2, third step: blocks are allocated on
 *          demand and return to a global pool when the request finishes.
 *
 * Status codes are those of pa.h.  No C++ exception crosses this interface.
 */
#ifndef PA_BLOCKS_H_
#define PA_BLOCKS_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------
 * Device block copies.  A pool is any array whose first axis is the block
 * id and whose blocks are block_bytes apart (the K and V pools of pa.h, in
 * any element type, 8-bit pools included).  Copies are bit-exact.
 *
 * block_mapping: int64 [num_pairs][2] of (src, dst) block ids, readable by
 * the device (device memory, or pinned host memory from hipHostMalloc).
 * A pair whose src or dst lies outside its pool is skipped.  Destinations
 * must be distinct, and for pa_copy_blocks no destination may also be a
 * source; otherwise the result is undefined.  num_pairs == 0 is a no-op.
 * block_bytes must be a positive multiple of 16 and the pools 16-byte
 * aligned.  Both calls only enqueue one kernel on `stream` and return.
 */

/*
 * pa_copy_blocks -- [Q67] §3.8 copy-on-write: for every pair,
 *   k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src]
 * (whole blocks: every KV head, token slot and channel).  Device pools.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                         int64_t block_bytes, int64_t num_blocks, void* stream);

/*
 * pa_swap_blocks -- [Q67] §3.9 swap: for every pair,
 *   dst_k[dst] = src_k[src] and dst_v[dst] = src_v[src]
 * between two pools of the same block size, one of which is usually pinned
 * host memory (swap out: device -> host, swap in: host -> device).  Host
 * pools must come from hipHostMalloc (or torch's pinned allocator) and be
 * mapped at the same address on the device (the runtime's attributes are
 * checked); the kernel reads or writes them over the host link.  A pageable
 * host pointer, or pinned memory mapped elsewhere, is rejected with
 * PA_ERR_UNSUPPORTED before anything is enqueued.  The source and
 * destination pools must not overlap (PA_ERR_SHAPE).
 */
pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int64_t* block_mapping, int64_t num_pairs, int64_t block_bytes,
                         int64_t src_num_blocks, int64_t dst_num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * Host block manager: the free pool, per-sequence block tables, reference
 * counts with copy-on-write, prefix keys with LRU eviction, and a host pool
 * for swapped-out sequences.  Host memory only; no call touches the GPU.
 * A manager is not thread-safe: one caller at a time.
 *
 * Rules (readings of the pages where they leave a step open):
 *   - Free blocks are handed out first in, first out, starting with block
 *     ids 0, 1, 2, ... in order.
 *   - A full block is registered under its key when it becomes full (at
 *     allocation for full prompt blocks, on the append that fills it, on
 *     swap-in), unless that key is registered already.  Its key covers the
 *     tokens of the block and of every block before it.
 *   - A block whose count falls to zero returns to the free pool, or, if it
 *     is registered, stays cached and joins the eviction order.  A free
 *     sequence releases its blocks last to first.  Cached blocks are evicted
 *     (least recently released first) only when the free pool is empty.
 *   - Prefix lookup walks the prompt's full blocks from the first and stops
 *     at the first miss; it never covers the block holding the last prompt
 *     token.  A hit adds a reference (taking a cached block back out of the
 *     eviction order).
 *   - Copy-on-write happens while the last block's count is above one; the
 *     last sharer writes in place.
 *   - Any call that lacks blocks returns PA_ERR_NO_BLOCKS and changes
 *     nothing.
 * Keys are two independent 64-bit chained hashes (SplitMix64 finaliser
 * over the previous key and the block's tokens); a hit also compares the
 * stored tokens and the previous block's key, so only a full 128-bit
 * collision of two different prefixes could share a block wrongly.
 * ------------------------------------------------------------------------ */

typedef struct pa_block_manager pa_block_manager;

/* New manager for a device pool of num_blocks blocks of block_size tokens
 * and a host pool of num_host_blocks blocks (0: no swap).  prefix_caching
 * != 0 enables the prefix keys.  *out receives the handle (host memory the
 * library owns until pa_bm_destroy).  Errors: PA_ERR_NULL, PA_ERR_SHAPE
 * (num_blocks < 1 or > 2^31 - 1, block_size < 1, num_host_blocks < 0). */
pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int64_t num_host_blocks,
                       int32_t prefix_caching, pa_block_manager** out);

/* Frees the manager and everything it holds.  NULL is a no-op. */
void pa_bm_destroy(pa_block_manager* m);

/* Blocks for a new prompt of num_tokens token ids (host array).  Leading
 * full blocks found under their keys are shared; *num_cached_tokens (may
 * be NULL) receives how many leading tokens they hold -- the caller
 * computes and writes K/V only for the tokens after them.  Errors:
 * PA_ERR_STATE (seq_id exists), PA_ERR_SHAPE (num_tokens < 1),
 * PA_ERR_NO_BLOCKS. */
pa_status pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* tokens,
                             int64_t num_tokens, int64_t* num_cached_tokens);

/* child shares every block of parent (one more reference each) and copies
 * its tokens ([Q67] §3.5).  Errors: PA_ERR_STATE. */
pa_status pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child);

/* Room for the sequence's next token: *slot (= block * block_size +
 * offset) is where its K/V go.  If the last block was shared, it was copied:
 * *cow_src and *cow_dst name the device copy the caller must enqueue
 * (pa_copy_blocks) before writing the slot; both are -1 otherwise.  Errors:
 * PA_ERR_STATE (unknown or swapped out), PA_ERR_NO_BLOCKS. */
pa_status pa_bm_append_slot(pa_block_manager* m, int64_t seq_id, int32_t token, int64_t* slot,
                            int64_t* cow_src, int64_t* cow_dst);

/* Drops the sequence and releases its blocks (device or host).  Errors:
 * PA_ERR_STATE. */
pa_status pa_bm_free(pa_block_manager* m, int64_t seq_id);

/* Moves the sequence to host blocks: pairs (host array int64 [n][2], room
 * for `capacity` pairs) receives (device block, host block) for every block
 * of the sequence in table order, *num_pairs their count; the caller runs
 * pa_swap_blocks with them before the device blocks are reused.  Errors:
 * PA_ERR_STATE, PA_ERR_NO_BLOCKS (host pool), PA_ERR_SHAPE (capacity). */
pa_status pa_bm_swap_out(pa_block_manager* m, int64_t seq_id, int64_t* pairs, int64_t capacity,
                         int64_t* num_pairs);

/* Brings a swapped-out sequence back into fresh device blocks: pairs
 * receives (host block, device block).  Errors as pa_bm_swap_out (device
 * pool for PA_ERR_NO_BLOCKS). */
pa_status pa_bm_swap_in(pa_block_manager* m, int64_t seq_id, int64_t* pairs, int64_t capacity,
                        int64_t* num_pairs);

/* Block table of a sequence (host int32 array with room for `capacity`
 * entries; device block ids, or host block ids while swapped out), its
 * length in *num_entries.  Errors: PA_ERR_STATE, PA_ERR_SHAPE (capacity). */
pa_status pa_bm_block_table(const pa_block_manager* m, int64_t seq_id, int32_t* table, int64_t capacity,
                            int64_t* num_entries);

/* Padded block tables of several resident sequences, ready for
 * pa_attention_varlen: tables (host int32 [num_seqs][width]) row i holds the
 * table of seq_ids[i], padded with 0; seq_lens (host int32 [num_seqs], may
 * be NULL) their token counts.  Errors: PA_ERR_STATE, PA_ERR_SHAPE (a table
 * longer than width or a length beyond int32). */
pa_status pa_bm_block_tables(const pa_block_manager* m, const int64_t* seq_ids, int64_t num_seqs,
                             int32_t* tables, int32_t width, int32_t* seq_lens);

/* Slots of tokens start .. start+count-1 of a resident sequence (host
 * int64 array).  Errors: PA_ERR_STATE, PA_ERR_SHAPE (range past its end). */
pa_status pa_bm_slot_mapping(const pa_block_manager* m, int64_t seq_id, int64_t start, int64_t count,
                             int64_t* slots);

/* Token count and swap state (1 = swapped out) of a sequence; either output
 * may be NULL.  Errors: PA_ERR_STATE. */
pa_status pa_bm_seq_info(const pa_block_manager* m, int64_t seq_id, int64_t* num_tokens, int32_t* swapped);

/* Reference count of a device block (number of resident block-table
 * entries that hold it).  Errors: PA_ERR_SHAPE (block out of range). */
pa_status pa_bm_refcount(const pa_block_manager* m, int64_t block, int32_t* count);

/* Pool counters, each output may be NULL: blocks an allocation may take
 * (free plus cached-unreferenced), registered (cached) blocks, free host
 * blocks, live sequences. */
pa_status pa_bm_stats(const pa_block_manager* m, int64_t* num_free, int64_t* num_cached,
                      int64_t* num_host_free, int64_t* num_seqs);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H_ */
