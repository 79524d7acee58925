// Internal launch interface between the C ABI (pa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kDefaultPartition = 512;

// First key a row at position pos sees: 0, or the oldest of the last W
// positions with a sliding window W > 0.
__host__ __device__ inline int window_start(int pos, int window) {
  return window > 0 ? (pos - window + 1 > 0 ? pos - window + 1 : 0) : 0;
}

// Arguments of the split-K decode kernel and its partition merge.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  float* ws_o;       // [prows, Hq, max_parts, D] unnormalised partial outputs
  float* ws_ml;      // [prows, Hq, max_parts, 2] (running max in log2 units, sum)
  int64_t q_row_stride;   // elements
  int64_t o_row_stride;   // elements
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t part_size;      // tokens per partition, multiple of 16
  int32_t max_parts;      // ceil(max_seq_len / part_size)
  float scale_log2;       // softmax scale * log2(e)
  int32_t* plan;            // fast kernel's work list (header + items), in the workspace
  int64_t merge_off_ints;   // list of requests with more than one partition: plan + kPlanHeaderInts + this
  int32_t plan_capacity;    // decode entries the work list has room for (>= 1)
  float lsum_scale;         // the softmax sum is multiplied by this (1 / v_scale for 8-bit pools, else 1)
  int32_t row_mode;         // which requests this launch serves (RowMode)
  int32_t partial_by_seq;   // 1: partials indexed by request, else by packed row
  int32_t merge_capacity;   // entries the merge list has room for
  int32_t sliding_window;   // 0, or W > 0: a row sees only the last W positions up to its own
  int32_t block_size;       // tokens per physical block (the generic kernel takes 8, 16 or 32)
  int32_t head_split_log2;  // fast kernel: a KV head's query heads are served by 2^this work items
};

// Requests a decode launch serves: all of them, only those with exactly one
// query row, or only those with more than one row.  Empty requests never.
enum RowMode : int32_t { kAllRows = 0, kSingleRowOnly = 1, kMultiRowOnly = 2 };

// Arguments of the MFMA prefill kernel (bf16, requests with n_b > 1).
struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int64_t q_row_stride;
  int64_t o_row_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks_per_seq;
  int32_t* plan;          // work list (prefill entries at plan + kPlanHeaderInts + pref_off_ints; the header's
                          // prefill claim counters are updated by the kernel)
  int64_t pref_off_ints;
  float scale_log2;
  // Context split of short requests (see PlanArgs::split_rows): a request with
  // n <= split_rows rows and more than one partition of part_size tokens is
  // computed per partition into partials [partial row, Hq, max_parts, D] and
  // (m, l), partial row = num_seqs + packed row; the merge list combines them.
  int32_t split_rows;
  int32_t part_size;
  int32_t max_parts;
  float* ws_o;
  float* ws_ml;
  int32_t tile_pairs;   // (query row, head) pairs per list entry: 256 (64 at D = 256), or 64 (32) for short requests
  int32_t sliding_window;
  int32_t block_size;   // tokens per physical block: 8, 16 or 32
  int32_t head_split_log2;   // a KV head's query heads are served by 2^this items (set by launch_prefill)
  float lsum_scale;          // 8-bit pools: the softmax sum is multiplied by this (1 / v_scale)
  int32_t claim_items;       // 1: items after the first are claimed from the list header's counter (beside a
                             // decode launch); 0: dealt out statically
};

hipError_t launch_cache_write(const void* k_new, const void* v_new, int64_t kv_row_stride_bytes, void* k_cache,
                              void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_bytes, int32_t block_size, hipStream_t stream);
// bf16 rows quantised to OCP FP8 E4M3 codes with per-tensor scales (D = 64 or 128).
hipError_t launch_cache_write_fp8(const void* k_new, const void* v_new, int64_t kv_row_stride_bytes, void* k_cache,
                                  void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, float k_scale, float v_scale,
                                  hipStream_t stream);

// dtype: 0 fp32, 1 bf16.  Returns hipErrorInvalidValue for shapes not built.
hipError_t launch_decode(int dtype, int head_dim, int group, const DecodeArgs& a, int64_t partial_rows,
                         hipStream_t stream);
bool decode_supported(int dtype, int head_dim, int group, int part_size);

// Work lists of the persistent kernels (plan.hip), in the workspace.
constexpr int kPlanHeaderInts = 64;      // header words (256 bytes)
constexpr int kPlanCountInt = 8;         // header slot: number of decode entries
constexpr int kPlanPrefCountInt = 9;     // header slot: number of prefill entries
constexpr int kPlanMergeCountInt = 10;   // header slot: number of merge entries (rows with > 1 partition)
constexpr int kPlanClaimInt = 11;        // header slot: claim counter of the fast decode kernel (zeroed by the plan,
                                         // re-armed by the last wave of each decode launch)
constexpr int kPlanDoneInt = 12;         // header slot: workgroups of the fast decode launch that have finished
constexpr int kPlanPrefClaimInt = 13;    // header slot: claim counter of the prefill kernel (zeroed by the plan,
                                         // re-armed by the last workgroup of each prefill launch)
constexpr int kPlanPrefDoneInt = 14;     // header slot: workgroups of the prefill launch that have finished
constexpr int kMaxPartBuckets = 512;     // partition_size / 16 of the fast kernel, at most
constexpr int kPrefillKeys = 64;         // keys per prefill K/V tile

struct PlanArgs {
  const int32_t* cu_seqlens;
  const int32_t* seq_lens;
  int32_t* plan;
  int64_t pref_off_ints;   // prefill entries start at plan + kPlanHeaderInts + pref_off_ints
  int64_t merge_off_ints;  // merge list (request ids) starts at plan + kPlanHeaderInts + merge_off_ints
  int32_t num_seqs;
  int32_t part_size;       // decode partition size
  int32_t group;           // query heads per KV head
  int32_t decode;          // build the decode list
  int32_t prefill;         // build the prefill list
  int32_t max_query_len;   // requests beyond these bounds get no entries, so the
  int32_t max_seq_len;     // lists never outgrow the capacity the host sized
  // Multi-row requests with at most this many rows (0: none; at most one row
  // tile) get one prefill entry per context partition of part_size tokens when
  // they span more than one, and one merge entry per row.
  int32_t split_rows;
  int32_t tile_pairs;      // (query row, head) pairs per prefill list entry (32, 64 or 256)
  int32_t sliding_window;  // partitions wholly before a request's window get no entries
};
hipError_t launch_plan(const PlanArgs& a, hipStream_t stream);
// Bytes of a plan buffer for these capacities (entries), rounded to 256.
size_t plan_bytes(int64_t decode_capacity, int64_t prefill_capacity, int64_t merge_capacity);

// Fast single-row decode (bf16, D = 64 or 128, G in {1, 2, 4, 8}, blocks of 8,
// 16 or 32 tokens); partials by request.  Reads its work list from a.plan
// (built by launch_plan first).
bool decode_gqa_supported(int dtype, int head_dim, int group, int part_size, int block_size);
// Waves of the persistent fast decode kernel on the current device.
int decode_gqa_workers(int group);
// Work items per (KV head, partition) of the fast decode kernel: 1, or more
// where one item cannot hold all of a KV head's query heads.
int decode_gqa_head_split(int head_dim, int group);
// fp8_cache: the pools hold OCP FP8 E4M3 codes (scales folded into scale_log2 and lsum_scale).
// beside_prefill: a prefill launch runs at the same time on another stream;
// the kernel then uses workgroups of three workers (where no KV head is split
// over items) so a prefill workgroup fits beside each of them.
hipError_t launch_decode_gqa(int group, int head_dim, bool fp8_cache, const DecodeArgs& a, hipStream_t stream,
                             bool beside_prefill = false);
// Partition merge alone (for a DecodeArgs whose partials are already written).
hipError_t launch_merge(int dtype, int head_dim, const DecodeArgs& a, int64_t partial_rows, hipStream_t stream);
// Merge for the fast decode kernel's partials (bf16, D = 64 or 128): only the
// requests on the plan's merge list, one wave per (request, query head).
hipError_t launch_merge_list(int head_dim, const DecodeArgs& a, hipStream_t stream);
size_t decode_lds_bytes(int dtype, int head_dim, int group, int part_size);

// MFMA kernel for multi-row requests (bf16 q and out; bf16 or 8-bit pools; D = 64, 128 or 256; G a
// power of two up to 64, or at D = 128 also 3, 5 to 7 and 9 to 15 with padding head slots; blocks of
// 8, 16 or 32 tokens).
hipError_t launch_prefill(int head_dim, int group, bool fp8_cache, const PrefillArgs& a, hipStream_t stream);
bool prefill_supported(int head_dim, int group, int block_size);
// Query heads per prefill work item: the group, at most 8 (larger groups are
// served by several items per KV head; the work list's row tiles use this).
int prefill_item_group(int group);
// (query row, head) pairs per prefill list entry (row tile): 256 at D <= 128
// (64 at D = 256), or 64 (32) when every multi-row request is short.  A 256-pair
// entry is one item of an 8-wave workgroup when the prefill kernel runs alone,
// two items of a 4-wave workgroup beside the decode kernel (8-wave workgroups
// do not fit on a CU beside a decode workgroup).
int prefill_tile_pairs(int head_dim, bool short_rows);

hipError_t launch_validate(const int32_t* cu, const int32_t* seq_lens, const int32_t* bt, const int64_t* slots,
                           int64_t num_slots, int32_t num_seqs, int64_t total_q, int32_t max_query_len,
                           int32_t max_seq_len, int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size,
                           int32_t* result, hipStream_t stream);

}  // namespace pa
