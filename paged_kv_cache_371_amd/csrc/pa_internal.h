// Internal launch interface between the C ABI (pa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kDefaultPartition = 512;

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
  int32_t row_mode;         // which requests this launch serves (RowMode)
  int32_t partial_by_seq;   // 1: partials indexed by request, else by packed row
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
  int32_t m_tiles;        // query-row tiles per request = ceil(max_query_len / rows per tile)
  float scale_log2;
};

hipError_t launch_cache_write(const void* k_new, const void* v_new, int64_t kv_row_stride_bytes, void* k_cache,
                              void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_bytes, hipStream_t stream);

// dtype: 0 fp32, 1 bf16.  Returns hipErrorInvalidValue for shapes not built.
hipError_t launch_decode(int dtype, int head_dim, int group, const DecodeArgs& a, int64_t partial_rows,
                         hipStream_t stream);
bool decode_supported(int dtype, int head_dim, int group, int part_size);

// Fast single-row decode (bf16, D = 128, G in {1, 2, 4, 8}); partials by request.
// It needs decode_gqa_plan_bytes() of workspace for its work list (a.plan).
constexpr int kPlanHeaderInts = 64;      // claim counters, entry count, padding to 256 B
constexpr int kPlanCountInt = 8;         // header slot holding the number of list entries
constexpr int kMaxPartBuckets = 512;     // partition_size / 16 of the fast kernel, at most
bool decode_gqa_supported(int dtype, int head_dim, int group, int part_size);
size_t decode_gqa_plan_bytes(int64_t num_seqs, int64_t max_parts);
// Waves of the persistent fast decode kernel on the current device.
int decode_gqa_workers(int group);
hipError_t launch_decode_gqa(int group, const DecodeArgs& a, hipStream_t stream);
// Partition merge alone (for a DecodeArgs whose partials are already written).
hipError_t launch_merge(int dtype, int head_dim, const DecodeArgs& a, int64_t partial_rows, hipStream_t stream);
size_t decode_lds_bytes(int dtype, int head_dim, int group, int part_size);

hipError_t launch_prefill(int head_dim, int group, const PrefillArgs& a, hipStream_t stream);
bool prefill_supported(int head_dim, int group);
int prefill_rows_per_tile(int head_dim, int group);

hipError_t launch_validate(const int32_t* cu, const int32_t* seq_lens, const int32_t* bt, const int64_t* slots,
                           int64_t num_slots, int32_t num_seqs, int64_t total_q, int32_t max_query_len,
                           int32_t max_seq_len, int32_t max_blocks_per_seq, int64_t num_blocks, int32_t* result,
                           hipStream_t stream);

}  // namespace pa
