// C ABI of the paged-attention library: argument checks, kernel choice,
// grid and workspace sizing, launch on the caller's stream.  See include/pa.h
// for the contract of each entry point.
#include "../../include/pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <mutex>

#include "pa_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }

inline bool dtype_ok(pa_dtype d) { return d == PA_F32 || d == PA_BF16; }

// Block sizes built: 16 (the pages' default; every kernel) and 8 and 32 (the
// cache writes and the generic decode kernel).
inline bool block_size_ok(int32_t bs) { return bs == 8 || bs == 16 || bs == 32; }

// Tokens per split-K partition.  An explicit partition_size is used as given;
// then a request's result depends only on the request itself (bitwise the
// same in any batch).  The default (0) picks, for the fast decode kernel, the
// largest of 2048 / 1024 / 512 tokens that still gives every wave of the
// persistent grid 4 work items by the host's upper bound
// B * Hkv * S * ceil(max_seq_len / P) (S: work items per KV head, 1 unless a
// KV head has more query heads than one item holds): long partitions cost less per token (one
// merge per partition), but too few of them leave waves idle.  The bound
// counts every request at the longest length, so it overstates the items of
// batches with short requests.  Measured on one MI355X: the MHA decode layer
// (contexts 128..2048) takes 1024 with 4 items a wave, 191.7 us against 199.7
// with 2048 (2 a wave) and 203.2 with 512 (8 a wave); the GQA decode layer,
// the mixed chunked-prefill step and the other workloads keep 2048.
inline int effective_partition(const pa_attn_params* p) {
  if (p->partition_size > 0) return p->partition_size;
  const int g = p->num_kv_heads > 0 ? p->num_q_heads / p->num_kv_heads : 0;
  const int dt = p->dtype == PA_BF16 ? 1 : 0;
  if (!pa::decode_gqa_supported(dt, p->head_dim, g, pa::kDefaultPartition, p->block_size))
    return pa::kDefaultPartition;
  // Multi-row requests that the MFMA kernel does not take run on the generic
  // kernel, whose per-workgroup scores of one partition must fit its LDS.
  const bool generic_rows =
      p->max_query_len > 1 && !(dt == 1 && pa::prefill_supported(p->head_dim, g, p->block_size));
  const int64_t want = int64_t(4) * pa::decode_gqa_workers(g);
  for (int ps : {2048, 1024}) {
    const int64_t items = int64_t(p->num_seqs) * p->num_kv_heads * pa::decode_gqa_head_split(p->head_dim, g) *
                          ((int64_t(p->max_seq_len) + ps - 1) / ps);
    if (items >= want && (!generic_rows || pa::decode_supported(dt, p->head_dim, g, ps))) return ps;
  }
  return pa::kDefaultPartition;
}

// How one call is split between the kernels.  Single-row (decode) requests
// take the fast bf16 kernel when it is built for (D, G); in bf16, requests
// with more rows take the MFMA prefill kernel when it is built for (D, G).
// The generic decode kernel serves whatever is left.  Split-K partials live
// in two workspace regions: A, indexed by request (single-row requests), and
// B, indexed by packed row (requests the generic kernel serves row by row).
struct Plan {
  bool ok;            // every kernel the call needs is built for these parameters
  bool fast;          // fast single-row kernel
  bool prefill;       // MFMA prefill kernel for multi-row requests
  int generic_mode;   // -1: generic kernel not launched, else its pa::RowMode
  bool generic_by_seq;
  int64_t parts;      // partitions per request, upper bound
  int64_t rows_a;     // partial rows in region A
  int64_t rows_b;     // partial rows in region B
  int32_t split_rows; // short multi-row requests split over partitions (0: none)
  int32_t tile_pairs; // (row, head) pairs per prefill work item
};

inline int64_t max_parts(const pa_attn_params* p) {
  const int ps = effective_partition(p);
  return p->max_seq_len > 0 ? (int64_t(p->max_seq_len) + ps - 1) / ps : 1;
}

inline Plan make_plan(const pa_attn_params* p) {
  Plan pl{};
  const int dt = p->dtype == PA_BF16 ? 1 : 0;
  const int g = p->num_q_heads / p->num_kv_heads;
  const bool multi = p->max_query_len > 1;
  const int ps = effective_partition(p);
  pl.fast = pa::decode_gqa_supported(dt, p->head_dim, g, ps, p->block_size);
  pl.prefill = dt == 1 && multi && pa::prefill_supported(p->head_dim, g, p->block_size);
  pl.parts = max_parts(p);
  // Batches whose multi-row requests all fit one half-size tile (64 / G rows;
  // 32 / G at D = 256) use half-size prefill tiles; such short requests (one
  // row tile) are split over context partitions when the partition is a
  // whole number of prefill key tiles.
  // Full tiles at D <= 128 hold 256 pairs: alone on the GPU an 8-wave
  // workgroup serves one; beside the decode kernel (a mixed step with the
  // num_decode_rows hint) a 4-wave workgroup serves each half.  Each wave
  // computes the same pairs the same way in both, and the split rule counts
  // 128-pair tiles either way, so the hint changes neither the lists nor a bit.
  const int gp = pa::prefill_item_group(g);   // query heads per prefill work item
  const bool short_rows = p->max_query_len <= pa::prefill_tile_pairs(p->head_dim, true) / gp;
  const int split_pairs = short_rows ? pa::prefill_tile_pairs(p->head_dim, true) : (p->head_dim == 256 ? 64 : 128);
  pl.tile_pairs = pa::prefill_tile_pairs(p->head_dim, short_rows);
  pl.split_rows = (pl.fast && pl.prefill && pl.parts > 1 && ps % pa::kPrefillKeys == 0 &&
                   p->max_query_len <= split_pairs / gp)
                      ? split_pairs / gp
                      : 0;
  if (pl.fast) {
    pl.generic_mode = (multi && !pl.prefill) ? pa::kMultiRowOnly : -1;
    pl.generic_by_seq = false;
  } else if (pl.prefill) {
    pl.generic_mode = pa::kSingleRowOnly;
    pl.generic_by_seq = true;
  } else {
    pl.generic_mode = pa::kAllRows;
    pl.generic_by_seq = false;
  }
  pl.ok = pl.generic_mode < 0 || pa::decode_supported(dt, p->head_dim, g, ps);
  if (pl.parts > 1) {
    const bool a_used = pl.fast || (pl.generic_mode >= 0 && pl.generic_by_seq);
    const bool b_used = pl.generic_mode >= 0 && !pl.generic_by_seq;
    pl.rows_a = a_used ? p->num_seqs + (pl.split_rows ? p->total_q : 0) : 0;
    pl.rows_b = b_used ? p->total_q : 0;
  }
  return pl;
}

inline size_t region_floats(const pa_attn_params* p, int64_t rows, int64_t parts) {
  return size_t(rows) * p->num_q_heads * parts * (p->head_dim + 2);
}

// Entries the prefill work list can hold: tiles of pl.tile_pairs (row, head)
// pairs, or one per partition of a split short request.
inline int64_t prefill_capacity(const pa_attn_params* p, const Plan& pl) {
  const int64_t rows = pl.tile_pairs / pa::prefill_item_group(p->num_q_heads / p->num_kv_heads);
  const int64_t per_seq = (int64_t(p->max_query_len) + rows - 1) / rows;
  return int64_t(p->num_seqs) * (pl.split_rows ? std::max<int64_t>(per_seq, pl.parts) : per_seq);
}
inline int64_t decode_capacity(const pa_attn_params* p, const Plan& pl) { return int64_t(p->num_seqs) * pl.parts; }
// Merge entries: single-row requests, plus the rows of split short requests.
inline int64_t merge_capacity(const pa_attn_params* p, const Plan& pl) {
  return pl.fast ? int64_t(p->num_seqs) + (pl.split_rows ? p->total_q : 0) : 0;
}

// Workspace: [work lists of the persistent kernels][region A][region B].
inline size_t plan_bytes(const pa_attn_params* p, const Plan& pl) {
  if (!pl.fast && !pl.prefill) return 0;
  return pa::plan_bytes(pl.fast ? decode_capacity(p, pl) : 0, pl.prefill ? prefill_capacity(p, pl) : 0,
                        merge_capacity(p, pl));
}
// Offsets (ints after the header) of the prefill entries and the merge list.
inline int64_t pref_off(const pa_attn_params* p, const Plan& pl) { return pl.fast ? 4 * decode_capacity(p, pl) : 0; }
inline int64_t merge_off(const pa_attn_params* p, const Plan& pl) {
  return pref_off(p, pl) + (pl.prefill ? 4 * prefill_capacity(p, pl) : 0);
}

// Limits of the kernels' index arithmetic: a request's partition count sits
// in the upper 16 bits of a signed int (count << 16) and a prefill entry's
// row tile in the lower 16 bits; work items are indexed as int (list entries
// x head groups).
inline bool plan_fits(const pa_attn_params* p, const Plan& pl) {
  const int g = p->num_q_heads / p->num_kv_heads;
  if (pl.parts > 32767) return false;
  if (int64_t(p->num_seqs) * pl.parts * p->num_kv_heads * pa::decode_gqa_head_split(p->head_dim, g) > INT32_MAX)
    return false;
  if (pl.prefill) {
    const int gp = pa::prefill_item_group(g);
    const int64_t rows = pl.tile_pairs / gp;
    if ((int64_t(p->max_query_len) + rows - 1) / rows > 65535) return false;
    // items: entries x KV heads x head groups, x 2 where 4-wave workgroups serve halves of entries
    if (prefill_capacity(p, pl) * p->num_kv_heads * ((g + gp - 1) / gp) * 2 > INT32_MAX) return false;
  }
  return true;
}

pa_status check_params(const pa_attn_params* p) {
  if (!p) return PA_ERR_NULL;
  if (!dtype_ok(p->dtype)) return PA_ERR_UNSUPPORTED;
  if (!block_size_ok(p->block_size)) return PA_ERR_UNSUPPORTED;
  if (p->num_seqs < 0 || p->total_q < 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 ||
      p->num_blocks <= 0 || p->max_blocks_per_seq <= 0 || p->max_query_len < 0 || p->max_seq_len < 0)
    return PA_ERR_SHAPE;
  if (p->num_q_heads % p->num_kv_heads) return PA_ERR_SHAPE;
  if (p->num_seqs > 65535) return PA_ERR_SHAPE;
  if (p->max_query_len > p->max_seq_len) return PA_ERR_SHAPE;
  if (int64_t(p->max_blocks_per_seq) * p->block_size < p->max_seq_len) return PA_ERR_SHAPE;
  if (p->total_q > 0 && p->num_seqs == 0) return PA_ERR_SHAPE;
  const int64_t hd = int64_t(p->num_q_heads) * p->head_dim;
  if (p->q_row_stride < hd || p->o_row_stride < hd) return PA_ERR_SHAPE;
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return PA_ERR_SHAPE;
  if (p->partition_size != 0 && (p->partition_size < 16 || p->partition_size > 8192 || p->partition_size % 16))
    return PA_ERR_SHAPE;
  if (p->sliding_window < 0 || p->num_decode_rows < 0) return PA_ERR_SHAPE;
  const int eb = elem_bytes(p->dtype);
  if ((p->q_row_stride * eb) % 16 || (p->o_row_stride * eb) % 16) return PA_ERR_ALIGN;
  return PA_OK;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return 208; }

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size is out of range or inconsistent";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: dtype, head_dim, group size or block size not built";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: pointer or row stride not 16-byte aligned";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: kernel launch failed";
    case PA_ERR_METADATA: return "PA_ERR_METADATA: device metadata failed validation";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks (nothing changed)";
    case PA_ERR_STATE: return "PA_ERR_STATE: unknown, existing or swapped-out sequence";
    case PA_ERR_HOST_MEMORY: return "PA_ERR_HOST_MEMORY: host allocation failed";
  }
  return "unknown pa_status";
}

pa_status pa_cache_write(const void* k_new, const void* v_new, int64_t kv_row_stride, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int64_t num_blocks, pa_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (kv_row_stride < int64_t(num_kv_heads) * head_dim) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (kv_row_stride * eb) % 16)
    return PA_ERR_ALIGN;
  hipError_t e = pa::launch_cache_write(k_new, v_new, kv_row_stride * eb, k_cache, v_cache, slot_mapping, num_tokens,
                                        num_kv_heads, head_dim * eb, block_size, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

size_t pa_attention_workspace_size(const pa_attn_params* p) {
  if (check_params(p) != PA_OK) return 0;
  const Plan pl = make_plan(p);
  if (!pl.ok || !plan_fits(p, pl)) return 0;
  return plan_bytes(p, pl) +
         (region_floats(p, pl.rows_a, pl.parts) + region_floats(p, pl.rows_b, pl.parts)) * sizeof(float);
}

int32_t pa_attention_partition_size(const pa_attn_params* p) {
  if (check_params(p) != PA_OK) return 0;
  return effective_partition(p);
}

namespace {

// Stages of an attention call: the work lists (from the request lengths
// only, shared by every layer of a step) and the attention proper.
enum Stage : int { kPlanStage = 1, kRunStage = 2 };

// Every attention entry point.  fp8: the pools hold OCP FP8 E4M3 codes with
// per-tensor scales (decode rows only; q and out are bf16).
// The second stream of a run whose batch has both single-row and multi-row
// requests: the prefill kernel runs on it while the decode kernel runs on the
// caller's stream, so the decode kernel's HBM streaming and the prefill
// kernel's matrix-core work share the CUs ([ICE]: one forward over the packed
// decode and prefill rows of a step; prefill is compute-bound, decode
// bandwidth-bound).  One stream (default priority) and two events per device,
// created on first use; the lock is held over the short enqueue-only
// sequence, so the events' records and waits of two host threads never mix.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr;
  hipEvent_t join = nullptr;
  bool ready = false;
};
constexpr int kSideDevices = 64;
std::mutex g_side_mu[kSideDevices];
SideStream g_side[kSideDevices];

// The current device's side stream and its lock, or nullptr if there is none
// (the run then launches everything on the caller's stream).
SideStream* side_of_current_device(std::mutex** mu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kSideDevices) return nullptr;
  *mu = &g_side_mu[dev];
  SideStream& ss = g_side[dev];
  std::lock_guard<std::mutex> lock(g_side_mu[dev]);
  if (!ss.ready) {
    if (hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(ss.stream);
      ss.stream = nullptr;
      return nullptr;
    }
    ss.ready = true;
  }
  return &ss;
}

pa_status attention_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cu_seqlens_q, const int32_t* seq_lens, const int32_t* block_tables,
                         const pa_attn_params* p, void* workspace, size_t workspace_bytes, void* stream, bool fp8,
                         float k_scale, float v_scale, int stages) {
  pa_status st = check_params(p);
  if (st != PA_OK) return st;
  if (fp8) {
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
      return PA_ERR_SHAPE;
    const int g8 = p->num_q_heads / p->num_kv_heads;
    if (p->dtype != PA_BF16 ||
        !pa::decode_gqa_supported(1, p->head_dim, g8, effective_partition(p), p->block_size) ||
        (p->max_query_len > 1 && !pa::prefill_supported(p->head_dim, g8, p->block_size)))
      return PA_ERR_UNSUPPORTED;
  }
  if (p->num_seqs == 0 || p->total_q == 0) return PA_OK;
  if (!cu_seqlens_q || !seq_lens) return PA_ERR_NULL;
  if (stages & kRunStage) {
    if (!out || !q || !k_cache || !v_cache || !block_tables) return PA_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_ALIGN;
  }
  const size_t need = pa_attention_workspace_size(p);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return PA_ERR_ALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = p->dtype == PA_BF16 ? 1 : 0;
  const int g = p->num_q_heads / p->num_kv_heads;
  const Plan pl = make_plan(p);
  if (!pl.ok) return PA_ERR_UNSUPPORTED;
  if (!plan_fits(p, pl)) return PA_ERR_SHAPE;
  const float scale_log2 = p->scale * kLog2e * (fp8 ? k_scale : 1.f);
  const size_t pbytes = plan_bytes(p, pl);
  float* ws = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + pbytes) : nullptr;
  float* region_a = ws;
  float* region_b = ws ? ws + region_floats(p, pl.rows_a, pl.parts) : nullptr;

  pa::DecodeArgs d{};
  d.out = out;
  d.q = q;
  d.k_cache = k_cache;
  d.v_cache = v_cache;
  d.cu_seqlens = cu_seqlens_q;
  d.seq_lens = seq_lens;
  d.block_tables = block_tables;
  d.q_row_stride = p->q_row_stride;
  d.o_row_stride = p->o_row_stride;
  d.num_seqs = p->num_seqs;
  d.num_q_heads = p->num_q_heads;
  d.num_kv_heads = p->num_kv_heads;
  d.max_blocks_per_seq = p->max_blocks_per_seq;
  d.part_size = effective_partition(p);
  d.max_parts = int32_t(pl.parts);
  d.scale_log2 = scale_log2;
  d.lsum_scale = fp8 ? 1.f / v_scale : 1.f;
  d.plan = (pl.fast || pl.prefill) ? static_cast<int32_t*>(workspace) : nullptr;
  d.merge_off_ints = merge_off(p, pl);
  d.plan_capacity = int32_t(std::max<int64_t>(1, pl.fast ? decode_capacity(p, pl) : 1));
  d.merge_capacity = int32_t(merge_capacity(p, pl));
  d.sliding_window = p->sliding_window;
  d.block_size = p->block_size;

  // Partials of a region: o [rows, Hq, parts, D] followed by (m, l) [rows, Hq, parts, 2].
  auto point_at = [&](float* region, int64_t rows) {
    d.ws_o = region;
    d.ws_ml = region ? region + int64_t(rows) * p->num_q_heads * pl.parts * p->head_dim : nullptr;
  };

  hipError_t e = hipSuccess;
  if ((stages & kPlanStage) && (pl.fast || pl.prefill)) {
    pa::PlanArgs pa_{};
    pa_.cu_seqlens = cu_seqlens_q;
    pa_.seq_lens = seq_lens;
    pa_.plan = static_cast<int32_t*>(workspace);
    pa_.pref_off_ints = pref_off(p, pl);
    pa_.merge_off_ints = merge_off(p, pl);
    pa_.num_seqs = p->num_seqs;
    pa_.part_size = d.part_size;
    pa_.group = pa::prefill_item_group(g);
    pa_.decode = pl.fast ? 1 : 0;
    pa_.prefill = pl.prefill ? 1 : 0;
    pa_.max_query_len = p->max_query_len;
    pa_.max_seq_len = p->max_seq_len;
    pa_.split_rows = pl.split_rows;
    pa_.tile_pairs = pl.tile_pairs;
    pa_.sliding_window = p->sliding_window;
    if (pa::launch_plan(pa_, s) != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (!(stages & kRunStage)) return PA_OK;
  // Fork: the decode kernel goes first on the caller's stream, the prefill
  // kernel on the side stream from the same point; the partial-output regions
  // and output rows of the two are disjoint, and the merge waits for both.
  std::mutex* side_mu = nullptr;
  SideStream* side = (pl.fast && pl.prefill && pl.generic_mode < 0 && p->num_decode_rows > 0)
                         ? side_of_current_device(&side_mu)
                         : nullptr;
  std::unique_lock<std::mutex> side_lock;
  if (side) {
    side_lock = std::unique_lock<std::mutex>(*side_mu);
    if (hipEventRecord(side->fork, s) != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (pl.fast) {
    point_at(region_a, pl.rows_a);
    d.row_mode = pa::kSingleRowOnly;
    d.partial_by_seq = 1;
    e = pa::launch_decode_gqa(g, p->head_dim, fp8, d, s, side != nullptr);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (side && hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess) return PA_ERR_LAUNCH;
  if (pl.generic_mode >= 0) {
    point_at(pl.generic_by_seq ? region_a : region_b, pl.generic_by_seq ? pl.rows_a : pl.rows_b);
    d.row_mode = pl.generic_mode;
    d.partial_by_seq = pl.generic_by_seq ? 1 : 0;
    e = pa::launch_decode(dt, p->head_dim, g, d, pl.generic_by_seq ? pl.rows_a : pl.rows_b, s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  if (pl.prefill) {
    pa::PrefillArgs f{};
    f.out = out;
    f.q = q;
    f.k_cache = k_cache;
    f.v_cache = v_cache;
    f.cu_seqlens = cu_seqlens_q;
    f.seq_lens = seq_lens;
    f.block_tables = block_tables;
    f.q_row_stride = p->q_row_stride;
    f.o_row_stride = p->o_row_stride;
    f.num_seqs = p->num_seqs;
    f.num_q_heads = p->num_q_heads;
    f.num_kv_heads = p->num_kv_heads;
    f.max_blocks_per_seq = p->max_blocks_per_seq;
    f.plan = static_cast<int32_t*>(workspace);
    f.pref_off_ints = pref_off(p, pl);
    f.scale_log2 = scale_log2;
    f.split_rows = pl.split_rows;
    f.tile_pairs = pl.tile_pairs;
    f.sliding_window = p->sliding_window;
    f.block_size = p->block_size;
    f.part_size = d.part_size;
    f.max_parts = d.max_parts;
    f.ws_o = pl.split_rows ? region_a : nullptr;
    f.ws_ml = pl.split_rows ? region_a + int64_t(pl.rows_a) * p->num_q_heads * pl.parts * p->head_dim : nullptr;
    f.lsum_scale = d.lsum_scale;
    f.claim_items = side ? 1 : 0;
    e = pa::launch_prefill(p->head_dim, g, fp8, f, side ? side->stream : s);
    if (e != hipSuccess) return PA_ERR_LAUNCH;
  }
  // Join: the caller's stream waits for the prefill kernel.
  if (side && (hipEventRecord(side->join, side->stream) != hipSuccess ||
               hipStreamWaitEvent(s, side->join, 0) != hipSuccess))
    return PA_ERR_LAUNCH;
  if (side) side_lock.unlock();
  // partitions of single-row requests and of split short requests
  if (pl.fast && pl.parts > 1) {
    point_at(region_a, pl.rows_a);
    if (pa::launch_merge_list(p->head_dim, d, s) != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

// Scratch of pa_attention_varlen_noalloc: one copy per GPU, in the code
// object's static device memory, held until the process ends.  Host code
// never uses the array's name as an address (on the host it is a stand-in
// for the symbol); it uses the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kScratchDevices];

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept; nullptr if the lookup fails.
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    g_scratch_ptr[dev].store(addr, std::memory_order_release);
    ptr = addr;
  }
  return ptr;
}

}  // namespace

pa_status pa_attention_varlen_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* cu_seqlens_q, const int32_t* seq_lens,
                                      const int32_t* block_tables, const pa_attn_params* p, void* stream) {
  pa_status st = check_params(p);
  if (st != PA_OK) return st;
  const size_t need = pa_attention_workspace_size(p);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  if (p->num_seqs == 0 || p->total_q == 0) return PA_OK;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_of_current_device();
    if (!ws) return PA_ERR_LAUNCH;
  }
  // The plan stage rewrites the work lists and re-arms their counters at the
  // start of the scratch; the partials behind them are written before they
  // are read, so nothing left by an earlier call needs clearing.
  return attention_impl(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, p, ws,
                        ws ? size_t(PA_NOALLOC_SCRATCH_BYTES) : 0, stream, false, 1.f, 1.f, kPlanStage | kRunStage);
}

pa_status pa_attention_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cu_seqlens_q, const int32_t* seq_lens, const int32_t* block_tables,
                              const pa_attn_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, p, workspace, workspace_bytes,
                        stream, false, 1.f, 1.f, kPlanStage | kRunStage);
}

pa_status pa_attention_plan(const int32_t* cu_seqlens_q, const int32_t* seq_lens, const pa_attn_params* p,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(nullptr, nullptr, nullptr, nullptr, cu_seqlens_q, seq_lens, nullptr, p, workspace,
                        workspace_bytes, stream, false, 1.f, 1.f, kPlanStage);
}

pa_status pa_attention_run(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* cu_seqlens_q, const int32_t* seq_lens, const int32_t* block_tables,
                           const pa_attn_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, p, workspace, workspace_bytes,
                        stream, false, 1.f, 1.f, kRunStage);
}

pa_status pa_attention_varlen_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* cu_seqlens_q, const int32_t* seq_lens, const int32_t* block_tables,
                                  const pa_attn_params* p, float k_scale, float v_scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, p, workspace, workspace_bytes,
                        stream, true, k_scale, v_scale, kPlanStage | kRunStage);
}

pa_status pa_attention_run_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens_q, const int32_t* seq_lens, const int32_t* block_tables,
                               const pa_attn_params* p, float k_scale, float v_scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return attention_impl(out, q, k_cache, v_cache, cu_seqlens_q, seq_lens, block_tables, p, workspace, workspace_bytes,
                        stream, true, k_scale, v_scale, kRunStage);
}

pa_status pa_cache_write_fp8(const void* k_new, const void* v_new, int64_t kv_row_stride, void* k_cache,
                             void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, float k_scale, float v_scale,
                             void* stream) {
  if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (kv_row_stride < int64_t(num_kv_heads) * head_dim) return PA_ERR_SHAPE;
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) || (kv_row_stride * 2) % 16)
    return PA_ERR_ALIGN;
  hipError_t e = pa::launch_cache_write_fp8(k_new, v_new, kv_row_stride * 2, k_cache, v_cache, slot_mapping, num_tokens,
                                            num_kv_heads, head_dim, block_size, k_scale, v_scale,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

pa_status pa_validate_metadata(const int32_t* cu_seqlens_q, const int32_t* seq_lens, const int32_t* block_tables,
                               const int64_t* slot_mapping, int64_t num_slots, const pa_attn_params* p,
                               int32_t* result, void* stream) {
  if (!p || !result) return PA_ERR_NULL;
  if (!block_size_ok(p->block_size)) return PA_ERR_UNSUPPORTED;
  if (p->num_seqs < 0 || p->total_q < 0 || p->num_blocks <= 0 || p->max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (p->num_seqs > 0 && (!cu_seqlens_q || !seq_lens || !block_tables)) return PA_ERR_NULL;
  if (!slot_mapping) num_slots = 0;
  if (num_slots < 0) return PA_ERR_SHAPE;
  hipError_t e = pa::launch_validate(cu_seqlens_q, seq_lens, block_tables, slot_mapping, num_slots, p->num_seqs,
                                     p->total_q, p->max_query_len, p->max_seq_len, p->max_blocks_per_seq,
                                     p->num_blocks, p->block_size, result, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
