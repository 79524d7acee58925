// Work lists of the persistent attention kernels, built on the device from
// cu_seqlens and seq_lens so the host never reads request lengths.
//
// Layout of the plan buffer (int32 words):
//   [kPlanCountInt]      number of decode entries
//   [kPlanPrefCountInt]  number of prefill entries
//   [kPlanMergeCountInt] number of merge entries
//   [kPlanClaimInt]      claim counter of the decode kernel's dynamic rounds, zeroed here
//   [kPlanDoneInt]       finished workgroups of a decode launch, zeroed here (each launch's last one
//                        zeroes both again, so one list serves any number of launches)
//   [kPlanPrefClaimInt]  claim counter of the prefill kernel, zeroed here
//   [kPlanPrefDoneInt]   finished workgroups of a prefill launch, zeroed here (re-armed the same way)
//   [kPlanHeaderInts ..)                   decode entries, int4 (request, partition, query row, context length)
//   [kPlanHeaderInts + pref_off ..)        prefill entries, int4 (request, row tile | partition << 16,
//                                          first query row, query rows)
//   [kPlanHeaderInts + merge_off ..)       merge list, int4 (request, query row, partitions, partial row),
//                                          any order
//
// Decode list: one entry per non-empty context partition of every single-row
// request -- all full partitions first, then the partial last partitions by
// decreasing number of blocks.  Prefill list: one entry per tile of
// tile_pairs (query row, head) pairs of every multi-row request, by
// decreasing number of 64-key tiles the tile has to visit; a short request
// (at most split_rows rows) whose context spans several partitions instead
// gets one entry per partition, so no single work item has to stream a whole
// long context.  Both orders put the largest items first: the consumers deal
// or claim items in list order, and handing out the small ones last keeps the
// workers' finish times close.  Merge list: one entry per query row whose
// result is split over partitions -- single-row requests (partial row = the
// request) and rows of split short requests (partial row = num_seqs + row).
// Requests whose lengths break the bounds the host sized the buffer for get no
// entries (their output rows are left untouched).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPrefBuckets = 512;   // key-tile counts are clamped into this many buckets

// Exclusive positions of the buckets in decreasing bucket order, written over
// hist[0..n); returns base + the total.  n <= blockDim.x.  Each wave scans
// its 64 buckets with lane shuffles, one wave scans the wave totals.
__device__ int scan_desc(int* hist, int* tmp, int n, int base) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int x = tid < n ? hist[n - 1 - tid] : 0;
  int v = x;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) tmp[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < nw ? tmp[lane] : 0;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < nw) tmp[64 + lane] = t;
  }
  __syncthreads();
  const int before = w > 0 ? tmp[64 + w - 1] : 0;
  const int total = tmp[64 + nw - 1];
  if (tid < n) hist[n - 1 - tid] = base + before + v - x;
  __syncthreads();
  return base + total;
}

constexpr int kPlanThreads = 1024;
constexpr int kPerThread = 4;   // requests whose lengths a thread keeps in registers

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int s_hist[kPrefBuckets > kMaxPartBuckets ? kPrefBuckets : kMaxPartBuckets];
  __shared__ int s_tmp[kPrefBuckets > kMaxPartBuckets ? kPrefBuckets : kMaxPartBuckets];
  __shared__ int s_full;
  __shared__ int s_cursor;
  __shared__ int s_merge;
  const int tid = threadIdx.x;
  const int32_t* __restrict__ cu = a.cu_seqlens;
  const int32_t* __restrict__ seq_lens = a.seq_lens;

  // (first row, rows, context) of the first kPerThread requests of this
  // thread, read once; requests past kPerThread * kPlanThreads are re-read.
  int rq0[kPerThread], rn[kPerThread], rl[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int b = tid + k * kPlanThreads;
    rq0[k] = 0;
    rn[k] = 0;
    rl[k] = 0;
    if (b < a.num_seqs) {
      rq0[k] = cu[b];
      rn[k] = cu[b + 1] - rq0[k];
      rl[k] = seq_lens[b];
    }
  }
  auto for_each_request = [&](auto&& f) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int b = tid + k * kPlanThreads;
      if (b < a.num_seqs) f(b, rq0[k], rn[k], rl[k]);
    }
    for (int b = tid + kPerThread * kPlanThreads; b < a.num_seqs; b += kPlanThreads) {
      const int q0 = cu[b];
      f(b, q0, cu[b + 1] - q0, seq_lens[b]);
    }
  };

  if (tid == 0) s_merge = 0;
  if (a.decode) {
    const int P = a.part_size;
    const int nbk = P / kBlock;
    for (int i = tid; i < nbk; i += kPlanThreads) s_hist[i] = 0;
    if (tid == 0) {
      s_full = 0;
      s_cursor = 0;
    }
    __syncthreads();
    // Partitions [p_lo, p_end) of a request hold keys its row sees (a sliding
    // window drops the ones wholly before it); partitions p_lo+1 .. p_end-2 are
    // full, the first and the last are sized in blocks.
    auto blocks_of = [&](int L, int lo, int p) {
      return (min(L, (p + 1) * P) + kBlock - 1) / kBlock - max(p * P, lo) / kBlock;
    };
    for_each_request([&](int, int, int n, int L) {
      if (n != 1 || L > a.max_seq_len) return;
      const int lo = window_start(L - 1, a.sliding_window);
      const int p_lo = lo / P, np = (L + P - 1) / P - p_lo;
      int full = max(0, np - 2);
      for (int k = 0; k < min(np, 2); ++k) {   // the first and the last partition
        const int nb = blocks_of(L, lo, k ? p_lo + np - 1 : p_lo);
        if (nb == nbk) ++full; else atomicAdd(&s_hist[nb - 1], 1);
      }
      if (full) atomicAdd(&s_full, full);
    });
    __syncthreads();
    const int total = scan_desc(s_hist, s_tmp, nbk, s_full);
    if (tid == 0) a.plan[kPlanCountInt] = total;
    int4* entries = reinterpret_cast<int4*>(a.plan + kPlanHeaderInts);
    int4* merge = reinterpret_cast<int4*>(a.plan + kPlanHeaderInts + a.merge_off_ints);
    for_each_request([&](int b, int q0, int n, int L) {
      if (n != 1 || L > a.max_seq_len) return;
      const int lo = window_start(L - 1, a.sliding_window);
      const int p_lo = lo / P, p_end = (L + P - 1) / P;
      int nfull = 0;
      for (int p = p_lo; p < p_end; ++p) nfull += blocks_of(L, lo, p) == nbk;
      int pos = nfull ? atomicAdd(&s_cursor, nfull) : 0;
      for (int p = p_lo; p < p_end; ++p) {
        const int nb = blocks_of(L, lo, p);
        entries[nb == nbk ? pos++ : atomicAdd(&s_hist[nb - 1], 1)] = make_int4(b, p, q0, L);
      }
      if (p_end - p_lo > 1) merge[atomicAdd(&s_merge, 1)] = make_int4(b, q0, p_end - p_lo, b);
    });
    __syncthreads();
    if (tid == 0) {
      a.plan[kPlanClaimInt] = 0;
      a.plan[kPlanDoneInt] = 0;
    }
  }

  if (a.prefill) {
    const int rows = a.tile_pairs / a.group;   // query rows per tile
    for (int i = tid; i < kPrefBuckets; i += kPlanThreads) s_hist[i] = 0;
    __syncthreads();
    // key tiles (64 keys) in [k0, k1), clamped into the buckets
    auto tiles = [&](int k0, int k1) {
      return min((k1 + kPrefillKeys - 1) / kPrefillKeys - k0 / kPrefillKeys, kPrefBuckets - 1);
    };
    // bucket of row tile mt: the keys its rows see, from its first row's
    // window start to its last row's position
    auto bucket = [&](int L, int n, int mt) {
      const int last = min(n, (mt + 1) * rows);   // rows [mt*rows, last)
      return tiles(window_start(L - n + mt * rows, a.sliding_window), L - n + last);
    };
    auto usable = [&](int n, int L) { return n >= 2 && n <= a.max_query_len && L >= n && L <= a.max_seq_len; };
    // A short request is split over partitions [p_lo, p_end) of P tokens when
    // its rows' keys span more than one (p_lo: the partition of its first
    // row's window start).
    const int P = a.part_size;
    auto first_part = [&](int n, int L) { return window_start(L - n, a.sliding_window) / P; };
    auto split_parts = [&](int n, int L) { return n <= a.split_rows ? (L + P - 1) / P - first_part(n, L) : 1; };
    auto part_bucket = [&](int n, int L, int p) {
      return tiles(max(p * P, window_start(L - n, a.sliding_window)), min(L, (p + 1) * P));
    };
    for_each_request([&](int, int, int n, int L) {
      if (!usable(n, L)) return;
      const int parts = split_parts(n, L);
      if (parts > 1) {
        const int p_lo = first_part(n, L);
        for (int p = p_lo; p < p_lo + parts; ++p) atomicAdd(&s_hist[part_bucket(n, L, p)], 1);
      } else {
        for (int mt = 0; mt * rows < n; ++mt) atomicAdd(&s_hist[bucket(L, n, mt)], 1);
      }
    });
    __syncthreads();
    const int total = scan_desc(s_hist, s_tmp, kPrefBuckets, 0);
    if (tid == 0) {
      a.plan[kPlanPrefCountInt] = total;
      a.plan[kPlanPrefClaimInt] = 0;
      a.plan[kPlanPrefDoneInt] = 0;
    }
    int4* entries = reinterpret_cast<int4*>(a.plan + kPlanHeaderInts + a.pref_off_ints);
    int4* merge = reinterpret_cast<int4*>(a.plan + kPlanHeaderInts + a.merge_off_ints);
    for_each_request([&](int b, int q0, int n, int L) {
      if (!usable(n, L)) return;
      const int parts = split_parts(n, L);
      if (parts > 1) {
        const int p_lo = first_part(n, L);
        for (int p = p_lo; p < p_lo + parts; ++p)
          entries[atomicAdd(&s_hist[part_bucket(n, L, p)], 1)] = make_int4(b, p << 16, q0, n);
        const int m0 = atomicAdd(&s_merge, n);
        for (int j = 0; j < n; ++j) merge[m0 + j] = make_int4(b, q0 + j, parts, a.num_seqs + q0 + j);
      } else {
        for (int mt = 0; mt * rows < n; ++mt)
          entries[atomicAdd(&s_hist[bucket(L, n, mt)], 1)] = make_int4(b, mt, q0, n);
      }
    });
  }
  __syncthreads();
  if (tid == 0) {
    a.plan[kPlanMergeCountInt] = s_merge;
    // a list this call does not build is empty, with its counters at rest
    if (!a.decode) {
      a.plan[kPlanCountInt] = 0;
      a.plan[kPlanClaimInt] = 0;
      a.plan[kPlanDoneInt] = 0;
    }
    if (!a.prefill) {
      a.plan[kPlanPrefCountInt] = 0;
      a.plan[kPlanPrefClaimInt] = 0;
      a.plan[kPlanPrefDoneInt] = 0;
    }
  }
}

}  // namespace

size_t plan_bytes(int64_t decode_capacity, int64_t prefill_capacity, int64_t merge_capacity) {
  const size_t ints = size_t(kPlanHeaderInts) + 4 * size_t(decode_capacity) + 4 * size_t(prefill_capacity) +
                      4 * size_t(merge_capacity);
  return (ints * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
