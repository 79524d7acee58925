// Whole-block copies: copy-on-write inside a pool and swap between pools.
//
// quant67, "PagedAttention 与 Continuous Batching" §3.8: a sample that must
// write into a shared block first copies that block to a fresh one; §3.9:
// preemption by swap moves a sequence's blocks to host memory and back.
// Both are the same operation -- block dst of one pool receives block src of
// another (or the same) pool, in K and in V -- over a list of (src, dst)
// pairs.  One launch covers every pair, so the per-block cost is bytes, not
// launches: a COW step copies one 32 KiB block per sample and a swap moves
// hundreds of blocks at once.
//
// Work item = (pair, pool, 16 KiB chunk of the block).  A workgroup of 256
// threads moves one item: four 16-byte loads per thread, all issued before
// the first store, so each wave keeps 4 KiB in flight.  Items of one pair
// are consecutive, so consecutive workgroups (which land on different XCDs)
// stream adjacent bytes.  Pinned host pools are read or written by the same
// loads and stores over the host link.
#include <climits>

#include "../../include/pa_blocks.h"
#include "pa_common.h"

namespace pa {

namespace {
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int64_t kCopyChunkVecs = int64_t(kCopyThreads) * kCopyUnroll;   // 16-byte vectors per item
constexpr int64_t kStreamingBytes = int64_t(256) << 20;                   // bytes read per call
}  // namespace

template <bool Streaming>
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char* __restrict__ dst_k, char* __restrict__ dst_v, const char* __restrict__ src_k,
    const char* __restrict__ src_v, const int64_t* __restrict__ mapping, int64_t block_bytes, int64_t src_blocks,
    int64_t dst_blocks, int64_t chunks, int64_t items) {
  const int64_t block_vecs = block_bytes >> 4;
  for (int64_t w = blockIdx.x; w < items; w += gridDim.x) {
    const int64_t pp = w / chunks;
    const int64_t chunk = w - pp * chunks;
    const int64_t pair = pp >> 1;
    const bool is_v = (pp & 1) != 0;
    const int64_t src = mapping[2 * pair];
    const int64_t dst = mapping[2 * pair + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
    const u32x4_t* s = reinterpret_cast<const u32x4_t*>((is_v ? src_v : src_k) + src * block_bytes);
    u32x4_t* d = reinterpret_cast<u32x4_t*>((is_v ? dst_v : dst_k) + dst * block_bytes);
    const int64_t base = chunk * kCopyChunkVecs;
    u32x4_t r[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * kCopyThreads + threadIdx.x;
      if (i < block_vecs) r[u] = Streaming ? __builtin_nontemporal_load(s + i) : s[i];
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * kCopyThreads + threadIdx.x;
      if (i < block_vecs) {
        if (Streaming)
          __builtin_nontemporal_store(r[u], d + i);
        else
          d[i] = r[u];
      }
    }
  }
}

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int64_t* mapping, int64_t num_pairs, int64_t block_bytes, int64_t src_blocks,
                              int64_t dst_blocks, hipStream_t stream) {
  const int64_t chunks = ((block_bytes >> 4) + kCopyChunkVecs - 1) / kCopyChunkVecs;
  const int64_t items = num_pairs * 2 * chunks;
  const int64_t grid = items < (int64_t(1) << 20) ? items : (int64_t(1) << 20);
  // Copies larger than the last-level cache stream past it (non-temporal
  // loads and stores, about 5% faster there); smaller ones keep the copied
  // blocks cached for the cache write and attention that follow.
  if (num_pairs * 2 * block_bytes >= kStreamingBytes)
    hipLaunchKernelGGL(copy_blocks_kernel<true>, dim3(unsigned(grid)), dim3(kCopyThreads), 0, stream,
                       static_cast<char*>(dst_k), static_cast<char*>(dst_v), static_cast<const char*>(src_k),
                       static_cast<const char*>(src_v), mapping, block_bytes, src_blocks, dst_blocks, chunks, items);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<false>, dim3(unsigned(grid)), dim3(kCopyThreads), 0, stream,
                       static_cast<char*>(dst_k), static_cast<char*>(dst_v), static_cast<const char*>(src_k),
                       static_cast<const char*>(src_v), mapping, block_bytes, src_blocks, dst_blocks, chunks, items);
  return hipGetLastError();
}

}  // namespace pa

// ---- C ABI (include/pa_blocks.h) -------------------------------------------------

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Address the device uses for p: device memory as is, pinned host memory
// where it is mapped at its host address.  Pageable host memory (which a
// kernel cannot reach) is refused.
pa_status device_address(const void* p, const void** out) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_UNSUPPORTED;
  }
  switch (attr.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      *out = p;
      return PA_OK;
    case hipMemoryTypeHost:
      // Pinned host memory is used in place only where the runtime maps it
      // at the same address on the device; anything else is refused rather
      // than translated.
      if (!attr.devicePointer || attr.devicePointer != attr.hostPointer) return PA_ERR_UNSUPPORTED;
      *out = p;
      return PA_OK;
    default:
      return PA_ERR_UNSUPPORTED;
  }
}

bool overlap(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uint64_t(b_bytes) && y < x + uint64_t(a_bytes);
}

// Shared checks and launch of pa_copy_blocks / pa_swap_blocks.
pa_status block_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int64_t* mapping,
                     int64_t num_pairs, int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks, void* stream) {
  if (num_pairs < 0 || num_pairs > INT32_MAX || block_bytes <= 0 || src_blocks <= 0 || dst_blocks <= 0)
    return PA_ERR_SHAPE;
  if (block_bytes % 16) return PA_ERR_ALIGN;
  constexpr int64_t kMaxPoolBytes = int64_t(1) << 50;   // keeps every byte offset and item count in int64
  if (block_bytes > kMaxPoolBytes || src_blocks > kMaxPoolBytes / block_bytes ||
      dst_blocks > kMaxPoolBytes / block_bytes)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !mapping) return PA_ERR_NULL;
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v) ||
      (reinterpret_cast<uintptr_t>(mapping) & 7u))
    return PA_ERR_ALIGN;
  const void *dk, *dv, *sk, *sv, *mp;
  pa_status st;
  if ((st = device_address(dst_k, &dk)) != PA_OK || (st = device_address(dst_v, &dv)) != PA_OK ||
      (st = device_address(src_k, &sk)) != PA_OK || (st = device_address(src_v, &sv)) != PA_OK ||
      (st = device_address(mapping, &mp)) != PA_OK)
    return st;
  hipError_t e = pa::launch_copy_blocks(const_cast<void*>(dk), const_cast<void*>(dv), sk, sv,
                                        static_cast<const int64_t*>(mp), num_pairs, block_bytes, src_blocks,
                                        dst_blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int64_t num_pairs,
                         int64_t block_bytes, int64_t num_blocks, void* stream) {
  return block_copy(k_cache, v_cache, k_cache, v_cache, block_mapping, num_pairs, block_bytes, num_blocks, num_blocks,
                    stream);
}

pa_status pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                         const int64_t* block_mapping, int64_t num_pairs, int64_t block_bytes, int64_t src_num_blocks,
                         int64_t dst_num_blocks, void* stream) {
  if (num_pairs > 0 && dst_k && dst_v && src_k && src_v && block_bytes > 0 && src_num_blocks > 0 &&
      dst_num_blocks > 0 && src_num_blocks <= INT64_MAX / block_bytes && dst_num_blocks <= INT64_MAX / block_bytes) {
    const int64_t sb = src_num_blocks * block_bytes, db = dst_num_blocks * block_bytes;
    if (overlap(dst_k, db, src_k, sb) || overlap(dst_k, db, src_v, sb) || overlap(dst_v, db, src_k, sb) ||
        overlap(dst_v, db, src_v, sb))
      return PA_ERR_SHAPE;
  }
  return block_copy(dst_k, dst_v, src_k, src_v, block_mapping, num_pairs, block_bytes, src_num_blocks,
                    dst_num_blocks, stream);
}

}  // extern "C"
