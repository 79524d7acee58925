// Cache write: scatter this step's new K/V rows into the 16-token block pool.
//
// quant67, "PagedAttention 与 Continuous Batching" §3.3: every decode step
// computes the new token's K/V and appends it to the block that holds its
// position; the scheduler hands the kernel one slot per row (slot_mapping).
// Slot s names block s / 16, offset s % 16.  The pool layout is
// [num_blocks, Hkv, 16, D], so one (row, head) is a contiguous run of D
// elements both in the source and in the pool.
//
// One thread moves one 16-byte chunk; consecutive threads cover consecutive
// chunks of one row, so loads and stores are fully coalesced per (row, head).
// K and V are handled by the same thread (two independent streams in flight).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

template <int ChunksPerHead>
__global__ __launch_bounds__(256) void cache_write_kernel(const u32x4_t* __restrict__ k_new,
                                                          const u32x4_t* __restrict__ v_new,
                                                          int64_t row_stride_chunks, u32x4_t* __restrict__ k_cache,
                                                          u32x4_t* __restrict__ v_cache,
                                                          const int64_t* __restrict__ slot_mapping,
                                                          int64_t num_tokens, int32_t num_kv_heads) {
  const int64_t per_row = int64_t(num_kv_heads) * ChunksPerHead;
  const int64_t total = num_tokens * per_row;
  for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += int64_t(gridDim.x) * blockDim.x) {
    const int64_t row = idx / per_row;
    const int64_t rem = idx - row * per_row;
    const int64_t slot = slot_mapping[row];
    if (slot < 0) continue;
    const int64_t head = rem / ChunksPerHead;
    const int64_t c = rem - head * ChunksPerHead;
    const int64_t blk = slot >> 4;
    const int64_t off = slot & 15;
    const int64_t dst = ((blk * num_kv_heads + head) * kBlock + off) * ChunksPerHead + c;
    const int64_t src = row * row_stride_chunks + rem;
    const u32x4_t kv = k_new[src];
    const u32x4_t vv = v_new[src];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
  }
}

hipError_t launch_cache_write(const void* k_new, const void* v_new, int64_t kv_row_stride_bytes, void* k_cache,
                              void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_bytes, hipStream_t stream) {
  const int64_t chunks_per_head = head_bytes / 16;
  const int64_t total = num_tokens * num_kv_heads * chunks_per_head;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  const int64_t stride_chunks = kv_row_stride_bytes / 16;
  auto kn = static_cast<const u32x4_t*>(k_new);
  auto vn = static_cast<const u32x4_t*>(v_new);
  auto kc = static_cast<u32x4_t*>(k_cache);
  auto vc = static_cast<u32x4_t*>(v_cache);
  switch (chunks_per_head) {
    case 8:   // D=64 bf16
      hipLaunchKernelGGL(cache_write_kernel<8>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc, vc,
                         slot_mapping, num_tokens, num_kv_heads);
      break;
    case 16:  // D=128 bf16, D=64 fp32
      hipLaunchKernelGGL(cache_write_kernel<16>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads);
      break;
    case 32:  // D=128 fp32
      hipLaunchKernelGGL(cache_write_kernel<32>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
