// Cache write: scatter this step's new K/V rows into the block pool (8, 16 or
// 32 tokens per block; 16 is the pages' default).
//
// quant67, "PagedAttention 与 Continuous Batching" §3.3: every decode step
// computes the new token's K/V and appends it to the block that holds its
// position; the scheduler hands the kernel one slot per row (slot_mapping).
// Slot s names block s / bs, offset s % bs.  The pool layout is
// [num_blocks, Hkv, bs, D], so one (row, head) is a contiguous run of D
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
                                                          int64_t num_tokens, int32_t num_kv_heads, int bs_log2) {
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
    const int64_t blk = slot >> bs_log2;
    const int64_t off = slot & ((int64_t(1) << bs_log2) - 1);
    const int64_t dst = (((blk * num_kv_heads + head) << bs_log2) + off) * ChunksPerHead + c;
    const int64_t src = row * row_stride_chunks + rem;
    const u32x4_t kv = k_new[src];
    const u32x4_t vv = v_new[src];
    k_cache[dst] = kv;
    v_cache[dst] = vv;
  }
}

// ---- 8-bit float cache (OCP FP8 E4M3) --------------------------------------------
//
// The pages name 8-bit KV caches (quant67 §8.8, §10.3) as the way to halve KV
// memory; the format taken is OCP E4M3 (bias 7, subnormals m * 2^-9, largest
// finite 448, S.1111.111 = NaN, no infinities).  A new value x (bf16) is
// stored as the code nearest to x / scale, where the quotient is the
// correctly rounded fp32 division; ties go to the even code, magnitudes of
// 448 and beyond (and infinities) saturate to 448, NaN becomes 0x7F.

// E4M3 code of an fp32 value (round to nearest, ties to even, saturating).
__device__ __forceinline__ uint32_t fp8_e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;              // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;      // |x| >= 448, infinities included
  if (a >= 0x3c800000u) {                         // |x| >= 2^-6: normal codes
    // keep exponent and 3 mantissa bits; round the 20 dropped bits to even
    uint32_t r = a >> 20;
    const uint32_t rest = a & 0xfffffu;
    if (rest > 0x80000u || (rest == 0x80000u && (r & 1u))) ++r;
    return sign | (r - (120u << 3));              // rebias 127 -> 7
  }
  // subnormal codes: multiples of 2^-9, the count rounded to even (8 is the
  // smallest normal code, 0x08, which the same number encodes)
  const float m = __builtin_rintf(__uint_as_float(a) * 512.f);
  return sign | uint32_t(m);
}

// One thread quantises 8 bf16 values (16 bytes in) to 8 codes (8 bytes out).
template <int ChunksPerHead>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(const u32x4_t* __restrict__ k_new,
                                                              const u32x4_t* __restrict__ v_new,
                                                              int64_t row_stride_chunks, uint2* __restrict__ k_cache,
                                                              uint2* __restrict__ v_cache,
                                                              const int64_t* __restrict__ slot_mapping,
                                                              int64_t num_tokens, int32_t num_kv_heads, int bs_log2,
                                                              float k_scale, float v_scale) {
  const int64_t per_row = int64_t(num_kv_heads) * ChunksPerHead;
  const int64_t total = num_tokens * per_row;
  auto quantise = [](const u32x4_t& w, float scale) {
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[2 * i] = fp8_e4m3_code(bf16_lo(w[i]) / scale);
      c[2 * i + 1] = fp8_e4m3_code(bf16_hi(w[i]) / scale);
    }
    return make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
  };
  for (int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += int64_t(gridDim.x) * blockDim.x) {
    const int64_t row = idx / per_row;
    const int64_t rem = idx - row * per_row;
    const int64_t slot = slot_mapping[row];
    if (slot < 0) continue;
    const int64_t head = rem / ChunksPerHead;
    const int64_t c = rem - head * ChunksPerHead;
    const int64_t blk = slot >> bs_log2;
    const int64_t off = slot & ((int64_t(1) << bs_log2) - 1);
    const int64_t dst = (((blk * num_kv_heads + head) << bs_log2) + off) * ChunksPerHead + c;
    const int64_t src = row * row_stride_chunks + rem;
    const u32x4_t kv = k_new[src];
    const u32x4_t vv = v_new[src];
    k_cache[dst] = quantise(kv, k_scale);
    v_cache[dst] = quantise(vv, v_scale);
  }
}

namespace {
int log2_block(int32_t block_size) { return block_size == 8 ? 3 : block_size == 32 ? 5 : 4; }
}  // namespace

hipError_t launch_cache_write_fp8(const void* k_new, const void* v_new, int64_t kv_row_stride_bytes, void* k_cache,
                                  void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, float k_scale, float v_scale,
                                  hipStream_t stream) {
  const int lb = log2_block(block_size);
  const int64_t chunks_per_head = head_dim / 8;   // 16 source bytes, 8 cache bytes per chunk
  const int64_t total = num_tokens * num_kv_heads * chunks_per_head;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  const int64_t stride_chunks = kv_row_stride_bytes / 16;
  auto kn = static_cast<const u32x4_t*>(k_new);
  auto vn = static_cast<const u32x4_t*>(v_new);
  auto kc = static_cast<uint2*>(k_cache);
  auto vc = static_cast<uint2*>(v_cache);
  switch (chunks_per_head) {
    case 8:   // D=64
      hipLaunchKernelGGL(cache_write_fp8_kernel<8>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads, lb, k_scale, v_scale);
      break;
    case 16:  // D=128
      hipLaunchKernelGGL(cache_write_fp8_kernel<16>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks,
                         kc, vc, slot_mapping, num_tokens, num_kv_heads, lb, k_scale, v_scale);
      break;
    case 32:  // D=256
      hipLaunchKernelGGL(cache_write_fp8_kernel<32>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks,
                         kc, vc, slot_mapping, num_tokens, num_kv_heads, lb, k_scale, v_scale);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_cache_write(const void* k_new, const void* v_new, int64_t kv_row_stride_bytes, void* k_cache,
                              void* v_cache, const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                              int32_t head_bytes, int32_t block_size, hipStream_t stream) {
  const int lb = log2_block(block_size);
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
                         slot_mapping, num_tokens, num_kv_heads, lb);
      break;
    case 16:  // D=128 bf16, D=64 fp32
      hipLaunchKernelGGL(cache_write_kernel<16>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads, lb);
      break;
    case 32:  // D=256 bf16, D=128 fp32
      hipLaunchKernelGGL(cache_write_kernel<32>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads, lb);
      break;
    case 64:  // D=256 fp32
      hipLaunchKernelGGL(cache_write_kernel<64>, dim3(blocks), dim3(threads), 0, stream, kn, vn, stride_chunks, kc,
                         vc, slot_mapping, num_tokens, num_kv_heads, lb);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
