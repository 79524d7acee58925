// Debug-time checks of the device metadata that the hot kernels trust.
// Each failed check ORs one PA_BAD_* bit into a caller-owned device word.
#include "../../include/pa.h"
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

__global__ void validate_clear(int32_t* result) { *result = 0; }

__global__ __launch_bounds__(256) void validate_requests(const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ seq_lens,
                                                         const int32_t* __restrict__ bt, int32_t num_seqs,
                                                         int64_t total_q, int32_t max_query_len, int32_t max_seq_len,
                                                         int32_t mbs, int64_t num_blocks, int32_t block_size,
                                                         int32_t* result) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= num_seqs) return;
  int bad = 0;
  const int c0 = cu[b], c1 = cu[b + 1];
  if (b == 0 && c0 != 0) bad |= PA_BAD_CU_SEQLENS;
  if (c1 < c0) bad |= PA_BAD_CU_SEQLENS;
  if (b == num_seqs - 1 && int64_t(c1) != total_q) bad |= PA_BAD_CU_SEQLENS;
  const int n = c1 - c0, L = seq_lens[b];
  if (L < 0 || n > L || n > max_query_len || L > max_seq_len) bad |= PA_BAD_LENGTHS;
  const int64_t used = (int64_t(L) + block_size - 1) / block_size;
  if (used > mbs) {
    bad |= PA_BAD_TABLE_WIDTH;
  } else {
    for (int64_t i = 0; i < used; ++i) {
      const int32_t id = bt[int64_t(b) * mbs + i];
      if (id < 0 || id >= num_blocks) {
        bad |= PA_BAD_BLOCK_ID;
        break;
      }
    }
  }
  if (bad) atomicOr(result, bad);
}

__global__ __launch_bounds__(256) void validate_slots(const int64_t* __restrict__ slots, int64_t num_slots,
                                                      int64_t num_blocks, int32_t block_size, int32_t* result) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= num_slots) return;
  const int64_t s = slots[i];
  if (s < 0) return;
  int bad = 0;
  if (s >= num_blocks * block_size) bad |= PA_BAD_SLOT_RANGE;
  for (int64_t j = i + 1; j < num_slots; ++j) {
    if (slots[j] == s) {
      bad |= PA_BAD_SLOT_DUP;
      break;
    }
  }
  if (bad) atomicOr(result, bad);
}

hipError_t launch_validate(const int32_t* cu, const int32_t* seq_lens, const int32_t* bt, const int64_t* slots,
                           int64_t num_slots, int32_t num_seqs, int64_t total_q, int32_t max_query_len,
                           int32_t max_seq_len, int32_t max_blocks_per_seq, int64_t num_blocks, int32_t block_size,
                           int32_t* result, hipStream_t stream) {
  hipLaunchKernelGGL(validate_clear, dim3(1), dim3(1), 0, stream, result);
  if (num_seqs > 0)
    hipLaunchKernelGGL(validate_requests, dim3((num_seqs + 255) / 256), dim3(256), 0, stream, cu, seq_lens, bt,
                       num_seqs, total_q, max_query_len, max_seq_len, max_blocks_per_seq, num_blocks, block_size,
                       result);
  if (num_slots > 0)
    hipLaunchKernelGGL(validate_slots, dim3((num_slots + 255) / 256), dim3(256), 0, stream, slots, num_slots,
                       num_blocks, block_size, result);
  return hipGetLastError();
}

}  // namespace pa
