// Split-K paged attention for decode rows, and the partition merge.
//
// quant67, "PagedAttention 与 Continuous Batching" §3.6: the kernel walks the
// request's block table, loads each physical block's K/V tile and folds it
// into a softmax; §3.3 fixes the block size at 16 tokens.  Here one
// workgroup (4 waves) owns one (request, KV head, context partition of
// part_size tokens).  The G query heads that share the KV head are served by
// the same K/V bytes, so each byte is read from HBM once per KV head.
//
// Lane layout (per wave, for one 16-token block of one KV head):
//   every lane issues 16-byte loads; kLpr lanes cover one token row of D
//   elements and kTpl rows are covered per load instruction, so each load
//   instruction reads kTpl * D * elem bytes of consecutive memory.  A lane
//   owns d-slice dl = lane % kLpr of tokens tg, tg + kTpl, ... of the block.
//
// Phases per (row, partition):
//   1. Q.K: per token, each lane forms G partial dot products over its
//      d-slice (bf16: v_dot2_f32_bf16, fp32 accumulate) and a DPP butterfly
//      over the kLpr lanes of the row completes them.  Scores, scaled by
//      scale*log2(e), land in LDS.
//   2. softmax: per head, max and exp2 over the partition's scores in LDS
//      (the result equals the online softmax of §3.6 folded block by block;
//      a partition is short enough to hold all its scores).
//   3. P.V: each lane accumulates G x vec fp32 outputs over its tokens.
//      Tokens past the context are selected away, never multiplied by 0,
//      so NaN in unused slots cannot leak.
//   4. Lanes and waves are summed through LDS.  A request whose context fits
//      in one partition is normalised and stored; otherwise the partition's
//      (max, sum, unnormalised output) go to the workspace and the merge
//      kernel combines them with log-sum-exp weights.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

template <typename E, int D, int G>
struct DecodeCfg {
  static constexpr int kVec = 16 / E::bytes;   // elements per 16-byte lane load
  static constexpr int kLpr = D / kVec;        // lanes per token row
  static constexpr int kTpl = kWave / kLpr;    // token rows per load instruction
  static constexpr int kLoads = kBlock / kTpl; // loads per lane per 16-token unit
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * kWave;
  static_assert(kLpr >= 1 && kLpr <= kWave && kTpl <= kBlock, "layout");
};

template <typename E>
__device__ __forceinline__ void widen16(const u32x4_t& w, float* f);

template <>
__device__ __forceinline__ void widen16<BF16>(const u32x4_t& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void widen16<F32>(const u32x4_t& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}

// Partial dot product of one 16-byte slice of q and k.
template <typename E>
__device__ __forceinline__ float dot16(const u32x4_t& q, const u32x4_t& k);

template <>
__device__ __forceinline__ float dot16<BF16>(const u32x4_t& q, const u32x4_t& k) {
  float s = dot2_bf16(q[0], k[0], 0.f);
  s = dot2_bf16(q[1], k[1], s);
  s = dot2_bf16(q[2], k[2], s);
  s = dot2_bf16(q[3], k[3], s);
  return s;
}

template <>
__device__ __forceinline__ float dot16<F32>(const u32x4_t& q, const u32x4_t& k) {
  float s = __uint_as_float(q[0]) * __uint_as_float(k[0]);
  s = fmaf(__uint_as_float(q[1]), __uint_as_float(k[1]), s);
  s = fmaf(__uint_as_float(q[2]), __uint_as_float(k[2]), s);
  s = fmaf(__uint_as_float(q[3]), __uint_as_float(k[3]), s);
  return s;
}

template <typename E>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v);

template <>
__device__ __forceinline__ void store_out<BF16>(void* out, int64_t idx, float v) {
  static_cast<__bf16*>(out)[idx] = (__bf16)v;   // round to nearest even
}

template <>
__device__ __forceinline__ void store_out<F32>(void* out, int64_t idx, float v) {
  static_cast<float*>(out)[idx] = v;
}

template <typename E, int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<E, D, G>;
  constexpr int kVec = C::kVec, kLpr = C::kLpr, kTpl = C::kTpl, kLoads = C::kLoads;
  constexpr int kRowBytes = D * E::bytes;
  constexpr float kNegInf = -__builtin_inff();
  const int bs = a.block_size;   // tokens per physical block: 8, 16 or 32

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int q0 = a.cu_seqlens[b];
  const int n = a.cu_seqlens[b + 1] - q0;
  if (n == 0 || (a.row_mode == kSingleRowOnly && n > 1) || (a.row_mode == kMultiRowOnly && n == 1)) return;
  const int L = a.seq_lens[b];
  const int tok0 = part * a.part_size;
  if (tok0 >= L) return;

  extern __shared__ float smem[];
  float* logits = smem;                                   // [part_size][G]
  const int red_off = (a.part_size * G > C::kWaves * G * D) ? a.part_size * G : C::kWaves * G * D;
  float* stats = smem + red_off;                          // [G][2]: max, sum

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;
  const int dl = lane % kLpr;
  const int tg = lane / kLpr;
  const int32_t* table = a.block_tables + int64_t(b) * a.max_blocks_per_seq;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  const int64_t head_tile = int64_t(kvh) * bs * kRowBytes;
  const int64_t block_stride = int64_t(a.num_kv_heads) * bs * kRowBytes;
  const int lane_off = tg * kRowBytes + dl * 16;
  // Rows tok .. tok + kTpl - 1 of one load instruction lie in one physical
  // block (tok is a multiple of kTpl, and kTpl <= 8 divides the block size).
  // A load wholly past tok_end (the partition's end) is never used: it reads
  // the load group holding the last used row instead, so every address stays
  // inside a block the context owns and no unused table entry is read.
  auto row_addr = [&](const char* pool, int tok, int tok_end) {
    const int tc = min(tok, (tok_end - 1) / kTpl * kTpl);
    const int64_t blk = table[tc / bs];
    return pool + blk * block_stride + head_tile + int64_t(tc - (tc / bs) * bs) * kRowBytes + lane_off;
  };

  for (int j = 0; j < n; ++j) {
    const int ctx = L - n + j + 1;  // keys lo .. ctx-1 are visible to row j
    if (tok0 >= ctx) continue;
    const int lo = window_start(ctx - 1, a.sliding_window);
    const int tok1 = min(tok0 + a.part_size, ctx);
    const int nparts = (ctx + a.part_size - 1) / a.part_size;
    const int row = q0 + j;
    const int lb0 = tok0 / kBlock;
    const int nblk = (tok1 + kBlock - 1) / kBlock - lb0;
    if (tok1 <= lo) {
      // the partition lies wholly before the row's window: an empty partial
      // (max -inf, sum 0) that the merge weighs by zero
      const int64_t prow = a.partial_by_seq ? b : row;
      for (int idx = tid; idx < G * D; idx += C::kThreads) {
        const int g = idx / D;
        const int d = idx - g * D;
        const int64_t slot = (prow * a.num_q_heads + kvh * G + g) * a.max_parts + part;
        a.ws_o[slot * D + d] = 0.f;
        if (d == 0) {
          a.ws_ml[2 * slot] = kNegInf;
          a.ws_ml[2 * slot + 1] = 0.f;
        }
      }
      continue;
    }

    // q slice of this lane for the G heads of the group.
    u32x4_t qf[G];
    {
      const char* qrow = static_cast<const char*>(a.q) + (int64_t(row) * a.q_row_stride + int64_t(kvh) * G * D) * E::bytes;
#pragma unroll
      for (int g = 0; g < G; ++g) qf[g] = *reinterpret_cast<const u32x4_t*>(qrow + g * kRowBytes + dl * 16);
    }

    // ---- phase 1: scores -------------------------------------------------
    {
      u32x4_t cur[kLoads];
      int i = wave;
      if (i < nblk) {
#pragma unroll
        for (int l = 0; l < kLoads; ++l)
          cur[l] = *reinterpret_cast<const u32x4_t*>(row_addr(kpool, (lb0 + i) * kBlock + l * kTpl, tok1));
      }
      for (; i < nblk; i += C::kWaves) {
        u32x4_t nxt[kLoads];
        const int in = i + C::kWaves;
        if (in < nblk) {
#pragma unroll
          for (int l = 0; l < kLoads; ++l)
            nxt[l] = *reinterpret_cast<const u32x4_t*>(row_addr(kpool, (lb0 + in) * kBlock + l * kTpl, tok1));
        }
#pragma unroll
        for (int l = 0; l < kLoads; ++l) {
          float s[G];
#pragma unroll
          for (int g = 0; g < G; ++g) s[g] = group_sum<kLpr>(dot16<E>(qf[g], cur[l]));
          const int tl = i * kBlock + l * kTpl + tg;     // token index within the partition
          const bool valid = tok0 + tl < tok1 && tok0 + tl >= lo;
          if constexpr (kLpr >= G) {
            float v = s[0];
#pragma unroll
            for (int g = 1; g < G; ++g) v = (dl == g) ? s[g] : v;
            if (dl < G) logits[tl * G + dl] = valid ? v * a.scale_log2 : kNegInf;
          } else {
#pragma unroll
            for (int g = 0; g < G; ++g)
              if ((g % kLpr) == dl) logits[tl * G + g] = valid ? s[g] * a.scale_log2 : kNegInf;
          }
        }
#pragma unroll
        for (int l = 0; l < kLoads; ++l) cur[l] = nxt[l];
      }
    }
    __syncthreads();

    // ---- phase 2: softmax over the partition ---------------------------------
    {
      const int nt = nblk * kBlock;
      const int nvalid = tok1 - tok0;
      for (int g = wave; g < G; g += C::kWaves) {
        float m = kNegInf;
        for (int t = lane; t < nvalid; t += kWave) m = fmaxf(m, logits[t * G + g]);
        m = group_max<kWave>(m);
        float l = 0.f;
        for (int t = lane; t < nt; t += kWave) {
          const float e = (t < nvalid) ? fast_exp2(logits[t * G + g] - m) : 0.f;
          logits[t * G + g] = e;
          l += e;
        }
        l = group_sum<kWave>(l);
        if (lane == 0) {
          stats[2 * g] = m;
          stats[2 * g + 1] = l;
        }
      }
    }
    __syncthreads();

    // ---- phase 3: P.V ----------------------------------------------------------
    float acc[G][kVec];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[g][e] = 0.f;
    {
      u32x4_t cur[kLoads];
      int i = wave;
      if (i < nblk) {
#pragma unroll
        for (int l = 0; l < kLoads; ++l)
          cur[l] = *reinterpret_cast<const u32x4_t*>(row_addr(vpool, (lb0 + i) * kBlock + l * kTpl, tok1));
      }
      for (; i < nblk; i += C::kWaves) {
        u32x4_t nxt[kLoads];
        const int in = i + C::kWaves;
        if (in < nblk) {
#pragma unroll
          for (int l = 0; l < kLoads; ++l)
            nxt[l] = *reinterpret_cast<const u32x4_t*>(row_addr(vpool, (lb0 + in) * kBlock + l * kTpl, tok1));
        }
        const bool tail = (tok0 + (i + 1) * kBlock) > tok1;   // block holds tokens past the context
#pragma unroll
        for (int l = 0; l < kLoads; ++l) {
          const int tl = i * kBlock + l * kTpl + tg;
          float v[kVec];
          widen16<E>(cur[l], v);
          if (tail && tok0 + tl >= tok1) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) v[e] = 0.f;
          }
          float p[G];
#pragma unroll
          for (int g = 0; g < G; ++g) p[g] = logits[tl * G + g];
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < kVec; ++e) acc[g][e] = fmaf(p[g], v[e], acc[g][e]);
        }
#pragma unroll
        for (int l = 0; l < kLoads; ++l) cur[l] = nxt[l];
      }
    }

    // ---- phase 4: reduce over token groups and waves, store --------------------
#pragma unroll
    for (int off = kLpr; off < kWave; off <<= 1)
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[g][e] += __shfl_xor(acc[g][e], off);
    __syncthreads();   // all waves are done with the probabilities in LDS
    if (tg == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < kVec; ++e) smem[(wave * G + g) * D + dl * kVec + e] = acc[g][e];
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += C::kThreads) {
      const int g = idx / D;
      const int d = idx - g * D;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < C::kWaves; ++w) o += smem[(w * G + g) * D + d];
      const int h = kvh * G + g;
      if (nparts == 1) {
        store_out<E>(a.out, int64_t(row) * a.o_row_stride + int64_t(h) * D + d, o / stats[2 * g + 1]);
      } else {
        const int64_t prow = a.partial_by_seq ? b : row;
        const int64_t slot = (prow * a.num_q_heads + h) * a.max_parts + part;
        a.ws_o[slot * D + d] = o;
        if (d == 0) {
          a.ws_ml[2 * slot] = stats[2 * g];
          a.ws_ml[2 * slot + 1] = stats[2 * g + 1];
        }
      }
    }
    __syncthreads();   // LDS is reused by the next row
  }
}

// Merge of the context partitions of one (row, query head):
//   M = max_p m_p,  w_p = 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p l_p.
template <typename E, int D>
__global__ __launch_bounds__(64) void merge_kernel(DecodeArgs a) {
  const int prow = blockIdx.x;
  const int h = blockIdx.y;
  int row, ctx;
  if (a.partial_by_seq) {
    const int b = prow;
    const int q0 = a.cu_seqlens[b];
    if (a.cu_seqlens[b + 1] - q0 != 1) return;
    row = q0;
    ctx = a.seq_lens[b];
  } else {
    row = prow;
    int lo = 0, hi = a.num_seqs;   // largest b with cu[b] <= row
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.cu_seqlens[mid] <= row) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int q0 = a.cu_seqlens[b];
    const int n = a.cu_seqlens[b + 1] - q0;
    if ((a.row_mode == kSingleRowOnly && n > 1) || (a.row_mode == kMultiRowOnly && n == 1)) return;
    ctx = a.seq_lens[b] - n + (row - q0) + 1;
  }
  const int nparts = (ctx + a.part_size - 1) / a.part_size;
  if (nparts <= 1) return;
  const int64_t base = (int64_t(prow) * a.num_q_heads + h) * a.max_parts;
  float M = -__builtin_inff();
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_ml[2 * (base + p)]);
  float denom = 0.f;
  constexpr int kPer = D / 64;
  float o[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) o[e] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = fast_exp2(a.ws_ml[2 * (base + p)] - M);
    denom = fmaf(w, a.ws_ml[2 * (base + p) + 1], denom);
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] = fmaf(w, a.ws_o[(base + p) * D + e * 64 + threadIdx.x], o[e]);
  }
  const float inv = 1.f / denom;
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    store_out<E>(a.out, int64_t(row) * a.o_row_stride + int64_t(h) * D + e * 64 + threadIdx.x, o[e] * inv);
}

// Merge of the partials of the fast decode kernel and of split short prefill
// requests (bf16, D = 64 or 128): only the rows on the work list's merge list, one
// wave per (row, query head); an entry names the row, its partition count and
// the partial row its partials were written under.
// The list count and the wave's entry are read together; then partitions are
// taken in chunks of kChunk, each chunk's (max, sum) (scalar loads) and
// output slices (vector loads) issued at once, and folded into a running
// log-sum-exp.  A request with up to kChunk partitions costs two memory round
// trips.  Partitions are combined in order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(256) void merge_list_kernel(DecodeArgs a) {
  constexpr int kPer = D / 64;   // d values per lane: 1, 2 or 4
  constexpr int kChunk = 8;
  const int4* list = reinterpret_cast<const int4*>(a.plan + kPlanHeaderInts + a.merge_off_ints);
  const int lane = threadIdx.x & 63;
  const int64_t NW = int64_t(gridDim.x) * 4;
  const int64_t cap = int64_t(a.merge_capacity) * a.num_q_heads;   // list capacity in (row, head) pairs
  for (int64_t t = int64_t(blockIdx.x) * 4 + uni(threadIdx.x >> 6); t < cap; t += NW) {
    const int e = int(t / a.num_q_heads);
    const int h = int(t - int64_t(e) * a.num_q_heads);
    const int32_t* ep = reinterpret_cast<const int32_t*>(list + e);
    const int q0 = load_const(ep, 1), nparts = load_const(ep, 2), prow = load_const(ep, 3);
    if (e >= load_const(a.plan, kPlanMergeCountInt)) break;
    const int64_t base = (int64_t(prow) * a.num_q_heads + h) * a.max_parts;
    const int32_t* ml = reinterpret_cast<const int32_t*>(a.ws_ml + 2 * base);
    const float* po = a.ws_o + base * D + kPer * lane;
    float M = -__builtin_inff(), denom = 0.f, acc[kPer] = {};
    for (int p0 = 0; p0 < nparts; p0 += kChunk) {
      float m[kChunk], l[kChunk], o[kChunk][kPer];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        m[j] = -__builtin_inff();
        l[j] = 0.f;
#pragma unroll
        for (int x = 0; x < kPer; ++x) o[j][x] = 0.f;
        if (p0 + j < nparts) {
          m[j] = __builtin_bit_cast(float, load_const(ml, 2 * (p0 + j)));
          l[j] = __builtin_bit_cast(float, load_const(ml, 2 * (p0 + j) + 1));
          if constexpr (kPer == 4) {
            const float4 v = *reinterpret_cast<const float4*>(po + int64_t(p0 + j) * D);
            o[j][0] = v.x;
            o[j][1] = v.y;
            o[j][2] = v.z;
            o[j][3] = v.w;
          } else if constexpr (kPer == 2) {
            const float2 v = *reinterpret_cast<const float2*>(po + int64_t(p0 + j) * D);
            o[j][0] = v.x;
            o[j][1] = v.y;
          } else {
            o[j][0] = po[int64_t(p0 + j) * D];
          }
        }
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) Mn = fmaxf(Mn, m[j]);
      const float c = fast_exp2(M - Mn);   // 0 for the first chunk
      denom *= c;
#pragma unroll
      for (int x = 0; x < kPer; ++x) acc[x] *= c;
      M = Mn;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (p0 + j < nparts) {
          const float w = fast_exp2(m[j] - M);
          denom = fmaf(w, l[j], denom);
#pragma unroll
          for (int x = 0; x < kPer; ++x) acc[x] = fmaf(w, o[j][x], acc[x]);
        }
      }
    }
    const float inv = 1.f / denom;
    __bf16* orow = static_cast<__bf16*>(a.out) + int64_t(q0) * a.o_row_stride + int64_t(h) * D;
    if constexpr (kPer == 4) {
      reinterpret_cast<uint2*>(orow)[lane] =
          make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));
    } else if constexpr (kPer == 2) {
      reinterpret_cast<uint32_t*>(orow)[lane] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      orow[lane] = (__bf16)(acc[0] * inv);
    }
  }
}

hipError_t launch_merge_list(int head_dim, const DecodeArgs& a, hipStream_t stream) {
  const int64_t waves = int64_t(a.merge_capacity) * a.num_q_heads;
  const int64_t grid = std::min<int64_t>((waves + 3) / 4, 1024);
  if (grid <= 0) return hipSuccess;
  if (head_dim == 256) {
    hipLaunchKernelGGL(merge_list_kernel<256>, dim3(grid), dim3(256), 0, stream, a);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(merge_list_kernel<128>, dim3(grid), dim3(256), 0, stream, a);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(merge_list_kernel<64>, dim3(grid), dim3(256), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------

template <typename E, int D, int G>
static size_t lds_bytes(int part_size) {
  const int a = part_size * G, b = DecodeCfg<E, D, G>::kWaves * G * D;
  return (size_t(a > b ? a : b) + 2 * G) * sizeof(float);
}

template <typename E, int D>
static hipError_t launch_merge_t(const DecodeArgs& a, int64_t partial_rows, hipStream_t stream) {
  if (a.max_parts <= 1 || partial_rows == 0) return hipSuccess;
  hipLaunchKernelGGL((merge_kernel<E, D>), dim3(partial_rows, a.num_q_heads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

// LDS a generic decode workgroup may take (its scores and partial outputs);
// gfx950 gives a workgroup up to 160 KiB.
constexpr size_t kGenericLdsMax = 128 * 1024;

template <typename E, int D, int G>
static hipError_t launch_one(const DecodeArgs& a, int64_t partial_rows, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_kernel<E, D, G>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(kGenericLdsMax));
  if (attr != hipSuccess) return attr;
  const size_t lds = lds_bytes<E, D, G>(a.part_size);
  dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_kernel<E, D, G>), grid, dim3(256), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge_t<E, D>(a, partial_rows, stream);
}

template <typename E, int D>
static hipError_t dispatch_group(int group, const DecodeArgs& a, int64_t partial_rows, hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<E, D, 1>(a, partial_rows, stream);
    case 2: return launch_one<E, D, 2>(a, partial_rows, stream);
    case 3: return launch_one<E, D, 3>(a, partial_rows, stream);
    case 4: return launch_one<E, D, 4>(a, partial_rows, stream);
    case 5: return launch_one<E, D, 5>(a, partial_rows, stream);
    case 6: return launch_one<E, D, 6>(a, partial_rows, stream);
    case 7: return launch_one<E, D, 7>(a, partial_rows, stream);
    case 8: return launch_one<E, D, 8>(a, partial_rows, stream);
    case 16: return launch_one<E, D, 16>(a, partial_rows, stream);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(int dtype, int head_dim, int group, int part_size) {
  if (dtype != 0 && dtype != 1) return false;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return false;
  // every group of up to 8 query heads per KV head (the kernel uses G only as a
  // count: one workgroup serves all G heads of a KV head), and 16
  if (!((group >= 1 && group <= 8) || group == 16)) return false;
  if (part_size < 16 || part_size > 8192 || part_size % 16) return false;
  return decode_lds_bytes(dtype, head_dim, group, part_size) <= kGenericLdsMax;
}

size_t decode_lds_bytes(int dtype, int head_dim, int group, int part_size) {
  const size_t a = size_t(part_size) * group, b = size_t(4) * group * head_dim;
  return ((a > b ? a : b) + 2 * group) * sizeof(float);
}

hipError_t launch_merge(int dtype, int head_dim, const DecodeArgs& a, int64_t partial_rows, hipStream_t stream) {
  if (dtype == 1) {
    if (head_dim == 128) return launch_merge_t<BF16, 128>(a, partial_rows, stream);
    if (head_dim == 64) return launch_merge_t<BF16, 64>(a, partial_rows, stream);
    if (head_dim == 256) return launch_merge_t<BF16, 256>(a, partial_rows, stream);
  } else if (dtype == 0) {
    if (head_dim == 128) return launch_merge_t<F32, 128>(a, partial_rows, stream);
    if (head_dim == 64) return launch_merge_t<F32, 64>(a, partial_rows, stream);
    if (head_dim == 256) return launch_merge_t<F32, 256>(a, partial_rows, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int dtype, int head_dim, int group, const DecodeArgs& a, int64_t partial_rows,
                         hipStream_t stream) {
  if (dtype == 1) {
    if (head_dim == 128) return dispatch_group<BF16, 128>(group, a, partial_rows, stream);
    if (head_dim == 64) return dispatch_group<BF16, 64>(group, a, partial_rows, stream);
    if (head_dim == 256) return dispatch_group<BF16, 256>(group, a, partial_rows, stream);
  } else if (dtype == 0) {
    if (head_dim == 128) return dispatch_group<F32, 128>(group, a, partial_rows, stream);
    if (head_dim == 64) return dispatch_group<F32, 64>(group, a, partial_rows, stream);
    if (head_dim == 256) return dispatch_group<F32, 256>(group, a, partial_rows, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
