// Split-K paged attention for single-row (decode) requests, bf16, D = 128.
//
// quant67, "PagedAttention 与 Continuous Batching" §3.6: the kernel walks the
// request's block table, loads each physical block's K/V and folds it into an
// online softmax; §3.7 fixes 16 tokens per block.  This is the bandwidth-bound
// half of the path (every decode step reads the whole context once), so the
// design goal is bytes in flight and few VALU instructions per byte.
//
// Work split: one workgroup of 4 waves per (request, KV head, context
// partition).  Wave w owns logical blocks w, w+4, w+8, ... of the partition
// and serves ALL G query heads of the KV head, so each K/V byte enters the
// chip once and is used G times from registers.
//
// Lane layout for one 16-token tile of one KV head (16 x 256 B, contiguous):
// lane l = 16*tg + r loads 16 B at token 4*i + tg, d-slice [8r, 8r+8), for
// load slots i = 0..3.  Every load instruction reads 1 KiB of consecutive
// memory.  Loads are raw buffer loads whose descriptor spans exactly one tile;
// a tile past the wave's range gets a zero-sized descriptor, so the pipeline
// issues a fixed number of loads per step without touching memory for it.
//
// Q.K: each lane forms G partial dot products (v_dot2_f32_bf16) over its
// 8-element slice.  A 4-step DPP reduce-scatter over the 16 lanes of a token
// row (row_ror:8, row_half_mirror, quad_perm x2, quad_perm x1) halves the
// number of values per step, so the G sums cost G-1 + (4-log2 G) DPP adds
// instead of 4G.  To make every step a single uniform instruction, lane r
// keeps its q heads in the order h(r ^ M_j) (M_j built from the step masks),
// and ends holding the full score of head h(r) = r >> (4 - log2 G).
//
// Softmax: each lane keeps (max, sum) of its (token row, head).  The
// reference max is raised only when a block's max exceeds it by more than 8
// (log2 units); otherwise p = 2^(s - m) <= 256 is used as is.  This is exact:
// the final normalisation uses the same reference.  p is rounded to bf16 once
// and the rounded values feed both the sum and P.V, so the output is a convex
// combination of V rows (a one-token context returns V exactly).
//
// P.V: p of token pairs (t, t+4) is packed as bf16x2, rotated within the row
// (row_ror) so lane r sees every head, and V pairs are re-packed with
// v_perm_b32; each v_dot2_f32_bf16 then adds two tokens' contributions to one
// fp32 accumulator.  Lane r's accumulator slot j holds head (h(r) +- j) mod G.
//
// End of the partition: the 4 token rows of a wave are combined with
// v_permlane32_swap / v_permlane16_swap (reduce-scatter), the 4 waves through
// LDS in a fixed order (deterministic).  A request whose context fits in one
// partition is normalised and stored as bf16 (round to nearest even); else
// the partition's (max, sum, unnormalised output) go to the workspace and the
// merge kernel combines them.
#include <algorithm>
#include <atomic>
#include <utility>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kD = 128;
constexpr int kTileBytes = kBlock * kD * 2;   // one (block, KV head) tile of bf16
constexpr int kWavesPerGroup = 4;
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr float kRescaleThreshold = 8.f;      // log2 units
constexpr float kMinusBig = -1e30f;           // finite "no token yet" max
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr int kMaxDevices = 64;

// Pairing masks of the 16-lane reduction steps and their DPP controls.
constexpr int kStepMask[4] = {8, 7, 2, 1};
constexpr int kStepCtrl[4] = {0x128 /*row_ror:8*/, 0x141 /*row_half_mirror*/, 0x4E /*quad_perm 2,3,0,1*/,
                              0xB1 /*quad_perm 1,0,3,2*/};

template <int G>
constexpr int log2_of() {
  return G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
}

// Offset mask of lane-relative q head j: XOR of the halving-step masks
// selected by the bits of j (bit b <-> step K-1-b).
template <int K>
constexpr int q_mask(int j) {
  int m = 0;
  for (int b = 0; b < K; ++b)
    if ((j >> b) & 1) m ^= kStepMask[K - 1 - b];
  return m;
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), Ctrl, 0xF, 0xF, true));
}

// Reduce-scatter of N per-head partial sums over the 16 lanes of a token row,
// steps S..3.  Returns the full sum of head h(r).
template <int N, int S>
__device__ __forceinline__ float row_reduce(const float* s) {
  if constexpr (S == 4) {
    return s[0];
  } else if constexpr (N > 1) {
    float t[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) t[i] = s[i] + dpp_f32<kStepCtrl[S]>(s[i + N / 2]);
    return row_reduce<N / 2, S + 1>(t);
  } else {
    const float t = s[0] + dpp_f32<kStepCtrl[S]>(s[0]);
    return row_reduce<1, S + 1>(&t);
  }
}

__device__ __forceinline__ float dot16_bf16(const u32x4_t& q, const u32x4_t& k) {
  float s = dot2_bf16(q[0], k[0], 0.f);
  s = dot2_bf16(q[1], k[1], s);
  s = dot2_bf16(q[2], k[2], s);
  s = dot2_bf16(q[3], k[3], s);
  return s;
}

__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// max / sum over the 4 token rows (lanes r, r+16, r+32, r+48); every lane gets the result.
__device__ __forceinline__ float rows_max(float v) {
  float a = v, b = v;
  swap32(a, b);
  v = fmaxf(a, b);
  a = v;
  b = v;
  swap16(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum(float v) {
  float a = v, b = v;
  swap32(a, b);
  v = a + b;
  a = v;
  b = v;
  swap16(a, b);
  return a + b;
}

template <int G>
struct GqaSmem {
  float m[kWavesPerGroup][G];
  float l[kWavesPerGroup][G];
  float M[G];
  float L[G];
  float o[kWavesPerGroup][G * kD];
};

// One work item: (request b, KV head kvh, partition part) of a single-row
// request whose partition holds at least one token.  Ends with a barrier, so
// the caller may reuse the shared memory right after.
template <int G>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int b, int kvh, int part, GqaSmem<G>& sm) {
  constexpr int K = log2_of<G>();
  constexpr int kRot = 16 / G;          // lanes between consecutive heads in a row
  constexpr int kNV = G * 8;            // accumulators per lane
  constexpr int kNZ = kNV / 4;          // accumulators per lane after the row reduce-scatter
  auto& s_m = sm.m;
  auto& s_l = sm.l;
  auto& s_M = sm.M;
  auto& s_L = sm.L;
  auto& s_o = sm.o;

  const int q0 = a.cu_seqlens[b];
  const int L = a.seq_lens[b];
  const int tok0 = part * a.part_size;
  const int tok1 = min(tok0 + a.part_size, L);
  const int nparts = (L + a.part_size - 1) / a.part_size;
  const int lb0 = tok0 / kBlock;
  const int nblk = (tok1 + kBlock - 1) / kBlock - lb0;
  const int lb_last = lb0 + nblk - 1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int tg = lane >> 4;
  const int hr = r >> (4 - K);

  // q slices of the G heads, in lane-relative order h(r ^ M_j).
  u32x4_t qreg[G];
  {
    const char* qrow = static_cast<const char*>(a.q) + (int64_t(q0) * a.q_row_stride + int64_t(kvh) * G * kD) * 2;
    static_for<G>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int hh = (r ^ q_mask<K>(j)) >> (4 - K);
      qreg[j] = *reinterpret_cast<const u32x4_t*>(qrow + hh * (kD * 2) + r * 16);
    });
  }

  const int nb = nblk > wave ? (nblk - wave + kWavesPerGroup - 1) / kWavesPerGroup : 0;
  const int32_t* __restrict__ table = a.block_tables + int64_t(b) * a.max_blocks_per_seq;
  const char* kbase = static_cast<const char*>(a.k_cache) + int64_t(kvh) * kTileBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + int64_t(kvh) * kTileBytes;
  const int64_t bstride = int64_t(a.num_kv_heads) * kTileBytes;
  const int voff = tg * (kD * 2) + r * 16;
  const float scale_log2 = a.scale_log2;

  auto issue = [&](u32x4_t(&kb)[4], u32x4_t(&vb)[4], int k) {
    const int lb = lb0 + wave + kWavesPerGroup * k;
    const int nrec = k < nb ? kTileBytes : 0;
    const int64_t phys = table[min(lb, lb_last)];
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + phys * bstride), 0, nrec, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + phys * bstride), 0, nrec, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 4; ++i) kb[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff + i * 1024, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + i * 1024, 0, 0);
  };

  float acc[G][8];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  float m = kMinusBig;   // reference max of this lane's (row, head), log2 units
  float l = 0.f;         // sum of rounded p relative to m

  auto process = [&](u32x4_t(&kb)[4], u32x4_t(&vb)[4], int k) {
    const int tb = (lb0 + wave + kWavesPerGroup * k) * kBlock;   // first token of the block
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s[G];
#pragma unroll
      for (int j = 0; j < G; ++j) s[j] = dot16_bf16(qreg[j], kb[i]);
      sc[i] = row_reduce<G, 0>(s) * scale_log2;
    }
    if (tb + kBlock > tok1) {   // the context ends inside this block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool dead = tb + 4 * i + tg >= tok1;
        sc[i] = dead ? -__builtin_inff() : sc[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) vb[i][w] = dead ? 0u : vb[i][w];
      }
    }
    const float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__builtin_amdgcn_ballot_w64(bm > m + kRescaleThreshold)) {
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
      static_for<G>([&](auto J) {
        constexpr int j = decltype(J)::value;
        float c = alpha;
        if constexpr (j > 0) c = dpp_f32<0x120 + j * kRot>(alpha);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] *= c;
      });
    }
    uint32_t p2[2];
    p2[0] = pack_bf16x2(fast_exp2(sc[0] - m), fast_exp2(sc[1] - m));
    p2[1] = pack_bf16x2(fast_exp2(sc[2] - m), fast_exp2(sc[3] - m));
    l = dot2_bf16(p2[0], kBf16OnePair, l);
    l = dot2_bf16(p2[1], kBf16OnePair, l);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      uint32_t pg[G];
      static_for<G>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (j == 0) pg[j] = p2[kp];
        else pg[j] = dpp_u32<0x120 + j * kRot>(p2[kp]);
      });
      uint32_t vp[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        vp[2 * w] = __builtin_amdgcn_perm(vb[2 * kp + 1][w], vb[2 * kp][w], 0x05040100u);
        vp[2 * w + 1] = __builtin_amdgcn_perm(vb[2 * kp + 1][w], vb[2 * kp][w], 0x07060302u);
      }
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = dot2_bf16(pg[j], vp[e], acc[j][e]);
    }
  };

  // ---- main loop: three tiles in flight per wave ---------------------------------
  // The scheduling barriers keep the loads of every stage in issue order, the
  // same before the loop as inside it, so each stage waits only for its own
  // tile (vmcnt = the 16 loads issued after it), never for the whole ring.
  {
    u32x4_t k0[4], v0[4], k1[4], v1[4], k2[4], v2[4];
    __builtin_amdgcn_sched_barrier(0);
    issue(k0, v0, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(k1, v1, 1);
    __builtin_amdgcn_sched_barrier(0);
    issue(k2, v2, 2);
    __builtin_amdgcn_sched_barrier(0);
    for (int k = 0; k < nb; k += 3) {
      process(k0, v0, k);
      __builtin_amdgcn_sched_barrier(0);
      issue(k0, v0, k + 3);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nb) process(k1, v1, k + 1);
      __builtin_amdgcn_sched_barrier(0);
      issue(k1, v1, k + 4);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 < nb) process(k2, v2, k + 2);
      __builtin_amdgcn_sched_barrier(0);
      issue(k2, v2, k + 5);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- combine the 4 token rows of the wave, then the 4 waves -----------------------
  const float mw = rows_max(m);
  const float lw = rows_sum(l * fast_exp2(m - mw));
  if (tg == 0 && (r & (kRot - 1)) == 0) {
    s_m[wave][hr] = mw;
    s_l[wave][hr] = lw;
  }
  __syncthreads();
  float M = s_m[0][hr];
#pragma unroll
  for (int w = 1; w < kWavesPerGroup; ++w) M = fmaxf(M, s_m[w][hr]);
  if (threadIdx.x < G * kRot && (r & (kRot - 1)) == 0) {   // one lane per head (wave 0, row 0)
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerGroup; ++w) Lt += s_l[w][hr] * fast_exp2(s_m[w][hr] - M);
    s_M[hr] = M;
    s_L[hr] = Lt;
  }
  // scale this lane's row to the common max and rotate the factor to each slot
  const float c = fast_exp2(m - M);
  static_for<G>([&](auto J) {
    constexpr int j = decltype(J)::value;
    float cj = c;
    if constexpr (j > 0) cj = dpp_f32<0x120 + j * kRot>(c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] *= cj;
  });
  // direction of row_ror within the row: head of slot j is (hr + dir*j) mod G
  int dir = 1;
  if constexpr (G > 1) {
    const int src = int(dpp_u32<0x120 + kRot>(uint32_t(r)));
    dir = ((src >> (4 - K)) == ((hr + 1) & (G - 1))) ? 1 : -1;
  }
  // reduce-scatter over the rows: after it, row rho holds accumulator x + rho*kNZ
  float* flat = &acc[0][0];
#pragma unroll
  for (int x = 0; x < kNV / 2; ++x) {
    float p = flat[x], q = flat[x + kNV / 2];
    swap32(p, q);
    flat[x] = p + q;
  }
#pragma unroll
  for (int x = 0; x < kNZ; ++x) {
    float p = flat[x], q = flat[x + kNZ];
    swap16(p, q);
    flat[x] = p + q;
  }
#pragma unroll
  for (int x = 0; x < kNZ; ++x) {
    const int v = x + tg * kNZ;
    const int j = v >> 3;
    const int e = v & 7;
    const int head = (hr + dir * j) & (G - 1);
    s_o[wave][head * kD + r * 8 + e] = flat[x];
  }
  __syncthreads();

  const int64_t row = q0;
  for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
    float o = s_o[0][idx];
#pragma unroll
    for (int w = 1; w < kWavesPerGroup; ++w) o += s_o[w][idx];
    const int h = idx >> 7;
    const int d = idx & (kD - 1);
    const int hq = kvh * G + h;
    if (nparts == 1) {
      static_cast<__bf16*>(a.out)[row * a.o_row_stride + int64_t(hq) * kD + d] = (__bf16)(o / s_L[h]);
    } else {
      const int64_t slot = (int64_t(b) * a.num_q_heads + hq) * a.max_parts + part;
      a.ws_o[slot * kD + d] = o;
      if (d == 0) {
        a.ws_ml[2 * slot] = s_M[h];
        a.ws_ml[2 * slot + 1] = s_L[h];
      }
    }
  }
  __syncthreads();
}

// Persistent kernel.  Item t is entry t / Hkv of the list plan_kernel built,
// KV head t % Hkv (the KV heads of one partition run side by side).  Round i
// hands items [i*W, (i+1)*W) to the W workgroups, in reverse order on odd
// rounds; with the list sorted by decreasing size this zig-zag keeps every
// workgroup's total within a few percent of the mean, with no atomics.
template <int G>
__global__ __launch_bounds__(256, 2) void decode_gqa_kernel(DecodeArgs a) {
  __shared__ GqaSmem<G> sm;
  const int32_t* items = a.plan + kPlanHeaderInts;
  const int hkv = a.num_kv_heads;
  const int total = __builtin_amdgcn_readfirstlane(a.plan[1]) * hkv;
  const int W = gridDim.x;
  for (int i = 0, base = 0; base < total; ++i, base += W) {
    const int t = base + ((i & 1) ? W - 1 - int(blockIdx.x) : int(blockIdx.x));
    if (t >= total) continue;
    const int e = t / hkv;
    const int kvh = t - e * hkv;
    const int b = __builtin_amdgcn_readfirstlane(items[2 * e]);
    const int part = __builtin_amdgcn_readfirstlane(items[2 * e + 1]);
    decode_item<G>(a, b, kvh, part, sm);
  }
}

// Builds the item list of the persistent kernel for the single-row requests:
// plan[1] = number of list entries (plan[0] and the rest of the 256-byte
// header are unused), then
// (request, partition) pairs -- every full partition first, then the partial
// last partitions by decreasing length, so the small items run at the end.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ seq_lens,
                                                    int32_t num_seqs, int32_t part_size, int32_t* __restrict__ plan) {
  __shared__ int s_hist[kMaxPartBuckets];
  __shared__ int s_cursor[kMaxPartBuckets];
  __shared__ int s_full;
  __shared__ int s_fullcur;
  const int nbk = part_size / kBlock;
  for (int i = threadIdx.x; i < nbk; i += blockDim.x) s_hist[i] = 0;
  if (threadIdx.x == 0) {
    s_full = 0;
    s_fullcur = 0;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < num_seqs; b += blockDim.x) {
    if (cu[b + 1] - cu[b] != 1) continue;
    const int L = seq_lens[b];
    const int nf = L / part_size;
    const int rem = L - nf * part_size;
    atomicAdd(&s_full, nf);
    if (rem > 0) atomicAdd(&s_hist[(rem - 1) / kBlock], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = s_full;
    for (int k = nbk - 1; k >= 0; --k) {
      s_cursor[k] = run;
      run += s_hist[k];
    }
    plan[1] = run;
  }
  __syncthreads();
  int32_t* items = plan + kPlanHeaderInts;
  for (int b = threadIdx.x; b < num_seqs; b += blockDim.x) {
    if (cu[b + 1] - cu[b] != 1) continue;
    const int L = seq_lens[b];
    const int nf = L / part_size;
    const int rem = L - nf * part_size;
    int pos = atomicAdd(&s_fullcur, nf);
    for (int p = 0; p < nf; ++p, ++pos) {
      items[2 * pos] = b;
      items[2 * pos + 1] = p;
    }
    if (rem > 0) {
      pos = atomicAdd(&s_cursor[(rem - 1) / kBlock], 1);
      items[2 * pos] = b;
      items[2 * pos + 1] = nf;
    }
  }
}

}  // namespace

bool decode_gqa_supported(int dtype, int head_dim, int group, int part_size) {
  return dtype == 1 && head_dim == kD && (group == 1 || group == 2 || group == 4 || group == 8) &&
         part_size % kBlock == 0 && part_size / kBlock <= kMaxPartBuckets;
}

size_t decode_gqa_plan_bytes(int64_t num_seqs, int64_t max_parts) {
  return (size_t(kPlanHeaderInts) + 2 * size_t(num_seqs) * size_t(max_parts)) * sizeof(int32_t);
}

namespace {

// Resident workgroups per device for kernel K: CUs x occupancy, queried once per device.
template <int G>
int persistent_groups() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_gqa_kernel<G>, 256, 0) != hipSuccess || occ <= 0)
    occ = 1;
  v = cus * occ;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const int64_t upper = int64_t(a.num_seqs) * a.max_parts * a.num_kv_heads;
  const int64_t grid = std::min<int64_t>(upper, persistent_groups<G>());
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.seq_lens, a.num_seqs, a.part_size,
                     a.plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_gqa_kernel<G>, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_gqa(int group, const DecodeArgs& a, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
