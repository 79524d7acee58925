// MFMA attention for multi-row (chunked-prefill) requests, bf16, D = 64, 128 or 256.
//
// quant67, "PagedAttention 与 Continuous Batching" §4.2: a long prompt is
// processed in chunks batched with decode rows; a chunk's rows attend to the
// cached prefix plus the causal part of their own chunk (bottom-right
// alignment: row j of a request with n rows and context L sees keys
// 0 .. L-n+j).  Every K/V byte serves many query rows here, so Q.K^T and P.V
// are dense contractions and run on the matrix cores
// (v_mfma_f32_32x32x16_bf16, or 16x16x32 at D = 256; fp32 accumulation).
//
// Work list entry: (request, KV head, tile of 256 -- or, for batches of short
// requests, 64 -- (query row, head) pairs; 64 and 32 at D = 256), the pairs
// packed as m = row * G + head over the G query heads of the KV head.  Every
// wave owns 32 pairs (16 at D = 256).  Alone on the GPU an 8-wave workgroup
// serves a 256-pair entry, its two groups of four waves taking turns on the
// matrix cores; beside the decode kernel two 4-wave items serve it (an 8-wave
// workgroup does not fit on a CU beside a decode workgroup).  A short request
// whose context spans several partitions is one entry per partition (its key
// tiles only), and leaves unnormalised partials and (max, sum) for the merge
// kernel.  Keys are visited in tiles of 64 (four 16-key units of paged
// blocks; every load of a wave has a wave-uniform base), staged through two
// LDS stages: K as 16-byte d-chunks, chunk major (the MFMA reads of one chunk
// are contiguous), V transposed (V^T, d-major) by a 4 x 8 register transpose,
// in a row layout that lets one 16-byte read feed a 32 x 32 x 16 operand.
// The layouts keep the staging writes and the MFMA operand reads free of bank
// conflicts.
//
// Per tile and wave: S^T = K Q^T (keys x pairs), so a lane holds scores of
// one pair and the online softmax over keys is in-lane plus one permlane swap
// between the wave's two 32-lane halves (two swaps over the four 16-lane rows
// at D = 256).  32 x 32 x 16 MFMAs take half the instructions of 16 x 16 x 32
// ones for the same products, and leave the vector ALUs more issue cycles for
// the softmax beside them.  P^T then feeds O^T = V^T P^T as the B operand
// without moving data: inside each MFMA step of P.V the keys are taken in the
// order the S^T accumulators hold them (two runs of 4 keys per lane), and V^T
// is read from LDS in that same order.  P is rounded
// to bf16 for the MFMA, and the softmax sum uses the rounded values.  The
// running max is raised only when a tile's max exceeds it by more than 8
// (log2 units), so most tiles neither rescale the accumulators nor spend a
// multiply on scaling the scores: p = 2^(s * scale * log2(e) - m) is one
// FMA and one exp2 per score.
//
// Positions past the context (the partial last block, clamped block ids)
// are zeroed when staged and masked as keys, so NaN in unused slots cannot
// reach the output.
#include <atomic>
#include <cstddef>
#include <type_traits>
#include <utility>

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr unsigned kRsrcWord3 = 0x00020000u;
constexpr float kMinusBig = -1e30f;
constexpr float kRescaleThreshold = 8.f;      // log2 units
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr int kWavesPerSimd = 2;              // register budget: 256 per lane

// Workgroup shape: W waves, each owning 32 (row, head) pairs (16 at D = 256).
// W = 4: 128 pairs, 64-key tiles, each wave fetching one 16-key unit of every
// tile, two workgroups per CU (the LDS holds two).  W = 2: 64 pairs, 32-key
// tiles, four workgroups per CU -- the same waves per SIMD, half the LDS reads
// per pair (each wave reads the whole staged tile).  W = 8: 256 pairs and
// 64-key tiles, one workgroup per CU, the waves in two groups of four that
// share every staged tile and take turns on the matrix cores (wave w fetches
// the K of unit w, wave w + 4 its V).
template <int W, int D>
struct Shape {
  static constexpr int kWaves = W;
  static constexpr int kThreads = 64 * W;
  static constexpr int kUnits = W == 8 ? 4 : W;      // 16-key units per tile
  static constexpr int kKeys = kBlock * kUnits;      // keys per tile
  static constexpr int kCB = kKeys / 16;             // 16-key column blocks of S^T
  static constexpr int kU = kKeys / 32;              // 32-key MFMA steps of O^T
  static constexpr int kKChunk = kKeys * 16 + 16;    // LDS bytes per 8-wide d-chunk of K (+ pad)
  // LDS bytes per d row of V^T.  At D <= 128 (32 x 32 x 16 products) a lane
  // reads 8 keys of a row as one 16-byte load: rows are 16-byte aligned and
  // padded by 16 bytes, so the 8 rows of an 8-lane read phase land on distinct
  // banks.  At D = 256 (16 x 16 x 32) a lane reads two 8-byte runs: keys + pad
  // chosen so that the 16 rows x 4 row groups of a 32-lane 8-byte read land on
  // distinct banks.
  static constexpr int kVRow = D != 256 || kKeys != 64 ? kKeys * 2 + 16 : kKeys * 2 + 8;
  static constexpr int kKBytes = (D / 8) * kKChunk;
  static constexpr int kVBytes = D * kVRow;
  static constexpr int kStageBytes = kKBytes + kVBytes;
  static constexpr int kLdsBytes = 2 * kStageBytes;
  static_assert(kKeys % 32 == 0, "whole 32-key MFMA steps");
};

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A kernel argument read from the kernel-argument segment where it is used,
// with a volatile scalar load.  The arguments a work item needs once are read
// this way, so they do not occupy scalar registers across the tile loop,
// which needs most of them.  The argument block is the PrefillArgs value at
// offset 0 of the segment.
template <typename T>
__device__ __forceinline__ T karg(size_t offset) {
  typedef const volatile T __attribute__((address_space(4))) CT;
  typedef const char __attribute__((address_space(4))) CC;
  CC* base = (CC*)__builtin_amdgcn_kernarg_segment_ptr();
  return *(CT*)(base + offset);
}
#define PA_KARG(field) karg<decltype(PrefillArgs::field)>(offsetof(PrefillArgs, field))
static_assert(std::is_standard_layout<PrefillArgs>::value, "offsetof on the argument block");

__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                  0);
}
// 32 x 32 x 16: lane l holds row (A) / column (B) l % 32 with k = 8 (l / 32) .. +7;
// element r of the result is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                  0);
}

// One thread's share of a wave's 16-key unit of a tile (d-chunks of 8 values):
//   D = 128: k[kk]: key 4*(lane/16) + kk, d-chunk lane%16;
//            v[kk]: key 4*(lane%4) + kk, d-chunk lane/4
//   D = 64:  the same for lanes 0..31 with d-chunk lane%8 for k
//   D = 256: k[kk]: key 8*(lane/32) + kk, d-chunk lane%32 (kk < 8);
//            v[4g + kk]: key 4*(lane%4) + kk, d-chunk lane/4 + 16g
//   The registers hold the cached encoding: 16 bytes (8 bf16) per chunk, or
//   with 8-bit pools 8 bytes (8 E4M3 codes), widened to bf16 when staged.
template <int D, bool F8>
struct TileRegs {
  static constexpr int kN = D == 256 ? 8 : 4;
  using Raw = typename std::conditional<F8, u32x2_t, u32x4_t>::type;
  Raw k[kN];
  Raw v[kN];
  // a chunk of 8 cached elements at byte offset off of the range rsrc
  static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t rsrc, int off) {
    if constexpr (F8)
      return __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, 0);
    else
      return __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
  }
  // the chunk as 8 bf16 values; E4M3 -> bf16 is exact (every E4M3 value is a
  // bf16 value), the pool's scale is applied elsewhere
  static __device__ __forceinline__ u32x4_t widen(const Raw& w) {
    if constexpr (F8) {
      auto cvt = [](uint32_t x, auto hi) {
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.f, decltype(hi)::value));
      };
      return u32x4_t{cvt(w[0], std::false_type{}), cvt(w[0], std::true_type{}), cvt(w[1], std::false_type{}),
                     cvt(w[1], std::true_type{})};
    } else {
      return w;
    }
  }
};

// W = 8 for chunked prefill alone on the GPU, W = 4 beside the decode kernel
// (and at D = 256); W = 2 for batches whose multi-row requests are short
// (speculative-decode verification), where a larger tile would be mostly
// empty and the LDS reads per tile, not HBM, would set the pace.
template <int G, int W, int BS, int D, bool F8>
__global__ __launch_bounds__((Shape<W, D>::kThreads), kWavesPerSimd) void prefill_kernel(PrefillArgs a) {
  using S = Shape<W, D>;
  constexpr int kEB = F8 ? 1 : 2;                // bytes per cached element
  constexpr int kTileBytes = kBlock * D * kEB;   // one 16-key unit of one KV head
  constexpr int kSteps = D / 32;               // 32-wide d steps of S^T = K Q^T
  constexpr int kDB = D / 16;                  // 16-row d blocks of O^T
  constexpr int kMB = D == 256 ? 1 : 2;       // 16-column MFMA blocks per wave (registers at D = 256)
  constexpr int kNK = TileRegs<D, F8>::kN;    // 8-element K (and V) chunks a lane stages per unit
  constexpr int kPairs = 16 * kMB * W;
  constexpr int kKeys = S::kKeys;
  constexpr int kCB = S::kCB;
  constexpr int kU = S::kU;
  constexpr int kKChunk = S::kKChunk;
  constexpr int kVRow = S::kVRow;
  constexpr int kKBytes = S::kKBytes;
  constexpr int kStageBytes = S::kStageBytes;
  constexpr int kRows = kPairs / G;   // query rows per work item
  // With 32 pairs per wave the products are 32 x 32 x 16 MFMAs (half the
  // instructions of 16 x 16 x 32 for the same work, which leaves more issue
  // cycles to the softmax); D = 256 keeps 16 pairs per wave on 16 x 16 x 32.
  constexpr bool kM32 = kMB == 2;
  constexpr int kNP = kM32 ? 1 : kMB;            // pairs per lane
  constexpr int kQSteps = kM32 ? D / 16 : kSteps;   // d steps of S^T
  constexpr int kAB = kM32 ? D / 32 : kDB;          // d blocks of O^T
  using Acc = typename std::conditional<kM32, f32x16_t, f32x4_t>::type;
  extern __shared__ __align__(16) char smem[];

  const int hkv = a.num_kv_heads;
  const int split_log2 = PA_KARG(head_split_log2);
  const int nh = hkv << split_log2;   // head groups of G query heads; group hg reads KV head hg >> split_log2
  const int group = a.num_q_heads / hkv;   // query heads per KV head
  // A list entry holds tile_pairs pairs: one item, or (256-pair entries on
  // 4-wave workgroups) two items, its first and second half of rows.
  const int subs = PA_KARG(tile_pairs) > kPairs ? 2 : 1;
  const int nhs = nh * subs;   // items per list entry
  const int total = load_const(a.plan, kPlanPrefCountInt) * nhs;
  const int ngroups = gridDim.x;
  const int wg = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int h = lane >> 4;    // 16-lane row of the wave
  const int lc = lane & 15;   // 16 x 16 MFMA column of the lane
  const int hf = lane >> 5;   // 32-lane half of the wave
  // staging coordinates (see TileRegs): at D = 64 the unit's 8 d-chunks per key
  // are staged by lanes 0..31 and lanes 32..63 stage nothing
  const int kkey = D == 256 ? 8 * (lane >> 5) : D == 128 ? 4 * (lane >> 4) : 4 * ((lane >> 3) & 3);
  const int kchunk = D == 256 ? lane & 31 : D == 128 ? lane & 15 : lane & 7;
  const int vkey = 4 * (lane & 3), vchunk = lane >> 2;
  const bool stager = D != 64 || lane < 32;
  constexpr int kHeadBytes = BS * D * kEB;   // one KV head's rows of a physical block
  const int64_t bstride = int64_t(hkv) * kHeadBytes;
  const float scale_log2 = a.scale_log2;
  const int32_t* entries = a.plan + kPlanHeaderInts + a.pref_off_ints;

  // Items in list order (largest first); workgroup wg's first item is item
  // wg.  Alone on the GPU, later items are dealt out round-robin, every other
  // round in reverse, so the large items spread over the workgroups.  Beside
  // a decode launch (claim_items), a CU holds one prefill workgroup until the
  // decode workgroups leave, so later items are claimed from a counter in the
  // list's header instead: the workgroups that run longer, or start later,
  // take more of the small items at the end.  The next claim is issued when
  // an item starts and its value read when the item ends, so the round trip
  // overlaps the item's tiles (a claim costs about 4% of a lone prefill
  // launch, which is why the lone one keeps the static deal).
  const bool claim_items = PA_KARG(claim_items) != 0;
  // Beside a decode launch each SIMD also runs a decode worker, which streams
  // K/V and waits on memory most of the time; the prefill waves take issue
  // priority over it (measured on the mixed chunked-prefill step: 580 -> 510
  // us; raising the decode waves' priority instead changed nothing).
  if (claim_items) __builtin_amdgcn_s_setprio(2);
  // There, a wave takes one level more while it issues its matrix-core
  // products (mixed chunked-prefill step: 490.5 -> 473.5 us).  Alone on the
  // GPU the same raise made the prefill kernel 4% slower, so it is not done.
  auto matrix_phase = [&](bool on) {
    if (claim_items) {
      if (on)
        __builtin_amdgcn_s_setprio(3);
      else
        __builtin_amdgcn_s_setprio(2);
    }
  };
  int* claim_counter = a.plan + kPlanPrefClaimInt;
  int* done_counter = a.plan + kPlanPrefDoneInt;
  __shared__ int s_next;
  for (int t = wg, round = 0; t < total;) {
    int claimed = 0;
    if (claim_items && tid == 0)
      claimed = __hip_atomic_fetch_add(claim_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int e = t / nhs;
    const int sub = t - e * nhs >= nh ? 1 : 0;
    const int hg = t - e * nhs - sub * nh;
    const int kvh = hg >> split_log2;
    // The item's query heads h0 .. h0 + gv - 1: a KV head's heads cut into
    // groups of G in order; where the group is not a power of two the last
    // item of a KV head has fewer, and its other head slots are padding.
    const int hsub = hg & ((1 << split_log2) - 1);
    const int h0 = kvh * group + hsub * G;
    const int gv = min(G, group - hsub * G);
    const int b = load_const(entries, 4 * int64_t(e));
    const int tile_part = load_const(entries, 4 * int64_t(e) + 1);
    const int q0 = load_const(entries, 4 * int64_t(e) + 2);
    const int n = load_const(entries, 4 * int64_t(e) + 3);
    const int mt = tile_part & 0xffff;
    const int part = tile_part >> 16;
    const int L = load_const(PA_KARG(seq_lens), b);
    const int P = L - n;                  // cached tokens before this request's rows
    const int j0 = (mt * subs + sub) * kRows;   // rows [j0, j1) of the request
    const bool empty = j0 >= n;   // the second half of a short entry: no rows, no tiles
    const int j1 = min(n, j0 + kRows);
    const int kmax = P + j1;              // keys visible to the last row
    const int KT = (kmax + kKeys - 1) / kKeys;
    // Keys from the first row's window start on.  A split short request
    // covers the key tiles of partition `part` (partitions before p_lo get no
    // item) and leaves partials for the merge; otherwise the item covers all
    // its tiles.
    const int window = PA_KARG(sliding_window);
    const int part_size = PA_KARG(part_size);
    const int lo_first = window_start(P + j0, window);
    const int lo_last = window_start(P + j1 - 1, window);
    const int p_lo = lo_first / part_size;
    const bool split = n <= PA_KARG(split_rows) && (L + part_size - 1) / part_size - p_lo > 1;
    const int part_tiles = part_size / kKeys;
    const int kt_lo = lo_first / kKeys;
    const int kt0 = split ? max(part * part_tiles, kt_lo) : kt_lo;
    const int kt1 = empty ? kt0 : split ? min(KT, (part + 1) * part_tiles) : KT;
    const int mbps = PA_KARG(max_blocks_per_seq);
    // the request's table entries, and its 16-key units (a wave's share of a key tile)
    const int nblk = max(1, min((L + BS - 1) / BS, mbps));
    const int nunits = max(1, min((L + kBlock - 1) / kBlock, (mbps * BS + kBlock - 1) / kBlock));
    const int32_t* table = PA_KARG(block_tables) + int64_t(b) * mbps;
    const char* kbase = static_cast<const char*>(PA_KARG(k_cache)) + int64_t(kvh) * kHeadBytes;
    const char* vbase = static_cast<const char*>(PA_KARG(v_cache)) + int64_t(kvh) * kHeadBytes;

    // ---- this lane's pairs -----------------------------------------------------
    // 32 pairs per wave (D <= 128): one pair per lane, m = wave*32 + lane % 32;
    // lanes l and l + 32 hold the same pair (each half of every 32-key block).
    // 16 pairs per wave (D = 256): m = wave*16 + lc, one per 16-lane row.
    // Visible keys of a pair: lolim .. lolim + span (one unsigned compare per score).
    int jrow[kNP], hq[kNP], lolim[kNP], span[kNP];
    bool mvalid[kNP];
    u32x4_t qb[kNP][kQSteps];   // B operand Q^T: pair m, d = 16s + 8hf .. +7 (32-pair) or 32s + 8h .. +7
#pragma unroll
    for (int mb = 0; mb < kNP; ++mb) {
      const int m = kM32 ? wave * 32 + (lane & 31) : wave * (16 * kMB) + mb * 16 + lc;
      jrow[mb] = j0 + m / G;
      hq[mb] = h0 + m % G;
      mvalid[mb] = jrow[mb] < j1 && m % G < gv;   // a padding head slot is never valid
      lolim[mb] = mvalid[mb] ? window_start(P + jrow[mb], window) : 0;
      span[mb] = mvalid[mb] ? P + jrow[mb] - lolim[mb] : 0;
      const char* qrow = static_cast<const char*>(PA_KARG(q)) +
                         (int64_t(q0 + (mvalid[mb] ? jrow[mb] : 0)) * PA_KARG(q_row_stride) +
                          int64_t(mvalid[mb] ? hq[mb] : h0) * D) * 2;
#pragma unroll
      for (int s = 0; s < kQSteps; ++s) {
        const int d0 = kM32 ? 16 * s + 8 * hf : 32 * s + 8 * h;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qrow + d0 * 2);
        qb[mb][s] = mvalid[mb] ? v : u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    // O^T blocks: d = 32*db + 8*(r/4) + 4*hf + r%4 (32-pair), or 16*db + 4h + r; pair m
    Acc acc[kNP][kAB];
#pragma unroll
    for (int mb = 0; mb < kNP; ++mb)
#pragma unroll
      for (int db = 0; db < kAB; ++db) acc[mb][db] = Acc{};
    float mrun[kNP], lrun[kNP];
#pragma unroll
    for (int mb = 0; mb < kNP; ++mb) {
      mrun[mb] = kMinusBig;
      lrun[mb] = 0.f;
    }

    // ---- K/V tile staging -----------------------------------------------------
    // Physical block of this wave's part of tile kt (clamped into the table;
    // positions past the context are zeroed when staged).  Read with a vector
    // load one tile ahead: a scalar load would share the LDS reads' wait
    // counter, and every tile's first LDS wait would then also wait out a
    // memory round trip for the table.
    //
    // Unit u (keys 16u .. 16u+15) lives in block u of 16 tokens, in half u & 1
    // of block u / 2 of 32 tokens, or in blocks 2u and 2u+1 of 8 tokens (the
    // second read only when it holds a key below L: past the context it may
    // not be the request's).  The ids travel packed in one 64-bit value.
    const __amdgpu_buffer_rsrc_t rtab =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(table), 0, nblk * 4, kRsrcWord3);
    constexpr int kUnits = S::kUnits;
    const int wunit = wave % kUnits;   // the 16-key unit of every tile this wave fetches
    auto unit_of = [&](int kt) { return min(kt * kUnits + wunit, nunits - 1); };
    auto phys_of = [&](int kt) -> uint64_t {
      const int u = unit_of(kt);
      if constexpr (BS == 16) {
        return __builtin_amdgcn_raw_buffer_load_b32(rtab, u * 4, 0, 0);
      } else if constexpr (BS == 32) {
        return __builtin_amdgcn_raw_buffer_load_b32(rtab, (u >> 1) * 4, 0, 0);
      } else {
        const uint32_t first = __builtin_amdgcn_raw_buffer_load_b32(rtab, 2 * u * 4, 0, 0);
        const uint32_t second =
            __builtin_amdgcn_raw_buffer_load_b32(rtab, (u * kBlock + 8 < L ? 2 * u + 1 : 2 * u) * 4, 0, 0);
        return uint64_t(first) | (uint64_t(second) << 32);
      }
    };
    using Regs = TileRegs<D, F8>;
    using Raw = typename Regs::Raw;
    // The lane's chunks of this wave's unit of tile kt from the K pool (base
    // kbase) or the V pool, in the K mapping (key kkey + i, d-chunk kchunk) or
    // the V mapping (key vkey + i % 4, d-chunk vchunk + 16 (i / 4)).
    auto load_part = [&](Raw* r, int kt, uint64_t phys_v, const char* base, bool kmap) {
      if (!stager) return;
      const int u = unit_of(kt);
      const int64_t phys = uni(int(uint32_t(phys_v)));
      auto off_of = [&](int i, int key_base) {
        return kmap ? (key_base + i) * (D * kEB) + kchunk * 8 * kEB
                    : (key_base + (i & 3)) * (D * kEB) + (vchunk + 16 * (i >> 2)) * 8 * kEB;
      };
      const int key = kmap ? kkey : vkey;
      if constexpr (BS == 8) {
        // keys 0..7 of the unit from the first block, 8..15 from the second
        const int64_t phys2 = uni(int(uint32_t(phys_v >> 32)));
        const int nrec = kt < kt1 ? kHeadBytes : 0;
        const int nrec2 = kt < kt1 && u * kBlock + 8 < L ? kHeadBytes : 0;
        const __amdgpu_buffer_rsrc_t r1 =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + phys * bstride), 0, nrec, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t r2 =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + phys2 * bstride), 0, nrec2, kRsrcWord3);
        if (key < 8) {
#pragma unroll
          for (int i = 0; i < kNK; ++i) r[i] = Regs::load(r1, off_of(i, key));
        } else {
#pragma unroll
          for (int i = 0; i < kNK; ++i) r[i] = Regs::load(r2, off_of(i, key - 8));
        }
      } else {
        const int64_t off = BS == 32 ? phys * bstride + (u & 1) * kTileBytes : phys * bstride;
        const int nrec = kt < kt1 ? kTileBytes : 0;
        const __amdgpu_buffer_rsrc_t r1 =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), 0, nrec, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < kNK; ++i) r[i] = Regs::load(r1, off_of(i, key));
      }
    };
    // Positions past the context in the lane's chunks (K or V mapping) become
    // zeros: code 0 is +0 in both encodings.
    auto zero_past = [&](Raw* r, int kt, bool kmap) {
      if (kt * kKeys + kKeys > L) {   // the context ends in this tile
        const int key0 = kt * kKeys + wunit * kBlock + (kmap ? kkey : vkey);
#pragma unroll
        for (int i = 0; i < kNK; ++i)
          if (key0 + (kmap ? i : (i & 3)) >= L) r[i] = Raw{};
      }
    };
    // K chunks of tile kt to the K half of stage st
    auto write_k = [&](Raw* r, int kt, int st) {
      if (!stager) return;
      zero_past(r, kt, true);
      char* ks = smem + st * kStageBytes;
#pragma unroll
      for (int i = 0; i < kNK; ++i)
        *reinterpret_cast<u32x4_t*>(ks + kchunk * kKChunk + (wunit * kBlock + kkey + i) * 16) = Regs::widen(r[i]);
    };
    // V chunks of tile kt to the V half of stage st, transposed: d rows
    // 8*(vchunk + 16g) + 2w (+1) get this lane's 4 keys (8 bytes each).  At D <=
    // 128 the 16-key group of unit u sits at group slot u ^ ((d / 16) % units)
    // of row d, and inside a group the keys come as 0-3, 8-11, 4-7, 12-15 (a
    // lane of the wave's first half takes keys 0-3 and 8-11 for a 32 x 32 x 16
    // step, of the second half 4-7 and 12-15).  With 64 LDS banks and 144-byte
    // rows, the 16 rows of a 16-lane read phase then share one slot and fall on
    // distinct banks, and so do the 8 chunks x 4 lanes of a 32-lane write phase
    // (rows 8 apart: the slot separates the pairs of chunks that the row
    // stride alone would put on one bank).
    auto write_v = [&](Raw* r, int kt, int st) {
      if (!stager) return;
      zero_past(r, kt, false);
      const int vslot = kM32 ? 16 * (wunit ^ ((vchunk >> 1) & (kUnits - 1))) + 8 * ((vkey >> 2) & 1) +
                                   4 * ((vkey >> 3) & 1)
                             : wunit * kBlock + vkey;
      char* vcol = smem + st * kStageBytes + kKBytes + vslot * 2;
#pragma unroll
      for (int g = 0; g < kNK / 4; ++g) {
        const u32x4_t vv[4] = {Regs::widen(r[4 * g]), Regs::widen(r[4 * g + 1]), Regs::widen(r[4 * g + 2]),
                               Regs::widen(r[4 * g + 3])};
        const int dc = vchunk + 16 * g;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo01 = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x05040100u);
          const uint32_t lo23 = __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x05040100u);
          const uint32_t hi01 = __builtin_amdgcn_perm(vv[1][w], vv[0][w], 0x07060302u);
          const uint32_t hi23 = __builtin_amdgcn_perm(vv[3][w], vv[2][w], 0x07060302u);
          *reinterpret_cast<u32x2_t*>(vcol + (8 * dc + 2 * w) * kVRow) = u32x2_t{lo01, lo23};
          *reinterpret_cast<u32x2_t*>(vcol + (8 * dc + 2 * w + 1) * kVRow) = u32x2_t{hi01, hi23};
        }
      }
    };
    auto fetch = [&](TileRegs<D, F8>& rg, int kt, uint64_t phys_v) {
      load_part(rg.k, kt, phys_v, kbase, true);
      load_part(rg.v, kt, phys_v, vbase, false);
    };
    auto stage_write = [&](TileRegs<D, F8>& rg, int kt, int st) {
      write_k(rg.k, kt, st);
      write_v(rg.v, kt, st);
    };

    // ---- one tile from LDS stage st -----------------------------------------------
    // The lazy rescale of one pair's state, given the tile's max in log2 units
    // (the same value in every lane that holds the pair).  The reference max is
    // raised only when the tile's max exceeds it by more than kRescaleThreshold
    // (log2 units); otherwise p <= 2^8 is used as is.  Exact: the normalisation
    // uses the same reference.  The wave rescales when any of its valid pairs
    // asks; pairs past the item's last row (zero queries, written nowhere) take
    // no part, so a pair's bits depend only on the valid pairs beside it and not
    // on how far the item's tile range reaches below the window of its rows.
    auto rescale = [&](int mb, float tmax) {
      if (__builtin_amdgcn_ballot_w64(mvalid[mb] && tmax > mrun[mb] + kRescaleThreshold)) {
        const float mnew = fmaxf(mrun[mb], tmax);
        const float alpha = fast_exp2(mrun[mb] - mnew);
        mrun[mb] = mnew;
        lrun[mb] *= alpha;
#pragma unroll
        for (int db = 0; db < kAB; ++db) acc[mb][db] *= alpha;
      }
    };
    // p = 2^(s * scale_log2 - m) of 8 scores, packed as bf16 pairs; the sum of the
    // rounded values goes into lsum
    auto softmax8 = [&](float s0, float s1, float s2, float s3, float s4, float s5, float s6, float s7, float nm,
                        float& lsum) {
      uint32_t w[4];
      w[0] = pack_bf16x2(fast_exp2(fmaf(s0, scale_log2, nm)), fast_exp2(fmaf(s1, scale_log2, nm)));
      w[1] = pack_bf16x2(fast_exp2(fmaf(s2, scale_log2, nm)), fast_exp2(fmaf(s3, scale_log2, nm)));
      w[2] = pack_bf16x2(fast_exp2(fmaf(s4, scale_log2, nm)), fast_exp2(fmaf(s5, scale_log2, nm)));
      w[3] = pack_bf16x2(fast_exp2(fmaf(s6, scale_log2, nm)), fast_exp2(fmaf(s7, scale_log2, nm)));
#pragma unroll
      for (int x = 0; x < 4; ++x) lsum = dot2_bf16(w[x], kBf16OnePair, lsum);
      return u32x4_t{w[0], w[1], w[2], w[3]};
    };
    // Keys past a row's limit, or before its window, get a score of -inf (raw
    // scores: the scale is positive, so the order and the masking survive
    // scaling).  Only tiles that reach past the first row's limit or before
    // the last row's window start need it.
    auto needs_mask = [&](int kt) { return kt * kKeys + kKeys - 1 > P + j0 || kt * kKeys < lo_last; };
    // ---- 32 pairs per wave: the pieces of a tile ------------------------------------
    // S^T block c of a tile: keys 32c + 8(r/4) + 4hf + r%4 (element r), pair lane % 32.
    constexpr int kKB = kKeys / 32;
    using STile = f32x16_t[kKB];
    // S^T of the tile whose K is in stage kst
    // Operand reads run kReadAhead MFMAs ahead of their products in the 8-wave
    // loop, where one wave per SIMD issues the products of a phase with no
    // other wave's products to hide its LDS round trips: the reads of the next
    // group of operands are issued, then the products of the current group,
    // and scheduling barriers keep the compiler from sinking the reads back
    // next to their use.  The 4-wave loops leave the schedule to the compiler.
    constexpr int kReadAhead = W == 8 ? 2 : 0;   // 2: 202.7 us alone on the mixed step's chunks, 1: 206.4, 4: 209.6
    auto pipelined = [&](auto nops, auto read, auto product) {
      constexpr int N = decltype(nops)::value;
      if constexpr (kReadAhead == 0) {
#pragma unroll
        for (int q = 0; q < N; ++q) product(q, read(q));
      } else {
        constexpr int B = kReadAhead;
        static_assert(N % B == 0, "whole groups of operands");
        u32x4_t buf[2][B];
#pragma unroll
        for (int x = 0; x < B; ++x) buf[0][x] = read(x);
#pragma unroll
        for (int g = 0; g < N / B; ++g) {
          if (g + 1 < N / B) {
#pragma unroll
            for (int x = 0; x < B; ++x) buf[(g + 1) & 1][x] = read((g + 1) * B + x);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int x = 0; x < B; ++x) product(g * B + x, buf[g & 1][x]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // S^T of the tile whose K is in stage kst; operand q: d step q / kKB, block q % kKB
    auto qk32 = [&](STile& sacc, int kst) {
      const char* ks = smem + kst * kStageBytes;
#pragma unroll
      for (int c = 0; c < kKB; ++c) sacc[c] = f32x16_t{};
      pipelined(
          std::integral_constant<int, kQSteps * kKB>{},
          [&](int q) {
            return *reinterpret_cast<const u32x4_t*>(ks + (2 * (q / kKB) + hf) * kKChunk +
                                                     (32 * (q % kKB) + (lane & 31)) * 16);
          },
          [&](int q, const u32x4_t& ka) { sacc[q % kKB] = mfma32(ka, qb[0][q / kKB], sacc[q % kKB]); });
    };
    auto mask32 = [&](STile& sacc, int kt) {
#pragma unroll
      for (int c = 0; c < kKB; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * kKeys + 32 * c + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (uint32_t(key - lolim[0]) > uint32_t(span[0])) sacc[c][r] = -__builtin_inff();
        }
    };
    // the tile's max over the pair's keys, in log2 units
    auto max32 = [&](const STile& sacc) {
      float tmax = -__builtin_inff();
#pragma unroll
      for (int c = 0; c < kKB; ++c)
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          tmax = fmaxf(fmaxf(tmax, fmaxf(sacc[c][r], sacc[c][r + 1])), fmaxf(sacc[c][r + 2], sacc[c][r + 3]));
      return halves_max(tmax) * scale_log2;
    };
    // B operands P^T of the tile's 16-key steps 2c + u: keys 32c + 16u + 8(t/4) +
    // 4hf + t%4 for the lane's slots t = 0..7, i.e. elements 8u .. 8u+7 of block c
    auto probs32 = [&](const STile& sacc, u32x4_t* pb) {
      const float nm = -mrun[0];
      float lsum = lrun[0];
#pragma unroll
      for (int c = 0; c < kKB; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x16_t& sv = sacc[c];
          pb[2 * c + u] = softmax8(sv[8 * u], sv[8 * u + 1], sv[8 * u + 2], sv[8 * u + 3], sv[8 * u + 4], sv[8 * u + 5],
                                   sv[8 * u + 6], sv[8 * u + 7], nm, lsum);
        }
      lrun[0] = lsum;
    };
    // O^T += V^T P^T with V from stage vst.  A operand of step k, d block db: row
    // 32db + lane % 32 and the same keys as P^T's slots, two runs of 4 keys.
    // operand q: 16-key step k = q / kAB, d block db = q % kAB, row 32 db + lane
    // % 32.  The lane's 8 keys are the 16 bytes at 32 * slot + 16 hf of the row,
    // slot = k ^ ((row / 16) % units) = k2 ^ hl with k2 = k ^ (2 (db & 1)) (4
    // units) or k (2 units) and hl = (lane / 16) % 2.  32 (k2 ^ hl) is 32 k2 +
    // 32 hl for even k2 and 32 k2 - 32 hl for odd k2, so each read is one of two
    // per-lane bases plus an immediate offset.
    const int vrow_lane = (lane & 31) * kVRow + 16 * hf;
    const int vbase_even = vrow_lane + 32 * ((lane >> 4) & 1);
    const int vbase_odd = vrow_lane - 32 * ((lane >> 4) & 1);
    auto pv32 = [&](const u32x4_t* pb, int vst) {
      if constexpr (kM32) {
        const char* vs = smem + vst * kStageBytes + kKBytes;
        pipelined(
            std::integral_constant<int, 2 * kKB * kAB>{},
            [&](int q) {
              const int db = q % kAB;
              const int k2 = (q / kAB) ^ (kUnits == 4 ? 2 * (db & 1) : 0);
              return *reinterpret_cast<const u32x4_t*>(vs + 32 * db * kVRow + 32 * k2 +
                                                       ((k2 & 1) ? vbase_odd : vbase_even));
            },
            [&](int q, const u32x4_t& va) { acc[0][q % kAB] = mfma32(va, pb[q / kAB], acc[0][q % kAB]); });
      }
    };

    // ---- one tile from LDS stage st -------------------------------------------------
    auto compute = [&](int kt, int st) {
      const char* ks = smem + st * kStageBytes;
      const char* vs = ks + kKBytes;
      if constexpr (kM32) {
        f32x16_t sacc[kKB];
        matrix_phase(true);
        qk32(sacc, st);
        matrix_phase(false);
        if (needs_mask(kt)) mask32(sacc, kt);
        rescale(0, max32(sacc));
        u32x4_t pb[2 * kKB];
        probs32(sacc, pb);
        matrix_phase(true);
        pv32(pb, st);
        matrix_phase(false);
      } else {   // 16 pairs per wave (D = 256)
        f32x4_t sacc[kCB][kMB];
#pragma unroll
        for (int c = 0; c < kCB; ++c)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) sacc[c][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
          for (int c = 0; c < kCB; ++c) {
            const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(ks + (4 * s + h) * kKChunk + (16 * c + lc) * 16);
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) sacc[c][mb] = mfma16(ka, qb[mb][s], sacc[c][mb]);
          }
        if (needs_mask(kt)) {
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int c = 0; c < kCB; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int key = kt * kKeys + 16 * c + 4 * h + r;
                if (uint32_t(key - lolim[mb]) > uint32_t(span[mb])) sacc[c][mb][r] = -__builtin_inff();
              }
        }
        u32x4_t pb[kMB][kU];   // B operand P^T per (pair block, 32-key step)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
          float tmax = -__builtin_inff();
#pragma unroll
          for (int c = 0; c < kCB; ++c)
            tmax = fmaxf(fmaxf(tmax, fmaxf(sacc[c][mb][0], sacc[c][mb][1])), fmaxf(sacc[c][mb][2], sacc[c][mb][3]));
          rescale(mb, rows_max(tmax) * scale_log2);
          const float nm = -mrun[mb];
          float lsum = lrun[mb];
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const f32x4_t& a0 = sacc[2 * u][mb];
            const f32x4_t& a1 = sacc[2 * u + 1][mb];
            pb[mb][u] = softmax8(a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3], nm, lsum);
          }
          lrun[mb] = lsum;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            const char* vrow = vs + (16 * db + lc) * kVRow;
            const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow + (32 * u + 4 * h) * 2);
            const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + (32 * u + 16 + 4 * h) * 2);
            const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) acc[mb][db] = mfma16(va, pb[mb][u], acc[mb][db]);
          }
      }
    };

    __syncthreads();   // the previous item is done with both stages
    if constexpr (W == 8) {
      // ---- two groups of four waves taking turns on the matrix cores -----------------
      // Group g (waves 4g .. 4g+3) runs phase t - g in tick t: phase 2i is the
      // products of tile i (P.V of tile i-1, then Q.K^T of tile i) and phase
      // 2i+1 its softmax (mask, max, rescale, P), so in every tick one wave per
      // SIMD feeds the matrix cores while the other does its vector work.  Every
      // tick ends at a barrier, and every wave runs the same 2T + 2 ticks.  The
      // two groups share the staged tiles: at the end of tick 2j group 0 writes
      // K of tile j+1 (wave w: unit w) and group 1 V of tile j (wave 4+w: unit
      // w), tile i in stage i & 1.  Phase 2i reads K of tile i and V of tile
      // i-1, in ticks 2i and 2i+1, and nothing writes those stage halves then.
      // A wave issues the loads of its next share right after writing one, two
      // ticks before they are written.  Each wave computes the same pairs with
      // the same arithmetic as a wave of the one-tile-at-a-time loop below.
      static_assert(W != 8 || kM32, "8-wave items need 32 pairs per wave");
      const int grp = wave >> 2;
      const int T = kt1 - kt0;
      Raw r[kNK];
      f32x16_t sacc[kKB];
      u32x4_t pb[2 * kKB];
      // phase 2i: the products of tile i (i = 0 .. T)
      auto gemm = [&](int i) {
        if (i >= 1) pv32(pb, (i - 1) & 1);
        if (i < T) qk32(sacc, i & 1);
      };
      // phase 2i+1: the softmax of tile i
      auto valu = [&](int i) {
        if (needs_mask(kt0 + i)) mask32(sacc, kt0 + i);
        rescale(0, max32(sacc));
        probs32(sacc, pb);
      };
      // Both groups run one loop body; group 1 enters it one tick late (its
      // idle first tick writes V of tile 0) and skips the loop's last barrier,
      // so every wave passes the same 2T + 3 barriers.
      const bool kpart = grp == 0;
      const char* pbase = kpart ? kbase : vbase;
      load_part(r, kt0, phys_of(kt0), pbase, kpart);
      if (kpart) {
        write_k(r, kt0, 0);
        load_part(r, kt0 + 1, phys_of(kt0 + 1), kbase, true);
      }
      uint64_t ph_next = phys_of(kt0 + (kpart ? 2 : 1));
      __syncthreads();
      if (!kpart) {   // tick 0 of group 1
        write_v(r, kt0, 0);
        load_part(r, kt0 + 1, ph_next, vbase, false);
        ph_next = phys_of(kt0 + 2);
        __syncthreads();
      }
      for (int j = 0; j <= T; ++j) {
        gemm(j);   // tick 2j (group 0), 2j + 1 (group 1)
        if (kpart) {
          write_k(r, kt0 + j + 1, (j + 1) & 1);
          load_part(r, kt0 + j + 2, ph_next, kbase, true);
          ph_next = phys_of(kt0 + j + 3);
        }
        __syncthreads();
        if (j < T) {
          valu(j);   // tick 2j + 1 (group 0), 2j + 2 (group 1)
          if (!kpart) {
            write_v(r, kt0 + j + 1, (j + 1) & 1);
            load_part(r, kt0 + j + 2, ph_next, vbase, false);
            ph_next = phys_of(kt0 + j + 3);
          }
        }
        if (kpart || j < T) __syncthreads();
      }
    } else {
      // Registers one or two tiles ahead.  With two register sets (where they
      // fit without spills: D <= 128 on 16- and 32-token blocks), tile kt+2 is
      // fetched while tile kt is computed from its stage and tile kt+1, fetched a
      // step earlier, is written to the other stage, so each load has two tiles
      // of compute to arrive; with one set, tile kt+1 is fetched and staged in
      // the step of tile kt.  Each barrier separates the staging write of a
      // stage from the computes that read it, before and after.  The loop is
      // unrolled by the two stages (tile kt is in stage (kt - kt0) & 1), so every
      // LDS address is a base plus an immediate offset.
      constexpr int kAhead = (D <= 128 && BS != 8) ? 2 : 1;
      TileRegs<D, F8> rg0, rg1;
      uint64_t ph_next = phys_of(kt0 + kAhead);
      fetch(rg0, kt0, phys_of(kt0));
      if constexpr (kAhead == 2) fetch(rg1, kt0 + 1, phys_of(kt0 + 1));
      stage_write(rg0, kt0, 0);
      __syncthreads();
      auto step = [&](int kt, TileRegs<D, F8>& free_rg, TileRegs<D, F8>& next_rg, auto st) {
        TileRegs<D, F8>& fetch_rg = kAhead == 2 ? free_rg : rg0;
        TileRegs<D, F8>& stage_rg = kAhead == 2 ? next_rg : rg0;
        fetch(fetch_rg, kt + kAhead, ph_next);
        ph_next = phys_of(kt + kAhead + 1);
        compute(kt, st);
        if (kt + 1 < kt1) stage_write(stage_rg, kt + 1, st ^ 1);
        __syncthreads();
      };
      if constexpr (D == 256 && BS == 8) {
        // not unrolled: the unrolled loop needs more registers than this shape has
        for (int kt = kt0; kt < kt1; ++kt) {
          const int st = (kt - kt0) & 1;
          fetch(rg0, kt + 1, ph_next);
          ph_next = phys_of(kt + 2);
          compute(kt, st);
          if (kt + 1 < kt1) stage_write(rg0, kt + 1, st ^ 1);
          __syncthreads();
        }
      } else {
        for (int kt = kt0; kt < kt1; kt += 2) {
          step(kt, rg0, rg1, std::integral_constant<int, 0>{});
          if (kt + 1 >= kt1) break;
          step(kt + 1, rg1, rg0, std::integral_constant<int, 1>{});
        }
      }
    }

    // A lane's output values come in runs of 4 consecutive d: run x of pair mb
    // starts at d = run_d(x) and holds run_v(mb, x).
    constexpr int kRuns = kM32 ? 4 * kAB : kAB;
    auto run_d = [&](int x) { return kM32 ? 32 * (x >> 2) + 8 * (x & 3) + 4 * hf : 16 * x + 4 * h; };
    auto run_v = [&](int mb, int x) -> f32x4_t {
      if constexpr (kM32) {
        const f32x16_t& v = acc[mb][x >> 2];
        const int r = 4 * (x & 3);
        return f32x4_t{v[r], v[r + 1], v[r + 2], v[r + 3]};
      } else {
        return acc[mb][x];
      }
    };
    // the pair's sum over every key: lanes l, l^32 (32-pair) or the four rows
    auto pair_sum = [&](float v) { return kM32 ? halves_sum(v) : rows_sum(v); };
    if (split) {
      // unnormalised partial output and (max, sum) of this partition
#pragma unroll
      for (int mb = 0; mb < kNP; ++mb) {
        const float lsum = pair_sum(lrun[mb]) * (F8 ? PA_KARG(lsum_scale) : 1.f);
        if (mvalid[mb]) {
          const int64_t idx = (int64_t(PA_KARG(num_seqs) + q0 + jrow[mb]) * PA_KARG(num_q_heads) + hq[mb]) *
                                  PA_KARG(max_parts) +
                              (part - p_lo);
          float* po = PA_KARG(ws_o) + idx * D;
#pragma unroll
          for (int x = 0; x < kRuns; ++x) *reinterpret_cast<f32x4_t*>(po + run_d(x)) = run_v(mb, x);
          if ((kM32 ? hf : h) == 0) *reinterpret_cast<float2*>(PA_KARG(ws_ml) + 2 * idx) = make_float2(mrun[mb], lsum);
        }
      }
    } else {
      // ---- normalise and store --------------------------------------------------
#pragma unroll
      for (int mb = 0; mb < kNP; ++mb) {
        const float inv = 1.f / (pair_sum(lrun[mb]) * (F8 ? PA_KARG(lsum_scale) : 1.f));
        if (mvalid[mb]) {
          __bf16* orow =
              static_cast<__bf16*>(PA_KARG(out)) + int64_t(q0 + jrow[mb]) * PA_KARG(o_row_stride) + int64_t(hq[mb]) * D;
#pragma unroll
          for (int x = 0; x < kRuns; ++x) {
            const f32x4_t v = run_v(mb, x);
            const u32x2_t o = {pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
            *reinterpret_cast<u32x2_t*>(orow + run_d(x)) = o;
          }
        }
      }
    }
    if (claim_items) {   // the item claimed when this one started
      if (tid == 0) s_next = ngroups + claimed;
      __syncthreads();
      t = uni(s_next);
    } else {   // the next round of the static deal; later rounds only hold larger indices
      ++round;
      t = round * ngroups + ((round & 1) ? ngroups - 1 - wg : wg);
    }
  }
  // With claims, every workgroup counts itself out once its last claim has
  // returned; the last one re-arms the claim counter (and this count), so the
  // next launch on the same list starts from zero.  No claim of this launch is
  // in flight then.
  if (claim_items && tid == 0 &&
      __hip_atomic_fetch_add(done_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngroups - 1) {
    __hip_atomic_store(claim_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int G, int W, int BS, int D, bool F8>
int prefill_groups() {
  static std::atomic<int> cache{0};
  int v = cache.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0, cus = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, prefill_kernel<G, W, BS, D, F8>, Shape<W, D>::kThreads,
                                                   Shape<W, D>::kLdsBytes) != hipSuccess ||
      occ <= 0)
    occ = 1;
  v = cus * occ;
  cache.store(v, std::memory_order_relaxed);
  return v;
}

template <int G, int W, int BS, int D, bool F8>
hipError_t launch_g(const PrefillArgs& a, hipStream_t stream) {
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(prefill_kernel<G, W, BS, D, F8>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, Shape<W, D>::kLdsBytes);
  if (attr != hipSuccess) return attr;
  using Sh = Shape<W, D>;
  const int groups = prefill_groups<G, W, BS, D, F8>();
  hipLaunchKernelGGL((prefill_kernel<G, W, BS, D, F8>), dim3(groups), dim3(Sh::kThreads), Sh::kLdsBytes, stream, a);
  return hipGetLastError();
}

}  // namespace

// A group that is not a power of two (D = 128 only) takes items of the next
// power of two, 8 at most, with padding head slots: 3 heads in items of 4, 5 to
// 7 in items of 8, 9 to 15 in two items of 8.
int prefill_item_group(int group) {
  if (group >= 8) return 8;
  int gi = 1;
  while (gi < group) gi <<= 1;
  return gi;
}

bool prefill_supported(int head_dim, int group, int block_size) {
  const bool pow2 = group >= 1 && group <= 64 && (group & (group - 1)) == 0;
  const bool padded = head_dim == 128 && group >= 3 && group < 16;
  return (head_dim == 64 || head_dim == 128 || head_dim == 256) && (pow2 || padded) &&
         (block_size == 8 || block_size == 16 || block_size == 32);
}

template <int W, int BS, int D, bool F8>
hipError_t launch_w(int group, const PrefillArgs& a, hipStream_t stream) {
  switch (group) {
    case 1: return launch_g<1, W, BS, D, F8>(a, stream);
    case 2: return launch_g<2, W, BS, D, F8>(a, stream);
    case 4: return launch_g<4, W, BS, D, F8>(a, stream);
    case 8: return launch_g<8, W, BS, D, F8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int W, int D, bool F8>
hipError_t launch_b(int group, const PrefillArgs& a, hipStream_t stream) {
  switch (a.block_size) {
    case 8: return launch_w<W, 8, D, F8>(group, a, stream);
    case 16: return launch_w<W, 16, D, F8>(group, a, stream);
    case 32: return launch_w<W, 32, D, F8>(group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

// W waves of 16 * kMB pairs each: 256 / 64 pairs per entry (32 per wave), or
// 64 / 32 at D = 256 (16 per wave).  A 256-pair entry is one 8-wave item, or
// beside the decode kernel two 4-wave items.
template <int D, bool F8>
hipError_t launch_d(int group, const PrefillArgs& a, hipStream_t stream) {
  const int per_wave = D == 256 ? 16 : 32;
  if (a.tile_pairs == 2 * per_wave) return launch_b<2, D, F8>(group, a, stream);
  if (a.tile_pairs == 4 * per_wave) return launch_b<4, D, F8>(group, a, stream);
  if constexpr (D != 256) {
    if (a.tile_pairs == 8 * per_wave)
      return a.claim_items ? launch_b<4, D, F8>(group, a, stream) : launch_b<8, D, F8>(group, a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(int head_dim, int group, bool fp8_cache, const PrefillArgs& a, hipStream_t stream) {
  if (!prefill_supported(head_dim, group, a.block_size)) return hipErrorInvalidValue;
  const int gi = prefill_item_group(group);
  PrefillArgs b = a;
  b.head_split_log2 = 0;
  while ((gi << b.head_split_log2) < group) ++b.head_split_log2;
  if (fp8_cache) {
    if (head_dim == 128) return launch_d<128, true>(gi, b, stream);
    if (head_dim == 64) return launch_d<64, true>(gi, b, stream);
    return launch_d<256, true>(gi, b, stream);
  }
  if (head_dim == 128) return launch_d<128, false>(gi, b, stream);
  if (head_dim == 64) return launch_d<64, false>(gi, b, stream);
  return launch_d<256, false>(gi, b, stream);
}

int prefill_tile_pairs(int head_dim, bool short_rows) {
  if (head_dim == 256) return short_rows ? 32 : 64;
  return short_rows ? 64 : 256;
}

}  // namespace pa
