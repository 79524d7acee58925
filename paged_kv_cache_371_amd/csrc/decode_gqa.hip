// Split-K paged attention for single-row (decode) requests, bf16, D = 64, 128
// or 256 (G <= 2).
//
// quant67, "PagedAttention 与 Continuous Batching" §3.6: the kernel walks the
// request's block table, loads each physical block's K/V and folds it into an
// online softmax; §3.7 fixes 16 tokens per block.  This is the bandwidth-bound
// half of the path (every decode step reads the whole context once), so the
// design goal is bytes in flight and few VALU instructions per byte.
//
// Work split: one wave per work item (request, KV head, context partition);
// the wave streams the partition's 16-token tiles and serves ALL G query
// heads of the KV head, so each K/V byte enters the chip once and is used G
// times from registers.  Items come from a device-built list (largest first):
// the first round is dealt statically, the rest is claimed at run time (see
// below).
//
// Lane layout for one 16-token tile of one KV head (16 rows of D elements,
// contiguous): lane l = 16*tg + r loads the E = D/16 elements of d-slice
// [E r, E r + E) of token 4*i + tg, for load slots i = 0..3 (16 B per lane at
// D = 128, 8 B at D = 64, 32 B as two loads at D = 256).  Every load instruction reads 64 E elements of
// consecutive memory.  Loads are raw buffer loads whose descriptor spans exactly one tile;
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
// End of the partition: the 4 token rows of the wave are combined with
// v_permlane32_swap / v_permlane16_swap (a reduce-scatter, fixed order, so
// the result is deterministic).  A request whose context fits in one
// partition is normalised and stored as bf16 (round to nearest even); else
// the partition's (max, sum, unnormalised output) go to the workspace and the
// merge kernel combines them.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "pa_common.h"
#include "pa_internal.h"

#ifndef PA_DECODE_RING
#define PA_DECODE_RING 3
#endif

namespace pa {
namespace {

// Worker waves per workgroup (each workgroup also has one scheduler wave).
// Four by default.  Three where a prefill launch runs beside this one and no
// KV head is split over items: a workgroup is then four waves, one per SIMD,
// and a four-wave prefill workgroup fits on the same CU (184 + 256 of the 512
// registers per lane of each SIMD), where five would leave one SIMD without
// room for it.
constexpr int kWorkersDefault = 4;
constexpr int kWorkersBesidePrefill = 3;
constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr float kRescaleThreshold = 8.f;      // log2 units
constexpr float kMinusBig = -1e30f;           // finite "no token yet" max
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr int kMaxDevices = 64;
#ifndef PA_DECODE_RING_FP8
#define PA_DECODE_RING_FP8 6
#endif
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(8))) uint32_t u32x8_t;

// Cache element types.  bf16: a lane loads 16 bytes (8 elements) per load
// slot.  OCP FP8 E4M3: a lane loads 8 bytes (the same 8 elements) and widens
// them to bf16 pairs with v_cvt_scalef32_pk_bf16_fp8 (exact: every E4M3 value
// is a bf16 value); the per-tensor scales are folded into the softmax scale
// and the output normalisation.
//
// Tiles in flight per wave (kRing): one workgroup per CU (one worker wave per
// SIMD), so registers go to a deep ring; an 8-bit tile, or a tile of D = 64,
// is half the bytes, so its ring is twice as deep for the same bytes in flight.
template <bool F8, int D>
struct Kv {
  static_assert(D == 64 || D == 128 || D == 256, "head dims 64, 128 and 256");
  static constexpr int kE = D / 16;                                  // elements of a row per lane
  static constexpr int kW = kE / 2;                                  // the same as bf16 pairs
  static constexpr int kTileBytes = kBlock * D * (F8 ? 1 : 2);       // 16 rows of one KV head
  static constexpr int kLoadBytes = kE * (F8 ? 1 : 2);               // per lane and load slot
  // the same bytes in flight for every tile size: twice the tiles at half the
  // bytes; a D = 256 tile (twice the bytes) keeps two in flight
  static constexpr int kRing = D == 256 ? (F8 ? PA_DECODE_RING : 2)
                                        : (F8 ? PA_DECODE_RING_FP8 : PA_DECODE_RING) * (128 / D);
  using Raw = typename std::conditional<
      kLoadBytes == 32, u32x8_t,
      typename std::conditional<kLoadBytes == 16, u32x4_t,
                                typename std::conditional<kLoadBytes == 8, u32x2_t, uint32_t>::type>::type>::type;
  // kE elements as bf16 pairs
  using Words = typename std::conditional<kW == 8, u32x8_t,
                                          typename std::conditional<kW == 4, u32x4_t, u32x2_t>::type>::type;
  static __device__ __forceinline__ Raw load(__amdgpu_buffer_rsrc_t rsrc, int off) {
    if constexpr (kLoadBytes == 32) {
      const u32x4_t lo = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
      const u32x4_t hi = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16, 0, 0);
      return u32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else if constexpr (kLoadBytes == 16) {
      return __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
    } else if constexpr (kLoadBytes == 8) {
      return __builtin_amdgcn_raw_buffer_load_b64(rsrc, off, 0, 0);
    } else {
      return __builtin_amdgcn_raw_buffer_load_b32(rsrc, off, 0, 0);
    }
  }
  template <bool Hi>   // the low or high two codes of w as a bf16 pair
  static __device__ __forceinline__ uint32_t cvt(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, Hi));
  }
  // the lane's kE elements as bf16 pairs
  static __device__ __forceinline__ Words widen(const Raw& w) {
    if constexpr (!F8) {
      return w;
    } else if constexpr (kW == 8) {
      return Words{cvt<false>(w[0]), cvt<true>(w[0]), cvt<false>(w[1]), cvt<true>(w[1]),
                   cvt<false>(w[2]), cvt<true>(w[2]), cvt<false>(w[3]), cvt<true>(w[3])};
    } else if constexpr (kW == 4) {
      return Words{cvt<false>(w[0]), cvt<true>(w[0]), cvt<false>(w[1]), cvt<true>(w[1])};
    } else {
      return Words{cvt<false>(w), cvt<true>(w)};
    }
  }
};
// Paging of the kernel's 16-token tiles onto blocks of BS tokens (8, 16 or
// 32).  A tile's key, kept in scalar registers, names where it lives: BS =
// 16: the block id; BS = 32: block id * 2 + which half of the block; BS = 8:
// the ids of its two blocks (low and high 32 bits), the high one -1 when the
// second block holds no token below tok1 (it may not be owned by the
// request, so neither its table entry past the owned ones nor its memory is
// read).  Tile T covers tokens [16 T, 16 T + 16) and starts below tok1.
template <int BS>
__device__ __forceinline__ int64_t tile_key(const int32_t* table, int T, int tok1) {
  if constexpr (BS == 16) {
    return load_const_early(table, T);
  } else if constexpr (BS == 32) {
    return int64_t(load_const_early(table, T >> 1)) * 2 + (T & 1);
  } else {
    static_assert(BS == 8, "block sizes 8, 16, 32");
    const bool second = T * kBlock + 8 < tok1;
    const int first_id = load_const_early(table, 2 * T);
    const int second_id = load_const_early(table, second ? 2 * T + 1 : 2 * T);
    return int64_t(uint64_t(uint32_t(first_id)) | (uint64_t(uint32_t(second ? second_id : -1)) << 32));
  }
}

#ifndef PA_DECODE_STATIC_ROUNDS
#define PA_DECODE_STATIC_ROUNDS 1
#endif
constexpr int kStaticRounds = PA_DECODE_STATIC_ROUNDS;   // rounds dealt without claims
static_assert(kStaticRounds >= 1, "round 0 is static");
#ifndef PA_DECODE_CLAIM_BATCH
#define PA_DECODE_CLAIM_BATCH 2
#endif
constexpr int kQueue = 16;                         // LDS queue slots of claimed items per workgroup
constexpr int kClaimBatch = PA_DECODE_CLAIM_BATCH; // items per claim
#ifndef PA_DECODE_REQUEST_TILES
#define PA_DECODE_REQUEST_TILES 6
#endif
constexpr int kRequestTiles = PA_DECODE_REQUEST_TILES;   // tiles before an item's end its worker asks for the next

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


typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

// S^T += K Q^T over 32 d (16 keys x 16 head columns).
__device__ __forceinline__ f32x4_t mfma_k32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                  0, 0, 0);
}
// O += P V over 16 keys (16 head rows x 16 d columns).
__device__ __forceinline__ f32x4_t mfma_k16(const u32x2_t& a, const u32x2_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
// Two E4M3 codes as a bf16 pair (exact), the low (Hi = false) or high two of w.
template <bool Hi>
__device__ __forceinline__ uint32_t cvt8(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, Hi));
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

// Dot product of a lane's slices of q and k (N bf16 pairs each).
template <int N, typename V>
__device__ __forceinline__ float dot_bf16(const V& q, const V& k) {
  float s = dot2_bf16(q[0], k[0], 0.f);
#pragma unroll
  for (int i = 1; i < N; ++i) s = dot2_bf16(q[i], k[i], s);
  return s;
}


// Geometry of one work item: (request b, head group hg, partition part) of a
// single-row request, served by one wave.  All fields are wave-uniform.
struct Item {
  int valid;
  int b, hg, q0;   // hg: head group, the item's index among its request's items of one partition
  int h0, gv;      // the item's query heads: h0 .. h0 + gv - 1 (gv < G: the rest are padding)
  int parts;     // partition index among the request's visible partitions (the partial
                 // slot) | their count << 16
  int lo;        // first visible key (sliding window), 0 without one
  int tok1;      // end of the partition's tokens
  int lb0;       // first logical block of the partition
  int nb;        // blocks (tiles) in the partition; >= 1 for a valid item
  int nbr;       // nb rounded up to a multiple of kRing (the item's stream length)
  const int32_t* table;
  const char* kbase;
  const char* vbase;
};


// Item t of the list plan_kernel built: entry t / H, head group t % H of the
// H = Hkv * 2^head_split_log2 groups of up to G query heads; the group's KV head is
// its index >> head_split_log2.  A KV head's Hq / Hkv query heads are cut into
// groups of G in order; where Hq / Hkv is not a multiple of G (a group that is
// not a power of two) the last group of a KV head has fewer, and its other
// head slots are padding (zero q, nothing written).  An index past the list
// gives a placeholder with in-range addresses and no tiles.  Every field goes
// through readfirstlane, so the descriptors and table loads built from it stay scalar.
template <bool F8, int BS, int D>
__device__ __forceinline__ Item make_item(const DecodeArgs& a, int total, int t, int4 ent, int G) {
  constexpr int kRing = Kv<F8, D>::kRing;
  constexpr int kHeadBytes = BS * D * (F8 ? 1 : 2);   // one KV head's rows of a block
  Item it;
  it.valid = t < total;
  int b = 0, part = 0, q0 = 0, L = 1, hg = 0;
  if (it.valid) {
    hg = t % (a.num_kv_heads << a.head_split_log2);
    b = ent.x;
    part = ent.y;
    q0 = ent.z;
    L = ent.w;
  }
  const int P = a.part_size;
  // keys [lo, L) are visible; partitions before lo's have no items
  const int lo = window_start(L - 1, a.sliding_window);
  const int p_lo = lo / P;
  const int tok0 = max(part * P, lo);
  const int tok1 = min(part * P + P, L);
  const int lb0 = tok0 / kBlock;
  const int nb = it.valid ? (tok1 + kBlock - 1) / kBlock - lb0 : 0;
  const int group = a.num_q_heads / a.num_kv_heads;   // query heads per KV head
  const int hsub = hg & ((1 << a.head_split_log2) - 1);
  it.b = uni(b);
  it.hg = uni(hg);
  it.h0 = uni((hg >> a.head_split_log2) * group + hsub * G);
  it.gv = uni(min(G, group - hsub * G));
  it.parts = uni((part - p_lo) | (((L + P - 1) / P - p_lo) << 16));
  it.q0 = uni(q0);
  it.lo = uni(lo);
  it.tok1 = uni(tok1);
  it.lb0 = uni(lb0);
  it.nb = uni(nb);
  it.nbr = uni(kRing * ((nb + kRing - 1) / kRing));
  it.valid = uni(it.valid);
  it.table = uni_ptr(a.block_tables + int64_t(b) * a.max_blocks_per_seq);
  it.kbase = uni_ptr(static_cast<const char*>(a.k_cache) + int64_t(hg >> a.head_split_log2) * kHeadBytes);
  it.vbase = uni_ptr(static_cast<const char*>(a.v_cache) + int64_t(hg >> a.head_split_log2) * kHeadBytes);
  return it;
}

// Persistent kernel.  Each workgroup has WK worker waves, which
// never synchronise with each other, plus one scheduler wave.  The list is
// sorted by decreasing size.  Rounds 0 .. kStaticRounds-1 are dealt
// statically: worker w of NW takes item i*NW + w in even rounds i and
// i*NW + NW-1-w in odd ones.  Later items are claimed from a counter in the
// list header, in list order, so faster workers take more of the small items
// at the end (the 8 XCDs stream at rates up to ~20% apart, which a static
// split cannot absorb).  The scheduler wave makes the claims and hands the
// items to its workgroup's workers through a small LDS queue: under a
// saturated HBM queue a device-scope atomic takes microseconds to return,
// and a worker that issued one would stall its tile stream on it (vector
// memory counters complete in order).
//
// A wave sees its items as one stream of tiles: an item contributes nbr
// stream slots (its nb tiles padded with empty ones to a multiple of kRing), so
// the last load group of an item already fetches the next item's first kRing
// tiles and the HBM queue of the wave never drains at item boundaries.  The
// physical block id of the slot issued next is fetched one issue ahead.
//
// MF: the matrix-core form of the tile math (D = 128, items of 4 or 8 heads).  S^T = K Q^T runs on v_mfma_f32_16x16x32_bf16
// with the tile's 16 keys as rows and the item's heads as columns (padded to
// 16 with zero q), so lane l holds head l % 16's scores of keys 4(l/16) ..
// 4(l/16)+3; those scores, exponentiated and rounded to bf16, are directly the
// A operand of O = P V on v_mfma_f32_16x16x16_bf16, whose B operand is V in
// its stored order: lane l loads keys 4(l/16) .. +3 at d = 8(l%16) .. +7 and
// output column n of product j is d = 8n + j.  K is loaded with key l % 16 per
// lane (the A-operand order), 16 bytes per load; the contraction order over d
// is a fixed permutation shared by K and q.  The VALU work per tile drops from
// ~G * D / 4 dot instructions per lane to the softmax and the operand
// conversions.
template <int G, bool F8, int BS, int D, bool MF, int WK>
__global__ __launch_bounds__(64 * (WK + 1), 1) void decode_gqa_kernel(DecodeArgs a) {
  static_assert(!MF || (D == 128 && (G == 4 || G == 8)), "matrix-core tiles: D = 128, items of 4 or 8 heads");
  static_assert(kClaimBatch <= WK && WK <= kQueue, "one queued item per worker at most");
  // Claims of a KV head's head groups (up to 4 items) start aligned when the
  // static rounds hand out a multiple of 4 items; three workers are launched
  // only where no KV head is split over items.
  static_assert(WK == kWorkersBesidePrefill || kStaticRounds * WK % 4 == 0, "claims of up to 4 items start aligned");
  using T = Kv<F8, D>;
  constexpr int kRing = T::kRing;
  constexpr int kTileBytes = T::kTileBytes;
  constexpr int kE = T::kE;             // elements of a row per lane
  constexpr int kW = T::kW;
  using Words = typename T::Words;
  constexpr int kHeadBytes = BS * D * (F8 ? 1 : 2);   // one KV head's rows of a block
  using Raw = typename T::Raw;
  constexpr int K = log2_of<G>();
  constexpr int kRot = 16 / G;          // lanes between consecutive heads in a row
  constexpr int kNV = G * kE;           // accumulators per lane
  constexpr int kNZ = kNV / 4;          // accumulators per lane after the row reduce-scatter
  constexpr int kRun = kNZ < kE ? kNZ : kE;   // consecutive d values per output run

  const int nh = a.num_kv_heads << a.head_split_log2;   // head groups (work items per list entry)
  const int total = load_const(a.plan, kPlanCountInt) * nh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NW = gridDim.x * WK;
  const int wid = int(blockIdx.x) * WK + wave;
  auto item_of_round = [&](int i) {   // item index of static round i, or total if none
    const int64_t base = int64_t(i) * NW;
    const int64_t t = base + ((i & 1) ? NW - 1 - wid : wid);
    return t < total ? int(t) : total;
  };
  const int64_t dyn0 = int64_t(kStaticRounds) * NW;   // first item handed out by claims
  // List entry of static round i (scalar loads).  The entry index is clamped
  // into the list's capacity instead of checked against the count, so round
  // 0's entry is fetched together with the count at kernel start; make_item
  // discards it when the round has no item.
  auto static_entry = [&](int i) -> int4 {
    const int64_t t = int64_t(i) * NW + ((i & 1) ? NW - 1 - wid : wid);
    const int e = int(min<int64_t>(t / nh, a.plan_capacity - 1));
    const int32_t* ep = a.plan + kPlanHeaderInts + 4 * int64_t(e);
    return make_int4(load_const_early(ep, 0), load_const_early(ep, 1), load_const_early(ep, 2), load_const_early(ep, 3));
  };
  const int4 entry0 = static_entry(0);
  int* claim_counter = a.plan + kPlanClaimInt;
  // Every wave counts itself out when it leaves, in its workgroup's LDS; the
  // workgroup's last wave counts the workgroup out on a device-scope counter,
  // and the last workgroup re-arms the claim counter (and this count) for the
  // next run on the same work list.  Each scheduler's claims have returned
  // their values before it counts out, so when the count completes no claim of
  // this launch is still in flight.  (One device-scope atomic per workgroup,
  // not per wave: a launch whose list is empty has all its waves leave at
  // once, and 1280 atomics on one address took about 13 us.)
  int* done_counter = a.plan + kPlanDoneInt;
  __shared__ int s_out;   // waves of this workgroup that have left
  auto count_out = [&]() {
    if ((threadIdx.x & 63) == 0 &&
        __hip_atomic_fetch_add(&s_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == WK &&
        __hip_atomic_fetch_add(done_counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == int(gridDim.x) - 1) {
      __hip_atomic_store(claim_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(done_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // Queue of claimed items with their list entries.  Slot s receives queue
  // index p = s, s + kQueue, ...; s_qfree[s] is the index it may receive next
  // (the consumer of index p sets it to p + kQueue once it has read the
  // item), so the scheduler never overwrites an item that has not been taken.
  __shared__ int s_qitem[kQueue];
  __shared__ int4 s_qent[kQueue];
  __shared__ int s_qfree[kQueue];
  __shared__ int s_qhead;   // queue indices handed to workers
  __shared__ int s_qtail;   // queue indices filled
  __shared__ int s_qend;    // final number of filled indices, once known
  __shared__ int s_qreq;    // requests made by the workers
  if (threadIdx.x < kQueue) s_qfree[threadIdx.x] = threadIdx.x;
  if (threadIdx.x == 0) {
    s_qreq = 0;
    s_qhead = 0;
    s_qtail = 0;
    s_qend = 0x7fffffff;
    s_out = 0;
  }
  __syncthreads();
  auto lds_load = [](int* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); };
  auto lds_store = [](int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); };
  const int4* entries = reinterpret_cast<const int4*>(a.plan + kPlanHeaderInts);

  if (wave == WK) {   // the scheduler: one claim per batch of requests
    if (lane == 0) {
      const int64_t ndyn = int64_t(total) - dyn0;
      // The items of one KV head's head groups are claimed together (up to
      // one per worker, aligned), so this workgroup's workers stream the same
      // tiles side by side and the repeated reads are served by L2.
      const int unit = min(1 << a.head_split_log2, WK);
      int pushed = 0, served = 0;
      for (bool more = ndyn > 0; more;) {
        int req;
        while ((req = lds_load(&s_qreq)) <= served) __builtin_amdgcn_s_sleep(1);
        const int want = (min(req - served, kClaimBatch) + unit - 1) / unit * unit;
        const int c = __hip_atomic_fetch_add(claim_counter, want, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int n = int(max<int64_t>(0, min<int64_t>(want, ndyn - c)));
        for (int j = 0; j < n; ++j) {
          const int q = pushed + j;
          const int t = int(dyn0 + c + j);
          const int4 e = entries[t / nh];
          while (lds_load(&s_qfree[q % kQueue]) != q) __builtin_amdgcn_s_sleep(1);
          s_qitem[q % kQueue] = t;
          s_qent[q % kQueue] = e;
        }
        pushed += n;
        served += want;
        lds_store(&s_qtail, pushed);
        more = n == want;
      }
      lds_store(&s_qend, pushed);
    }
    count_out();
    return;
  }
  // A worker asks for its next claimed item (once per item, before taking it).
  auto request = [&]() {
    if (lane == 0) __hip_atomic_fetch_add(&s_qreq, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // Next claimed item for this worker (index and list entry); index total
  // when there is none left.
  auto take = [&](int& t, int4& e) {
    int q = 0;
    if (lane == 0) q = __hip_atomic_fetch_add(&s_qhead, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    q = uni(q);
    for (;;) {
      if (q < uni(lds_load(&s_qtail))) {
        t = uni(s_qitem[q % kQueue]);
        const int4 v = s_qent[q % kQueue];
        e = make_int4(uni(v.x), uni(v.y), uni(v.z), uni(v.w));
        if (lane == 0) lds_store(&s_qfree[q % kQueue], q + kQueue);
        return;
      }
      if (q >= uni(lds_load(&s_qend))) {
        t = total;
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };

  const int r = lane & 15;
  const int tg = lane >> 4;
  const int hr = r >> (4 - K);
  const int voff = tg * D * (F8 ? 1 : 2) + r * T::kLoadBytes;   // token tg of the slot, d-slice r
  const int64_t bstride = int64_t(a.num_kv_heads) * kHeadBytes;   // bytes per physical block
  const float scale_log2 = a.scale_log2;
  // direction of row_ror within a row: the head of accumulator slot j is (hr + dir*j) mod G
  int dir = 1;
  if constexpr (G > 1) {
    const int src = int(dpp_u32<0x120 + kRot>(uint32_t(r)));
    dir = ((src >> (4 - K)) == ((hr + 1) & (G - 1))) ? 1 : -1;
  }

  // Each wave stages the next item's q rows in its own LDS slot: fetched into a
  // few VGPRs when the item starts (not used by the tile loop, so the loop
  // never waits for them) and moved to qreg through LDS after the item.
  constexpr int kQD = G * D / 2;                    // q dwords of an item: G rows of D bf16
  constexpr int kQDw = kQD >= 64 ? kQD / 64 : 1;    // per lane (lanes >= kQD idle when kQD < 64)
  __shared__ uint32_t sq[WK][64 * kQDw];
  // (padding heads of the item read nothing and park zeros)
  auto fetch_q = [&](const Item& it, uint32_t(&qt)[kQDw]) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(
        static_cast<const char*>(a.q) + (int64_t(it.q0) * a.q_row_stride + int64_t(it.h0) * D) * 2);
    if constexpr (kQDw >= 4) {
      // a lane's dwords lie in one head's row (kQDw divides D / 2)
      const bool live = lane * kQDw / (D / 2) < it.gv;
#pragma unroll
      for (int c = 0; c < kQDw / 4; ++c) {
        const u32x4_t v = live ? reinterpret_cast<const u32x4_t*>(src)[lane * (kQDw / 4) + c] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int w = 0; w < 4; ++w) qt[4 * c + w] = v[w];
      }
    } else {
#pragma unroll
      for (int c = 0; c < kQDw; ++c) {
        const int i = lane * kQDw + c;
        qt[c] = i < kQD && i / (D / 2) < it.gv ? src[i] : 0u;
      }
    }
  };
  auto park_q = [&](const uint32_t(&qt)[kQDw]) {
#pragma unroll
    for (int c = 0; c < kQDw; ++c) sq[wave][lane * kQDw + c] = qt[c];
  };
  auto read_q = [&](Words(&qreg)[G]) {   // q slices, lane-relative order h(r ^ M_j)
    const char* base = reinterpret_cast<const char*>(&sq[wave][0]);
    static_for<G>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int hh = (r ^ q_mask<K>(j)) >> (4 - K);
      qreg[j] = *reinterpret_cast<const Words*>(base + hh * (D * 2) + r * (kE * 2));
    });
  };

  Item cur = make_item<F8, BS, D>(a, total, item_of_round(0), entry0, G);
  if (!cur.valid) {
    count_out();
    return;
  }

  // ---- matrix-core form: lane geometry and q operands ----------------------------
  constexpr int kEB = F8 ? 1 : 2;                  // bytes per cached element
  constexpr int kKLoads = F8 ? 2 : 4;              // 16-byte K loads per lane and tile
  const int mrow = lane & 15;                      // MFMA row / column of the lane
  const int mg = lane >> 4;                        // its group of 4 (k slots, output rows)
  const int kmf_off = mrow * (D * kEB) + 16 * mg;  // K: key mrow, then + 64 per load
  const int vmf_off = 4 * mg * (D * kEB) + 8 * mrow * kEB;   // V: key 4 mg, d 8 mrow; + D*kEB per key
  // d of element 0 of the lane's K (and q) operand of 32-d step st: bf16 loads hold
  // d 8 mg + 32 st; 8-bit loads hold 16 codes, d 16 mg + 64 (st / 2), split in halves
  auto mf_d0 = [&](int st) { return F8 ? 16 * mg + 64 * (st >> 1) + 8 * (st & 1) : 8 * mg + 32 * st; };
  // registers of one tile as loaded: K, V
  using KR = typename std::conditional<MF, u32x4_t, Raw>::type;
  using VR = typename std::conditional<MF, typename std::conditional<F8, u32x2_t, u32x4_t>::type, Raw>::type;
  constexpr int kKR = MF ? kKLoads : 4;
  u32x4_t qmf[4];   // B operand of step st: head mrow's q at d mf_d0(st) .. +7, zero for padding heads
  auto q_mf_from = [&](const char* rows, int gv) {   // rows: the item's gv q rows of D bf16
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qmf[st] = mrow < gv ? *reinterpret_cast<const u32x4_t*>(rows + mrow * (D * 2) + mf_d0(st) * 2)
                          : u32x4_t{0u, 0u, 0u, 0u};
  };

  // The dot-product form serves groups that are powers of two only (padding
  // head slots exist only in the matrix-core form), so there h0 = hg * G and gv = G.
  auto load_q = [&](Words(&qreg)[G], const Item& it) {   // q slices, lane-relative order h(r ^ M_j)
    const char* qrow =
        static_cast<const char*>(a.q) + (int64_t(it.q0) * a.q_row_stride + int64_t(it.hg) * G * D) * 2;
    static_for<G>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const int hh = (r ^ q_mask<K>(j)) >> (4 - K);
      qreg[j] = *reinterpret_cast<const Words*>(qrow + hh * (D * 2) + r * (kE * 2));
    });
  };
  // Load slot i reads rows 4i .. 4i+3 of the tile.  With BS = 8 slots 0, 1
  // read the first block and slots 2, 3 the second (rows 0..7 of each).
  auto load_tile = [&](KR(&kb)[kKR], VR(&vb)[4], const char* kbase, const char* vbase, bool live, int64_t key) {
    if constexpr (MF && BS == 8) {
      // Keys 0..7 of the tile are rows 0..7 of the first block, keys 8..15 of
      // the second.  Each lane reads its rows from both blocks at row index
      // r (first) and r ^ 8 (second): exactly one of the two lies inside its
      // block's 8-row range, the other reads past it and returns zeros without
      // touching memory, so the OR of the two is the lane's data.
      const int64_t id0 = int64_t(uint32_t(uint64_t(key)));
      const int id1 = int(uint32_t(uint64_t(key) >> 32));
      const int nrec0 = live ? kHeadBytes : 0;
      const int nrec1 = live && id1 >= 0 ? kHeadBytes : 0;
      const int64_t off1 = int64_t(id1 >= 0 ? id1 : 0) * bstride;
      const __amdgpu_buffer_rsrc_t rk0 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + id0 * bstride), 0, nrec0, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rk1 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + off1), 0, nrec1, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv0 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + id0 * bstride), 0, nrec0, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv1 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + off1), 0, nrec1, kRsrcWord3);
      constexpr int kRow = D * kEB;
      const int k_alt = kmf_off ^ (8 * kRow);   // key row mrow ^ 8
#pragma unroll
      for (int i = 0; i < kKR; ++i)
        kb[i] = __builtin_amdgcn_raw_buffer_load_b128(rk0, kmf_off + 64 * i, 0, 0) |
                __builtin_amdgcn_raw_buffer_load_b128(rk1, k_alt + 64 * i, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // key 4 mg + i: rows 0..7 of block 0 for mg < 2, else of block 1
        const int v0 = vmf_off + i * kRow;
        const int v1 = v0 ^ (8 * kRow);
        if constexpr (F8)
          vb[i] = __builtin_amdgcn_raw_buffer_load_b64(rv0, v0, 0, 0) | __builtin_amdgcn_raw_buffer_load_b64(rv1, v1, 0, 0);
        else
          vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rv0, v0, 0, 0) |
                  __builtin_amdgcn_raw_buffer_load_b128(rv1, v1, 0, 0);
      }
    } else if constexpr (MF) {
      const int64_t off = BS == 32 ? (key >> 1) * bstride + (key & 1) * kTileBytes : key * bstride;
      const int nrec = live ? kTileBytes : 0;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + off), 0, nrec, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + off), 0, nrec, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kKR; ++i) kb[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, kmf_off + 64 * i, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (F8)
          vb[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, vmf_off + i * (D * kEB), 0, 0);
        else
          vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vmf_off + i * (D * kEB), 0, 0);
      }
    } else if constexpr (BS == 8) {
      const int64_t id0 = int64_t(uint32_t(uint64_t(key)));
      const int id1 = int(uint32_t(uint64_t(key) >> 32));
      const int nrec0 = live ? kHeadBytes : 0;
      const int nrec1 = live && id1 >= 0 ? kHeadBytes : 0;
      const int64_t off1 = int64_t(id1 >= 0 ? id1 : 0) * bstride;
      const __amdgpu_buffer_rsrc_t rk0 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + id0 * bstride), 0, nrec0, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rk1 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + off1), 0, nrec1, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv0 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + id0 * bstride), 0, nrec0, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv1 =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + off1), 0, nrec1, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i) kb[i] = T::load(i < 2 ? rk0 : rk1, voff + (i & 1) * (kTileBytes / 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) vb[i] = T::load(i < 2 ? rv0 : rv1, voff + (i & 1) * (kTileBytes / 4));
    } else {
      const int64_t off = BS == 32 ? (key >> 1) * bstride + (key & 1) * kTileBytes : key * bstride;
      const int nrec = live ? kTileBytes : 0;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase + off), 0, nrec, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase + off), 0, nrec, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i) kb[i] = T::load(rk, voff + i * (kTileBytes / 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) vb[i] = T::load(rv, voff + i * (kTileBytes / 4));
    }
  };

  Words qreg[G];
  // the ring: K and V of kRing tiles, as loaded
  KR kr[kRing][kKR];
  VR vr[kRing][4];
  if constexpr (MF)
    q_mf_from(static_cast<const char*>(a.q) + (int64_t(cur.q0) * a.q_row_stride + int64_t(cur.h0) * D) * 2, cur.gv);
  else
    load_q(qreg, cur);
  int64_t ph0[kRing];   // keys of the first tiles, all requested before any is used
  static_for<kRing>([&](auto S) {
    constexpr int st = decltype(S)::value;
    ph0[st] = tile_key<BS>(cur.table, cur.lb0 + min(st, cur.nb - 1), cur.tok1);
  });
  __builtin_amdgcn_sched_barrier(0);
  static_for<kRing>([&](auto S) {
    constexpr int st = decltype(S)::value;
    load_tile(kr[st], vr[st], cur.kbase, cur.vbase, st < cur.nb, ph0[st]);
    __builtin_amdgcn_sched_barrier(0);
  });

  for (int i = 0;; ++i) {
    // The next item.  A static one is known now.  A claimed one is requested
    // kRequestTiles tiles before this item ends and taken at the start of its
    // second-to-last load group, just before its first block ids are needed,
    // so it is handed out as late as the tile stream allows.
    const bool dyn = i + 1 >= kStaticRounds;
    Item nxt = make_item<F8, BS, D>(a, total, total, make_int4(0, 0, 0, 1), G);
    uint32_t qt[kQDw];
    bool requested = false;
    auto get_next = [&]() {
      if (!requested) request();
      requested = true;
      int t;
      int4 e;
      take(t, e);
      nxt = make_item<F8, BS, D>(a, total, t, e, G);
      if (nxt.valid) fetch_q(nxt, qt);
    };
    if (!dyn) {
      nxt = make_item<F8, BS, D>(a, total, item_of_round(i + 1), static_entry(i + 1), G);
      if (nxt.valid) fetch_q(nxt, qt);
    } else if (cur.nb <= 2 * kRing) {
      get_next();
    }
    __builtin_amdgcn_sched_barrier(0);

    float acc[G][kE];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[j][e] = 0.f;
    float m = kMinusBig;   // reference max of this lane's (row, head), log2 units
    float l = 0.f;         // sum of rounded p relative to m

    // Stream slot j of this item: its own tile j, or tile j - nbr of the next
    // item.  Every field is a scalar select, so a slot costs one scalar load.
    auto slot_phys = [&](int j) -> int64_t {
      const bool own = j < cur.nbr;
      const int jj = own ? j : j - cur.nbr;
      const int32_t* tb = own ? cur.table : nxt.table;
      const int lb0 = own ? cur.lb0 : nxt.lb0;
      const int nbl = own ? cur.nb : nxt.nb;
      return tile_key<BS>(tb, lb0 + max(min(jj, nbl - 1), 0), own ? cur.tok1 : nxt.tok1);
    };
    int64_t pf = slot_phys(kRing);   // tile key of the next slot to issue
    auto issue = [&](KR(&kb)[kKR], VR(&vb)[4], int j) {
      const int64_t phys = pf;
      pf = slot_phys(j + 1);
      const bool own = j < cur.nbr;
      const int jj = own ? j : j - cur.nbr;
      const int nbl = own ? cur.nb : nxt.nb;
      load_tile(kb, vb, own ? cur.kbase : nxt.kbase, own ? cur.vbase : nxt.vbase, jj < nbl, phys);
    };

    // matrix-core form: O accumulators (product j: rows heads 4 mg .. +3, column
    // mrow = d 8 mrow + j) and the tile step
    f32x4_t oacc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto process_mf = [&](auto& kraw, auto& vraw, int k) {   // generic: instantiated only where called
      f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        u32x4_t ka;
        if constexpr (F8) {
          const u32x4_t& w = kraw[st >> 1];
          ka = (st & 1) ? u32x4_t{cvt8<false>(w[2]), cvt8<true>(w[2]), cvt8<false>(w[3]), cvt8<true>(w[3])}
                        : u32x4_t{cvt8<false>(w[0]), cvt8<true>(w[0]), cvt8<false>(w[1]), cvt8<true>(w[1])};
        } else {
          ka = kraw[st];
        }
        s4 = mfma_k32(ka, qmf[st], s4);
      }
      const int tb = (cur.lb0 + k) * kBlock;   // first token of the tile
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = s4[i] * scale_log2;   // key tb + 4 mg + i, head mrow
      using VV = std::remove_cv_t<std::remove_reference_t<decltype(vraw[0])>>;   // VR (dependent)
      VV vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = vraw[i];
      if (tb + kBlock > cur.tok1 || tb < cur.lo) {   // the context ends, or the window starts, in this tile
        const uint32_t span = uint32_t(cur.tok1 - cur.lo);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = uint32_t(tb + 4 * mg + i - cur.lo) >= span;
          sc[i] = dead ? -__builtin_inff() : sc[i];
          vv[i] = dead ? VV{} : vv[i];   // rows past the context may hold anything
        }
      }
      // every lane: the tile max of head mrow (its 4 keys, then the 4 lane groups)
      const float bm = rows_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
      if (__builtin_amdgcn_ballot_w64(bm > m + kRescaleThreshold)) {
        const float mn = fmaxf(m, bm);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {   // output row i of the lane is head 4 mg + i
          const float ai = __shfl(alpha, 4 * mg + i);
#pragma unroll
          for (int j = 0; j < 8; ++j) oacc[j][i] *= ai;
        }
      }
      const u32x2_t pa = {pack_bf16x2(fast_exp2(sc[0] - m), fast_exp2(sc[1] - m)),
                          pack_bf16x2(fast_exp2(sc[2] - m), fast_exp2(sc[3] - m))};
      l = dot2_bf16(pa[0], kBf16OnePair, l);
      l = dot2_bf16(pa[1], kBf16OnePair, l);
      // B operand of product j: keys 4 mg .. +3 at d 8 mrow + j, as two bf16 pairs
      if constexpr (F8) {
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
          for (int b = 0; b < 4; b += 2) {
            // codes b, b+1 of word w of keys (0, 1) and (2, 3), interleaved by key
            const uint32_t sel = b == 0 ? 0x05010400u : 0x07030602u;
            const uint32_t x01 = __builtin_amdgcn_perm(vv[1][w], vv[0][w], sel);
            const uint32_t x23 = __builtin_amdgcn_perm(vv[3][w], vv[2][w], sel);
            const int j = 4 * w + b;
            oacc[j] = mfma_k16(pa, u32x2_t{cvt8<false>(x01), cvt8<false>(x23)}, oacc[j]);
            oacc[j + 1] = mfma_k16(pa, u32x2_t{cvt8<true>(x01), cvt8<true>(x23)}, oacc[j + 1]);
          }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          const u32x2_t vb = {__builtin_amdgcn_perm(vv[1][j >> 1], vv[0][j >> 1], sel),
                              __builtin_amdgcn_perm(vv[3][j >> 1], vv[2][j >> 1], sel)};
          oacc[j] = mfma_k16(pa, vb, oacc[j]);
        }
      }
    };

    auto process = [&](Raw(&kraw)[4], Raw(&vraw)[4], int k) {
      Words kb[4], vb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kb[i] = T::widen(kraw[i]);
        vb[i] = T::widen(vraw[i]);
      }
      const int tb = (cur.lb0 + k) * kBlock;   // first token of the block
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s[G];
#pragma unroll
        for (int j = 0; j < G; ++j) s[j] = dot_bf16<kW>(qreg[j], kb[i]);
        sc[i] = row_reduce<G, 0>(s) * scale_log2;
      }
      if (tb + kBlock > cur.tok1 || tb < cur.lo) {   // the context ends, or the window starts, in this block
        const uint32_t span = uint32_t(cur.tok1 - cur.lo);   // visible keys: lo .. tok1 - 1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool dead = uint32_t(tb + 4 * i + tg - cur.lo) >= span;
          sc[i] = dead ? -__builtin_inff() : sc[i];
#pragma unroll
          for (int w = 0; w < kW; ++w) vb[i][w] = dead ? 0u : vb[i][w];
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
          for (int e = 0; e < kE; ++e) acc[j][e] *= c;
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
        uint32_t vp[kE];
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          vp[2 * w] = __builtin_amdgcn_perm(vb[2 * kp + 1][w], vb[2 * kp][w], 0x05040100u);
          vp[2 * w + 1] = __builtin_amdgcn_perm(vb[2 * kp + 1][w], vb[2 * kp][w], 0x07060302u);
        }
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int e = 0; e < kE; ++e) acc[j][e] = dot2_bf16(pg[j], vp[e], acc[j][e]);
      }
    };

    // ---- this item's tiles; the last group issues the next item's first tiles ----
    // The scheduling barriers keep the loads of every stage in issue order, so
    // each stage waits only for its own tile (vmcnt = the 16 loads after it).
    for (int k = 0; k < cur.nb; k += kRing) {
      if (dyn && cur.nb > 2 * kRing) {
        if (!requested && cur.nb - k <= kRequestTiles) {
          request();
          requested = true;
        }
        if (k + 2 * kRing >= cur.nb && k + kRing < cur.nb) {
          get_next();
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      static_for<kRing>([&](auto S) {
        constexpr int st = decltype(S)::value;
        if (st == 0 || k + st < cur.nb) {
          if constexpr (MF)
            process_mf(kr[st], vr[st], k + st);
          else
            process(kr[st], vr[st], k + st);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(kr[st], vr[st], k + kRing + st);
        __builtin_amdgcn_sched_barrier(0);
      });
      // Last group: park the next item's q in LDS.  Here, in the loop body, the
      // compiler sees the 8*kRing loads of this group issued after the q fetch
      // and waits for vmcnt(8*kRing), leaving the next item's first tiles in
      // flight (after the loop it could only wait for vmcnt(0) and drain them).
      if (k + kRing >= cur.nb && nxt.valid) park_q(qt);
    }

    if constexpr (MF) {
      // ---- matrix-core form: normalise or leave partials -------------------------
      // m is already common to the lane groups of a head; the sum is not
      const float lw = rows_sum(l) * a.lsum_scale;   // every lane: sum of head mrow (carries 1 / v_scale)
      if (nxt.valid) q_mf_from(reinterpret_cast<const char*>(&sq[wave][0]), nxt.gv);   // parked in the last group
      const bool whole = (cur.parts >> 16) == 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // output row i: head 4 mg + i, d 8 mrow .. +7
        const int head = 4 * mg + i;
        const float Lh = __shfl(lw, head);
        if (head < cur.gv) {
          const int hq = cur.h0 + head;
          if (whole) {
            const float inv = 1.f / Lh;
            u32x4_t o;
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = pack_bf16x2(oacc[2 * w][i] * inv, oacc[2 * w + 1][i] * inv);
            *reinterpret_cast<u32x4_t*>(static_cast<__bf16*>(a.out) + int64_t(cur.q0) * a.o_row_stride +
                                        int64_t(hq) * D + 8 * mrow) = o;
          } else {
            const int64_t slot = (int64_t(cur.b) * a.num_q_heads + hq) * a.max_parts + (cur.parts & 0xffff);
            float* dst = a.ws_o + slot * D + 8 * mrow;
            *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{oacc[0][i], oacc[1][i], oacc[2][i], oacc[3][i]};
            *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{oacc[4][i], oacc[5][i], oacc[6][i], oacc[7][i]};
          }
        }
      }
      if (!whole && mg == 0 && mrow < cur.gv) {
        const int64_t slot = (int64_t(cur.b) * a.num_q_heads + cur.h0 + mrow) * a.max_parts + (cur.parts & 0xffff);
        a.ws_ml[2 * slot] = m;
        a.ws_ml[2 * slot + 1] = lw;
      }
      if (!nxt.valid) break;
      cur = nxt;
      continue;
    }

    // ---- combine the 4 token rows: common max, rescale, reduce-scatter -----------
    const float mw = rows_max(m);
    const float c = fast_exp2(m - mw);
    // every lane: (max, sum) of head hr over the partition; the sum carries
    // 1 / v_scale, so dividing by it also applies the V scale
    const float lw = rows_sum(l * c) * a.lsum_scale;
    static_for<G>([&](auto J) {
      constexpr int j = decltype(J)::value;
      float cj = c;
      if constexpr (j > 0) cj = dpp_f32<0x120 + j * kRot>(c);
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[j][e] *= cj;
    });
    // after the reduce-scatter, row rho holds accumulator x + rho*kNZ of d-slice r
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
    if (nxt.valid) read_q(qreg);   // the next item's q, parked in the last group
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int x0 = 0; x0 < kNZ; x0 += kRun) {
      const int v = x0 + tg * kNZ;
      const int j = v / kE;
      const int e0 = v % kE;
      const int head = (hr + dir * j) & (G - 1);
      const int src = head * kRot;   // a lane of row 0 whose head is `head`
      const float Lh = __shfl(lw, src);
      const int hq = cur.hg * G + head;
      if ((cur.parts >> 16) == 1) {
        const float inv = 1.f / Lh;
        __bf16* orow = static_cast<__bf16*>(a.out) + int64_t(cur.q0) * a.o_row_stride + int64_t(hq) * D + r * kE + e0;
        if constexpr (kRun >= 8) {
#pragma unroll
          for (int c = 0; c < kRun / 8; ++c) {
            u32x4_t o;
#pragma unroll
            for (int w = 0; w < 4; ++w)
              o[w] = pack_bf16x2(flat[x0 + 8 * c + 2 * w] * inv, flat[x0 + 8 * c + 2 * w + 1] * inv);
            *reinterpret_cast<u32x4_t*>(orow + 8 * c) = o;
          }
        } else if constexpr (kRun == 4) {
          u32x2_t o;
#pragma unroll
          for (int w = 0; w < 2; ++w) o[w] = pack_bf16x2(flat[x0 + 2 * w] * inv, flat[x0 + 2 * w + 1] * inv);
          *reinterpret_cast<u32x2_t*>(orow) = o;
        } else {
#pragma unroll
          for (int x = 0; x < kRun; ++x) orow[x] = (__bf16)(flat[x0 + x] * inv);
        }
      } else {
        const int64_t slot = (int64_t(cur.b) * a.num_q_heads + hq) * a.max_parts + (cur.parts & 0xffff);
        float* dst = a.ws_o + slot * D + r * kE + e0;
#pragma unroll
        for (int x = 0; x < kRun; ++x) dst[x] = flat[x0 + x];
      }
    }
    if ((cur.parts >> 16) > 1 && tg == 0 && (r & (kRot - 1)) == 0) {   // one lane per head
      const int64_t slot = (int64_t(cur.b) * a.num_q_heads + cur.hg * G + hr) * a.max_parts + (cur.parts & 0xffff);
      a.ws_ml[2 * slot] = mw;
      a.ws_ml[2 * slot + 1] = lw;
    }
    if (!nxt.valid) break;
    cur = nxt;
  }
  count_out();
}

}  // namespace

// Query heads per work item.  At D = 256 the accumulators and q slices of
// G = 4 or more leave no registers for the tile ring, so a KV head's heads are
// served two at a time; above 8 heads (any D) eight at a time.  The items of
// one KV head are adjacent in the list, so they are dealt to waves of one
// workgroup and stream the same tiles at about the same time: the second
// read of a tile is mostly served by L2.
// A group that is not a power of two (D = 128 only) is served by items of the
// next power of two, 8 at most, whose extra head slots are padding: 3 heads as
// an item of 4, 5 to 7 as one of 8, 9 to 15 as two of 8.  The matrix-core tile
// form pads its products to 16 heads anyway, so the padding costs no extra work.
static int item_group(int head_dim, int group) {
  const int cap = head_dim == 256 ? 2 : 8;
  if (group >= cap) return cap;
  int gi = 1;
  while (gi < group) gi <<= 1;
  return gi;
}

constexpr int kMaxGroup = 64;   // query heads per KV head served by this kernel, at most

int decode_gqa_head_split(int head_dim, int group) {
  const int gi = item_group(head_dim, group);
  return gi > 0 ? (group + gi - 1) / gi : 1;
}

bool decode_gqa_supported(int dtype, int head_dim, int group, int part_size, int block_size) {
  const bool pow2 = group >= 1 && group <= kMaxGroup && (group & (group - 1)) == 0;
  const bool padded = head_dim == 128 && group >= 3 && group < 16;   // items with padding heads
  return dtype == 1 && (head_dim == 64 || head_dim == 128 || head_dim == 256) && (pow2 || padded) &&
         (block_size == 8 || block_size == 16 || block_size == 32) && part_size % kBlock == 0 &&
         part_size / kBlock <= kMaxPartBuckets;
}

namespace {

// Resident workgroups per device for kernel K: CUs x occupancy, queried once per device.
template <int G, bool F8, int BS, int D, bool MF, int WK>
int persistent_groups() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0, occ = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_gqa_kernel<G, F8, BS, D, MF, WK>, 64 * (WK + 1), 0) !=
          hipSuccess ||
      occ <= 0)
    occ = 1;
  v = cus * std::min(occ, 1);
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// The matrix-core tile form serves D = 128 with items of 4 or 8 heads, on
// bf16 and 8-bit pools, at every block size (so results stay bitwise the same
// across block sizes).  On 8-bit pools the dot-product form is bound by the
// VALU issue of the code conversions and v_dot2 instructions (205 -> 153 us
// on the GQA decode layer); on bf16 pools the kernel streams at the HBM
// ceiling either way, and the form's lighter vector work shortens the tail
// (273.8 -> 272.4 us) and leaves more issue slots to a prefill launch beside
// it (mixed chunked-prefill step 507.7 -> 499 us).
template <int G, bool F8, int BS, int D>
constexpr bool use_mfma_tiles() {
  return D == 128 && (G == 4 || G == 8);
}

template <int G, bool F8, int BS, int D, int WK>
hipError_t launch_wk(const DecodeArgs& a, hipStream_t stream) {
  constexpr bool MF = use_mfma_tiles<G, F8, BS, D>();
  const int64_t upper = (int64_t(a.num_seqs) * a.max_parts * a.num_kv_heads) << a.head_split_log2;
  const int64_t grid = std::min<int64_t>(upper, persistent_groups<G, F8, BS, D, MF, WK>());
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_gqa_kernel<G, F8, BS, D, MF, WK>), dim3(grid), dim3(64 * (WK + 1)), 0, stream, a);
  return hipGetLastError();
}

// Three workers also where four would not fit the registers a wave needs: the
// matrix-core form with 8-token blocks needs more than the 256 a wave may take
// when one SIMD holds two of a workgroup's five waves.
template <int G, bool F8, int BS, int D>
constexpr bool three_workers_fit_better() {
  return use_mfma_tiles<G, F8, BS, D>() && BS == 8;
}

template <int G, bool F8, int BS, int D>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream, bool beside_prefill) {
  if ((beside_prefill || three_workers_fit_better<G, F8, BS, D>()) && a.head_split_log2 == 0)
    return launch_wk<G, F8, BS, D, kWorkersBesidePrefill>(a, stream);
  return launch_wk<G, F8, BS, D, kWorkersDefault>(a, stream);
}

template <bool F8, int BS, int D>
hipError_t launch_bs(int group, const DecodeArgs& a, hipStream_t stream, bool bp) {
  switch (group) {
    case 1: return launch_g<1, F8, BS, D>(a, stream, bp);
    case 2: return launch_g<2, F8, BS, D>(a, stream, bp);
    case 4: return launch_g<4, F8, BS, D>(a, stream, bp);
    case 8: return launch_g<8, F8, BS, D>(a, stream, bp);
    default: return hipErrorInvalidValue;
  }
}

template <bool F8, int D>
hipError_t launch_d(int group, const DecodeArgs& a, hipStream_t stream, bool bp) {
  switch (a.block_size) {
    case 8: return launch_bs<F8, 8, D>(group, a, stream, bp);
    case 16: return launch_bs<F8, 16, D>(group, a, stream, bp);
    case 32: return launch_bs<F8, 32, D>(group, a, stream, bp);
    default: return hipErrorInvalidValue;
  }
}

template <bool F8, int BS>
hipError_t launch_bs256(int group, const DecodeArgs& a, hipStream_t stream, bool bp) {   // G <= 2 at D = 256
  switch (group) {
    case 1: return launch_g<1, F8, BS, 256>(a, stream, bp);
    case 2: return launch_g<2, F8, BS, 256>(a, stream, bp);
    default: return hipErrorInvalidValue;
  }
}

template <bool F8>
hipError_t launch_f(int group, int head_dim, const DecodeArgs& a, hipStream_t stream, bool bp) {
  switch (head_dim) {
    case 64: return launch_d<F8, 64>(group, a, stream, bp);
    case 128: return launch_d<F8, 128>(group, a, stream, bp);
    case 256:
      switch (a.block_size) {
        case 8: return launch_bs256<F8, 8>(group, a, stream, bp);
        case 16: return launch_bs256<F8, 16>(group, a, stream, bp);
        case 32: return launch_bs256<F8, 32>(group, a, stream, bp);
        default: return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int decode_gqa_workers(int group) {
  int g = 0;
  switch (item_group(128, group)) {
    case 1: g = persistent_groups<1, false, 16, 128, false, kWorkersDefault>(); break;
    case 2: g = persistent_groups<2, false, 16, 128, false, kWorkersDefault>(); break;
    case 4: g = persistent_groups<4, false, 16, 128, false, kWorkersDefault>(); break;
    case 8: g = persistent_groups<8, false, 16, 128, false, kWorkersDefault>(); break;
    default: g = 256;
  }
  return g * kWorkersDefault;
}

// a.block_size selects the paging (8, 16 or 32 tokens per block); the kernel
// is instantiated for the item group, and a.head_split_log2 is set here.
hipError_t launch_decode_gqa(int group, int head_dim, bool fp8_cache, const DecodeArgs& a, hipStream_t stream,
                             bool beside_prefill) {
  const int gi = item_group(head_dim, group);
  const int split = decode_gqa_head_split(head_dim, group);
  // every item holds at least one head, and a KV head's items number a power of two
  if (gi <= 0 || gi * split < group || gi * (split - 1) >= group || (split & (split - 1)) != 0 ||
      group > kMaxGroup)
    return hipErrorInvalidValue;
  if (gi * split != group && !(head_dim == 128 && (gi == 4 || gi == 8))) return hipErrorInvalidValue;
  DecodeArgs b = a;
  b.head_split_log2 = 0;
  while ((1 << b.head_split_log2) < split) ++b.head_split_log2;
  return fp8_cache ? launch_f<true>(gi, head_dim, b, stream, beside_prefill)
                   : launch_f<false>(gi, head_dim, b, stream, beside_prefill);
}

}  // namespace pa
