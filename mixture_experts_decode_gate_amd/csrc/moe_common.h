// Device helpers shared by the routed-MoE kernels' translation units: routing
// (top-k, the union), the NVFP4 row loads, the slot table, the down-sweep
// segments, and the host-side launch helpers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- routing
// Router GEMV.  Top-k runs in the next kernel: every gate/up block takes top-k,
// the union and the slot table itself from the stored logits (moe_forward), or
// topk_kernel does (moe_route).  The kernel boundary makes every router
// block's results visible to the reader without a grid-wide hand-off.
//
// Block e (of E+1) computes router row e for every input row (e == E is the
// shared expert's gate vector): wave c < nkc takes the kRouterChunk-column
// chunk c, issues all its loads before any arithmetic and accumulates in
// fp64.  The sum runs in a fixed order that does not depend on the number of
// rows: each quad of lanes per chunk, those partials in chunk order, then the
// 16 quads; it is rounded once: logits[r][e] = fp32(sum),
// gamma[r] = fp32(sigmoid(sum)), and for sigmoid routing
// score[r][e] = sigmoid(fp32(sum)) in fp64.
constexpr int kRouterChunk = 512;
constexpr int kMaxRouterChunks = MOE_MAX_DIM / kRouterChunk;
constexpr int kRouteThreads = 64 * kMaxRouterChunks;  // a wave per router chunk
constexpr int kTopkThreads = 64 * kMaxRows;           // a wave per row
static_assert(MOE_MAX_EXPERTS <= 64 * 16, "top-k holds at most 16 keys per lane");

// A set of up to 128 slots: bit t of lo (t < 64) or of hi (t >= 64).
struct Slots128 {
  uint64_t lo, hi;
};

// Bits [lo, hi) of a 64-bit word, both bounds clamped to [0, 64].  This and
// the other plain bit-arithmetic helpers below are host-callable too, so a
// host program can check them against bit-by-bit references.
__host__ __device__ __forceinline__ uint64_t bit_range64(int lo, int hi) {
  lo = lo < 0 ? 0 : lo;
  hi = hi > 64 ? 64 : hi;
  if (hi <= lo) return 0ull;
  const uint64_t up = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  return up & ~((1ull << lo) - 1ull);
}

// The lowest slot of a slot set in [a, a + k) (a row's slots: a = r*k), or
// -1 when none; a + k <= 128, so a row's window may span both words (one
// row with top_k past 64).
__host__ __device__ __forceinline__ int slot_first(const Slots128& s, int a, int k) {
  const uint64_t lo = s.lo & bit_range64(a, a + k);
  const uint64_t hi = s.hi & bit_range64(a - 64, a + k - 64);
  if (lo) return __builtin_ctzll(lo);
  if (hi) return 64 + __builtin_ctzll(hi);
  return -1;
}

// t / k without a divide, for 0 <= t < 128 and 1 <= k <= 128.  With
// m = ceil(2^16 / k) = (2^16 + e) / k, 0 <= e < k, t*m / 2^16 exceeds t/k by
// t*e / (k * 2^16) < 1/k (t*e < 2^16); the fraction of t/k is at most
// (k - 1)/k, so the sum stays below the next integer.
__host__ __device__ __forceinline__ uint32_t small_div_magic(int k) {
  return (65536u + (uint32_t)k - 1u) / (uint32_t)k;
}
__host__ __device__ __forceinline__ int small_div(int t, uint32_t magic) {
  return (int)(((uint32_t)t * magic) >> 16);
}

// One lane's part of the union: its slots t = 64*q + lane, q = 0, 1.
struct UnionLane {
  int pos[2];        // union position of slot t when it is a first occurrence, else -1
  uint32_t mask[2];  // rows that chose slot t's id
  Slots128 eq[2];    // slots that hold slot t's id
};

// Union of the n <= 128 ids in ids_lds (slot t = r*k + j; 128 entries
// readable) that lie in [lo, hi).  Each slot compares its id with every slot
// at once (broadcast LDS reads, no sort): slot t is a first occurrence when
// its id is in range and no earlier slot holds it.  First occurrences, in slot
// order, form the union; a slot whose id is out of range maps to -1 (under
// expert parallelism forward_ep.rs splits the selected ids into local and
// remote ones by local_expert_range).  Up to 64 ids this is the one-wave,
// one-tile union of the "RETRACTED (2026-08-29)" and "WIDENED (2026-08-31)"
// notes; past 64 the wave takes the slots in two tiles of 64 and the second
// tile's union positions continue the first's.  Returns U; the union outputs
// are written when union_ids is not null (row_mask may be null on its own).
inline __device__ int union_wave(const int32_t* ids_lds, int n, int k, int rows, int lo, int hi, int lane,
                          int32_t* union_ids, int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask,
                          UnionLane& ul) {
  const int tiles = n > 64 ? 2 : 1;
  bool first[2] = {false, false}, local[2] = {false, false};
  int id[2] = {-1, -1}, f[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    ul.pos[q] = -1;
    ul.mask[q] = 0u;
    ul.eq[q] = Slots128{0ull, 0ull};
    if (q >= tiles) continue;
    const int t = 64 * q + lane;
    id[q] = t < n ? ids_lds[t] : -1;
    local[q] = id[q] >= lo && id[q] < hi;
    Slots128 eq{0ull, 0ull};
    auto match4 = [&](int t4) {
      const int4 v = reinterpret_cast<const int4*>(ids_lds)[t4];
      return (uint64_t)(v.x == id[q]) | ((uint64_t)(v.y == id[q]) << 1) | ((uint64_t)(v.z == id[q]) << 2) |
             ((uint64_t)(v.w == id[q]) << 3);
    };
#pragma unroll
    for (int t4 = 0; t4 < 16; ++t4) eq.lo |= match4(t4) << (4 * t4);
    if (tiles > 1) {
#pragma unroll
      for (int t4 = 16; t4 < 32; ++t4) eq.hi |= match4(t4) << (4 * (t4 - 16));
    }
    // slots past n hold stale ids
    if (n < 64) {
      eq.lo &= (1ull << n) - 1ull;
      eq.hi = 0ull;
    } else if (n < 128) {
      eq.hi &= (1ull << (n - 64)) - 1ull;
    }
    // a slot below n holds its own id, so its set is not empty
    f[q] = t >= n ? t : (eq.lo ? __builtin_ctzll(eq.lo) : 64 + __builtin_ctzll(eq.hi));
    first[q] = t < n && local[q] && f[q] == t;
    ul.eq[q] = eq;
    for (int r = 0; r < rows; ++r)
      if (slot_first(eq, r * k, k) >= 0) ul.mask[q] |= 1u << r;
  }
  const uint64_t bal0 = __ballot(first[0]), bal1 = __ballot(first[1]);
  const int U = __popcll(bal0) + __popcll(bal1);
  auto pos_of = [&](int t) {
    return t < 64 ? __popcll(bal0 & ((1ull << t) - 1ull)) : __popcll(bal0) + __popcll(bal1 & ((1ull << (t - 64)) - 1ull));
  };
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (q >= tiles) continue;
    const int t = 64 * q + lane;
    if (first[q]) ul.pos[q] = pos_of(t);
    if (union_ids != nullptr) {
      if (t < n) slot_to_union[t] = local[q] ? pos_of(f[q]) : -1;
      if (first[q]) {
        union_ids[ul.pos[q]] = id[q];
        if (row_mask) row_mask[ul.pos[q]] = ul.mask[q];
      }
    }
  }
  if (union_ids != nullptr && lane == 0) *union_count = U;
  return U;
}

// The same union over at most 256 experts through two LDS tables indexed by
// expert id, in place of comparing every slot with every other: each slot t
// whose id is in [lo, hi) takes the minimum of t into first[id] and sets its
// row's bit in mask[id] (LDS atomics), and slot t is a first occurrence when
// first[id] == t.  One wave's LDS operations run in issue order, so the reset
// before the atomics and the reads after them need no barrier.  Writes what
// union_wave writes, plus each first occurrence's slot table entry (built by
// entry(id, row_mask) with no pairs) and then every slot's pair index into its
// entry.  first and mask hold 256 entries; k <= 128 and n <= 128.
template <typename EntryFn>
inline __device__ int union_lds(const int32_t* ids_lds, int n, int k, int lo, int hi, int lane, uint32_t* first_tab,
                                uint32_t* mask_tab, int32_t* union_ids, int32_t* union_count, int32_t* slot_to_union,
                                uint32_t* row_mask, SlotInfo* slots, EntryFn&& entry) {
  const int tiles = n > 64 ? 2 : 1;
  const uint32_t kmagic = small_div_magic(k);
  int id[2], row[2];
  bool use[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 64 * q + lane;
    id[q] = q < tiles && t < n ? ids_lds[t] : -1;
    use[q] = q < tiles && t < n && id[q] >= lo && id[q] < hi;
    row[q] = small_div(t, kmagic);
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (use[q]) {
      first_tab[id[q]] = 0xFFFFFFFFu;
      mask_tab[id[q]] = 0u;
    }
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (use[q]) {
      atomicMin(&first_tab[id[q]], (uint32_t)(64 * q + lane));
      atomicOr(&mask_tab[id[q]], 1u << row[q]);
    }
  int f[2];
  uint32_t msk[2];
  bool first[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 64 * q + lane;
    f[q] = use[q] ? (int)first_tab[id[q]] : t;
    msk[q] = use[q] ? mask_tab[id[q]] : 0u;
    first[q] = use[q] && f[q] == t;
  }
  const uint64_t bal0 = __ballot(first[0]), bal1 = __ballot(first[1]);
  const int U = __popcll(bal0) + __popcll(bal1);
  auto pos_of = [&](int t) {
    return t < 64 ? __popcll(bal0 & ((1ull << t) - 1ull)) : __popcll(bal0) + __popcll(bal1 & ((1ull << (t - 64)) - 1ull));
  };
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 64 * q + lane;
    if (q < tiles && t < n) slot_to_union[t] = use[q] ? pos_of(f[q]) : -1;
    if (first[q]) {
      const int pos = pos_of(t);
      union_ids[pos] = id[q];
      row_mask[pos] = msk[q];
      slots[pos] = entry(id[q], msk[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (use[q]) slots[pos_of(f[q])].pair[row[q]] = (uint8_t)(64 * q + lane);
  if (lane == 0) *union_count = U;
  return U;
}

// The token-major slot list (MoeLayer::forward_token_major_decode runs every
// (row, selected expert) pair on its own): slot t = r*k + j holds id[t] for
// row r alone, so an expert chosen by several rows is swept once per row.
// Same outputs as union_wave, with U = n.
inline __device__ int identity_slots(const int32_t* ids_lds, int n, int k, int lane, int32_t* union_ids,
                              int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask, UnionLane& ul) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 64 * q + lane;
    const bool used = t < n;
    ul.pos[q] = used ? t : -1;
    ul.mask[q] = used ? 1u << (t / k) : 0u;
    ul.eq[q] = Slots128{used && q == 0 ? 1ull << lane : 0ull, used && q == 1 ? 1ull << lane : 0ull};
    if (used) {
      slot_to_union[t] = t;
      union_ids[t] = ids_lds[t];
      row_mask[t] = ul.mask[q];
    }
  }
  if (lane == 0) *union_count = n;
  return n;
}


// Order-preserving map of a float key to uint32 (larger float -> larger
// integer); +0 and -0 map to neighbours, never to 0 except the all-ones NaN.
__host__ __device__ __forceinline__ uint32_t key_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__host__ __device__ __forceinline__ float key_float(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Weight pointers of one expert, staged in LDS by the block that runs top-k.
struct ExpertPtrs {
  const uint8_t* p[6];  // gate, up, down: packed codes then block scales
  float scale2[3];
};

// Global-memory load through an address-space-1 pointer: a flat load would
// also count against the LDS counter, and its wait would drain both.
template <typename T>
__device__ __forceinline__ T ld_global(const T* ptr) {
  typedef __attribute__((address_space(1))) const T global_t;
  return *(global_t*)ptr;
}

// The values top-k reads for one row, as lane l sees them (experts
// l*G .. l*G+G-1, clamped in range).
template <int G>
struct TopkIn {
  float lv[G], bv[G];
  double sv[G];  // sigmoid score (sigmoid routing)
};

template <int G>
__device__ __forceinline__ void topk_load(const RouteParams& p, int r, int lane, TopkIn<G>& in) {
  const int E = p.E;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int e = min(lane * G + i, E - 1);
    in.lv[i] = ld_global(p.logits + r * E + e);
    in.sv[i] = ld_global(p.score + r * E + e);
    in.bv[i] = ld_global(p.bias + e);
  }
}

// Top-k of row r (one wave) from values loaded by topk_load.  Lane l holds
// experts l*G .. l*G+G-1, so a lower (lane, position) pair is a lower expert
// id.  Each of the k rounds takes the lane's largest remaining key (lowest
// position on ties), the wave-wide maximum of those, and the lowest lane
// holding it: the largest key, ties to the lower id.  Sigmoid keys are
// fp32(s) + bias with s the fp64 score the router pass stored.  Writes the
// row's ids to ids_lds (and ids_out when not null) and, when w_out is not
// null, the weights (fp64, rounded once).
template <int G>
__device__ void topk_select(const RouteParams& p, int r, int lane, TopkIn<G>& in, int32_t* ids_lds,
                            int32_t* ids_out, float* w_out) {
  const int E = p.E, k = p.k;
  const bool softmax = p.route_kind == MOE_ROUTE_SOFTMAX;
  uint32_t key[G];  // 0: not a candidate (past E, or already taken)
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const bool valid = lane * G + i < E;
    const float kf = softmax ? in.lv[i] : (float)in.sv[i] + in.bv[i];
    key[i] = valid ? key_bits(kf) : 0u;
  }
  // Round j's id goes to lane j % 64 of sel[j / 64] (k <= 128); the ids are
  // stored after the last round, so a round carries no store and no branch.
  int sel[2] = {0, 0};
  float top_logit = 0.f;
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bool better = key[i] > best;
      best = better ? key[i] : best;
      bi = better ? i : bi;
    }
    const uint32_t m = wave_max(best);
    const uint64_t cand = __ballot(best == m);
    const int wl = (int)__builtin_ctzll(cand | (1ull << 63));
    const int wi = __builtin_amdgcn_readlane(bi, wl);
    // k <= E valid keys keep m > 0; the clamp only guards ids against keys
    // outside the contract (NaN).
    const int taken = wl * G + wi;
    const int be = min(taken, E - 1);
#pragma unroll
    for (int i = 0; i < G; ++i) key[i] = lane * G + i == taken ? 0u : key[i];
    if (j == 0) top_logit = key_float(m);  // softmax: the largest logit
    if (j < 64)
      sel[0] = lane == j ? be : sel[0];
    else
      sel[1] = lane == j - 64 ? be : sel[1];
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = 64 * q + lane;
    if (j < k) {
      if (ids_out != nullptr) ids_out[r * k + j] = sel[q];
      ids_lds[r * k + j] = sel[q];
    }
  }
  if (w_out == nullptr) return;
  // round that took each of this lane's experts, -1 if none
  int selj[G];
#pragma unroll
  for (int i = 0; i < G; ++i) selj[i] = -1;
  for (int j = 0; j < k; ++j) {
    const int e = __builtin_amdgcn_readlane(sel[j >> 6], j & 63);
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (lane * G + i == e) selj[i] = j;
  }
  // Weights.  Softmax: exp(L - max), normalised over all experts, or over the
  // k selected when norm_topk_prob.  Sigmoid: s, optionally normalised over
  // the selected, times routed_scaling_factor.
  double sv[G], all_part = 0.0, sel_part = 0.0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    sv[i] = 0.0;
    if (lane * G + i < E) {
      double v = in.sv[i];
      if (softmax) v = (!p.norm || selj[i] >= 0) ? exp((double)in.lv[i] - (double)top_logit) : 0.0;
      sv[i] = v;
      all_part += v;
      if (selj[i] >= 0) sel_part += v;
    }
  }
  double sums[2] = {all_part, sel_part};
  wave_sum_n<2>(sums);
  const double all_sum = softmax && !p.norm ? sums[0] : 1.0;
  const double sel_sum = p.norm ? sums[1] : 1.0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    if (selj[i] >= 0) {
      double wgt;
      if (softmax) {
        wgt = p.norm ? sv[i] / sel_sum : sv[i] / all_sum;
      } else {
        wgt = p.norm ? sv[i] / sel_sum : sv[i];
        wgt *= (double)p.rsf;
      }
      w_out[r * k + selj[i]] = (float)wgt;
    }
  }
}

// ---------------------------------------------------------------- sweeps
// Copy the slot table into LDS (all kNumSlots entries: those past U are stale
// and never read, and not waiting for U saves a round trip).  Later reads come
// from LDS: a global load issued after the prefetched weights would make the
// in-order load counter drain the prefetch.  Each thread issues all its loads
// before its first store, so the copy costs one memory round trip, not one
// per pass of a strided loop.
template <int kThreads>
__device__ __forceinline__ void load_slot_table(SlotInfo* dst, const SlotInfo* src) {
  constexpr int kWords = (int)(sizeof(SlotInfo) / 4);
  constexpr int kPerThread = (kNumSlots * kWords + kThreads - 1) / kThreads;
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst);
  uint32_t v[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int i = (int)threadIdx.x + q * kThreads;
    v[q] = i < kNumSlots * kWords ? s32[i] : 0u;
  }
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int i = (int)threadIdx.x + q * kThreads;
    if (i < kNumSlots * kWords) d32[i] = v[q];
  }
}

constexpr int kMaxSweepThreads = 512;
constexpr int kSweepWaves = kMaxSweepThreads / 64;
// The gate/up sweep stages R * NCH chunks of x (4 KB each) in LDS: at most
// kMaxChunkRows of them, and the LDS copy of every expert's pointers only up
// to kPtabMaxChunkRows.
constexpr int kMaxChunkRows = 36;
constexpr int kPtabMaxChunkRows = 24;

// One row of a K-contiguous NVFP4 matrix as this lane sees it: NCH 16-byte
// code loads (32 columns each, 2048 columns per chunk across the wave) and
// the two E4M3 block scales of each.
template <int NCH>
struct RowRegs {
  u32x4 q[NCH];
  uint32_t s[NCH];
};

// Lanes whose columns lie past K load the row's last 32 columns instead (an
// in-bounds, finite copy); scale_pair zeroes their two block scales, so they
// add exactly 0 whatever the activations hold there.  No branch guards the
// loads (a branch here makes the compiler drain the prefetched loads early),
// and nothing is computed on the loaded values until they are used (an
// operation here would make the compiler wait for them at the fetch).
// packed, scales, n and K are wave-uniform (scalar registers): each load is
// a scalar row base plus the lane's unsigned 32-bit offset, with no vector
// address arithmetic.
template <int NCH>
__device__ __forceinline__ void load_row(RowRegs<NCH>& b, const uint8_t* packed, const uint8_t* scales, int n,
                                         int K, int lane) {
  const uint8_t* rc = packed + (size_t)n * (size_t)(K >> 1);
  const uint8_t* rs = scales + (size_t)n * (size_t)(K >> 4);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = c * kChunk + lane * 32;
    const uint32_t cc = (uint32_t)(col < K ? col : K - 32);
    b.q[c] = ld_stream(rc + (cc >> 1));
    b.s[c] = ld_stream_u16(rs + (cc >> 4));
  }
}

// Reads the row's loaded registers here, on every path.  Where a path skips
// the use of a prefetched row (a branch on the rows that use it, an item that
// is not computed), the compiler's wait-count pass counts the row's loads as
// still in flight after it, and the next write to those registers (at the
// top of the loop) waits for every load issued since.
template <int NCH>
__device__ __forceinline__ void consume(const RowRegs<NCH>& b) {
#pragma unroll
  for (int c = 0; c < NCH; ++c) asm volatile("" ::"v"(b.q[c]), "v"(b.s[c]));
}

// The two E4M3 block scales of chunk c for this lane, zero past K.
template <int NCH>
__device__ __forceinline__ uint32_t scale_pair(const RowRegs<NCH>& b, int c, int K, int lane) {
  return c * kChunk + lane * 32 < K ? b.s[c] : 0u;
}

// Weight pointers of expert ex, as read from the expert tables.
__device__ __forceinline__ ExpertPtrs expert_ptrs(const RouteParams& rp, int ex) {
  ExpertPtrs e;
  e.p[0] = ld_global(rp.gate.packed + ex);
  e.p[1] = ld_global(rp.gate.scales + ex);
  e.p[2] = ld_global(rp.up.packed + ex);
  e.p[3] = ld_global(rp.up.scales + ex);
  e.p[4] = ld_global(rp.down.packed + ex);
  e.p[5] = ld_global(rp.down.scales + ex);
  e.scale2[0] = ld_global(rp.gate.scale2 + ex);
  e.scale2[1] = ld_global(rp.up.scale2 + ex);
  e.scale2[2] = ld_global(rp.down.scale2 + ex);
  return e;
}

// Slot table entry of a routed expert.  ``eq`` holds the slots t = r*k + j
// whose id is this expert: row r's pair is r*k + j for the one j its bits
// name (a row's ids are distinct).
__device__ __forceinline__ SlotInfo slot_info(const ExpertPtrs& e, int ex, int inter, uint32_t row_mask,
                                              const Slots128& eq, int k, int rows) {
  SlotInfo si;
  si.gate_packed = e.p[0];
  si.gate_scales = e.p[1];
  si.up_packed = e.p[2];
  si.up_scales = e.p[3];
  si.down_packed = e.p[4];
  si.down_scales = e.p[5];
  si.gate_scale2 = e.scale2[0];
  si.up_scale2 = e.scale2[1];
  si.down_scale2 = e.scale2[2];
  si.inter = inter;
  si.row_mask = row_mask;
  si.expert = ex;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) si.pair[r] = (uint8_t)0xFF;
  for (int r = 0; r < rows; ++r) {
    const int f = slot_first(eq, r * k, k);
    if (f >= 0) si.pair[r] = (uint8_t)f;
  }
  return si;
}

// A routed slot's table entry with no pair indices yet (all 0xFF).
__device__ __forceinline__ SlotInfo slot_info_base(const ExpertPtrs& e, int ex, int inter, uint32_t row_mask) {
  SlotInfo si;
  si.gate_packed = e.p[0];
  si.gate_scales = e.p[1];
  si.up_packed = e.p[2];
  si.up_scales = e.p[3];
  si.down_packed = e.p[4];
  si.down_scales = e.p[5];
  si.gate_scale2 = e.scale2[0];
  si.up_scale2 = e.scale2[1];
  si.down_scale2 = e.scale2[2];
  si.inter = inter;
  si.row_mask = row_mask;
  si.expert = ex;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) si.pair[r] = (uint8_t)0xFF;
  return si;
}

// Slot table entry of the shared expert (used by every row; row r's pair is
// rows*k + r).
__device__ __forceinline__ SlotInfo shared_slot_info(const RouteParams& rp, uint32_t row_mask) {
  SlotInfo si;
  si.gate_packed = rp.shared_gate.packed;
  si.gate_scales = rp.shared_gate.scales;
  si.up_packed = rp.shared_up.packed;
  si.up_scales = rp.shared_up.scales;
  si.down_packed = rp.shared_down.packed;
  si.down_scales = rp.shared_down.scales;
  si.gate_scale2 = rp.shared_gate.scale2;
  si.up_scale2 = rp.shared_up.scale2;
  si.down_scale2 = rp.shared_down.scale2;
  si.inter = rp.shared_inter;
  si.row_mask = row_mask;
  si.expert = -1;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) si.pair[r] = r < rp.rows ? (uint8_t)(rp.rows * rp.k + r) : (uint8_t)0xFF;
  return si;
}

// Down-sweep segments (one wave): one segment per slot -- the shared slot
// first (all R rows), then the routed slots in union order.  Lane l holds the
// row masks of union slots l (mask0) and 64 + l (mask1), 0 past U.
// seg_rows[s] holds the segment's row mask in bits 0..15 and its number of
// row groups (of up to ``group`` rows) in bits 16..23; seg_cum[s] is the
// summed work weight of the segments before s (kSegCostBase per group plus
// one per row; seg_cum[count] the total).  Returns the number of segments.
inline __device__ int build_segments(uint32_t mask0, uint32_t mask1, int lane, int R, int group,
                                     int32_t* seg_slot, uint32_t* seg_rows, int32_t* seg_cum) {
  const int sh_groups = (R + group - 1) / group;
  if (lane == 0) {
    seg_slot[0] = kSharedSlot;
    seg_rows[0] = ((1u << R) - 1u) | ((uint32_t)sh_groups << 16);
    seg_cum[0] = 0;
  }
  int total = 1, wtotal = kSegCostBase * sh_groups + R;  // segments and weight so far
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t mask = q ? mask1 : mask0;
    const int cnt = __popc(mask);
    const int groups = (cnt + group - 1) / group;
    const int has = cnt > 0 ? 1 : 0;
    const int cost = kSegCostBase * groups + cnt;
    int incl = has, wincl = cost;  // inclusive prefix sums over lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o), wv = __shfl_up(wincl, o);
      if (lane >= o) {
        incl += v;
        wincl += wv;
      }
    }
    if (has) {
      const int seg = total + incl - 1;
      seg_slot[seg] = 64 * q + lane;
      seg_rows[seg] = mask | ((uint32_t)groups << 16);
      seg_cum[seg] = wtotal + wincl - cost;
    }
    total += __shfl(incl, 63);
    wtotal += __shfl(wincl, 63);
  }
  if (lane == 0) seg_cum[total] = wtotal;
  return total;
}

// ---------------------------------------------------------------- launch helpers
// Per-device launch caches hold this many devices; a device index past it is
// served without caching.
constexpr int kMaxDevices = 64;

// Launch shapes, measured on MI355X: the gate/up sweep runs 8 waves per CU
// (one 512-thread block: its staged x and 196 VGPRs allow no more), the down
// sweep 12 (three 256-thread blocks), the read probe 16 blocks per CU with 16
// loads in flight per lane (the fastest of 4 / 8 / 16 each).
constexpr int kGateupWavesPerCU = 8;
constexpr int kDownWavesPerCU = 12;
constexpr int kNumXcds = 8;  // accelerator dies; workgroups go to them round-robin
constexpr int kProbeBlocksPerCU = 16;
constexpr int kProbeUnroll = 16;

// Workgroup b runs on XCD b % kNumXcds.  Its XCD-major index numbers the
// blocks die by die (the blocks of one XCD get consecutive indices), so work
// split by that index gives each die contiguous runs of weight rows rather
// than every kNumXcds-th row, whose addresses can fall unevenly on the HBM
// channels.  A bijection on [0, gridDim.x) when the grid is a multiple of
// kNumXcds, the identity otherwise.
__device__ __forceinline__ int xcd_major_block() {
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  return nb % kNumXcds == 0 ? (b % kNumXcds) * (nb / kNumXcds) + b / kNumXcds : b;
}

inline int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  return dev;
}

inline int cu_count() {
  static int cached[kMaxDevices] = {0};
  const int dev = current_device();
  if (dev >= 0 && dev < kMaxDevices && cached[dev]) return cached[dev];
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev] = n;
  return n;
}

template <class T>
struct no_deduce {
  using type = T;
};

// Launch ``kernel``; with stage events, through hipExtLaunchKernel so the
// events record the kernel's own start and end.
template <typename... KArgs>
hipError_t launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, StageEvents ev,
                    typename no_deduce<KArgs>::type... args) {
  if (ev.start != nullptr || ev.stop != nullptr) {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, s, ev.start, ev.stop, 0);
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}

// Blocks per CU for a sweep kernel: the occupancy limit (queried once per
// kernel instance and device), capped at ``waves_per_cu`` waves.
template <typename K>
int blocks_per_cu(K kernel, int threads, size_t lds, int waves_per_cu, int (&cache)[kMaxDevices]) {
  const int dev = current_device();
  int local = 0;
  int& per_cu = (dev >= 0 && dev < kMaxDevices) ? cache[dev] : local;
  if (per_cu <= 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, lds) != hipSuccess || occ <= 0) occ = 1;
    const int want = (waves_per_cu * 64 + threads - 1) / threads;
    per_cu = occ < want ? occ : (want < 1 ? 1 : want);
  }
  return per_cu;
}


// The gate/up sweep's launchers, one translation unit per four row counts.
hipError_t launch_gateup_rows_1_4(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                  StageEvents ev);
hipError_t launch_gateup_rows_5_8(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                  StageEvents ev);
hipError_t launch_gateup_rows_9_12(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                   StageEvents ev);
hipError_t launch_gateup_rows_13_16(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                    StageEvents ev);

}  // namespace moe
