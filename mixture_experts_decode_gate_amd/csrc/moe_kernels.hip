// Routed-MoE decode/verify kernels for MI355X (gfx950).
//
// Stage order follows MoeLayer::forward_token_major_decode
// (metrale_model_layers/layers/moe/forward_token_major.rs): router GEMM,
// batched top-k, gate+up, silu+down, weighted sum and shared-expert blend.
// The gate+up and down stages sweep the *union* of the experts the rows chose,
// each union expert's weights read once for every row that chose it
// ("Function forward_moe" rustdoc, "RETRACTED (2026-08-29)" note), and the
// shared expert once for all rows (same page, SHARED-expert note).
//
// Numerics: router dot products and the routing math run in fp64 and round
// once to fp32, so top-k decisions are taken on the same fp32 keys a float64
// reference produces.  Expert dot products use bf16 x bf16 -> fp32 dot2 on
// weights decoded exactly from E2M1 (block scale applied per 16 columns), and
// silu(gate)*up is stored as bf16.  Every per-(row, expert) value is reduced
// in an order that does not depend on the other rows, so a call with R rows
// writes each row's output bytes exactly as a one-row call would.

#include <hip/hip_ext.h>

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
// chunk c, issues all its loads before any arithmetic, accumulates in fp64
// and reduces in a fixed order; the chunk partials are summed in chunk order
// and rounded once: logits[r][e] = fp32(sum), gamma[r] = fp32(sigmoid(sum)),
// and for sigmoid routing score[r][e] = sigmoid(sum) in fp64.
constexpr int kRouterChunk = 512;
constexpr int kMaxRouterChunks = MOE_MAX_DIM / kRouterChunk;
constexpr int kRouteThreads = 64 * kMaxRouterChunks;  // a wave per router chunk
constexpr int kTopkThreads = 64 * kMaxRows;           // a wave per row
static_assert(MOE_MAX_EXPERTS <= 64 * 16, "top-k holds at most 16 keys per lane");

// Union of the n <= 64 ids in ids_lds (slot t = r*k + j) that lie in
// [lo, hi).  Lane t compares its id with every slot at once (broadcast LDS
// reads, no sort): slot t is a first occurrence when its id is in range and no
// earlier slot holds it.  First occurrences, in slot order, form the union;
// a slot whose id is out of range maps to -1 (under expert parallelism
// forward_ep.rs splits the selected ids into local and remote ones by
// local_expert_range).  Returns the lane's union position if it is a first
// occurrence (else -1), in *mask_out the rows that chose its id and in
// *count_out the union size U, in *eq_out the slots that hold its id (bit t).
// The union outputs are written when union_ids is not null (row_mask may be
// null on its own).
__device__ int union_wave(const int32_t* ids_lds, int n, int k, int rows, int lo, int hi, int lane,
                          int32_t* union_ids, int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask,
                          uint32_t* mask_out, int* count_out, uint64_t* eq_out) {
  const int id = lane < n ? ids_lds[lane] : -1;
  const bool local = id >= lo && id < hi;
  uint64_t eq = 0;
#pragma unroll
  for (int t4 = 0; t4 < kMaxIds / 4; ++t4) {
    const int4 v = reinterpret_cast<const int4*>(ids_lds)[t4];
    eq |= (uint64_t)(v.x == id) << (4 * t4 + 0);
    eq |= (uint64_t)(v.y == id) << (4 * t4 + 1);
    eq |= (uint64_t)(v.z == id) << (4 * t4 + 2);
    eq |= (uint64_t)(v.w == id) << (4 * t4 + 3);
  }
  eq &= n >= 64 ? ~0ull : ((1ull << n) - 1ull);
  const int first = lane < n ? __builtin_ctzll(eq) : lane;
  uint32_t mask = 0;
  const uint64_t kmask = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
  for (int r = 0; r < rows; ++r)
    if ((eq >> (r * k)) & kmask) mask |= 1u << r;
  const bool is_first = (lane < n) && local && (first == lane);
  const unsigned long long bal = __ballot(is_first);
  const int pos_self = __popcll(bal & ((1ull << lane) - 1ull));
  const int pos_first = __popcll(bal & ((1ull << first) - 1ull));
  if (union_ids != nullptr) {
    if (lane < n) slot_to_union[lane] = local ? pos_first : -1;
    if (is_first) {
      union_ids[pos_self] = id;
      if (row_mask) row_mask[pos_self] = mask;
    }
    if (lane == 0) *union_count = __popcll(bal);
  }
  *mask_out = mask;
  *count_out = __popcll(bal);
  *eq_out = eq;
  return is_first ? pos_self : -1;
}

// The token-major slot list (MoeLayer::forward_token_major_decode runs every
// (row, selected expert) pair on its own): slot t = r*k + j holds id[t] for
// row r alone, so an expert chosen by several rows is swept once per row.
// Same outputs and return value as union_wave, with U = n.
__device__ int identity_slots(const int32_t* ids_lds, int n, int k, int lane, int32_t* union_ids,
                              int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask,
                              uint32_t* mask_out, int* count_out, uint64_t* eq_out) {
  const bool used = lane < n;
  const uint32_t mask = used ? 1u << (lane / k) : 0u;
  if (used) {
    slot_to_union[lane] = lane;
    union_ids[lane] = ids_lds[lane];
    row_mask[lane] = mask;
  }
  if (lane == 0) *union_count = n;
  *mask_out = mask;
  *count_out = n;
  *eq_out = used ? 1ull << lane : 0ull;
  return used ? lane : -1;
}

__global__ __launch_bounds__(64) void union_kernel(const int32_t* __restrict__ ids, int rows, int k, int lo, int hi,
                                                   int32_t* union_ids, int32_t* union_count,
                                                   int32_t* slot_to_union, uint32_t* row_mask) {
  __shared__ __align__(16) int32_t s_ids[kMaxIds];
  const int lane = threadIdx.x;
  const int n = rows * k;
  s_ids[lane] = lane < n ? ids[lane] : -1;
  __syncthreads();
  uint32_t mask;
  int count;
  uint64_t eq;
  union_wave(s_ids, n, k, rows, lo, hi, lane, union_ids, union_count, slot_to_union, row_mask, &mask, &count, &eq);
}

// Order-preserving map of a float key to uint32 (larger float -> larger
// integer); +0 and -0 map to neighbours, never to 0 except the all-ones NaN.
__device__ __forceinline__ uint32_t key_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
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
  int selj[G];      // round that took the expert, -1 if none
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const bool valid = lane * G + i < E;
    const float kf = softmax ? in.lv[i] : (float)in.sv[i] + in.bv[i];
    key[i] = valid ? key_bits(kf) : 0u;
    selj[i] = -1;
  }
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
    const int be = min(wl * G + wi, E - 1);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < G; ++i)
        if (i == wi) {
          key[i] = 0u;
          selj[i] = j;
        }
    }
    if (j == 0) top_logit = key_float(m);  // softmax: the largest logit
    if (lane == 0) {
      if (ids_out != nullptr) ids_out[r * k + j] = be;
      ids_lds[r * k + j] = be;
    }
  }
  if (w_out == nullptr) return;
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

// This lane's share of chunk c of one dense fp32 router row (or the gate
// vector) times the R input rows, in fp64: bf16 x fp32 products are exact in
// fp64.  Lanes past h load an in-bounds copy and add zeros.
template <int R>
__device__ __forceinline__ void router_dot_f32(const RouteParams& p, const float* row, int c, int lane,
                                               double (&acc)[R]) {
  const int h = p.h;
  constexpr int kIt = kRouterChunk / 256;
  float4 wv[kIt];
  uint2 xv[R][kIt];
  bool ok[kIt];
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int col = c * kRouterChunk + it * 256 + lane * 4;
    ok[it] = col < h;
    const int cc = ok[it] ? col : h - 4;  // in-bounds; the contribution is dropped below
    const u32x4 w4 = ld_stream(reinterpret_cast<const uint8_t*>(row + cc));
    wv[it] = make_float4(__uint_as_float(w4.x), __uint_as_float(w4.y), __uint_as_float(w4.z), __uint_as_float(w4.w));
#pragma unroll
    for (int r = 0; r < R; ++r) xv[r][it] = *reinterpret_cast<const uint2*>(p.x + (size_t)r * h + cc);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const double w0 = ok[it] ? (double)wv[it].x : 0.0, w1 = ok[it] ? (double)wv[it].y : 0.0;
      const double w2 = ok[it] ? (double)wv[it].z : 0.0, w3 = ok[it] ? (double)wv[it].w : 0.0;
      acc[r] = __builtin_fma((double)bf16_to_f32(xv[r][it].x & 0xFFFFu), w0, acc[r]);
      acc[r] = __builtin_fma((double)bf16_to_f32(xv[r][it].x >> 16), w1, acc[r]);
      acc[r] = __builtin_fma((double)bf16_to_f32(xv[r][it].y & 0xFFFFu), w2, acc[r]);
      acc[r] = __builtin_fma((double)bf16_to_f32(xv[r][it].y >> 16), w3, acc[r]);
    }
  }
}

// The same for an NVFP4 router row e: lane covers 8 consecutive columns (4
// bytes of E2M1 codes, even column in the low nibble, and their E4M3 block
// scale).  code x scale is exact in fp32 (at most 6 significant bits) and its
// product with a bf16 input exact in fp64; the per-tensor scale2 multiplies
// the row's finished fp64 sum.  Lanes past h load an in-bounds copy and take
// a zero scale.
template <int R>
__device__ __forceinline__ void router_dot_nvfp4(const RouteParams& p, int e, int c, int lane, double (&acc)[R]) {
  typedef __attribute__((address_space(1))) const uint32_t global_u32;
  typedef __attribute__((address_space(1))) const uint8_t global_u8;
  const int h = p.h;
  const int col = c * kRouterChunk + lane * 8;
  const bool ok = col < h;
  const int cc = ok ? col : h - 8;
  const uint32_t q = __builtin_nontemporal_load((global_u32*)(p.router_packed + (size_t)e * (size_t)(h >> 1) + (cc >> 1)));
  const uint32_t sb = __builtin_nontemporal_load((global_u8*)(p.router_scales + (size_t)e * (size_t)(h >> 4) + (cc >> 4)));
  u32x4 xv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) xv[r] = *reinterpret_cast<const u32x4*>(p.x + (size_t)r * h + cc);
  const double sc = ok ? (double)e4m3<0>(sb) : 0.0;
  double wv[8];
  const bf16x2 d0 = e2m1x2<0>(q), d1 = e2m1x2<1>(q), d2 = e2m1x2<2>(q), d3 = e2m1x2<3>(q);
  const uint32_t du[4] = {__builtin_bit_cast(uint32_t, d0), __builtin_bit_cast(uint32_t, d1),
                          __builtin_bit_cast(uint32_t, d2), __builtin_bit_cast(uint32_t, d3)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wv[2 * i] = (double)bf16_to_f32(du[i] & 0xFFFFu) * sc;
    wv[2 * i + 1] = (double)bf16_to_f32(du[i] >> 16) * sc;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    acc[r] = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[r] = __builtin_fma((double)bf16_to_f32(xv[r][i] & 0xFFFFu), wv[2 * i], acc[r]);
      acc[r] = __builtin_fma((double)bf16_to_f32(xv[r][i] >> 16), wv[2 * i + 1], acc[r]);
    }
  }
}

template <int R>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteParams p) {
  __shared__ double part[kMaxRouterChunks][kMaxRows];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h = p.h, E = p.E;
  const int nkc = (h + kRouterChunk - 1) / kRouterChunk;
  const int e = blockIdx.x;

  if (wave < nkc) {
    const int c = wave;
    double acc[R];
    if (p.router_fp4 && e < E)
      router_dot_nvfp4<R>(p, e, c, lane, acc);
    else
      router_dot_f32<R>(p, (e < E) ? p.router_w + (size_t)e * h : p.gate_vec, c, lane, acc);
    wave_sum_n<R>(acc);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) part[c][r] = acc[r];
    }
  }
  __syncthreads();
  // Wave 0: lane r sums row r's chunk partials in chunk order and takes the
  // sigmoid (the gate row always; router rows for sigmoid routing), and lane
  // 0 writes every row's results.  The kernel that follows reads them after
  // the kernel boundary.
  if (wave == 0) {
    double z = 0.0, sg = 0.0;
    if (lane < R) {
      for (int cc = 0; cc < nkc; ++cc) z += part[cc][lane];
      if (p.router_fp4 && e < E) z *= (double)p.router_scale2;
      // The gate takes the fp64 sum; routing scores take the fp32 logit, the
      // value top-k sees.
      if (e == E)
        sg = p.ungated ? 1.0 : 1.0 / (1.0 + exp(-z));
      else if (p.route_kind == MOE_ROUTE_SIGMOID_BIAS)
        sg = 1.0 / (1.0 + exp(-(double)(float)z));
    }
    double zr[R], sr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint64_t zb = __builtin_bit_cast(uint64_t, z), sb = __builtin_bit_cast(uint64_t, sg);
      zr[r] = __builtin_bit_cast(double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(zb >> 32), r) << 32) |
                                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)zb, r));
      sr[r] = __builtin_bit_cast(double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(sb >> 32), r) << 32) |
                                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)sb, r));
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (e < E) {
          p.logits[r * E + e] = (float)zr[r];
          p.score[r * E + e] = sr[r];
        } else {
          p.gamma[r] = (float)sr[r];
        }
      }
    }
  }
}

// moe_route's top-k: one block, one wave per row, on the logits and scores
// route_kernel stored (visible across the kernel boundary).
template <int G>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(RouteParams p) {
  __shared__ __align__(16) int32_t s_ids[kMaxIds];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  if (wave >= p.rows) return;
  TopkIn<G> in;
  topk_load<G>(p, wave, lane, in);
  topk_select<G>(p, wave, lane, in, s_ids, p.ids_out, p.w_out);
}

// ---------------------------------------------------------------- sweeps
// Copy the slot table into LDS (all 65 entries: those past U are stale and
// never read, and not waiting for U saves a round trip).  Later reads come
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
// whose id is this expert (bit t): row r's pair is r*k + j for the one j its
// bits name (a row's ids are distinct).
__device__ __forceinline__ SlotInfo slot_info(const ExpertPtrs& e, int ex, int inter, uint32_t row_mask, uint64_t eq,
                                              int k) {
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
  const uint64_t kmask = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    const uint64_t m = r * k < 64 ? (eq >> (r * k)) & kmask : 0ull;
    si.pair[r] = m ? (uint8_t)(r * k + __builtin_ctzll(m)) : (uint8_t)0xFF;
  }
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

// Down-sweep segments (one wave): a segment is one union slot and a group of
// up to kDownGroup of the rows that use it, routed slots in union order (lane
// su holds slot su's row mask, 0 past U), then the shared slot's groups of all
// R rows.  seg_rows[s] holds row i of the group in bits 4i..4i+3 and the row
// count in bits 28..31; seg_cum[s] is the summed work weight of the segments
// before s (seg_cum[count] the total).  Returns the number of segments.
__device__ int build_segments(uint32_t mask, int lane, int R, int32_t* seg_slot, uint32_t* seg_rows,
                              int32_t* seg_cum) {
  const int cnt = __popc(mask);
  const int groups = (cnt + kDownGroup - 1) / kDownGroup;
  int incl = groups;                          // inclusive prefix sums over lanes: segments
  int wincl = groups * kSegCostBase + cnt;    // and weight
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o), wv = __shfl_up(wincl, o);
    if (lane >= o) {
      incl += v;
      wincl += wv;
    }
  }
  const int seg = incl - groups;
  int wcum = wincl - (groups * kSegCostBase + cnt);
  for (int g = 0; g < groups; ++g) {
    uint32_t packed = 0;
    int n = 0;
    for (int r = 0; r < kMaxRows && n < kDownGroup; ++r) {
      // rows of earlier groups are skipped
      if (((mask >> r) & 1u) && __popc(mask & ((1u << r) - 1u)) >= g * kDownGroup) {
        packed |= (uint32_t)r << (4 * n);
        ++n;
      }
    }
    seg_slot[seg + g] = lane;
    seg_rows[seg + g] = packed | ((uint32_t)n << 28);
    seg_cum[seg + g] = wcum;
    wcum += kSegCostBase + n;
  }
  int total = __shfl(incl, 63);
  wcum = __shfl(wincl, 63);
  for (int g = 0; g * kDownGroup < R; ++g) {
    uint32_t packed = 0;
    int n = 0;
    for (int r = g * kDownGroup; r < R && n < kDownGroup; ++r, ++n) packed |= (uint32_t)r << (4 * n);
    if (lane == 0) {
      seg_slot[total] = kSharedSlot;
      seg_rows[total] = packed | ((uint32_t)n << 28);
      seg_cum[total] = wcum;
    }
    wcum += kSegCostBase + n;
    ++total;
  }
  if (lane == 0) seg_cum[total] = wcum;
  return total;
}

// Gate+up sweep.  It starts with the routing decisions: every block runs
// top-k on the logits the router pass stored (one wave per row), the union
// and the slot table, all in LDS; block 0 also writes them to the workspace
// for the down sweep and the blend.  Redundant work in every block costs a
// few microseconds of arithmetic on 24 KB of L2 reads, against a grid-wide
// hand-off that would cost a ticket, fences and an extra memory round trip.
//
// Work items are rows n of each union slot's gate and up matrices (the shared
// expert's Is rows first, then each routed slot's I rows).
// Block b owns items b, b + B, b + 2B, ... (B blocks), so all blocks sweep
// the weights front to back together; its waves claim the block's items in
// order from a counter in LDS.  Waves that share a SIMD are not issued evenly
// (the oldest goes first): with claims, one that is issued less simply takes
// fewer items, instead of finishing far behind its neighbours.  A claim is an
// LDS atomic, tracked apart from the weight loads, so taking one never waits
// for prefetched weights.  A wave loads its next items while it computes the
// current one.  For each row r that uses the slot:
//   act[slot][r][n] = bf16(silu(g) * v), g = W_gate[n,:] . x_r, v = W_up[n,:] . x_r.
template <int R, int NCH, int G>
__global__ __launch_bounds__(kMaxSweepThreads) void gateup_kernel(SweepParams p) {
  constexpr int kXUnits = R * NCH * kChunkUnits;  // 16-byte units of staged x
  constexpr int kXPer = (kXUnits + kMaxSweepThreads - 1) / kMaxSweepThreads;
  constexpr bool kPtab = G == 4;  // E <= 256: every expert's pointers fit in LDS
  extern __shared__ u32x4 xs[];  // [R][NCH][256] staged x rows
  __shared__ SlotInfo s_slots[kNumSlots];
  __shared__ ExpertPtrs s_ptab[kPtab ? 64 * G : 1];
  __shared__ __align__(16) int32_t s_ids[kMaxIds];
  __shared__ float s_w[kMaxIds];
  __shared__ int32_t s_uids[kMaxIds], s_s2u[kMaxIds];
  __shared__ uint32_t s_rmask[kMaxIds];
  __shared__ int s_next;  // the block's next unclaimed item
  __shared__ int s_union;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h = p.h;
  const RouteParams& rp = p.route;
  const bool publish = blockIdx.x == 0;

  // Prologue.  Every load that does not depend on routing is issued first --
  // x, the top-k inputs, every expert's weight pointers, then the first
  // item's weights -- and each is consumed in issue order, so no wait on the
  // in-order load counter covers a load issued after it.  No global store
  // precedes a barrier (a barrier after a store waits for every outstanding
  // load): block 0 writes the routing results to the workspace only after
  // the last barrier.
  u32x4 xv[kXPer];
  auto x_unit = [&](int i, int& r, int& dst) {  // unit i of the staged x: its row, LDS slot and column
    r = i / (NCH * kChunkUnits);
    const int rem = i - r * NCH * kChunkUnits;
    const int c = rem / kChunkUnits, un = rem - c * kChunkUnits;
    dst = (r * NCH + c) * kChunkUnits + swz_unit(un);
    return c * kChunk + un * 8;
  };
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    int r, dst;
    const int col = x_unit(min((int)threadIdx.x + q * kMaxSweepThreads, kXUnits - 1), r, dst);
    xv[q] = ld_global(reinterpret_cast<const u32x4*>(p.x + (size_t)r * h + (col < h ? col : h - 8)));
  }
  // Unconditional, with clamped indices: a branch around a load would leave
  // the wait-count pass unsure of the count and make it wait for everything.
  TopkIn<G> tin;
  topk_load<G>(rp, wave < R ? wave : R - 1, lane, tin);
  ExpertPtrs ep;
  if (kPtab) ep = expert_ptrs(rp, min((int)threadIdx.x, rp.E - 1));
  if (threadIdx.x == 0) {
    s_next = 0;
    s_slots[kSharedSlot] = shared_slot_info(rp, (1u << R) - 1u);
  }
  __syncthreads();

  // Items: the shared expert's Is rows first, then each routed slot's I rows.
  // The item id of the block's claim i is b + i * B (not yet checked against
  // the item count, which needs U).
  auto claim_id = [&]() -> long long {
    int i = 0;
    if (lane == 0) i = atomicAdd(&s_next, 1);
    i = __builtin_amdgcn_readfirstlane(i);
    return (long long)blockIdx.x + (long long)i * gridDim.x;
  };
  // What the compute needs of an item's slot, in scalar registers: the rows
  // that use it, the per-tensor scales and each row's pair index (byte r).
  constexpr int kPairWords = (R + 3) / 4;
  struct ItemSlot {
    uint32_t row_mask;
    float gate_scale2, up_scale2;
    uint32_t pairw[kPairWords];
  };
  RowRegs<NCH> ga, ua, gb, ub;
  ItemSlot sa, sb;
  int na = 0, nb = 0;
  auto fetch = [&](int id, RowRegs<NCH>& g, RowRegs<NCH>& u, ItemSlot& si, int& n) {
    int slot;
    if (id < p.shared_inter) {
      slot = kSharedSlot;
      n = id;
    } else {
      slot = (id - p.shared_inter) / p.inter;
      n = id - p.shared_inter - slot * p.inter;
    }
    const SlotInfo& e = s_slots[slot];
    load_row<NCH>(g, uniform_ptr(e.gate_packed), uniform_ptr(e.gate_scales), n, h, lane);
    load_row<NCH>(u, uniform_ptr(e.up_packed), uniform_ptr(e.up_scales), n, h, lane);
    si.row_mask = uniform_u32(e.row_mask);
    si.gate_scale2 = uniform_f32(e.gate_scale2);
    si.up_scale2 = uniform_f32(e.up_scale2);
#pragma unroll
    for (int q = 0; q < kPairWords; ++q) si.pairw[q] = uniform_u32(reinterpret_cast<const uint32_t*>(e.pair)[q]);
  };
  // A first claim on a shared-expert row needs no routing: its weights are
  // requested now and arrive while the block runs top-k.  A wave whose first
  // claim is a routed row loads a shared row some other wave claimed (a cache
  // hit; it is not computed) so the load stays unconditional, and fetches its
  // item later.  That shared row also stands in for every item past the last
  // claim: its loads are always in bounds.
  long long first = claim_id();
  const bool early = first < p.shared_inter;
  const int any_id = early ? (int)first : (int)(first % p.shared_inter);
  fetch(any_id, ga, ua, sa, na);
  // Nothing that reads a loaded value may be scheduled above the fetch.
  __builtin_amdgcn_sched_barrier(0);

  // Consume, in issue order: x (zero past h), top-k, the pointer table.
#pragma unroll
  for (int q = 0; q < kXPer; ++q) {
    const int i = (int)threadIdx.x + q * kMaxSweepThreads;
    if (i < kXUnits) {
      int r, dst;
      const int col = x_unit(i, r, dst);
      xs[dst] = col < h ? xv[q] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Every prologue load is waited for here on every path (see consume()),
  // used or not.
#pragma unroll
  for (int q = 0; q < kXPer; ++q) asm volatile("" ::"v"(xv[q]));
#pragma unroll
  for (int i = 0; i < G; ++i) asm volatile("" ::"v"(tin.lv[i]), "v"(tin.bv[i]), "v"(tin.sv[i]));
  if (kPtab) {
#pragma unroll
    for (int i = 0; i < 6; ++i) asm volatile("" ::"v"(ep.p[i]));
#pragma unroll
    for (int i = 0; i < 3; ++i) asm volatile("" ::"v"(ep.scale2[i]));
  }
  if (wave < R) topk_select<G>(rp, wave, lane, tin, s_ids, nullptr, publish ? s_w : nullptr);
  if (kPtab && (int)threadIdx.x < rp.E) s_ptab[threadIdx.x] = ep;
  __syncthreads();
  if (wave == 0) {
    uint32_t mask;
    int count;
    uint64_t eq;
    const int pos = p.token_major ? identity_slots(s_ids, R * rp.k, rp.k, lane, s_uids, &s_union, s_s2u, s_rmask,
                                                   &mask, &count, &eq)
                                  : union_wave(s_ids, R * rp.k, rp.k, R, rp.expert_lo, rp.expert_hi, lane, s_uids,
                                               &s_union, s_s2u, s_rmask, &mask, &count, &eq);
    if (pos >= 0) {  // lane is the union entry's first slot
      const int ex = s_ids[lane];
      s_slots[pos] = slot_info(kPtab ? s_ptab[ex] : expert_ptrs(rp, ex), ex, rp.inter, mask, eq, rp.k);
    }
  }
  __syncthreads();
  const int U = s_union;
  const long long total = (long long)p.shared_inter + (long long)U * p.inter;
  // Item id of the block's next claim, or -1 once the block's items run out
  // (claims only grow, so every later claim fails too).
  auto claim = [&]() -> int {
    const long long id = claim_id();
    return id < total ? (int)id : -1;
  };

  auto compute = [&](const RowRegs<NCH>& g, const RowRegs<NCH>& u, const ItemSlot& si, int n) {
    float ag[R], au[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      ag[r] = 0.f;
      au[r] = 0.f;
    }
    // Lanes past the last column hold zero codes and scales, and the staged
    // x is zero there too, so every lane runs the same code.
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      bf16x2 gw[16], uw[16];
      decode32(g.q[c], gw);
      decode32(u.q[c], uw);
      const uint32_t gsc = scale_pair<NCH>(g, c, h, lane), usc = scale_pair<NCH>(u, c, h, lane);
      const float gs0 = e4m3<0>(gsc), gs1 = e4m3<1>(gsc);
      const float us0 = e4m3<0>(usc), us1 = e4m3<1>(usc);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if ((si.row_mask >> r) & 1u) {
          const u32x4* xr = xs + (r * NCH + c) * kChunkUnits;
          const u32x4 x0 = xr[lane], x1 = xr[64 + lane], x2 = xr[128 + lane], x3 = xr[192 + lane];
          ag[r] = dot32(gw, x0, x1, x2, x3, gs0, gs1, ag[r]);
          au[r] = dot32(uw, x0, x1, x2, x3, us0, us1, au[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if ((si.row_mask >> r) & 1u) {
        float gu[2] = {ag[r], au[r]};
        wave_sum_n<2>(gu);
        const float gv = gu[0] * si.gate_scale2;
        const float uv = gu[1] * si.up_scale2;
        if (lane == 0) {
          const float a = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
          const uint32_t pr = (si.pairw[r >> 2] >> (8 * (r & 3))) & 0xFFu;
          p.act[(size_t)pr * p.act_stride + n] = f32_to_bf16(a);
        }
      }
    }
  };

  // Three register buffers in rotation: while one item is computed, the next
  // two are in flight.  Loads are always issued (the stand-in row once the
  // claims run out) so no branch separates them from the compute they
  // overlap.  An item id of -1 is loaded and waited for but not computed:
  // the first buffer of a wave whose first claim is a routed row, and every
  // buffer past the last claim.
  RowRegs<NCH> gc, uc;
  ItemSlot sc;
  int nc = 0;
  int id_a, id_b;
  if (early) {
    id_a = (int)first;  // first < Is <= total
    id_b = claim();
  } else {
    id_a = -1;
    id_b = first < total ? (int)first : -1;
  }
  const bool has_work = id_a >= 0 || id_b >= 0;
  fetch(id_b >= 0 ? id_b : any_id, gb, ub, sb, nb);
  // Block 0 publishes the routing results for the down sweep and the blend.
  if (publish && wave == 0) {
    const int n = R * rp.k;
    if (lane < n) {
      rp.ids_out[lane] = s_ids[lane];
      rp.w_out[lane] = s_w[lane];
      rp.slot_to_union[lane] = s_s2u[lane];
    }
    if (lane < U) {
      rp.union_ids[lane] = s_uids[lane];
      rp.row_mask[lane] = s_rmask[lane];
      rp.slots[lane] = s_slots[lane];
    }
    if (lane == 0) {
      *rp.union_count = U;
      rp.slots[kSharedSlot] = s_slots[kSharedSlot];
    }
    const int nseg =
        build_segments(lane < U ? s_slots[lane].row_mask : 0u, lane, R, p.seg_slot, p.seg_rows, p.seg_cum);
    if (lane == 0) *p.seg_count = nseg;
  }
  if (!has_work) return;
  // One exit, after a whole rotation: an exit after each item would give the
  // compiler paths back to the top with items still in flight, and the waits
  // it derives for those paths would drain the loads on every pass.  Items
  // past the last claim are waited for (their loads repeat a valid item) but
  // not computed.
  while (true) {
    const int id_c = id_b >= 0 ? claim() : -1;
    fetch(id_c >= 0 ? id_c : any_id, gc, uc, sc, nc);
    consume<NCH>(ga);
    consume<NCH>(ua);
    if (id_a >= 0) compute(ga, ua, sa, na);
    const int id_a2 = id_c >= 0 ? claim() : -1;
    fetch(id_a2 >= 0 ? id_a2 : any_id, ga, ua, sa, na);
    consume<NCH>(gb);
    consume<NCH>(ub);
    if (id_b >= 0) compute(gb, ub, sb, nb);
    const int id_b2 = id_a2 >= 0 ? claim() : -1;
    fetch(id_b2 >= 0 ? id_b2 : any_id, gb, ub, sb, nb);
    consume<NCH>(gc);
    consume<NCH>(uc);
    if (id_c >= 0) compute(gc, uc, sc, nc);
    if (id_a2 < 0) break;
    id_a = id_a2;
    id_b = id_b2;
  }
}

// Down sweep.  The work is the row space of "segments": a segment is one
// union slot and a group of up to kGroup of the rows that use it (a slot used
// by more rows than that is swept once per group).  Every wave takes an equal
// contiguous share of segments x h output rows -- at most two segments -- so
// waves never wait for each other.  A wave holds its group's act rows in
// registers (loaded once per segment) and loads its next batch of weight rows
// while it computes the current batch.  For row r of union slot u, with
// pair t the (row, expert) pair of (u, r):
//   y[t][n] = W_down[u][n,:] . act[t][:]
constexpr int kDownThreads = 256;
constexpr int kDownBatch = 4;  // weight rows per prefetch batch (stored as float4s)
constexpr int kDownBufs = 3;   // batches in the prefetch rotation

template <int NCH>
struct DownBatch {
  RowRegs<NCH> row[kDownBatch];
};

template <int NCH>
__global__ __launch_bounds__(kDownThreads) void down_kernel(SweepParams p) {
  constexpr int kGroup = kDownGroup;  // act rows held per segment (16 VGPRs each per 2048 columns)
  constexpr int kMaxSegs = kMaxDownSegs;
  __shared__ SlotInfo s_slots[kNumSlots];
  __shared__ int s_seg_slot[kMaxSegs];
  __shared__ uint32_t s_seg_rows[kMaxSegs];  // row i of the group in bits 4i..4i+3, count in bits 28..31
  __shared__ int s_seg_cum[kMaxSegs + 1];    // work weight before segment s
  __shared__ int s_nseg;
  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int nwaves = blockDim.x >> 6;
  const int h = p.h;
  // The slot table and the segment table (written by the gate/up sweep's
  // block 0), each thread's loads all issued before its first store.
  {
    constexpr int kPer = (kMaxSegs + 1 + kDownThreads - 1) / kDownThreads;
    int sl[kPer], sw[kPer];
    uint32_t sr[kPer];
    const int nseg = *p.seg_count;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = (int)threadIdx.x + q * kDownThreads;
      const int ic = i < kMaxSegs ? i : kMaxSegs - 1;
      sl[q] = p.seg_slot[ic];
      sr[q] = p.seg_rows[ic];
      sw[q] = p.seg_cum[i <= kMaxSegs ? i : kMaxSegs];
    }
    load_slot_table<kDownThreads>(s_slots, p.slots);
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int i = (int)threadIdx.x + q * kDownThreads;
      if (i < kMaxSegs) {
        s_seg_slot[i] = sl[q];
        s_seg_rows[i] = sr[q];
      }
      if (i <= kMaxSegs) s_seg_cum[i] = sw[q];
    }
    if (threadIdx.x == 0) s_nseg = nseg;
  }
  __syncthreads();

  // Each segment gets a group of waves in proportion to its work weight
  // (kSegCostBase + rows per weight row: a two-row segment costs more
  // arithmetic per byte): with cumulative weights c_s and total C, virtual
  // wave v of V works on the segment s with c_s <= v * C / V < c_{s+1}.  The
  // group's waves take interleaved batches of kDownBatch rows: every group
  // sweeps its matrix front to back together.  V >= C gives every segment
  // at least one virtual wave; with fewer waves than that a wave takes
  // several virtual waves in turn.
  const int W = gridDim.x * nwaves;
  const int nseg = s_nseg;
  const int C = s_seg_cum[nseg];
  const int V = W > C ? W : C;

  DownBatch<NCH> buf[kDownBufs];
  u32x4 act[kGroup][NCH][4];
  for (int v = blockIdx.x * nwaves + wave; v < V; v += W) {
    const long long key = (long long)v * C / V;  // in [0, C)
    int seg = 0;
    for (int span = 64; span > 0; span >>= 1)  // largest s with c_s <= key (nseg <= 128)
      if (seg + span < nseg && s_seg_cum[seg + span] <= key) seg += span;
    seg = uniform_int(seg);
    const long long c0 = s_seg_cum[seg], c1 = s_seg_cum[seg + 1];
    const int first = (int)(((long long)V * c0 + C - 1) / C);  // first virtual wave of the segment
    const int last = (int)(((long long)V * c1 + C - 1) / C);
    const int n_end = h;
    const int slot = uniform_int(s_seg_slot[seg]);
    const uint32_t rows = uniform_u32(s_seg_rows[seg]);
    const int cnt = (int)(rows >> 28);
    const SlotInfo& si = s_slots[slot];
    const int K = uniform_int(si.inter);
    const uint8_t* const d_packed = uniform_ptr(si.down_packed);
    const uint8_t* const d_scales = uniform_ptr(si.down_scales);
    const float d2 = uniform_f32(si.down_scale2);
    const int stride = (last - first) * kDownBatch;
    const int n0 = (v - first) * kDownBatch;
    if (n0 >= n_end) continue;
    // Pair index of each group row (unused entries repeat the last row).
    int prs[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int r = (int)((rows >> (4 * (i < cnt ? i : cnt - 1))) & 0xFu);
      prs[i] = uniform_int(si.pair[r]);
    }
    // act rows of the group.  Lanes past K read the row's first columns:
    // finite values that meet zeroed scales.
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const uint16_t* src = p.act + (size_t)prs[i] * p.act_stride;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int col = c * kChunk + lane * 32;
        const u32x4* q = reinterpret_cast<const u32x4*>(src + (col < K ? col : 0));
#pragma unroll
        for (int u = 0; u < 4; ++u) act[i][c][u] = q[u];
      }
    }
    auto fetch = [&](int nb, DownBatch<NCH>& b) {
#pragma unroll
      for (int i = 0; i < kDownBatch; ++i) {
        const int n = nb + i < n_end ? nb + i : n_end - 1;  // rows past the range are loaded, not computed
        load_row<NCH>(b.row[i], d_packed, d_scales, n, K, lane);
      }
    };
    // Rows of a batch: per group row, the batch's dot products are reduced
    // together and written with 16-byte stores (batches start at multiples
    // of 4 and h is a multiple of 32).
    auto compute = [&](int nb, const DownBatch<NCH>& b) {
      float acc[kGroup][kDownBatch];
#pragma unroll
      for (int g = 0; g < kGroup; ++g)
#pragma unroll
        for (int i = 0; i < kDownBatch; ++i) acc[g][i] = 0.f;
#pragma unroll
      for (int i = 0; i < kDownBatch; ++i) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          bf16x2 dw[16];
          decode32(b.row[i].q[c], dw);
          const uint32_t sc = scale_pair<NCH>(b.row[i], c, K, lane);
          const float s0 = e4m3<0>(sc), s1 = e4m3<1>(sc);
#pragma unroll
          for (int g = 0; g < kGroup; ++g)
            if (g < cnt)
              acc[g][i] = dot32(dw, act[g][c][0], act[g][c][1], act[g][c][2], act[g][c][3], s0, s1, acc[g][i]);
        }
      }
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        if (g < cnt) {
          wave_sum_n<kDownBatch>(acc[g]);
          float* dst = p.y + (size_t)prs[g] * h + nb;
          if (lane == 0) {

#pragma unroll
            for (int i = 0; i < kDownBatch; i += 4) {
              if (nb + i + 4 <= n_end) {
                *reinterpret_cast<float4*>(dst + i) =
                    make_float4(acc[g][i] * d2, acc[g][i + 1] * d2, acc[g][i + 2] * d2, acc[g][i + 3] * d2);
              } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                  if (nb + i + q < n_end) dst[i + q] = acc[g][i + q] * d2;
              }
            }
          }
        }
      }
    };
    // kDownBufs batches in rotation: while one is computed, the next
    // kDownBufs - 1 are in flight.  Batches past the range reload the last
    // row (no branch around the loads); they are waited for but not
    // computed.  The loop runs whole rotations with one way back to the top:
    // an exit after each batch would give the compiler paths back to the top
    // with batches still in flight, and the waits it derives for those paths
    // would drain the loads on every pass.
    int nf = n0;  // next batch to fetch
#pragma unroll
    for (int i = 0; i < kDownBufs - 1; ++i) {
      fetch(nf < n_end ? nf : n_end - 1, buf[i]);
      nf += stride;
    }
    // The act rows are waited for here, on every path (see consume()).
#pragma unroll
    for (int i = 0; i < kGroup; ++i)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int u = 0; u < 4; ++u) asm volatile("" ::"v"(act[i][c][u]));
    const int rounds = ((n_end - n0 + stride - 1) / stride + kDownBufs - 1) / kDownBufs;
    int nc = n0;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int i = 0; i < kDownBufs; ++i) {
        fetch(nf < n_end ? nf : n_end - 1, buf[(i + kDownBufs - 1) % kDownBufs]);
        nf += stride;
#pragma unroll
        for (int q = 0; q < kDownBatch; ++q) consume<NCH>(buf[i].row[q]);
        if (nc < n_end) compute(nc, buf[i]);
        nc += stride;
      }
    }
  }
}

// ---------------------------------------------------------------- down sweep + blend, few rows
// With few rows the activations of every (row, expert) pair fit in LDS, and a
// single kernel runs the down projections and the weighted sum.  Block b owns
// output rows [b*nr, (b+1)*nr) of every union slot and of the shared expert,
// so every term of out[r][n] is computed inside the block: the blend needs no
// kernel of its own and the expert outputs no round trip through memory.
//   y[t][n]   = W_down[u][n,:] . act[t][:]        (t: the pair of slot u and row r)
//   out[r][n] = bf16( sum_{j<k} w[r][j] * y[r*k + j][n] + gamma[r] * y[rows*k + r][n] )
// Each y value is computed exactly as down_kernel computes it (same lane
// columns, same chunk order, same reduction, scale2 last) and the sum runs in
// blend_kernel's order, so both paths write the same bytes; y is also written
// to the workspace.  Work units are (slot, batch of kDownBatch output rows),
// the shared expert's first; the block's waves claim them from an LDS counter
// and keep two units in flight while they compute one.
constexpr int kDbThreads = 768;  // 12 waves, one block per CU
constexpr int kDbMaxRows = 4;    // rows served by this kernel (act of every pair in LDS)
constexpr int kDbActPer = 12;    // act staging loads per thread (16 bytes each)

template <int R, int NCH>
__global__ __launch_bounds__(kDbThreads) void down_blend_kernel(SweepParams p, int nr) {
  static_assert(R <= kDbMaxRows, "down_blend_kernel serves at most kDbMaxRows rows");
  extern __shared__ u32x4 s_act[];  // [P][NCH][256] act rows (swizzled), then y as floats [P][nr]
  __shared__ SlotInfo s_slots[kNumSlots];
  __shared__ float s_w[kMaxIds];
  __shared__ float s_gamma[kDbMaxRows];
  __shared__ int32_t s_local[kMaxIds];  // slot_to_union >= 0 (EP share: local expert)
  __shared__ int s_next, s_union;
  const RouteParams& rp = p.route;
  const int lane = threadIdx.x & 63;
  const int h = p.h, k = rp.k;
  const int P = R * k + R;  // pairs
  float* s_y = reinterpret_cast<float*>(s_act + (size_t)P * NCH * kChunkUnits);
  const int n_begin = blockIdx.x * nr;
  const int nbat = nr / kDownBatch;

  // Prologue: the loads that do not depend on the slot table are issued
  // first (slot table, U, weights, gates, act rows), then a shared-expert
  // unit's weights, and each is consumed in issue order.
  constexpr int kSlotWords = (int)(sizeof(SlotInfo) / 4);
  constexpr int kTabPer = (kNumSlots * kSlotWords + kDbThreads - 1) / kDbThreads;
  uint32_t tab[kTabPer];
#pragma unroll
  for (int q = 0; q < kTabPer; ++q) {
    const int i = (int)threadIdx.x + q * kDbThreads;
    tab[q] = ld_global(reinterpret_cast<const uint32_t*>(p.slots) + (i < kNumSlots * kSlotWords ? i : 0));
  }
  const int ucount = ld_global(p.union_count);
  const int tw = (int)threadIdx.x < R * k ? (int)threadIdx.x : 0;
  const float wv = ld_global(rp.w_out + tw);
  const int s2u = ld_global(rp.slot_to_union + tw);
  const float gv = ld_global(rp.gamma + ((int)threadIdx.x < R ? (int)threadIdx.x : 0));
  // act rows: unit i of the staging is 16 bytes of pair t, chunk c, unit un
  // (columns past the pair's K read a valid copy and are stored as zeros);
  // the launcher serves this kernel only when one pass of kDbActPer loads per
  // thread covers every unit
  const int units = P * NCH * kChunkUnits;
  constexpr int kActPer = kDbActPer;
  auto act_src = [&](int i, int& dst, bool& valid) {
    const int t = i / (NCH * kChunkUnits);
    const int rem = i - t * NCH * kChunkUnits;
    const int c = rem / kChunkUnits, un = rem - c * kChunkUnits;
    const int K = t < R * k ? p.inter : p.shared_inter;
    const int col = c * kChunk + un * 8;
    valid = col < K;
    dst = (t * NCH + c) * kChunkUnits + swz_unit(un);
    return reinterpret_cast<const u32x4*>(p.act + (size_t)t * p.act_stride + (valid ? col : 0));
  };
  u32x4 av[kActPer];
#pragma unroll
  for (int q = 0; q < kActPer; ++q) {
    const int i = (int)threadIdx.x + q * kDbThreads;
    int dst;
    bool valid;
    av[q] = ld_global(act_src(i < units ? i : 0, dst, valid));
  }
  if (threadIdx.x == 0) {
    s_next = 0;
    s_slots[kSharedSlot] = shared_slot_info(rp, (1u << R) - 1u);
  }
  __syncthreads();

  auto claim_id = [&]() -> int {
    int i = 0;
    if (lane == 0) i = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(i);
  };
  // What the compute needs of a unit, in scalar registers.
  constexpr int kPairWords = (R + 3) / 4;
  struct UnitInfo {
    int n, K;
    float d2;
    uint32_t mask;
    uint32_t pairw[kPairWords];
  };
  // unit id: slot s = id / nbat (0: the shared expert, then union slot s - 1),
  // output rows n_begin + (id % nbat) * kDownBatch + 0..3
  auto fetch = [&](int id, DownBatch<NCH>& b, UnitInfo& ui) {
    const int sidx = id / nbat;
    const int slot = sidx == 0 ? kSharedSlot : sidx - 1;
    const int n = n_begin + (id - sidx * nbat) * kDownBatch;
    const SlotInfo& e = s_slots[slot];
    const uint8_t* const dp = uniform_ptr(e.down_packed);
    const uint8_t* const ds = uniform_ptr(e.down_scales);
    const int K = uniform_int(e.inter);
#pragma unroll
    for (int i = 0; i < kDownBatch; ++i) load_row<NCH>(b.row[i], dp, ds, n + i < h ? n + i : h - 1, K, lane);
    ui.n = n;
    ui.K = K;
    ui.d2 = uniform_f32(e.down_scale2);
    ui.mask = uniform_u32(e.row_mask);
#pragma unroll
    for (int q = 0; q < kPairWords; ++q) ui.pairw[q] = uniform_u32(reinterpret_cast<const uint32_t*>(e.pair)[q]);
  };
  // Shared-expert units need no slot table: the first claim is fetched now
  // when it is one; otherwise a shared unit stands in (loaded, not computed).
  // That stand-in also serves every unit past the last claim.
  const int first = claim_id();
  const bool early = first < nbat;
  const int any_id = early ? first : 0;
  DownBatch<NCH> ba, bb, bc;
  UnitInfo ia, ib, ic;
  fetch(any_id, ba, ia);
  __builtin_amdgcn_sched_barrier(0);

  // Consume, in issue order: the slot table, U, weights and gates, act rows.
  {
#pragma unroll
    for (int q = 0; q < kTabPer; ++q) {
      const int i = (int)threadIdx.x + q * kDbThreads;
      // the shared slot's entry is this call's (set above); every other is the gate/up sweep's
      if (i < kNumSlots * kSlotWords && i / kSlotWords != kSharedSlot)
        reinterpret_cast<uint32_t*>(s_slots)[i] = tab[q];
    }
    if (threadIdx.x == 0) s_union = ucount;
    if ((int)threadIdx.x < R * k) {
      s_w[threadIdx.x] = wv;
      s_local[threadIdx.x] = s2u >= 0;
    }
    if ((int)threadIdx.x < R) s_gamma[threadIdx.x] = gv;
#pragma unroll
    for (int q = 0; q < kActPer; ++q) {
      const int i = (int)threadIdx.x + q * kDbThreads;
      if (i < units) {
        int dst;
        bool valid;
        act_src(i, dst, valid);
        s_act[dst] = valid ? av[q] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < kTabPer; ++q) asm volatile("" ::"v"(tab[q]));
#pragma unroll
    for (int q = 0; q < kActPer; ++q) asm volatile("" ::"v"(av[q]));
  }
  __syncthreads();
  const int total = (s_union + 1) * nbat;
  auto claim = [&]() -> int {
    const int id = claim_id();
    return id < total ? id : -1;
  };

  // Rows of a unit in groups of two (act rows from LDS), each weight row
  // decoded once per group; y to LDS and the workspace.
  auto compute = [&](const DownBatch<NCH>& b, const UnitInfo& ui) {
#pragma unroll
    for (int g = 0; g < (R + 1) / 2; ++g) {
      const int r0 = 2 * g, r1 = 2 * g + 1;
      const bool u0 = (ui.mask >> r0) & 1u;
      const bool u1 = r1 < R && ((ui.mask >> r1) & 1u);
      if (!u0 && !u1) continue;
      const int p0 = (int)((ui.pairw[r0 >> 2] >> (8 * (r0 & 3))) & 0xFFu);
      const int p1 = r1 < R ? (int)((ui.pairw[r1 >> 2] >> (8 * (r1 & 3))) & 0xFFu) : p0;
      u32x4 x0[NCH][4], x1[NCH][4];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const u32x4* a0 = s_act + (p0 * NCH + c) * kChunkUnits;
        const u32x4* a1 = s_act + ((u1 ? p1 : p0) * NCH + c) * kChunkUnits;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x0[c][q] = a0[q * 64 + lane];
          x1[c][q] = a1[q * 64 + lane];
        }
      }
      float acc0[kDownBatch], acc1[kDownBatch];
#pragma unroll
      for (int i = 0; i < kDownBatch; ++i) {
        acc0[i] = 0.f;
        acc1[i] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          bf16x2 dw[16];
          decode32(b.row[i].q[c], dw);
          const uint32_t sc = scale_pair<NCH>(b.row[i], c, ui.K, lane);
          const float s0 = e4m3<0>(sc), s1 = e4m3<1>(sc);
          if (u0) acc0[i] = dot32(dw, x0[c][0], x0[c][1], x0[c][2], x0[c][3], s0, s1, acc0[i]);
          if (u1) acc1[i] = dot32(dw, x1[c][0], x1[c][1], x1[c][2], x1[c][3], s0, s1, acc1[i]);
        }
      }
      auto emit = [&](float (&acc)[kDownBatch], int pr) {
        wave_sum_n<kDownBatch>(acc);
        if (lane == 0) {
          const int nl = ui.n - n_begin;
          float* dst = p.y + (size_t)pr * h + ui.n;
          if (ui.n + kDownBatch <= h) {
            *reinterpret_cast<float4*>(dst) =
                make_float4(acc[0] * ui.d2, acc[1] * ui.d2, acc[2] * ui.d2, acc[3] * ui.d2);
          } else {
#pragma unroll
            for (int i = 0; i < kDownBatch; ++i)
              if (ui.n + i < h) dst[i] = acc[i] * ui.d2;
          }
#pragma unroll
          for (int i = 0; i < kDownBatch; ++i) s_y[pr * nr + nl + i] = acc[i] * ui.d2;
        }
      };
      if (u0) emit(acc0, p0);
      if (u1) emit(acc1, p1);
    }
  };

  int id_a, id_b;
  if (early) {
    id_a = first;  // < nbat <= total
    id_b = claim();
  } else {
    id_a = -1;
    id_b = first < total ? first : -1;
  }
  if (id_a >= 0 || id_b >= 0) {
    fetch(id_b >= 0 ? id_b : any_id, bb, ib);
    // One exit, after a whole rotation (see the gate/up sweep).
    while (true) {
      const int id_c = id_b >= 0 ? claim() : -1;
      fetch(id_c >= 0 ? id_c : any_id, bc, ic);
#pragma unroll
      for (int q = 0; q < kDownBatch; ++q) consume<NCH>(ba.row[q]);
      if (id_a >= 0) compute(ba, ia);
      const int id_a2 = id_c >= 0 ? claim() : -1;
      fetch(id_a2 >= 0 ? id_a2 : any_id, ba, ia);
#pragma unroll
      for (int q = 0; q < kDownBatch; ++q) consume<NCH>(bb.row[q]);
      if (id_b >= 0) compute(bb, ib);
      const int id_b2 = id_a2 >= 0 ? claim() : -1;
      fetch(id_b2 >= 0 ? id_b2 : any_id, bb, ib);
#pragma unroll
      for (int q = 0; q < kDownBatch; ++q) consume<NCH>(bc.row[q]);
      if (id_c >= 0) compute(bc, ic);
      if (id_a2 < 0) break;
      id_a = id_a2;
      id_b = id_b2;
    }
#pragma unroll
    for (int q = 0; q < kDownBatch; ++q) {
      consume<NCH>(ba.row[q]);
      consume<NCH>(bb.row[q]);
    }
  }
  __syncthreads();

  // The weighted sum of the block's rows, in blend_kernel's order.
  const int t = (int)threadIdx.x;
  if (t < R * nr) {
    const int r = t / nr, i = t - (t / nr) * nr;
    const int n = n_begin + i;
    if (n < h) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j)
        if (p.partial == nullptr || s_local[r * k + j]) acc = __builtin_fmaf(s_w[r * k + j], s_y[(r * k + j) * nr + i], acc);
      if (p.partial != nullptr) {
        p.partial[(size_t)r * h + n] = acc;
      } else {
        acc = __builtin_fmaf(s_gamma[r], s_y[(R * k + r) * nr + i], acc);
        p.out[(size_t)r * h + n] = f32_to_bf16(acc);
      }
    }
  }
}

// Weighted sum and shared-expert blend, one thread per (row, column):
//   out[r][n] = bf16( sum_{j<k} w[r][j] * y[r*k + j][n] + gamma[r] * y[rows*k + r][n] )
// summed in fp32 in ascending j.  With partial non-null (one rank's share
// under expert parallelism) it writes the routed sum alone, in fp32, over the
// slots whose expert is local (slot_to_union >= 0): forward_token_major.rs
// blends with a zeroed shared term before the all-reduce.
__global__ __launch_bounds__(256) void blend_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                    const int32_t* __restrict__ slot_to_union,
                                                    const float* __restrict__ gamma, uint16_t* __restrict__ out,
                                                    float* __restrict__ partial, int h, int k, int rows) {
  constexpr int kB = 8;  // slots whose loads are issued together
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= h) return;
  // Outputs are stored by pair, so no load waits for another: each batch of
  // eight slots issues its weight and output loads together, then adds in
  // ascending j.
  const float g = gamma[r];
  const float ys = y[(size_t)(rows * k + r) * h + n];
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += kB) {
    float wv[kB], yv[kB];
    bool use[kB];
#pragma unroll
    for (int q = 0; q < kB; ++q) {
      const int j = j0 + q < k ? j0 + q : k - 1;
      wv[q] = w[r * k + j];
      yv[q] = y[(size_t)(r * k + j) * h + n];
      use[q] = j0 + q < k && (partial == nullptr || slot_to_union[r * k + j] >= 0);
    }
#pragma unroll
    for (int q = 0; q < kB; ++q)
      if (use[q]) acc = __builtin_fmaf(wv[q], yv[q], acc);
  }
  if (partial != nullptr) {
    partial[(size_t)r * h + n] = acc;
    return;
  }
  acc = __builtin_fmaf(g, ys, acc);
  out[(size_t)r * h + n] = f32_to_bf16(acc);
}

// The shared expert added after the all-reduce of the ranks' partials
// (forward_token_major.rs: moe_batched_blend, or residual_add when the gate
// weight is null, where gamma = 1):
//   out[r][n] = bf16( reduced[r][n] + gamma[r] * y[rows*k + r][n] )
__global__ __launch_bounds__(256) void ep_combine_kernel(const float* __restrict__ reduced,
                                                         const float* __restrict__ y,
                                                         const float* __restrict__ gamma,
                                                         uint16_t* __restrict__ out, int h, int k, int rows) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= h) return;
  const float acc = __builtin_fmaf(gamma[r], y[(size_t)(rows * k + r) * h + n], reduced[(size_t)r * h + n]);
  out[(size_t)r * h + n] = f32_to_bf16(acc);
}

// Read-bandwidth probe: every 16-byte unit of ``src`` read once with the
// sweeps' non-temporal 16-byte loads (each wave reads 1 KB contiguous per
// load, waves grid-strided), folded by XOR into one word per block so the
// loads cannot be dropped.  Measures the achievable streaming-read rate for
// comparison with the sweeps' algorithmic GB/s.
constexpr int kProbeThreads = 256;

template <int kProbeUnroll>
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t* __restrict__ src, size_t units,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_x[kProbeThreads / 64];
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < units; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int q = 0; q < kProbeUnroll; ++q) v[q] = ld_stream(src + (i + q * stride) * 16);
#pragma unroll
    for (int q = 0; q < kProbeUnroll; ++q) acc ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
  }
  for (; i < units; i += stride) {
    const u32x4 v = ld_stream(src + i * 16);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if ((threadIdx.x & 63) == 0) s_x[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) t ^= s_x[w];
    sink[blockIdx.x] = t;
  }
}

// ---------------------------------------------------------------- launchers
namespace {

// Per-device launch caches hold this many devices; a device index past it is
// served without caching.
constexpr int kMaxDevices = 64;

// Launch shapes, measured on MI355X: the gate/up sweep runs 8 waves per CU
// (one 512-thread block: its staged x and 196 VGPRs allow no more), the down
// sweep 12 (three 256-thread blocks), the read probe 16 blocks per CU with 16
// loads in flight per lane (the fastest of 4 / 8 / 16 each).
constexpr int kGateupWavesPerCU = 8;
constexpr int kDownWavesPerCU = 12;
constexpr int kProbeBlocksPerCU = 16;
constexpr int kProbeUnroll = 16;

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  return dev;
}

int cu_count() {
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

template <int R>
hipError_t route_r(const RouteParams& p, hipStream_t s, StageEvents ev) {
  return launch_k(route_kernel<R>, dim3(p.E + 1), dim3(kRouteThreads), 0, s, ev, p);
}

template <int R, int NCH, int G>
hipError_t gateup_rng(const SweepParams& p, int max_items, hipStream_t s, StageEvents ev) {
  const size_t lds = (size_t)R * NCH * kChunkUnits * 16;
  // The dynamic LDS limit is set once per device (the attribute is per device).
  static bool attr_set[kMaxDevices] = {false};
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices || !attr_set[dev]) {
    const hipError_t e = hipFuncSetAttribute((const void*)gateup_kernel<R, NCH, G>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) attr_set[dev] = true;
  }
  static int per_cu[kMaxDevices] = {0};
  constexpr int threads = kMaxSweepThreads;
  int grid = cu_count() * blocks_per_cu(gateup_kernel<R, NCH, G>, threads, lds, kGateupWavesPerCU, per_cu);
  // no more waves than work items
  if (grid * (threads / 64) > max_items) grid = (max_items * 64 + threads - 1) / threads;
  return launch_k(gateup_kernel<R, NCH, G>, dim3(grid < 1 ? 1 : grid), dim3(threads), lds, s, ev, p);
}

template <int R, int NCH>
hipError_t gateup_rn(const SweepParams& p, int max_items, hipStream_t s, StageEvents ev) {
  // top-k keys per lane: 4 covers up to 256 experts, 16 up to MOE_MAX_EXPERTS
  return p.route.E <= 256 ? gateup_rng<R, NCH, 4>(p, max_items, s, ev) : gateup_rng<R, NCH, 16>(p, max_items, s, ev);
}

template <int NCH>
hipError_t down_n(const SweepParams& p, hipStream_t s, StageEvents ev) {
  static int per_cu[kMaxDevices] = {0};
  const int grid = cu_count() * blocks_per_cu(down_kernel<NCH>, kDownThreads, 0, kDownWavesPerCU, per_cu);
  return launch_k(down_kernel<NCH>, dim3(grid), dim3(kDownThreads), 0, s, ev, p);
}

// LDS the few-row down+blend kernel needs beyond its static arrays: every
// pair's act row padded to whole 2048-column chunks, and the block's y values.
size_t down_blend_dyn_lds(int rows, int k, int nr) {
  const size_t P = (size_t)rows * k + rows;
  return P * kChunkUnits * 16 + P * (size_t)nr * sizeof(float);
}

int max_lds_per_block() {
  static int cached[kMaxDevices] = {0};
  const int dev = current_device();
  if (dev >= 0 && dev < kMaxDevices && cached[dev]) return cached[dev];
  int v = 0;
  if (dev < 0 || hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
    v = 64 * 1024;
  if (dev >= 0 && dev < kMaxDevices) cached[dev] = v;
  return v;
}

template <int R>
hipError_t down_blend_r(const SweepParams& p, int nr, hipStream_t s, StageEvents ev) {
  const size_t lds = down_blend_dyn_lds(R, p.route.k, nr);
  static size_t attr_set[kMaxDevices] = {0};  // dynamic LDS limit set so far, per device
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices || attr_set[dev] < lds) {
    const hipError_t e = hipFuncSetAttribute((const void*)down_blend_kernel<R, 1>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) attr_set[dev] = lds;
  }
  const int grid = (p.h + nr - 1) / nr;
  return launch_k(down_blend_kernel<R, 1>, dim3(grid), dim3(kDbThreads), lds, s, ev, p, nr);
}

template <int R>
hipError_t gateup_r(const SweepParams& p, int nch, int max_items, hipStream_t s, StageEvents ev) {
  switch (nch) {
    case 1: return gateup_rn<R, 1>(p, max_items, s, ev);
    case 2: return gateup_rn<R, 2>(p, max_items, s, ev);
    case 3: return gateup_rn<R, 3>(p, max_items, s, ev);
    case 4: return gateup_rn<R, 4>(p, max_items, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route(const RouteParams& p, hipStream_t s, StageEvents ev) {
  switch (p.rows) {
#define MOE_ROUTE_CASE(R) \
  case R:                 \
    return route_r<R>(p, s, ev);
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(3)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(5)
    MOE_ROUTE_CASE(6)
    MOE_ROUTE_CASE(7)
    MOE_ROUTE_CASE(8)
#undef MOE_ROUTE_CASE
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const RouteParams& p, hipStream_t s) {
  // keys per lane: 4 covers up to 256 experts, 16 up to MOE_MAX_EXPERTS
  if (p.E <= 256) return launch_k(topk_kernel<4>, dim3(1), dim3(kTopkThreads), 0, s, StageEvents{}, p);
  return launch_k(topk_kernel<16>, dim3(1), dim3(kTopkThreads), 0, s, StageEvents{}, p);
}

hipError_t launch_union(const int32_t* ids, int rows, int k, int32_t* union_ids, int32_t* union_count,
                        int32_t* slot_to_union, uint32_t* row_mask, hipStream_t s) {
  return launch_k(union_kernel, dim3(1), dim3(64), 0, s, StageEvents{}, ids, rows, k, 0, (int)MOE_MAX_EXPERTS,
                  union_ids, union_count, slot_to_union, row_mask);
}

hipError_t launch_union_local(const int32_t* ids, int rows, int k, int lo, int hi, int32_t* union_ids,
                              int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask, hipStream_t s) {
  return launch_k(union_kernel, dim3(1), dim3(64), 0, s, StageEvents{}, ids, rows, k, lo, hi, union_ids, union_count,
                  slot_to_union, row_mask);
}

hipError_t launch_gateup(const SweepParams& p, int rows, int max_slots, hipStream_t s, StageEvents ev) {
  const int nch = (p.h + kChunk - 1) / kChunk;
  const int max_items = max_slots * p.inter + p.shared_inter;  // work items (weight rows)
  switch (rows) {
    case 1: return gateup_r<1>(p, nch, max_items, s, ev);
    case 2: return gateup_r<2>(p, nch, max_items, s, ev);
    case 3: return gateup_r<3>(p, nch, max_items, s, ev);
    case 4: return gateup_r<4>(p, nch, max_items, s, ev);
    case 5: return gateup_r<5>(p, nch, max_items, s, ev);
    case 6: return gateup_r<6>(p, nch, max_items, s, ev);
    case 7: return gateup_r<7>(p, nch, max_items, s, ev);
    case 8: return gateup_r<8>(p, nch, max_items, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down(const SweepParams& p, hipStream_t s, StageEvents ev) {
  const int kmax = p.inter > p.shared_inter ? p.inter : p.shared_inter;
  switch ((kmax + kChunk - 1) / kChunk) {
    case 1: return down_n<1>(p, s, ev);
    case 2: return down_n<2>(p, s, ev);
  }
  return hipErrorInvalidValue;
}

int down_blend_rows_per_block(int rows, int k, int h, int imax) {
  if (rows < 1 || rows > kDbMaxRows || imax > kChunk) return 0;
  const int P = rows * k + rows;
  if (P * kChunkUnits > kDbActPer * kDbThreads) return 0;  // one staging pass
  // one block per CU, a whole number of batches per block
  const int per = (h + cu_count() - 1) / cu_count();
  const int nr = (per + kDownBatch - 1) / kDownBatch * kDownBatch;
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, (const void*)down_blend_kernel<kDbMaxRows, 1>) != hipSuccess) return 0;
  if (fa.sharedSizeBytes + down_blend_dyn_lds(rows, k, nr) > (size_t)max_lds_per_block()) return 0;
  return nr;
}

hipError_t launch_down_blend(const SweepParams& p, int rows, int nr, hipStream_t s, StageEvents ev) {
  switch (rows) {
    case 1: return down_blend_r<1>(p, nr, s, ev);
    case 2: return down_blend_r<2>(p, nr, s, ev);
    case 3: return down_blend_r<3>(p, nr, s, ev);
    case 4: return down_blend_r<4>(p, nr, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_blend(const float* y, const float* w, const int32_t* slot_to_union, const float* gamma,
                        uint16_t* out, float* partial, int rows, int h, int k, hipStream_t s, StageEvents ev) {
  return launch_k(blend_kernel, dim3((h + 255) / 256, rows), dim3(256), 0, s, ev, y, w, slot_to_union, gamma, out,
                  partial, h, k, rows);
}

hipError_t launch_ep_combine(const float* reduced, const float* y, const float* gamma, uint16_t* out, int rows, int h,
                             int k, hipStream_t s) {
  return launch_k(ep_combine_kernel, dim3((h + 255) / 256, rows), dim3(256), 0, s, StageEvents{}, reduced, y, gamma,
                  out, h, k, rows);
}

hipError_t launch_read_probe(const uint8_t* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
  return launch_k(read_probe_kernel<kProbeUnroll>, dim3(blocks), dim3(kProbeThreads), 0, s, StageEvents{}, src,
                  bytes / 16, sink);
}

int read_probe_blocks() { return cu_count() * kProbeBlocksPerCU; }

}  // namespace moe

static_assert(sizeof(moe::SlotInfo) == moe::kSlotInfoBytes, "SlotInfo size changed: update kSlotInfoBytes");
