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

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- router
// One wave per (router row e, 2048-column chunk c).  e == E is the shared
// expert's gate vector.  Each lane accumulates in fp64 over its columns; the
// chunk partials are summed in chunk order by the top-k kernel.
template <int R>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ router_w,
                                                     const float* __restrict__ gate_vec,
                                                     double* __restrict__ partials, int h, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int c = blockIdx.y;
  if (e > E) return;
  const float* row = (e < E) ? router_w + (size_t)e * h : gate_vec;
  double acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0;
#pragma unroll 2
  for (int it = 0; it < kChunk / 256; ++it) {
    const int col = c * kChunk + it * 256 + lane * 4;
    if (col < h) {
      const float4 wv = *reinterpret_cast<const float4*>(row + col);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)r * h + col);
        acc[r] = __builtin_fma((double)bf16_to_f32(xv.x & 0xFFFFu), (double)wv.x, acc[r]);
        acc[r] = __builtin_fma((double)bf16_to_f32(xv.x >> 16), (double)wv.y, acc[r]);
        acc[r] = __builtin_fma((double)bf16_to_f32(xv.y & 0xFFFFu), (double)wv.z, acc[r]);
        acc[r] = __builtin_fma((double)bf16_to_f32(xv.y >> 16), (double)wv.w, acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double s = wave_sum(acc[r]);
    if (lane == 0) partials[((size_t)c * kMaxRows + r) * (E + 1) + e] = s;
  }
}

// ---------------------------------------------------------------- union
// One wave deduplicates n <= 64 ids held in LDS: lane t compares its id with
// every slot (pairwise scan, no sort).  A slot is a first occurrence when no
// earlier slot holds its id; first occurrences, in slot order, form the union.
__device__ void union_wave(const int32_t* ids_lds, int n, int k, int lane, int32_t* union_ids,
                           int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask,
                           int32_t* first_out, uint32_t* mask_out) {
  const int id = lane < n ? ids_lds[lane] : -1;
  int first = lane;
  uint32_t mask = 0;
  int row = 0, col = 0;
  for (int t = 0; t < n; ++t) {
    const int v = ids_lds[t];
    const bool eq = (lane < n) && (v == id);
    if (eq && t < first) first = t;
    if (eq) mask |= 1u << row;
    if (++col == k) { col = 0; ++row; }
  }
  const bool is_first = (lane < n) && (first == lane);
  const unsigned long long bal = __ballot(is_first);
  const int pos_self = __popcll(bal & ((1ull << lane) - 1ull));
  const int pos_first = __popcll(bal & ((1ull << first) - 1ull));
  if (lane < n) slot_to_union[lane] = pos_first;
  if (is_first) {
    union_ids[pos_self] = id;
    if (row_mask) row_mask[pos_self] = mask;
  }
  if (lane == 0) *union_count = __popcll(bal);
  *first_out = is_first ? pos_self : -1;
  *mask_out = mask;
}

__global__ __launch_bounds__(64) void union_kernel(const int32_t* __restrict__ ids, int n, int k,
                                                   int32_t* union_ids, int32_t* union_count,
                                                   int32_t* slot_to_union, uint32_t* row_mask) {
  __shared__ int32_t s_ids[kMaxIds];
  const int lane = threadIdx.x;
  if (lane < n) s_ids[lane] = ids[lane];
  __syncthreads();
  int pos;
  uint32_t mask;
  union_wave(s_ids, n, k, lane, union_ids, union_count, slot_to_union, row_mask, &pos, &mask);
}

// ---------------------------------------------------------------- top-k
// One wave per row: logits (fp32 rounding of the fp64 sum over chunks),
// selection keys, k rounds of wave argmax (ties to the lower id), weights in
// fp64.  With UNION, wave 0 then builds the union and resolves each union
// slot's weight pointers for the sweeps.
constexpr int kKeysPerLane = MOE_MAX_EXPERTS / 64;

template <bool UNION>
__global__ __launch_bounds__(512) void topk_kernel(TopkParams p) {
  __shared__ int32_t s_ids[kMaxIds];
  const int lane = threadIdx.x & 63;
  const int r = threadIdx.x >> 6;
  const int E = p.E, k = p.k;
  if (r < p.rows) {
    float kv[kKeysPerLane];
    float lv[kKeysPerLane];
    int selj[kKeysPerLane];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
      const int e = lane + 64 * i;
      kv[i] = -__builtin_huge_valf();
      lv[i] = 0.f;
      selj[i] = -1;
      if (e < E) {
        double L = 0.0;
        for (int c = 0; c < p.nkc; ++c) L += p.partials[((size_t)c * kMaxRows + r) * (E + 1) + e];
        const float L32 = (float)L;
        p.logits[r * E + e] = L32;
        lv[i] = L32;
        if (p.route_kind == MOE_ROUTE_SOFTMAX) {
          kv[i] = L32;
        } else {
          const float s32 = (float)(1.0 / (1.0 + exp(-(double)L32)));
          kv[i] = s32 + p.bias[e];
        }
      }
    }
    if (lane == 0) {
      double z = 0.0;
      for (int c = 0; c < p.nkc; ++c) z += p.partials[((size_t)c * kMaxRows + r) * (E + 1) + E];
      p.gamma[r] = (float)(1.0 / (1.0 + exp(-z)));
    }
    float top_logit = 0.f;
    for (int j = 0; j < k; ++j) {
      float bk = -__builtin_huge_valf();
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < kKeysPerLane; ++i) {
        const int e = lane + 64 * i;
        if (e < E && selj[i] < 0 && kv[i] > bk) {
          bk = kv[i];
          be = e;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ok = __shfl_xor(bk, o);
        const int oe = __shfl_xor(be, o);
        if (ok > bk || (ok == bk && oe < be)) {
          bk = ok;
          be = oe;
        }
      }
      // NaN keys (outside the contract) can leave no winner; keep the id in
      // range so no later stage indexes the weight tables out of bounds.
      if (be >= E) be = 0;
      if ((be & 63) == lane) {
#pragma unroll
        for (int i = 0; i < kKeysPerLane; ++i)
          if (i == (be >> 6)) selj[i] = j;
      }
      if (j == 0) top_logit = bk;  // softmax: the largest logit
      if (lane == 0) {
        p.ids_out[r * k + j] = be;
        s_ids[r * k + j] = be;
      }
    }
    // Weights.  Softmax: exp(L - max) normalised over all experts, or over the
    // k selected when norm_topk_prob.  Sigmoid: s, optionally normalised over
    // the selected, times routed_scaling_factor.
    double num[kKeysPerLane];
    double all_part = 0.0, sel_part = 0.0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
      const int e = lane + 64 * i;
      num[i] = 0.0;
      if (e < E) {
        double v;
        if (p.route_kind == MOE_ROUTE_SOFTMAX)
          v = exp((double)lv[i] - (double)top_logit);
        else
          v = 1.0 / (1.0 + exp(-(double)lv[i]));
        num[i] = v;
        all_part += v;
        if (selj[i] >= 0) sel_part += v;
      }
    }
    const double all_sum = wave_sum(all_part);
    const double sel_sum = wave_sum(sel_part);
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
      if (selj[i] >= 0) {
        double wgt;
        if (p.route_kind == MOE_ROUTE_SOFTMAX) {
          wgt = p.norm ? num[i] / sel_sum : num[i] / all_sum;
        } else {
          wgt = p.norm ? num[i] / sel_sum : num[i];
          wgt *= (double)p.rsf;
        }
        p.w_out[r * k + selj[i]] = (float)wgt;
      }
    }
  }
  if constexpr (UNION) {
    __syncthreads();
    if (threadIdx.x < 64) {
      int pos;
      uint32_t mask;
      union_wave(s_ids, p.rows * k, k, lane, p.union_ids, p.union_count, p.slot_to_union, p.row_mask,
                 &pos, &mask);
      if (pos >= 0) {
        const int e = s_ids[lane];
        SlotInfo si;
        si.gate_packed = p.gate.packed[e];
        si.gate_scales = p.gate.scales[e];
        si.up_packed = p.up.packed[e];
        si.up_scales = p.up.scales[e];
        si.down_packed = p.down.packed[e];
        si.down_scales = p.down.scales[e];
        si.gate_scale2 = p.gate.scale2[e];
        si.up_scale2 = p.up.scale2[e];
        si.down_scale2 = p.down.scale2[e];
        si.inter = p.inter;
        si.row_mask = mask;
        si.expert = e;
        p.slots[pos] = si;
      }
      if (lane == 0) {
        SlotInfo si;
        si.gate_packed = p.shared_gate.packed;
        si.gate_scales = p.shared_gate.scales;
        si.up_packed = p.shared_up.packed;
        si.up_scales = p.shared_up.scales;
        si.down_packed = p.shared_down.packed;
        si.down_scales = p.shared_down.scales;
        si.gate_scale2 = p.shared_gate.scale2;
        si.up_scale2 = p.shared_up.scale2;
        si.down_scale2 = p.shared_down.scale2;
        si.inter = p.shared_inter;
        si.row_mask = (1u << p.rows) - 1u;
        si.expert = -1;
        p.slots[kSharedSlot] = si;
      }
    }
  }
}

// ---------------------------------------------------------------- sweeps
// Stage R rows of a bf16 [R][cols] matrix (row stride `stride` elements) into
// LDS as NCH chunks of 256 swizzled 16-byte units, zero beyond `cols`.  Only
// rows in `mask` are staged.
template <int R, int NCH>
__device__ __forceinline__ void stage_rows(u32x4* dst, const uint16_t* src, size_t stride, int cols,
                                           uint32_t mask) {
  for (int i = threadIdx.x; i < R * NCH * kChunkUnits; i += blockDim.x) {
    const int r = i / (NCH * kChunkUnits);
    if (!((mask >> r) & 1u)) continue;
    const int rem = i - r * NCH * kChunkUnits;
    const int c = rem / kChunkUnits;
    const int un = rem - c * kChunkUnits;
    const int col = c * kChunk + un * 8;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < cols) v = *reinterpret_cast<const u32x4*>(src + (size_t)r * stride + col);
    dst[(r * NCH + c) * kChunkUnits + swz_unit(un)] = v;
  }
}

constexpr int kSweepThreads = 512;
constexpr int kSweepWaves = kSweepThreads / 64;
constexpr int kGateUpRowsPerWave = 2;
constexpr int kGateUpTile = kSweepWaves * kGateUpRowsPerWave;  // gate/up rows per tile
constexpr int kDownRowsPerWave = 8;
constexpr int kDownTile = kSweepWaves * kDownRowsPerWave;      // output rows per tile

// Gate+up sweep.  A tile is kGateUpTile consecutive rows n of one union
// slot's gate and up matrices; each wave takes kGateUpRowsPerWave of them.
// For each row n and each row r that uses the slot:
//   act[slot][r][n] = bf16(silu(g) * v), g = W_gate[n,:] . x_r, v = W_up[n,:] . x_r.
template <int R, int NCH>
__global__ __launch_bounds__(kSweepThreads) void gateup_kernel(SweepParams p) {
  extern __shared__ u32x4 xs[];  // [R][NCH][256] staged x rows
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = p.h;
  stage_rows<R, NCH>(xs, p.x, (size_t)h, h, (1u << R) - 1u);
  __syncthreads();

  const int U = *p.union_count;
  const int tpe_r = (p.inter + kGateUpTile - 1) / kGateUpTile;
  const int tpe_s = (p.shared_inter + kGateUpTile - 1) / kGateUpTile;
  const int ntiles = U * tpe_r + tpe_s;
  const size_t code_stride = (size_t)h >> 1;
  const size_t scale_stride = (size_t)h >> 4;

  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    int slot, nb;
    if (t < U * tpe_r) {
      slot = t / tpe_r;
      nb = t - slot * tpe_r;
    } else {
      slot = kSharedSlot;
      nb = t - U * tpe_r;
    }
    const SlotInfo si = p.slots[slot];
    const int n0 = nb * kGateUpTile + wave * kGateUpRowsPerWave;

    // Issue every load of this wave's rows before any arithmetic.
    u32x4 gq[kGateUpRowsPerWave][NCH], uq[kGateUpRowsPerWave][NCH];
    uint32_t gsc[kGateUpRowsPerWave][NCH], usc[kGateUpRowsPerWave][NCH];
#pragma unroll
    for (int i = 0; i < kGateUpRowsPerWave; ++i) {
      const int n = n0 + i;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int col = c * kChunk + lane * 32;
        gq[i][c] = u32x4{0u, 0u, 0u, 0u};
        uq[i][c] = u32x4{0u, 0u, 0u, 0u};
        gsc[i][c] = 0u;
        usc[i][c] = 0u;
        if (n < si.inter && col < h) {
          const size_t co = (size_t)n * code_stride + (col >> 1);
          const size_t so = (size_t)n * scale_stride + (col >> 4);
          gq[i][c] = *reinterpret_cast<const u32x4*>(si.gate_packed + co);
          uq[i][c] = *reinterpret_cast<const u32x4*>(si.up_packed + co);
          gsc[i][c] = *reinterpret_cast<const uint16_t*>(si.gate_scales + so);
          usc[i][c] = *reinterpret_cast<const uint16_t*>(si.up_scales + so);
        }
      }
    }

#pragma unroll
    for (int i = 0; i < kGateUpRowsPerWave; ++i) {
      const int n = n0 + i;
      if (n >= si.inter) break;
      float ag[R], au[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        ag[r] = 0.f;
        au[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int col = c * kChunk + lane * 32;
        if (col < h) {
          bf16x2 gw[16], uw[16];
          decode32(gq[i][c], gw);
          decode32(uq[i][c], uw);
          const float gs0 = e4m3<0>(gsc[i][c]), gs1 = e4m3<1>(gsc[i][c]);
          const float us0 = e4m3<0>(usc[i][c]), us1 = e4m3<1>(usc[i][c]);
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
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if ((si.row_mask >> r) & 1u) {
          const float g = wave_sum(ag[r]) * si.gate_scale2;
          const float v = wave_sum(au[r]) * si.up_scale2;
          if (lane == 0) {
            const float a = g / (1.0f + __expf(-g)) * v;
            p.act[((size_t)slot * kMaxRows + r) * p.act_stride + n] = f32_to_bf16(a);
          }
        }
      }
    }
  }
}

// Down sweep.  A tile is kDownTile consecutive output rows n of one union
// slot's down matrix [h, inter]; the slot's act rows are staged in LDS.
//   y[slot][r][n] = W_down[n,:] . act[slot][r][:]
template <int R, int NCH>
__global__ __launch_bounds__(kSweepThreads) void down_kernel(SweepParams p) {
  extern __shared__ u32x4 as_[];  // [R][NCH][256] staged act rows
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = p.h;
  const int U = *p.union_count;
  const int tpe = (h + kDownTile - 1) / kDownTile;
  const int ntiles = (U + 1) * tpe;

  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int su = t / tpe;
    const int nb = t - su * tpe;
    const int slot = su < U ? su : kSharedSlot;
    const SlotInfo si = p.slots[slot];
    const int K = si.inter;
    __syncthreads();  // the previous tile's LDS reads are done
    stage_rows<R, NCH>(as_, p.act + (size_t)slot * kMaxRows * p.act_stride, (size_t)p.act_stride, K,
                       si.row_mask);
    __syncthreads();

    const size_t code_stride = (size_t)K >> 1;
    const size_t scale_stride = (size_t)K >> 4;
    const int n0 = nb * kDownTile + wave * kDownRowsPerWave;
    u32x4 dq[kDownRowsPerWave][NCH];
    uint32_t dsc[kDownRowsPerWave][NCH];
#pragma unroll
    for (int i = 0; i < kDownRowsPerWave; ++i) {
      const int n = n0 + i;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int col = c * kChunk + lane * 32;
        dq[i][c] = u32x4{0u, 0u, 0u, 0u};
        dsc[i][c] = 0u;
        if (n < h && col < K) {
          dq[i][c] = *reinterpret_cast<const u32x4*>(si.down_packed + (size_t)n * code_stride + (col >> 1));
          dsc[i][c] = *reinterpret_cast<const uint16_t*>(si.down_scales + (size_t)n * scale_stride + (col >> 4));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kDownRowsPerWave; ++i) {
      const int n = n0 + i;
      if (n >= h) break;
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int col = c * kChunk + lane * 32;
        if (col < K) {
          bf16x2 dw[16];
          decode32(dq[i][c], dw);
          const float s0 = e4m3<0>(dsc[i][c]), s1 = e4m3<1>(dsc[i][c]);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            if ((si.row_mask >> r) & 1u) {
              const u32x4* ar = as_ + (r * NCH + c) * kChunkUnits;
              acc[r] = dot32(dw, ar[lane], ar[64 + lane], ar[128 + lane], ar[192 + lane], s0, s1, acc[r]);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if ((si.row_mask >> r) & 1u) {
          const float yv = wave_sum(acc[r]) * si.down_scale2;
          if (lane == 0) p.y[((size_t)slot * kMaxRows + r) * h + n] = yv;
        }
      }
    }
  }
}

// Weighted sum and shared-expert blend, one thread per (row, column):
//   out[r][n] = bf16( sum_{j<k} w[r][j] * y[slot(r,j)][r][n] + gamma[r] * y[shared][r][n] )
// summed in fp32 in ascending j.
__global__ __launch_bounds__(256) void blend_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                    const int32_t* __restrict__ slot_to_union,
                                                    const float* __restrict__ gamma, uint16_t* __restrict__ out,
                                                    int h, int k) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= h) return;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int s = slot_to_union[r * k + j];
    acc = __builtin_fmaf(w[r * k + j], y[((size_t)s * kMaxRows + r) * h + n], acc);
  }
  acc = __builtin_fmaf(gamma[r], y[((size_t)kSharedSlot * kMaxRows + r) * h + n], acc);
  out[(size_t)r * h + n] = f32_to_bf16(acc);
}

// ---------------------------------------------------------------- launchers
namespace {

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Persistent grid: every CU holds as many blocks as occupancy allows (queried
// once per kernel instance), capped by the largest possible tile count.
template <typename K>
int sweep_grid(K kernel, size_t lds, int max_tiles, int& per_cu_cache) {
  if (per_cu_cache <= 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kSweepThreads, lds) != hipSuccess ||
        per_cu <= 0)
      per_cu = 1;
    per_cu_cache = per_cu;
  }
  int grid = cu_count() * per_cu_cache;
  if (grid > max_tiles) grid = max_tiles;
  return grid < 1 ? 1 : grid;
}

template <int R>
hipError_t router_r(const uint16_t* x, const float* rw, const float* gv, double* partials, int h, int E,
                    hipStream_t s) {
  const int nkc = (h + kChunk - 1) / kChunk;
  dim3 grid((E + 1 + 3) / 4, nkc);
  hipLaunchKernelGGL((router_kernel<R>), grid, dim3(256), 0, s, x, rw, gv, partials, h, E);
  return hipGetLastError();
}

template <int R, int NCH>
hipError_t gateup_rn(const SweepParams& p, int max_tiles, hipStream_t s) {
  const size_t lds = (size_t)R * NCH * kChunkUnits * 16;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)gateup_kernel<R, NCH>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  static int per_cu = 0;
  const int grid = sweep_grid(gateup_kernel<R, NCH>, lds, max_tiles, per_cu);
  hipLaunchKernelGGL((gateup_kernel<R, NCH>), dim3(grid), dim3(kSweepThreads), lds, s, p);
  return hipGetLastError();
}

template <int R, int NCH>
hipError_t down_rn(const SweepParams& p, int max_tiles, hipStream_t s) {
  const size_t lds = (size_t)R * NCH * kChunkUnits * 16;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)down_kernel<R, NCH>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  static int per_cu = 0;
  const int grid = sweep_grid(down_kernel<R, NCH>, lds, max_tiles, per_cu);
  hipLaunchKernelGGL((down_kernel<R, NCH>), dim3(grid), dim3(kSweepThreads), lds, s, p);
  return hipGetLastError();
}

template <int R>
hipError_t gateup_r(const SweepParams& p, int nch, int max_tiles, hipStream_t s) {
  switch (nch) {
    case 1: return gateup_rn<R, 1>(p, max_tiles, s);
    case 2: return gateup_rn<R, 2>(p, max_tiles, s);
    case 3: return gateup_rn<R, 3>(p, max_tiles, s);
    case 4: return gateup_rn<R, 4>(p, max_tiles, s);
  }
  return hipErrorInvalidValue;
}

template <int R>
hipError_t down_r(const SweepParams& p, int nch, int max_tiles, hipStream_t s) {
  switch (nch) {
    case 1: return down_rn<R, 1>(p, max_tiles, s);
    case 2: return down_rn<R, 2>(p, max_tiles, s);
    case 3: return down_rn<R, 3>(p, max_tiles, s);
    case 4: return down_rn<R, 4>(p, max_tiles, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const float* router_w, const float* gate_vec, double* partials,
                         int rows, int h, int E, hipStream_t s) {
  switch (rows) {
    case 1: return router_r<1>(x, router_w, gate_vec, partials, h, E, s);
    case 2: return router_r<2>(x, router_w, gate_vec, partials, h, E, s);
    case 3: return router_r<3>(x, router_w, gate_vec, partials, h, E, s);
    case 4: return router_r<4>(x, router_w, gate_vec, partials, h, E, s);
    case 5: return router_r<5>(x, router_w, gate_vec, partials, h, E, s);
    case 6: return router_r<6>(x, router_w, gate_vec, partials, h, E, s);
    case 7: return router_r<7>(x, router_w, gate_vec, partials, h, E, s);
    case 8: return router_r<8>(x, router_w, gate_vec, partials, h, E, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const TopkParams& p, bool with_union, hipStream_t s) {
  if (with_union)
    hipLaunchKernelGGL((topk_kernel<true>), dim3(1), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((topk_kernel<false>), dim3(1), dim3(512), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_union(const int32_t* ids, int rows, int k, int32_t* union_ids, int32_t* union_count,
                        int32_t* slot_to_union, uint32_t* row_mask, hipStream_t s) {
  hipLaunchKernelGGL(union_kernel, dim3(1), dim3(64), 0, s, ids, rows * k, k, union_ids, union_count,
                     slot_to_union, row_mask);
  return hipGetLastError();
}

hipError_t launch_gateup(const SweepParams& p, int rows, int max_union, hipStream_t s) {
  const int nch = (p.h + kChunk - 1) / kChunk;
  const int tpe_r = (p.inter + kGateUpTile - 1) / kGateUpTile;
  const int tpe_s = (p.shared_inter + kGateUpTile - 1) / kGateUpTile;
  const int max_tiles = max_union * tpe_r + tpe_s;
  switch (rows) {
    case 1: return gateup_r<1>(p, nch, max_tiles, s);
    case 2: return gateup_r<2>(p, nch, max_tiles, s);
    case 3: return gateup_r<3>(p, nch, max_tiles, s);
    case 4: return gateup_r<4>(p, nch, max_tiles, s);
    case 5: return gateup_r<5>(p, nch, max_tiles, s);
    case 6: return gateup_r<6>(p, nch, max_tiles, s);
    case 7: return gateup_r<7>(p, nch, max_tiles, s);
    case 8: return gateup_r<8>(p, nch, max_tiles, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down(const SweepParams& p, int rows, int max_union, hipStream_t s) {
  const int kmax = p.inter > p.shared_inter ? p.inter : p.shared_inter;
  const int nch = (kmax + kChunk - 1) / kChunk;
  const int tpe = (p.h + kDownTile - 1) / kDownTile;
  const int max_tiles = (max_union + 1) * tpe;
  switch (rows) {
    case 1: return down_r<1>(p, nch, max_tiles, s);
    case 2: return down_r<2>(p, nch, max_tiles, s);
    case 3: return down_r<3>(p, nch, max_tiles, s);
    case 4: return down_r<4>(p, nch, max_tiles, s);
    case 5: return down_r<5>(p, nch, max_tiles, s);
    case 6: return down_r<6>(p, nch, max_tiles, s);
    case 7: return down_r<7>(p, nch, max_tiles, s);
    case 8: return down_r<8>(p, nch, max_tiles, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_blend(const float* y, const float* w, const int32_t* slot_to_union, const float* gamma,
                        uint16_t* out, int rows, int h, int k, hipStream_t s) {
  dim3 grid((h + 255) / 256, rows);
  hipLaunchKernelGGL(blend_kernel, grid, dim3(256), 0, s, y, w, slot_to_union, gamma, out, h, k);
  return hipGetLastError();
}

}  // namespace moe

static_assert(sizeof(moe::SlotInfo) == moe::kSlotInfoBytes, "SlotInfo size changed: update kSlotInfoBytes");
