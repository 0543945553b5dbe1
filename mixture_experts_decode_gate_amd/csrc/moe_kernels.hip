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

#include "moe_common.h"

namespace moe {

__global__ __launch_bounds__(64) void union_kernel(const int32_t* __restrict__ ids, int rows, int k, int lo, int hi,
                                                   int32_t* union_ids, int32_t* union_count,
                                                   int32_t* slot_to_union, uint32_t* row_mask) {
  __shared__ __align__(16) int32_t s_ids[kMaxIds];
  const int lane = threadIdx.x;
  const int n = rows * k;
  s_ids[lane] = lane < n ? ids[lane] : -1;
  s_ids[64 + lane] = 64 + lane < n ? ids[64 + lane] : -1;
  __syncthreads();
  UnionLane ul;
  union_wave(s_ids, n, k, rows, lo, hi, lane, union_ids, union_count, slot_to_union, row_mask, ul);
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
  // part[c][r][q]: chunk c's partial for row r over the quad of lanes 4q..4q+3
  __shared__ double part[kMaxRouterChunks][R][16];
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
    quad_sum_n<R>(acc);
    if ((lane & 3) == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) part[c][r][lane >> 2] = acc[r];
    }
  }
  __syncthreads();
  // Thread 16r + q finishes quad q of row r: its chunk partials summed in
  // chunk order, then the row's 16 quads reduced across its DPP row (row r
  // sits on lanes 16(r % 4) .. +15 of wave r / 4).  The row's first lane
  // takes the sigmoid (the gate row always; router rows for sigmoid routing)
  // and writes the row's results; the kernel that follows reads them after
  // the kernel boundary.
  if ((int)threadIdx.x < 16 * R) {
    const int r = (int)threadIdx.x >> 4, q = (int)threadIdx.x & 15;
    double v[kMaxRouterChunks];
#pragma unroll
    for (int cc = 0; cc < kMaxRouterChunks; ++cc) v[cc] = part[cc < nkc ? cc : 0][r][q];
    double z = v[0];
#pragma unroll
    for (int cc = 1; cc < kMaxRouterChunks; ++cc)
      if (cc < nkc) z += v[cc];
    z = row16_sum(z);
    if (q == 0) {
      if (p.router_fp4 && e < E) z *= (double)p.router_scale2;
      // The gate takes the fp64 sum; routing scores take the fp32 logit, the
      // value top-k sees.
      if (e < E) {
        p.logits[r * E + e] = (float)z;
        p.score[r * E + e] = p.route_kind == MOE_ROUTE_SIGMOID_BIAS ? 1.0 / (1.0 + exp(-(double)(float)z)) : 0.0;
      } else {
        p.gamma[r] = p.ungated ? 1.0f : (float)(1.0 / (1.0 + exp(-z)));
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

// Down sweep.  The work is one "segment" per union slot (and one for the
// shared expert): the slot's down matrix times the act rows of every row that
// uses it.  A wave holds up to kGroup act rows in registers (loaded once per
// segment), so a slot used by more rows is swept by several row groups side
// by side (see the wave mapping below).  Each wave loads its next batches of
// weight rows while it computes the current one.  For row r of union slot u,
// with pair t the (row, expert) pair of (u, r):
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
  constexpr int kGroup = down_group(NCH);  // act rows a wave holds (the segment table's group size)
  constexpr int kMaxSegs = kMaxDownSegs;
  static_assert(kMaxSegs < 256, "the segment search spans at most 255 segments");
  __shared__ SlotInfo s_slots[kNumSlots];
  __shared__ int s_seg_slot[kMaxSegs];
  __shared__ uint32_t s_seg_rows[kMaxSegs];  // row mask in bits 0..15, row groups in bits 16..23
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

  // Each segment (a slot) gets waves in proportion to its work weight
  // (kSegCostBase + rows per weight row and group of rows: a two-row group
  // costs more arithmetic per byte): with cumulative weights c_s and total C,
  // virtual wave v of V works on the segment s with c_s <= v * C / V <
  // c_{s+1}.  Within a segment of G row groups, consecutive virtual waves take
  // groups 0, 1, .., G-1 of the same batch: the waves that read a weight row
  // for the slot's different row groups sit side by side (the shared slot
  // comes first and starts at wave 0, so its groups share a block) and the
  // repeated reads are served by the cache.  Each group's waves take
  // interleaved batches of kDownBatch rows: every group sweeps its matrix
  // front to back together.  V >= C gives every segment at least 4 G virtual
  // waves (a segment weighs at least 4 per group); with fewer waves than that
  // a wave takes several virtual waves in turn.
  const int W = gridDim.x * nwaves;
  const int nseg = s_nseg;
  const int C = s_seg_cum[nseg];
  const int V = W > C ? W : C;

  // Numbering the blocks XCD by XCD gives each XCD (and its L2) a contiguous
  // run of virtual waves, so the row groups of one slot and the readers of one
  // act row mostly share an L2.
  const int lb = xcd_major_block();

  DownBatch<NCH> buf[kDownBufs];
  u32x4 act[kGroup][NCH][4];
  for (int v = lb * nwaves + wave; v < V; v += W) {
    const long long key = (long long)v * C / V;  // in [0, C)
    int seg = 0;
    for (int span = 128; span > 0; span >>= 1)  // largest s with c_s <= key (nseg <= kMaxSegs)
      if (seg + span < nseg && s_seg_cum[seg + span] <= key) seg += span;
    seg = uniform_int(seg);
    const long long c0 = s_seg_cum[seg], c1 = s_seg_cum[seg + 1];
    const int first = (int)(((long long)V * c0 + C - 1) / C);  // first virtual wave of the segment
    const int last = (int)(((long long)V * c1 + C - 1) / C);
    const int n_end = h;
    const int slot = uniform_int(s_seg_slot[seg]);
    const uint32_t segw = uniform_u32(s_seg_rows[seg]);
    const uint32_t mask = segw & 0xFFFFu;
    const int ngroups = (int)(segw >> 16);
    const int vi = v - first, nvs = last - first;
    // Every row group gets the same number of waves, so that the i-th waves
    // of all groups read the same batches; the at most ngroups - 1 virtual
    // waves left over stay idle.
    const int wg = nvs / ngroups;  // >= 1: the segment weighs at least 4 per group
    if (vi >= wg * ngroups) continue;
    const int grp = vi % ngroups;  // this wave's row group
    const SlotInfo& si = s_slots[slot];
    const int K = uniform_int(si.inter);
    const uint8_t* const d_packed = uniform_ptr(si.down_packed);
    const uint8_t* const d_scales = uniform_ptr(si.down_scales);
    const float d2 = uniform_f32(si.down_scale2);
    const int stride = wg * kDownBatch;
    const int n0 = (vi / ngroups) * kDownBatch;
    if (n0 >= n_end) continue;
    // The group's rows: the (kGroup * grp)-th and following rows of the mask;
    // their pair indices (unused entries repeat the last row).
    int grow[kGroup], cnt = 0;
    for (int r = 0; r < kMaxRows; ++r) {
      if ((mask >> r) & 1u) {
        const int idx = __popc(mask & ((1u << r) - 1u)) - kGroup * grp;
        if (idx >= 0 && idx < kGroup) {
          grow[idx] = r;
          ++cnt;
        }
      }
    }
    cnt = uniform_int(cnt);
    int prs[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) prs[i] = uniform_int(si.pair[grow[i < cnt ? i : cnt - 1]]);
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
          const float t = wave_sum4_scatter(acc[g], lane);
          const int j = sum4_value(lane);
          if (lane < kDownBatch && nb + j < n_end) p.y[(size_t)prs[g] * h + nb + j] = t * d2;
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
// single kernel runs the down projections and the weighted sum.  The block
// with XCD-major index v (xcd_major_block) owns output rows [v*nr, (v+1)*nr)
// of every union slot and of the shared expert, so every term of out[r][n]
// is computed inside the block: the blend needs no
// kernel of its own and the expert outputs no round trip through memory.
//   y[t][n]   = W_down[u][n,:] . act[t][:]        (t: the pair of slot u and row r)
//   out[r][n] = bf16( sum_{j<k} w[r][j] * y[r*k + j][n] + gamma[r] * y[rows*k + r][n] )
// Each y value is computed exactly as down_kernel computes it (same lane
// columns, same chunk order, same reduction, scale2 last) and the sum runs in
// blend_kernel's order, so both paths write the same bytes; y is also written
// to the workspace.  Work units are (slot, batch of kDownBatch output rows),
// the shared expert's first; the block's waves claim them from an LDS counter
// and keep two units in flight while they compute one.  It serves one or two
// rows: with more, the registers of 12 waves per CU no longer hold two rows'
// activations beside three weight batches, and the down sweep + blend kernels
// take over.
constexpr int kDbThreads = 768;  // 12 waves, one block per CU
constexpr int kDbMaxRows = 2;    // rows served by this kernel (act of every pair in LDS)
constexpr int kDbActPer = 12;    // act staging loads per thread (16 bytes each), at most

// A: act staging loads per thread, enough for every pair of this call (the
// loads are unconditional, so fewer of them when fewer pairs need staging).
template <int R, int NCH, int A>
__global__ __launch_bounds__(kDbThreads) void down_blend_kernel(SweepParams p, int nr) {
  static_assert(A <= kDbActPer, "at most kDbActPer act staging loads per thread");
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
  const int n_begin = xcd_major_block() * nr;
  const int nbat = nr / kDownBatch;

  // Prologue, in two steps so the first weight loads go out early: (1) the
  // slot table, U, routing weights and gates and every act row, then a
  // shared-expert unit's weights (their pointers are this kernel's
  // arguments); (2) once the slot table is in LDS, the first routed unit's
  // weights.  Loads are consumed in issue order.
  const int units = P * NCH * kChunkUnits;
  // Unit i of the act staging is 16 bytes of pair t, chunk c, unit un
  // (columns past the pair's K read a valid copy and are stored as zeros).
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
  auto act_issue = [&](u32x4* av, int base, int n) {
#pragma unroll
    for (int q = 0; q < n; ++q) {
      const int i = base + (int)threadIdx.x + q * kDbThreads;
      int dst;
      bool valid;
      av[q] = ld_global(act_src(i < units ? i : 0, dst, valid));
    }
  };
  auto act_store = [&](const u32x4* av, int base, int n) {
#pragma unroll
    for (int q = 0; q < n; ++q) {
      const int i = base + (int)threadIdx.x + q * kDbThreads;
      if (i < units) {
        int dst;
        bool valid;
        act_src(i, dst, valid);
        s_act[dst] = valid ? av[q] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int q = 0; q < n; ++q) asm volatile("" ::"v"(av[q]));
  };
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
  u32x4 av_first[A];
  act_issue(av_first, 0, A);
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
  // output rows n_begin + (id % nbat) * kDownBatch + 0..3.  id -1 is the
  // stand-in loaded where there is no unit: rows 0..3 of the shared expert,
  // the same address in every wave, so it is served from the cache.
  auto fetch = [&](int id, DownBatch<NCH>& b, UnitInfo& ui) {
    const int sidx = id < 0 ? 0 : id / nbat;
    const int slot = sidx == 0 ? kSharedSlot : sidx - 1;
    const int n = id < 0 ? 0 : n_begin + (id - sidx * nbat) * kDownBatch;
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
  // when it is one; otherwise the stand-in (loaded, not computed).
  const int first = claim_id();
  const bool early = first < nbat;
  DownBatch<NCH> ba, bb, bc;
  UnitInfo ia, ib, ic;
  fetch(early ? first : -1, ba, ia);
  __builtin_amdgcn_sched_barrier(0);

  // Consume, in issue order: the slot table, U, weights and gates.
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
    for (int q = 0; q < kTabPer; ++q) asm volatile("" ::"v"(tab[q]));
    act_store(av_first, 0, A);
  }
  __syncthreads();
  const int total = (s_union + 1) * nbat;
  auto claim = [&]() -> int {
    const int id = claim_id();
    return id < total ? id : -1;
  };
  int id_a, id_b;
  if (early) {
    id_a = first;  // < nbat <= total
    id_b = claim();
  } else {
    id_a = -1;
    id_b = first < total ? first : -1;
  }
  fetch(id_b, bb, ib);

  // The unit's one or two rows (act rows from LDS), each weight row decoded
  // once; y to LDS and the workspace.
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
        const float t = wave_sum4_scatter(acc, lane);
        const int j = sum4_value(lane);
        if (lane < kDownBatch) {
          const float yv = t * ui.d2;
          if (ui.n + j < h) p.y[(size_t)pr * h + ui.n + j] = yv;
          s_y[pr * nr + (ui.n - n_begin) + j] = yv;
        }
      };
      if (u0) emit(acc0, p0);
      // the two rows' sums one after the other: fewer registers live at once
      __builtin_amdgcn_sched_barrier(0);
      if (u1) emit(acc1, p1);
      // the next group's act rows are read from LDS after this group is done
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (id_a >= 0 || id_b >= 0) {
    // One exit, after a whole rotation (see the gate/up sweep).
    while (true) {
      const int id_c = id_b >= 0 ? claim() : -1;
      fetch(id_c, bc, ic);
#pragma unroll
      for (int q = 0; q < kDownBatch; ++q) consume<NCH>(ba.row[q]);
      if (id_a >= 0) compute(ba, ia);
      const int id_a2 = id_c >= 0 ? claim() : -1;
      fetch(id_a2, ba, ia);
#pragma unroll
      for (int q = 0; q < kDownBatch; ++q) consume<NCH>(bb.row[q]);
      if (id_b >= 0) compute(bb, ib);
      const int id_b2 = id_a2 >= 0 ? claim() : -1;
      fetch(id_b2, bb, ib);
#pragma unroll
      for (int q = 0; q < kDownBatch; ++q) consume<NCH>(bc.row[q]);
      if (id_c >= 0) compute(bc, ic);
      if (id_a2 < 0) break;
      id_a = id_a2;
      id_b = id_b2;
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

template <int R>
hipError_t route_r(const RouteParams& p, hipStream_t s, StageEvents ev) {
  return launch_k(route_kernel<R>, dim3(p.E + 1), dim3(kRouteThreads), 0, s, ev, p);
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

template <int R, int A>
hipError_t down_blend_ra(const SweepParams& p, int nr, hipStream_t s, StageEvents ev) {
  const size_t lds = down_blend_dyn_lds(R, p.route.k, nr);
  static size_t attr_set[kMaxDevices] = {0};  // dynamic LDS limit set so far, per device
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices || attr_set[dev] < lds) {
    const hipError_t e = hipFuncSetAttribute((const void*)down_blend_kernel<R, 1, A>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) attr_set[dev] = lds;
  }
  const int grid = (p.h + nr - 1) / nr;
  return launch_k(down_blend_kernel<R, 1, A>, dim3(grid), dim3(kDbThreads), lds, s, ev, p, nr);
}

// 3 R staging loads per thread cover R (k + 1) pairs for k <= 8; larger k
// takes kDbActPer.
template <int R>
hipError_t down_blend_r(const SweepParams& p, int nr, hipStream_t s, StageEvents ev) {
  constexpr int kFew = 3 * R;
  const int pairs = R * p.route.k + R;
  if (pairs * kChunkUnits <= kFew * kDbThreads) return down_blend_ra<R, kFew>(p, nr, s, ev);
  return down_blend_ra<R, kDbActPer>(p, nr, s, ev);
}

}  // namespace

#define MOE_ROWS_CASES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
static_assert(kMaxRows == 16, "MOE_ROWS_CASES lists every row count");

hipError_t launch_route(const RouteParams& p, hipStream_t s, StageEvents ev) {
  switch (p.rows) {
#define MOE_ROUTE_CASE(R) \
  case R:                 \
    return route_r<R>(p, s, ev);
    MOE_ROWS_CASES(MOE_ROUTE_CASE)
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
  if (rows >= 1 && rows <= 4) return launch_gateup_rows_1_4(p, rows, nch, max_items, s, ev);
  if (rows >= 5 && rows <= 8) return launch_gateup_rows_5_8(p, rows, nch, max_items, s, ev);
  if (rows >= 9 && rows <= 12) return launch_gateup_rows_9_12(p, rows, nch, max_items, s, ev);
  if (rows >= 13 && rows <= 16) return launch_gateup_rows_13_16(p, rows, nch, max_items, s, ev);
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
  if (hipFuncGetAttributes(&fa, (const void*)down_blend_kernel<kDbMaxRows, 1, kDbActPer>) != hipSuccess) return 0;
  if (fa.sharedSizeBytes + down_blend_dyn_lds(rows, k, nr) > (size_t)max_lds_per_block()) return 0;
  return nr;
}

hipError_t launch_down_blend(const SweepParams& p, int rows, int nr, hipStream_t s, StageEvents ev) {
  switch (rows) {
    case 1: return down_blend_r<1>(p, nr, s, ev);
    case 2: return down_blend_r<2>(p, nr, s, ev);
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
static_assert(moe::kMaxRows == MOE_MAX_ROWS && moe::kMaxIds == MOE_MAX_IDS && moe::kNumSlots == MOE_MAX_IDS + 1,
              "device and ABI limits differ");
static_assert(moe::kMaxChunkRows == MOE_MAX_CHUNK_ROWS, "device and ABI staging limits differ");
