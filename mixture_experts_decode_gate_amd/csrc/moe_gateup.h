// The gate+up sweep kernel and its launch templates (instantiated by the
// moe_gateup_rows_*.hip translation units).
#pragma once

#include "moe_common.h"

namespace moe {

// Gate+up sweep.  It starts with the routing decisions: every block runs
// top-k on the logits the router pass stored (one wave per row), the union
// and the slot table, all in LDS; block 0 also writes them to the workspace
// for the down sweep and the blend.  Redundant work in every block costs a
// few microseconds of arithmetic on 24 KB of L2 reads, against a grid-wide
// hand-off that would cost a ticket, fences and an extra memory round trip.
//
// Work items are rows n of each union slot's gate and up matrices (the shared
// expert's Is rows first, then each routed slot's I rows).
// The block with XCD-major index v (xcd_major_block) owns items v, v + B,
// v + 2B, ... (B blocks), so all blocks sweep the weights front to back
// together, each die over contiguous runs of rows; its waves claim the
// block's items in order from a counter in LDS.  Waves that share a SIMD are not issued evenly
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
  // x is staged in two passes when a thread's share exceeds kXPass loads
  // (fewer with 16 top-k keys per lane): the second goes out after the first
  // is in LDS and lands during top-k.
  constexpr int kXPassMax = G == 4 ? 12 : 6;
  constexpr int kXPass = kXPer < kXPassMax ? kXPer : kXPassMax;
  constexpr int kXRest = kXPer - kXPass;
  // Every expert's pointers are copied to LDS when E <= 256 and the staged x
  // leaves room for them; otherwise each union slot's pointers are read from
  // the expert tables once the union is known.
  constexpr bool kPtab = G == 4 && R * NCH <= kPtabMaxChunkRows;
  constexpr int kTopkRows = (R + kSweepWaves - 1) / kSweepWaves;  // rows each wave runs top-k for
  extern __shared__ u32x4 xs[];  // [R][NCH][256] staged x rows
  __shared__ SlotInfo s_slots[kNumSlots];
  __shared__ ExpertPtrs s_ptab[kPtab ? 64 * G : 1];
  __shared__ __align__(16) int32_t s_ids[kMaxIds];
  __shared__ float s_w[kMaxIds];
  __shared__ int32_t s_uids[kMaxIds], s_s2u[kMaxIds];
  __shared__ uint32_t s_rmask[kMaxIds];
  __shared__ uint32_t s_first[G == 4 ? 256 : 1], s_umask[G == 4 ? 256 : 1];  // union_lds tables
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
  u32x4 xv[kXPass];
  auto x_unit = [&](int i, int& r, int& dst) {  // unit i of the staged x: its row, LDS slot and column
    r = i / (NCH * kChunkUnits);
    const int rem = i - r * NCH * kChunkUnits;
    const int c = rem / kChunkUnits, un = rem - c * kChunkUnits;
    dst = (r * NCH + c) * kChunkUnits + swz_unit(un);
    return c * kChunk + un * 8;
  };
  // Units q0 .. q0 + n - 1 of this thread's share: load, then store (zero past h).
  auto x_load = [&](u32x4* v, int q0, int n) {
#pragma unroll
    for (int q = 0; q < n; ++q) {
      int r, dst;
      const int col = x_unit(min((int)threadIdx.x + (q0 + q) * kMaxSweepThreads, kXUnits - 1), r, dst);
      v[q] = ld_global(reinterpret_cast<const u32x4*>(p.x + (size_t)r * h + (col < h ? col : h - 8)));
    }
  };
  auto x_store = [&](const u32x4* v, int q0, int n) {
#pragma unroll
    for (int q = 0; q < n; ++q) {
      const int i = (int)threadIdx.x + (q0 + q) * kMaxSweepThreads;
      if (i < kXUnits) {
        int r, dst;
        const int col = x_unit(i, r, dst);
        xs[dst] = col < h ? v[q] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  x_load(xv, 0, kXPass);
  // Wave w runs top-k for rows w, w + 8, ...; the prologue loads the inputs
  // of all of them, or with 16 keys per lane (past 256 experts) of the first
  // only (the second row's are loaded when its turn comes).  A wave with no
  // row (w >= R) loads none: its redundant loads would sit in the in-order
  // queue ahead of its first item's weights.  The branch is wave-uniform and
  // every load after it is issued on both paths in the same order, so the
  // waits below stay exact; the loads that do not depend on the wave
  // (x, the pointer table) stay unconditional with clamped indices.
  constexpr int kTopkPre = G == 4 ? kTopkRows : 1;
  TopkIn<G> tin[kTopkPre] = {};
#pragma unroll
  for (int i = 0; i < kTopkPre; ++i) {
    const int r = wave + i * kSweepWaves;
    if (r < R) topk_load<G>(rp, r, lane, tin[i]);
  }
  ExpertPtrs ep;
  if (kPtab) ep = expert_ptrs(rp, min((int)threadIdx.x, rp.E - 1));
  if (threadIdx.x == 0) {
    s_next = 0;
    s_slots[kSharedSlot] = shared_slot_info(rp, (1u << R) - 1u);
  }
  __syncthreads();

  // Items: the shared expert's Is rows first, then each routed slot's I rows.
  // The item id of the block's claim i is v + i * B (not yet checked against
  // the item count, which needs U).
  const int vblock = xcd_major_block();
  auto claim_id = [&]() -> long long {
    int i = 0;
    if (lane == 0) i = atomicAdd(&s_next, 1);
    i = __builtin_amdgcn_readfirstlane(i);
    return (long long)vblock + (long long)i * gridDim.x;
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
  // claim is a routed row loads the stand-in instead (it is not computed) so
  // the load stays unconditional, and fetches its item later.  The stand-in,
  // loaded wherever there is no item (also past the last claim), is the
  // shared expert's row 0: the same address in every wave, so it is served
  // from the cache and its loads are always in bounds.
  constexpr int kStandin = 0;
  long long first = claim_id();
  const bool early = first < p.shared_inter;
  fetch(early ? (int)first : kStandin, ga, ua, sa, na);
  // Nothing that reads a loaded value may be scheduled above the fetch.
  __builtin_amdgcn_sched_barrier(0);

  // Consume, in issue order: x (zero past h), top-k, the pointer table.
  x_store(xv, 0, kXPass);
  // Every prologue load is waited for here on every path (see consume()),
  // used or not.
#pragma unroll
  for (int q = 0; q < kXPass; ++q) asm volatile("" ::"v"(xv[q]));
#pragma unroll
  for (int t = 0; t < kTopkPre; ++t)
#pragma unroll
    for (int i = 0; i < G; ++i) asm volatile("" ::"v"(tin[t].lv[i]), "v"(tin[t].bv[i]), "v"(tin[t].sv[i]));
  if (kPtab) {
#pragma unroll
    for (int i = 0; i < 6; ++i) asm volatile("" ::"v"(ep.p[i]));
#pragma unroll
    for (int i = 0; i < 3; ++i) asm volatile("" ::"v"(ep.scale2[i]));
  }
  // the rest of x, if any: issued now, it lands while top-k runs
  u32x4 xv2[kXRest > 0 ? kXRest : 1];
  if (kXRest > 0) x_load(xv2, kXPass, kXRest);
#pragma unroll
  for (int i = 0; i < kTopkRows; ++i) {
    const int r = wave + i * kSweepWaves;
    if (i < kTopkPre) {
      if (r < R) topk_select<G>(rp, r, lane, tin[i < kTopkPre ? i : 0], s_ids, nullptr, publish ? s_w : nullptr);
    } else {
      TopkIn<G> late;
      topk_load<G>(rp, r < R ? r : R - 1, lane, late);
      if (r < R) topk_select<G>(rp, r, lane, late, s_ids, nullptr, publish ? s_w : nullptr);
    }
  }
  if (kXRest > 0) {
    x_store(xv2, kXPass, kXRest);
#pragma unroll
    for (int q = 0; q < kXRest; ++q) asm volatile("" ::"v"(xv2[q]));
  }
  if (kPtab && (int)threadIdx.x < rp.E) s_ptab[threadIdx.x] = ep;
  __syncthreads();
  if (wave == 0) {
    UnionLane ul;
    // One row's top-k ids are distinct and already in first-occurrence order:
    // its union over the full expert range is the slot list itself.
    const bool identity = p.token_major || (R == 1 && rp.expert_lo == 0 && rp.expert_hi >= rp.E);
    if (G == 4 && !identity) {
      union_lds(s_ids, R * rp.k, rp.k, rp.expert_lo, rp.expert_hi, lane, s_first, s_umask, s_uids, &s_union, s_s2u,
                s_rmask, s_slots, [&](int ex, uint32_t mask) {
                  return slot_info_base(kPtab ? s_ptab[ex] : expert_ptrs(rp, ex), ex, rp.inter, mask);
                });
    } else {
      if (identity)
        identity_slots(s_ids, R * rp.k, rp.k, lane, s_uids, &s_union, s_s2u, s_rmask, ul);
      else
        union_wave(s_ids, R * rp.k, rp.k, R, rp.expert_lo, rp.expert_hi, lane, s_uids, &s_union, s_s2u, s_rmask, ul);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (ul.pos[q] >= 0) {  // slot 64*q + lane is the union entry's first slot
          const int ex = s_ids[64 * q + lane];
          s_slots[ul.pos[q]] = slot_info(kPtab ? s_ptab[ex] : expert_ptrs(rp, ex), ex, rp.inter, ul.mask[q],
                                         ul.eq[q], rp.k, R);
        }
      }
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
  fetch(id_b >= 0 ? id_b : kStandin, gb, ub, sb, nb);
  // Block 0 publishes the routing results for the down sweep and the blend.
  if (publish && wave == 0) {
    const int n = R * rp.k;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int t = 64 * q + lane;
      if (t < n) {
        rp.ids_out[t] = s_ids[t];
        rp.w_out[t] = s_w[t];
        rp.slot_to_union[t] = s_s2u[t];
      }
      if (t < U) {
        rp.union_ids[t] = s_uids[t];
        rp.row_mask[t] = s_rmask[t];
        rp.slots[t] = s_slots[t];
      }
    }
    if (lane == 0) {
      *rp.union_count = U;
      rp.slots[kSharedSlot] = s_slots[kSharedSlot];
    }
    const int kdown = p.inter > p.shared_inter ? p.inter : p.shared_inter;  // the down sweep's K
    const int nseg = build_segments(lane < U ? s_slots[lane].row_mask : 0u,
                                    64 + lane < U ? s_slots[64 + lane].row_mask : 0u, lane, R,
                                    down_group((kdown + kChunk - 1) / kChunk), p.seg_slot, p.seg_rows, p.seg_cum);
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
    fetch(id_c >= 0 ? id_c : kStandin, gc, uc, sc, nc);
    consume<NCH>(ga);
    consume<NCH>(ua);
    if (id_a >= 0) compute(ga, ua, sa, na);
    const int id_a2 = id_c >= 0 ? claim() : -1;
    fetch(id_a2 >= 0 ? id_a2 : kStandin, ga, ua, sa, na);
    consume<NCH>(gb);
    consume<NCH>(ub);
    if (id_b >= 0) compute(gb, ub, sb, nb);
    const int id_b2 = id_a2 >= 0 ? claim() : -1;
    fetch(id_b2 >= 0 ? id_b2 : kStandin, gb, ub, sb, nb);
    consume<NCH>(gc);
    consume<NCH>(uc);
    if (id_c >= 0) compute(gc, uc, sc, nc);
    if (id_a2 < 0) break;
    id_a = id_a2;
    id_b = id_b2;
  }
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

// Instances exist for R * NCH <= kMaxChunkRows (the staged x fits in LDS);
// the ABI refuses larger row counts before any launch.
template <int R>
hipError_t gateup_r(const SweepParams& p, int nch, int max_items, hipStream_t s, StageEvents ev) {
  switch (nch) {
    case 1:
      if constexpr (R * 1 <= kMaxChunkRows) return gateup_rn<R, 1>(p, max_items, s, ev);
      break;
    case 2:
      if constexpr (R * 2 <= kMaxChunkRows) return gateup_rn<R, 2>(p, max_items, s, ev);
      break;
    case 3:
      if constexpr (R * 3 <= kMaxChunkRows) return gateup_rn<R, 3>(p, max_items, s, ev);
      break;
    case 4:
      if constexpr (R * 4 <= kMaxChunkRows) return gateup_rn<R, 4>(p, max_items, s, ev);
      break;
  }
  return hipErrorInvalidValue;
}


}  // namespace moe
