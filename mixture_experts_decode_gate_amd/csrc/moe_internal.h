// Host <-> kernel interface of libmoe (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

struct SlotInfo;

// Expert activations and outputs are stored by (row, selected expert) pair:
// pair t = r * k + j for row r's j-th routed expert, rows * k + r for row r's
// shared expert.
constexpr int kMaxPairs = MOE_MAX_IDS + MOE_MAX_ROWS;
// act rows a down-sweep wave holds in registers (16 VGPRs per row per 2048
// columns): four with one 2048-column chunk, two with two
constexpr int down_group(int nch) { return nch == 1 ? 4 : 2; }
constexpr int kMaxDownSegs = MOE_MAX_IDS + 1;  // one segment per union slot and the shared slot
// Down-sweep work weight of a group of n rows: kSegCostBase + n per weight
// row (decode and loads, plus one dot product per row).
constexpr int kSegCostBase = 3;

struct RouteParams {
  const uint16_t* x;       // [rows][h] bf16
  const float* router_w;   // [E][h] fp32 (dense router), or null with router_fp4
  const uint8_t* router_packed;  // NVFP4 router [E][h/2] codes (router_fp4)
  const uint8_t* router_scales;  // NVFP4 router [E][h/16] E4M3 block scales
  float router_scale2;
  int router_fp4;
  const float* gate_vec;   // [h] shared-expert gate vector
  int h;
  const float* bias;       // [E]; for softmax any readable [E] floats (ignored)
  int E, k, rows, route_kind, norm;
  float rsf;
  float* logits;           // [MOE_MAX_ROWS][E]
  double* score;           // [MOE_MAX_ROWS][E] sigmoid(logit) in fp64 (sigmoid routing)
  float* gamma;            // [MOE_MAX_ROWS]
  int32_t* ids_out;        // [rows][k]
  float* w_out;            // [rows][k]
  // union outputs (moe_forward only)
  int32_t* union_ids;
  int32_t* union_count;
  int32_t* slot_to_union;
  uint32_t* row_mask;
  SlotInfo* slots;         // [MOE_MAX_IDS + 1]
  int expert_lo, expert_hi; // experts swept: the union keeps ids in [lo, hi) (all of [0, E) but under EP)
  int ungated;             // 1: no shared-expert gate vector, gamma = 1 (gate_vec then points at any h floats)
  moe_expert_table gate, up, down;
  moe_nvfp4 shared_gate, shared_up, shared_down;
  int inter, shared_inter;
};

struct SweepParams {
  const uint16_t* x;          // [rows][h] bf16
  const SlotInfo* slots;      // [MOE_MAX_IDS + 1] (down sweep; written by the gate/up sweep)
  const int32_t* union_count; // device U (down sweep)
  uint16_t* act;              // [pairs][act_stride] bf16, by (row, expert) pair
  float* y;                   // [pairs][h] fp32, by (row, expert) pair
  int h;
  int act_stride;             // max(inter, shared_inter)
  int inter;                  // routed expert intermediate size
  int shared_inter;
  RouteParams route;          // the gate/up sweep takes top-k from route.logits / route.score
  int32_t* seg_slot;          // [kMaxDownSegs] down segments: union slot
  uint32_t* seg_rows;         // [kMaxDownSegs] down segments: packed rows and count
  int32_t* seg_cum;           // [kMaxDownSegs + 1] down segments: weight before segment s
  int32_t* seg_count;         // [1]
  int token_major;            // 1: one slot per (row, selected expert), no dedup
  uint16_t* out;              // [rows][h] bf16 (down+blend kernel), or null with partial
  float* partial;             // [rows][h] fp32 routed partial (expert-parallel share), or null
};

constexpr size_t kSlotInfoBytes = 88;  // sizeof(SlotInfo), checked in the kernels file

// Optional kernel start/stop events (hipExtLaunchKernel): the events record
// the kernel's own start and end, with nothing enqueued between kernels.
struct StageEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Router GEMV: logits, sigmoid scores and the shared-expert gate.
hipError_t launch_route(const RouteParams& p, hipStream_t s, StageEvents ev = {});
// Top-k of every row from what launch_route left (moe_route only).
hipError_t launch_topk(const RouteParams& p, hipStream_t s);
hipError_t launch_union(const int32_t* ids, int rows, int k, int32_t* union_ids, int32_t* union_count,
                        int32_t* slot_to_union, uint32_t* row_mask, hipStream_t s);
hipError_t launch_gateup(const SweepParams& p, int rows, int max_slots, hipStream_t s, StageEvents ev = {});
hipError_t launch_down(const SweepParams& p, hipStream_t s, StageEvents ev = {});
// Down sweep and blend in one kernel for one or two rows: the rows of output
// each block owns when this call can run it (at most two rows, every pair's
// act fits in LDS), else 0.
int down_blend_rows_per_block(int rows, int k, int h, int imax);
hipError_t launch_down_blend(const SweepParams& p, int rows, int nr, hipStream_t s, StageEvents ev = {});
// out = bf16(sum_j w*y + gamma*s); with partial non-null, partial = sum_j w*y
// (fp32, slots mapped to -1 skipped) and out is not written.
hipError_t launch_blend(const float* y, const float* w, const int32_t* slot_to_union, const float* gamma,
                        uint16_t* out, float* partial, int rows, int h, int k, hipStream_t s, StageEvents ev = {});
hipError_t launch_union_local(const int32_t* ids, int rows, int k, int lo, int hi, int32_t* union_ids,
                              int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask, hipStream_t s);
// Streaming-read probe over ``bytes`` (a multiple of 16) of ``src``; writes
// one word per block to sink[0 .. blocks).
hipError_t launch_read_probe(const uint8_t* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s);
int read_probe_blocks();
// out = bf16(reduced + gamma * shared), the shared expert's output at pair rows*k + r.
hipError_t launch_ep_combine(const float* reduced, const float* y, const float* gamma, uint16_t* out, int rows, int h,
                             int k, hipStream_t s);

}  // namespace moe
