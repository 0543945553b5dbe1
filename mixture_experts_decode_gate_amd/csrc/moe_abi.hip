// C ABI of libmoe: argument validation, workspace layout and stage launches.
//
// Every refusal happens here, before any HIP call, and leaves a message for
// moe_last_error() -- the C form of the refusals the pages make with a message
// (forward_token_major.rs and forward_ep.rs refuse a router whose width differs
// from num_experts; forward_token_major.rs routes layers without a shared
// expert or with other formats to another path).

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "moe_internal.h"

// Workspace of moe_forward_static: one array per GPU, in the library's own
// device memory, held until the process ends.  In host code ``scratch`` names a
// host-side stand-in, not a device address: the address each GPU holds it at
// comes from hipGetSymbolAddress (scratch_address below) and only that address
// is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Stage 2 is one kernel (down sweep and blend together) for one or two rows
// whose pairs' activations all fit in LDS, else the down sweep and then the
// blend kernel.
const char* const kStageNames[] = {"route", "gate_up_sweep", "down_sweep_blend"};
constexpr int kNumStages = 3;

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->hidden < MOE_DIM_ALIGN || c->hidden > MOE_MAX_DIM || c->hidden % MOE_DIM_ALIGN)
    return fail(MOE_ERR_INVALID_ARG, "hidden=%d must be a multiple of %d in [%d, %d]", c->hidden, MOE_DIM_ALIGN,
                MOE_DIM_ALIGN, MOE_MAX_DIM);
  if (c->moe_inter < MOE_DIM_ALIGN || c->moe_inter > MOE_MAX_INTER || c->moe_inter % MOE_DIM_ALIGN)
    return fail(MOE_ERR_INVALID_ARG, "moe_inter=%d must be a multiple of %d in [%d, %d]", c->moe_inter,
                MOE_DIM_ALIGN, MOE_DIM_ALIGN, MOE_MAX_INTER);
  if (c->shared_inter < MOE_DIM_ALIGN || c->shared_inter > MOE_MAX_INTER || c->shared_inter % MOE_DIM_ALIGN)
    return fail(MOE_ERR_INVALID_ARG, "shared_inter=%d must be a multiple of %d in [%d, %d]", c->shared_inter,
                MOE_DIM_ALIGN, MOE_DIM_ALIGN, MOE_MAX_INTER);
  if (c->num_experts < 1 || c->num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "num_experts=%d outside [1, %d]", c->num_experts, MOE_MAX_EXPERTS);
  if (c->top_k < 1 || c->top_k > c->num_experts || c->top_k > MOE_MAX_IDS)
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside [1, min(num_experts=%d, %d)]", c->top_k, c->num_experts,
                MOE_MAX_IDS);
  if (c->route_kind != MOE_ROUTE_SOFTMAX && c->route_kind != MOE_ROUTE_SIGMOID_BIAS)
    return fail(MOE_ERR_INVALID_ARG, "unknown route_kind %d", c->route_kind);
  if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1)
    return fail(MOE_ERR_INVALID_ARG, "norm_topk_prob=%d must be 0 or 1", c->norm_topk_prob);
  const float rsf = c->routed_scaling_factor;
  if (!(rsf == rsf) || rsf > 3.0e38f || rsf < -3.0e38f)
    return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor is not finite");
  return MOE_OK;
}

// Column chunks of 2048 the gate/up sweep stages per row of x.
int x_chunks(const moe_config* c) { return (c->hidden + 2047) / 2048; }

// Largest rows one call serves for this config: MOE_MAX_ROWS, top_k * rows
// <= MOE_MAX_IDS, and rows * x_chunks <= MOE_MAX_CHUNK_ROWS (the gate/up
// sweep holds every row of x in LDS).
int max_rows(const moe_config* c) {
  int r = MOE_MAX_ROWS;
  if (MOE_MAX_IDS / c->top_k < r) r = MOE_MAX_IDS / c->top_k;
  if (MOE_MAX_CHUNK_ROWS / x_chunks(c) < r) r = MOE_MAX_CHUNK_ROWS / x_chunks(c);
  return r;
}

// Rows routing alone takes: MOE_MAX_ROWS, and top_k * rows ids for the union.
moe_status check_route_rows(const moe_config* c, int32_t rows) {
  if (rows < 1 || rows > MOE_MAX_ROWS)
    return fail(MOE_ERR_INVALID_ARG, "rows=%d outside [1, %d]", rows, MOE_MAX_ROWS);
  if (c->top_k * rows > MOE_MAX_IDS)
    return fail(MOE_ERR_INVALID_ARG, "top_k*rows=%d exceeds the %d ids the union takes", c->top_k * rows,
                MOE_MAX_IDS);
  return MOE_OK;
}

// Rows the whole layer takes: also every row of x in the gate/up sweep's LDS.
moe_status check_rows(const moe_config* c, int32_t rows) {
  moe_status st = check_route_rows(c, rows);
  if (st) return st;
  if (rows * x_chunks(c) > MOE_MAX_CHUNK_ROWS)
    return fail(MOE_ERR_UNSUPPORTED,
                "rows=%d at hidden=%d stages %d chunks of x in LDS (at most %d): at most %d rows per call here; "
                "moe_forward_prefill takes any number",
                rows, c->hidden, rows * x_chunks(c), MOE_MAX_CHUNK_ROWS, MOE_MAX_CHUNK_ROWS / x_chunks(c));
  return MOE_OK;
}

moe_status check_nvfp4(const moe_nvfp4& t, const char* name) {
  if (!t.packed || !t.scales) return fail(MOE_ERR_UNSUPPORTED, "%s: the layer has no shared expert", name);
  if (!aligned(t.packed, 16) || !aligned(t.scales, 16))
    return fail(MOE_ERR_INVALID_ARG, "%s: packed and scales must be 16-byte aligned", name);
  if (!(t.scale2 == t.scale2)) return fail(MOE_ERR_INVALID_ARG, "%s: scale2 is NaN", name);
  return MOE_OK;
}

moe_status check_table(const moe_expert_table& t, const char* name) {
  if (!t.packed || !t.scales || !t.scale2) return fail(MOE_ERR_INVALID_ARG, "%s table has a NULL array", name);
  if (!aligned(t.packed, 8) || !aligned(t.scales, 8) || !aligned(t.scale2, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s table arrays are misaligned", name);
  return MOE_OK;
}

moe_status check_route_weights(const moe_config* c, const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  if (w->router_w) {
    if (!aligned(w->router_w, 16)) return fail(MOE_ERR_INVALID_ARG, "router_w must be 16-byte aligned");
    if (w->router_nvfp4.packed || w->router_nvfp4.scales)
      return fail(MOE_ERR_INVALID_ARG, "router_w and router_nvfp4 are both set");
  } else {
    const moe_nvfp4& r = w->router_nvfp4;
    if (!r.packed || !r.scales) return fail(MOE_ERR_INVALID_ARG, "no router: router_w and router_nvfp4 are NULL");
    if (!aligned(r.packed, 16) || !aligned(r.scales, 16))
      return fail(MOE_ERR_INVALID_ARG, "router_nvfp4 packed and scales must be 16-byte aligned");
    const float s2 = r.scale2;
    if (!(s2 == s2) || s2 > 3.0e38f || s2 < -3.0e38f) return fail(MOE_ERR_INVALID_ARG, "router scale2 is not finite");
  }
  if (c->route_kind == MOE_ROUTE_SIGMOID_BIAS) {
    if (!w->correction_bias || !aligned(w->correction_bias, 4))
      return fail(MOE_ERR_INVALID_ARG, "sigmoid routing needs an aligned correction_bias");
  } else if (w->correction_bias) {
    return fail(MOE_ERR_INVALID_ARG, "softmax routing takes no correction_bias");
  }
  // A NULL gate is the ungated shared expert (gamma = 1).
  if (w->shared_expert_gate && !aligned(w->shared_expert_gate, 16))
    return fail(MOE_ERR_INVALID_ARG, "shared_expert_gate must be 16-byte aligned");
  return MOE_OK;
}

moe_status check_all_weights(const moe_config* c, const moe_weights* w) {
  moe_status st = check_route_weights(c, w);
  if (st) return st;
  if ((st = check_nvfp4(w->shared_gate, "shared_gate"))) return st;
  if ((st = check_nvfp4(w->shared_up, "shared_up"))) return st;
  if ((st = check_nvfp4(w->shared_down, "shared_down"))) return st;
  if ((st = check_table(w->gate, "gate"))) return st;
  if ((st = check_table(w->up, "up"))) return st;
  if ((st = check_table(w->down, "down"))) return st;
  return MOE_OK;
}

void compute_layout(const moe_config* c, moe_ws_layout* L) {
  const size_t R = MOE_MAX_ROWS, E = (size_t)c->num_experts, k = (size_t)c->top_k, h = (size_t)c->hidden;
  const size_t imax = (size_t)(c->moe_inter > c->shared_inter ? c->moe_inter : c->shared_inter);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L->logits = take(R * E * sizeof(float));
  L->score = take(R * E * sizeof(double));
  L->gamma = take(R * sizeof(float));
  L->topk_ids = take(R * k * sizeof(int32_t));
  L->topk_w = take(R * k * sizeof(float));
  L->union_ids = take(MOE_MAX_IDS * sizeof(int32_t));
  L->union_count = take(sizeof(int32_t));
  L->slot_to_union = take(MOE_MAX_IDS * sizeof(int32_t));
  L->row_mask = take(MOE_MAX_IDS * sizeof(uint32_t));
  L->slot_info = take((size_t)(MOE_MAX_IDS + 1) * moe::kSlotInfoBytes);
  L->segments = take(sizeof(int32_t) + (size_t)moe::kMaxDownSegs * (sizeof(int32_t) + sizeof(uint32_t)) +
                     (size_t)(moe::kMaxDownSegs + 1) * sizeof(int32_t));
  L->act = take((size_t)moe::kMaxPairs * imax * sizeof(uint16_t));
  L->y = take((size_t)moe::kMaxPairs * h * sizeof(float));
  L->total = off;
}

moe_status check_ws(const moe_config* c, void* ws, size_t ws_bytes, moe_ws_layout* L) {
  compute_layout(c, L);
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  if (ws_bytes < L->total)
    return fail(MOE_ERR_WORKSPACE, "ws_bytes=%zu < %zu required", ws_bytes, L->total);
  return MOE_OK;
}

moe_status check_xy(const moe_config* c, const uint16_t* x, const uint16_t* out, int32_t rows, void* ws,
                    const moe_ws_layout& L) {
  const size_t xb = (size_t)rows * c->hidden * sizeof(uint16_t);
  if (!x || !aligned(x, 16)) return fail(MOE_ERR_INVALID_ARG, "x must be a 16-byte aligned device pointer");
  if (overlaps(x, xb, ws, L.total)) return fail(MOE_ERR_INVALID_ARG, "x overlaps the workspace");
  if (out) {
    if (!aligned(out, 16)) return fail(MOE_ERR_INVALID_ARG, "out must be 16-byte aligned");
    if (overlaps(x, xb, out, xb)) return fail(MOE_ERR_INVALID_ARG, "x and out overlap");
    if (overlaps(out, xb, ws, L.total)) return fail(MOE_ERR_INVALID_ARG, "out overlaps the workspace");
  }
  return MOE_OK;
}

moe_status check_union_args(const int32_t* topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                            const int32_t* union_ids, const int32_t* union_count, const int32_t* slot_to_union,
                            const uint32_t* row_mask) {
  if (rows < 1 || rows > MOE_MAX_ROWS) return fail(MOE_ERR_INVALID_ARG, "rows=%d outside [1, %d]", rows, MOE_MAX_ROWS);
  if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "num_experts=%d outside [1, %d]", num_experts, MOE_MAX_EXPERTS);
  if (top_k < 1 || top_k > num_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside [1, num_experts=%d]", top_k, num_experts);
  if (top_k * rows > MOE_MAX_IDS)
    return fail(MOE_ERR_INVALID_ARG, "top_k*rows=%d exceeds %d", top_k * rows, MOE_MAX_IDS);
  if (!topk_ids || !union_ids || !union_count || !slot_to_union)
    return fail(MOE_ERR_INVALID_ARG, "NULL id buffer");
  if (!aligned(topk_ids, 4) || !aligned(union_ids, 4) || !aligned(union_count, 4) || !aligned(slot_to_union, 4) ||
      (row_mask && !aligned(row_mask, 4)))
    return fail(MOE_ERR_INVALID_ARG, "id buffers must be 4-byte aligned");
  const size_t n = (size_t)rows * top_k * 4;
  if (overlaps(union_ids, MOE_MAX_IDS * 4, slot_to_union, n) || overlaps(union_count, 4, union_ids, MOE_MAX_IDS * 4) ||
      overlaps(union_count, 4, slot_to_union, n) ||
      (row_mask && (overlaps(row_mask, MOE_MAX_IDS * 4, union_ids, MOE_MAX_IDS * 4) ||
                    overlaps(row_mask, MOE_MAX_IDS * 4, slot_to_union, n) || overlaps(row_mask, MOE_MAX_IDS * 4, union_count, 4))))
    return fail(MOE_ERR_INVALID_ARG, "union output buffers overlap");
  return MOE_OK;
}

moe_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// Device address of ``scratch`` on the current device, looked up once per
// device with that device current (each GPU holds its own copy).
constexpr int kScratchDevices = 64;
struct ScratchAddress {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddress g_scratch[kScratchDevices];

moe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d: the static workspace serves devices 0..%d", dev, kScratchDevices - 1);
  ScratchAddress& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess) return device_status(s.err, "hipGetSymbolAddress(scratch)");
  if (!s.ptr) return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
  *out = s.ptr;
  return MOE_OK;
}

void fill_route(moe::RouteParams& p, const moe_config* c, const moe_weights* w, const uint16_t* x, int32_t rows,
                char* ws, const moe_ws_layout& L, int32_t* ids_out, float* w_out) {
  memset(&p, 0, sizeof p);
  p.x = x;
  p.router_w = w->router_w;
  p.router_fp4 = w->router_w ? 0 : 1;
  p.router_packed = w->router_nvfp4.packed;
  p.router_scales = w->router_nvfp4.scales;
  p.router_scale2 = w->router_nvfp4.scale2;
  // Without a gate vector the gate pass reads the workspace's expert outputs
  // (any h readable floats; written later in the call) and writes gamma = 1.
  p.gate_vec = w->shared_expert_gate ? w->shared_expert_gate : reinterpret_cast<const float*>(ws + L.y);
  p.ungated = w->shared_expert_gate ? 0 : 1;
  p.expert_lo = 0;
  p.expert_hi = c->num_experts;
  p.h = c->hidden;
  // Top-k reads bias[e] unconditionally; softmax routing ignores the value,
  // so it reads the workspace's expert outputs (at least E floats) instead.
  p.bias = w->correction_bias ? w->correction_bias : reinterpret_cast<const float*>(ws + L.y);
  p.E = c->num_experts;
  p.k = c->top_k;
  p.rows = rows;
  p.route_kind = c->route_kind;
  p.norm = c->norm_topk_prob;
  p.rsf = c->routed_scaling_factor;
  p.logits = reinterpret_cast<float*>(ws + L.logits);
  p.score = reinterpret_cast<double*>(ws + L.score);
  p.gamma = reinterpret_cast<float*>(ws + L.gamma);
  p.ids_out = ids_out;
  p.w_out = w_out;
  p.union_ids = reinterpret_cast<int32_t*>(ws + L.union_ids);
  p.union_count = reinterpret_cast<int32_t*>(ws + L.union_count);
  p.slot_to_union = reinterpret_cast<int32_t*>(ws + L.slot_to_union);
  p.row_mask = reinterpret_cast<uint32_t*>(ws + L.row_mask);
  p.slots = reinterpret_cast<moe::SlotInfo*>(ws + L.slot_info);
  p.gate = w->gate;
  p.up = w->up;
  p.down = w->down;
  p.shared_gate = w->shared_gate;
  p.shared_up = w->shared_up;
  p.shared_down = w->shared_down;
  p.inter = c->moe_inter;
  p.shared_inter = c->shared_inter;
}

// Options of one layer evaluation beyond moe_forward's arguments.
struct ForwardMode {
  bool token_major = false;  // one slot per (row, selected expert), no union
  int lo = 0, hi = -1;       // experts swept: [lo, hi) (hi < 0: all)
  float* partial = nullptr;  // EP share: fp32 routed partial instead of out
};

moe_status forward_impl(const moe_config* cfg, const moe_weights* w, const uint16_t* x, uint16_t* out,
                        int32_t rows, void* ws, size_t ws_bytes, void* stream, void* const* events,
                        const ForwardMode& mode) {
  moe_status st = check_config(cfg);
  if (st) return st;
  if ((st = check_rows(cfg, rows))) return st;
  if ((st = check_all_weights(cfg, w))) return st;
  moe_ws_layout L;
  if ((st = check_ws(cfg, ws, ws_bytes, &L))) return st;
  const int lo = mode.lo, hi = mode.hi < 0 ? cfg->num_experts : mode.hi;
  if (lo < 0 || lo > hi || hi > cfg->num_experts)
    return fail(MOE_ERR_INVALID_ARG, "expert range [%d, %d) outside [0, num_experts=%d]", lo, hi, cfg->num_experts);
  if (mode.partial) {
    const size_t pb = (size_t)rows * cfg->hidden * sizeof(float);
    if (!aligned(mode.partial, 16)) return fail(MOE_ERR_INVALID_ARG, "partial must be 16-byte aligned");
    if (overlaps(mode.partial, pb, x, (size_t)rows * cfg->hidden * 2) || overlaps(mode.partial, pb, ws, L.total))
      return fail(MOE_ERR_INVALID_ARG, "partial overlaps x or the workspace");
    if ((st = check_xy(cfg, x, nullptr, rows, ws, L))) return st;
  } else {
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    if ((st = check_xy(cfg, x, out, rows, ws, L))) return st;
  }
  const bool token_major = mode.token_major;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  // Stage i's kernel records events[2i] at its start and events[2i+1] at its end.
  auto stage_ev = [&](int i) {
    moe::StageEvents ev;
    if (events) {
      ev.start = reinterpret_cast<hipEvent_t>(events[2 * i]);
      ev.stop = reinterpret_cast<hipEvent_t>(events[2 * i + 1]);
    }
    return ev;
  };
  // Slots the sweeps may see: the union holds at most min(k*rows, E) experts;
  // the token-major list holds every one of the k*rows pairs.
  const int max_slots = token_major ? cfg->top_k * rows : (cfg->top_k * rows < hi - lo ? cfg->top_k * rows : hi - lo);

  moe::RouteParams rp;
  int32_t* ids = reinterpret_cast<int32_t*>(wsb + L.topk_ids);
  float* wts = reinterpret_cast<float*>(wsb + L.topk_w);
  fill_route(rp, cfg, w, x, rows, wsb, L, ids, wts);
  rp.expert_lo = lo;
  rp.expert_hi = hi;

  moe::SweepParams sp;
  sp.x = x;
  sp.slots = reinterpret_cast<const moe::SlotInfo*>(wsb + L.slot_info);
  sp.union_count = reinterpret_cast<const int32_t*>(wsb + L.union_count);
  sp.act = reinterpret_cast<uint16_t*>(wsb + L.act);
  sp.y = reinterpret_cast<float*>(wsb + L.y);
  sp.h = cfg->hidden;
  sp.act_stride = cfg->moe_inter > cfg->shared_inter ? cfg->moe_inter : cfg->shared_inter;
  sp.inter = cfg->moe_inter;
  sp.shared_inter = cfg->shared_inter;
  sp.route = rp;
  sp.seg_count = reinterpret_cast<int32_t*>(wsb + L.segments);
  sp.seg_slot = sp.seg_count + 1;
  sp.seg_rows = reinterpret_cast<uint32_t*>(sp.seg_slot + moe::kMaxDownSegs);
  sp.seg_cum = reinterpret_cast<int32_t*>(sp.seg_rows + moe::kMaxDownSegs);
  sp.token_major = token_major ? 1 : 0;
  sp.out = out;
  sp.partial = mode.partial;

  hipError_t e;
  if ((e = moe::launch_route(rp, s, stage_ev(0))) != hipSuccess) return device_status(e, "route launch");
  if ((e = moe::launch_gateup(sp, rows, max_slots, s, stage_ev(1))) != hipSuccess)
    return device_status(e, "gate/up launch");
  const moe::StageEvents ev2 = stage_ev(2);
  const int nr = moe::down_blend_rows_per_block(rows, cfg->top_k, cfg->hidden, sp.act_stride);
  if (nr > 0) {
    if ((e = moe::launch_down_blend(sp, rows, nr, s, ev2)) != hipSuccess) return device_status(e, "down+blend launch");
    return ok();
  }
  if ((e = moe::launch_down(sp, s, {ev2.start, nullptr})) != hipSuccess) return device_status(e, "down launch");
  e = moe::launch_blend(sp.y, wts, rp.slot_to_union, reinterpret_cast<const float*>(wsb + L.gamma), out,
                        mode.partial, rows, cfg->hidden, cfg->top_k, s, {nullptr, ev2.stop});
  if (e != hipSuccess) return device_status(e, "blend launch");
  return ok();
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  moe_ws_layout L;
  compute_layout(cfg, &L);
  return L.total;
}

moe_status moe_workspace_layout(const moe_config* cfg, moe_ws_layout* out) {
  moe_status st = check_config(cfg);
  if (st) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  compute_layout(cfg, out);
  return ok();
}

moe_status moe_route(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16, int32_t rows,
                     int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st) return st;
  if ((st = check_route_rows(cfg, rows))) return st;
  if ((st = check_route_weights(cfg, w))) return st;
  moe_ws_layout L;
  if ((st = check_ws(cfg, ws, ws_bytes, &L))) return st;
  if ((st = check_xy(cfg, x_bf16, nullptr, rows, ws, L))) return st;
  if (!topk_ids || !aligned(topk_ids, 4) || !topk_w || !aligned(topk_w, 4))
    return fail(MOE_ERR_INVALID_ARG, "topk_ids and topk_w must be aligned device pointers");
  const size_t nb = (size_t)rows * cfg->top_k * 4;
  if (overlaps(topk_ids, nb, topk_w, nb)) return fail(MOE_ERR_INVALID_ARG, "topk_ids and topk_w overlap");
  char* wsb = static_cast<char*>(ws);
  if (overlaps(topk_ids, nb, wsb, L.topk_ids) || overlaps(topk_w, nb, wsb, L.topk_ids))
    return fail(MOE_ERR_INVALID_ARG, "topk outputs overlap the router intermediates of the workspace");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  moe::RouteParams rp;
  fill_route(rp, cfg, w, x_bf16, rows, wsb, L, topk_ids, topk_w);
  hipError_t e = moe::launch_route(rp, s);
  if (e != hipSuccess) return device_status(e, "route launch");
  if ((e = moe::launch_topk(rp, s)) != hipSuccess) return device_status(e, "top-k launch");
  return ok();
}

moe_status moe_union(const int32_t* topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                     int32_t* union_ids, int32_t* union_count, int32_t* slot_to_union, uint32_t* row_mask,
                     void* stream) {
  moe_status st = check_union_args(topk_ids, rows, top_k, num_experts, union_ids, union_count, slot_to_union, row_mask);
  if (st) return st;
  hipError_t e = moe::launch_union(topk_ids, rows, top_k, union_ids, union_count, slot_to_union, row_mask,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_status(e, "union launch");
  return ok();
}

moe_status moe_union_local(const int32_t* topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                           int32_t expert_lo, int32_t expert_hi, int32_t* union_ids, int32_t* union_count,
                           int32_t* slot_to_union, uint32_t* row_mask, void* stream) {
  moe_status st = check_union_args(topk_ids, rows, top_k, num_experts, union_ids, union_count, slot_to_union, row_mask);
  if (st) return st;
  if (expert_lo < 0 || expert_lo > expert_hi || expert_hi > num_experts)
    return fail(MOE_ERR_INVALID_ARG, "expert range [%d, %d) outside [0, num_experts=%d]", expert_lo, expert_hi,
                num_experts);
  hipError_t e = moe::launch_union_local(topk_ids, rows, top_k, expert_lo, expert_hi, union_ids, union_count,
                                         slot_to_union, row_mask, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_status(e, "union launch");
  return ok();
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16, uint16_t* out_bf16,
                       int32_t rows, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(cfg, w, x_bf16, out_bf16, rows, ws, ws_bytes, stream, nullptr, ForwardMode());
}

moe_status moe_forward_static(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16, uint16_t* out_bf16,
                              int32_t rows, void* stream) {
  // Every refusal before any HIP call, as moe_forward's: the layout of this
  // config must fit the static workspace.
  moe_status st = check_config(cfg);
  if (st) return st;
  if ((st = check_rows(cfg, rows))) return st;
  moe_ws_layout L;
  compute_layout(cfg, &L);
  if (L.total > (size_t)MOE_STATIC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED, "the layer's workspace needs %zu bytes; the static workspace holds %d",
                L.total, (int)MOE_STATIC_SCRATCH_BYTES);
  if ((st = check_all_weights(cfg, w))) return st;
  if (!x_bf16 || !aligned(x_bf16, 16)) return fail(MOE_ERR_INVALID_ARG, "x must be a 16-byte aligned device pointer");
  if (!out_bf16 || !aligned(out_bf16, 16)) return fail(MOE_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const size_t xb = (size_t)rows * cfg->hidden * sizeof(uint16_t);
  if (overlaps(x_bf16, xb, out_bf16, xb)) return fail(MOE_ERR_INVALID_ARG, "x and out overlap");
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return forward_impl(cfg, w, x_bf16, out_bf16, rows, ws, (size_t)MOE_STATIC_SCRATCH_BYTES, stream, nullptr,
                      ForwardMode());
}

moe_status moe_forward_prefill(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                               uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 1) return fail(MOE_ERR_INVALID_ARG, "rows=%d must be positive", rows);
  moe_status st = check_config(cfg);
  if (st) return st;
  const int chunk = max_rows(cfg);
  if (!x_bf16 || !out_bf16) return fail(MOE_ERR_INVALID_ARG, "x and out must be device pointers");
  const size_t xb = (size_t)rows * cfg->hidden * sizeof(uint16_t);
  if (overlaps(x_bf16, xb, out_bf16, xb)) return fail(MOE_ERR_INVALID_ARG, "x and out overlap");
  if (ws && overlaps(x_bf16, xb, ws, ws_bytes)) return fail(MOE_ERR_INVALID_ARG, "x overlaps the workspace");
  if (ws && overlaps(out_bf16, xb, ws, ws_bytes)) return fail(MOE_ERR_INVALID_ARG, "out overlaps the workspace");
  // Each sub-chunk is one moe_forward on the same stream and workspace, in row
  // order; every argument check runs on the first sub-chunk before any launch.
  for (int32_t r0 = 0; r0 < rows; r0 += chunk) {
    const int32_t n = rows - r0 < chunk ? rows - r0 : chunk;
    const size_t off = (size_t)r0 * cfg->hidden;
    st = forward_impl(cfg, w, x_bf16 + off, out_bf16 + off, n, ws, ws_bytes, stream, nullptr, ForwardMode());
    if (st) return st;
  }
  return ok();
}

moe_status moe_forward_token_major(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                                   uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes, void* stream) {
  ForwardMode m;
  m.token_major = true;
  return forward_impl(cfg, w, x_bf16, out_bf16, rows, ws, ws_bytes, stream, nullptr, m);
}

moe_status moe_forward_ep_partial(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                                  float* partial, int32_t rows, int32_t expert_lo, int32_t expert_hi, void* ws,
                                  size_t ws_bytes, void* stream) {
  if (!partial) return fail(MOE_ERR_INVALID_ARG, "partial is NULL");
  ForwardMode m;
  m.lo = expert_lo;
  m.hi = expert_hi;
  m.partial = partial;
  if (expert_hi < 0) return fail(MOE_ERR_INVALID_ARG, "expert_hi=%d is negative", expert_hi);
  return forward_impl(cfg, w, x_bf16, nullptr, rows, ws, ws_bytes, stream, nullptr, m);
}

moe_status moe_ep_combine(const moe_config* cfg, const float* reduced, uint16_t* out_bf16, int32_t rows, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st) return st;
  if ((st = check_rows(cfg, rows))) return st;
  moe_ws_layout L;
  if ((st = check_ws(cfg, ws, ws_bytes, &L))) return st;
  const size_t rb = (size_t)rows * cfg->hidden * sizeof(float), ob = (size_t)rows * cfg->hidden * 2;
  if (!reduced || !aligned(reduced, 16)) return fail(MOE_ERR_INVALID_ARG, "reduced must be a 16-byte aligned pointer");
  if (!out_bf16 || !aligned(out_bf16, 16)) return fail(MOE_ERR_INVALID_ARG, "out must be a 16-byte aligned pointer");
  if (overlaps(reduced, rb, out_bf16, ob)) return fail(MOE_ERR_INVALID_ARG, "reduced and out overlap");
  if (overlaps(reduced, rb, ws, L.total) || overlaps(out_bf16, ob, ws, L.total))
    return fail(MOE_ERR_INVALID_ARG, "reduced or out overlaps the workspace");
  char* wsb = static_cast<char*>(ws);
  hipError_t e = moe::launch_ep_combine(reduced, reinterpret_cast<const float*>(wsb + L.y),
                                        reinterpret_cast<const float*>(wsb + L.gamma), out_bf16, rows, cfg->hidden,
                                        cfg->top_k, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_status(e, "combine launch");
  return ok();
}

moe_status moe_forward_timed(const moe_config* cfg, const moe_weights* w, const uint16_t* x_bf16,
                             uint16_t* out_bf16, int32_t rows, void* ws, size_t ws_bytes, void* stream,
                             void* const* stage_events) {
  return forward_impl(cfg, w, x_bf16, out_bf16, rows, ws, ws_bytes, stream, stage_events, ForwardMode());
}

int32_t moe_read_probe_sink_words(void) { return moe::read_probe_blocks(); }

moe_status moe_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !aligned(src, 16)) return fail(MOE_ERR_INVALID_ARG, "src must be a 16-byte aligned device pointer");
  if (bytes == 0 || bytes % 16) return fail(MOE_ERR_INVALID_ARG, "bytes=%zu must be a positive multiple of 16", bytes);
  if (!sink || !aligned(sink, 4)) return fail(MOE_ERR_INVALID_ARG, "sink must be a 4-byte aligned device pointer");
  const int blocks = moe::read_probe_blocks();
  if (overlaps(src, bytes, sink, (size_t)blocks * 4)) return fail(MOE_ERR_INVALID_ARG, "sink overlaps src");
  hipError_t e = moe::launch_read_probe(static_cast<const uint8_t*>(src), bytes, sink, blocks,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_status(e, "probe launch");
  return ok();
}

int32_t moe_num_stages(void) { return kNumStages; }

const char* moe_stage_name(int32_t i) { return (i >= 0 && i < kNumStages) ? kStageNames[i] : nullptr; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
