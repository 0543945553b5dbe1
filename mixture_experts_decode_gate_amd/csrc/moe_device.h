// Device-side helpers shared by the routed-MoE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kChunk = 2048;        // K columns one wave covers per pass: 64 lanes x 32 columns
constexpr int kChunkUnits = 256;    // 16-byte bf16 units per chunk (2048 * 2 B / 16 B)
constexpr int kMaxRows = 16;
constexpr int kMaxIds = 128;
constexpr int kSharedSlot = 128;    // slot table index of the shared expert
constexpr int kNumSlots = 129;

// Weight pointers of one union slot (a routed expert, or the shared expert at
// kSharedSlot), resolved once per call so the sweeps need a single load.
struct SlotInfo {
  const uint8_t* gate_packed;
  const uint8_t* gate_scales;
  const uint8_t* up_packed;
  const uint8_t* up_scales;
  const uint8_t* down_packed;
  const uint8_t* down_scales;
  float gate_scale2;
  float up_scale2;
  float down_scale2;
  int32_t inter;      // rows of gate/up, columns of down
  uint32_t row_mask;  // bit r: row r uses this slot
  int32_t expert;     // expert id, -1 for the shared expert
  uint8_t pair[kMaxRows];  // pair index of (this slot, row r) where row r uses the slot
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Round to nearest even; inputs are finite.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Two E2M1 codes (byte SEL of w, low nibble first) -> two bf16 values.  The
// hardware conversion is exact: every E2M1 value is a bf16 value.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}

// OCP E4M3FN byte SEL of w -> fp32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// DPP lane move: lanes outside ROW_MASK read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)src, CTRL, ROW_MASK, 0xF, false);
}

// Sum over the 64 lanes with DPP: pairs, quads, half rows, rows (16 lanes),
// then row 1 += row 0 and row 3 += row 2 (row_bcast:15), and rows 2-3 +=
// lane 31 (row_bcast:31).  Lane 63 ends with the total, which is returned to
// every lane.  The order of additions is fixed, so the result is
// deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += __builtin_bit_cast(float, dpp_u32<0xB1, 0xF>(__builtin_bit_cast(uint32_t, v)));   // quad_perm [1,0,3,2]
  v += __builtin_bit_cast(float, dpp_u32<0x4E, 0xF>(__builtin_bit_cast(uint32_t, v)));   // quad_perm [2,3,0,1]
  v += __builtin_bit_cast(float, dpp_u32<0x141, 0xF>(__builtin_bit_cast(uint32_t, v)));  // row_half_mirror
  v += __builtin_bit_cast(float, dpp_u32<0x140, 0xF>(__builtin_bit_cast(uint32_t, v)));  // row_mirror
  v += __builtin_bit_cast(float, dpp_u32<0x142, 0xA>(__builtin_bit_cast(uint32_t, v)));  // row_bcast:15
  v += __builtin_bit_cast(float, dpp_u32<0x143, 0xC>(__builtin_bit_cast(uint32_t, v)));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// wave_sum of N independent values, step by step, so each DPP step of one
// value fills the hazard slots of the others.  Same addition order as
// wave_sum for every value.  The totals are valid in lane 63 only.
template <int N>
__device__ __forceinline__ void wave_sum_lane63_n(float (&v)[N]) {
#define MOE_SUM_STEP(CTRL, MASK)                                                                   \
  _Pragma("unroll") for (int i = 0; i < N; ++i) v[i] += __builtin_bit_cast(                        \
      float, dpp_u32<CTRL, MASK>(__builtin_bit_cast(uint32_t, v[i])));
  MOE_SUM_STEP(0xB1, 0xF)
  MOE_SUM_STEP(0x4E, 0xF)
  MOE_SUM_STEP(0x141, 0xF)
  MOE_SUM_STEP(0x140, 0xF)
  MOE_SUM_STEP(0x142, 0xA)
  MOE_SUM_STEP(0x143, 0xC)
#undef MOE_SUM_STEP
}

// The same, with the totals broadcast to every lane.
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
  wave_sum_lane63_n<N>(v);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[i]), 63));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)b);
  const uint64_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xB1, 0xF>(v);
  v += dpp_f64<0x4E, 0xF>(v);
  v += dpp_f64<0x141, 0xF>(v);
  v += dpp_f64<0x140, 0xF>(v);
  v += dpp_f64<0x142, 0xA>(v);
  v += dpp_f64<0x143, 0xC>(v);
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

// wave_sum(double) of N independent values, step by step (same addition
// order as wave_sum for every value).
template <int N>
__device__ __forceinline__ void wave_sum_n(double (&v)[N]) {
#define MOE_SUM_STEP64(CTRL, MASK) \
  _Pragma("unroll") for (int i = 0; i < N; ++i) v[i] += dpp_f64<CTRL, MASK>(v[i]);
  MOE_SUM_STEP64(0xB1, 0xF)
  MOE_SUM_STEP64(0x4E, 0xF)
  MOE_SUM_STEP64(0x141, 0xF)
  MOE_SUM_STEP64(0x140, 0xF)
  MOE_SUM_STEP64(0x142, 0xA)
  MOE_SUM_STEP64(0x143, 0xC)
#undef MOE_SUM_STEP64
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v[i]);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    v[i] = __builtin_bit_cast(double, (hi << 32) | lo);
  }
}

// Lane moves past a quad: ds_swizzle in bit-mask mode (lane l reads lane
// l ^ M within its 32-lane half) and ds_bpermute (lane l reads lane l ^ 32).
template <int M>
__device__ __forceinline__ float swizzle_xor(float v) {
  static_assert(M > 0 && M < 32, "ds_swizzle exchanges within 32 lanes");
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), (M << 10) | 0x1F));
}
__device__ __forceinline__ float xor32_lane(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

// Sum over the 64 lanes of four values at once: lane l ends with the total of
// value sum4_value(l) = 2 (l & 1) + ((l >> 1) & 1).  Across lane pairs each
// lane keeps two of the values and receives the partner's copy of them, across
// quads one; the remaining steps are a butterfly on that one value (lanes
// l ^ 4, 8, 16, 32).  Each value's additions form the same xor tree over the
// lanes whatever the other values hold, and every lane with the same value
// index ends with the same bits.
__device__ __forceinline__ int sum4_value(int lane) { return 2 * (lane & 1) + ((lane >> 1) & 1); }

__device__ __forceinline__ float wave_sum4_scatter(const float (&v)[4], int lane) {
  const bool p = lane & 1, q = lane & 2;
  const float k0 = p ? v[2] : v[0], k1 = p ? v[3] : v[1];
  const float s0 = p ? v[0] : v[2], s1 = p ? v[1] : v[3];
  const float a0 = k0 + __builtin_bit_cast(float, dpp_u32<0xB1, 0xF>(__builtin_bit_cast(uint32_t, s0)));
  const float a1 = k1 + __builtin_bit_cast(float, dpp_u32<0xB1, 0xF>(__builtin_bit_cast(uint32_t, s1)));
  const float kq = q ? a1 : a0, sq = q ? a0 : a1;
  float b = kq + __builtin_bit_cast(float, dpp_u32<0x4E, 0xF>(__builtin_bit_cast(uint32_t, sq)));
  b += swizzle_xor<4>(b);
  b += swizzle_xor<8>(b);
  b += swizzle_xor<16>(b);
  b += xor32_lane(b, lane);
  return b;
}

// The first two steps of wave_sum(double) on N independent values: every lane
// of a quad ends with the quad's sum (both additions are commutative, so the
// four lanes hold the same bits).
template <int N>
__device__ __forceinline__ void quad_sum_n(double (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f64<0xB1, 0xF>(v[i]);  // quad_perm [1,0,3,2]
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f64<0x4E, 0xF>(v[i]);  // quad_perm [2,3,0,1]
}

// Sum over each DPP row of 16 lanes (the first four steps of wave_sum):
// every lane of the row ends with the row's sum.
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_f64<0x140, 0xF>(v);  // row_mirror
  return v;
}

// Maximum over the 64 lanes (same DPP pattern as wave_sum; lanes a step
// does not reach read 0, the identity), returned to every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  v = mx(v, dpp_u32<0xB1, 0xF>(v));   // quad_perm [1,0,3,2]
  v = mx(v, dpp_u32<0x4E, 0xF>(v));   // quad_perm [2,3,0,1]
  v = mx(v, dpp_u32<0x141, 0xF>(v));  // row_half_mirror
  v = mx(v, dpp_u32<0x140, 0xF>(v));  // row_mirror
  v = mx(v, dpp_u32<0x142, 0xA>(v));  // row_bcast:15
  v = mx(v, dpp_u32<0x143, 0xC>(v));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The wave's index within its block, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// A wave-uniform value read from LDS, moved to scalar registers, so the
// address arithmetic built on it runs on the scalar unit.
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* q) {
  const uint64_t v = reinterpret_cast<uint64_t>(q);
  const uint64_t lo = uniform_u32((uint32_t)v), hi = uniform_u32((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((hi << 32) | lo);
}

typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
typedef __attribute__((address_space(1))) const uint16_t global_u16;

// Weight bytes are read once per call: non-temporal global loads keep them
// from displacing reused data in the caches.
__device__ __forceinline__ u32x4 ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load((global_u32x4*)p);
}
__device__ __forceinline__ uint32_t ld_stream_u16(const uint8_t* p) {
  return __builtin_nontemporal_load((global_u16*)p);
}

// Decode 32 E2M1 codes (one 16-byte load) into 16 bf16 pairs, column order.
__device__ __forceinline__ void decode32(const u32x4& q, bf16x2 (&w)[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    w[d * 4 + 0] = e2m1x2<0>(q[d]);
    w[d * 4 + 1] = e2m1x2<1>(q[d]);
    w[d * 4 + 2] = e2m1x2<2>(q[d]);
    w[d * 4 + 3] = e2m1x2<3>(q[d]);
  }
}

// Dot of 32 decoded weights with 32 bf16 activations (4 units of 8), applying
// each 16-column block scale once: s0 * (cols 0..15) + s1 * (cols 16..31),
// accumulated into acc in that order.
__device__ __forceinline__ float dot32(const bf16x2 (&w)[16], const u32x4& x0, const u32x4& x1,
                                       const u32x4& x2, const u32x4& x3, float s0, float s1, float acc) {
  float p0 = 0.f, p1 = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) p0 = dot2(w[b], as_bf16x2(x0[b]), p0);
#pragma unroll
  for (int b = 0; b < 4; ++b) p0 = dot2(w[4 + b], as_bf16x2(x1[b]), p0);
#pragma unroll
  for (int b = 0; b < 4; ++b) p1 = dot2(w[8 + b], as_bf16x2(x2[b]), p1);
#pragma unroll
  for (int b = 0; b < 4; ++b) p1 = dot2(w[12 + b], as_bf16x2(x3[b]), p1);
  acc = __builtin_fmaf(s0, p0, acc);
  acc = __builtin_fmaf(s1, p1, acc);
  return acc;
}

// LDS position of natural 16-byte unit `u` (0..255) of a 2048-column chunk.
// Lane l reads units 4l..4l+3; storing unit u at (u & 3) * 64 + (u >> 2) makes
// each of the four reads cover 64 consecutive units (no bank conflicts).
__device__ __forceinline__ int swz_unit(int u) { return (u & 3) * 64 + (u >> 2); }

}  // namespace moe
