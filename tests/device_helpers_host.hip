// Host-side checks of the plain bit-arithmetic helpers of the routing kernels
// (moe_common.h), each against a bit-by-bit or arithmetic reference written
// here.  Built and run by test_device_helpers_host.py; prints one summary line
// and exits non-zero on any mismatch.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "moe_common.h"

using namespace moe;

static long g_fails = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      if (g_fails++ < 10) {              \
        std::printf("mismatch: ");       \
        std::printf(__VA_ARGS__);        \
        std::printf("\n");               \
      }                                  \
    }                                    \
  } while (0)

static bool slot_bit(const Slots128& s, int t) { return t < 64 ? (s.lo >> t) & 1u : (s.hi >> (t - 64)) & 1u; }

static uint32_t bits_of_float(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
static float float_of_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int main() {
  // t / k for every slot index t < 128 and every k <= 128 (the row of slot t).
  long n_div = 0;
  for (int k = 1; k <= 128; ++k) {
    const uint32_t m = small_div_magic(k);
    for (int t = 0; t < 128; ++t, ++n_div) CHECK(small_div(t, m) == t / k, "small_div(%d) k=%d", t, k);
  }

  // bit_range64 for every pair of bounds in [-70, 140), both sides clamped.
  long n_range = 0;
  for (int lo = -70; lo < 140; ++lo)
    for (int hi = -70; hi < 140; ++hi, ++n_range) {
      uint64_t ref = 0;
      for (int b = 0; b < 64; ++b)
        if (b >= lo && b < hi) ref |= 1ull << b;
      CHECK(bit_range64(lo, hi) == ref, "bit_range64(%d, %d)", lo, hi);
    }

  // slot_first over every window [a, a + k) with a + k <= 128 of random slot
  // sets: dense, sparse, one word empty, a single slot in the upper word.
  std::mt19937_64 g(20240611);
  long n_slot = 0;
  for (int it = 0; it < 1200; ++it) {
    Slots128 s{g(), g()};
    if (it % 3 == 0) {
      s.lo &= g() & g() & g();
      s.hi &= g() & g() & g();
    }
    if (it % 5 == 0) s.lo = 0;
    if (it % 7 == 0) s.hi = 0;
    if (it % 11 == 0) s = Slots128{0ull, 1ull << (g() % 64)};
    for (int k = 1; k <= 128; ++k)
      for (int a = 0; a + k <= 128; ++a, ++n_slot) {
        int ref = -1;
        for (int t = a; t < a + k; ++t)
          if (slot_bit(s, t)) {
            ref = t;
            break;
          }
        CHECK(slot_first(s, a, k) == ref, "slot_first(a=%d, k=%d) set %d", a, k, it);
      }
  }

  // key_bits along the non-NaN floats in increasing order (-inf .. -0, then
  // +0 .. +inf; every float near the ends, near zero and near the smallest
  // normals, every 251st elsewhere): keys strictly increase and are never 0,
  // and key_float inverts key_bits.  Ordinal o runs over that order.
  const uint64_t last = 2ull * 0x7F800000ull + 1ull;  // +inf
  auto bits_at = [](uint64_t o) -> uint32_t {
    return o <= 0x7F800000ull ? (uint32_t)(0xFF800000ull - o) : (uint32_t)(o - 0x7F800001ull);
  };
  auto dense = [&](uint64_t o) {
    const uint64_t w = 1ull << 16, zero = 0x7F800001ull, nmin = 0x00800000ull;
    auto near = [&](uint64_t c) { return o + w > c && o < c + w; };
    return o < w || last - o < w || near(zero) || near(zero - nmin) || near(zero + nmin);
  };
  long n_key = 0;
  uint32_t prev = 0;
  for (uint64_t o = 0; o <= last; o += dense(o) ? 1 : 251, ++n_key) {
    const uint32_t b = bits_at(o);
    const uint32_t key = key_bits(float_of_bits(b));
    CHECK(key != 0u, "key_bits(0x%08x) is 0", b);
    CHECK(o == 0 || key > prev, "key_bits(0x%08x) not above the previous float's key", b);
    CHECK(bits_of_float(key_float(key)) == b, "key_float(key_bits(0x%08x))", b);
    prev = key;
  }
  CHECK(key_bits(float_of_bits(0x80000000u)) + 1u == key_bits(0.0f), "-0 and +0 are not neighbours");
  CHECK(key_bits(float_of_bits(0xFFFFFFFFu)) == 0u, "the all-ones NaN does not map to 0");

  std::printf("%s div=%ld range=%ld slot=%ld key=%ld fails=%ld\n", g_fails ? "FAIL" : "ok", n_div, n_range, n_slot,
              n_key, g_fails);
  return g_fails ? 1 : 0;
}
