// Gate+up sweep instances for 13..16 rows (a translation unit of its own so
// the instances compile in parallel).
#include "moe_gateup.h"

namespace moe {

hipError_t launch_gateup_rows_13_16(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                   StageEvents ev) {
  switch (rows) {
    case 13: return gateup_r<13>(p, nch, max_items, s, ev);
    case 14: return gateup_r<14>(p, nch, max_items, s, ev);
    case 15: return gateup_r<15>(p, nch, max_items, s, ev);
    case 16: return gateup_r<16>(p, nch, max_items, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
