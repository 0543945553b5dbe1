// Gate+up sweep instances for 5..8 rows (a translation unit of its own so
// the instances compile in parallel).
#include "moe_gateup.h"

namespace moe {

hipError_t launch_gateup_rows_5_8(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                   StageEvents ev) {
  switch (rows) {
    case 5: return gateup_r<5>(p, nch, max_items, s, ev);
    case 6: return gateup_r<6>(p, nch, max_items, s, ev);
    case 7: return gateup_r<7>(p, nch, max_items, s, ev);
    case 8: return gateup_r<8>(p, nch, max_items, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
