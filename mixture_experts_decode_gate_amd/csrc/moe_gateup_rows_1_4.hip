// Gate+up sweep instances for 1..4 rows (a translation unit of its own so
// the instances compile in parallel).
#include "moe_gateup.h"

namespace moe {

hipError_t launch_gateup_rows_1_4(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                   StageEvents ev) {
  switch (rows) {
    case 1: return gateup_r<1>(p, nch, max_items, s, ev);
    case 2: return gateup_r<2>(p, nch, max_items, s, ev);
    case 3: return gateup_r<3>(p, nch, max_items, s, ev);
    case 4: return gateup_r<4>(p, nch, max_items, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
