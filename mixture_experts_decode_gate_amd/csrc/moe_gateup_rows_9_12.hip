// Gate+up sweep instances for 9..12 rows (a translation unit of its own so
// the instances compile in parallel).
#include "moe_gateup.h"

namespace moe {

hipError_t launch_gateup_rows_9_12(const SweepParams& p, int rows, int nch, int max_items, hipStream_t s,
                                   StageEvents ev) {
  switch (rows) {
    case 9: return gateup_r<9>(p, nch, max_items, s, ev);
    case 10: return gateup_r<10>(p, nch, max_items, s, ev);
    case 11: return gateup_r<11>(p, nch, max_items, s, ev);
    case 12: return gateup_r<12>(p, nch, max_items, s, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
