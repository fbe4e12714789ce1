// Partial attention on MFMA: the sliding-window variants (packed cache, and
// paged with rows addressed lane by lane), trees up to and above 64 nodes.
#include "attn_partial_mfma_impl.h"

namespace ltree {

hipError_t launch_mfma_window(bool big, bool lane_paged, int D, int tpw, dim3 grid, PartialArgs a,
                              hipStream_t s) {
  if (lane_paged) {
    return big ? launch_dd<true, true, 2>(D, tpw, grid, a, s)
               : launch_dd<true, false, 2>(D, tpw, grid, a, s);
  }
  return big ? launch_dd<true, true, 0>(D, tpw, grid, a, s)
             : launch_dd<true, false, 0>(D, tpw, grid, a, s);
}

}  // namespace ltree
