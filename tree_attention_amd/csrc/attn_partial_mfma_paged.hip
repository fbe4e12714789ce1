// Partial attention on MFMA: the paged-cache variants (whole 64-key tiles
// per page, or rows addressed lane by lane), trees up to and above 64 nodes.
#include "attn_partial_mfma_impl.h"

namespace ltree {

hipError_t launch_mfma_paged(bool big, bool lane_paged, int D, int tpw, dim3 grid, PartialArgs a,
                             hipStream_t s) {
  if (lane_paged) {
    return big ? launch_dd<false, true, 2>(D, tpw, grid, a, s)
               : launch_dd<false, false, 2>(D, tpw, grid, a, s);
  }
  return big ? launch_dd<false, true, 1>(D, tpw, grid, a, s)
             : launch_dd<false, false, 1>(D, tpw, grid, a, s);
}

}  // namespace ltree
