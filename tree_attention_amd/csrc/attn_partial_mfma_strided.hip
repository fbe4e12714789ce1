// Partial attention on MFMA: the verification variants over a prefix cache
// whose K and V rows sit at the caller's strides (tree rows stay packed).
#include "attn_partial_mfma_impl.h"

namespace ltree {

hipError_t launch_mfma_strided(bool big, int D, int tpw, dim3 grid, PartialArgs a, hipStream_t s) {
  return big ? launch_dd<false, true, 0, true>(D, tpw, grid, a, s)
             : launch_dd<false, false, 0, true>(D, tpw, grid, a, s);
}

}  // namespace ltree
