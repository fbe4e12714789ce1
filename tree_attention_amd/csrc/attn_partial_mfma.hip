// Partial attention on MFMA for bf16 inputs (steps a2 and a3): the launch
// plan and the verification variants over a packed cache.  The kernel and
// its description are in attn_partial_mfma_impl.h.
#include "attn_partial_mfma_impl.h"

namespace ltree {

hipError_t launch_partials_mfma(const Plan& p, PartialArgs a, hipStream_t stream) {
  // Row blocking: at most kMaxTPW tiles of 16 rows per wave, 8 waves.  Fewer
  // row tiles per wave (more workgroups, each re-reading its split's keys)
  // when the (sequence, KV head, split) workgroups alone would leave compute
  // units idle: the smallest count whose grid still fits the chip once.
  const int tiles = (p.R + 15) / 16;
  const long units = static_cast<long>(p.B) * p.Hkv * p.slots;
  const int cus = device_cu_count();
  int max_tpw = kMaxTPW;
  for (int t = 1; t < kMaxTPW; ++t) {
    if (units * ((tiles + kWaves * t - 1) / (kWaves * t)) <= cus) {
      max_tpw = t;
      break;
    }
  }
  const int row_blocks = (tiles + kWaves * max_tpw - 1) / (kWaves * max_tpw);
  const int tiles_per_block = (tiles + row_blocks - 1) / row_blocks;
  const int tpw = (tiles_per_block + kWaves - 1) / kWaves;
  a.rows_per_wg = 16 * tiles_per_block;
  a.row_blocks = (p.R + a.rows_per_wg - 1) / a.rows_per_wg;
  const dim3 grid(p.Hkv, p.slots, p.B * a.row_blocks);
  const bool big = a.T > 64;
  // a window starts at any key, so over a paged cache its rows go by lane;
  // whole 64-key tiles per page when the page size allows
  const bool paged = a.block_table != nullptr;
  const bool lane_paged = paged && (a.window > 0 || a.page_size % kTile != 0);
  if (a.window > 0) return launch_mfma_window(big, lane_paged, p.D, tpw, grid, a, stream);
  if (a.kstride != a.Hkv * p.D || a.vstride != a.Hkv * p.D) {
    return launch_mfma_strided(big, p.D, tpw, grid, a, stream);
  }
  if (paged) return launch_mfma_paged(big, lane_paged, p.D, tpw, grid, a, stream);
  return launch_mfma_plain(big, p.D, tpw, grid, a, stream);
}

hipError_t launch_mfma_plain(bool big, int D, int tpw, dim3 grid, PartialArgs a, hipStream_t s) {
  return big ? launch_dd<false, true, 0>(D, tpw, grid, a, s)
             : launch_dd<false, false, 0>(D, tpw, grid, a, s);
}

}  // namespace ltree
