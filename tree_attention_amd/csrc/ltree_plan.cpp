// Work planning and numeric argument checks of libltree (see ltree_plan.h).
// Plain C++: built into the library by hipcc and, for the host tests, alone
// by g++ under address and undefined-behaviour sanitizers.
#include "ltree_plan.h"

#include <limits.h>

#include "ltree.h"

namespace ltree {

namespace {
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

bool make_plan(int B, int T, int Hq, int Hkv, int D, int max_prefix_len, int cus, Plan* p,
               int window, int page_size, long row_stride) {
  if (page_size < 0 || cus < 1) return false;
  if (window < 0 || window > LTREE_MAX_WINDOW || (window > 0 && window < T)) return false;
  if (window > 0) max_prefix_len = window - 1;
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_prefix_len < 0) return false;
  if (D != 64 && D != 128) return false;
  if (T > LTREE_MAX_TREE) return false;
  // output rows (b, h, i) are indexed with 32-bit integers in the merge
  // (B * Hq alone fits 64 bits; T <= 256)
  if (static_cast<long>(B) * Hq >= (1L << 31) / T + 1 ||
      static_cast<long>(B) * Hq * T >= (1L << 31)) {
    return false;
  }
  const long packed = static_cast<long>(Hkv) * D;
  if (row_stride == 0) row_stride = packed;
  if (row_stride < packed || row_stride > kMaxRowStride) return false;
  p->B = B;
  p->T = T;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->D = D;
  p->G = Hq / Hkv;
  p->R = p->G * T;
  p->max_prefix_len = max_prefix_len;
  p->window = window;
  p->seq_cap = INT_MAX;

  // Split size: enough prefix splits per KV head that the Hkv heads of one
  // sequence cover every compute unit once; never below 256 keys, so that a
  // split's partial output stays small next to the keys it reads (a window of
  // a few hundred keys, whose call is latency-bound, splits down to 64).
  const long per_head = (static_cast<long>(cus) + Hkv - 1) / Hkv;
  long chunk = (static_cast<long>(max_prefix_len) + per_head - 1) / per_head;
  chunk = (chunk + 63) / 64 * 64;
  const long min_chunk = window > 0 ? 64 : 256;
  if (chunk < min_chunk) chunk = min_chunk;
  // keys of one split are addressed with 32-bit element offsets
  const long cap = ((1L << 31) - 1) / row_stride / 64 * 64;
  if (chunk > cap) chunk = cap;
  // a paged split's page numbers fit the kernels' LDS table (a split that
  // starts inside a page touches one page more than it fills)
  if (page_size > 0 && chunk > static_cast<long>(kMaxSplitPages - 1) * page_size) {
    chunk = static_cast<long>(kMaxSplitPages - 1) * page_size / 64 * 64;
  }
  if (chunk < 64) return false;
  p->chunk = static_cast<int>(chunk);
  p->max_chunks = static_cast<int>((max_prefix_len + chunk - 1) / chunk);
  // the last split of a sequence also takes the tree keys; an empty prefix
  // still needs one partial for them
  p->slots = p->max_chunks > 0 ? p->max_chunks : 1;

  const size_t rows = static_cast<size_t>(B) * Hkv * p->slots * p->R;
  p->o_part_off = 0;
  p->scale_part_off = align_up(rows * D * sizeof(float), 256);
  p->lse_part_off = align_up(p->scale_part_off + rows * sizeof(float), 256);
  p->bytes = align_up(p->lse_part_off + rows * sizeof(float), 256);
  return true;
}

int check_sizes(int B, int T, int Hq, int Hkv, int D, int max_prefix_len) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_prefix_len < 0) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (T > LTREE_MAX_TREE || (D != 64 && D != 128)) return LTREE_ERR_UNSUPPORTED;
  // every flat index the kernels form from the query/output sizes fits in int
  // (B * Hq alone fits 64 bits; T * D <= 2^15)
  if (static_cast<long>(B) * Hq > ((1L << 31) - 1) / (static_cast<long>(T) * D)) {
    return LTREE_ERR_UNSUPPORTED;
  }
  return LTREE_OK;
}

int check_paged(int elt_bytes, int Hkv, int D, int num_pages, int page_size, int max_pages_per_seq,
                int max_prefix_len, int window, uint32_t* pool_bytes32, int* seq_cap) {
  if (page_size < 1 || num_pages < 1 || max_pages_per_seq < 1 || Hkv < 1 || D < 1) {
    return LTREE_ERR_INVALID_ARG;
  }
  const long reach = static_cast<long>(max_pages_per_seq) * page_size;
  if (window == 0 && (max_prefix_len < 0 || static_cast<long>(max_prefix_len) > reach)) {
    return LTREE_ERR_INVALID_ARG;
  }
  // page rows are addressed with 64-bit offsets; a page's rows with 32-bit ones
  if (static_cast<long>(page_size) * Hkv * D > (1L << 30)) return LTREE_ERR_UNSUPPORTED;
  // rows addressed lane by lane from the start of the pool (a page size that
  // is not a multiple of 64, or any window) use 32-bit byte offsets
  const long pool_bytes = static_cast<long>(num_pages) * page_size * Hkv * D * elt_bytes;
  const bool lane_rows = window > 0 || page_size % 64 != 0;
  if (lane_rows && pool_bytes >= (1L << 31)) return LTREE_ERR_UNSUPPORTED;
  *pool_bytes32 = static_cast<uint32_t>(pool_bytes < (1L << 31) ? pool_bytes : 0);
  *seq_cap = static_cast<int>(reach < INT_MAX ? reach : INT_MAX);
  return LTREE_OK;
}

int check_strides(int Hkv, int D, long k_row_stride, long v_row_stride) {
  const long packed = static_cast<long>(Hkv) * D;
  for (long s : {k_row_stride, v_row_stride}) {
    if (s < packed || s % 8 != 0) return LTREE_ERR_INVALID_ARG;
    if (s > kMaxRowStride) return LTREE_ERR_UNSUPPORTED;
  }
  return LTREE_OK;
}

}  // namespace ltree
