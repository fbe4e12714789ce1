// Work planning and the numeric argument checks of libltree, in plain C++ (no
// device code), so that a host-only build can run them under sanitizers over
// extreme sizes.  The HIP side (ltree_api.hip) queries the device and launches.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace ltree {

// How one attention call is cut into work.  Derived only from the sizes, the
// prefix row strides and the device's compute-unit count, so the workspace
// size query and the calls that use the workspace agree on one device.
struct Plan {
  int B, T, Hq, Hkv, D, G, R;  // R = G*T query rows per (sequence, KV head)
  int max_prefix_len;
  int window;      // 0, or the sliding window W (then max_prefix_len = W - 1)
  int seq_cap;     // largest L_b the call may address (paged: the block table's reach)
  int chunk;       // prefix keys per split (multiple of 64)
  int max_chunks;  // ceil(max_prefix_len / chunk): prefix splits per (b, g)
  int slots;       // max(max_chunks, 1).  Slot s of sequence b holds prefix
                   // keys [s*chunk, min((s+1)*chunk, L_b)); its last
                   // non-empty slot (slot 0 when L_b = 0) also the T tree keys
  size_t o_part_off, scale_part_off, lse_part_off, bytes;  // workspace layout
};

// Page numbers of one split that the paged kernels hold in LDS: a split
// covers at most (kMaxSplitPages - 1) * page_size keys.
constexpr int kMaxSplitPages = 448;

// Largest prefix row stride (elements between consecutive keys of one KV
// head): a 64-key tile of one head is addressed with 32-bit byte offsets.
constexpr long kMaxRowStride = 1L << 24;

// Returns false when the sizes are invalid (the caller reports the status).
// cus: compute units of the device; the prefix is cut into enough splits
// that the KV heads of one sequence cover them once.
// window > 0: the prefix part of each sequence is at most its last window - 1
// keys, and max_prefix_len is taken as window - 1.
// page_size > 0: a paged prefix (any page size); splits are capped so their
// pages fit the kernels' LDS table.
// row_stride: the larger of the prefix K and V row strides in elements
// (0: packed rows, Hkv * D).
bool make_plan(int B, int T, int Hq, int Hkv, int D, int max_prefix_len, int cus, Plan* p,
               int window = 0, int page_size = 0, long row_stride = 0);

// The status (LTREE_OK, LTREE_ERR_INVALID_ARG, LTREE_ERR_UNSUPPORTED) of the
// sizes every attention call shares.
int check_sizes(int B, int T, int Hq, int Hkv, int D, int max_prefix_len);

// A paged prefix: pool of num_pages pages of page_size rows (Hkv * D elements
// of elt_bytes each), block table of max_pages_per_seq entries per sequence.
// window > 0 for the sliding-window call (max_prefix_len unused).  On
// success *pool_bytes32 is the pool's size when it is below 2^31 bytes, else 0,
// and *seq_cap the longest sequence the block table can address.
int check_paged(int elt_bytes, int Hkv, int D, int num_pages, int page_size, int max_pages_per_seq,
                int max_prefix_len, int window, uint32_t* pool_bytes32, int* seq_cap);

// Prefix row strides of a strided cache: each at least Hkv * D, a multiple of
// 8 elements (16-byte rows), at most kMaxRowStride.
int check_strides(int Hkv, int D, long k_row_stride, long v_row_stride);

}  // namespace ltree
