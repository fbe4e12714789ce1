// Internal declarations shared by the host API and the kernel files of libltree.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ltree.h"
#include "ltree_plan.h"

namespace ltree {

// The prefix keys sequence b's partials read, [start, start + n) of its L_b
// rows.  Without a window all of them; with a window W the last
// min(L_b, W - 1), the cache keys a token at the tree's first position can
// see.  False when L_b is out of range: negative, above seq_cap (what a paged
// call's block table can address), or (no window) above max_prefix_len.
__device__ inline bool key_range(int L, int window, int max_prefix_len, int seq_cap, int* start,
                                 int* n) {
  if (L < 0 || L > seq_cap || (window == 0 && L > max_prefix_len)) return false;
  *n = window > 0 ? min(L, window - 1) : L;
  *start = L - *n;
  return true;
}

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Arguments of the partial-attention kernels (steps 1 and 2).
//
// Workspace layout, written by the partial kernels and read by the merge:
//   o_part    [B][Hkv][slots][R][D] each partial normalised by its own sum:
//             fp32 (fp32 inputs), or int16 snorm values o / scale_part
//             (bf16 inputs; the region is sized for fp32)
//   scale_part[B][Hkv][slots][R]    fp32, the row's largest |o| (bf16 inputs)
//   lse_part  [B][Hkv][slots][R]    fp32, log2 of the partial's sum of
//                                   2^(scale*log2(e)*score), i.e. lse / ln 2
// Row r of (b, g) is tree node i = r / G of query head g*G + r % G.
struct PartialArgs {
  const void* q;
  const void* kp;
  const void* vp;
  const int32_t* offsets;
  const void* kt;
  const void* vt;
  const uint64_t* mask;
  void* o_part;
  float* scale_part;
  float* lse_part;
  int B, T, Hq, Hkv, G, R;
  int W;             // mask words per row, ceil(T / 64)
  int chunk, max_chunks, slots, max_prefix_len;
  int seq_cap;       // largest L_b the call may address
  int rows_per_wg, row_blocks;
  int has_tree;      // 0: prefix keys only (no tree part; the tree arguments are unused)
  int window;        // 0, or W: node i sees the last W - depth(i) prefix keys (and its branch)
  // prefix row strides in elements (key j, KV head g at row (off + j) * stride
  // + g * D); the packed layout has Hkv * D.  Tree rows are always packed.
  int kstride, vstride;
  // paged prefix (block_table != nullptr): kp/vp are page pools
  // [num_pages][page_size][Hkv][D]; key j of sequence b is row j % page_size
  // of page block_table[b * max_pages + j / page_size]; L_b = seq_lens[b]
  const int32_t* seq_lens;
  const int32_t* block_table;
  int page_size, max_pages, num_pages;
  int page_shift;    // log2(page_size) when it is a power of two, else -1
  uint32_t pool_bytes;  // bytes of one pool when page_size is not a multiple of 64 (< 4 GB)
  int simple_tpr;    // fp32 kernel: threads per query row (set by its launcher)
  float scale_log2;  // scale * log2(e)
  float headroom;    // 15 / scale_log2: raw-score margin of the lazy softmax reference
  float neg_inv_scale_log2;  // -1 / scale_log2
};

hipError_t launch_mask_build(const int32_t* parent, int B, int T, uint64_t* mask,
                             int32_t* status, hipStream_t stream);

// bf16 inputs, D in {64, 128}: MFMA kernel.
hipError_t launch_partials_mfma(const Plan& plan, PartialArgs args, hipStream_t stream);

// fp32 inputs (or any dtype, for checking): fp32 FMA kernel.
hipError_t launch_partials_simple(ltree_dtype dtype, const Plan& plan, PartialArgs args,
                                  hipStream_t stream);

hipError_t launch_kv_commit(const void* k_tree, const void* v_tree, const int32_t* accepted,
                            const int32_t* n_accepted, const int32_t* dst_row, void* k_cache,
                            void* v_cache, int B, int T, int row_bytes, int cache_rows,
                            int32_t* status, hipStream_t stream);

hipError_t launch_tree_rope(bool bf16, void* q, void* k_tree, const uint64_t* mask,
                            const int32_t* offsets, int B, int T, int Hq, int Hkv, int D,
                            double base, hipStream_t stream);

// snorm: o_part holds int16 snorm values with per-row scales (bf16 path).
// seq_lens != nullptr: L_b = seq_lens[b] (paged prefix), else offsets[b+1] - offsets[b].
hipError_t launch_merge(const Plan& plan, bool snorm, const int32_t* offsets,
                        const int32_t* seq_lens, const void* o_part, const float* scale_part,
                        const float* lse_part, float* o, float* lse, hipStream_t stream);

}  // namespace ltree
