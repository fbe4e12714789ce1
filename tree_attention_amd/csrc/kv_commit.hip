// KV-cache commit of the accepted draft tokens.
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", opening explanation: the target model
// checks the draft's proposals and keeps (writes down) the ones it accepts;
// section 3 "Wichtige Ergebnisse": about 3.5 to 4 tokens are accepted per
// verification pass.  The keys and values the verification computed for the
// accepted branch of the tree become part of the cached prefix for the next
// step, so their rows are copied from the tree buffers into the KV cache.
//
// Row j < n_accepted[b] of sequence b:
//   k_cache[dst_row[b] + j] = k_tree[b, accepted[b, j]]   (all KV heads)
//   v_cache[dst_row[b] + j] = v_tree[b, accepted[b, j]]
// Pure data movement, 16 bytes per lane; one workgroup per (sequence,
// accepted row).  A sequence whose arguments are out of range is not written
// and is reported in the status word.
#include "ltree_internal.h"

namespace ltree {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCommitThreads = 256;

// true when sequence b's accepted rows are all inside the tree and the cache
__device__ inline bool commit_ok(const int32_t* accepted, const int32_t* n_accepted,
                                 const int32_t* dst_row, int T, int cache_rows, int b) {
  const int n = n_accepted[b];
  const int d = dst_row[b];
  if (n < 0 || n > T || d < 0 || d > cache_rows - n) return false;
  for (int j = 0; j < n; ++j) {
    const int id = accepted[static_cast<size_t>(b) * T + j];
    if (id < 0 || id >= T) return false;
  }
  return true;
}

// grid (T, B): block (j, b) copies accepted row j of sequence b (if j < n_b).
// Block (0, 0) also writes the status: 0, or 1 + the first bad sequence.
__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(
    const char* __restrict__ k_tree, const char* __restrict__ v_tree,
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ n_accepted,
    const int32_t* __restrict__ dst_row, char* __restrict__ k_cache, char* __restrict__ v_cache,
    int B, int T, int row_bytes, int cache_rows, int32_t* __restrict__ status) {
  const int j = blockIdx.x, b = blockIdx.y;
  if (status != nullptr && j == 0 && b == 0) {
    __shared__ int first_bad;
    if (threadIdx.x == 0) first_bad = B;
    __syncthreads();
    for (int s = threadIdx.x; s < B; s += kCommitThreads) {
      if (!commit_ok(accepted, n_accepted, dst_row, T, cache_rows, s)) atomicMin(&first_bad, s);
    }
    __syncthreads();
    if (threadIdx.x == 0) *status = first_bad == B ? 0 : 1 + first_bad;
  }
  if (j >= n_accepted[b] || !commit_ok(accepted, n_accepted, dst_row, T, cache_rows, b)) return;
  const int node = accepted[static_cast<size_t>(b) * T + j];
  const size_t src = (static_cast<size_t>(b) * T + node) * row_bytes;
  const size_t dst = static_cast<size_t>(dst_row[b] + j) * row_bytes;
  // row_bytes is a multiple of 16 (D in {64, 128}, 2- or 4-byte elements)
  for (int o = threadIdx.x * 16; o < row_bytes; o += kCommitThreads * 16) {
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k_tree + src + o);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v_tree + src + o);
    *reinterpret_cast<u32x4*>(k_cache + dst + o) = kv;
    *reinterpret_cast<u32x4*>(v_cache + dst + o) = vv;
  }
}

}  // namespace

hipError_t launch_kv_commit(const void* k_tree, const void* v_tree, const int32_t* accepted,
                            const int32_t* n_accepted, const int32_t* dst_row, void* k_cache,
                            void* v_cache, int B, int T, int row_bytes, int cache_rows,
                            int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(kv_commit_kernel, dim3(T, B), dim3(kCommitThreads), 0, stream,
                     static_cast<const char*>(k_tree), static_cast<const char*>(v_tree), accepted,
                     n_accepted, dst_row, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), B, T, row_bytes, cache_rows, status);
  return hipGetLastError();
}

}  // namespace ltree
