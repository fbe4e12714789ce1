// Ancestor-or-self bitmask of speculation trees (step a1).
//
// The tree mask of the speculative part: gist.science page "LongSpec:
// Long-Context Lossless Speculative Decoding with Efficient Drafting and
// Verification", section 2 part C ("Schnelle Tree Attention"), item 2 of the
// split, and section 1 item "Ineffiziente Verifikation".  A draft token sees
// itself and its ancestors.
//
// One wavefront per tree, one lane per node (T <= 64).  Pointer jumping: lane i
// keeps A_i = the nodes on its path from i up to (not including) J_i, starting
// with A_i = {i}, J_i = parent(i).  Each round sets A_i |= A_{J_i} and
// J_i = J_{J_i}, so after k rounds A_i spans 2^k path nodes; six rounds cover
// any path of a 64-node tree.  Reads of other lanes go through cross-lane
// shuffles, which see the values of the previous round.
//
// Trees of 65..256 nodes (W = ceil(T/64) words per row) take the same pointer
// jumping with one thread per node of a 256-thread workgroup, A_i held as W
// words, the previous round's values exchanged through LDS, and eight rounds.
//
// Up to 16 trees of at most 64 nodes take one workgroup, which also forms the
// status word (the smallest invalid entry over all trees).  More trees, or
// trees of more than 64 nodes, are spread over workgroups (16 trees, or one
// wide tree, each), and a one-wave kernel forms the status afterwards: the
// rows of a tree with an invalid entry are all zero, while row 0 of a valid
// tree always holds bit 0, so the first tree whose row 0 is zero is the first
// invalid one, and its parent entries give the first invalid index.
#include <algorithm>
#include <climits>

#include "ltree_internal.h"

namespace ltree {
namespace {

__device__ inline uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  const uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// status != nullptr only for a one-workgroup launch
__global__ __launch_bounds__(1024) void mask_build_kernel(const int32_t* __restrict__ parent,
                                                          int B, int T,
                                                          uint64_t* __restrict__ mask,
                                                          int32_t* __restrict__ status) {
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = INT_MAX;
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const bool node = lane < T;

  for (int b = blockIdx.x * nwaves + wave; b < B; b += gridDim.x * nwaves) {
    const size_t row0 = static_cast<size_t>(b) * T;
    int p = -1;
    bool bad = false;
    if (node) {
      p = parent[row0 + lane];
      bad = p < -1 || p >= lane;
    }
    const uint64_t bad_lanes = __ballot(bad);

    uint64_t anc = node ? (1ull << lane) : 0ull;
    int jump = (node && !bad) ? p : -1;
#pragma unroll
    for (int round = 0; round < 6; ++round) {
      const int src = jump >= 0 ? jump : lane;
      const uint64_t a = shfl_u64(anc, src);
      const int j2 = __shfl(jump, src);
      if (jump >= 0) {
        anc |= a;
        jump = j2;
      }
    }
    if (bad_lanes) {
      anc = 0;
      if (lane == 0) atomicMin(&first_bad, static_cast<int>(row0) + __ffsll(static_cast<unsigned long long>(bad_lanes)) - 1);
    }
    if (node) mask[row0 + lane] = anc;
  }

  __syncthreads();
  if (threadIdx.x == 0 && status != nullptr) {
    *status = first_bad == INT_MAX ? 0 : first_bad + 1;
  }
}

constexpr int kWideThreads = 256;  // nodes of the largest tree
constexpr int kWideWords = 4;      // mask words per row of the largest tree

// status != nullptr only for a one-workgroup launch
__global__ __launch_bounds__(kWideThreads) void mask_build_wide_kernel(
    const int32_t* __restrict__ parent, int B, int T, int W, uint64_t* __restrict__ mask,
    int32_t* __restrict__ status) {
  __shared__ uint64_t anc_s[kWideThreads][kWideWords];
  __shared__ int jump_s[kWideThreads];
  __shared__ int first_bad;
  const int i = threadIdx.x;
  if (i == 0) first_bad = INT_MAX;
  __syncthreads();
  const bool node = i < T;

  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const size_t row0 = static_cast<size_t>(b) * T;
    int p = -1;
    bool bad = false;
    if (node) {
      p = parent[row0 + i];
      bad = p < -1 || p >= i;
    }
    uint64_t anc[kWideWords] = {0ull, 0ull, 0ull, 0ull};
    if (node) anc[i >> 6] = 1ull << (i & 63);
    int jump = (node && !bad) ? p : -1;
#pragma unroll 1
    for (int round = 0; round < 8; ++round) {
#pragma unroll
      for (int w = 0; w < kWideWords; ++w) anc_s[i][w] = anc[w];
      jump_s[i] = jump;
      __syncthreads();
      if (jump >= 0) {  // an earlier node of the same tree
#pragma unroll
        for (int w = 0; w < kWideWords; ++w) anc[w] |= anc_s[jump][w];
        jump = jump_s[jump];
      }
      __syncthreads();
    }
    const bool tree_bad = __syncthreads_or(bad) != 0;
    if (bad) atomicMin(&first_bad, static_cast<int>(row0) + i);
    if (node) {
      for (int w = 0; w < W; ++w) mask[(row0 + i) * W + w] = tree_bad ? 0ull : anc[w];
    }
  }

  __syncthreads();
  if (i == 0 && status != nullptr) {
    *status = first_bad == INT_MAX ? 0 : first_bad + 1;
  }
}

// The status word after a build spread over workgroups (one wave): the
// first tree whose row 0 is zero, then its first invalid parent entry.
__global__ __launch_bounds__(64) void mask_status_kernel(const int32_t* __restrict__ parent, int B,
                                                         int T, int W,
                                                         const uint64_t* __restrict__ mask,
                                                         int32_t* __restrict__ status) {
  const int lane = threadIdx.x;
  int first = INT_MAX;
  for (int b = lane; b < B; b += 64) {
    if (mask[static_cast<size_t>(b) * T * W] == 0ull) {
      first = b;
      break;
    }
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) first = min(first, __shfl_xor(first, s));
  int st = 0;
  if (first != INT_MAX) {
    const size_t row0 = static_cast<size_t>(first) * T;
    int bad_i = INT_MAX;
    for (int i = lane; i < T; i += 64) {
      const int p = parent[row0 + i];
      if (p < -1 || p >= i) {
        bad_i = i;
        break;
      }
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) bad_i = min(bad_i, __shfl_xor(bad_i, s));
    st = static_cast<int>(row0) + bad_i + 1;
  }
  if (lane == 0) *status = st;
}

}  // namespace

hipError_t launch_mask_build(const int32_t* parent, int B, int T, uint64_t* mask,
                             int32_t* status, hipStream_t stream) {
  const int W = (T + 63) / 64;
  if (T <= 64 && B <= 16) {  // one workgroup, status formed in place
    hipLaunchKernelGGL(mask_build_kernel, dim3(1), dim3(64 * B), 0, stream, parent, B, T, mask,
                       status);
    return hipGetLastError();
  }
  if (T <= 64) {
    const int wgs = std::min((B + 15) / 16, 1024);
    hipLaunchKernelGGL(mask_build_kernel, dim3(wgs), dim3(1024), 0, stream, parent, B, T, mask,
                       static_cast<int32_t*>(nullptr));
  } else {
    hipLaunchKernelGGL(mask_build_wide_kernel, dim3(std::min(B, 4096)), dim3(kWideThreads), 0, stream,
                       parent, B, T, W, mask, static_cast<int32_t*>(nullptr));
  }
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && status != nullptr) {
    hipLaunchKernelGGL(mask_status_kernel, dim3(1), dim3(64), 0, stream, parent, B, T, W, mask,
                       status);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace ltree
