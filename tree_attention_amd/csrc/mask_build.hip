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
#include <climits>

#include "ltree_internal.h"

namespace ltree {
namespace {

__device__ inline uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl(static_cast<uint32_t>(v), src);
  const uint32_t hi = __shfl(static_cast<uint32_t>(v >> 32), src);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

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

  for (int b = wave; b < B; b += nwaves) {
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

}  // namespace

hipError_t launch_mask_build(const int32_t* parent, int B, int T, uint64_t* mask,
                             int32_t* status, hipStream_t stream) {
  // One workgroup: the status word needs the minimum over all trees, and the
  // mask is built once per verification step, so B trees per 16 waves is ample.
  const int waves = B < 16 ? B : 16;
  hipLaunchKernelGGL(mask_build_kernel, dim3(1), dim3(64 * waves), 0, stream, parent, B, T,
                     mask, status);
  return hipGetLastError();
}

}  // namespace ltree
