// Log-sum-exp merge of the partial results (step a4).
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 2 part C, "Aggregation": the
// partial softmax results of the cached part and of the speculative part are
// joined exactly with a log-sum-exp step.  Here the cached part itself arrives
// as several prefix splits, so the same merge also reduces the splits.
//
// For one output row with partials (o_s, l_s), l_s = log2 of the partial sum:
//   M = max_s l_s,  w_s = 2^(l_s - M),  Z = sum_s w_s,
//   o = sum_s (w_s / Z) o_s,  lse = ln 2 * (M + log2 Z).
//
// One wavefront per output row (b, h, i).  Lanes first scan the partial lse
// values (max, then sum), then read the partial outputs one split at a time in
// a fixed order, so the result is bitwise deterministic.  Each lane owns D/64
// consecutive features, so every partial row is one coalesced 4*D-byte read.
#include "ltree_internal.h"

namespace ltree {
namespace {

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(
    const int32_t* __restrict__ offsets, const float* __restrict__ o_part,
    const float* __restrict__ lse_part, float* __restrict__ o, float* __restrict__ lse, int B,
    int T, int Hq, int Hkv, int G, int R, int chunk, int max_chunks, int slots,
    int max_prefix_len) {
  constexpr int E = D / 64;  // features per lane
  const int lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<long>(B) * Hq * T) return;
  // rows are ordered (b, h, i) so the lse writes [B, Hq, T] are contiguous
  const int i = static_cast<int>(row % T);
  const int h = static_cast<int>((row / T) % Hq);
  const int b = static_cast<int>(row / (static_cast<long>(T) * Hq));
  const int g = h / G;
  const int r = i * G + (h % G);

  float* orow = o + ((static_cast<size_t>(b) * T + i) * Hq + h) * D + lane * E;
  const int L = offsets[b + 1] - offsets[b];
  if (L < 0 || L > max_prefix_len) {
    // The prefix-length table disagrees with max_prefix_len: fail loudly.
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = __builtin_nanf("");
    if (lane == 0) lse[(static_cast<size_t>(b) * Hq + h) * T + i] = __builtin_nanf("");
    return;
  }
  const int npre = (L + chunk - 1) / chunk;
  const int nparts = npre + 1;  // prefix splits, then the tree partial
  const size_t base = static_cast<size_t>(b * Hkv + g) * slots;
  auto slot_of = [&](int s) { return s < npre ? s : max_chunks; };

  float mx = -INFINITY;
  for (int s = lane; s < nparts; s += 64) mx = fmaxf(mx, lse_part[(base + slot_of(s)) * R + r]);
  mx = wave_max(mx);
  float z = 0.f;
  for (int s = lane; s < nparts; s += 64) z += exp2f(lse_part[(base + slot_of(s)) * R + r] - mx);
  z = wave_sum(z);
  const float inv_z = 1.f / z;

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  int s = 0;
  // four partials in flight per step
  for (; s + 4 <= nparts; s += 4) {
    float w[4];
    float v[4][E];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t pr = (base + slot_of(s + u)) * R + r;
      w[u] = exp2f(lse_part[pr] - mx) * inv_z;
      const float* src = o_part + pr * D + lane * E;
#pragma unroll
      for (int e = 0; e < E; ++e) v[u][e] = src[e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(w[u], v[u][e], acc[e]);
  }
  for (; s < nparts; ++s) {
    const size_t pr = (base + slot_of(s)) * R + r;
    const float w = exp2f(lse_part[pr] - mx) * inv_z;
    const float* src = o_part + pr * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(w, src[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) orow[e] = acc[e];
  if (lane == 0) {
    lse[(static_cast<size_t>(b) * Hq + h) * T + i] = (mx + log2f(z)) * 0.6931471805599453f;
  }
}

}  // namespace

hipError_t launch_merge(const Plan& p, const int32_t* offsets, const float* o_part,
                        const float* lse_part, float* o, float* lse, hipStream_t stream) {
  const long rows = static_cast<long>(p.B) * p.Hq * p.T;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  if (p.D == 128) {
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(256), 0, stream, offsets, o_part,
                       lse_part, o, lse, p.B, p.T, p.Hq, p.Hkv, p.G, p.R, p.chunk,
                       p.max_chunks, p.slots, p.max_prefix_len);
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(256), 0, stream, offsets, o_part,
                       lse_part, o, lse, p.B, p.T, p.Hq, p.Hkv, p.G, p.R, p.chunk,
                       p.max_chunks, p.slots, p.max_prefix_len);
  }
  return hipGetLastError();
}

}  // namespace ltree
