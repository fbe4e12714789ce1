// Log-sum-exp merge of the partial results (step a4).
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 2 part C, "Aggregation": the
// partial softmax results of the cached part and of the speculative part are
// joined exactly with a log-sum-exp step.  Here the cached part itself arrives
// as several prefix splits (the last of which has also taken in the tree
// keys), so the same merge reduces the splits.
//
// For one output row with partials (o_s, l_s), l_s = log2 of the partial sum:
//   M = max_s l_s,  w_s = 2^(l_s - M),  Z = sum_s w_s,
//   o = sum_s (w_s / Z) o_s,  lse = ln 2 * (M + log2 Z).
//
// Each output row (b, h, i) is served by NSG groups of D/4 lanes; a lane owns
// four consecutive features, so every partial row is one coalesced read of 16
// bytes per lane.  Each group first scans all partial lse values (max, then
// sum), then accumulates its share of the partial outputs (splits q, q+NSG,
// ...) in a fixed order; the groups' sums are added in LDS in a fixed order,
// so the result is bitwise deterministic.  Splitting the partials over groups
// keeps several times more loads in flight than one group per row would.
#include "ltree_internal.h"

namespace ltree {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int LPR>
__device__ inline float group_max(float v) {
#pragma unroll
  for (int s = LPR / 2; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}

template <int LPR>
__device__ inline float group_sum(float v) {
#pragma unroll
  for (int s = LPR / 2; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

constexpr int kMergeThreads = 256;
constexpr int kSplitGroups = 4;  // lane groups sharing one output row

// Four features of partial row pr for lane j: fp32, or int16 snorm values
// times the row's scale.
template <int D, bool SNORM>
__device__ inline f32x4 load_part(const void* o_part, const float* scale_part, size_t pr, int j) {
  if constexpr (SNORM) {
    const s16x4 q = reinterpret_cast<const s16x4*>(static_cast<const int16_t*>(o_part) + pr * D)[j];
    const float sc = scale_part[pr] * (1.f / 32767.f);
    return (f32x4){static_cast<float>(q[0]), static_cast<float>(q[1]), static_cast<float>(q[2]),
                   static_cast<float>(q[3])} * sc;
  } else {
    return reinterpret_cast<const f32x4*>(static_cast<const float*>(o_part) + pr * D)[j];
  }
}

template <int D, bool SNORM>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(
    const int32_t* __restrict__ offsets, const void* __restrict__ o_part,
    const float* __restrict__ scale_part, const float* __restrict__ lse_part,
    float* __restrict__ o, float* __restrict__ lse, int B, int T, int Hq, int Hkv, int G, int R,
    int chunk, int slots, int max_prefix_len) {
  constexpr int LPR = D / 4;                             // lanes per group
  constexpr int NSG = kSplitGroups;
  constexpr int RPB = kMergeThreads / (LPR * NSG);       // rows per workgroup
  __shared__ f32x4 red[NSG - 1][RPB][LPR];

  const int j = threadIdx.x % LPR;                       // lane within the group
  const int q = (threadIdx.x / LPR) % NSG;               // split group
  const int rl = threadIdx.x / (LPR * NSG);              // row within the workgroup
  // rows are ordered (b, h, i) so the lse writes [B, Hq, T] are contiguous;
  // B * Hq * T < 2^31 is checked by the host
  const unsigned row = blockIdx.x * RPB + rl;
  const unsigned nrows = static_cast<unsigned>(B) * Hq * T;
  const bool valid = row < nrows;
  const unsigned i = valid ? row % T : 0;
  const unsigned bh = valid ? row / T : 0;
  const unsigned h = bh % Hq;
  const unsigned b = bh / Hq;
  const unsigned g = h / G;
  const unsigned r = i * G + (h % G);

  const int L = offsets[b + 1] - offsets[b];
  const bool bad = L < 0 || L > max_prefix_len;
  // one partial per prefix split, the last of which also covers the tree
  // keys; one tree-only partial when the prefix is empty
  const int nparts = bad || L == 0 ? 1 : (L + chunk - 1) / chunk;
  const size_t base = static_cast<size_t>(b * Hkv + g) * slots;
  auto part_row = [&](int s) { return (base + s) * R + r; };

  float mx = -INFINITY;
  for (int s = j; s < nparts; s += LPR) mx = fmaxf(mx, lse_part[part_row(s)]);
  mx = group_max<LPR>(mx);
  float z = 0.f;
  for (int s = j; s < nparts; s += LPR) z += exp2f(lse_part[part_row(s)] - mx);
  z = group_sum<LPR>(z);
  const float inv_z = 1.f / z;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;  // partials in flight per lane and step
  int s = q;
  for (; s + (U - 1) * NSG < nparts; s += U * NSG) {
    float w[U];
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t pr = part_row(s + u * NSG);
      w[u] = lse_part[pr];
      v[u] = load_part<D, SNORM>(o_part, scale_part, pr, j);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc += (exp2f(w[u] - mx) * inv_z) * v[u];
  }
  for (; s < nparts; s += NSG) {
    const size_t pr = part_row(s);
    acc += (exp2f(lse_part[pr] - mx) * inv_z) * load_part<D, SNORM>(o_part, scale_part, pr, j);
  }

  if (q > 0) red[q - 1][rl][j] = acc;
  __syncthreads();
  if (q > 0 || !valid) return;
#pragma unroll
  for (int k = 0; k < NSG - 1; ++k) acc += red[k][rl][j];
  f32x4* orow = reinterpret_cast<f32x4*>(o + ((static_cast<size_t>(b) * T + i) * Hq + h) * D) + j;
  float* lrow = lse + (static_cast<size_t>(b) * Hq + h) * T + i;
  if (bad) {
    // The prefix-length table disagrees with max_prefix_len: fail loudly.
    const float nan = __builtin_nanf("");
    *orow = (f32x4){nan, nan, nan, nan};
    if (j == 0) *lrow = nan;
    return;
  }
  *orow = acc;
  if (j == 0) *lrow = (mx + log2f(z)) * 0.6931471805599453f;
}

}  // namespace

template <int D, bool SNORM>
void launch_typed(const Plan& p, dim3 grid, const int32_t* offsets, const void* o_part,
                  const float* scale_part, const float* lse_part, float* o, float* lse,
                  hipStream_t stream) {
  hipLaunchKernelGGL((lse_merge_kernel<D, SNORM>), grid, dim3(kMergeThreads), 0, stream, offsets,
                     o_part, scale_part, lse_part, o, lse, p.B, p.T, p.Hq, p.Hkv, p.G, p.R,
                     p.chunk, p.slots, p.max_prefix_len);
}

hipError_t launch_merge(const Plan& p, bool snorm, const int32_t* offsets, const void* o_part,
                        const float* scale_part, const float* lse_part, float* o, float* lse,
                        hipStream_t stream) {
  const long rows = static_cast<long>(p.B) * p.Hq * p.T;
  const long rows_per_block = kMergeThreads / (p.D / 4 * kSplitGroups);
  const dim3 grid(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block));
  if (p.D == 128) {
    if (snorm) {
      launch_typed<128, true>(p, grid, offsets, o_part, scale_part, lse_part, o, lse, stream);
    } else {
      launch_typed<128, false>(p, grid, offsets, o_part, scale_part, lse_part, o, lse, stream);
    }
  } else {
    if (snorm) {
      launch_typed<64, true>(p, grid, offsets, o_part, scale_part, lse_part, o, lse, stream);
    } else {
      launch_typed<64, false>(p, grid, offsets, o_part, scale_part, lse_part, o, lse, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace ltree
