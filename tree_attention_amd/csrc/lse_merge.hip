// Log-sum-exp merge of the partial results (step a4).
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 2 part C, "Aggregation": the
// partial softmax results of the cached part and of the speculative part are
// joined exactly with a log-sum-exp step.  Here the cached part itself arrives
// as several prefix splits (the last of which has also taken in the tree
// keys), so the same merge reduces the splits.
//
// The same merge serves prefix-only attention (no tree part); a row whose
// partials are all empty (empty prefix) gets o = 0 and lse = -inf.
//
// For one output row with partials (o_s, l_s), l_s = log2 of the partial sum:
//   M = max_s l_s,  w_s = 2^(l_s - M),  Z = sum_s w_s,
//   o = sum_s (w_s / Z) o_s,  lse = ln 2 * (M + log2 Z).
//
// One wavefront per output row (b, h, i).  Lane s first loads the lse (and,
// on the bf16 path, the scale) of partial s, 64 partials at a time (the
// first 64 together with the prefix length, and kept in registers); the
// wavefront reduces max and sum across lanes and forms each partial's weight
// in its lane.  Then every lane owns D/64 consecutive features: per partial it
// reads them (one coalesced row read per partial, several partials in flight)
// and adds them with the partial's weight, read from lane s as a scalar.  The
// order of additions is fixed, so the result is bitwise deterministic.
#include "ltree_internal.h"

namespace ltree {
namespace {

constexpr int kMergeWaves = 4;  // rows per workgroup
constexpr int kBatch = 64;      // partials per pass (one per lane)
constexpr int kUnroll = 8;      // partial rows in flight per lane

// Reductions over the wavefront without LDS round trips: the two halves and
// the two 16-lane groups of each half are paired by lane swaps, then each
// 16-lane row by rotations of 8, 4, 2 and 1 lanes (DPP).  Every pair combines
// the same two values in every lane (addition is commutative), so all lanes
// end with bitwise the same result.
template <int K>
__device__ inline float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + K, 0xf, 0xf, false));
}
__device__ inline float wave_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
__device__ inline float wave_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  return v + row_ror<1>(v);
}

// lane s's value as a wavefront-uniform scalar
__device__ inline float lane_value(float v, int s) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), s));
}

// The D/64 features of partial row pr owned by lane j: fp32, or int16 snorm
// values (the row's scale is applied through the weight).
template <int D, bool SNORM>
__device__ inline void load_part(const void* o_part, size_t pr, int j, float (&v)[D / 64]) {
  constexpr int FPL = D / 64;
  if constexpr (SNORM) {
    const int16_t* p = static_cast<const int16_t*>(o_part) + pr * D + j * FPL;
    if constexpr (FPL == 2) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      v[0] = static_cast<float>(static_cast<int16_t>(u & 0xffffu));
      v[1] = static_cast<float>(static_cast<int16_t>(u >> 16));
    } else {
      v[0] = static_cast<float>(*p);
    }
  } else {
    const float* p = static_cast<const float*>(o_part) + pr * D + j * FPL;
#pragma unroll
    for (int f = 0; f < FPL; ++f) v[f] = p[f];
  }
}

template <int D, bool SNORM>
__global__ __launch_bounds__(64 * kMergeWaves) void lse_merge_kernel(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ seq_lens,
    const void* __restrict__ o_part,
    const float* __restrict__ scale_part, const float* __restrict__ lse_part,
    float* __restrict__ o, float* __restrict__ lse, int B, int T, int Hq, int Hkv, int G, int R,
    int chunk, int slots, int max_prefix_len, int window, int seq_cap) {
  constexpr int FPL = D / 64;  // features per lane
  const int j = threadIdx.x & 63;
  // rows are ordered (b, h, i) so the lse writes [B, Hq, T] are contiguous;
  // B * Hq * T < 2^31 is checked by the host
  const unsigned row = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= static_cast<unsigned>(B) * Hq * T) return;  // whole wavefronts
  const unsigned i = row % T;
  const unsigned bh = row / T;
  const unsigned h = bh % Hq;
  const unsigned b = bh / Hq;
  const unsigned g = h / G;
  const unsigned r = i * G + (h % G);
  float* orow = o + ((static_cast<size_t>(b) * T + i) * Hq + h) * D + j * FPL;
  float* lrow = lse + (static_cast<size_t>(b) * Hq + h) * T + i;

  const size_t base = static_cast<size_t>(b * Hkv + g) * slots;
  auto part_row = [&](int s) { return (base + s) * R + r; };
  // the first kBatch partials' lse and scale, loaded together with the
  // prefix length (slots below `slots` lie inside the workspace; what lies
  // past the last partial is dropped below)
  const bool pre = j < slots && j < kBatch;
  float l0 = pre ? lse_part[part_row(j)] : -INFINITY;
  float sc0 = (SNORM && pre) ? scale_part[part_row(j)] : 0.f;

  int start, n;
  const int L = seq_lens != nullptr ? seq_lens[b] : offsets[b + 1] - offsets[b];
  const float nan = __builtin_nanf("");
  if (!key_range(L, window, max_prefix_len, seq_cap, &start, &n)) {
    // The prefix-length table disagrees with max_prefix_len: fail loudly.
#pragma unroll
    for (int f = 0; f < FPL; ++f) orow[f] = nan;
    if (j == 0) *lrow = nan;
    return;
  }
  // one partial per prefix split, the last of which also covers the tree
  // keys; one tree-only partial when the prefix is empty
  const int nparts = n == 0 ? 1 : (n + chunk - 1) / chunk;
  if (j >= nparts) {
    l0 = -INFINITY;
    sc0 = 0.f;
  }

  // max and sum of 2^lse over all partials; a NaN partial (a paged split
  // with a page outside the pool) makes the row NaN
  float mx = l0;
  bool bad = l0 != l0;
  for (int s0 = kBatch; s0 < nparts; s0 += kBatch) {
    if (s0 + j < nparts) {
      const float l = lse_part[part_row(s0 + j)];
      bad = bad || l != l;
      mx = fmaxf(mx, l);
    }
  }
  if (__any(bad)) {
#pragma unroll
    for (int f = 0; f < FPL; ++f) orow[f] = nan;
    if (j == 0) *lrow = nan;
    return;
  }
  mx = wave_max(mx);
  if (mx == -INFINITY) {
    // no key at all (prefix-only attention over an empty prefix): the
    // softmax of an empty set, taken as o = 0 and lse = -inf
#pragma unroll
    for (int f = 0; f < FPL; ++f) orow[f] = 0.f;
    if (j == 0) *lrow = -INFINITY;
    return;
  }
  float z = exp2f(l0 - mx);
  for (int s0 = kBatch; s0 < nparts; s0 += kBatch) {
    if (s0 + j < nparts) z += exp2f(lse_part[part_row(s0 + j)] - mx);
  }
  z = wave_sum(z);
  const float inv_z = 1.f / z;

  float acc[FPL];
#pragma unroll
  for (int f = 0; f < FPL; ++f) acc[f] = 0.f;
  for (int s0 = 0; s0 < nparts; s0 += kBatch) {
    const int n = min(kBatch, nparts - s0);
    // this lane's weight: partial s0 + j
    float wl = 0.f;
    if (s0 == 0) {
      wl = exp2f(l0 - mx) * inv_z;
      if constexpr (SNORM) wl *= sc0 * (1.f / 32767.f);
    } else if (j < n) {
      const size_t pr = part_row(s0 + j);
      wl = exp2f(lse_part[pr] - mx) * inv_z;
      if constexpr (SNORM) wl *= scale_part[pr] * (1.f / 32767.f);
    }
    int s = 0;
    for (; s + kUnroll <= n; s += kUnroll) {
      float v[kUnroll][FPL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) load_part<D, SNORM>(o_part, part_row(s0 + s + u), j, v[u]);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float w = lane_value(wl, s + u);
#pragma unroll
        for (int f = 0; f < FPL; ++f) acc[f] = fmaf(w, v[u][f], acc[f]);
      }
    }
    for (; s < n; ++s) {
      float v[FPL];
      load_part<D, SNORM>(o_part, part_row(s0 + s), j, v);
      const float w = lane_value(wl, s);
#pragma unroll
      for (int f = 0; f < FPL; ++f) acc[f] = fmaf(w, v[f], acc[f]);
    }
  }
#pragma unroll
  for (int f = 0; f < FPL; ++f) orow[f] = acc[f];
  if (j == 0) *lrow = (mx + log2f(z)) * 0.6931471805599453f;
}

template <int D, bool SNORM>
void launch_typed(const Plan& p, dim3 grid, const int32_t* offsets, const int32_t* seq_lens,
                  const void* o_part,
                  const float* scale_part, const float* lse_part, float* o, float* lse,
                  hipStream_t stream) {
  hipLaunchKernelGGL((lse_merge_kernel<D, SNORM>), grid, dim3(64 * kMergeWaves), 0, stream,
                     offsets, seq_lens, o_part, scale_part, lse_part, o, lse, p.B, p.T, p.Hq, p.Hkv, p.G,
                     p.R, p.chunk, p.slots, p.max_prefix_len, p.window, p.seq_cap);
}

}  // namespace

hipError_t launch_merge(const Plan& p, bool snorm, const int32_t* offsets,
                        const int32_t* seq_lens, const void* o_part, const float* scale_part,
                        const float* lse_part, float* o, float* lse, hipStream_t stream) {
  const long rows = static_cast<long>(p.B) * p.Hq * p.T;
  const dim3 grid(static_cast<unsigned>((rows + kMergeWaves - 1) / kMergeWaves));
  if (p.D == 128) {
    if (snorm) {
      launch_typed<128, true>(p, grid, offsets, seq_lens, o_part, scale_part, lse_part, o, lse, stream);
    } else {
      launch_typed<128, false>(p, grid, offsets, seq_lens, o_part, scale_part, lse_part, o, lse, stream);
    }
  } else {
    if (snorm) {
      launch_typed<64, true>(p, grid, offsets, seq_lens, o_part, scale_part, lse_part, o, lse, stream);
    } else {
      launch_typed<64, false>(p, grid, offsets, seq_lens, o_part, scale_part, lse_part, o, lse, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace ltree
