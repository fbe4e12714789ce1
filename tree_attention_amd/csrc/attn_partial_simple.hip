// Partial attention with plain fp32 FMA arithmetic (steps a2 and a3), used for
// fp32 inputs, where the contraction is tiny and precision is the point.
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 2 part C: item 1 of the split
// (cached part: prefix keys, no mask) and item 2 (speculative part: tree keys,
// tree mask).  Each workgroup computes one partial: the softmax of its query
// rows over one prefix split, or over the tree tokens, normalised by its own
// sum, plus log2 of that sum.  The log-sum-exp merge joins the partials.
//
// Grid (Hkv, slots, B * row blocks); `tpr` threads per query row (a power of
// two up to 32, more when there are few rows, so that small problems still
// occupy the workgroup): each takes every tpr-th key with its own online
// softmax state, and the tpr states are joined by wavefront shuffles at the
// end.  Keys are staged 32 at a time in LDS as fp32 and read by every thread
// (broadcast reads).  The last prefix split of a sequence (slot 0 when its
// prefix is empty) continues over the tree keys.
#include "ltree_internal.h"

namespace ltree {
namespace {

template <typename Tin>
__device__ inline float to_f32(Tin x);
template <>
__device__ inline float to_f32<float>(float x) {
  return x;
}
template <>
__device__ inline float to_f32<__bf16>(__bf16 x) {
  return static_cast<float>(x);
}

constexpr int kKeysPerTile = 32;
constexpr int kThreadsWG = 256;

template <typename Tin, int D>
__global__ __launch_bounds__(kThreadsWG) void partial_simple_kernel(PartialArgs a) {
  __shared__ float ks[kKeysPerTile][D + 1];
  __shared__ float vs[kKeysPerTile][D + 1];

  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int slot = blockIdx.y;
  const int tpr = a.simple_tpr;                  // threads per row
  const int rows_per_wg = kThreadsWG / tpr;
  const int sub = tid % tpr;                     // this thread's share of the keys
  const int rblocks = (a.R + rows_per_wg - 1) / rows_per_wg;
  const int b = blockIdx.z / rblocks;
  const int rb = blockIdx.z % rblocks;
  const bool paged = a.block_table != nullptr;
  const int off0 = paged ? 0 : a.offsets[b];
  const int L = paged ? a.seq_lens[b] : a.offsets[b + 1] - off0;
  int start, n;
  if (!key_range(L, a.window, a.max_prefix_len, a.seq_cap, &start, &n)) return;  // the merge reports it
  // slot s: prefix keys start + [s*chunk, min((s+1)*chunk, n)); the last one
  // (slot 0 when n = 0) also the tree keys
  const int nparts = n > 0 ? (n + a.chunk - 1) / a.chunk : 1;
  if (slot >= nparts) return;
  const int k0 = slot * a.chunk;
  const int npk = max(0, min(a.chunk, n - k0));
  const bool tree = a.has_tree && slot == nparts - 1;
  // prefix rows at the caller's strides (a paged pool, and the tree, are packed)
  const size_t tstride = static_cast<size_t>(a.Hkv) * D;
  const size_t kstr = paged ? tstride : static_cast<size_t>(a.kstride);
  const size_t vstr = paged ? tstride : static_cast<size_t>(a.vstride);
  const size_t row0 = static_cast<size_t>(off0) + start + k0;
  const Tin* kp = static_cast<const Tin*>(a.kp) + row0 * kstr + static_cast<size_t>(g) * D;
  const Tin* vp = static_cast<const Tin*>(a.vp) + row0 * vstr + static_cast<size_t>(g) * D;
  const Tin* kt = static_cast<const Tin*>(a.kt) + (static_cast<size_t>(b) * a.T * a.Hkv + g) * D;
  const Tin* vt = static_cast<const Tin*>(a.vt) + (static_cast<size_t>(b) * a.T * a.Hkv + g) * D;

  const int r = rb * rows_per_wg + tid / tpr;
  const bool active = r < a.R;
  // paged prefix: row of key k (within the sequence) in the page pool; a page
  // outside the pool makes this partial NaN and nothing is read
  auto page_row = [&](int k) -> size_t {
    const int pg = a.block_table[static_cast<size_t>(b) * a.max_pages + k / a.page_size];
    return static_cast<size_t>(pg) * a.page_size + k % a.page_size;
  };
  if (paged) {
    bool bad = false;
    const int p0 = (start + k0) / a.page_size;
    const int np = npk > 0 ? (start + k0 + npk - 1) / a.page_size - p0 + 1 : 0;
    for (int k = tid; k < np; k += kThreadsWG) {
      const int pg = a.block_table[static_cast<size_t>(b) * a.max_pages + p0 + k];
      bad = bad || pg < 0 || pg >= a.num_pages;
    }
    if (__syncthreads_or(bad)) {
      if (active && sub == 0) a.lse_part[(static_cast<size_t>(b * a.Hkv + g) * a.slots + slot) * a.R + r] = __builtin_nanf("");
      return;
    }
  }
  const int i = active ? r / a.G : 0;
  const int h = g * a.G + (active ? r % a.G : 0);
  float qv[D];
  {
    const Tin* qp = static_cast<const Tin*>(a.q) + ((static_cast<size_t>(b) * a.T + i) * a.Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] = active ? to_f32(qp[d]) * a.scale_log2 : 0.f;
  }
  // this row's mask words (W per row)
  const uint64_t* mrow =
      a.mask != nullptr ? a.mask + (static_cast<size_t>(b) * a.T + i) * a.W : nullptr;
  int depth = 0;
  if (a.window > 0 && active) {
    for (int w = 0; w < a.W; ++w) depth += static_cast<int>(__popcll(mrow[w]));
  }
  // window W: this row sees prefix keys from key n - W + depth(i) of the range
  const int first = a.window > 0 ? n - a.window + depth - k0 : 0;

  float m = -INFINITY, l = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;

  // prefix keys (tiles 0 .. ptiles-1), then the tree keys (one more pass).
  // The elements of tile tt+1 are loaded into registers while tile tt is
  // computed, so each tile's memory latency hides behind the one before.
  const int ptiles = (npk + kKeysPerTile - 1) / kKeysPerTile;
  const int ttiles = tree ? (a.T + kKeysPerTile - 1) / kKeysPerTile : 0;
  const int ntiles = ptiles + ttiles;
  static_assert(kKeysPerTile * D % kThreadsWG == 0, "whole staging rounds");
  constexpr int kPer = kKeysPerTile * D / kThreadsWG;  // elements per thread and tile
  float kr[kPer], vr[kPer];
  auto fetch = [&](int tt) {
    const bool intree = tt >= ptiles;
    const int t0 = (intree ? tt - ptiles : tt) * kKeysPerTile;
    const int n = min(kKeysPerTile, (intree ? a.T : npk) - t0);
    const Tin* kb = intree ? kt : kp;  // (a paged prefix tile addresses the pools itself)
    const Tin* vb = intree ? vt : vp;
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int e = tid + it * kThreadsWG;
      const int j = e / D, d = e % D;
      const int key = t0 + min(j, n - 1);
      size_t koff = key * (intree ? tstride : kstr) + d;
      size_t voff = key * (intree ? tstride : vstr) + d;
      if (paged && !intree) {
        koff = voff = page_row(start + k0 + key) * tstride + static_cast<size_t>(g) * D + d;
        kb = static_cast<const Tin*>(a.kp);
        vb = static_cast<const Tin*>(a.vp);
      }
      kr[it] = to_f32(kb[koff]);
      vr[it] = to_f32(vb[voff]);
    }
  };
  if (ntiles > 0) fetch(0);
  for (int tt = 0; tt < ntiles; ++tt) {
    const bool intree = tt >= ptiles;
    const int t0 = (intree ? tt - ptiles : tt) * kKeysPerTile;
    const int n = min(kKeysPerTile, (intree ? a.T : npk) - t0);
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int e = tid + it * kThreadsWG;
      ks[e / D][e % D] = kr[it];
      vs[e / D][e % D] = vr[it];
    }
    __syncthreads();
    if (tt + 1 < ntiles) fetch(tt + 1);
    // tree keys t0 .. t0 + 31 lie in mask word t0 / 64
    const uint64_t mwt = (intree && active) ? mrow[t0 / 64] : 0ull;
    for (int j = sub; j < n; j += tpr) {
      if (intree ? !((mwt >> ((t0 + j) & 63)) & 1) : t0 + j < first) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qv[d], ks[j][d], s);
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(s - mn);
      l = fmaf(l, alpha, p);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], alpha, p * vs[j][d]);
      m = mn;
    }
  }

  // join the tpr states of the row (consecutive lanes of one wavefront)
  for (int off = 1; off < tpr; off <<= 1) {
    const float mo = __shfl_xor(m, off);
    const float lo = __shfl_xor(l, off);
    const float mn = fmaxf(m, mo);
    const float a0 = m == -INFINITY ? 0.f : exp2f(m - mn);  // a state without keys weighs 0
    const float a1 = mo == -INFINITY ? 0.f : exp2f(mo - mn);
    l = l * a0 + lo * a1;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * a0 + __shfl_xor(acc[d], off) * a1;
    m = mn;
  }
  if (!active || sub != 0) return;
  const size_t pr = (static_cast<size_t>(b * a.Hkv + g) * a.slots + slot) * a.R + r;  // active row
  const float inv = l > 0.f ? 1.f / l : 0.f;  // no keys: o = 0, lse = -inf
  float* op = static_cast<float*>(a.o_part) + pr * D;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  a.lse_part[pr] = m + log2f(l);
}

template <typename Tin>
hipError_t launch_typed(const Plan& p, PartialArgs a, hipStream_t stream) {
  // threads per row: the largest power of two up to 32 that still fits all
  // rows of a (sequence, KV head) into one workgroup, else 1
  int tpr = 1;
  while (tpr < 32 && p.R * tpr * 2 <= kThreadsWG) tpr *= 2;
  a.simple_tpr = tpr;
  const int rows_per_wg = kThreadsWG / tpr;
  const int rblocks = (p.R + rows_per_wg - 1) / rows_per_wg;
  const dim3 grid(p.Hkv, p.slots, p.B * rblocks);
  if (p.D == 128) {
    hipLaunchKernelGGL((partial_simple_kernel<Tin, 128>), grid, dim3(kThreadsWG), 0, stream, a);
  } else {
    hipLaunchKernelGGL((partial_simple_kernel<Tin, 64>), grid, dim3(kThreadsWG), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partials_simple(ltree_dtype dtype, const Plan& p, PartialArgs a,
                                  hipStream_t stream) {
  return dtype == LTREE_F32 ? launch_typed<float>(p, a, stream) : launch_typed<__bf16>(p, a, stream);
}

}  // namespace ltree
