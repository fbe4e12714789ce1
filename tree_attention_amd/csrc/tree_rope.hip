// Rotary position embedding of the tree tokens at their tree positions.
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 1 "Problemstellung", item
// "Trainings-Inferenz-Diskrepanz": positions enter through RoPE, and the draft's
// positions must agree with the target model's; the mlsanity.com page lists
// RoFormer (rotary position embedding) among the paper's references.  A tree
// token continues the prefix along its own branch, so node i of sequence b sits
// at position p = L_b + depth(i) - 1 (depth counts the nodes from the root,
// root = 1); siblings share a position.
//
// For each query head and each KV head of the token, and k < D/2 with
// theta_k = base^(-2k/D) and a = p * theta_k:
//   x'[k]       = x[k] cos a - x[k + D/2] sin a
//   x'[k + D/2] = x[k + D/2] cos a + x[k] sin a
// (the half-split pairing of the target models' rotary layers).  Applied in
// place to q [B,T,Hq,D] and k_tree [B,T,Hkv,D].  The angle and the rotation are
// evaluated in fp64 (positions reach 10^6 radians at theta_0 = 1), then
// rounded to the storage type.  depth(i) is the popcount of the node's mask
// row (its W = ceil(T/64) words); a zero row (a tree with an invalid parent)
// is left unrotated.
#include <algorithm>

#include "ltree_internal.h"

namespace ltree {
namespace {

template <typename Tx>
__device__ inline double load_d(const Tx* p) {
  if constexpr (sizeof(Tx) == 2) {
    return static_cast<double>(__uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(p)) << 16));
  } else {
    return static_cast<double>(*p);
  }
}

template <typename Tx>
__device__ inline void store_d(Tx* p, double v) {
  if constexpr (sizeof(Tx) == 2) {
    // fp64 -> bf16 rounded to nearest even, exactly: first to fp32 rounding
    // to odd (truncate, then set the last bit if anything was dropped), whose
    // 16 extra bits make the second rounding, to bf16, the correct one
    float f = __double2float_rz(v);
    uint32_t u = __float_as_uint(f);
    if (static_cast<double>(f) != v) u |= 1u;
    u += 0x7fffu + ((u >> 16) & 1u);
    *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(u >> 16);
  } else {
    *p = static_cast<float>(v);  // round to nearest even
  }
}

constexpr int kRopeThreads = 256;
constexpr int kRopeBatch = 16;  // head passes whose elements are loaded ahead

// grid (T, B, S); 256 threads: thread t rotates pair k = t mod D/2 of heads
// t / (D/2) + n * 256 / (D/2) of the token (pass n), the query heads first,
// then the key heads.  The token's passes are shared by its S workgroups,
// which fill the chip when T * B is small.  The elements of up to
// kRopeBatch passes are loaded before the token's position and angle are
// known, so those loads overlap the mask and prefix-table reads and the fp64
// angle instead of following them.
template <typename Tx, int D>
__global__ __launch_bounds__(kRopeThreads) void tree_rope_kernel(
    Tx* __restrict__ q, Tx* __restrict__ kt, const uint64_t* __restrict__ mask,
    const int32_t* __restrict__ offsets, int T, int Hq, int Hkv, double base) {
  constexpr int kHalf = D / 2;
  constexpr int kHeadsPerPass = kRopeThreads / kHalf;
  const int i = blockIdx.x, b = blockIdx.y;
  const int k = threadIdx.x % kHalf, h0 = threadIdx.x / kHalf;
  const int W = (T + 63) / 64;  // mask words per row
  const int H = Hq + Hkv;
  const int passes = (H + kHeadsPerPass - 1) / kHeadsPerPass;
  const int per = (passes + gridDim.z - 1) / gridDim.z;
  const int pbeg = blockIdx.z * per, pend = min(passes, pbeg + per);
  if (pbeg >= pend) return;
  Tx* qrow = q + (static_cast<size_t>(b) * T + i) * Hq * D;
  Tx* krow = kt + (static_cast<size_t>(b) * T + i) * Hkv * D;
  auto head_row = [&](int h) -> Tx* {
    return h < Hq ? qrow + static_cast<size_t>(h) * D : krow + static_cast<size_t>(h - Hq) * D;
  };
  const uint64_t* mrow = mask + (static_cast<size_t>(b) * T + i) * W;
  const int L = offsets[b + 1] - offsets[b];
  double x0[kRopeBatch], x1[kRopeBatch];
  // (a pass past the last head reads the last head's row: no branch per
  // load, and the value is never stored)
  auto load_batch = [&](int pass0) {
#pragma unroll
    for (int j = 0; j < kRopeBatch; ++j) {
      const Tx* row = head_row(min(h0 + min(pass0 + j, pend - 1) * kHeadsPerPass, H - 1));
      x0[j] = load_d(row + k);
      x1[j] = load_d(row + k + kHalf);
    }
  };
  load_batch(pbeg);
  int depth = 0;
  for (int w = 0; w < W; ++w) depth += static_cast<int>(__popcll(mrow[w]));
  if (depth == 0) return;
  const long p = static_cast<long>(L) + depth - 1;
  const double theta = pow(base, -2.0 * k / D);
  double s, c;
  sincos(static_cast<double>(p) * theta, &s, &c);
  for (int pass0 = pbeg;; pass0 += kRopeBatch) {
#pragma unroll
    for (int j = 0; j < kRopeBatch; ++j) {
      const int h = h0 + (pass0 + j) * kHeadsPerPass;
      if (pass0 + j < pend && h < H) {
        Tx* row = head_row(h);
        store_d(row + k, x0[j] * c - x1[j] * s);
        store_d(row + k + kHalf, x1[j] * c + x0[j] * s);
      }
    }
    if (pass0 + kRopeBatch >= pend) break;
    load_batch(pass0 + kRopeBatch);
  }
}

template <typename Tx>
void launch_typed(void* q, void* kt, const uint64_t* mask, const int32_t* offsets, int B, int T,
                  int Hq, int Hkv, int D, double base, hipStream_t stream) {
  // workgroups per token: enough for T * B tokens to cover the compute units
  // once, at most one per pass
  const int passes = (Hq + Hkv + kRopeThreads / (D / 2) - 1) / (kRopeThreads / (D / 2));
  const long tokens = static_cast<long>(T) * B;
  const int S = static_cast<int>(std::max(1L, std::min<long>(passes, device_cu_count() / tokens)));
  const dim3 grid(T, B, S);
  if (D == 128) {
    hipLaunchKernelGGL((tree_rope_kernel<Tx, 128>), grid, dim3(kRopeThreads), 0, stream,
                       static_cast<Tx*>(q), static_cast<Tx*>(kt), mask, offsets, T, Hq, Hkv, base);
  } else {
    hipLaunchKernelGGL((tree_rope_kernel<Tx, 64>), grid, dim3(kRopeThreads), 0, stream,
                       static_cast<Tx*>(q), static_cast<Tx*>(kt), mask, offsets, T, Hq, Hkv, base);
  }
}

}  // namespace

hipError_t launch_tree_rope(bool bf16, void* q, void* k_tree, const uint64_t* mask,
                            const int32_t* offsets, int B, int T, int Hq, int Hkv, int D,
                            double base, hipStream_t stream) {
  if (bf16) {
    launch_typed<uint16_t>(q, k_tree, mask, offsets, B, T, Hq, Hkv, D, base, stream);
  } else {
    launch_typed<float>(q, k_tree, mask, offsets, B, T, Hq, Hkv, D, base, stream);
  }
  return hipGetLastError();
}

}  // namespace ltree
