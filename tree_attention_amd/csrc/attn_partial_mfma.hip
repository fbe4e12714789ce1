// Partial attention on MFMA for bf16 inputs (steps a2 and a3).
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 2 part C ("Schnelle Tree
// Attention"): item 1 of the split is the cached part (the long prefix KV
// cache, no mask), item 2 the speculative part (the tree tokens, tree mask).
// Each workgroup produces one partial softmax result: its query rows against
// one prefix split, or against the tree tokens under the mask.  The
// log-sum-exp merge ("Aggregation") joins the partials.
//
// Work decomposition.  All G*T query rows that read one KV head (the GQA group
// times the tree tokens) share every key, so one workgroup takes all of them
// (up to 320 rows) and each key byte is read from memory once per split.  With
// 320 rows the key/value stream carries 320 MFMA flops per byte, near the
// chip's flop:byte balance point, which is why the rows are not split further.
//
// Grid (Hkv, slots, B * row_blocks), 256 threads = 4 wavefronts.  Consecutive
// workgroups differ in KV head first, so with 8 KV heads every head keeps to
// one XCD (workgroups are dealt to the 8 XCDs round-robin) and its queries
// stay in that XCD's L2.
//
// Keys arrive in 64-key LDS tiles and are consumed in 32-key blocks.  Per
// block, per wavefront (TPW row tiles of 16 rows each):
//   S^T[key][row] = K . Q^T   on v_mfma_f32_16x16x32_bf16, A = K from LDS,
//                              B = Q^T held in registers for the whole split;
//   online softmax in fp32, row max over the 4 lane groups by two xor shuffles;
//   O^T[d][row] += V^T . P^T  on v_mfma_f32_16x16x32_f16, A = V^T from LDS,
//                              B = P^T straight from the S^T accumulators.
// Result layout of a 16x16 MFMA: lane (g = lane/16, c = lane%16) holds rows
// 4g..4g+3 of column c.  Reading K rows in the order key(m) = 8(m/4) + 4s +
// m%4 for the two 16-key halves s of a 32-key block makes lane group g hold
// keys 8g..8g+7 of the block, exactly the k-slots the P.V MFMA expects from
// lane group g, so probabilities never move between lanes.
//
// LDS per buffer: K tile [64 keys][D] bf16 with the 16-byte chunks of each row
// XOR-swizzled by key (the 16 rows read together hit different banks), and V^T
// tile [D][64 keys] fp16 with padded rows (converted from bf16 while staging:
// exact, since every finite bf16 below 65504 is an fp16).  Two buffers; the
// global loads of tile t+1 are in flight while tile t is computed.
#include <type_traits>

#include "ltree_internal.h"

namespace ltree {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;  // keys per tile

template <int D>
struct Cfg {
  static constexpr int KC16 = D / 8;                        // 16-byte chunks per key row
  static constexpr int KROW = D * 2;                        // bytes per K row in LDS
  static constexpr int KBUF = kTile * KROW;                 // bytes per K buffer
  static constexpr int VSTR = kTile * 2 + 16;               // bytes per V^T row (padded)
  static constexpr int VBUF = D * VSTR;                     // bytes per V^T buffer
  static constexpr int DC = D / 32;                         // d chunks of the QK MFMA
  static constexpr int DT = D / 16;                         // d tiles of the PV MFMA
  static constexpr int KLOADS = kTile * KC16 / 256;         // K 16-byte loads per thread
  static constexpr int VITEMS = (kTile / 2) * KC16 / 256;   // V (key pair, chunk) items
  static constexpr int SMEM = 2 * (KBUF + VBUF);
};

// Chunk swizzle of a K row: the 16 rows read by one lane group in a QK step
// are keys 8a + b (+4) with a, b in 0..3, so the swizzle uses key bits 0,1,3,4.
template <int D>
__device__ inline int kswz(int key) {
  if constexpr (D == 128) {
    return (key & 3) | ((key >> 1) & 12);
  } else {
    return (key & 3) | ((key >> 1) & 4);
  }
}

__device__ inline uint32_t pack_f16(float lo, float hi) {
  const f16x2 h = __builtin_convertvector((f32x2){lo, hi}, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

template <int D, int TPW>
__global__ __launch_bounds__(256, 1) void partial_mfma_kernel(PartialArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  const int g = blockIdx.x;
  const int slot = blockIdx.y;
  const int b = blockIdx.z / a.row_blocks;
  const int rb = blockIdx.z % a.row_blocks;
  const int off0 = a.offsets[b];
  const int L = a.offsets[b + 1] - off0;
  const bool tree = slot == a.max_chunks;
  const size_t kstride = static_cast<size_t>(a.Hkv) * D;

  int k0, k1;
  const __bf16* kbase;
  const __bf16* vbase;
  if (!tree) {
    if (L < 0 || L > a.max_prefix_len) return;  // the merge reports it
    k0 = slot * a.chunk;
    if (k0 >= L) return;
    k1 = min(k0 + a.chunk, L);
    kbase = static_cast<const __bf16*>(a.kp) + (static_cast<size_t>(off0) * a.Hkv + g) * D;
    vbase = static_cast<const __bf16*>(a.vp) + (static_cast<size_t>(off0) * a.Hkv + g) * D;
  } else {
    k0 = 0;
    k1 = a.T;
    kbase = static_cast<const __bf16*>(a.kt) + (static_cast<size_t>(b) * a.T * a.Hkv + g) * D;
    vbase = static_cast<const __bf16*>(a.vt) + (static_cast<size_t>(b) * a.T * a.Hkv + g) * D;
  }

  // ---- queries of this wave's rows, as the B operand (Q^T) of the QK MFMA.
  const int rbase = rb * a.rows_per_wg + wave * TPW * 16;
  bf16x8 qf[TPW][C::DC];
  uint64_t mw[TPW];
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt) {
    const int r = rbase + rt * 16 + l16;
    const bool ok = r < a.R;
    const int i = ok ? r / a.G : 0;
    const int hh = ok ? r % a.G : 0;
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<size_t>(b) * a.T + i) * a.Hq + g * a.G + hh) * D + grp * 8;
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
      if (ok) {
        qf[rt][c] = *reinterpret_cast<const bf16x8*>(qp + c * 32);
      } else {
        qf[rt][c] = __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u});
      }
    }
    mw[rt] = (tree && ok) ? a.mask[static_cast<size_t>(b) * a.T + i] : ~0ull;
  }

  f32x4 acc[C::DT][TPW];
  float mrow[TPW], lrow[TPW];
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt) {
    mrow[rt] = -INFINITY;
    lrow[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt][rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale_log2;
  uint32_t vbits[TPW];  // tree workgroup: this lane's 16 mask bits per row tile

  // ---- staging registers for the next tile
  u32x4 kreg[C::KLOADS];
  u32x4 vreg[C::VITEMS][2];

  auto gload = [&](int t) {
    const int tb = k0 + t * kTile;
#pragma unroll
    for (int j = 0; j < C::KLOADS; ++j) {
      const int e = tid + 256 * j;
      const int key = min(tb + e / C::KC16, k1 - 1);
      kreg[j] = *reinterpret_cast<const u32x4*>(kbase + key * kstride + (e % C::KC16) * 8);
    }
#pragma unroll
    for (int j = 0; j < C::VITEMS; ++j) {
      const int e = tid + 256 * j;
      const int p = e / C::KC16;
      const int cc = e % C::KC16;
      const int ka = min(tb + 2 * p, k1 - 1);
      const int kb = min(tb + 2 * p + 1, k1 - 1);
      vreg[j][0] = *reinterpret_cast<const u32x4*>(vbase + ka * kstride + cc * 8);
      vreg[j][1] = *reinterpret_cast<const u32x4*>(vbase + kb * kstride + cc * 8);
    }
  };

  auto lstore = [&](int buf) {
    char* kl = smem + buf * C::KBUF;
    char* vl = smem + 2 * C::KBUF + buf * C::VBUF;
#pragma unroll
    for (int j = 0; j < C::KLOADS; ++j) {
      const int e = tid + 256 * j;
      const int key = e / C::KC16;
      const int cc = e % C::KC16;
      *reinterpret_cast<u32x4*>(kl + key * C::KROW + ((cc ^ kswz<D>(key)) << 4)) = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < C::VITEMS; ++j) {
      const int e = tid + 256 * j;
      const int p = e / C::KC16;
      const int cc = e % C::KC16;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = vreg[j][0][w];  // v[2p][8cc+2w], v[2p][8cc+2w+1]
        const uint32_t y = vreg[j][1][w];  // v[2p+1][...]
        const float x0 = __uint_as_float(x << 16), x1 = __uint_as_float(x & 0xffff0000u);
        const float y0 = __uint_as_float(y << 16), y1 = __uint_as_float(y & 0xffff0000u);
        const int d = 8 * cc + 2 * w;
        *reinterpret_cast<uint32_t*>(vl + d * C::VSTR + p * 4) = pack_f16(x0, y0);
        *reinterpret_cast<uint32_t*>(vl + (d + 1) * C::VSTR + p * 4) = pack_f16(x1, y1);
      }
    }
  };

  // One 32-key block: S^T = K . Q^T, masking, online softmax, O^T += V^T . P^T.
  // MASK: apply the tree mask (tree workgroup); TAIL: keys may pass k1.
  auto block = [&](const char* kl, const char* vl, int kb, int key0, auto mask_tag,
                   bool tail) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x4 s[2][TPW];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int key = kb * 32 + 8 * (l16 >> 2) + 4 * sub + (l16 & 3);
      const char* krow = kl + key * C::KROW;
      const int sw = kswz<D>(key);
#pragma unroll
      for (int rt = 0; rt < TPW; ++rt) s[sub][rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C::DC; ++c) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(krow + (((c * 4 + grp) ^ sw) << 4));
#pragma unroll
        for (int rt = 0; rt < TPW; ++rt) {
          s[sub][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qf[rt][c], s[sub][rt], 0, 0, 0);
        }
      }
    }

    // lane holds keys key0 + 8*grp + 4*sub + v, v = 0..3, of its row
    if (MASK || tail) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int kk = key0 + 8 * grp + 4 * sub + v;
          const bool in = kk < k1;
#pragma unroll
          for (int rt = 0; rt < TPW; ++rt) {
            bool vis = in;
            if constexpr (MASK) vis = vis && ((vbits[rt] >> (4 * sub + v)) & 1u);
            if (!vis) s[sub][rt][v] = -INFINITY;
          }
        }
    }

    // online softmax in base 2 on scores scaled by scale*log2(e).  The running
    // max moves only when a row's block max exceeds it by more than 8/c2, i.e.
    // when a probability would exceed 2^8; otherwise probabilities up to 2^8
    // are kept against the stale max (exact: the final normalisation and the
    // lse use that same max), and the accumulator is not rescaled.
    float mt[TPW];
    bool need = false;
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
      float m = fmaxf(fmaxf(fmaxf(s[0][rt][0], s[0][rt][1]), fmaxf(s[0][rt][2], s[0][rt][3])),
                      fmaxf(fmaxf(s[1][rt][0], s[1][rt][1]), fmaxf(s[1][rt][2], s[1][rt][3])));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      mt[rt] = m;
      need = need || (m - mrow[rt]) * c2 > 8.f;
    }
    if (__any(need)) {
#pragma unroll
      for (int rt = 0; rt < TPW; ++rt) {
        const float mn = fmaxf(mrow[rt], mt[rt]);
        // a tree row can have no visible key yet (a forest): keep it empty
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mrow[rt] - mn) * c2);
        mrow[rt] = mn;
        lrow[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc[dt][rt] *= alpha;
      }
    }
    f16x8 pb[TPW];
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
      const float mc = mrow[rt] == -INFINITY ? 0.f : mrow[rt] * c2;  // then every s is -inf
      float p[8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 4; ++v) p[4 * sub + v] = __builtin_amdgcn_exp2f(fmaf(s[sub][rt][v], c2, -mc));
      lrow[rt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      const u32x4 w = (u32x4){pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]),
                              pack_f16(p[6], p[7])};
      pb[rt] = __builtin_bit_cast(f16x8, w);
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const f16x8 A =
          *reinterpret_cast<const f16x8*>(vl + (dt * 16 + l16) * C::VSTR + (kb * 32 + 8 * grp) * 2);
#pragma unroll
      for (int rt = 0; rt < TPW; ++rt) {
        acc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, pb[rt], acc[dt][rt], 0, 0, 0);
      }
    }
  };

  if (tree) {
    // The speculative part: T <= 64 tree keys, one tile, under the tree mask.
    // Lane group grp needs mask bits 8*grp..8*grp+7 of each 32-key block.
#pragma unroll
    for (int rt = 0; rt < TPW; ++rt) {
      vbits[rt] = static_cast<uint32_t>((mw[rt] >> (8 * grp)) & 0xffu) |
                  (static_cast<uint32_t>((mw[rt] >> (32 + 8 * grp)) & 0xffu) << 8);
    }
    gload(0);
    lstore(0);
    __syncthreads();
    block(smem, smem + 2 * C::KBUF, 0, 0, std::true_type{}, true);
    if (k1 > 32) {
#pragma unroll
      for (int rt = 0; rt < TPW; ++rt) vbits[rt] >>= 8;
      block(smem, smem + 2 * C::KBUF, 1, 32, std::true_type{}, true);
    }
  } else {
    // The cached part: one prefix split, no mask; tile t computes from buffer
    // t&1 while the global loads of tile t+1 are in flight.
    const int ntiles = (k1 - k0 + kTile - 1) / kTile;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      if (more) gload(t + 1);
      const char* kl = smem + (t & 1) * C::KBUF;
      const char* vl = smem + 2 * C::KBUF + (t & 1) * C::VBUF;
      const int tb = k0 + t * kTile;
      block(kl, vl, 0, tb, std::false_type{}, tb + 32 > k1);
      if (tb + 32 < k1) block(kl, vl, 1, tb + 32, std::false_type{}, tb + 64 > k1);
      if (more) lstore((t + 1) & 1);
      __syncthreads();
    }
  }

  // ---- normalise and write the partial
  const size_t pbase = (static_cast<size_t>(b * a.Hkv + g) * a.slots + slot) * a.R;
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt) {
    float l = lrow[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = rbase + rt * 16 + l16;
    if (r < a.R) {
      const float inv = 1.f / l;
      float* op = a.o_part + (pbase + r) * D + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        *reinterpret_cast<f32x4*>(op + dt * 16) = acc[dt][rt] * inv;
      }
      if (grp == 0) a.lse_part[pbase + r] = mrow[rt] * c2 + __builtin_amdgcn_logf(l);
    }
  }
}

template <int D>
hipError_t launch_d(int tpw, dim3 grid, PartialArgs a, hipStream_t stream) {
  switch (tpw) {
    case 1: hipLaunchKernelGGL((partial_mfma_kernel<D, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((partial_mfma_kernel<D, 2>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((partial_mfma_kernel<D, 3>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((partial_mfma_kernel<D, 4>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((partial_mfma_kernel<D, 5>), grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partials_mfma(const Plan& p, PartialArgs a, hipStream_t stream) {
  // Row blocking: at most 5 row tiles of 16 per wave (320 rows per workgroup).
  constexpr int kMaxTPW = 5;
  const int row_blocks = (p.R + 64 * kMaxTPW - 1) / (64 * kMaxTPW);
  const int rows_per_block = (p.R + row_blocks - 1) / row_blocks;
  const int tpw = (rows_per_block + 63) / 64;
  a.rows_per_wg = 64 * tpw;
  a.row_blocks = (p.R + a.rows_per_wg - 1) / a.rows_per_wg;
  const dim3 grid(p.Hkv, p.slots, p.B * a.row_blocks);
  return p.D == 128 ? launch_d<128>(tpw, grid, a, stream) : launch_d<64>(tpw, grid, a, stream);
}

}  // namespace ltree
