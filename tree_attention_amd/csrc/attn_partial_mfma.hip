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
// (up to 384 rows) and each key byte is read from memory once per split.  With
// 320 rows the key/value stream carries 320 MFMA flops per byte, near the
// chip's flop:byte balance point, which is why the rows are not split further.
//
// Grid (Hkv, slots, B * row_blocks), 512 threads = 8 wavefronts, two per SIMD.
// The 16-row tiles of the workgroup's rows are dealt round-robin: tile t goes
// to wave t % 8, so with 20 tiles (G*T = 320) waves 0-3 take three and waves
// 4-7 two, and each SIMD (waves w and w+4) carries five.  Two waves per SIMD
// let the matrix cores run one wave's MFMAs while the other wave does its
// softmax arithmetic, and keep each wave within 256 registers.  Consecutive
// workgroups differ in KV head first, so with 8 KV heads every head keeps to
// one XCD (workgroups are dealt to the 8 XCDs round-robin) and its queries
// stay in that XCD's L2.
//
// Keys arrive in 64-key tiles and are consumed in 32-key blocks.  Per block,
// per wavefront and per 16-row tile:
//   S^T[key][row] = K . Q^T   v_mfma_f32_16x16x32_bf16, A = K from LDS,
//                              B = Q^T held in registers for the whole split;
//   online softmax in fp32 (row max over the 4 lane groups by two permlane
//                              swaps);
//   O^T[d][row] += V^T . P^T  v_mfma_f32_16x16x32_f16, A = V^T from LDS,
//                              B = P^T straight from the S^T accumulators.
// Result layout of a 16x16 MFMA: lane (g = lane/16, c = lane%16) holds rows
// 4g..4g+3 of column c.  Reading K rows in the order key(m) = 8(m/4) + 4s +
// m%4 for the two 16-key halves s of a block makes lane group g hold keys
// 8g..8g+7 of the block, exactly the k-slots the P.V MFMA expects from lane
// group g, so probabilities never move between lanes.
//
// LDS, three stages of one tile each:
//   K   [64 keys][D] bf16, filled straight from memory by global_load_lds
//       (16 bytes per lane); the 16-byte chunks of a key row are XOR-swizzled
//       by key so the 16 rows one lane group reads together hit distinct banks.
//   V^T [D][64 keys] fp16, 160-byte rows, 16-byte chunks XOR-swizzled by d/8;
//       converted from bf16 in registers while staging (exact: every finite
//       bf16 below 65504 is an fp16).
// Loads run two tiles ahead of the tile being computed; one barrier per tile.
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

constexpr int kTile = 64;    // keys per LDS tile
constexpr int kStages = 3;   // LDS tiles in flight
constexpr int kWaves = 8;    // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxTPW = 3;   // row tiles per wave at most (384 rows per workgroup)

template <int D>
struct Cfg {
  static constexpr int KC16 = D / 8;                    // 16-byte chunks per key row
  static constexpr int KROW = D * 2;                    // bytes per K row in LDS
  static constexpr int KBUF = kTile * KROW;             // bytes per K stage
  static constexpr int VSTR = 160;                      // bytes per V^T row
  static constexpr int VBUF = D * VSTR;                 // bytes per V^T stage
  static constexpr int DC = D / 32;                     // d chunks of the QK MFMA
  static constexpr int DT = D / 16;                     // d tiles of the PV MFMA
  static constexpr int KDMA = kTile * KC16 / kThreads;  // K 16-byte DMA loads per thread
  static constexpr int KEYS_PER_DMA = 1024 / KROW;      // keys per wave DMA instruction
  static constexpr int VITEMS = (kTile / 2) * KC16;     // V (key pair, chunk) items per tile
  static constexpr int SMEM = kStages * (KBUF + VBUF);
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

// Byte offset of the 16-byte chunk (row d, keys 8*chunk .. 8*chunk+7) of V^T.
__device__ inline int vt_off(int d, int chunk) {
  return d * 160 + ((chunk ^ ((d >> 3) & 7)) << 4);
}

__device__ inline uint32_t pack_f16(float lo, float hi) {
  const f16x2 h = __builtin_convertvector((f32x2){lo, hi}, f16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// max / sum over the four lane groups (lanes l, l^16, l^32, l^48)
__device__ inline float group_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Everything one workgroup shares.
struct Ctx {
  const PartialArgs* a;
  char* kl0;            // K stages
  char* vl0;            // V^T stages
  const __bf16* kbase;  // first key of this partial, KV head g
  const __bf16* vbase;
  int kstride;          // elements between consecutive keys
  int nkeys;            // keys of this partial
  int tid, lane, wave, l16, grp;
  int b, g, slot, rbase, rend;  // rows [rbase, rend) belong to this workgroup
  bool tree;
};

// The per-wave body: NT row tiles (rows rbase + 16*(wave + 8*rt) + l16).
template <int D, int NT>
__device__ __attribute__((always_inline)) inline void run(const Ctx& x) {
  using C = Cfg<D>;
  const PartialArgs& a = *x.a;
  const int lane = x.lane, l16 = x.l16, grp = x.grp, tid = x.tid, wave = x.wave;
  const int nkeys = x.nkeys;
  const bool tree = x.tree;

  // ---- queries of this wave's rows, as the B operand (Q^T) of the QK MFMA
  bf16x8 qf[NT][C::DC];
  uint32_t vbits[NT];  // tree: this lane's mask bits (keys 8grp..8grp+7 of each block)
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
    const bool ok = r < x.rend;
    const int i = ok ? r / a.G : 0;
    const int hh = ok ? r % a.G : 0;
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<size_t>(x.b) * a.T + i) * a.Hq + x.g * a.G + hh) * D + grp * 8;
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
      if (ok) {
        qf[rt][c] = *reinterpret_cast<const bf16x8*>(qp + c * 32);
      } else {
        qf[rt][c] = __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u});
      }
    }
    vbits[rt] = 0xffffu;
    if (tree && ok) {
      const uint64_t mw = a.mask[static_cast<size_t>(x.b) * a.T + i];
      vbits[rt] = static_cast<uint32_t>((mw >> (8 * grp)) & 0xffu) |
                  (static_cast<uint32_t>((mw >> (32 + 8 * grp)) & 0xffu) << 8);
    }
  }

  f32x4 acc[C::DT][NT];
  float mrow[NT], lrow[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    mrow[rt] = -INFINITY;
    lrow[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt][rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale_log2;
  const int ntiles = (nkeys + kTile - 1) / kTile;
  const int nblocks = (nkeys + 31) / 32;
  const int kstride = x.kstride;

  // ---- staging: K straight to LDS, V through registers
  auto kdma = [&](int t) {
    char* kl = x.kl0 + (t % kStages) * C::KBUF;
    const int last = nkeys - 1 - t * kTile;  // clamp keys past the end
#pragma unroll
    for (int j = 0; j < C::KDMA; ++j) {
      const int blk = j * kWaves + wave;  // 1 KB block of this wave instruction
      const int key = blk * C::KEYS_PER_DMA + lane / C::KC16;
      const int slotc = lane % C::KC16;
      const int kk = min(key, last);
      const __bf16* src = x.kbase + (t * kTile + kk) * kstride + ((slotc ^ kswz<D>(key)) * 8);
      __builtin_amdgcn_global_load_lds(src, kl + blk * 1024, 16, 0, 0);
    }
  };
  u32x4 vreg[2];
  const bool vitem = tid < C::VITEMS;
  const int vcc = tid % C::KC16;  // d chunk of this thread's V item
  const int vp = tid / C::KC16;   // key pair of this thread's V item
  auto vload = [&](int t) {
    if (vitem) {
      const int last = nkeys - 1 - t * kTile;
      const __bf16* src = x.vbase + (t * kTile) * kstride + vcc * 8;
      vreg[0] = *reinterpret_cast<const u32x4*>(src + min(2 * vp, last) * kstride);
      vreg[1] = *reinterpret_cast<const u32x4*>(src + min(2 * vp + 1, last) * kstride);
    }
  };
  auto vstore = [&](int t) {
    if (vitem) {
      char* vl = x.vl0 + (t % kStages) * C::VBUF;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u0 = vreg[0][w];  // v[2p][8cc+2w], v[2p][8cc+2w+1]
        const uint32_t u1 = vreg[1][w];  // v[2p+1][...]
        const float x0 = __uint_as_float(u0 << 16), x1 = __uint_as_float(u0 & 0xffff0000u);
        const float y0 = __uint_as_float(u1 << 16), y1 = __uint_as_float(u1 & 0xffff0000u);
        const int d = 8 * vcc + 2 * w;
        // key pair p sits at dword p%4 of 16-byte chunk p/4
        *reinterpret_cast<uint32_t*>(vl + vt_off(d, vp >> 2) + (vp & 3) * 4) = pack_f16(x0, y0);
        *reinterpret_cast<uint32_t*>(vl + vt_off(d + 1, vp >> 2) + (vp & 3) * 4) = pack_f16(x1, y1);
      }
    }
  };

  // ---- prologue: tiles 0 and 1 in flight, tile 0 ready
  kdma(0);
  vload(0);
  wait_vmem_all();
  vstore(0);
  if (ntiles > 1) {
    vload(1);
    kdma(1);
  }
  __syncthreads();

  for (int jb = 0; jb < nblocks; ++jb) {
    const char* kl = x.kl0 + ((jb >> 1) % kStages) * C::KBUF;
    const char* vl = x.vl0 + ((jb >> 1) % kStages) * C::VBUF;

    // S^T = K . Q^T for keys jb*32 .. +31: all eight K operands are read
    // first so their LDS latency overlaps, then the MFMAs
    bf16x8 ka[2][C::DC];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int key = (jb & 1) * 32 + 8 * (l16 >> 2) + 4 * sub + (l16 & 3);
      const char* krow = kl + key * C::KROW;
      const int sw = kswz<D>(key);
#pragma unroll
      for (int c = 0; c < C::DC; ++c) {
        ka[sub][c] = *reinterpret_cast<const bf16x8*>(krow + (((c * 4 + grp) ^ sw) << 4));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s[2][NT];
#pragma unroll
    for (int c = 0; c < C::DC; ++c) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          s[sub][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              ka[sub][c], qf[rt][c], c == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : s[sub][rt], 0, 0, 0);
        }
      }
    }
    // the V^T operands of this block's P.V, read now, used after the softmax
    f16x8 va[C::DT];
    {
      const int chunk = (jb & 1) * 4 + grp;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        va[dt] = *reinterpret_cast<const f16x8*>(vl + vt_off(dt * 16 + l16, chunk));
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // keys past the end of the partial, and tree keys outside the row's branch
    const int key0 = jb * 32;
    if (tree || key0 + 32 > nkeys) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const bool in = key0 + 8 * grp + 4 * sub + v < nkeys;
#pragma unroll
          for (int rt = 0; rt < NT; ++rt) {
            const uint32_t bits = (jb & 1) ? (vbits[rt] >> 8) : vbits[rt];
            if (!(in && ((bits >> (4 * sub + v)) & 1u))) s[sub][rt][v] = -INFINITY;
          }
        }
    }

    // Online softmax in base 2 on scores scaled by c2 = scale*log2(e).  The
    // running max moves only when a row's block max exceeds it by more than
    // 8/c2, i.e. when a probability would exceed 2^8; otherwise probabilities
    // up to 2^8 are kept against the stale max (exact: the final normalisation
    // and the lse use that same max) and the accumulator is not rescaled.
    float mt[NT];
    bool need = false;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const float m0 = fmaxf(fmaxf(s[0][rt][0], s[0][rt][1]), s[0][rt][2]);
      const float m1 = fmaxf(fmaxf(s[0][rt][3], s[1][rt][0]), s[1][rt][1]);
      const float m2 = fmaxf(fmaxf(s[1][rt][2], s[1][rt][3]), m0);
      mt[rt] = group_max(fmaxf(m1, m2));
      need = need || (mt[rt] - mrow[rt]) * c2 > 8.f;
    }
    if (__any(need)) {
      // Rare.  The scaled accumulator goes back through an MFMA (0*0 + C) so
      // that every definition of acc inside the loop is an MFMA result and acc
      // stays in the accumulation registers.
      const f16x8 z8 = __builtin_bit_cast(f16x8, (u32x4){0u, 0u, 0u, 0u});
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const float mn = fmaxf(mrow[rt], mt[rt]);
        // a tree row can have no visible key yet (a forest): keep it empty
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((mrow[rt] - mn) * c2);
        mrow[rt] = mn;
        lrow[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          acc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(z8, z8, acc[dt][rt] * alpha, 0, 0, 0);
        }
      }
    }

    // p = 2^(s*c2 - m*c2), row sums from the fp32 p, fp16 pack for P.V
    f16x8 pb[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      const float mc = mrow[rt] == -INFINITY ? 0.f : mrow[rt] * c2;  // then every s is -inf
      float p[8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[4 * sub + v] = __builtin_amdgcn_exp2f(fmaf(s[sub][rt][v], c2, -mc));
        }
      lrow[rt] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      const u32x4 w = (u32x4){pack_f16(p[0], p[1]), pack_f16(p[2], p[3]), pack_f16(p[4], p[5]),
                              pack_f16(p[6], p[7])};
      pb[rt] = __builtin_bit_cast(f16x8, w);
    }

    // O^T += V^T . P^T
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        acc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[dt], pb[rt], acc[dt][rt], 0, 0, 0);
      }
    }

    // After the first block of tile t: stage V^T of tile t+1, barrier (tile
    // t+1 is then complete in LDS), start the loads of tile t+2.
    if ((jb & 1) == 0) {
      const int t = jb >> 1;
      if (t + 1 < ntiles) {
        vstore(t + 1);
        wait_vmem_all();  // this thread's K DMA of tile t+1 has landed
        __syncthreads();
        if (t + 2 < ntiles) {
          // V loads first: the compiler waits for outstanding loads before
          // reusing their registers, and at this point none are outstanding
          vload(t + 2);
          kdma(t + 2);
        }
      }
    }
  }

  // ---- normalise and write the partial
  const size_t pbase = (static_cast<size_t>(x.b * a.Hkv + x.g) * a.slots + x.slot) * a.R;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const float l = group_sum(lrow[rt]);
    const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
    if (r < x.rend) {
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

template <int D, int TPW>
__global__ __launch_bounds__(kThreads, 2) void partial_mfma_kernel(PartialArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];

  Ctx x;
  x.a = &a;
  x.kl0 = smem;
  x.vl0 = smem + kStages * C::KBUF;
  x.tid = threadIdx.x;
  x.lane = x.tid & 63;
  x.wave = x.tid >> 6;
  x.l16 = x.lane & 15;
  x.grp = x.lane >> 4;
  x.g = blockIdx.x;
  x.slot = blockIdx.y;
  x.b = blockIdx.z / a.row_blocks;
  const int rb = blockIdx.z % a.row_blocks;
  x.rbase = rb * a.rows_per_wg;
  const int off0 = a.offsets[x.b];
  const int L = a.offsets[x.b + 1] - off0;
  x.tree = x.slot == a.max_chunks;
  x.kstride = a.Hkv * D;
  if (!x.tree) {
    if (L < 0 || L > a.max_prefix_len) return;  // the merge reports it
    const int k0 = x.slot * a.chunk;
    if (k0 >= L) return;
    x.nkeys = min(a.chunk, L - k0);
    const size_t row0 = static_cast<size_t>(off0) + k0;
    x.kbase = static_cast<const __bf16*>(a.kp) + (row0 * a.Hkv + x.g) * D;
    x.vbase = static_cast<const __bf16*>(a.vp) + (row0 * a.Hkv + x.g) * D;
  } else {
    x.nkeys = a.T;
    x.kbase = static_cast<const __bf16*>(a.kt) + (static_cast<size_t>(x.b) * a.T * a.Hkv + x.g) * D;
    x.vbase = static_cast<const __bf16*>(a.vt) + (static_cast<size_t>(x.b) * a.T * a.Hkv + x.g) * D;
  }

  // Row tiles of this workgroup and how many fall to this wave.  Every wave
  // runs the same sequence of tiles, blocks and barriers; only the number of
  // row tiles it computes differs.
  x.rend = min(a.R, x.rbase + a.rows_per_wg);
  const int tiles = (x.rend - x.rbase + 15) / 16;
  const int ntw = (tiles - x.wave + kWaves - 1) / kWaves;  // tiles wave, wave+8, ... < tiles
  if constexpr (TPW >= 3) {
    if (ntw >= 3) {
      run<D, 3>(x);
      return;
    }
  }
  if constexpr (TPW >= 2) {
    if (ntw == 2) {
      run<D, 2>(x);
      return;
    }
  }
  run<D, 1>(x);  // one tile, or none: a wave without rows still stages and syncs
}

template <int D>
hipError_t launch_d(int tpw, dim3 grid, PartialArgs a, hipStream_t stream) {
  switch (tpw) {
    case 1: hipLaunchKernelGGL((partial_mfma_kernel<D, 1>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((partial_mfma_kernel<D, 2>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((partial_mfma_kernel<D, 3>), grid, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partials_mfma(const Plan& p, PartialArgs a, hipStream_t stream) {
  // Row blocking: at most kMaxTPW tiles of 16 rows per wave, 8 waves.
  const int tiles = (p.R + 15) / 16;
  const int row_blocks = (tiles + kWaves * kMaxTPW - 1) / (kWaves * kMaxTPW);
  const int tiles_per_block = (tiles + row_blocks - 1) / row_blocks;
  const int tpw = (tiles_per_block + kWaves - 1) / kWaves;
  a.rows_per_wg = 16 * tiles_per_block;
  a.row_blocks = (p.R + a.rows_per_wg - 1) / a.rows_per_wg;
  const dim3 grid(p.Hkv, p.slots, p.B * a.row_blocks);
  return p.D == 128 ? launch_d<128>(tpw, grid, a, stream) : launch_d<64>(tpw, grid, a, stream);
}

}  // namespace ltree
