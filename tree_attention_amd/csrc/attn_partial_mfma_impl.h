// Partial attention on MFMA for bf16 inputs (steps a2 and a3).
//
// gist.science page "LongSpec: Long-Context Lossless Speculative Decoding with
// Efficient Drafting and Verification", section 2 part C ("Schnelle Tree
// Attention"): item 1 of the split is the cached part (the long prefix KV
// cache, no mask), item 2 the speculative part (the tree tokens, tree mask).
// Each workgroup produces one partial softmax result: its query rows against
// one prefix split; the last split of a sequence (the only one when the prefix
// is empty) continues over the tree tokens under the mask, so no workgroup is
// spent on the tiny tree part alone.  The log-sum-exp merge ("Aggregation")
// joins the partials.
//
// Work decomposition.  All G*T query rows that read one KV head (the GQA group
// times the tree tokens) share every key, so one workgroup takes all of them
// (up to 384 rows) and each key byte is read from memory once per split.  With
// 320 rows the key/value stream carries 320 MFMA flops per byte, near the
// chip's flop:byte balance point, which is why the rows are not split further.
//
// Grid (Hkv, slots, B * row_blocks), 512 threads = 8 wavefronts, two per SIMD.
// One sequence: workgroup (g, s, rb) takes split s of row block rb.  A batch
// of 2 to 256 sequences: the j-th workgroup of KV head g (j = y + slots * z)
// takes the j-th (sequence, split) pair that exists, row blocks innermost,
// so every workgroup with work comes before the empty ones in dispatch
// order.  (Mapped directly, the unused slots of a short sequence would be
// dispatched between the splits of the longer ones: each such workgroup
// holds a CU for a memory round trip, and the CUs they leave are not the
// ones the next real workgroups go to.)
// The 16-row tiles of the workgroup's rows are dealt round-robin: tile t goes
// to wave t % 8, so with 20 tiles (G*T = 320) waves 0-3 take three and waves
// 4-7 two, and each SIMD (waves w and w+4) carries five.  Consecutive
// workgroups differ in KV head first, so with 8 KV heads every head keeps to
// one XCD (workgroups are dealt to the 8 XCDs round-robin).
//
// Keys arrive in 64-key tiles and are consumed in 32-key blocks.  Per block,
// per wavefront and per 16-row tile:
//   S^T[key][row] = K . Q^T   v_mfma_f32_16x16x32_bf16, A = K rows from LDS,
//                              B = Q^T held in registers for the whole split;
//   online softmax in fp32 (lazy reference max, see below);
//   O^T[d][row] += V^T . P^T  v_mfma_f32_16x16x32_f16, A = V^T (fp16) from
//                              LDS, B = P^T (fp16) straight from the S^T
//                              accumulators.
// Result layout of a 16x16 MFMA: lane (g = lane/16, c = lane%16) holds rows
// 4g..4g+3 of column c.  Reading K rows in the order key(m) = 8(m/4) + 4s +
// m%4 for the two 16-key halves s of a block makes lane group g hold keys
// 8g..8g+7 of the block, exactly the k-slots the P.V MFMA expects from lane
// group g, so probabilities never move between lanes.
//
// Order within a block: the K operands of the block are already in
// registers (loaded during the previous P.V); the QK products run one row
// tile at a time, each row tile's softmax overlapping the products of the
// next; then the P.V products, one d tile at a time, while the K operands of
// the following block are read.
//
// LDS.  Three stages of one tile each hold K [64 keys][D] and the raw V tile,
// both filled straight from memory by buffer loads to LDS (16 bytes per lane;
// the buffer range ends at the tile's last real key, so rows past it read as
// zeros), so no staging registers are needed and tiles t+1 and t+2 are in
// flight while tile t is computed.  Once a thread's V loads of the next tile
// have landed it converts them to fp16 and writes them transposed into one of
// three V^T buffers [D][64 keys] (exact for |v| < 65504).  Probabilities
// enter the P.V product as fp16, whose rounding (2^-11) keeps the output
// within tolerance even where a few large values dominate a row, which bf16
// (2^-8) does not.  LDS has 64 banks of 4 bytes.  The K chunk swizzle puts
// the 16 lanes of a lane group on 16 different 16-byte bank groups, so the K
// operand reads have no bank conflicts; the V^T buffers use a 144-byte row
// pitch and a cell swizzle, and their reads and the transposed writes still
// register a few conflict cycles per instruction (measured), most of which the
// LDS pipeline hides.  One barrier per tile.
//
// Shared by the translation units that instantiate the kernel's variants
// (attn_partial_mfma*.hip), so that they compile in parallel.
#pragma once

#include <type_traits>

#include "ltree_internal.h"

namespace ltree {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;    // keys per LDS tile
constexpr int kStages = 3;   // LDS buffers of each kind (K, raw V, V^T); tile t uses t % 3
constexpr int kWaves = 8;    // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxTPW = 3;   // row tiles per wave at most (384 rows per workgroup)
constexpr int kVtRow = 144;  // bytes per V^T row: 64 fp16 keys + 16 bytes of pitch
constexpr int kMaskStash = LTREE_MAX_TREE * ((LTREE_MAX_TREE + 63) / 64) * 8;  // LDS bytes, BIGT
constexpr int kPageStash = kMaxSplitPages * 4;  // LDS bytes, PAGED: the split's page numbers
constexpr int kHeadKeys = 256;  // window: keys at the start of the range a row may hide
// fourth word of a raw buffer descriptor (32-bit data format; no swizzle)
constexpr int kBufferFlags = 0x00020000;
constexpr int kCompactBatch = 256;  // batches of 2..256 sequences: splits packed in dispatch order

template <int D>
struct Cfg {
  static constexpr int KC16 = D / 8;                      // 16-byte chunks per key row
  static constexpr int ROW = D * 2;                       // bytes per K (or raw V) row
  static constexpr int BUF = kTile * ROW;                 // bytes of one K (or raw V) tile
  static constexpr int VT = D * kVtRow;                   // bytes of one V^T buffer
  // LDS: kStages K tiles, then kStages raw V tiles, then kStages V^T buffers
  static constexpr int K0 = 0;
  static constexpr int R0 = kStages * BUF;
  static constexpr int T0 = 2 * kStages * BUF;
  static constexpr int SMEM = T0 + kStages * VT;
  static constexpr int DC = D / 32;                       // d chunks of the QK MFMA
  static constexpr int DT = D / 16;                       // d tiles of the PV MFMA
  static constexpr int KDMA = kTile * KC16 / kThreads;    // K 16-byte DMA loads per thread
  static constexpr int ROWS_PER_DMA = 1024 / ROW;         // K rows per wave DMA instruction
  static constexpr int VITEMS = (kTile / 2) * KC16;       // V items: (key pair, d chunk)
  static constexpr int VIPT = VITEMS > kThreads ? VITEMS / kThreads : 1;  // V items per thread
  static constexpr int VTHREADS = VITEMS / VIPT;          // threads that stage V
  static constexpr int DPT_V = KDMA + 2 * VIPT;           // DMA per tile, V-staging threads
  static constexpr int DPT_K = KDMA;                      // DMA per tile, other threads
  static constexpr int OUT_PITCH = 2 * D + 16;            // LDS bytes per partial row (epilogue)
  static_assert(kMaxTPW * kWaves * 16 * OUT_PITCH <= SMEM, "the partial rows fit in LDS");
};

// K rows: the 16 lanes of one lane group read keys 8a + b (+4), a, b in 0..3,
// at one 16-byte chunk index; the swizzle spreads them over all 64 banks.  It
// does not use key bits 2 or 5, so a lane's offsets hold for both 4-key halves
// of a 16-key step and both 32-key blocks of a tile.
template <int D>
__device__ inline int kswz(int key) {
  if constexpr (D == 128) {
    return (key & 3) | ((key >> 1) & 12);
  } else {  // 128-byte rows: two rows per bank line
    return ((key >> 1) & 1) | ((key >> 2) & 2) | ((key >> 2) & 4);
  }
}

// V^T: row d at d * kVtRow, its 16-byte cell q (keys 8q..8q+7) at position
// q ^ ((d / 16) % 8).  With the 144-byte pitch the 16 rows one lane group reads
// (a d tile) hit distinct bank groups, and the XOR spreads the cells the
// staging threads write together (features 8c + e for 16 values of c).
__device__ inline int vt_off(int d, int q) { return d * kVtRow + ((q ^ ((d >> 4) & 7)) << 4); }

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

// This thread's LDS DMA writes are complete except for those of the `n` (0..1)
// most recently issued tiles, DPT loads per tile (the loop issues nothing
// else to memory).
template <int DPT>
__device__ inline void wait_dma_except(int n) {
  if (n >= 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DPT) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// Workgroup barrier for the hand-off of LDS buffers: this wave's LDS reads
// and writes are complete; its tile loads in flight are not waited for
// (__syncthreads would wait for them all: each thread waits for its own
// loads of a tile before the barrier that publishes it).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// acc + lo + hi of two fp16 (the row sums)
__device__ inline float add_f16x2(f16x2 h, float acc) {
  const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
  return __builtin_amdgcn_fdot2(h, ones, acc, false);
}

// fp16 pair (lo, hi) from the low halves (hi = false) or high halves of two
// bf16 pairs (exact below 65504)
__device__ inline uint32_t pack_f16_of_bf16(uint32_t lo, uint32_t hi, bool upper) {
  const float a = __uint_as_float(upper ? (lo & 0xffff0000u) : (lo << 16));
  const float b = __uint_as_float(upper ? (hi & 0xffff0000u) : (hi << 16));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}

// Everything one workgroup shares.
struct Ctx {
  const PartialArgs* a;
  char* smem;
  const __bf16* kbase;  // first prefix key of this partial, KV head g
  const __bf16* vbase;
  const __bf16* ktree;  // tree key 0 of this sequence, KV head g
  const __bf16* vtree;
  int kstride;          // elements between consecutive prefix keys: K (the packed pool when paged)
  int vstride;          // ... of V
  int tstride;          // ... of the tree keys (Hkv * D)
  int kfirst;           // key index (within the sequence) of this partial's first prefix key
  int npk;              // prefix keys of this partial
  bool tree;            // the tree keys follow them
  bool head;            // sliding window, a split within the first 256 keys of the range:
                        // its tiles there are masked per row
  int hbase;            // row i sees keys hbase + depth(i) .. of the range
  int hk0;              // the split's first key, counted from the start of the range
  int tid, lane, wave, l16, grp;
  int b, g, slot, rbase, rend;  // rows [rbase, rend) belong to this workgroup
};

// Splits of a sequence whose key range holds n keys: one per chunk, or one
// (the tree's, or an empty partial) when n = 0.
__device__ inline int split_count(int n, int chunk) { return n > 0 ? (n + chunk - 1) / chunk : 1; }

// Batches of 2..kCompactBatch sequences: the (sequence, split) pair of
// index p in the order (sequence, split), sequences whose length is out of
// the call's bounds holding none.  Every wave computes it on its own (no
// LDS, no barrier): lane l counts the splits of sequences 4l..4l+3, a
// prefix sum over the lanes finds the lane and then the sequence that holds
// pair p.  False when p is past the batch's last split.
template <int PAGED>
__device__ inline bool find_split(const PartialArgs& a, int lane, int p, int* b_out, int* s_out) {
  int len[4];
  if constexpr (PAGED != 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) len[k] = a.seq_lens[min(4 * lane + k, a.B - 1)];
  } else {
    int off[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) off[k] = a.offsets[min(4 * lane + k, a.B)];
#pragma unroll
    for (int k = 0; k < 4; ++k) len[k] = off[k + 1] - off[k];
  }
  int np[4];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int start, n;
    const bool ok = 4 * lane + k < a.B &&
                    key_range(len[k], a.window, a.max_prefix_len, a.seq_cap, &start, &n);
    np[k] = ok ? split_count(n, a.chunk) : 0;
    sum += np[k];
  }
  int inc = sum;  // splits of sequences 0 .. 4*lane+3
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  const uint64_t hit = __ballot(inc > p);
  if (hit == 0) return false;
  const int l = __builtin_ctzll(hit);
  int q = p - __builtin_amdgcn_readlane(inc - sum, l);  // index among lane l's splits
  int b = 4 * l;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int n = __builtin_amdgcn_readlane(np[k], l);
    if (q < n) break;
    q -= n;
    ++b;
  }
  *b_out = b;
  *s_out = q;
  return true;
}

// The prefix keys of this workgroup's split (and whether the tree keys
// follow them), from the sequence's entry in the prefix table.  False when
// the split holds nothing: past the sequence's last split, or a length
// outside the call's bounds (the merge reports that one).
template <int D, int PAGED>
__device__ inline bool locate(Ctx& x) {
  const PartialArgs& a = *x.a;
  const int off0 = PAGED ? 0 : a.offsets[x.b];
  const int L = PAGED ? a.seq_lens[x.b] : a.offsets[x.b + 1] - off0;
  int start, n;
  if (!key_range(L, a.window, a.max_prefix_len, a.seq_cap, &start, &n)) return false;
  // slot s: prefix keys start + [s*chunk, min((s+1)*chunk, n)); the last one
  // (slot 0 when n = 0) also the tree keys
  const int nparts = split_count(n, a.chunk);
  if (x.slot >= nparts) return false;
  const int k0 = x.slot * a.chunk;
  x.npk = max(0, min(a.chunk, n - k0));
  x.kfirst = start + k0;
  x.tree = a.has_tree && x.slot == nparts - 1;
  // window W: node i sees prefix keys from L - W + depth(i) on, i.e. from
  // key n - W + depth(i) <= depth(i) - 1 of the range (within its first 64
  // keys for trees of up to 64 nodes, its first 256 for larger ones)
  x.head = a.window > 0 && x.npk > 0 && k0 < kHeadKeys;
  x.hbase = n - a.window;
  x.hk0 = k0;
  // prefix rows at the caller's strides (a paged pool is packed: Hkv * D)
  x.tstride = a.Hkv * D;
  x.kstride = PAGED ? x.tstride : a.kstride;
  x.vstride = PAGED ? x.tstride : a.vstride;
  const size_t row0 = static_cast<size_t>(off0) + start + k0;
  x.kbase = static_cast<const __bf16*>(a.kp) + row0 * x.kstride + x.g * D;
  x.vbase = static_cast<const __bf16*>(a.vp) + row0 * x.vstride + x.g * D;
  x.ktree = static_cast<const __bf16*>(a.kt) + (static_cast<size_t>(x.b) * a.T * a.Hkv + x.g) * D;
  x.vtree = static_cast<const __bf16*>(a.vt) + (static_cast<size_t>(x.b) * a.T * a.Hkv + x.g) * D;
  if (x.npk == 0) {  // tree only: the prefix pointers may not be dereferenceable
    x.kbase = x.ktree;
    x.vbase = x.vtree;
  }
  return true;
}

// The per-wave body: NT row tiles (rows rbase + 16*(wave + 8*rt) + l16).
// WIN: the sliding-window variant (the head tile's per-row masking exists
// only there, so the other variant's registers are not spent on it).
// BIGT: trees of more than 64 nodes: ceil(T/64) tree tiles, whose mask bits
// each row tile reads from a copy of the sequence's mask words in LDS at the
// start of the tile (W = ceil(T/64) words per row).
// STR: prefix K and V rows at the caller's strides (tree rows packed).
// PAGED: the prefix keys live in pages of a shared pool; the page numbers of
// the split are copied to LDS first.  PAGED == 1 (page size a multiple of
// 64): each 64-key tile lies in one page and gets its own base.  PAGED == 2
// (any page size, a pool below 4 GB): one buffer spans the pool and every
// lane finds its own row's page.
template <int D, int NT, bool WIN, bool BIGT, int PAGED, bool STR>
__device__ __attribute__((always_inline)) inline void run(Ctx& x) {
  using C = Cfg<D>;
  const PartialArgs& a = *x.a;
  const int lane = x.lane, l16 = x.l16, grp = x.grp, wave = x.wave, tid = x.tid;
  const int T = x.a->T;

  // ---- queries of this wave's rows, as the B operand (Q^T) of the QK MFMA,
  // and (trees of up to 64 nodes) the rows' mask words.  Neither depends on
  // the prefix table, so they are issued before it is read and the two
  // memory latencies overlap.
  bf16x8 qf[NT][C::DC];
  uint64_t mws[NT];
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    // a row past the workgroup's rows reads the last real row (without a
    // branch per load): its results are never written
    const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
    const int rr = r < x.rend ? r : x.rend - 1;
    const int i = rr / a.G;
    const int hh = rr % a.G;
    const __bf16* qp = static_cast<const __bf16*>(a.q) +
                       ((static_cast<size_t>(x.b) * a.T + i) * a.Hq + x.g * a.G + hh) * D + grp * 8;
#pragma unroll
    for (int c = 0; c < C::DC; ++c) qf[rt][c] = *reinterpret_cast<const bf16x8*>(qp + c * 32);
    mws[rt] = (!BIGT && a.mask != nullptr) ? a.mask[static_cast<size_t>(x.b) * a.T + i] : 0;
  }
  // this workgroup's keys; none (a split past the sequence's last, or an
  // invalid length, which the merge reports): nothing to do
  if (!locate<D, PAGED>(x)) return;
  const int npk = x.npk;
  const bool tree = x.tree;
  const bool head = WIN && x.head;

  uint32_t vbits[NT];  // tree: this lane's mask bits (keys 8grp..8grp+7 of each block)
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
    const bool ok = r < x.rend;
    const int i = (ok ? r : x.rend - 1) / a.G;
    vbits[rt] = 0xffffu;
    if (!BIGT && (tree || head) && ok) {
      const uint64_t mw = mws[rt];
      if (tree) {
        vbits[rt] = static_cast<uint32_t>((mw >> (8 * grp)) & 0xffu) |
                    (static_cast<uint32_t>((mw >> (32 + 8 * grp)) & 0xffu) << 8);
      }
      if (head) {  // bits 16..23: the row's first visible key of the window
        const int sh = min(max(x.hbase + static_cast<int>(__popcll(mw)), 0), 63);
        vbits[rt] |= static_cast<uint32_t>(sh) << 16;
      }
    }
    if (BIGT && head && ok) {  // depth over the row's W mask words; up to 255 keys hidden
      int depth = 0;
      for (int w = 0; w < a.W; ++w) {
        depth += static_cast<int>(__popcll(a.mask[(static_cast<size_t>(x.b) * a.T + i) * a.W + w]));
      }
      vbits[rt] |= static_cast<uint32_t>(min(max(x.hbase + depth, 0), 255)) << 16;
    }
  }

  // Wait for these loads here, before any tile load is in flight (a later
  // first use would make the wait cover the tile loads too).
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
    for (int c = 0; c < C::DC; ++c) asm volatile("" : "+v"(qf[rt][c]));
    asm volatile("" : "+v"(vbits[rt]));
  }

  // Online softmax state per row, in raw score units s = q.k, relative to a
  // reference max m of the row:
  //   nmc   -m*c2, the exponent offset (kNoRef while the row has seen no
  //         key: far above any real offset, so the first key moves the
  //         reference and scales the empty accumulator by 2^-kNoRef = 0,
  //         and masked scores still give 2^-inf = 0, never inf - inf),
  //   thr   m + 15/c2 = -nmc/c2 + 15/c2, updated with the reference: a score
  //         above it would give a probability above 2^15 (fp16 holds up to
  //         65504),
  //   lsum  sum of this lane's probabilities as rounded to fp16 for P.V (the
  //         output is normalised by the same values it accumulates).
  constexpr float kNoRef = 1e30f;
  f32x4 acc[C::DT][NT];
  float nmc[NT], lsum[NT], thr[NT];
  const float c2 = a.scale_log2;
  const float t8 = a.headroom;             // 15 / c2
  const float nic2 = a.neg_inv_scale_log2;  // -1 / c2
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    nmc[rt] = kNoRef;
    thr[rt] = fmaf(kNoRef, nic2, t8);
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt][rt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  // prefix tiles, then the tree tiles (one for T <= 64)
  const int ptiles = (npk + kTile - 1) / kTile;
  const int ntiles = ptiles + (tree ? (BIGT ? (T + kTile - 1) / kTile : 1) : 0);
  // STR: a strided prefix cache (other row strides than the packed tree);
  // otherwise one stride serves every tile
  const int kstride = x.kstride;
  const int vstride = STR ? x.vstride : kstride;
  const int tstride = STR ? x.tstride : kstride;

  // ---- per-lane LDS offsets of the MFMA operands.  Stage, block half, sub
  // block, d tile and V^T buffer are compile-time and go into the 16-bit
  // offset field of the LDS instructions; the region bases above 64 KB are
  // folded into the lane offsets (kept opaque so the compiler does not split
  // them back out).
  int koff[C::DC];
  {
    const int key = 8 * (l16 >> 2) + (l16 & 3);  // block-relative key of sub 0
    const int sw = kswz<D>(key);                  // the same for key + 4 and key + 32
#pragma unroll
    for (int c = 0; c < C::DC; ++c) koff[c] = C::K0 + key * C::ROW + (((c * 4 + grp) ^ sw) << 4);
  }
  // V^T operand of d tile dt for lane (grp, l16): row 16dt + l16, cell
  // 4h + grp for block half h; the XOR term of cell 4h + grp in a row of
  // d tile dt is ((4h + grp) ^ dt), whose bit 2 is uniform.
  int voff[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) {
    voff[d4] = C::T0 + l16 * kVtRow + (((grp ^ d4) & 3) << 4);
    asm volatile("" : "+v"(voff[d4]));
  }

  // ---- staging.  Tile t uses K tile, raw V tile and V^T buffer t % 3;
  // every stage index below is a compile-time constant (the tile loop is
  // unrolled by three).
  // K: 16-byte chunks straight to the K tile, swizzled by key.
  // V: item (key pair m, d chunk c), VIPT per thread: item tid + i * kThreads
  // (threads below VTHREADS); keys 2m and 2m+1 of chunk c land in two 1 KB
  // slots of the raw V tile at this lane's position, so only this thread
  // reads them back.
  char* const sm = x.smem;
  const bool vstage = C::VTHREADS == kThreads || tid < C::VTHREADS;  // compile-time true when every thread stages V
  // Loads go through buffer descriptors whose range ends with the tile's last
  // real key, so rows past it read as zeros (and are masked); per-thread byte
  // offsets within a tile:
  int ksoff[C::KDMA];
#pragma unroll
  for (int j = 0; j < C::KDMA; ++j) {
    const int row = (j * kWaves + wave) * C::ROWS_PER_DMA + lane / C::KC16;
    ksoff[j] = (row * kstride + (((lane % C::KC16) ^ kswz<D>(row)) * 8)) * 2;
  }
  int vsoff[C::VIPT][2];
#pragma unroll
  for (int i = 0; i < C::VIPT; ++i) {
    const int it = tid + i * kThreads, vm = it / C::KC16, vc = it % C::KC16;
    vsoff[i][0] = ((2 * vm) * vstride + vc * 8) * 2;
    vsoff[i][1] = vsoff[i][0] + vstride * 2;
  }
  // PAGED: the split's page numbers in LDS (after the mask words, if any)
  const int32_t* pst = reinterpret_cast<const int32_t*>(sm + C::SMEM + (BIGT ? kMaskStash : 0));
  const int p0 = PAGED ? (a.page_shift >= 0 ? x.kfirst >> a.page_shift : x.kfirst / a.page_size) : 0;
  // PAGED == 2: pool row of the split's key k (relative to kfirst), from the
  // LDS page table
  auto pool_row = [&](int k) -> uint32_t {
    const int key = x.kfirst + k;
    const int slot = a.page_shift >= 0 ? key >> a.page_shift : key / a.page_size;
    const int in_page = a.page_shift >= 0 ? key & (a.page_size - 1) : key % a.page_size;
    return static_cast<uint32_t>(pst[slot - p0]) * static_cast<uint32_t>(a.page_size) +
           static_cast<uint32_t>(in_page);
  };
  auto dma = [&](int S, int t) {
    const bool tt = BIGT ? t >= ptiles : t == ptiles;  // a tree tile
    const int u = BIGT ? t - ptiles : 0;                // its index among the tree tiles
    const int nrows = tt ? (BIGT ? min(kTile, T - u * kTile) : T) : min(kTile, npk - t * kTile);
    // first row of the tile; row strides: the caller's for prefix tiles, the
    // packed tree layout for tree tiles
    const size_t trow = tt ? (BIGT ? static_cast<size_t>(u) * kTile : 0) : static_cast<size_t>(t) * kTile;
    const int ks = tt ? tstride : kstride;
    const int vs = tt ? tstride : vstride;
    const __bf16* kb = (tt ? x.ktree : x.kbase) + trow * ks;
    const __bf16* vb = (tt ? x.vtree : x.vbase) + trow * vs;
    if constexpr (PAGED == 2) {
      if (!tt) {  // one buffer over the pool (from KV head g on); rows by lane below
        kb = static_cast<const __bf16*>(a.kp) + x.g * D;
        vb = static_cast<const __bf16*>(a.vp) + x.g * D;
      }
    }
    if constexpr (PAGED == 1) {
      if (!tt) {  // tile t: keys kfirst + 64t .. of page pst[(kfirst + 64t) / P - p0]
        const int key = x.kfirst + t * kTile;
        const int slot = a.page_shift >= 0 ? key >> a.page_shift : key / a.page_size;
        const int in_page = a.page_shift >= 0 ? key & (a.page_size - 1) : key % a.page_size;
        const int pg = __builtin_amdgcn_readfirstlane(pst[slot - p0]);
        const size_t row = static_cast<size_t>(pg) * a.page_size + in_page;
        kb = static_cast<const __bf16*>(a.kp) + row * kstride + x.g * D;
        vb = static_cast<const __bf16*>(a.vp) + row * kstride + x.g * D;
      }
    }
    const bool lane_rows = PAGED == 2 && !tt;
    const int pool_range = static_cast<int>(a.pool_bytes - static_cast<uint32_t>(x.g * D * 2));
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(kb), 0,
                                                      lane_rows ? pool_range : nrows * ks * 2, kBufferFlags);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(vb), 0,
                                                      lane_rows ? pool_range : nrows * vs * 2, kBufferFlags);
    // a strided prefix with other strides than the tree: the tree tile's
    // per-thread offsets at the tree stride
    const bool restride = STR && tt && (kstride != tstride || vstride != tstride);
#pragma unroll
    for (int j = 0; j < C::KDMA; ++j) {
      char* dst = sm + Cfg<D>::K0 + S * Cfg<D>::BUF + (j * kWaves + wave) * 1024;
      int vo = ksoff[j];
      if (restride) {
        const int row = (j * kWaves + wave) * C::ROWS_PER_DMA + lane / C::KC16;
        vo = (row * tstride + (((lane % C::KC16) ^ kswz<D>(row)) * 8)) * 2;
      }
      if constexpr (PAGED == 2) {
        if (lane_rows) {  // rows past the tile's last key repeat it (they are masked)
          const int row = (j * kWaves + wave) * C::ROWS_PER_DMA + lane / C::KC16;
          const uint32_t pr = pool_row(t * kTile + min(row, nrows - 1));
          vo = static_cast<int>((pr * static_cast<uint32_t>(kstride) +
                                 static_cast<uint32_t>(((lane % C::KC16) ^ kswz<D>(row)) * 8)) * 2u);
        }
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)dst, 16, vo, 0, 0, 0);
    }
    if (vstage) {
#pragma unroll
      for (int i = 0; i < C::VIPT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          char* dst = sm + Cfg<D>::R0 + S * Cfg<D>::BUF +
                      (j * (Cfg<D>::VITEMS / 64) + i * kWaves + wave) * 1024;
          int vo = vsoff[i][j];
          if (restride) {
            const int it = tid + i * kThreads, vm = it / C::KC16, vc = it % C::KC16;
            vo = ((2 * vm + j) * tstride + vc * 8) * 2;
          }
          if constexpr (PAGED == 2) {
            if (lane_rows) {
              const int it = tid + i * kThreads, vm = it / C::KC16, vc = it % C::KC16;
              const uint32_t pr = pool_row(min(t * kTile + 2 * vm + j, t * kTile + nrows - 1));
              vo = static_cast<int>((pr * static_cast<uint32_t>(kstride) + static_cast<uint32_t>(vc * 8)) * 2u);
            }
          }
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)dst, 16, vo, 0, 0, 0);
        }
    }
  };
  // This thread's V items, bf16 -> fp16, transposed into V^T buffer S: for
  // each feature d = 8c + e, the dword (key 2m, key 2m+1); the eight cells of
  // an item are 144 bytes apart (vt_off is linear in e for d = 8c + e).
  int rdoff = C::R0 + wave * 1024 + 16 * lane;
  int wroff[C::VIPT];
#pragma unroll
  for (int i = 0; i < C::VIPT; ++i) {
    const int it = tid + i * kThreads, vm = it / C::KC16, vc = it % C::KC16;
    wroff[i] = C::T0 + vt_off(8 * vc, vm >> 2) + 4 * (vm & 3);
    asm volatile("" : "+v"(wroff[i]));
  }
  asm volatile("" : "+v"(rdoff));
  auto convert = [&](int S) {
    if (vstage) {
#pragma unroll
      for (int i = 0; i < C::VIPT; ++i) {
        const char* rb = sm + rdoff + S * C::BUF + i * kWaves * 1024;
        const u32x4 u0 = *reinterpret_cast<const u32x4*>(rb);
        const u32x4 u1 = *reinterpret_cast<const u32x4*>(rb + (C::VITEMS / 64) * 1024);
        char* wb = sm + wroff[i] + S * C::VT;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          *reinterpret_cast<uint32_t*>(wb + e * kVtRow) = pack_f16_of_bf16(u0[e >> 1], u1[e >> 1], e & 1);
        }
      }
    }
  };
  auto wait_own = [&](int later) {
    if (vstage) {
      wait_dma_except<C::DPT_V>(later);
    } else {
      wait_dma_except<C::DPT_K>(later);
    }
  };

  // ---- one 32-key block: block half H of the tile in stage S, whose first
  // `valid` keys are real (prefix or tree keys); tree blocks also apply the
  // ancestor mask.
  //
  // The K operands of a block (all d chunks, both 16-key halves) are loaded
  // into registers ahead of it, during the P.V of the block before, so its
  // QK products start at once.  The QK products run one row tile at a time,
  // and the softmax of row tile rt is computed while the products of row tile
  // rt+1 are in the matrix cores.  The P.V products follow once every row
  // tile has its probabilities, one d tile of V^T at a time.
  bf16x8 ka[C::DC][2];
  auto kload = [&](int S, auto H_) {
    constexpr int H = decltype(H_)::value;
    // (by 16-key half: the order in which the QK chains use them)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int c = 0; c < C::DC; ++c)
        ka[c][sub] = *reinterpret_cast<const bf16x8*>(sm + koff[c] + S * C::BUF + H * 32 * C::ROW +
                                                      sub * 4 * C::ROW);
  };
  f16x8 P[NT];  // probabilities of the current block (the B operand P^T of P.V)

  // S^T = K . Q^T for row tile rt; keys past the end, tree keys outside the
  // row's branch and, in the window's head tile, keys before the row's window
  // get -inf
  // hk >= 0: a window head tile whose first key is key hk of the range
  auto qk = [&](f32x4 (&s)[2], int rt, int H, int valid, bool treeblk, int hk, auto MASK_) {
    if constexpr (D == 128) {
      // the two accumulation chains (16-key halves) one after the other:
      // products into the accumulator the previous one wrote issue sooner
      // (1% fewer cycles per tile than alternating them)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int c = 0; c < C::DC; ++c) {
          s[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              ka[c][sub], qf[rt][c], c == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : s[sub], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
    } else {  // (the D = 64 variants spill with that order)
#pragma unroll
      for (int c = 0; c < C::DC; ++c)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
          s[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              ka[c][sub], qf[rt][c], c == 0 ? (f32x4){0.f, 0.f, 0.f, 0.f} : s[sub], 0, 0, 0);
    }
    if constexpr (decltype(MASK_)::value) {
      // one bit per key of this lane: real key and (tree) an ancestor; made
      // opaque so the per-key conditions are formed here, not kept for the
      // whole loop
      const int nin = min(max(valid - 8 * grp, 0), 8);
      uint32_t bits = (!treeblk ? 0xffu : H ? (vbits[rt] >> 8) : vbits[rt]) & ((1u << nin) - 1u);
      if (WIN && hk >= 0) {  // this lane's keys are hk + 32H + 8grp + 0..7
        const int sh = static_cast<int>(vbits[rt] >> 16) - (hk + 32 * H + 8 * grp);
        bits &= sh <= 0 ? 0xffu : sh >= 8 ? 0u : (0xffu << sh);
      }
      asm volatile("" : "+v"(bits));
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (!((bits >> (4 * sub + v)) & 1u)) s[sub][v] = -INFINITY;
        }
    }
  };
  // p = 2^(s*c2 - m*c2) in fp16 for P.V, and their sum (the same fp16
  // values, accumulated in fp32)
  auto probs = [&](const f32x4 (&s)[2], int rt) {
    float p[8];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int v = 0; v < 4; ++v) p[4 * sub + v] = __builtin_amdgcn_exp2f(fmaf(s[sub][v], c2, nmc[rt]));
    f16x2 hp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      hp[k] = __builtin_convertvector((f32x2){p[2 * k], p[2 * k + 1]}, f16x2);
      lsum[rt] = add_f16x2(hp[k], lsum[rt]);
    }
    P[rt] = __builtin_bit_cast(f16x8, (u32x4){__builtin_bit_cast(uint32_t, hp[0]),
                                              __builtin_bit_cast(uint32_t, hp[1]),
                                              __builtin_bit_cast(uint32_t, hp[2]),
                                              __builtin_bit_cast(uint32_t, hp[3])});
  };
  auto lane_max = [](const f32x4 (&s)[2]) {
    const float m0 = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
    const float m1 = fmaxf(fmaxf(s[0][3], s[1][0]), s[1][1]);
    return fmaxf(fmaxf(s[1][2], s[1][3]), fmaxf(m0, m1));
  };

  // Move row tile rt's references to the block's row maxima where a score
  // passed the threshold, and rescale what it has accumulated.
  auto rescale = [&](int rt, float lm) {
    const float mt = group_max(lm);
    const bool up = mt > thr[rt];  // this row's reference moves to mt
    const float n_new = up ? -mt * c2 : nmc[rt];
    const float alpha = up ? __builtin_amdgcn_exp2f(n_new - nmc[rt]) : 1.f;
    nmc[rt] = n_new;
    thr[rt] = fmaf(n_new, nic2, t8);
    lsum[rt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt][rt] *= alpha;
  };

  // Online softmax in base 2, with a lazily moved reference max.  Each lane
  // checks its own eight scores of a row against the row threshold; only
  // when some score would give a probability above 2^15 does the wave reduce
  // the row maxima across lane groups, move the reference and rescale.
  // Keeping probabilities up to 2^15 against a stale reference is exact: the
  // final normalisation and the lse use the same reference.
  //
  // Row tile by row tile: the check of row tile rt, then its exponentials
  // with the QK products of row tile rt+1 in flight.
  auto qk_softmax = [&](auto H_, int valid, bool treeblk, int hk, auto MASK_) {
    constexpr int H = decltype(H_)::value;
    f32x4 s[2][2];
    float lm[2];
    qk(s[0], 0, H, valid, treeblk, hk, MASK_);
    lm[0] = lane_max(s[0]);
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
      if (__builtin_expect(__any(lm[rt & 1] > thr[rt]), 0)) rescale(rt, lm[rt & 1]);
      probs(s[rt & 1], rt);
      if (rt + 1 < NT) {
        qk(s[(rt + 1) & 1], rt + 1, H, valid, treeblk, hk, MASK_);
        lm[(rt + 1) & 1] = lane_max(s[(rt + 1) & 1]);
        // issue order: the products of row tile rt+1 one at a time between
        // the vector instructions of row tile rt
#pragma unroll
        for (int k = 0; k < 2 * C::DC; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
    }
  };

  // O^T += V^T . P^T for block half H of stage S, one d tile at a time;
  // `next` loads the K operands of the following block meanwhile
  auto pv = [&](int S, auto H_, auto next) {
    constexpr int H = decltype(H_)::value;
    // V^T rows 16dt + l16, cell 4H + grp
    f16x8 va[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int uni = S * C::VT + dt * 16 * kVtRow + ((((4 * H) ^ dt) & 4) << 4);
      va[dt] = *reinterpret_cast<const f16x8*>(sm + voff[dt & 3] + uni);
    }
    next();
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
        acc[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[dt], P[rt], acc[dt][rt], 0, 0, 0);
    // issue order: three V^T reads ahead, then per d tile its products and
    // one more read (the last two d tiles: the next block's K operands, DC
    // each)
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int dt = 0; dt + 3 < C::DT; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, Cfg<D>::DC, 0);
    }
  };

  // ---- Schedule.  One barrier per tile, before the P.V of its last block:
  // by then every thread has converted its V items of tile t+1 (so V^T of
  // tile t+1 and, through the loads it waited for, K of tile t+1 are
  // complete), and every wave has finished reading K of tile t (whose stage
  // then takes the loads of tile t+3) and the V^T of tile t-1.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // S = t % kStages; a compile-time constant in the unrolled main loop.
  auto tile = [&](int S, int t, auto MASK_) {
    const int SN = S + 1 < kStages ? S + 1 : 0;
    const bool tt = BIGT ? t >= ptiles : t == ptiles;
    const int u = BIGT ? t - ptiles : 0;
    const int nk = tt ? (BIGT ? min(kTile, T - u * kTile) : T) : min(kTile, npk - t * kTile);  // real keys of this tile
    if constexpr (BIGT) {
      if (tt) {  // this lane's mask bits of tree tile u, from the LDS copy
        const uint64_t* mst = reinterpret_cast<const uint64_t*>(sm + C::SMEM);
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
          const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
          const uint64_t mw = r < x.rend ? mst[(r / a.G) * a.W + u] : ~0ull;
          vbits[rt] = (vbits[rt] & 0xffff0000u) |  // (keeps a window's first-key bits)
                      static_cast<uint32_t>((mw >> (8 * grp)) & 0xffu) |
                      (static_cast<uint32_t>((mw >> (32 + 8 * grp)) & 0xffu) << 8);
        }
      }
    }
    // window head tiles: those within the first 256 keys of the range (a row
    // hides at most depth - 1 <= 255 of them; 63 for trees of up to 64 nodes)
    const int hb = (head && !tt && x.hk0 + t * kTile < kHeadKeys) ? x.hk0 + t * kTile : -1;
    const bool more = t + 1 < ntiles;
    // a tile whose real keys all lie in its first block (the last tile of a
    // split, a tree of up to 32 nodes) skips the second: fully masked, it
    // would add exact zeros
    const bool two = !decltype(MASK_)::value || nk > 32;
    qk_softmax(I0{}, min(nk, 32), tt, hb, MASK_);
    pv(S, I0{}, [&] { kload(S, I1{}); });
    if (two) qk_softmax(I1{}, nk - 32, tt, hb, MASK_);
    if (more) {
      wait_own(min(1, ntiles - 2 - t));
      convert(SN);
    }
    lds_barrier();
    // (after the last tile the K operand load reads a stage nobody uses;
    // harmless)
    if (two) {
      pv(S, I1{}, [&] { kload(SN, I0{}); });
    } else {
      kload(SN, I0{});
    }
    // stage S is free since the barrier; issued here rather than right after
    // it, the loads no longer hold up the P.V products of every wave at once
    if (t + 3 < ntiles) dma(S, t + 3);
  };
  if constexpr (BIGT) {
    if (tree) {  // the sequence's mask words to LDS, before any tile load is in flight
      const uint64_t* mrow = a.mask + static_cast<size_t>(x.b) * a.T * a.W;
      uint64_t* mst = reinterpret_cast<uint64_t*>(sm + C::SMEM);
      for (int k = tid; k < a.T * a.W; k += kThreads) mst[k] = mrow[k];
    }
  }
  if constexpr (PAGED) {
    // page numbers of this split's keys; a page outside the pool makes the
    // partial NaN (the merge then writes NaN rows) and reads nothing
    const int np = npk > 0 ? (x.kfirst + npk - 1) / a.page_size - p0 + 1 : 0;
    int32_t* pw = reinterpret_cast<int32_t*>(sm + C::SMEM + (BIGT ? kMaskStash : 0));
    bool bad = false;
    for (int k = tid; k < np; k += kThreads) {
      const int pg = a.block_table[static_cast<size_t>(x.b) * a.max_pages + p0 + k];
      bad = bad || pg < 0 || pg >= a.num_pages;
      pw[k] = pg;
    }
    if (__syncthreads_or(bad)) {
      const size_t pb = (static_cast<size_t>(x.b * a.Hkv + x.g) * a.slots + x.slot) * a.R;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
        if (r < x.rend && grp == 0) {
          a.lse_part[pb + r] = __builtin_nanf("");
          a.scale_part[pb + r] = 0.f;
        }
      }
      return;
    }
  }
  // Tile 0 alone first: every workgroup starts at once, and tile 0 arrives
  // sooner when the loads of the next tiles are not competing with it.
  // (no tile at all only for an empty prefix without tree keys: the partial
  // is then empty, lse -inf)
  if (ntiles > 0) {
    dma(0, 0);
    wait_own(0);
    if (ntiles > 1) dma(1, 1);
    if (ntiles > 2) dma(2, 2);
    convert(0);
  }
  lds_barrier();
  kload(0, I0{});
  // Full prefix tiles need no mask; the last prefix tile when partial and
  // the tree tile run masked after them, with the stage a run-time value.
  // The window variant runs every tile that way (its splits hold a few
  // tiles, and the first of a sequence is masked per row).
  const int nfull = WIN ? 0 : npk / kTile;
  int t = 0;
  for (; t + kStages <= nfull; t += kStages) {
    tile(0, t, std::false_type{});
    tile(1, t + 1, std::false_type{});
    tile(2, t + 2, std::false_type{});
  }
  for (; t < ntiles; ++t) tile(t % kStages, t, std::true_type{});

  // ---- normalise and write the partial.  A row of o = acc / l goes out as
  // int16 snorm values acc / max|acc| with the row's max|o| as its scale
  // (the 16-bit form halves the partials' memory traffic; its error is at most
  // 2^-16 of the row's largest magnitude).  Row r's D features are spread
  // over the four lane groups, so the max takes a reduction across them.
  // The workgroup's rows are consecutive in the partial buffer: they are
  // gathered in LDS (free once every wave is past its last tile) and leave
  // as whole 16-byte chunks, each store instruction covering 1 KB of
  // contiguous memory (written from the MFMA layout directly, a store would
  // cover 16 separate 32-byte pieces).
  const size_t pbase = (static_cast<size_t>(x.b * a.Hkv + x.g) * a.slots + x.slot) * a.R;
  lds_barrier();
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    const float l = group_sum(lsum[rt]);
    float mx = 0.f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(acc[dt][rt][i]));
    mx = group_max(mx);
    const float inv = mx > 0.f ? 1.f / mx : 0.f;
    const int r = x.rbase + 16 * (wave + kWaves * rt) + l16;
    if (r < x.rend) {
      char* ob = sm + (r - x.rbase) * C::OUT_PITCH + 8 * grp;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const f32x4 v = acc[dt][rt] * inv;
        const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(v[0], v[1]));
        const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(v[2], v[3]));
        *reinterpret_cast<u32x2*>(ob + dt * 32) = (u32x2){lo, hi};
      }
      if (grp == 0) {
        a.lse_part[pbase + r] = -nmc[rt] + __builtin_amdgcn_logf(l);
        a.scale_part[pbase + r] = l > 0.f ? mx / l : 0.f;
      }
    }
  }
  lds_barrier();
  char* const og = reinterpret_cast<char*>(static_cast<int16_t*>(a.o_part) + (pbase + x.rbase) * D);
  const int nchunks = (x.rend - x.rbase) * C::KC16;
  for (int k = tid; k < nchunks; k += kThreads) {
    const int rr = k / C::KC16, c = k % C::KC16;
    *reinterpret_cast<u32x4*>(og + 16 * k) = *reinterpret_cast<const u32x4*>(sm + rr * C::OUT_PITCH + 16 * c);
  }
}

template <int D, int TPW, bool WIN, bool BIGT, int PAGED, bool STR>
__global__ __launch_bounds__(kThreads, 2) void partial_mfma_kernel(PartialArgs a) {
  using C = Cfg<D>;
  static_assert(!(WIN && PAGED == 1), "a window starts anywhere: rows by lane over a paged cache");
  static_assert(!(STR && (WIN || PAGED)), "strided rows only for the packed-cache verification variant");
  __shared__ __attribute__((aligned(1024)))
  char smem[C::SMEM + (BIGT ? kMaskStash : 0) + (PAGED ? kPageStash : 0)];

  Ctx x;
  x.a = &a;
  x.smem = smem;
  x.tid = threadIdx.x;
  x.lane = threadIdx.x & 63;
  x.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  x.l16 = x.lane & 15;
  x.grp = x.lane >> 4;
  x.g = blockIdx.x;
  int rb;
  if (a.B > 1 && a.B <= kCompactBatch) {  // splits packed in dispatch order
    const int j = blockIdx.y + gridDim.y * blockIdx.z;
    if (!find_split<PAGED>(a, x.lane, j / a.row_blocks, &x.b, &x.slot)) return;
    rb = j % a.row_blocks;
  } else {
    x.slot = blockIdx.y;
    x.b = blockIdx.z / a.row_blocks;
    rb = blockIdx.z % a.row_blocks;
  }
  x.rbase = rb * a.rows_per_wg;

  // Row tiles of this workgroup and how many fall to this wave.  Every wave
  // runs the same sequence of tiles, blocks and barriers; only the number of
  // row tiles it computes differs.  (Its keys are located inside run(),
  // once the query loads are in flight.)
  x.rend = min(a.R, x.rbase + a.rows_per_wg);
  const int tiles = (x.rend - x.rbase + 15) / 16;
  const int ntw = (tiles - x.wave + kWaves - 1) / kWaves;  // tiles wave, wave+8, ... < tiles
  if constexpr (TPW >= 3) {
    if (ntw >= 3) {
      run<D, 3, WIN, BIGT, PAGED, STR>(x);
      return;
    }
  }
  if constexpr (TPW >= 2) {
    if (ntw == 2) {
      run<D, 2, WIN, BIGT, PAGED, STR>(x);
      return;
    }
  }
  run<D, 1, WIN, BIGT, PAGED, STR>(x);  // one tile, or none: a wave without rows still stages and syncs
}

template <int D, bool WIN, bool BIGT, int PAGED, bool STR>
hipError_t launch_d(int tpw, dim3 grid, PartialArgs a, hipStream_t stream) {
  switch (tpw) {
    case 1: hipLaunchKernelGGL((partial_mfma_kernel<D, 1, WIN, BIGT, PAGED, STR>), grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((partial_mfma_kernel<D, 2, WIN, BIGT, PAGED, STR>), grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((partial_mfma_kernel<D, 3, WIN, BIGT, PAGED, STR>), grid, dim3(kThreads), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <bool WIN, bool BIGT, int PAGED, bool STR = false>
hipError_t launch_dd(int D, int tpw, dim3 grid, PartialArgs a, hipStream_t stream) {
  return D == 128 ? launch_d<128, WIN, BIGT, PAGED, STR>(tpw, grid, a, stream)
                  : launch_d<64, WIN, BIGT, PAGED, STR>(tpw, grid, a, stream);
}

}  // namespace

// Launchers of the variants, one translation unit per group (external
// linkage; the kernels themselves stay local to their unit).
hipError_t launch_mfma_plain(bool big, int D, int tpw, dim3 grid, PartialArgs a, hipStream_t s);
hipError_t launch_mfma_strided(bool big, int D, int tpw, dim3 grid, PartialArgs a, hipStream_t s);
hipError_t launch_mfma_window(bool big, bool lane_paged, int D, int tpw, dim3 grid, PartialArgs a,
                              hipStream_t s);
hipError_t launch_mfma_paged(bool big, bool lane_paged, int D, int tpw, dim3 grid, PartialArgs a,
                             hipStream_t s);

}  // namespace ltree
