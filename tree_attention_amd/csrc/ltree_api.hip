// C ABI of libltree: argument checks, work planning, kernel launches.
// The operations are defined in include/ltree.h.
#include <atomic>
#include <cmath>

#include "ltree_internal.h"

// The partials of ltree_attn_noalloc: each device the library runs on holds
// its own copy from the first call there until the process ends.  In host
// code this name is a stand-in, not a device address: kernels get the
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[LTREE_NOALLOC_SCRATCH_BYTES];

namespace ltree {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];        // 0 = not queried yet
std::atomic<void*> g_scratch_ptr[kMaxDevices];   // nullptr = not looked up yet
}  // namespace

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  const bool cached = dev < kMaxDevices;  // devices past the table are asked every time
  int n = cached ? g_cu_count[dev].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    n = 256;
  }
  if (cached) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Device address of device dev's copy of `scratch` (dev current), looked up
// once per device; nullptr if the lookup fails.
static void* scratch_on(int dev) {
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

// The plan of a call on the current device.
static bool plan_here(int B, int T, int Hq, int Hkv, int D, int max_prefix_len, Plan* p,
                      int window = 0, int page_size = 0, long row_stride = 0) {
  return make_plan(B, T, Hq, Hkv, D, max_prefix_len, device_cu_count(), p, window, page_size,
                   row_stride);
}

}  // namespace ltree

using ltree::Plan;
using ltree::aligned;
using ltree::plan_here;

extern "C" {

int ltree_version(void) { return LTREE_VERSION; }

const char* ltree_status_string(int status) {
  switch (status) {
    case LTREE_OK: return "ok";
    case LTREE_ERR_INVALID_ARG: return "invalid argument";
    case LTREE_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case LTREE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case LTREE_ERR_HIP: return "HIP runtime error";
    case LTREE_ERR_SCRATCH: return "needs more scratch than LTREE_NOALLOC_SCRATCH_BYTES";
    default: return "unknown status";
  }
}

int ltree_build_mask(const int32_t* parent, int B, int T, uint64_t* mask, int32_t* status,
                     hipStream_t stream) {
  if (parent == nullptr || mask == nullptr || B < 1 || T < 1) return LTREE_ERR_INVALID_ARG;
  if (T > LTREE_MAX_TREE) return LTREE_ERR_UNSUPPORTED;
  if (static_cast<long>(B) * T > (1L << 30)) return LTREE_ERR_INVALID_ARG;
  return ltree::launch_mask_build(parent, B, T, mask, status, stream) == hipSuccess
             ? LTREE_OK
             : LTREE_ERR_HIP;
}

size_t ltree_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_prefix_len) {
  Plan p;
  return plan_here(B, T, Hq, Hkv, D, max_prefix_len, &p) ? p.bytes : 0;
}

using ltree::check_sizes;

// A paged prefix: pools of pages and the table that maps each sequence's
// keys to them (see ltree_attn_paged).
struct Paging {
  const int32_t* seq_lens = nullptr;
  const int32_t* block_table = nullptr;
  int page_size = 0, max_pages = 0, num_pages = 0;
  uint32_t pool_bytes = 0;
  int seq_cap = 0;
};

// Prefix row strides in elements (0, 0: packed rows of Hkv * D).
struct Strides {
  long k = 0, v = 0;
};

// Partials of prefix (+ tree, when has_tree) attention into the workspace;
// window > 0: sliding-window attention (max_prefix_len is then window - 1);
// pg.block_table != nullptr: a paged prefix (k_prefix/v_prefix are the pools).
static int partials(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                    const void* q, const void* k_prefix, const void* v_prefix,
                    const int32_t* prefix_offsets, int max_prefix_len, bool has_tree,
                    const void* k_tree, const void* v_tree, const uint64_t* mask,
                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                    int window = 0, const Paging& pg = Paging(), const Strides& rs = Strides()) {
  if (dtype != LTREE_F32 && dtype != LTREE_BF16) return LTREE_ERR_INVALID_ARG;
  const int st = check_sizes(B, T, Hq, Hkv, D, max_prefix_len);
  if (st != LTREE_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.f)) return LTREE_ERR_INVALID_ARG;
  if (q == nullptr || workspace == nullptr) return LTREE_ERR_INVALID_ARG;
  if (pg.block_table == nullptr ? prefix_offsets == nullptr : pg.seq_lens == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (has_tree && (k_tree == nullptr || v_tree == nullptr || mask == nullptr)) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (max_prefix_len > 0 && (k_prefix == nullptr || v_prefix == nullptr)) {
    return LTREE_ERR_INVALID_ARG;
  }
  // 16-byte vector loads of q/k/v rows
  if (!aligned(q, 16) || (has_tree && (!aligned(k_tree, 16) || !aligned(v_tree, 16))) ||
      (k_prefix && !aligned(k_prefix, 16)) || (v_prefix && !aligned(v_prefix, 16))) {
    return LTREE_ERR_INVALID_ARG;
  }
  const long packed = static_cast<long>(Hkv) * D;
  const long kstride = rs.k > 0 ? rs.k : packed, vstride = rs.v > 0 ? rs.v : packed;
  Plan p;
  if (!plan_here(B, T, Hq, Hkv, D, max_prefix_len, &p, window, pg.page_size,
                 kstride > vstride ? kstride : vstride)) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (workspace_bytes < p.bytes || !aligned(workspace, 256)) return LTREE_ERR_WORKSPACE;

  ltree::PartialArgs a{};
  a.q = q;
  a.kp = k_prefix;
  a.vp = v_prefix;
  a.offsets = prefix_offsets;
  a.kt = k_tree;
  a.vt = v_tree;
  a.mask = mask;
  a.o_part = static_cast<char*>(workspace) + p.o_part_off;
  a.scale_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.scale_part_off);
  a.lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.lse_part_off);
  a.B = B;
  a.T = T;
  a.W = (T + 63) / 64;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = p.G;
  a.R = p.R;
  a.chunk = p.chunk;
  a.max_chunks = p.max_chunks;
  a.slots = p.slots;
  a.max_prefix_len = p.max_prefix_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.headroom = 15.f / a.scale_log2;
  a.neg_inv_scale_log2 = -1.f / a.scale_log2;
  a.has_tree = has_tree ? 1 : 0;
  a.window = window;
  a.kstride = static_cast<int>(kstride);
  a.vstride = static_cast<int>(vstride);
  a.seq_cap = pg.block_table != nullptr ? pg.seq_cap : p.seq_cap;
  a.seq_lens = pg.seq_lens;
  a.block_table = pg.block_table;
  a.page_size = pg.page_size;
  a.max_pages = pg.max_pages;
  a.num_pages = pg.num_pages;
  a.pool_bytes = pg.pool_bytes;
  a.page_shift = -1;
  if (pg.page_size > 0 && (pg.page_size & (pg.page_size - 1)) == 0) {
    a.page_shift = __builtin_ctz(static_cast<unsigned>(pg.page_size));
  }

  hipError_t err;
  if (dtype == LTREE_BF16) {
    err = ltree::launch_partials_mfma(p, a, stream);
  } else {
    err = ltree::launch_partials_simple(dtype, p, a, stream);
  }
  return err == hipSuccess ? LTREE_OK : LTREE_ERR_HIP;
}

int ltree_attn_partials(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                        const void* q, const void* k_prefix, const void* v_prefix,
                        const int32_t* prefix_offsets, int max_prefix_len, const void* k_tree,
                        const void* v_tree, const uint64_t* mask, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return partials(dtype, B, T, Hq, Hkv, D, scale, q, k_prefix, v_prefix, prefix_offsets,
                  max_prefix_len, true, k_tree, v_tree, mask, workspace, workspace_bytes, stream);
}

// Merge of the partials in the workspace into o and lse.
static int merge(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D,
                 const int32_t* prefix_offsets, int max_prefix_len, float* o, float* lse,
                 const void* workspace, size_t workspace_bytes, hipStream_t stream,
                 int window = 0, const Paging& pg = Paging(), const Strides& rs = Strides()) {
  if (dtype != LTREE_F32 && dtype != LTREE_BF16) return LTREE_ERR_INVALID_ARG;
  const int st = check_sizes(B, T, Hq, Hkv, D, max_prefix_len);
  if (st != LTREE_OK) return st;
  if ((pg.seq_lens == nullptr && prefix_offsets == nullptr) || o == nullptr || lse == nullptr ||
      workspace == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  Plan p;
  if (!plan_here(B, T, Hq, Hkv, D, max_prefix_len, &p, window, pg.page_size,
                 rs.k > rs.v ? rs.k : rs.v)) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (pg.block_table != nullptr) p.seq_cap = pg.seq_cap;
  if (workspace_bytes < p.bytes || !aligned(workspace, 256)) return LTREE_ERR_WORKSPACE;
  const char* ws = static_cast<const char*>(workspace);
  const hipError_t err = ltree::launch_merge(
      p, dtype == LTREE_BF16, prefix_offsets, pg.seq_lens, ws + p.o_part_off,
      reinterpret_cast<const float*>(ws + p.scale_part_off),
      reinterpret_cast<const float*>(ws + p.lse_part_off), o, lse, stream);
  return err == hipSuccess ? LTREE_OK : LTREE_ERR_HIP;
}

int ltree_attn_merge(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D,
                     const int32_t* prefix_offsets, int max_prefix_len, float* o, float* lse,
                     const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return merge(dtype, B, T, Hq, Hkv, D, prefix_offsets, max_prefix_len, o, lse, workspace,
               workspace_bytes, stream);
}

int ltree_attn(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
               const void* q, const void* k_prefix, const void* v_prefix,
               const int32_t* prefix_offsets, int max_prefix_len, const void* k_tree,
               const void* v_tree, const uint64_t* mask, float* o, float* lse, void* workspace,
               size_t workspace_bytes, hipStream_t stream) {
  if (o == nullptr || lse == nullptr) return LTREE_ERR_INVALID_ARG;
  int st = ltree_attn_partials(dtype, B, T, Hq, Hkv, D, scale, q, k_prefix, v_prefix,
                               prefix_offsets, max_prefix_len, k_tree, v_tree, mask, workspace,
                               workspace_bytes, stream);
  if (st != LTREE_OK) return st;
  return ltree_attn_merge(dtype, B, T, Hq, Hkv, D, prefix_offsets, max_prefix_len, o, lse,
                          workspace, workspace_bytes, stream);
}

int ltree_attn_noalloc(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                       const void* q, const void* k_prefix, const void* v_prefix,
                       const int32_t* prefix_offsets, int max_prefix_len, const void* k_tree,
                       const void* v_tree, const uint64_t* mask, float* o, float* lse,
                       hipStream_t stream) {
  const int st = check_sizes(B, T, Hq, Hkv, D, max_prefix_len);
  if (st != LTREE_OK) return st;
  Plan p;
  if (!plan_here(B, T, Hq, Hkv, D, max_prefix_len, &p)) return LTREE_ERR_INVALID_ARG;
  if (p.bytes > LTREE_NOALLOC_SCRATCH_BYTES) return LTREE_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LTREE_ERR_HIP;
  if (dev >= ltree::kMaxDevices) return LTREE_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return LTREE_ERR_HIP;
    if (sdev != dev) return LTREE_ERR_INVALID_ARG;
  }
  void* ws = ltree::scratch_on(dev);
  if (ws == nullptr) return LTREE_ERR_HIP;
  return ltree_attn(dtype, B, T, Hq, Hkv, D, scale, q, k_prefix, v_prefix, prefix_offsets,
                    max_prefix_len, k_tree, v_tree, mask, o, lse, ws, LTREE_NOALLOC_SCRATCH_BYTES,
                    stream);
}

int ltree_prefix_attn(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                      const void* q, const void* k_prefix, const void* v_prefix,
                      const int32_t* prefix_offsets, int max_prefix_len, float* o, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (o == nullptr || lse == nullptr) return LTREE_ERR_INVALID_ARG;
  int st = partials(dtype, B, T, Hq, Hkv, D, scale, q, k_prefix, v_prefix, prefix_offsets,
                    max_prefix_len, false, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                    stream);
  if (st != LTREE_OK) return st;
  return ltree_attn_merge(dtype, B, T, Hq, Hkv, D, prefix_offsets, max_prefix_len, o, lse,
                          workspace, workspace_bytes, stream);
}

size_t ltree_attn_strided_workspace_bytes(int B, int T, int Hq, int Hkv, int D,
                                          int max_prefix_len, int64_t k_row_stride,
                                          int64_t v_row_stride) {
  Plan p;
  if (ltree::check_strides(Hkv, D, k_row_stride, v_row_stride) != LTREE_OK) return 0;
  const long s = k_row_stride > v_row_stride ? k_row_stride : v_row_stride;
  return plan_here(B, T, Hq, Hkv, D, max_prefix_len, &p, 0, 0, s) ? p.bytes : 0;
}

int ltree_attn_strided(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                       const void* q, const void* k_prefix, const void* v_prefix,
                       int64_t k_row_stride, int64_t v_row_stride, const int32_t* prefix_offsets,
                       int max_prefix_len, const void* k_tree, const void* v_tree,
                       const uint64_t* mask, float* o, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (o == nullptr || lse == nullptr) return LTREE_ERR_INVALID_ARG;
  const int cs = ltree::check_strides(Hkv, D, k_row_stride, v_row_stride);
  if (cs != LTREE_OK) return cs;
  Strides rs;
  rs.k = k_row_stride;
  rs.v = v_row_stride;
  const bool has_tree = k_tree != nullptr || v_tree != nullptr || mask != nullptr;
  int st = partials(dtype, B, T, Hq, Hkv, D, scale, q, k_prefix, v_prefix, prefix_offsets,
                    max_prefix_len, has_tree, k_tree, v_tree, mask, workspace, workspace_bytes,
                    stream, 0, Paging(), rs);
  if (st != LTREE_OK) return st;
  return merge(dtype, B, T, Hq, Hkv, D, prefix_offsets, max_prefix_len, o, lse, workspace,
               workspace_bytes, stream, 0, Paging(), rs);
}

size_t ltree_window_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window) {
  Plan p;
  if (window < 1) return 0;
  return plan_here(B, T, Hq, Hkv, D, window - 1, &p, window) ? p.bytes : 0;
}

int ltree_window_attn(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                      int window, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cache_offsets, const void* k_tree, const void* v_tree,
                      const uint64_t* mask, float* o, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (o == nullptr || lse == nullptr || k_cache == nullptr || v_cache == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (window < 1 || window < T) return LTREE_ERR_INVALID_ARG;
  if (window > LTREE_MAX_WINDOW) return LTREE_ERR_UNSUPPORTED;
  int st = partials(dtype, B, T, Hq, Hkv, D, scale, q, k_cache, v_cache, cache_offsets,
                    window - 1, true, k_tree, v_tree, mask, workspace, workspace_bytes, stream,
                    window);
  if (st != LTREE_OK) return st;
  return merge(dtype, B, T, Hq, Hkv, D, cache_offsets, window - 1, o, lse, workspace,
               workspace_bytes, stream, window);
}

size_t ltree_attn_paged_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_prefix_len,
                                        int page_size) {
  Plan p;
  if (page_size < 1) return 0;
  return plan_here(B, T, Hq, Hkv, D, max_prefix_len, &p, 0, page_size) ? p.bytes : 0;
}

int ltree_attn_paged(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                     const void* q, const void* k_pages, const void* v_pages, int num_pages,
                     int page_size, const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int max_prefix_len, const void* k_tree,
                     const void* v_tree, const uint64_t* mask, float* o, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (o == nullptr || lse == nullptr || k_pages == nullptr || v_pages == nullptr ||
      block_table == nullptr || seq_lens == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  Paging pg;
  const int cp = ltree::check_paged(dtype == LTREE_BF16 ? 2 : 4, Hkv, D, num_pages, page_size,
                                    max_pages_per_seq, max_prefix_len, 0, &pg.pool_bytes,
                                    &pg.seq_cap);
  if (cp != LTREE_OK) return cp;
  const bool has_tree = k_tree != nullptr || v_tree != nullptr || mask != nullptr;
  pg.seq_lens = seq_lens;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.max_pages = max_pages_per_seq;
  pg.num_pages = num_pages;
  int st = partials(dtype, B, T, Hq, Hkv, D, scale, q, k_pages, v_pages, nullptr, max_prefix_len,
                    has_tree, k_tree, v_tree, mask, workspace, workspace_bytes, stream, 0, pg);
  if (st != LTREE_OK) return st;
  return merge(dtype, B, T, Hq, Hkv, D, nullptr, max_prefix_len, o, lse, workspace,
               workspace_bytes, stream, 0, pg);
}

size_t ltree_window_attn_paged_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window,
                                               int page_size) {
  Plan p;
  if (window < 1 || page_size < 1) return 0;
  return plan_here(B, T, Hq, Hkv, D, window - 1, &p, window, page_size) ? p.bytes : 0;
}

int ltree_window_attn_paged(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                            int window, const void* q, const void* k_pages, const void* v_pages,
                            int num_pages, int page_size, const int32_t* block_table,
                            int max_pages_per_seq, const int32_t* seq_lens, const void* k_tree,
                            const void* v_tree, const uint64_t* mask, float* o, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (o == nullptr || lse == nullptr || k_pages == nullptr || v_pages == nullptr ||
      block_table == nullptr || seq_lens == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (window < 1 || window < T) return LTREE_ERR_INVALID_ARG;
  if (window > LTREE_MAX_WINDOW) return LTREE_ERR_UNSUPPORTED;
  // a window starts at any key, so rows are addressed lane by lane from the
  // start of the pool (32-bit byte offsets); a sequence longer than the block
  // table reaches gives NaN rows, like an over-long sequence of ltree_attn_paged
  Paging pg;
  const int cp = ltree::check_paged(dtype == LTREE_BF16 ? 2 : 4, Hkv, D, num_pages, page_size,
                                    max_pages_per_seq, 0, window, &pg.pool_bytes, &pg.seq_cap);
  if (cp != LTREE_OK) return cp;
  pg.seq_lens = seq_lens;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.max_pages = max_pages_per_seq;
  pg.num_pages = num_pages;
  int st = partials(dtype, B, T, Hq, Hkv, D, scale, q, k_pages, v_pages, nullptr, window - 1,
                    true, k_tree, v_tree, mask, workspace, workspace_bytes, stream, window, pg);
  if (st != LTREE_OK) return st;
  return merge(dtype, B, T, Hq, Hkv, D, nullptr, window - 1, o, lse, workspace, workspace_bytes,
               stream, window, pg);
}

int ltree_commit_kv(ltree_dtype dtype, int B, int T, int Hkv, int D, const void* k_tree,
                    const void* v_tree, const int32_t* accepted, const int32_t* n_accepted,
                    const int32_t* dst_row, void* k_cache, void* v_cache, int cache_rows,
                    int32_t* status, hipStream_t stream) {
  if (dtype != LTREE_F32 && dtype != LTREE_BF16) return LTREE_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || Hkv < 1 || cache_rows < 0) return LTREE_ERR_INVALID_ARG;
  if (T > LTREE_MAX_TREE || (D != 64 && D != 128)) return LTREE_ERR_UNSUPPORTED;
  if (k_tree == nullptr || v_tree == nullptr || accepted == nullptr || n_accepted == nullptr ||
      dst_row == nullptr || k_cache == nullptr || v_cache == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (!aligned(k_tree, 16) || !aligned(v_tree, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16)) {
    return LTREE_ERR_INVALID_ARG;
  }
  const long row_bytes = static_cast<long>(Hkv) * D * (dtype == LTREE_BF16 ? 2 : 4);
  // byte offsets of tree rows and cache rows stay below 2^63; the row itself
  // is addressed with an int
  if (row_bytes > (1L << 30) || static_cast<long>(B) * T > (1L << 30)) return LTREE_ERR_UNSUPPORTED;
  return ltree::launch_kv_commit(k_tree, v_tree, accepted, n_accepted, dst_row, k_cache,
                                 v_cache, B, T, static_cast<int>(row_bytes), cache_rows, status,
                                 stream) == hipSuccess
             ? LTREE_OK
             : LTREE_ERR_HIP;
}

int ltree_tree_rope(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, void* q,
                    void* k_tree, const uint64_t* mask, const int32_t* prefix_offsets,
                    double rope_base, hipStream_t stream) {
  if (dtype != LTREE_F32 && dtype != LTREE_BF16) return LTREE_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1) return LTREE_ERR_INVALID_ARG;
  if (T > LTREE_MAX_TREE || (D != 64 && D != 128)) return LTREE_ERR_UNSUPPORTED;
  if (!(std::isfinite(rope_base) && rope_base > 1.0)) return LTREE_ERR_INVALID_ARG;
  if (q == nullptr || k_tree == nullptr || mask == nullptr || prefix_offsets == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (static_cast<long>(B) * T * (Hq + Hkv) * D > (1L << 40)) return LTREE_ERR_UNSUPPORTED;
  return ltree::launch_tree_rope(dtype == LTREE_BF16, q, k_tree, mask, prefix_offsets, B, T, Hq,
                                 Hkv, D, rope_base, stream) == hipSuccess
             ? LTREE_OK
             : LTREE_ERR_HIP;
}

}  // extern "C"
