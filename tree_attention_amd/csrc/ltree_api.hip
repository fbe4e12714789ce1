// C ABI of libltree: argument checks, work planning, kernel launches.
// The operations are defined in include/ltree.h.
#include <atomic>
#include <cmath>
#include <cstdlib>

#include "ltree_internal.h"

namespace ltree {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev >= kMaxDevices) dev = kMaxDevices - 1;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    n = 256;
  }
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool make_plan(int B, int T, int Hq, int Hkv, int D, int max_prefix_len, Plan* p, int window,
               int page_size) {
  if (page_size < 0) return false;
  if (window < 0 || window > LTREE_MAX_WINDOW || (window > 0 && window < T)) return false;
  if (window > 0) max_prefix_len = window - 1;
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_prefix_len < 0) return false;
  if (D != 64 && D != 128) return false;
  if (T > LTREE_MAX_TREE) return false;
  // output rows (b, h, i) are indexed with 32-bit integers in the merge
  if (static_cast<long>(B) * Hq * T >= (1L << 31)) return false;
  p->B = B;
  p->T = T;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->D = D;
  p->G = Hq / Hkv;
  p->R = p->G * T;
  p->max_prefix_len = max_prefix_len;
  p->window = window;

  // Split size: enough prefix splits per KV head that the Hkv heads of one
  // sequence cover every compute unit once; never below 256 keys, so that a
  // split's partial output stays small next to the keys it reads (a window of
  // a few hundred keys, whose call is latency-bound, splits down to 64).
  const int cus = device_cu_count();
  const int per_head = (cus + Hkv - 1) / Hkv;
  long chunk = (static_cast<long>(max_prefix_len) + per_head - 1) / per_head;
  chunk = (chunk + 63) / 64 * 64;
  const long min_chunk = window > 0 ? 64 : 256;
  if (chunk < min_chunk) chunk = min_chunk;
  if (const char* env = std::getenv("LTREE_SPLIT_KEYS")) {  // tuning sweeps only
    const long v = std::atol(env);
    if (v >= 64 && v % 64 == 0) chunk = v;
  }
  // keys of one split are addressed with 32-bit element offsets
  const long cap = ((1L << 31) - 1) / (static_cast<long>(Hkv) * D) / 64 * 64;
  if (chunk > cap) chunk = cap;
  // a paged split's page numbers fit the kernels' LDS table (a split that
  // starts inside a page touches one page more than it fills)
  if (page_size > 0 && chunk > static_cast<long>(kMaxSplitPages - 1) * page_size) {
    chunk = static_cast<long>(kMaxSplitPages - 1) * page_size / 64 * 64;
  }
  if (chunk < 64) return false;
  p->chunk = static_cast<int>(chunk);
  p->max_chunks = static_cast<int>((max_prefix_len + chunk - 1) / chunk);
  // the last split of a sequence also takes the tree keys; an empty prefix
  // still needs one partial for them
  p->slots = p->max_chunks > 0 ? p->max_chunks : 1;

  const size_t rows = static_cast<size_t>(B) * Hkv * p->slots * p->R;
  p->o_part_off = 0;
  p->scale_part_off = align_up(rows * D * sizeof(float), 256);
  p->lse_part_off = align_up(p->scale_part_off + rows * sizeof(float), 256);
  p->bytes = align_up(p->lse_part_off + rows * sizeof(float), 256);
  return true;
}

}  // namespace ltree

using ltree::Plan;
using ltree::aligned;

extern "C" {

int ltree_version(void) { return LTREE_VERSION; }

const char* ltree_status_string(int status) {
  switch (status) {
    case LTREE_OK: return "ok";
    case LTREE_ERR_INVALID_ARG: return "invalid argument";
    case LTREE_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case LTREE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case LTREE_ERR_HIP: return "HIP runtime error";
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
  return ltree::make_plan(B, T, Hq, Hkv, D, max_prefix_len, &p) ? p.bytes : 0;
}

static int check_sizes(int B, int T, int Hq, int Hkv, int D, int max_prefix_len) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || max_prefix_len < 0) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (T > LTREE_MAX_TREE || (D != 64 && D != 128)) return LTREE_ERR_UNSUPPORTED;
  // every flat index the kernels form from the query/output sizes fits in int
  if (static_cast<long>(B) * T * Hq * D > (1L << 31) - 1) return LTREE_ERR_UNSUPPORTED;
  return LTREE_OK;
}

// A paged prefix: pools of pages and the table that maps each sequence's
// keys to them (see ltree_attn_paged).
struct Paging {
  const int32_t* seq_lens = nullptr;
  const int32_t* block_table = nullptr;
  int page_size = 0, max_pages = 0, num_pages = 0;
  uint32_t pool_bytes = 0;
};

// Partials of prefix (+ tree, when has_tree) attention into the workspace;
// window > 0: sliding-window attention (max_prefix_len is then window - 1);
// pg.block_table != nullptr: a paged prefix (k_prefix/v_prefix are the pools).
static int partials(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                    const void* q, const void* k_prefix, const void* v_prefix,
                    const int32_t* prefix_offsets, int max_prefix_len, bool has_tree,
                    const void* k_tree, const void* v_tree, const uint64_t* mask,
                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                    int window = 0, const Paging& pg = Paging()) {
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
  Plan p;
  if (!ltree::make_plan(B, T, Hq, Hkv, D, max_prefix_len, &p, window, pg.page_size)) {
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
                 int window = 0, const Paging& pg = Paging()) {
  if (dtype != LTREE_F32 && dtype != LTREE_BF16) return LTREE_ERR_INVALID_ARG;
  const int st = check_sizes(B, T, Hq, Hkv, D, max_prefix_len);
  if (st != LTREE_OK) return st;
  if ((pg.seq_lens == nullptr && prefix_offsets == nullptr) || o == nullptr || lse == nullptr ||
      workspace == nullptr) {
    return LTREE_ERR_INVALID_ARG;
  }
  Plan p;
  if (!ltree::make_plan(B, T, Hq, Hkv, D, max_prefix_len, &p, window, pg.page_size)) {
    return LTREE_ERR_INVALID_ARG;
  }
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

size_t ltree_window_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window) {
  Plan p;
  if (window < 1) return 0;
  return ltree::make_plan(B, T, Hq, Hkv, D, window - 1, &p, window) ? p.bytes : 0;
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
  return ltree::make_plan(B, T, Hq, Hkv, D, max_prefix_len, &p, 0, page_size) ? p.bytes : 0;
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
  if (page_size < 1 || num_pages < 1 || max_pages_per_seq < 1 ||
      max_prefix_len < 0 ||
      static_cast<long>(max_prefix_len) > static_cast<long>(max_pages_per_seq) * page_size) {
    return LTREE_ERR_INVALID_ARG;
  }
  // page rows are addressed with 64-bit offsets; a page's rows with 32-bit ones
  if (static_cast<long>(page_size) * Hkv * D > (1L << 30)) return LTREE_ERR_UNSUPPORTED;
  // a page size that is not a multiple of 64 addresses every row from the
  // start of the pool with a 32-bit byte offset
  const long pool_bytes = static_cast<long>(num_pages) * page_size * Hkv * D *
                          (dtype == LTREE_BF16 ? 2 : 4);
  if (page_size % 64 != 0 && pool_bytes >= (1L << 31)) return LTREE_ERR_UNSUPPORTED;
  const bool has_tree = k_tree != nullptr || v_tree != nullptr || mask != nullptr;
  Paging pg;
  pg.seq_lens = seq_lens;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.max_pages = max_pages_per_seq;
  pg.num_pages = num_pages;
  pg.pool_bytes = static_cast<uint32_t>(pool_bytes < (1L << 31) ? pool_bytes : 0);
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
  return ltree::make_plan(B, T, Hq, Hkv, D, window - 1, &p, window, page_size) ? p.bytes : 0;
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
  if (window < 1 || window < T || page_size < 1 || num_pages < 1 || max_pages_per_seq < 1) {
    return LTREE_ERR_INVALID_ARG;
  }
  if (window > LTREE_MAX_WINDOW) return LTREE_ERR_UNSUPPORTED;
  if (static_cast<long>(page_size) * Hkv * D > (1L << 30)) return LTREE_ERR_UNSUPPORTED;
  // a window starts at any key, so rows are addressed lane by lane from the
  // start of the pool (32-bit byte offsets)
  const long pool_bytes = static_cast<long>(num_pages) * page_size * Hkv * D *
                          (dtype == LTREE_BF16 ? 2 : 4);
  if (pool_bytes >= (1L << 31)) return LTREE_ERR_UNSUPPORTED;
  Paging pg;
  pg.seq_lens = seq_lens;
  pg.block_table = block_table;
  pg.page_size = page_size;
  pg.max_pages = max_pages_per_seq;
  pg.num_pages = num_pages;
  pg.pool_bytes = static_cast<uint32_t>(pool_bytes);
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
