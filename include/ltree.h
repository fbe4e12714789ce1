/*
 * ltree.h -- hybrid tree-verification attention on AMD Instinct MI355X (gfx950).
 *
 * A speculative-decoding verifier scores a tree of T draft tokens against a long
 * cached prefix.  Following the split described on the gist.science page
 * "LongSpec: Long-Context Lossless Speculative Decoding with Efficient Drafting
 * and Verification" (section 2 "Methodik", part C "Schnelle Tree Attention"),
 * the attention of every tree token is computed in two parts:
 *
 *   - the cached part: the long prefix KV cache, attended with no mask;
 *   - the speculative part: the T draft tokens, attended under a tree mask;
 *
 * and the two partial softmax results are joined exactly by a log-sum-exp
 * merge (same section, "Aggregation").  The arXiv abstract of the paper
 * (mlsanity.com page, section "Abstract (arXiv)") describes the same thing as
 * fast prefix computation combined with standard tree attention.
 *
 * The result equals one softmax over [prefix | tree] in which tree node i sees
 * every prefix key and the tree nodes in anc*(i) = {i} U ancestors(i):
 *
 *     lse[b,h,i] = ln sum_{j visible} exp(scale * <q[b,i,h], k_j>)
 *     o[b,i,h]   = sum_{j visible} exp(scale * <q[b,i,h], k_j> - lse[b,h,i]) v_j
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns all
 *     buffers; the library never allocates or frees device memory.
 *   - Every tensor is dense row-major with the last dimension contiguous.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  The return
 *     value only reports checks of host-visible arguments and launch errors;
 *     device-side findings go to the documented device outputs.
 *   - Query head h reads KV head h / G, with G = Hq / Hkv (contiguous groups).
 *   - Thread safety: calls may be issued from several host threads; calls that
 *     share a workspace must be ordered by the caller (same stream, or events).
 */
#ifndef LTREE_H
#define LTREE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LTREE_VERSION 130 /* 1.3.0: ltree_attn_noalloc */
#define LTREE_MAX_TREE 256 /* largest tree; a mask row has W = ceil(T / 64) 64-bit words */
#define LTREE_MAX_WINDOW (1 << 20) /* largest sliding window of ltree_window_attn */

typedef enum {
  LTREE_OK = 0,
  LTREE_ERR_INVALID_ARG = -1, /* null pointer, bad size, Hq % Hkv != 0, scale <= 0, ... */
  LTREE_ERR_UNSUPPORTED = -2, /* valid but not built: D not 64/128, T > 256, ...       */
  LTREE_ERR_WORKSPACE = -3,   /* workspace too small or misaligned                     */
  LTREE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed            */
  LTREE_ERR_SCRATCH = -5      /* ltree_attn_noalloc: the call needs more scratch memory
                                 than LTREE_NOALLOC_SCRATCH_BYTES                       */
} ltree_status;

typedef enum {
  LTREE_F32 = 0, /* fp32 q/k/v: exact-arithmetic path (fp32 FMA), for checking */
  LTREE_BF16 = 1 /* bf16 q/k/v: the MFMA path                                   */
} ltree_dtype;

/* Library version, LTREE_VERSION of the build. */
int ltree_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* ltree_status_string(int status);

/* Words of one mask row for a tree of T nodes: W = ceil(T / 64). */
#define LTREE_MASK_WORDS(T) (((T) + 63) / 64)

/*
 * ltree_build_mask -- ancestor-or-self bitmask of B speculation trees.
 *
 * Defines the tree mask of the speculative part (gist.science page, section 2
 * part C, item 2 of the split; section 1 "Problemstellung", item "Ineffiziente
 * Verifikation", on tree-attention masks).  A draft token sees its own branch:
 * itself and its ancestors, no siblings or cousins.
 *
 *   parent  [B, T] int32.  parent[b*T+i] = -1 hangs node i directly under the
 *           prefix; otherwise it is an earlier node, 0 <= parent < i.  Several
 *           -1 entries (a forest) are allowed.
 *   B, T    1 <= B, 1 <= T <= LTREE_MAX_TREE.
 *   mask    [B, T, W] uint64 out, W = LTREE_MASK_WORDS(T) (1 for T <= 64).
 *           Bit j % 64 of word j / 64 of row (b, i) is set iff j == i or j is
 *           an ancestor of i.  Bits j >= T are zero.
 *   status  [1] int32 out, or NULL.  0 when every parent entry is valid; else
 *           1 + the smallest flat index b*T+i whose entry is invalid.  All mask
 *           rows of a tree with an invalid entry are written as zero.
 *
 * Returns LTREE_OK, LTREE_ERR_INVALID_ARG (null pointer, B < 1, T < 1),
 * LTREE_ERR_UNSUPPORTED (T > 256) or LTREE_ERR_HIP.  No workspace; one launch,
 * or (more than 16 trees, or T > 64) one launch spread over workgroups and,
 * when status is requested, a one-wave launch that forms it.
 */
int ltree_build_mask(const int32_t* parent, int B, int T, uint64_t* mask,
                     int32_t* status, hipStream_t stream);

/*
 * ltree_attn_workspace_bytes -- size of the scratch buffer `ltree_attn`,
 * `ltree_attn_partials` and `ltree_attn_merge` need for these sizes on the
 * current device.  The workspace holds the partial results of the prefix
 * splits (the last split of a sequence also covers its tree tokens): fp32 for
 * fp32 inputs; for bf16 inputs 16-bit normalised values with one fp32 scale
 * per row.  Returns 0 if the sizes are invalid.
 */
size_t ltree_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D,
                                  int max_prefix_len);

/*
 * ltree_attn -- hybrid tree-verification attention, all three steps.
 *
 * Step 1 (cached part, gist.science section 2 part C item 1): every tree
 * query attends the whole prefix of its sequence with no mask.  The prefix is
 * cut into splits that run in parallel; each split yields a normalised partial
 * output and its log-sum-exp.  Step 2 (speculative part, item 2): every tree
 * query attends the T tree tokens under `mask`.  Step 3 ("Aggregation"): all
 * partials are joined by a log-sum-exp merge into `o` and `lse`.
 *
 *   dtype          LTREE_BF16 or LTREE_F32 for q, k_prefix, v_prefix, k_tree, v_tree.
 *   B, T, Hq, Hkv, D
 *                  batch, tree size (1..256), query heads, KV heads (Hq % Hkv == 0),
 *                  head dim (64 or 128).
 *   scale          score scale (usually 1/sqrt(D)); finite and > 0.
 *   q              [B, T, Hq, D] queries of the tree tokens (after RoPE).
 *   k_prefix, v_prefix
 *                  [sum_b L_b, Hkv, D] packed prefix cache; sequence b owns rows
 *                  prefix_offsets[b] .. prefix_offsets[b+1]-1.
 *   prefix_offsets [B+1] int32, offsets[0] = 0, non-decreasing; L_b may be 0.
 *   max_prefix_len host int >= every L_b; it sizes the grid and the workspace.
 *                  A sequence whose L_b exceeds it, or whose offsets decrease,
 *                  gets NaN in all its o and lse entries.
 *   k_tree, v_tree [B, T, Hkv, D] keys/values of the tree tokens.
 *   mask           [B, T, W] uint64 from ltree_build_mask (bit j of row i: node
 *                  j visible to node i).  Row i must have bit i set; a row with
 *                  no visible tree node and L_b = 0 has no defined result.
 *   o              [B, T, Hq, D] fp32 out.
 *   lse            [B, Hq, T] fp32 out, natural logarithm.
 *   workspace      >= ltree_attn_workspace_bytes(...) bytes, 256-byte aligned.
 *                  Its contents on entry do not matter.
 *
 * Numerics (bf16): q.k on bf16 MFMA with fp32 accumulation; softmax in fp32;
 * probabilities are rounded to fp16 and v converted from bf16 to fp16 (round
 * to nearest; exact for 2^-14 <= |v| < 65504, an absolute error of at most
 * 2^-25 for smaller |v|, where fp16 is subnormal) for the fp16 MFMA P.v
 * product with fp32 accumulation; the row sums add the same fp16-rounded
 * probabilities.  Each split's normalised output row is
 * stored as 16-bit values relative to the row's largest magnitude (error at
 * most 2^-16 of it) for the merge.  |v| must stay below the fp16 limit 65504;
 * larger values give non-finite o.  fp32 path: fp32 throughout.
 *
 * Returns LTREE_OK, LTREE_ERR_INVALID_ARG, LTREE_ERR_UNSUPPORTED,
 * LTREE_ERR_WORKSPACE or LTREE_ERR_HIP.  Two kernel launches on `stream`.
 */
int ltree_attn(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
               const void* q, const void* k_prefix, const void* v_prefix,
               const int32_t* prefix_offsets, int max_prefix_len,
               const void* k_tree, const void* v_tree, const uint64_t* mask,
               float* o, float* lse, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * ltree_attn_noalloc -- ltree_attn for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same kernels and the same results as ltree_attn
 * with the same arguments; the partials live in a static device array of
 * LTREE_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs
 * on, from the first call on that device until the process ends, instead of
 * a workspace argument.  The call allocates nothing.
 *
 *   arguments      as for ltree_attn, without the workspace.
 *   stream         must belong to the current device (the one whose copy of
 *                  the array is used); LTREE_ERR_INVALID_ARG otherwise.
 *
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (on different streams, or from different threads with
 * their kernels still running) race and give wrong results.  Calls ordered on
 * one stream are safe.  Nothing in the array has to start at zero: the merge
 * uses only values the partial kernel wrote in the same call.
 *
 * Returns as ltree_attn, and LTREE_ERR_SCRATCH when
 * ltree_attn_workspace_bytes(B, T, Hq, Hkv, D, max_prefix_len) exceeds
 * LTREE_NOALLOC_SCRATCH_BYTES (nothing is launched then).  Two kernel
 * launches on `stream`.
 */
#define LTREE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20) /* 96 MiB per device */
int ltree_attn_noalloc(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                       const void* q, const void* k_prefix, const void* v_prefix,
                       const int32_t* prefix_offsets, int max_prefix_len,
                       const void* k_tree, const void* v_tree, const uint64_t* mask,
                       float* o, float* lse, hipStream_t stream);

/*
 * ltree_attn_strided_workspace_bytes -- workspace size of ltree_attn_strided
 * for these sizes and row strides on the current device (0 if invalid).
 */
size_t ltree_attn_strided_workspace_bytes(int B, int T, int Hq, int Hkv, int D,
                                          int max_prefix_len, int64_t k_row_stride,
                                          int64_t v_row_stride);

/*
 * ltree_attn_strided -- ltree_attn over a prefix cache whose key rows are not
 * packed: key j of sequence b, KV head g, feature d is
 *
 *     k_prefix[(prefix_offsets[b] + j) * k_row_stride + g * D + d]
 *
 * (likewise v_prefix with v_row_stride).  An interleaved cache [rows, 2, Hkv, D]
 * is k_prefix = base, v_prefix = base + Hkv * D, both strides 2 * Hkv * D; a
 * cache with padded rows has a stride above Hkv * D.  The computation is that
 * of ltree_attn on the packed rows (gist.science section 2 part C); no copy
 * is made.
 *
 *   k_row_stride, v_row_stride
 *                  host, in elements: >= Hkv * D, a multiple of 8 (16-byte rows),
 *                  at most 2^24.  LTREE_ERR_INVALID_ARG otherwise
 *                  (LTREE_ERR_UNSUPPORTED above 2^24).
 *   k_tree, v_tree, mask
 *                  as for ltree_attn, packed [B, T, Hkv, D]; all three NULL
 *                  computes the prefix part alone (as ltree_prefix_attn: an
 *                  empty prefix gives o = 0 and lse = -inf).
 *   workspace      >= ltree_attn_strided_workspace_bytes(...), 256-byte aligned.
 *   other arguments as for ltree_attn.
 *
 * Returns as ltree_attn.  Two kernel launches.
 */
int ltree_attn_strided(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                       const void* q, const void* k_prefix, const void* v_prefix,
                       int64_t k_row_stride, int64_t v_row_stride,
                       const int32_t* prefix_offsets, int max_prefix_len,
                       const void* k_tree, const void* v_tree, const uint64_t* mask,
                       float* o, float* lse, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * ltree_attn_partials -- steps 1 and 2 of ltree_attn alone (same arguments
 * minus o and lse): writes the partial results of every prefix split and of
 * the tree part into `workspace`.  The layout is internal; the only consumer
 * is ltree_attn_merge called with the same sizes.  One kernel launch.
 */
int ltree_attn_partials(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D,
                        float scale, const void* q, const void* k_prefix,
                        const void* v_prefix, const int32_t* prefix_offsets,
                        int max_prefix_len, const void* k_tree, const void* v_tree,
                        const uint64_t* mask, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * ltree_attn_merge -- step 3 of ltree_attn alone: the log-sum-exp merge
 * (gist.science section 2 part C, "Aggregation") of the partials that
 * ltree_attn_partials left in `workspace` into o [B,T,Hq,D] and lse [B,Hq,T].
 * dtype and sizes must equal those of the ltree_attn_partials call (dtype
 * selects the partial format).  One kernel launch.
 */
int ltree_attn_merge(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D,
                     const int32_t* prefix_offsets, int max_prefix_len,
                     float* o, float* lse, const void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * ltree_prefix_attn -- attention of T query tokens over the prefix KV cache
 * alone, no mask and no tree part: the draft model's cross-attention into the
 * target model's shared KV cache (gist.science page, section 2 "Methodik",
 * part A, item "Cross-Attention mit geteiltem KV-Cache": the draft reads the
 * target's cache directly).  The same kernels as ltree_attn (split-K partials,
 * then the log-sum-exp merge) with the tree part left out.
 *
 *   dtype, B, T, Hq, Hkv, D, scale, q, k_prefix, v_prefix, prefix_offsets,
 *   max_prefix_len, o, lse, workspace, workspace_bytes, stream
 *                  as for ltree_attn; T (1..256) counts the query tokens.  The
 *                  workspace size is ltree_attn_workspace_bytes(B, T, Hq, Hkv,
 *                  D, max_prefix_len).
 *   A sequence with L_b = 0 has no key: its rows get o = 0 and lse = -inf.
 *
 * Returns as ltree_attn.  Two kernel launches.
 */
int ltree_prefix_attn(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                      const void* q, const void* k_prefix, const void* v_prefix,
                      const int32_t* prefix_offsets, int max_prefix_len, float* o, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ltree_attn_paged_workspace_bytes -- bytes of workspace ltree_attn_paged needs
 * for these sizes and page size (0 when they are invalid).
 */
size_t ltree_attn_paged_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int max_prefix_len,
                                        int page_size);

/*
 * ltree_attn_paged -- ltree_attn over a paged prefix cache: the same
 * computation (gist.science page, section 2 part C: prefix without mask, tree
 * under the mask, log-sum-exp merge), with the prefix keys and values kept in
 * fixed-size pages of a shared pool instead of one packed array.  With
 * k_tree, v_tree and mask all NULL it is the prefix-only attention of
 * ltree_prefix_attn over the paged cache (the draft's cross-attention into the
 * target's cache, section 2 part A).
 *
 *   k_pages, v_pages  [num_pages, page_size, Hkv, D] page pools (dtype as q).
 *   num_pages         >= 1, pages in each pool.
 *   page_size         keys per page, >= 1.  A multiple of 64 (every 64-key tile
 *                     within one page) takes any pool size; other page sizes
 *                     address rows lane by lane from the start of the pool and
 *                     need num_pages * page_size * Hkv * D * element bytes
 *                     below 2^31 (else LTREE_ERR_UNSUPPORTED).
 *   block_table       [B, max_pages_per_seq] int32: key j of sequence b is row
 *                     j % page_size of page block_table[b, j / page_size].
 *                     Entries past a sequence's last page are not read.  A page
 *                     number outside [0, num_pages) is never dereferenced: the
 *                     rows of that sequence become NaN.
 *   seq_lens          [B] int32, L_b = prefix keys of sequence b, 0 <= L_b <=
 *                     max_prefix_len (a larger one makes its rows NaN).
 *   max_prefix_len    host int, <= max_pages_per_seq * page_size.
 *   workspace         ltree_attn_paged_workspace_bytes(B, T, Hq, Hkv, D,
 *                     max_prefix_len, page_size) bytes, 256-byte aligned.
 *   everything else   as for ltree_attn (T up to LTREE_MAX_TREE).
 *
 * Returns as ltree_attn.  Two kernel launches.
 */
int ltree_attn_paged(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                     const void* q, const void* k_pages, const void* v_pages, int num_pages,
                     int page_size, const int32_t* block_table, int max_pages_per_seq,
                     const int32_t* seq_lens, int max_prefix_len, const void* k_tree,
                     const void* v_tree, const uint64_t* mask, float* o, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ltree_window_attn_workspace_bytes -- bytes of workspace ltree_window_attn
 * needs for these sizes and window (0 when they are invalid).
 */
size_t ltree_window_attn_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window);

/*
 * ltree_window_attn -- the draft model's sliding-window self-attention over a
 * draft tree (gist.science page, section 2 "Methodik", part A, item
 * "Sliding-Window Self-Attention": the draft's self-attention sees a window of
 * recent tokens, e.g. 512, so its own cache stays bounded).
 *
 * Positions: key k of sequence b's draft cache (k = 0 .. L_b - 1; the last is
 * the token just before the tree) is at position k; tree node i is at
 * L_b + depth(i) - 1 (depth = nodes on its root path, root = 1), the position
 * ltree_tree_rope uses.  Node i sees exactly the keys on its own branch (all
 * cache keys, the tree nodes of anc*(i)) whose position p satisfies
 * pos(i) - window < p <= pos(i): the last window - depth(i) cache keys and
 * every ancestor.  Otherwise as ltree_attn (scores, lse, GQA, fp32 outputs).
 *
 *   dtype, B, T, Hq, Hkv, D, scale, q, k_tree, v_tree, mask, o, lse, stream
 *                  as for ltree_attn.
 *   window         T <= window <= LTREE_MAX_WINDOW.
 *   k_cache, v_cache  [sum L_b, Hkv, D] packed by cache_offsets [B+1] (as
 *                  k_prefix/v_prefix of ltree_attn), not NULL; L_b may exceed
 *                  the window: only the last min(L_b, window - 1) rows of each
 *                  sequence are read, so a caller may pass the whole history
 *                  or only a bounded ring of recent rows laid out in order.
 *   workspace      ltree_window_attn_workspace_bytes(B, T, Hq, Hkv, D, window)
 *                  bytes, 256-byte aligned, caller-owned.
 *
 * Returns as ltree_attn (LTREE_ERR_INVALID_ARG also for window < T).  A
 * decreasing cache_offsets table (L_b < 0) turns that sequence's rows into
 * NaN.  Two kernel launches.
 */
int ltree_window_attn(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                      int window, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cache_offsets, const void* k_tree, const void* v_tree,
                      const uint64_t* mask, float* o, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * ltree_window_attn_paged_workspace_bytes -- bytes of workspace
 * ltree_window_attn_paged needs (0 when the sizes are invalid).
 */
size_t ltree_window_attn_paged_workspace_bytes(int B, int T, int Hq, int Hkv, int D, int window,
                                               int page_size);

/*
 * ltree_window_attn_paged -- ltree_window_attn over a paged draft cache: the
 * window rule of ltree_window_attn, the cache addressed as in
 * ltree_attn_paged (k_pages, v_pages, num_pages, page_size, block_table,
 * max_pages_per_seq, seq_lens; only the last min(L_b, window - 1) keys of
 * each sequence are read, so only their pages need valid entries).  A
 * sequence with L_b above max_pages_per_seq * page_size (more keys than its
 * block-table row can address) gets NaN in all its o and lse entries, and
 * nothing of it is read, as for ltree_attn_paged.  A window
 * starts at any key, so rows are addressed lane by lane from the start of the
 * pool: num_pages * page_size * Hkv * D * element bytes must stay below 2^31
 * (else LTREE_ERR_UNSUPPORTED).  The workspace is
 * ltree_window_attn_paged_workspace_bytes(B, T, Hq, Hkv, D, window, page_size)
 * bytes.  Returns as ltree_window_attn.  Two kernel launches.
 */
int ltree_window_attn_paged(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, float scale,
                            int window, const void* q, const void* k_pages, const void* v_pages,
                            int num_pages, int page_size, const int32_t* block_table,
                            int max_pages_per_seq, const int32_t* seq_lens, const void* k_tree,
                            const void* v_tree, const uint64_t* mask, float* o, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ltree_commit_kv -- copy the keys and values of the accepted draft tokens from
 * the tree buffers into the KV cache, so they join the cached prefix of the
 * next verification step (gist.science page, opening explanation: the target
 * keeps the proposals it accepts; section 3 "Wichtige Ergebnisse": about 3.5
 * to 4 accepted tokens per pass).
 *
 *   dtype       element type of all four K/V arrays (LTREE_BF16 or LTREE_F32).
 *   B, T, Hkv, D  1 <= T <= LTREE_MAX_TREE, D in {64, 128}.
 *   k_tree, v_tree  [B, T, Hkv, D], as given to ltree_attn.
 *   accepted    [B, T] int32: tree node ids of the accepted tokens of sequence
 *               b in cache order (root side first); entries from n_accepted[b]
 *               on are ignored.
 *   n_accepted  [B] int32, 0 <= n <= T.
 *   dst_row     [B] int32: cache row that takes accepted token 0 of sequence b;
 *               tokens 1.. follow in consecutive rows.
 *   k_cache, v_cache  [cache_rows, Hkv, D] in/out: rows dst_row[b] ..
 *               dst_row[b] + n_accepted[b] - 1 are overwritten, nothing else.
 *               Ranges of different sequences must not overlap.
 *   status      [1] int32 out or NULL: 0, or 1 + the first sequence whose
 *               n_accepted, dst_row or accepted ids are out of range; such a
 *               sequence is not written.
 *
 * Returns LTREE_OK, LTREE_ERR_INVALID_ARG (null or misaligned pointer, bad
 * sizes), LTREE_ERR_UNSUPPORTED or LTREE_ERR_HIP.  One kernel launch; all
 * pointers 16-byte aligned.
 */
int ltree_commit_kv(ltree_dtype dtype, int B, int T, int Hkv, int D, const void* k_tree,
                    const void* v_tree, const int32_t* accepted, const int32_t* n_accepted,
                    const int32_t* dst_row, void* k_cache, void* v_cache, int cache_rows,
                    int32_t* status, hipStream_t stream);

/*
 * ltree_tree_rope -- rotary position embedding of the tree tokens, in place, at
 * their tree positions (gist.science page, section 1 "Problemstellung", item
 * "Trainings-Inferenz-Diskrepanz": positions enter through RoPE and must agree
 * with the target model's; the mlsanity.com page lists RoFormer among the
 * paper's references).  Node i of sequence b takes position
 * p = L_b + depth(i) - 1, depth = popcount of the mask row (root = 1), so a token
 * continues the prefix along its own branch and siblings share a position.
 * For every head and k < D/2, with a = p * rope_base^(-2k/D):
 *   x[k]       <- x[k] cos a - x[k + D/2] sin a
 *   x[k + D/2] <- x[k + D/2] cos a + x[k] sin a
 * evaluated in fp64 and rounded to nearest even into the storage type.
 *
 *   dtype          LTREE_BF16 or LTREE_F32, the type of q and k_tree.
 *   q              [B, T, Hq, D] in/out.   k_tree  [B, T, Hkv, D] in/out.
 *   mask           [B, T, W] uint64 from ltree_build_mask.  A zero row (a tree
 *                  with an invalid parent) leaves that token unrotated.
 *   prefix_offsets [B+1] int32 as for ltree_attn (L_b = o[b+1] - o[b]).
 *   rope_base      > 1, the rotary base of the target model.
 *
 * Returns LTREE_OK, LTREE_ERR_INVALID_ARG, LTREE_ERR_UNSUPPORTED (T > 256,
 * D not 64/128) or LTREE_ERR_HIP.  One kernel launch; run it before ltree_attn.
 */
int ltree_tree_rope(ltree_dtype dtype, int B, int T, int Hq, int Hkv, int D, void* q,
                    void* k_tree, const uint64_t* mask, const int32_t* prefix_offsets,
                    double rope_base, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LTREE_H */
