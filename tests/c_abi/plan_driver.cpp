// Host-only driver of libltree's work planning and argument checks
// (tree_attention_amd/csrc/ltree_plan.cpp), built by tests/test_host_plan.py
// with g++ under the address and undefined-behaviour sanitizers.  It runs the
// planner over extreme and random sizes and checks, in 128-bit arithmetic,
// the invariants the kernels rely on: every split is a whole number of 64-key
// tiles, the splits cover the prefix, a split's keys are addressed with
// 32-bit offsets, a paged split's pages fit the LDS table, and the workspace
// holds every partial row.  Prints "plans checked: N" and exits 0, or prints
// the first failure and exits 1.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>

#include "ltree.h"
#include "ltree_plan.h"

using ltree::Plan;
typedef __int128 i128;

static long g_checked = 0;

#define REQUIRE(cond, ...)                                      \
  do {                                                          \
    if (!(cond)) {                                              \
      fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      fprintf(stderr, __VA_ARGS__);                             \
      fprintf(stderr, "\n");                                    \
      exit(1);                                                  \
    }                                                           \
  } while (0)

// make_plan and, when it succeeds, every invariant of the plan
static bool plan_and_check(int B, int T, int Hq, int Hkv, int D, int L, int cus, int window,
                           int page, long stride) {
  Plan p;
  const bool ok = ltree::make_plan(B, T, Hq, Hkv, D, L, cus, &p, window, page, stride);
  ++g_checked;
  if (!ok) return false;
  const char* fmt = "B=%d T=%d Hq=%d Hkv=%d D=%d L=%d cus=%d window=%d page=%d stride=%ld";
  const int Le = window > 0 ? window - 1 : L;
  REQUIRE(p.G * Hkv == Hq && p.R == p.G * T, fmt, B, T, Hq, Hkv, D, L, cus, window, page, stride);
  REQUIRE(p.chunk >= 64 && p.chunk % 64 == 0, fmt, B, T, Hq, Hkv, D, L, cus, window, page, stride);
  // the splits cover the (longest) prefix, none of them empty
  REQUIRE((i128)p.max_chunks * p.chunk >= Le, fmt, B, T, Hq, Hkv, D, L, cus, window, page, stride);
  REQUIRE(p.max_chunks == 0 || (i128)(p.max_chunks - 1) * p.chunk < Le, fmt, B, T, Hq, Hkv, D, L,
          cus, window, page, stride);
  REQUIRE(p.slots == (p.max_chunks > 0 ? p.max_chunks : 1), fmt, B, T, Hq, Hkv, D, L, cus, window,
          page, stride);
  // a split's keys at the row stride fit 32-bit element offsets
  const long s = stride > 0 ? stride : (long)Hkv * D;
  REQUIRE((i128)p.chunk * s <= INT_MAX, fmt, B, T, Hq, Hkv, D, L, cus, window, page, stride);
  // a paged split touches at most kMaxSplitPages pages
  if (page > 0) {
    REQUIRE((i128)p.chunk <= (i128)(ltree::kMaxSplitPages - 1) * page, fmt, B, T, Hq, Hkv, D, L,
            cus, window, page, stride);
  }
  // the workspace holds o (fp32-sized), scale and lse of every partial row, in order
  const i128 rows = (i128)B * Hkv * p.slots * p.R;
  REQUIRE(p.o_part_off == 0 && (i128)p.scale_part_off >= rows * D * 4, fmt, B, T, Hq, Hkv, D, L,
          cus, window, page, stride);
  REQUIRE((i128)p.lse_part_off >= (i128)p.scale_part_off + rows * 4, fmt, B, T, Hq, Hkv, D, L, cus,
          window, page, stride);
  REQUIRE((i128)p.bytes >= (i128)p.lse_part_off + rows * 4 && p.bytes % 256 == 0, fmt, B, T, Hq,
          Hkv, D, L, cus, window, page, stride);
  // output rows are indexed with 32-bit integers
  REQUIRE((i128)B * Hq * T < ((i128)1 << 31), fmt, B, T, Hq, Hkv, D, L, cus, window, page, stride);
  return true;
}

int main() {
  // ---- extreme sizes
  // B * Hq * T just below and at 2^31 (the merge's 32-bit row index)
  REQUIRE(plan_and_check(8388607, 256, 1, 1, 128, 4096, 256, 0, 0, 0), "B*Hq*T = 2^31 - 256");
  REQUIRE(!plan_and_check(8388608, 256, 1, 1, 128, 4096, 256, 0, 0, 0), "B*Hq*T = 2^31");
  REQUIRE(plan_and_check(1, 256, 8388607, 1, 64, 0, 256, 0, 0, 0), "Hq = 2^23 - 1, T = 256");
  // the longest prefix, with the largest heads and rows (split capped by 32-bit offsets)
  REQUIRE(plan_and_check(1, 64, 40, 8, 128, INT_MAX, 256, 0, 0, 0), "L = INT_MAX");
  REQUIRE(plan_and_check(1, 64, 4096, 4096, 128, INT_MAX, 256, 0, 0, 0), "Hkv*D = 2^19");
  REQUIRE(plan_and_check(1, 64, 8, 8, 128, INT_MAX, 256, 0, 0, ltree::kMaxRowStride),
          "largest stride");
  REQUIRE(!plan_and_check(1, 64, 8, 8, 128, 100, 256, 0, 0, ltree::kMaxRowStride + 8),
          "stride above the cap");
  REQUIRE(!plan_and_check(1, 64, 8, 8, 128, 100, 256, 0, 0, 1000), "stride below Hkv*D");
  REQUIRE(plan_and_check(1, 1, 1, 1, 64, 0, 1, 0, 0, 0), "smallest problem");
  REQUIRE(plan_and_check(1, 1, 1, 1, 64, INT_MAX, 1, 0, 0, 0), "one CU, longest prefix");
  REQUIRE(plan_and_check(1, 64, 40, 8, 128, 32768, 1 << 20, 0, 0, 0), "very many CUs");
  // windows: the largest, one equal to T, one shorter than T
  REQUIRE(plan_and_check(1, 64, 40, 8, 128, 0, 256, LTREE_MAX_WINDOW, 0, 0), "largest window");
  REQUIRE(!plan_and_check(1, 64, 40, 8, 128, 0, 256, LTREE_MAX_WINDOW + 1, 0, 0), "window > max");
  REQUIRE(plan_and_check(1, 64, 40, 8, 128, 0, 256, 64, 0, 0), "window = T");
  REQUIRE(!plan_and_check(1, 64, 40, 8, 128, 0, 256, 63, 0, 0), "window < T");
  // paged: one-key pages, vLLM-sized, huge pages
  REQUIRE(plan_and_check(1, 64, 40, 8, 128, 1 << 20, 256, 0, 1, 0), "1-key pages");
  REQUIRE(plan_and_check(4, 64, 32, 8, 128, INT_MAX, 256, 0, 16, 0), "16-key pages");
  REQUIRE(plan_and_check(1, 64, 40, 8, 128, INT_MAX, 256, 0, 1 << 20, 0), "huge pages");
  // invalid sizes
  const int bad[][6] = {{0, 8, 8, 8, 128, 10}, {1, 0, 8, 8, 128, 10}, {1, 257, 8, 8, 128, 10},
                        {1, 8, 8, 3, 128, 10}, {1, 8, 8, 8, 96, 10}, {1, 8, 8, 8, 128, -1},
                        {-5, 8, 8, 8, 128, 10}, {1, 8, 0, 8, 128, 10}, {1, 8, 8, 0, 128, 10}};
  for (const auto& b : bad) {
    REQUIRE(!plan_and_check(b[0], b[1], b[2], b[3], b[4], b[5], 256, 0, 0, 0), "bad sizes");
  }
  REQUIRE(!plan_and_check(1, 8, 8, 8, 128, 10, 0, 0, 0, 0), "zero CUs");
  REQUIRE(!plan_and_check(1, 8, 8, 8, 128, 10, 256, 0, -1, 0), "negative page size");

  // ---- the size checks shared by every call
  REQUIRE(ltree::check_sizes(1, 64, 40, 8, 128, 32768) == LTREE_OK, "qwq layer");
  REQUIRE(ltree::check_sizes(1, 257, 40, 8, 128, 1) == LTREE_ERR_UNSUPPORTED, "T > 256");
  REQUIRE(ltree::check_sizes(1, 64, 40, 8, 96, 1) == LTREE_ERR_UNSUPPORTED, "D = 96");
  REQUIRE(ltree::check_sizes(1, 64, 40, 7, 128, 1) == LTREE_ERR_INVALID_ARG, "Hq % Hkv");
  REQUIRE(ltree::check_sizes(INT_MAX, 256, INT_MAX, 1, 128, 1) == LTREE_ERR_UNSUPPORTED,
          "B*T*Hq*D overflow");
  REQUIRE(ltree::check_sizes(65536, 256, 1, 1, 128, 1) == LTREE_ERR_UNSUPPORTED, "2^31 exactly");
  REQUIRE(ltree::check_sizes(65535, 256, 1, 1, 128, 1) == LTREE_OK, "below 2^31");

  // ---- paged checks
  uint32_t pool = 0;
  int cap = 0;
  REQUIRE(ltree::check_paged(2, 8, 128, 256, 256, 128, 32768, 0, &pool, &cap) == LTREE_OK,
          "qwq pages");
  REQUIRE(pool == 256u * 256 * 8 * 128 * 2 && cap == 32768, "pool %u cap %d", pool, cap);
  REQUIRE(ltree::check_paged(2, 8, 128, 256, 256, 128, 32769, 0, &pool, &cap) ==
              LTREE_ERR_INVALID_ARG, "max_prefix_len past the block table");
  REQUIRE(ltree::check_paged(2, 8, 128, INT_MAX, 64, INT_MAX, INT_MAX, 0, &pool, &cap) == LTREE_OK,
          "huge pool, 64-key pages");
  REQUIRE(pool == 0 && cap == INT_MAX, "pool %u cap %d", pool, cap);
  REQUIRE(ltree::check_paged(2, 8, 128, INT_MAX, 16, 8, 100, 0, &pool, &cap) ==
              LTREE_ERR_UNSUPPORTED, "huge pool, 16-key pages");
  REQUIRE(ltree::check_paged(4, 8, 128, 1, 1 << 20, 1, 0, 0, &pool, &cap) == LTREE_OK,
          "page of 2^30 elements");
  REQUIRE(ltree::check_paged(4, 8, 128, 1, (1 << 20) + 64, 1, 0, 0, &pool, &cap) ==
              LTREE_ERR_UNSUPPORTED, "page above 2^30 elements");
  REQUIRE(ltree::check_paged(2, 8, 128, 64, 64, 4, 0, 512, &pool, &cap) == LTREE_OK,
          "window over pages");
  REQUIRE(cap == 256, "window cap %d", cap);
  REQUIRE(ltree::check_paged(2, 8, 128, 1 << 20, 256, 4, 0, 512, &pool, &cap) ==
              LTREE_ERR_UNSUPPORTED, "window over a pool of 2^31 bytes or more");
  for (int bad_page : {0, -1}) {
    REQUIRE(ltree::check_paged(2, 8, 128, 4, bad_page, 4, 0, 0, &pool, &cap) ==
                LTREE_ERR_INVALID_ARG, "page size %d", bad_page);
  }

  // ---- strides
  REQUIRE(ltree::check_strides(8, 128, 1024, 1024) == LTREE_OK, "packed");
  REQUIRE(ltree::check_strides(8, 128, 2048, 2048) == LTREE_OK, "interleaved");
  REQUIRE(ltree::check_strides(8, 128, 1020, 1024) == LTREE_ERR_INVALID_ARG, "short");
  REQUIRE(ltree::check_strides(8, 128, 1028, 1024) == LTREE_ERR_INVALID_ARG, "unaligned");
  REQUIRE(ltree::check_strides(8, 128, LONG_MAX / 8 * 8, 1024) == LTREE_ERR_UNSUPPORTED, "huge");
  REQUIRE(ltree::check_strides(8, 128, LONG_MAX, 1024) == LTREE_ERR_INVALID_ARG, "huge, unaligned");
  REQUIRE(ltree::check_strides(8, 128, LONG_MIN, 1024) == LTREE_ERR_INVALID_ARG, "negative");

  // ---- random sizes, extremes mixed in
  std::mt19937_64 rng(20261203);
  auto pick = [&](std::initializer_list<long> edges, long lo, long hi) -> long {
    if (rng() % 3 == 0) return *(edges.begin() + rng() % edges.size());
    return lo + (long)(rng() % (unsigned long)(hi - lo + 1));
  };
  for (int n = 0; n < 200000; ++n) {
    const int D = rng() % 2 ? 128 : 64;
    const int Hkv = (int)pick({1, 2, 8, 4096}, 1, 64);
    const int G = (int)pick({1, 5, 8, 1 << 16}, 1, 16);
    const int T = (int)pick({1, 64, 65, 256, 257}, 1, 256);
    const int B = (int)pick({1, 4, 1 << 20, INT_MAX}, 1, 4096);
    const int L = (int)pick({0, 1, 63, 64, 65, 32768, INT_MAX}, 0, 1 << 22);
    const int cus = (int)pick({1, 80, 256, 304, 1 << 16}, 1, 1024);
    const int window = rng() % 4 == 0 ? (int)pick({T, T + 1, 512, LTREE_MAX_WINDOW}, T, 1 << 16) : 0;
    const int page = rng() % 4 == 0 ? (int)pick({1, 16, 48, 64, 256, 1 << 20}, 1, 4096) : 0;
    const long stride = rng() % 4 == 0 ? (long)Hkv * D + 8 * (long)(rng() % 4096) : 0;
    if ((long)G * Hkv > INT_MAX) continue;
    plan_and_check(B, T, G * Hkv, Hkv, D, L, cus, window, page, stride);
  }
  printf("plans checked: %ld\n", g_checked);
  return 0;
}
