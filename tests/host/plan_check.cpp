// Host-only checks of the planner, built with g++ under ASan/UBSan by
// tests/test_host.py:
//  1. magic-number division agrees with '/' for random and edge operands;
//  2. the canonical iteration space visits exactly the same per-operand
//     offsets, in the same row-major order, as the uncanonicalised space,
//     for random shapes, broadcasts and strides.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "zk_plan.h"

using namespace zk;

static int fail(const char *what, long long a, long long b) {
  std::printf("FAIL %s %lld %lld\n", what, a, b);
  return 1;
}

static std::vector<std::vector<int64_t>> walk(int r, const int64_t *n, int nops,
                                              const int64_t (*st)[kMaxDims]) {
  int64_t total = 1;
  for (int k = 0; k < r; ++k) total *= n[k];
  std::vector<std::vector<int64_t>> out(nops);
  std::vector<int64_t> idx(r > 0 ? r : 1, 0);
  for (int64_t t = 0; t < total; ++t) {
    for (int o = 0; o < nops; ++o) {
      int64_t off = 0;
      for (int k = 0; k < r; ++k) off += idx[k] * st[o][k];
      out[o].push_back(off);
    }
    for (int k = r - 1; k >= 0; --k) {
      if (++idx[k] < n[k]) break;
      idx[k] = 0;
    }
  }
  return out;
}

int main() {
  std::mt19937_64 rng(1234);
  // 1. fast division
  const uint32_t ds[] = {1, 2, 3, 5, 7, 9, 10, 63, 64, 65, 255, 256, 1000,
                         1023, 1024, 4096, 4097, 65535, 65536, 1u << 20,
                         (1u << 30) + 1, 2147483647u};
  for (uint32_t d : ds) {
    FastDiv f = make_fastdiv(d);
    const uint32_t ns[] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2147483647u,
                           2147483646u, 123456789u};
    for (uint32_t n : ns) {
      if (n > 2147483647u) continue;
      if (fastdiv_eval(f, n) != n / d) return fail("fastdiv", n, d);
    }
    for (int t = 0; t < 20000; ++t) {
      uint32_t n = (uint32_t)(rng() & 0x7fffffffu);
      if (fastdiv_eval(f, n) != n / d) return fail("fastdiv", n, d);
    }
  }
  for (int t = 0; t < 200000; ++t) {
    uint32_t d = 1 + (uint32_t)(rng() % 0x7ffffffeu);
    uint32_t n = (uint32_t)(rng() & 0x7fffffffu);
    if (fastdiv_eval(make_fastdiv(d), n) != n / d) return fail("fastdiv", n, d);
  }
  // 2. canonicalisation preserves the offset sequence of every operand
  for (int t = 0; t < 3000; ++t) {
    int r = (int)(rng() % 6);
    int64_t n[kMaxDims];
    for (int k = 0; k < r; ++k) n[k] = 1 + (int64_t)(rng() % 4);
    int nops = 1 + (int)(rng() % 4);
    int64_t st[kMaxOps][kMaxDims];
    {
      int64_t d = 1;
      for (int k = r - 1; k >= 0; --k) { st[0][k] = d; d *= n[k]; }
    }
    for (int o = 1; o < nops; ++o) {
      int mode = (int)(rng() % 4);
      int64_t d = 1;
      for (int k = r - 1; k >= 0; --k) {
        if (mode == 0) { st[o][k] = d; d *= n[k]; }                 // dense
        else if (mode == 1) st[o][k] = (rng() % 2) ? 0 : st[0][k];  // broadcast
        else if (mode == 2) st[o][k] = (int64_t)(rng() % 7);        // random
        else st[o][k] = st[0][k];                                   // as out
      }
    }
    Canon c = canonicalise(r, n, nops, st);
    auto ref = walk(r, n, nops, st);
    auto got = walk(c.rank, c.n, nops, c.s);
    int64_t total = 1;
    for (int k = 0; k < r; ++k) total *= n[k];
    if (c.numel != total) return fail("numel", c.numel, total);
    for (int o = 0; o < nops; ++o) {
      if (ref[o].size() != got[o].size())
        return fail("count", (long long)ref[o].size(), (long long)got[o].size());
      for (size_t i = 0; i < ref[o].size(); ++i)
        if (ref[o][i] != got[o][i]) return fail("offset", ref[o][i], got[o][i]);
    }
    for (int k = 0; k < c.rank; ++k)
      if (c.n[k] == 1 && c.rank > 1) return fail("size-1 kept", k, c.rank);
  }
  std::printf("OK\n");
  return 0;
}
