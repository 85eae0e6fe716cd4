// Host-only checks of the planner, built with g++ under ASan/UBSan by
// tests/test_host.py:
//  1. magic-number division agrees with '/' for random and edge operands;
//  2. the canonical iteration space visits exactly the same per-operand
//     offsets, in the same row-major order, as the uncanonicalised space,
//     for random shapes, broadcasts and strides;
//  3. every reduction plan of random backward and reduce calls meets the
//     shape assumptions its stage-1 kernel and launch are written for
//     (patterns, divisibility, partial counts, grid limits, workspace).
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
  // 3. reduction plans against the assumptions of their kernels
  const int64_t sizes[] = {1, 2, 3, 4, 7, 9, 16, 64, 256, 260, 1024, 2048, 4096};
  int seen[K_COUNT] = {0};
  for (int t = 0; t < 20000; ++t) {
    zk_desc da{}, db{};
    const int r = 1 + (int)(rng() % 4);
    da.rank = r;
    int64_t numel = 1;
    for (int k = 0; k < r; ++k) {
      int64_t v = sizes[rng() % 13];
      if (numel * v > ((int64_t)1 << 26)) v = 1;
      da.sizes[k] = v;
      numel *= v;
    }
    // b: a's shape with random dims set to 1, possibly fewer leading dims
    const int rb = 1 + (int)(rng() % r);
    db.rank = rb;
    for (int k = 0; k < rb; ++k) {
      const int64_t v = da.sizes[r - rb + k];
      db.sizes[k] = (rng() % 2) ? v : 1;
    }
    for (zk_desc *d : {&da, &db}) {
      int64_t s = 1;
      for (int k = d->rank - 1; k >= 0; --k) { d->strides[k] = s; s *= d->sizes[k]; }
    }
    if (rng() % 2) std::swap(da, db);
    const uintptr_t q = (rng() % 4) ? 0 : 4;  // aligned or not
    BwdPlan p;
    const zk_op op = (zk_op)(rng() % 4);
    const zk_epi epi = (zk_epi)(rng() % 3);
    const bool wa = rng() % 4 != 0, wb = rng() % 4 != 0;
    zk_status st;
    if (rng() % 3 == 0) {
      st = plan_reduce(db.rank <= da.rank ? da : db, db.rank <= da.rank ? db.rank : da.rank,
                       db.rank <= da.rank ? db.sizes : da.sizes, q, q, &p);
    } else {
      st = plan_bwd(op, epi, da, db, wa, wb, q, q, q, q, q, q, q, &p);
    }
    if (st != ZK_OK) continue;
    const Canon &c = p.c;
    size_t need = 0;
    for (int i = 0; i < p.nred; ++i) {
      const RedPlan &rp = p.red[i];
      if (rp.kernel >= 0 && rp.kernel < K_COUNT) ++seen[rp.kernel];
      need += (size_t)rp.partials * (size_t)rp.kept * (size_t)rp.csub * 8u;
      if (rp.csub != 1 && rp.kernel != K_RED_COL) return fail("csub", rp.csub, rp.kernel);
      // a stage-1 class that leaves partials covers every term with >= 1 of them
      if (rp.red > 0 && (rp.kernel == K_RED_COL || rp.kernel == K_RED_ROW ||
                         rp.kernel == K_RED_TILE || rp.kernel == K_RED_GENERIC) &&
          (rp.partials < 1 || rp.chunk < 1))
        return fail("no partials", rp.partials, rp.chunk);
      const int64_t inner = c.rank > 0 ? c.n[c.rank - 1] : 1;
      switch (rp.kernel) {
        case K_RED_COL: {
          // [rows, cols] column sums: the canonical [R, K], or [R1, K * C] for
          // [R1, K, C] -> [K, 1] (each kept element owns C columns)
          if (rp.csub == 1) {
            if (c.rank != 2 || rp.kept != c.n[1] || rp.red != c.n[0] ||
                rp.col_rows != c.n[0] || rp.col_cols != c.n[1])
              return fail("col shape", rp.kept, c.rank);
          } else {
            if (c.rank != 3 || rp.csub != c.n[2] || rp.kept != c.n[1] ||
                rp.col_rows != c.n[0] || rp.col_cols != c.n[1] * c.n[2] ||
                rp.red != c.n[0] * c.n[2])
              return fail("col sub shape", rp.csub, c.rank);
            if (rp.partials * rp.csub >= ((int64_t)1 << 31)) return fail("col sub index", rp.partials, rp.csub);
          }
          const int64_t rows = rp.col_rows, cols = rp.col_cols;
          if (cols % 4 != 0) return fail("col K%4", cols, 0);
          if (!(rp.nw == 1 || rp.nw == 4 || rp.nw == 16)) return fail("col nw", rp.nw, 0);
          if (rp.chunk < 1) return fail("col rcw", rp.chunk, 0);
          // narrow columns fold rows into 256-wide ones: fold * K == 256
          const int64_t f = rp.fold;
          if (f < 1 || (f > 1 && (cols * f != 256 || rows % f != 0)))
            return fail("col fold", f, cols);
          const int64_t R0 = rows / f, Kw = cols * f;
          const int64_t P = (R0 + rp.nw * rp.chunk - 1) / (rp.nw * rp.chunk);
          if (P < 1 || rp.partials != P * f) return fail("col partials", rp.partials, P * f);
          // short columns: the one band of rows is split evenly over the waves
          if (P == 1 && rp.nw * rp.chunk > R0 + rp.nw - 1) return fail("col idle waves", rp.nw, rp.chunk);
          // the grid stays within the dispatch limit unless one band is left
          if (P > 1 && ((Kw + 255) / 256) * P > kMaxGridBlocks) return fail("col grid", P, 0);
          break;
        }
        case K_RED_ROW: {
          if (inner % 4 != 0 || inner < 256) return fail("row inner", inner, 0);
          if (rp.chunk != inner && rp.chunk % 256 != 0) return fail("row chunk", rp.chunk, inner);
          const int64_t R1 = c.numel / inner / rp.kept;
          const int64_t NC = (inner + rp.chunk - 1) / rp.chunk;
          if (R1 * inner * rp.kept != c.numel) return fail("row cover", R1, rp.kept);
          // blockwise: four chunks of a row share one partial
          if (rp.nw != 1 && (rp.nw != 4 || NC % 4 != 0)) return fail("row waves", rp.nw, NC);
          if (rp.partials != R1 * NC / rp.nw) return fail("row partials", rp.partials, R1 * NC);
          break;
        }
        case K_RED_ROWD: {
          if (rp.partials != 0 || inner % 4 != 0) return fail("rowd", rp.partials, inner);
          if (rp.kept * rp.red != c.numel) return fail("rowd cover", rp.kept, rp.red);
          if (rp.red < kDirMinTerms || rp.red > kDirMaxTerms) return fail("rowd terms", rp.red, 0);
          // plain row sums ([K, T]: the reduced run is the whole inner dim) of
          // many elements go to red_row
          if (rp.red == inner && c.numel > kDirRowSumMaxElems) return fail("rowd size", c.numel, 0);
          if (!(rp.chunk == 1 || rp.chunk == 2 || rp.chunk == 4) || rp.red > 4096 * rp.chunk)
            return fail("rowd vectors", rp.chunk, rp.red);
          break;
        }
        case K_RED_ROWSEG: {
          // dense rows of C = 4 * 2^j < 256 elements, the inner dim reduced;
          // rank 2 finishes in place, rank 3 leaves [R1, K] partials
          const int64_t C = rp.chunk;
          if (rp.kept * rp.red != c.numel || c.n[c.rank - 1] != C) return fail("rowseg", rp.kept, C);
          if (C < 4 || C > 256 || 256 % C != 0) return fail("rowseg C", C, 0);
          if (c.rank == 2 ? (rp.partials != 0 || rp.red != C)
                          : (c.rank != 3 || rp.partials != c.n[0] || rp.kept != c.n[1]))
            return fail("rowseg partials", rp.partials, c.rank);
          // rank 3: at most C (<= 256) row sums a kept element as partials
          if (rp.partials > C || rp.partials > kRowSegMaxPartials)
            return fail("rowseg partial bound", rp.partials, C);
          break;
        }
        case K_RED_GEND: {
          if (rp.partials != 0 || rp.kept * rp.red != c.numel) return fail("gend", rp.kept, rp.red);
          if (rp.red < kGenDirMinTerms || rp.red > kGenDirMaxTerms) return fail("gend terms", rp.red, 0);
          break;
        }
        case K_RED_RUN: {
          // the two innermost dims form a dense run of 64..256 elements, 32-bit
          // offsets, at least kRunMinBlocks blocks and two runs a block
          const int64_t L = c.n[c.rank - 1] * (c.rank >= 2 ? c.n[c.rank - 2] : 1);
          if (rp.partials != 0 || rp.kept * rp.red != c.numel || rp.chunk != L)
            return fail("run cover", rp.kept, rp.red);
          if (c.rank < 3 || L < kRunMinLen || L > kRunMaxLen || p.idx64) return fail("run shape", L, c.rank);
          if (c.s[0][c.rank - 1] != 1 || c.s[0][c.rank - 2] != c.n[c.rank - 1]) return fail("run dense", 0, 0);
          const int ko = rp.which == 0 ? 3 : 4;
          int64_t blocks = 1, runs = 1;
          for (int k = 0; k < c.rank - 2; ++k) (c.s[ko][k] != 0 ? blocks : runs) *= c.n[k];
          if (blocks < kRunMinBlocks || runs < 2 || blocks * runs * L != c.numel) return fail("run blocks", blocks, runs);
          break;
        }
        case K_RED_TILE: {
          if (c.rank != 2 || c.n[1] % 4 != 0) return fail("tile shape", c.rank, c.n[1]);
          if (rp.chunk != 64 && rp.chunk != 128) return fail("tile rows", rp.chunk, 0);
          if (rp.partials != (c.n[0] + rp.chunk - 1) / rp.chunk) return fail("tile partials", rp.partials, 0);
          break;
        }
        case K_RED_GENERIC: {
          if (rp.red > 0 && rp.partials * rp.chunk < rp.red) return fail("gen cover", rp.partials, rp.red);
          if (!p.empty_space && rp.kept * rp.red != c.numel) return fail("gen count", rp.kept, rp.red);
          break;
        }
        default:
          return fail("kernel", rp.kernel, 0);
      }
    }
    if (p.workspace < need) return fail("workspace", (long long)p.workspace, (long long)need);
  }
  for (int k : {K_RED_COL, K_RED_ROW, K_RED_ROWD, K_RED_GEND, K_RED_RUN, K_RED_TILE, K_RED_GENERIC})
    if (k != K_RED_TILE && seen[k] == 0) return fail("class never planned", k, 0);
  // 4. forward plans: the dense operand of fwd_row walks the output layout,
  //    128-bit paths only on multiples of 4 and aligned pointers, rank <= 3
  for (int t = 0; t < 20000; ++t) {
    zk_desc da{}, db{};
    const int r = 1 + (int)(rng() % 4);
    da.rank = r;
    int64_t numel = 1;
    for (int k = 0; k < r; ++k) {
      int64_t v = sizes[rng() % 13];
      if (numel * v > ((int64_t)1 << 26)) v = 1;
      da.sizes[k] = v;
      numel *= v;
    }
    const int rb = (int)(rng() % (r + 1));
    db.rank = rb;
    for (int k = 0; k < rb; ++k) db.sizes[k] = (rng() % 2) ? da.sizes[r - rb + k] : 1;
    for (zk_desc *d : {&da, &db}) {
      int64_t s2 = 1;
      for (int k = d->rank - 1; k >= 0; --k) { d->strides[k] = s2; s2 *= d->sizes[k]; }
    }
    if (r == 2 && rng() % 3 == 0) {  // a transposed view
      std::swap(da.sizes[0], da.sizes[1]);
      da.strides[0] = 1;
      da.strides[1] = da.sizes[0];
    }
    if (rng() % 2) std::swap(da, db);
    const uintptr_t pa = (rng() % 4) ? 0 : 4, pb = (rng() % 4) ? 0 : 4, po = (rng() % 4) ? 0 : 4;
    FwdPlan f;
    if (plan_fwd((zk_op)(rng() % 4), (zk_epi)(rng() % 3), da, db, pa, pb, po, &f) != ZK_OK)
      continue;
    if (f.empty) continue;
    const Canon &c = f.c;
    const int64_t inner = c.n[c.rank - 1];
    switch (f.kernel) {
      case K_FWD_FLAT:
        if (f.vec == 4 && (pa || pb || po)) return fail("flat vec align", f.vec, 0);
        break;
      case K_FWD_ROW: {
        if (c.rank > 3) return fail("row rank", c.rank, 0);
        const int big = f.swap ? 2 : 1;
        for (int k = 0; k < c.rank; ++k)
          if (c.n[k] > 1 && c.s[big][k] != c.s[0][k]) return fail("row dense", k, c.s[big][k]);
        if (f.vec == 4 && (inner % 4 != 0 || po || (f.swap ? pb : pa)))
          return fail("row vec", inner, 0);
        break;
      }
      case K_FWD_TILE:
        if (c.rank != 2 || f.vec != 4 || c.n[1] % 4 != 0 || po) return fail("tile", c.rank, c.n[1]);
        break;
      case K_FWD_GENERIC:
        if (f.vec == 4 && po) return fail("generic vec align", 0, 0);
        break;
      default:
        return fail("fwd kernel", f.kernel, 0);
    }
  }
  // 5. shapes far beyond the random range: more than 2^30 kept columns, and
  //    middle sums over many rows of short rows, plan in bounded time with
  //    at least one partial, within the kernels' index limits
  {
    const int64_t big = (int64_t)1 << 31;
    zk_desc din{}, dk{};
    din.rank = 2;
    din.sizes[0] = 2;
    din.sizes[1] = big;
    din.strides[0] = big;
    din.strides[1] = 1;
    const int64_t tgt[1] = {big};
    BwdPlan p;
    if (plan_reduce(din, 1, tgt, 0, 0, &p) != ZK_OK) return fail("huge reduce", 0, 0);
    if (p.nred != 1 || p.red[0].kernel != K_RED_COL || p.red[0].partials < 1 ||
        p.red[0].chunk < 1 || p.red[0].kept != big)
      return fail("huge reduce plan", p.red[0].kernel, p.red[0].partials);
    dk.rank = 1;
    dk.sizes[0] = big;
    dk.strides[0] = 1;
    BwdPlan q;
    if (plan_bwd(ZK_MUL, ZK_EPI_NONE, din, dk, true, true, 0, 0, 0, 0, 0, 0, 0, &q) != ZK_OK)
      return fail("huge bwd", 0, 0);
    if (q.nred != 1 || q.red[0].kernel != K_RED_COL || q.red[0].partials < 1 ||
        q.red[0].chunk < 1 || !q.fused_big)
      return fail("huge bwd plan", q.red[0].kernel, q.red[0].partials);
    // [2^22, 4, 4] -> [4, 1]: column sums of [2^22, 16] with bounded partials
    zk_desc m{};
    m.rank = 3;
    m.sizes[0] = (int64_t)1 << 22;
    m.sizes[1] = 4;
    m.sizes[2] = 4;
    m.strides[0] = 16;
    m.strides[1] = 4;
    m.strides[2] = 1;
    const int64_t t2[2] = {4, 1};
    BwdPlan r;
    if (plan_reduce(m, 2, t2, 0, 0, &r) != ZK_OK) return fail("middle", 0, 0);
    const RedPlan &rr = r.red[0];
    if (rr.kernel != K_RED_COL || rr.csub != 4 || rr.partials > 65536 ||
        r.workspace > ((size_t)64 << 20) / 16)
      return fail("middle plan", rr.kernel, (long long)r.workspace);
  }
  // 6. debug pointer checks: the decision on synthetic runtime records
  {
    const PtrRecord dev0{1, kMemDevice, 0}, dev1{1, kMemDevice, 1}, host{1, kMemHost, 0},
        unreg{1, kMemUnregistered, -1}, unknown{0, kMemUnregistered, -1},
        managed{1, kMemManaged, 3};
    const PtrRecord ok3[3] = {dev0, dev0, managed};
    if (check_ptr_records(ok3, 3, 0) != ZK_OK) return fail("debug ok", 0, 0);
    if (check_ptr_records(ok3, 0, 0) != ZK_OK) return fail("debug none", 0, 0);
    if (check_ptr_records(ok3, 3, -1) != ZK_ERR_DEVICE) return fail("debug no device", 0, 0);
    for (const PtrRecord &bad : {dev1, host, unreg, unknown}) {
      const PtrRecord mix[3] = {dev0, bad, dev0};
      if (check_ptr_records(mix, 3, 0) != ZK_ERR_DEVICE) return fail("debug bad", bad.mem_type, 0);
    }
    const PtrRecord on1[2] = {dev1, managed};
    if (check_ptr_records(on1, 2, 1) != ZK_OK) return fail("debug device 1", 0, 0);
    if (check_ptr_records(on1, 2, 0) != ZK_ERR_DEVICE) return fail("debug wrong device", 0, 0);
  }
  std::printf("OK\n");
  return 0;
}
