// zk_fwd.hip -- forward kernels for gfx950 (wave64).
//
// out[i] = epi(a[off_a(i)] (op) b[off_b(i)]) over the canonical iteration
// space (Operator chapter of the "Zero" book, "broadcast": a repeated operand
// dim reads coordinate 0, here a stride of 0).  The output is always dense.
// Classes:
//   flat    : a, b, out walk the same dense layout -> 128-bit streams
//   row     : one dense operand, the other rank <= 3 with any strides; its
//             inner dim is a broadcast scalar, a contiguous run, or a gather
//   tile    : rank 2 with a transposed operand (x[i,j] at i + j*ld); 64x64
//             tiles are staged through LDS so both HBM sides are coalesced
//   generic : any rank <= 8, per-element offsets
#include <atomic>
#include <type_traits>

#include "zk_device.h"

namespace zk {

constexpr int kBlock = 256;

// Vector accesses per thread of the streaming kernels.  On MI355X one
// 128-bit vector per lane and one tile per block, over a grid as large as
// the data, streams fastest (measured: a dense a+b reaches ~6.4 TB/s this
// way against ~5.7 TB/s with four vectors per lane); the operands that are
// read or written once also carry the non-temporal hint.  With the GeLU
// epilogue each block first copies the 5.4 KB erfc table into LDS, so a
// block takes two vectors per lane to halve that traffic.
constexpr int row_unroll(int epi) { (void)epi; return 1; }
// The GeLU row kernel (long arithmetic per element, 64 VGPRs) runs a grid of
// 2 blocks of 1024 lanes per CU (all resident at once, 8 waves per SIMD)
// that loops over the tiles and issues the next tile's loads before the
// current tile's arithmetic.  Each block stages the GeLU table in LDS once,
// so few large blocks stage it least often.  Measured on the [4096, 1024]
// step: 9.9 us, against 10.5 us with 8 blocks of 256 lanes per CU and
// 11.0 us with one tile per block.
constexpr bool kRowPrefetch = true;
// Rows (along the transposed operand's contiguous columns) per fwd_tile tile
// (128 and 256 measured slower on the [4096, 4096] transposed product).
constexpr int kTileRows = 64;
constexpr int kRowGeluBlocksPerCU = 2;
constexpr int kRowGeluBlk = 1024;  // threads per block of the GeLU row kernel

// Launches give one block per tile; kernels loop over tiles with a grid
// stride, so a grid capped here still covers any size.  (A dispatch counts
// its grid in work-items with 32 bits: blocks * kBlock must stay below 2^32.)
constexpr int64_t kMaxBlocks = (int64_t)1 << 22;

template <int V>
using IC = std::integral_constant<int, V>;

// Calls fn(IC<op>, IC<epi>) for the runtime (op, epi).
template <typename Fn>
static hipError_t with_op_epi(zk_op op, zk_epi epi, Fn &&fn) {
  switch ((int)op * 3 + (int)epi) {
    case 0: return fn(IC<ZK_ADD>{}, IC<ZK_EPI_NONE>{});
    case 1: return fn(IC<ZK_ADD>{}, IC<ZK_EPI_GELU>{});
    case 2: return fn(IC<ZK_ADD>{}, IC<ZK_EPI_RELU>{});
    case 3: return fn(IC<ZK_SUB>{}, IC<ZK_EPI_NONE>{});
    case 4: return fn(IC<ZK_SUB>{}, IC<ZK_EPI_GELU>{});
    case 5: return fn(IC<ZK_SUB>{}, IC<ZK_EPI_RELU>{});
    case 6: return fn(IC<ZK_MUL>{}, IC<ZK_EPI_NONE>{});
    case 7: return fn(IC<ZK_MUL>{}, IC<ZK_EPI_GELU>{});
    case 8: return fn(IC<ZK_MUL>{}, IC<ZK_EPI_RELU>{});
    case 9: return fn(IC<ZK_DIV>{}, IC<ZK_EPI_NONE>{});
    case 10: return fn(IC<ZK_DIV>{}, IC<ZK_EPI_GELU>{});
    case 11: return fn(IC<ZK_DIV>{}, IC<ZK_EPI_RELU>{});
  }
  return hipErrorInvalidValue;
}

Space make_space(const Canon &c) {
  Space s{};
  s.rank = c.rank;
  s.numel = c.numel;
  for (int k = 0; k < kMaxDims; ++k) {
    s.n[k] = k < c.rank ? c.n[k] : 1;
    for (int o = 0; o < kMaxOps; ++o) s.s[o][k] = k < c.rank ? c.s[o][k] : 0;
    uint32_t d = (s.n[k] >= 1 && s.n[k] < ((int64_t)1 << 31)) ? (uint32_t)s.n[k] : 1u;
    s.fd[k] = make_fastdiv(d);
  }
  return s;
}

// ------------------------------------------------------------------ flat
// Tiles of kBlock * U * VEC elements, t = blockIdx.x, +gridDim.x, ... (the
// launch gives one tile per block up to the grid cap).
template <int OP, int EPI, int VEC, int U>
__global__ __launch_bounds__(kBlock) void k_fwd_flat(const float *a,
                                                     const float *b,
                                                     float *out, int64_t n) {
  __shared__ double s_gelu[EPI == ZK_EPI_GELU ? kGeluTabLen : 1];
  if constexpr (EPI == ZK_EPI_GELU) gelu_tab_load(s_gelu);
  constexpr int64_t tile = (int64_t)kBlock * U * VEC;
  const int64_t ntiles = (n + tile - 1) / tile;
  // With one block per tile, block b takes tile (b % 8) * (ntiles / 8) +
  // b / 8: blocks go to the 8 XCDs in turn, so each XCD walks one contiguous
  // eighth of the arrays (measured on MI355X, the 1.6 GB residual add:
  // 245.2-245.6 us against 246.7-249.1 in tile order; a read-and-write
  // stream such as a copy measured slower that way, so only this kernel,
  // with its two reads and one write, does it).
  const bool xcd = (int64_t)gridDim.x == ntiles && ntiles % 8 == 0;
  for (int64_t t0 = blockIdx.x; t0 < ntiles; t0 += gridDim.x) {
    const int64_t t = xcd ? (t0 % 8) * (ntiles / 8) + t0 / 8 : t0;
    if constexpr (VEC == 4) {
      const int64_t base = t * tile + (int64_t)threadIdx.x * 4;
      float4 va[U], vb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kBlock * 4;
        if (i + 4 <= n) {
          va[u] = ld4_nt(a + i);
          vb[u] = ld4_nt(b + i);
        }
      }
      uint32_t redo_bits = 0;  // bit 4u+k: element needs the GeLU double-double path
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + (int64_t)u * kBlock * 4;
        if (i + 4 <= n) {
          const float x[4] = {va[u].x, va[u].y, va[u].z, va[u].w};
          const float y[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
          float r[4];
          uint32_t redo;
          fwd4_fast<OP, EPI>(x, y, r, redo, s_gelu);
          redo_bits |= redo << (4 * u);
          st4_nt(out + i, make_float4(r[0], r[1], r[2], r[3]));
        } else if (i < n) {
          for (int64_t j = i; j < n; ++j) out[j] = fwd32<OP, EPI>(a[j], b[j], s_gelu);
        }
      }
      if constexpr (EPI == ZK_EPI_GELU) {
        while (redo_bits) {  // rare: near a rounding tie
          const int bit = __builtin_ctz(redo_bits);
          redo_bits &= redo_bits - 1;
          const int64_t j = base + (int64_t)(bit >> 2) * kBlock * 4 + (bit & 3);
          out[j] = gelu32_slow(op32<OP>(a[j], b[j]));
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = t * tile + (int64_t)u * kBlock + threadIdx.x;
        if (i < n) out[i] = fwd32<OP, EPI>(a[i], b[i], s_gelu);
      }
    }
  }
}

// ------------------------------------------------------------------- row
// Offset of a non-dense operand (strides ss) at flat output index i of a
// rank <= 3 space.  Fully unrolled so kernel-argument arrays are indexed by
// constants.
struct RowArgs {
  int32_t rank;
  int64_t n[3];
  int64_t ss[3];
  FastDiv fd[3];
  int64_t numel;
  float sval;  // SM_ARG: the scalar operand
};

template <typename I>
__device__ __forceinline__ I row_offset(const RowArgs &ra, I i) {
  I off = 0;
  I rest = i;
#pragma unroll
  for (int k = 2; k >= 1; --k) {
    if (k < ra.rank) {
      I q;
      if constexpr (sizeof(I) == 4) q = (I)fdiv(ra.fd[k], (uint32_t)rest);
      else q = rest / (I)ra.n[k];
      I c = rest - q * (I)ra.n[k];
      off += c * (I)ra.ss[k];
      rest = q;
    }
  }
  off += rest * (I)ra.ss[0];
  return off;
}

template <int OP, int EPI, int VEC, int SMODE, bool SWAP, typename I, int BLK>
__global__ __launch_bounds__(BLK) __attribute__((amdgpu_waves_per_eu(4))) void k_fwd_row(const float *big,
                                                    const float *small,
                                                    float *out, RowArgs ra) {
  __shared__ double s_gelu[EPI == ZK_EPI_GELU ? kGeluTabLen : 1];
  constexpr int U = row_unroll(EPI);
  constexpr I tile = (I)BLK * U * VEC;
  const I n = (I)ra.numel;
  const I sin = (I)ra.ss[ra.rank - 1];
  if constexpr (VEC == 4) {
    // Tiles t = blockIdx.x, +gridDim.x, ... (the launch gives one per block).
    const I ntiles = (n + tile - 1) / tile;
    auto load = [&](I t, float4 *vb, float4 *vs) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const I i = t * tile + (I)threadIdx.x * 4 + (I)u * BLK * 4;
        if (i < n) {
          vb[u] = ld4_nt(big + i);
          if constexpr (SMODE == SM_ARG) {
            vs[u] = make_float4(ra.sval, ra.sval, ra.sval, ra.sval);
          } else if constexpr (SMODE == SM_BCAST) {
            const float s = small[row_offset<I>(ra, i)];
            vs[u] = make_float4(s, s, s, s);
          } else if constexpr (SMODE == SM_CONTIG) {
            vs[u] = ld4(small + row_offset<I>(ra, i));
          } else {
            const I off = row_offset<I>(ra, i);
#pragma unroll
            for (int k = 0; k < 4; ++k) el(vs[u], k) = small[off + (I)k * sin];
          }
        }
      }
    };
    auto process = [&](I t, const float4 *vb, const float4 *vs) {
      const I base = t * tile + (I)threadIdx.x * 4;
      uint32_t redo_bits = 0;  // bit 4u+k: element needs the GeLU double-double path
      float4 res[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const I i = base + (I)u * BLK * 4;
        if (i < n) {
          float x[4], y[4], r[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            x[k] = SWAP ? el(vs[u], k) : el(vb[u], k);
            y[k] = SWAP ? el(vb[u], k) : el(vs[u], k);
          }
          uint32_t redo;
          fwd4_fast<OP, EPI>(x, y, r, redo, s_gelu);
          redo_bits |= redo << (4 * u);
          res[u] = make_float4(r[0], r[1], r[2], r[3]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const I i = base + (I)u * BLK * 4;
        if (i < n) st4_nt(out + i, res[u]);
      }
      if constexpr (EPI == ZK_EPI_GELU) {
        while (redo_bits) {  // rare: near a rounding tie; reload the operands
          const int bit = __builtin_ctz(redo_bits);
          redo_bits &= redo_bits - 1;
          const I i = base + (I)(bit >> 2) * BLK * 4;
          const I off = SMODE == SM_ARG ? (I)0 : row_offset<I>(ra, i);
          const int k = bit & 3;
          float vsm;
          if constexpr (SMODE == SM_ARG) vsm = ra.sval;
          else if constexpr (SMODE == SM_BCAST) vsm = small[off];
          else if constexpr (SMODE == SM_CONTIG) vsm = small[off + k];
          else vsm = small[off + (I)k * sin];
          const float vbig = big[i + k];
          const float h = SWAP ? op32<OP>(vsm, vbig) : op32<OP>(vbig, vsm);
          out[i + k] = gelu32_slow(h);
        }
      }
    };
    // The first tile's loads are issued before the GeLU table is staged in
    // LDS, so the two latencies overlap.
    float4 vb[U], vs[U];
    I t = (I)blockIdx.x;
    if (t < ntiles) load(t, vb, vs);
    if constexpr (EPI == ZK_EPI_GELU) gelu_tab_load(s_gelu);
    for (; t < ntiles; t += (I)gridDim.x) {
      if constexpr (kRowPrefetch && EPI == ZK_EPI_GELU) {
        // the next tile's loads are issued before this tile's arithmetic
        float4 nb[U], ns[U];
        const I tn = t + (I)gridDim.x;
        if (tn < ntiles) load(tn, nb, ns);
        process(t, vb, vs);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          vb[u] = nb[u];
          vs[u] = ns[u];
        }
      } else {
        if (t != (I)blockIdx.x) load(t, vb, vs);
        process(t, vb, vs);
      }
    }
  } else {
    if constexpr (EPI == ZK_EPI_GELU) gelu_tab_load(s_gelu);
    // 64-bit loop counter: i + stride may pass 2^31 even when n does not
    for (int64_t i64 = (int64_t)blockIdx.x * BLK + threadIdx.x; i64 < (int64_t)n;
         i64 += (int64_t)gridDim.x * BLK) {
      const I i = (I)i64;
      const float vbig = big[i];
      const float vsm = SMODE == SM_ARG ? ra.sval : small[row_offset<I>(ra, i)];
      out[i] = SWAP ? fwd32<OP, EPI>(vsm, vbig, s_gelu) : fwd32<OP, EPI>(vbig, vsm, s_gelu);
    }
  }
}

// ------------------------------------------------------------- bcrows
// A dense operand of n0 rows of n1 elements (n1 % 4 == 0, n1 >=
// kBcRowsMinCols) combined with one contiguous row vector that every row shares (the other operand's outer
// stride is 0, as the attention mask [1,1,S,S] against scores [B,H,S,S]): a
// lane reads a 16-byte piece of the row vector once and applies it to the
// same piece of kBcRows rows (n0 % kBcRows == 0), so the shared vector crosses
// the L2 once per kBcRows rows instead of once per row.  Group g of rows
// covers rows g * kBcRows ...; vector v of the grid is piece v % (n1 / 4) of
// group v / (n1 / 4).  One binary32 operation per element, as everywhere.
constexpr int kBcRows = 2;
// Only for row vectors of at least this many elements (256 KiB): a short
// vector stays in each CU's L1 and costs nothing to re-read, and there the
// paired rows only disturb the stream (measured on MI355X: the 4 MiB mask
// row, add 174-178 -> 167-168 us; gamma[4096] against h[32768, 4096],
// 170 -> 171-173 us, so that one stays on the row kernel).  Four rows a
// lane measured 172.7 us on the mask add.
constexpr int64_t kBcRowsMinCols = (int64_t)1 << 16;
struct BcRowsArgs {
  int64_t n1;     // row length (elements)
  int64_t total;  // (n0 / kBcRows) * (n1 / 4) vectors
  uint32_t vpr;   // n1 / 4, 16-byte pieces per row
  FastDiv fv;     // divides by vpr (32-bit index path)
};

template <int OP, int EPI, bool SWAP, typename I>
__global__ __launch_bounds__(kBlock) void k_fwd_bcrows(const float *big, const float *small,
                                                       float *out, BcRowsArgs ba) {
  static_assert(EPI != ZK_EPI_GELU, "the GeLU epilogue takes the row kernel");
  const I n1 = (I)ba.n1;
  for (int64_t v64 = (int64_t)blockIdx.x * kBlock + threadIdx.x; v64 < ba.total;
       v64 += (int64_t)gridDim.x * kBlock) {
    I g;
    if constexpr (sizeof(I) == 4) g = (I)fdiv(ba.fv, (uint32_t)v64);
    else g = (I)(v64 / (int64_t)ba.vpr);
    const I j = ((I)v64 - g * (I)ba.vpr) * 4;
    const I i0 = g * (I)kBcRows * n1 + j;
    const float4 sv = ld4(small + j);
    // The rows one after another: a row's load follows the previous row's
    // store (out may alias big as far as the compiler knows), so a lane has
    // one 16-byte vector of the stream in flight; with both rows' loads
    // issued first the 4 MiB mask add measured 171-172 us against 167-168.
#pragma unroll
    for (int k = 0; k < kBcRows; ++k) {
      const float4 x = ld4_nt(big + i0 + (I)k * n1);
      float4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        el(r, e) = SWAP ? fwd32<OP, EPI>(el(sv, e), el(x, e), nullptr)
                        : fwd32<OP, EPI>(el(x, e), el(sv, e), nullptr);
      st4_nt(out + i0 + (I)k * n1, r);
    }
  }
}

// ------------------------------------------------------------------ tile
// out[R, C] row-major; T[i, j] at i + j*ld (transposed view); O[i, j] at
// i*os0 + j*os1.  64x64 tiles (one per block up to the grid cap): T is read
// down its contiguous columns into LDS, then rows of the tile are combined
// with O and written as 128-bit row segments.
struct TileArgs {
  int64_t R, C, ld, os0, os1;
  int64_t tiles_c, ntiles;
  int32_t tv;  // T's columns start 16-byte aligned: 128-bit loads
};

template <int OP, int EPI, int OMODE, bool SWAP, int TI>
__global__ __launch_bounds__(kBlock) void k_fwd_tile(const float *tr,
                                                     const float *oth,
                                                     float *out, TileArgs ta) {
  // TI rows (along T's contiguous columns) x 64 columns per tile
  __shared__ float tile[64][TI + 1];
  __shared__ double s_gelu[EPI == ZK_EPI_GELU ? kGeluTabLen : 1];
  if constexpr (EPI == ZK_EPI_GELU) gelu_tab_load(s_gelu);
  const int t = threadIdx.x;
  for (int64_t bt = blockIdx.x; bt < ta.ntiles; bt += gridDim.x) {
    // Diagonal order: blocks running together take different row tiles, so
    // their column runs of T start at different offsets within the column
    // stride (with one row tile for all, every concurrent read would share
    // its low address bits, and with them the same few HBM channels).
    const int64_t tiles_r = ta.ntiles / ta.tiles_c;
    const int64_t tr_j = bt % ta.tiles_c;
    const int64_t tr_i = (bt / ta.tiles_c + tr_j) % tiles_r;
    const int64_t i0 = tr_i * TI, j0 = tr_j * 64;
    if (ta.tv) {
      // 128-bit loads down T's columns: TI/4 lanes cover one column's run
      constexpr int LPC = TI / 4, CPT = kBlock / LPC;  // lanes per column, columns per trip
      const int i4 = (t % LPC) * 4, jq = t / LPC;
      const int64_t gi = i0 + i4;
      float4 v[64 / CPT];
#pragma unroll
      for (int p = 0; p < 64 / CPT; ++p) {
        const int64_t gj = j0 + jq + CPT * p;
        v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gj < ta.C) {
          const float *src = tr + gi + gj * ta.ld;
          if (gi + 3 < ta.R) {
            v[p] = ld4_nt(src);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (gi + k < ta.R) el(v[p], k) = src[k];
          }
        }
      }
#pragma unroll
      for (int p = 0; p < 64 / CPT; ++p)
#pragma unroll
        for (int k = 0; k < 4; ++k) tile[jq + CPT * p][i4 + k] = el(v[p], k);
    } else {
      constexpr int CPT = kBlock / TI;
      const int i = t % TI, jq = t / TI;
      const int64_t gi = i0 + i;
#pragma unroll
      for (int p = 0; p < 64 / CPT; ++p) {
        const int j = jq + CPT * p;
        const int64_t gj = j0 + j;
        float v = 0.f;
        if (gi < ta.R && gj < ta.C) v = __builtin_nontemporal_load(tr + gi + gj * ta.ld);
        tile[j][i] = v;
      }
    }
    __syncthreads();
    const int m = t & 15, q = t >> 4;
    const int j = 4 * m;
    const int64_t gj = j0 + j;
    if (gj < ta.C) {
#pragma unroll
      for (int p = 0; p < TI / 16; ++p) {
        const int i = q + 16 * p;
        const int64_t gi = i0 + i;
        if (gi >= ta.R) continue;
        float4 vo;
        const int64_t ooff = gi * ta.os0 + gj * ta.os1;
        if constexpr (OMODE == SM_BCAST) {
          float s = oth[ooff];
          vo = make_float4(s, s, s, s);
        } else if constexpr (OMODE == SM_CONTIG) {
          vo = ld4(oth + ooff);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) el(vo, k) = oth[ooff + k * ta.os1];
        }
        float4 r;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float vt = tile[j + k][i];
          float x = SWAP ? el(vo, k) : vt;
          float y = SWAP ? vt : el(vo, k);
          el(r, k) = fwd32<OP, EPI>(x, y, s_gelu);
        }
        st4_nt(out + gi * ta.C + gj, r);
      }
    }
    __syncthreads();  // the tile is refilled by the next trip
  }
}

// --------------------------------------------------------------- generic
template <typename I>
__device__ __forceinline__ void offsets_ab(const Space &sp, I i, I &oa, I &ob) {
  I rest = i;
  oa = 0;
  ob = 0;
#pragma unroll
  for (int k = kMaxDims - 1; k >= 1; --k) {
    if (k < sp.rank) {
      I q;
      if constexpr (sizeof(I) == 4) q = (I)fdiv(sp.fd[k], (uint32_t)rest);
      else q = rest / (I)sp.n[k];
      I c = rest - q * (I)sp.n[k];
      oa += c * (I)sp.s[1][k];
      ob += c * (I)sp.s[2][k];
      rest = q;
    }
  }
  oa += rest * (I)sp.s[1][0];
  ob += rest * (I)sp.s[2][0];
}

// side: -1, or which operand (0 = a, 1 = b) is the host scalar sv.
template <int OP, int EPI, typename I>
__global__ __launch_bounds__(kBlock) void k_fwd_generic(const float *a,
                                                        const float *b,
                                                        float *out, Space sp,
                                                        int flat_a, int flat_b,
                                                        int vec_out, ScalarArg sa) {
  __shared__ double s_gelu[EPI == ZK_EPI_GELU ? kGeluTabLen : 1];
  if constexpr (EPI == ZK_EPI_GELU) gelu_tab_load(s_gelu);
  const I n = (I)sp.numel;
  // 64-bit loop counter: i0 + stride may pass 2^31 even when n does not
  for (int64_t j0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4; j0 < (int64_t)n;
       j0 += (int64_t)gridDim.x * kBlock * 4) {
    const I i0 = (I)j0;
    float r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      I i = i0 + k;
      if (i < n) {
        I oa, ob;
        offsets_ab<I>(sp, i, oa, ob);
        float x = sa.side == 0 ? sa.value : a[flat_a ? i : oa];
        float y = sa.side == 1 ? sa.value : b[flat_b ? i : ob];
        r[k] = fwd32<OP, EPI>(x, y, s_gelu);
      }
    }
    if (vec_out && i0 + 4 <= n) {
      st4(out + i0, make_float4(r[0], r[1], r[2], r[3]));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k < n) out[i0 + k] = r[k];
    }
  }
}

// ------------------------------------------------------ fused forward
// out = (a op1 b) op2 c, each operator one binary32 operation (Operator
// chapter, "fusion": the same math in one pass; the intermediate is never
// stored).  ROW: canonical rank <= 3, inner dim a multiple of 4; each input
// walks the output's layout (IM_FLAT), repeats the first input (IM_SAME_A),
// or is read at its decoded offset with its own inner-dim mode.
struct In3 {
  const float *p;
  int64_t s[3];  // canonical strides (rank <= 3; unused dims 0)
  int32_t mode;
};
struct Space3 {
  int32_t rank;
  int64_t n[3];
  FastDiv fd[3];
  int64_t numel;
};

template <typename I>
__device__ __forceinline__ float4 load_in3(const In3 &x, I i, I c0, I c1, I c2) {
  if (x.mode == IM_FLAT) return ld4_nt(x.p + i);
  const I off = c0 * (I)x.s[0] + c1 * (I)x.s[1] + c2 * (I)x.s[2];
  if (x.mode == IM_BCAST) {
    const float v = x.p[off];
    return make_float4(v, v, v, v);
  }
  if (x.mode == IM_CONTIG) return ld4(x.p + off);
  float4 v;
  const I si = (I)x.s[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) el(v, k) = x.p[off + (I)k * si];
  return v;
}

template <int OP1, int OP2, typename I>
__global__ __launch_bounds__(kBlock) void k_fwd2_row(In3 a, In3 b, In3 c, float *out,
                                                     Space3 sp) {
  const I n = (I)sp.numel;
  const bool dec = a.mode != IM_FLAT || b.mode != IM_FLAT ||
                   (c.mode != IM_FLAT && c.mode != IM_SAME_A);
  // 64-bit loop counter: i + stride may pass 2^31 even when n does not
  for (int64_t j = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4; j < (int64_t)n;
       j += (int64_t)gridDim.x * kBlock * 4) {
    const I i = (I)j;
    // coordinates of element i over the (up to) 3 canonical dims
    I c0 = 0, c1 = 0, c2 = i;
    if (dec && sp.rank >= 2) {
      I q;
      if constexpr (sizeof(I) == 4) q = (I)fdiv(sp.fd[sp.rank - 1], (uint32_t)i);
      else q = i / (I)sp.n[sp.rank - 1];
      c2 = i - q * (I)sp.n[sp.rank - 1];
      if (sp.rank == 3) {
        I q2;
        if constexpr (sizeof(I) == 4) q2 = (I)fdiv(sp.fd[1], (uint32_t)q);
        else q2 = q / (I)sp.n[1];
        c1 = q - q2 * (I)sp.n[1];
        c0 = q2;
      } else {
        c1 = q;
      }
    }
    // the kernel's In3 strides are aligned to (c0, c1, c2) by the launcher
    const float4 va = load_in3<I>(a, i, c0, c1, c2);
    const float4 vb = load_in3<I>(b, i, c0, c1, c2);
    const float4 vc = c.mode == IM_SAME_A ? va : load_in3<I>(c, i, c0, c1, c2);
    float4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      el(r, k) = op32<OP2>(op32<OP1>(el(va, k), el(vb, k)), el(vc, k));
    st4_nt(out + i, r);
  }
}

// Fused (a op1 b) op2 c over rows of n1 elements where a is dense, one of b
// and c is a contiguous row vector that every row shares (outer strides 0,
// n1 >= kBcRowsMinCols) and the other a scalar per row (inner stride 0):
// the attention's scores * scale[1,H,1,1] + mask[1,1,S,S].  As in
// k_fwd_bcrows, a lane applies each 16-byte piece of the shared vector to
// kBcRows rows.  Row r's scalar sits at (r / nmid) * rs0 + (r % nmid) * rs1
// (rank 3 [n0, nmid, n1]; rank 2: nmid = 1, rs1 = 0).  VB: b is the vector,
// c the scalar; else the reverse.  Two binary32 roundings per element, as
// everywhere.
struct Bc2Args {
  int64_t n1;     // row length (elements)
  int64_t total;  // (rows / kBcRows) * (n1 / 4) vectors
  uint32_t vpr;   // n1 / 4
  FastDiv fv;     // divides by vpr
  uint32_t nmid;  // middle dim of a rank-3 space (1 for rank 2)
  FastDiv fmid;   // divides by nmid
  int64_t rs0, rs1;
};

template <int OP1, int OP2, bool VB, typename I>
__global__ __launch_bounds__(kBlock) void k_fwd2_bcrows(const float *a, const float *b,
                                                        const float *c, float *out,
                                                        Bc2Args ba) {
  const I n1 = (I)ba.n1;
  const float *vec = VB ? b : c;
  const float *sca = VB ? c : b;
  for (int64_t v64 = (int64_t)blockIdx.x * kBlock + threadIdx.x; v64 < ba.total;
       v64 += (int64_t)gridDim.x * kBlock) {
    I g;
    if constexpr (sizeof(I) == 4) g = (I)fdiv(ba.fv, (uint32_t)v64);
    else g = (I)(v64 / (int64_t)ba.vpr);
    const I j = ((I)v64 - g * (I)ba.vpr) * 4;
    const I r0 = g * (I)kBcRows;
    const float4 vv = ld4(vec + j);
    // the rows one after another, as in k_fwd_bcrows
#pragma unroll
    for (int k = 0; k < kBcRows; ++k) {
      const I r = r0 + (I)k;
      const float4 x = ld4_nt(a + r * n1 + j);
      I q;
      if constexpr (sizeof(I) == 4) q = (I)fdiv(ba.fmid, (uint32_t)r);
      else q = r / (I)ba.nmid;
      const float sv = sca[q * (I)ba.rs0 + (r - q * (I)ba.nmid) * (I)ba.rs1];
      float4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        el(o, e) = VB ? op32<OP2>(op32<OP1>(el(x, e), el(vv, e)), sv)
                      : op32<OP2>(op32<OP1>(el(x, e), sv), el(vv, e));
      st4_nt(out + r * n1 + j, o);
    }
  }
}

template <int OP1, int OP2, typename I>
__global__ __launch_bounds__(kBlock) void k_fwd2_generic(const float *a, const float *b,
                                                         const float *c, float *out,
                                                         Space sp, int vec_out) {
  const I n = (I)sp.numel;
  for (int64_t j0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4; j0 < (int64_t)n;
       j0 += (int64_t)gridDim.x * kBlock * 4) {
    const I i0 = (I)j0;
    float r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const I i = i0 + k;
      if (i < n) {
        I rest = i, oa = 0, ob = 0, oc = 0;
#pragma unroll
        for (int d = kMaxDims - 1; d >= 1; --d) {
          if (d < sp.rank) {
            I q;
            if constexpr (sizeof(I) == 4) q = (I)fdiv(sp.fd[d], (uint32_t)rest);
            else q = rest / (I)sp.n[d];
            const I cd = rest - q * (I)sp.n[d];
            oa += cd * (I)sp.s[1][d];
            ob += cd * (I)sp.s[2][d];
            oc += cd * (I)sp.s[3][d];
            rest = q;
          }
        }
        oa += rest * (I)sp.s[1][0];
        ob += rest * (I)sp.s[2][0];
        oc += rest * (I)sp.s[3][0];
        r[k] = op32<OP2>(op32<OP1>(a[oa], b[ob]), c[oc]);
      }
    }
    if (vec_out && i0 + 4 <= n) {
      st4(out + i0, make_float4(r[0], r[1], r[2], r[3]));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k < n) out[i0 + k] = r[k];
    }
  }
}

// ---------------------------------------------------------- materialise
// out (dense, target shape) = in read through its strides, broadcast to the
// target (Operator chapter, "view backward": the stride-aware copy that turns
// a view into contiguous storage).  A copy: no arithmetic, bit-exact.
template <typename I>
__global__ __launch_bounds__(kBlock) void k_copy_row(In3 x, float *out, Space3 sp) {
  const I n = (I)sp.numel;
  for (int64_t j = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4; j < (int64_t)n;
       j += (int64_t)gridDim.x * kBlock * 4) {
    const I i = (I)j;
    I c0 = 0, c1 = 0, c2 = i;
    if (x.mode != IM_FLAT && sp.rank >= 2) {
      I q;
      if constexpr (sizeof(I) == 4) q = (I)fdiv(sp.fd[sp.rank - 1], (uint32_t)i);
      else q = i / (I)sp.n[sp.rank - 1];
      c2 = i - q * (I)sp.n[sp.rank - 1];
      if (sp.rank == 3) {
        I q2;
        if constexpr (sizeof(I) == 4) q2 = (I)fdiv(sp.fd[1], (uint32_t)q);
        else q2 = q / (I)sp.n[1];
        c1 = q - q2 * (I)sp.n[1];
        c0 = q2;
      } else {
        c1 = q;
      }
    }
    st4_nt(out + i, load_in3<I>(x, i, c0, c1, c2));
  }
}

// T[i, j] at i + j*ld (a transposed view) -> out[R, C] row-major, through a
// 64x64 LDS tile (the layout of k_fwd_tile without the second operand).
__global__ __launch_bounds__(kBlock) void k_copy_tile(const float *tr, float *out, TileArgs ta) {
  __shared__ float tile[64][65];
  const int t = threadIdx.x;
  for (int64_t bt = blockIdx.x; bt < ta.ntiles; bt += gridDim.x) {
    const int64_t tiles_r = ta.ntiles / ta.tiles_c;
    const int64_t tr_j = bt % ta.tiles_c;
    const int64_t tr_i = (bt / ta.tiles_c + tr_j) % tiles_r;  // diagonal order
    const int64_t i0 = tr_i * 64, j0 = tr_j * 64;
    if (ta.tv) {
      const int i4 = (t & 15) * 4, jq = t >> 4;
      const int64_t gi = i0 + i4;
      float4 v[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int64_t gj = j0 + jq + 16 * p;
        v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gj < ta.C) {
          const float *src = tr + gi + gj * ta.ld;
          if (gi + 3 < ta.R) {
            v[p] = ld4_nt(src);
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (gi + k < ta.R) el(v[p], k) = src[k];
          }
        }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int k = 0; k < 4; ++k) tile[jq + 16 * p][i4 + k] = el(v[p], k);
    } else {
      const int i = t & 63, jq = t >> 6;
      const int64_t gi = i0 + i;
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int j = jq + 4 * p;
        const int64_t gj = j0 + j;
        tile[j][i] = (gi < ta.R && gj < ta.C) ? tr[gi + gj * ta.ld] : 0.f;
      }
    }
    __syncthreads();
    const int m = t & 15, q = t >> 4;
    const int64_t gj = j0 + 4 * m;
    if (gj < ta.C) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int i = q + 16 * p;
        const int64_t gi = i0 + i;
        if (gi < ta.R) {
          float4 r;
#pragma unroll
          for (int k = 0; k < 4; ++k) el(r, k) = tile[4 * m + k][i];
          st4_nt(out + gi * ta.C + gj, r);
        }
      }
    }
    __syncthreads();  // the tile is refilled by the next trip
  }
}

template <typename I>
__global__ __launch_bounds__(kBlock) void k_copy_generic(const float *in, float *out, Space sp,
                                                         int vec_out) {
  const I n = (I)sp.numel;
  for (int64_t j0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4; j0 < (int64_t)n;
       j0 += (int64_t)gridDim.x * kBlock * 4) {
    const I i0 = (I)j0;
    float r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const I i = i0 + k;
      if (i < n) {
        I rest = i, off = 0;
#pragma unroll
        for (int d = kMaxDims - 1; d >= 1; --d) {
          if (d < sp.rank) {
            I q;
            if constexpr (sizeof(I) == 4) q = (I)fdiv(sp.fd[d], (uint32_t)rest);
            else q = rest / (I)sp.n[d];
            off += (rest - q * (I)sp.n[d]) * (I)sp.s[1][d];
            rest = q;
          }
        }
        off += rest * (I)sp.s[1][0];
        r[k] = in[off];
      }
    }
    if (vec_out && i0 + 4 <= n) {
      st4(out + i0, make_float4(r[0], r[1], r[2], r[3]));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i0 + k < n) out[i0 + k] = r[k];
    }
  }
}

// -------------------------------------------------------------- launcher
// Compute units of the current device (queried once per process).
// Compute units of the current device, looked up once per device (a relaxed
// atomic cache: concurrent first calls store the same value).  It sizes the
// resident GeLU grid only; no result depends on it.
static int cu_count() {
  constexpr int kDevCache = 64;
  static std::atomic<int> cache[kDevCache] = {};
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kDevCache) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  if (dev < kDevCache) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static inline unsigned grid_of(int64_t n, int64_t per_block) {
  const int64_t g = (n + per_block - 1) / per_block;
  return (unsigned)(g < kMaxBlocks ? g : kMaxBlocks);
}

hipError_t launch_fwd(const FwdPlan &p, zk_op op, zk_epi epi, const float *a,
                      const float *b, float *out, hipStream_t st, const ScalarArg *sa) {
  const ScalarArg no_scalar{-1, 0.f};
  const ScalarArg sarg = sa ? *sa : no_scalar;
  if (p.empty) return hipSuccess;
  const Canon &c = p.c;
  return with_op_epi(op, epi, [&](auto OPc, auto EPIc) -> hipError_t {
    constexpr int OP = decltype(OPc)::value;
    constexpr int EPI = decltype(EPIc)::value;
    ProfScope prof(p.kernel);
    switch (p.kernel) {
      case K_FWD_FLAT: {
        constexpr int U = row_unroll(EPI);
        if (p.vec == 4)
          ZK_LAUNCH(prof, (k_fwd_flat<OP, EPI, 4, U>), dim3(grid_of(c.numel, kBlock * U * 4)),
                    dim3(kBlock), 0, st, a, b, out, c.numel);
        else
          ZK_LAUNCH(prof, (k_fwd_flat<OP, EPI, 1, U>), dim3(grid_of(c.numel, kBlock * U)),
                    dim3(kBlock), 0, st, a, b, out, c.numel);
        return hipGetLastError();
      }
      case K_FWD_ROW: {
        RowArgs ra{};
        ra.rank = c.rank;
        ra.numel = c.numel;
        ra.sval = sarg.value;
        int sm = p.swap ? 1 : 2;
        for (int k = 0; k < 3; ++k) {
          ra.n[k] = k < c.rank ? c.n[k] : 1;
          ra.ss[k] = k < c.rank ? c.s[sm][k] : 0;
          ra.fd[k] = make_fastdiv(ra.n[k] < ((int64_t)1 << 31) ? (uint32_t)ra.n[k] : 1u);
        }
        const float *big = p.swap ? b : a;
        const float *small = p.swap ? a : b;
        auto go = [&](auto VECc, auto SMc, auto SWc, auto Ic) -> hipError_t {
          constexpr int VEC = decltype(VECc)::value;
          constexpr int SM = decltype(SMc)::value;
          constexpr bool SW = decltype(SWc)::value != 0;
          using I = std::conditional_t<decltype(Ic)::value != 0, int64_t, int32_t>;
          constexpr int BLK = EPI == ZK_EPI_GELU ? kRowGeluBlk : kBlock;
          int64_t blocks = grid_of(c.numel, BLK * row_unroll(EPI) * VEC);
          // a dispatch counts work-items with 32 bits
          if (blocks > kMaxBlocks * kBlock / BLK) blocks = kMaxBlocks * kBlock / BLK;
          if (EPI == ZK_EPI_GELU && kRowGeluBlocksPerCU > 0) {
            const int64_t cap = (int64_t)kRowGeluBlocksPerCU * cu_count();
            if (blocks > cap) blocks = cap;
          }
          ZK_LAUNCH(prof, (k_fwd_row<OP, EPI, VEC, SM, SW, I, BLK>), dim3((unsigned)blocks),
                    dim3(BLK), 0, st,
                    big, small, out, ra);
          return hipGetLastError();
        };
        auto go_i = [&](auto VECc, auto SMc, auto SWc) -> hipError_t {
          return p.idx64 ? go(VECc, SMc, SWc, IC<1>{}) : go(VECc, SMc, SWc, IC<0>{});
        };
        auto go_sw = [&](auto VECc, auto SMc) -> hipError_t {
          return p.swap ? go_i(VECc, SMc, IC<1>{}) : go_i(VECc, SMc, IC<0>{});
        };
        if (p.small_mode == SM_ARG)
          return p.vec == 1 ? go_sw(IC<1>{}, IC<SM_ARG>{}) : go_sw(IC<4>{}, IC<SM_ARG>{});
        if (p.vec == 1) return go_sw(IC<1>{}, IC<SM_GATHER>{});
        if constexpr (EPI != ZK_EPI_GELU) {
          // rows sharing one contiguous row vector: k_fwd_bcrows
          const int sm = p.swap ? 1 : 2;
          if (p.small_mode == SM_CONTIG && c.rank == 2 && c.s[sm][0] == 0 &&
              c.n[0] % kBcRows == 0 && c.n[1] >= kBcRowsMinCols &&
              c.n[1] / 4 < ((int64_t)1 << 31)) {
            BcRowsArgs ba{};
            ba.n1 = c.n[1];
            ba.vpr = (uint32_t)(c.n[1] / 4);
            ba.total = (c.n[0] / kBcRows) * (c.n[1] / 4);
            ba.fv = make_fastdiv(ba.vpr);
            const int64_t need = (ba.total + kBlock - 1) / kBlock;
            const unsigned grid = (unsigned)(need < kMaxBlocks ? need : kMaxBlocks);
            auto go_bc = [&](auto SWc, auto Ic) -> hipError_t {
              constexpr bool SW = decltype(SWc)::value != 0;
              using I = std::conditional_t<decltype(Ic)::value != 0, int64_t, int32_t>;
              ZK_LAUNCH(prof, (k_fwd_bcrows<OP, EPI, SW, I>), dim3(grid), dim3(kBlock), 0, st,
                        p.swap ? b : a, p.swap ? a : b, out, ba);
              return hipGetLastError();
            };
            if (p.idx64) return p.swap ? go_bc(IC<1>{}, IC<1>{}) : go_bc(IC<0>{}, IC<1>{});
            return p.swap ? go_bc(IC<1>{}, IC<0>{}) : go_bc(IC<0>{}, IC<0>{});
          }
        }
        switch (p.small_mode) {
          case SM_BCAST: return go_sw(IC<4>{}, IC<SM_BCAST>{});
          case SM_CONTIG: return go_sw(IC<4>{}, IC<SM_CONTIG>{});
          default: return go_sw(IC<4>{}, IC<SM_GATHER>{});
        }
      }
      case K_FWD_TILE: {
        int tr_op = p.swap ? 2 : 1, ot_op = p.swap ? 1 : 2;
        const float *tr = p.swap ? b : a;
        const float *ot = p.swap ? a : b;
        TileArgs ta{};
        ta.R = c.n[0];
        ta.C = c.n[1];
        ta.ld = c.s[tr_op][1];
        ta.os0 = c.s[ot_op][0];
        ta.os1 = c.s[ot_op][1];
        ta.tiles_c = (ta.C + 63) / 64;
        ta.ntiles = ((ta.R + kTileRows - 1) / kTileRows) * ta.tiles_c;
        ta.tv = ta.ld % 4 == 0 && ((uintptr_t)tr & 15u) == 0;
        unsigned grid = (unsigned)(ta.ntiles < kMaxBlocks ? ta.ntiles : kMaxBlocks);
        int om = SM_GATHER;
        if (ta.os1 == 0) om = SM_BCAST;
        else if (ta.os1 == 1 && ta.os0 % 4 == 0 && ((uintptr_t)ot & 15u) == 0) om = SM_CONTIG;
        auto go = [&](auto OMc, auto SWc) -> hipError_t {
          constexpr int OM = decltype(OMc)::value;
          constexpr bool SW = decltype(SWc)::value != 0;
          ZK_LAUNCH(prof, (k_fwd_tile<OP, EPI, OM, SW, kTileRows>), dim3(grid), dim3(kBlock),
                    0, st, tr, ot, out, ta);
          return hipGetLastError();
        };
        auto go_sw = [&](auto OMc) -> hipError_t {
          return p.swap ? go(OMc, IC<1>{}) : go(OMc, IC<0>{});
        };
        if (om == SM_BCAST) return go_sw(IC<SM_BCAST>{});
        if (om == SM_CONTIG) return go_sw(IC<SM_CONTIG>{});
        return go_sw(IC<SM_GATHER>{});
      }
      default: {
        Space sp = make_space(c);
        int fa = 1, fb = 1;
        for (int k = 0; k < c.rank; ++k) {
          if (c.s[1][k] != c.s[0][k]) fa = 0;
          if (c.s[2][k] != c.s[0][k]) fb = 0;
        }
        unsigned grid = grid_of(c.numel, kBlock * 4);
        if (p.idx64)
          ZK_LAUNCH(prof, (k_fwd_generic<OP, EPI, int64_t>), dim3(grid), dim3(kBlock), 0, st,
                    a, b, out, sp, fa, fb, p.vec == 4 ? 1 : 0, sarg);
        else
          ZK_LAUNCH(prof, (k_fwd_generic<OP, EPI, int32_t>), dim3(grid), dim3(kBlock), 0, st,
                    a, b, out, sp, fa, fb, p.vec == 4 ? 1 : 0, sarg);
        return hipGetLastError();
      }
    }
  });
}

// Calls fn(IC<op1>, IC<op2>) for op1 in add..div, op2 in add/sub.
template <typename Fn>
static hipError_t with_op2(zk_op op1, zk_op op2, Fn &&fn) {
  switch ((int)op1 * 2 + (op2 == ZK_SUB ? 1 : 0)) {
    case 0: return fn(IC<ZK_ADD>{}, IC<ZK_ADD>{});
    case 1: return fn(IC<ZK_ADD>{}, IC<ZK_SUB>{});
    case 2: return fn(IC<ZK_SUB>{}, IC<ZK_ADD>{});
    case 3: return fn(IC<ZK_SUB>{}, IC<ZK_SUB>{});
    case 4: return fn(IC<ZK_MUL>{}, IC<ZK_ADD>{});
    case 5: return fn(IC<ZK_MUL>{}, IC<ZK_SUB>{});
    case 6: return fn(IC<ZK_DIV>{}, IC<ZK_ADD>{});
    case 7: return fn(IC<ZK_DIV>{}, IC<ZK_SUB>{});
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd2(const Fwd2Plan &p, zk_op op1, zk_op op2, const float *a,
                       const float *b, const float *c, float *out, hipStream_t st) {
  if (p.empty) return hipSuccess;
  const Canon &cn = p.c;
  return with_op2(op1, op2, [&](auto O1, auto O2) -> hipError_t {
    constexpr int OP1 = decltype(O1)::value;
    constexpr int OP2 = decltype(O2)::value;
    ProfScope prof(p.kernel);
    const unsigned grid = grid_of(cn.numel, kBlock * 4);
    if (p.kernel == K_FWD2_ROW && (cn.rank == 2 || cn.rank == 3) && p.mode[0] == IM_FLAT &&
        p.mode[2] != IM_SAME_A) {
      // a shared row vector and a per-row scalar: k_fwd2_bcrows
      const int R = cn.rank;
      const int64_t n1 = cn.n[R - 1];
      auto is_vec = [&](int x) {
        for (int k = 0; k + 1 < R; ++k)
          if (cn.s[1 + x][k] != 0) return false;
        return cn.s[1 + x][R - 1] == 1;
      };
      const bool vb = is_vec(1) && cn.s[3][R - 1] == 0;
      const bool vc = is_vec(2) && cn.s[2][R - 1] == 0;
      const float *vp = vb ? b : c;
      const int64_t rows = n1 > 0 ? cn.numel / n1 : 0;
      if ((vb || vc) && n1 >= kBcRowsMinCols && n1 % 4 == 0 && n1 / 4 < ((int64_t)1 << 31) &&
          rows % kBcRows == 0 && ((uintptr_t)a & 15u) == 0 && ((uintptr_t)out & 15u) == 0 &&
          ((uintptr_t)vp & 15u) == 0 && (R == 2 || cn.n[1] < ((int64_t)1 << 31))) {
        const int so = vb ? 3 : 2;  // the per-row scalar's stride set
        Bc2Args ba{};
        ba.n1 = n1;
        ba.vpr = (uint32_t)(n1 / 4);
        ba.total = (rows / kBcRows) * (n1 / 4);
        ba.fv = make_fastdiv(ba.vpr);
        ba.nmid = R == 3 ? (uint32_t)cn.n[1] : 1u;
        ba.fmid = make_fastdiv(ba.nmid);
        ba.rs0 = cn.s[so][0];
        ba.rs1 = R == 3 ? cn.s[so][1] : 0;
        const int64_t need = (ba.total + kBlock - 1) / kBlock;
        const unsigned g2 = (unsigned)(need < kMaxBlocks ? need : kMaxBlocks);
        auto go = [&](auto VBc, auto Ic) -> hipError_t {
          constexpr bool VB = decltype(VBc)::value != 0;
          using I = std::conditional_t<decltype(Ic)::value != 0, int64_t, int32_t>;
          ZK_LAUNCH(prof, (k_fwd2_bcrows<OP1, OP2, VB, I>), dim3(g2), dim3(kBlock), 0, st, a,
                    b, c, out, ba);
          return hipGetLastError();
        };
        if (p.idx64) return vb ? go(IC<1>{}, IC<1>{}) : go(IC<0>{}, IC<1>{});
        return vb ? go(IC<1>{}, IC<0>{}) : go(IC<0>{}, IC<0>{});
      }
    }
    if (p.kernel == K_FWD2_ROW) {
      // canonical dims right-aligned onto (c0, c1, c2)
      Space3 sp{};
      sp.rank = cn.rank;
      sp.numel = cn.numel;
      for (int k = 0; k < 3; ++k) {
        sp.n[k] = k < cn.rank ? cn.n[k] : 1;
        sp.fd[k] = make_fastdiv(sp.n[k] < ((int64_t)1 << 31) ? (uint32_t)sp.n[k] : 1u);
      }
      In3 in[3];
      const float *ptr[3] = {a, b, c};
      for (int x = 0; x < 3; ++x) {
        in[x].p = ptr[x];
        in[x].mode = p.mode[x];
        for (int k = 0; k < 3; ++k) in[x].s[k] = 0;
        // rank 1: (c2); rank 2: (c1, c2); rank 3: (c0, c1, c2)
        for (int k = 0; k < cn.rank; ++k) in[x].s[3 - cn.rank + k] = cn.s[1 + x][k];
      }
      // sp.n / sp.fd are indexed by canonical dim; the kernel divides by the
      // innermost (rank-1) and, for rank 3, by dim 1.
      if (p.idx64)
        ZK_LAUNCH(prof, (k_fwd2_row<OP1, OP2, int64_t>), dim3(grid), dim3(kBlock), 0, st,
                  in[0], in[1], in[2], out, sp);
      else
        ZK_LAUNCH(prof, (k_fwd2_row<OP1, OP2, int32_t>), dim3(grid), dim3(kBlock), 0, st,
                  in[0], in[1], in[2], out, sp);
      return hipGetLastError();
    }
    Space sp = make_space(cn);
    if (p.idx64)
      ZK_LAUNCH(prof, (k_fwd2_generic<OP1, OP2, int64_t>), dim3(grid), dim3(kBlock), 0, st,
                a, b, c, out, sp, p.vec == 4 ? 1 : 0);
    else
      ZK_LAUNCH(prof, (k_fwd2_generic<OP1, OP2, int32_t>), dim3(grid), dim3(kBlock), 0, st,
                a, b, c, out, sp, p.vec == 4 ? 1 : 0);
    return hipGetLastError();
  });
}

hipError_t launch_copy(const CopyPlan &p, const float *in, float *out, hipStream_t st) {
  if (p.empty) return hipSuccess;
  const Canon &cn = p.c;
  ProfScope prof(p.kernel);
  if (p.kernel == K_COPY_TILE) {
    TileArgs ta{};
    ta.R = cn.n[0];
    ta.C = cn.n[1];
    ta.ld = cn.s[1][1];
    ta.tiles_c = (ta.C + 63) / 64;
    ta.ntiles = ((ta.R + 63) / 64) * ta.tiles_c;
    ta.tv = ta.ld % 4 == 0 && ((uintptr_t)in & 15u) == 0;
    const unsigned grid = (unsigned)(ta.ntiles < kMaxBlocks ? ta.ntiles : kMaxBlocks);
    ZK_LAUNCH(prof, k_copy_tile, dim3(grid), dim3(kBlock), 0, st, in, out, ta);
    return hipGetLastError();
  }
  const unsigned grid = grid_of(cn.numel, kBlock * 4);
  if (p.kernel == K_COPY_ROW) {
    Space3 sp{};
    sp.rank = cn.rank;
    sp.numel = cn.numel;
    for (int k = 0; k < 3; ++k) {
      sp.n[k] = k < cn.rank ? cn.n[k] : 1;
      sp.fd[k] = make_fastdiv(sp.n[k] < ((int64_t)1 << 31) ? (uint32_t)sp.n[k] : 1u);
    }
    In3 x{};
    x.p = in;
    x.mode = p.mode;
    for (int k = 0; k < cn.rank; ++k) x.s[3 - cn.rank + k] = cn.s[1][k];
    if (p.idx64)
      ZK_LAUNCH(prof, (k_copy_row<int64_t>), dim3(grid), dim3(kBlock), 0, st, x, out, sp);
    else
      ZK_LAUNCH(prof, (k_copy_row<int32_t>), dim3(grid), dim3(kBlock), 0, st, x, out, sp);
    return hipGetLastError();
  }
  Space sp = make_space(cn);
  if (p.idx64)
    ZK_LAUNCH(prof, (k_copy_generic<int64_t>), dim3(grid), dim3(kBlock), 0, st, in, out, sp,
              p.vec == 4 ? 1 : 0);
  else
    ZK_LAUNCH(prof, (k_copy_generic<int32_t>), dim3(grid), dim3(kBlock), 0, st, in, out, sp,
              p.vec == 4 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace zk
