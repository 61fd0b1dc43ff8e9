// Wave-level tile engine shared by the forward, dQ and dK/dV kernels.
//
// A workgroup owns 128 "lane-side" rows (4 waves x 32; queries in the forward and dQ
// kernels, keys in the dK/dV kernel) and streams 64-row "other-side" tiles through LDS.
// Every 32x32x16 MFMA accumulator then has one lane-side row per lane (lane % 32) and
// other-side rows in its registers: register r of block b holds other-side row
// 32 b + 8 (r / 4) + 4 (lane / 32) + r % 4.
//
// Offset-aware tiling (abstract, item 1; zicq.com explainer, section on offset-aware
// tiling): a 32 x 64 wave tile touches only 95 offsets, so the table rows of those offsets
// are staged once per workgroup tile in LDS (a 192-row window shared by the 4 waves) and
// the relation products are computed once per offset (abstract, item 2; explainer, section
// on reusing query/key relation products) on MFMA as a [96 offsets x 32 rows] block.  The
// products are skew-gathered back into the score layout through a wave-private LDS buffer.
#pragma once

#include "relpos_device.h"

namespace relpos {

constexpr int NWAVE = 4;
constexpr int WROWS = 32;            // lane-side rows per wave
constexpr int BLANE = NWAVE * WROWS; // lane-side rows per workgroup
constexpr int BOTH = 64;             // other-side rows per step
constexpr int TSTR = 72;             // LDS row stride (elements) of 64-wide bf16 tiles
constexpr int WIN = 192;             // window rows (BLANE + BOTH - 1 = 191, padded)
constexpr int GS2 = 68;              // skew buffer row stride (floats): 64 offsets + pad

// A per-window-row fp32 value (T-XL v.r) kept in the 16-byte padding of the window's rows:
// window rows 4 q .. 4 q + 3 store theirs in the padding of row q.
__device__ __forceinline__ float* win_vec(uint16_t* win, int x) {
  return (float*)(win + (x >> 2) * TSTR + kHeadDim) + (x & 3);
}
// Where the values of window rows pb + 4 kh .. + 3 start (pb % 8 == 0, the same in every lane);
// rows pb + 8 q + 4 kh follow 2 q padded rows further on.
__device__ __forceinline__ const uint16_t* win_vec4_base(const uint16_t* win, int pb, int kh) {
  return win + ((pb >> 2) + kh) * TSTR + kHeadDim;
}

// ---------------------------------------------------------------------------------------
// Staging (all 256 threads).  Tiles hold NP bf16 planes of [rows][TSTR].
// ---------------------------------------------------------------------------------------
// base + e elements.  By default the offset is taken in 32 bits (e < 2^32 / sizeof(T)), so the
// address is the wave-uniform base in scalar registers plus one 32-bit vector register.  A
// translation unit that defines RELPOS_STAGE_ADDR64 keeps 64-bit per-lane addresses: the T-XL
// key-side pass, at its 256-register limit, is allocated better that way (measured).
template <typename T>
__device__ __forceinline__ const T* stage_addr(const T* base, int64_t e) {
#ifdef RELPOS_STAGE_ADDR64
  return base + e;
#else
  return (const T*)((const char*)base + (uint32_t)e * (uint32_t)sizeof(T));
#endif
}

// 64 consecutive rows of a [*, 64] tensor; rows >= nvalid are zero.
template <typename T, int NP>
__device__ __forceinline__ void stage64(uint16_t* tile, const T* base, int row0, int nvalid) {
  const int t = threadIdx.x;
  const int r = t >> 2;
  const int c = (t & 3) * 16;
  const int plane = BOTH * TSTR;
  if constexpr (NP == 1) {
    // bf16: the read without a branch (rows past nvalid read row nvalid - 1 and store zeros)
    const u32x4* g = (const u32x4*)stage_addr(base, (int64_t)min(row0 + r, nvalid - 1) * kHeadDim + c);
    const u32x4 v0 = g[0], v1 = g[1], z = {0u, 0u, 0u, 0u};
    const bool ok = row0 + r < nvalid;
    *(u32x4*)(tile + r * TSTR + c) = ok ? v0 : z;
    *(u32x4*)(tile + r * TSTR + c + 8) = ok ? v1 : z;
    return;
  }
  if (row0 + r < nvalid) {
    const T* g = stage_addr(base, (int64_t)(row0 + r) * kHeadDim + c);
    lds_store8<T>(tile, plane, r * TSTR + c, g);
    lds_store8<T>(tile, plane, r * TSTR + c + 8, g + 8);
  } else {
    lds_zero8<NP>(tile, plane, r * TSTR + c);
    lds_zero8<NP>(tile, plane, r * TSTR + c + 8);
  }
}

// Register prefetch of a 64-row tile: this thread's 16 elements (row t / 4, columns
// 16 (t % 4) ..).  load() issues the global reads early; store() writes them to LDS later.
template <typename T>
struct TilePrefetch {
  static constexpr int NCH = sizeof(T) == 2 ? 2 : 4;   // 16-byte chunks per thread
  u32x4 v[NCH];
  // Rows at or past nvalid (>= 1) repeat row nvalid - 1 instead of reading zeros: the attention
  // kernels mask every pair of such a row (its scores are -inf, its weights and dS exactly 0),
  // and a finite row times a zero weight adds nothing.  Loading unconditionally keeps the
  // registers free of a zero-fill branch.
  __device__ __forceinline__ void load(const T* base, int row0, int nvalid) {
    const int t = threadIdx.x;
    const int row = min(row0 + (t >> 2), nvalid - 1), c = (t & 3) * 16;
    const u32x4* g = (const u32x4*)stage_addr(base, (int64_t)row * kHeadDim + c);
#pragma unroll
    for (int i = 0; i < NCH; ++i) v[i] = g[i];
  }
  // rows row0 .. row0 + 63 of base, zero outside [lo, hi)
  __device__ __forceinline__ void load_range(const T* base, int row0, int lo, int hi) {
    const int t = threadIdx.x;
    const int r = t >> 2, c = (t & 3) * 16;
    if (row0 + r >= lo && row0 + r < hi) {
      const u32x4* g = (const u32x4*)stage_addr(base, (int64_t)(row0 + r) * kHeadDim + c);
#pragma unroll
      for (int i = 0; i < NCH; ++i) v[i] = g[i];
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* tile) const { store_at(tile, BOTH * TSTR, 0); }
  // into rows p0 .. p0 + 63 of a tile of NP planes `plane` elements apart
  __device__ __forceinline__ void store_at(uint16_t* tile, int plane, int p0) const {
    const int t = threadIdx.x;
    const int e = (p0 + (t >> 2)) * TSTR + (t & 3) * 16;
    if constexpr (NCH == 2) {
      *(u32x4*)(tile + e) = v[0];
      *(u32x4*)(tile + e + 8) = v[1];
    } else {
      // fp32: split into (hi, lo) bf16 planes
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // elements are copied out by value first: a bit cast of a vector-element lvalue
          // reads the vector's first element whatever the index
          const u32x4 ch = v[2 * half + i / 2];
          const uint32_t u0 = ch[2 * (i % 2)], u1 = ch[2 * (i % 2) + 1];
          const float x0 = __uint_as_float(u0), x1 = __uint_as_float(u1);
          uint16_t h0, l0, h1, l1;
          split_bf16(x0, h0, l0);
          split_bf16(x1, h1, l1);
          h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        *(u32x4*)(tile + e + 8 * half) = h;
        *(u32x4*)(tile + plane + e + 8 * half) = l;
      }
    }
  }
};

// WIN window rows; window row x reads table row rowfn(x) (< 0 = zero row).
template <typename T, int NP, typename F>
__device__ __forceinline__ void stage_window(uint16_t* win, const T* table, F rowfn) {
  const int t = threadIdx.x;
  const int c = (t & 3) * 16;
  const int plane = WIN * TSTR;
  if constexpr (NP == 1) {
    // bf16: every read first, without branches (a missing row reads row 0 and stores zeros),
    // so that the three row groups cost one round trip
    u32x4 v[3][2];
    bool ok[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int row = rowfn(64 * i + (t >> 2));
      ok[i] = row >= 0;
      const u32x4* g = (const u32x4*)stage_addr(table, (int64_t)max(row, 0) * kHeadDim + c);
      v[i][0] = g[0];
      v[i][1] = g[1];
    }
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int x = 64 * i + (t >> 2);
      *(u32x4*)(win + x * TSTR + c) = ok[i] ? v[i][0] : z;
      *(u32x4*)(win + x * TSTR + c + 8) = ok[i] ? v[i][1] : z;
    }
    return;
  }
#pragma unroll
  for (int x0 = 0; x0 < WIN; x0 += 64) {
    const int x = x0 + (t >> 2);
    const int row = rowfn(x);
    if (row >= 0) {
      const T* g = stage_addr(table, (int64_t)row * kHeadDim + c);
      lds_store8<T>(win, plane, x * TSTR + c, g);
      lds_store8<T>(win, plane, x * TSTR + c + 8, g + 8);
    } else {
      lds_zero8<NP>(win, plane, x * TSTR + c);
      lds_zero8<NP>(win, plane, x * TSTR + c + 8);
    }
  }
}

// Window rows x0 .. x0 + 63 into physical rows p0 .. p0 + 63 (a circular window's new rows);
// window row x reads table row rowfn(x) (< 0 = zero row).
template <typename T, int NP, typename F>
__device__ __forceinline__ void stage_window_rows(uint16_t* win, const T* table, F rowfn, int x0,
                                                  int p0) {
  const int t = threadIdx.x;
  const int c = (t & 3) * 16;
  const int plane = WIN * TSTR;
  const int row = rowfn(x0 + (t >> 2));
  const int e = (p0 + (t >> 2)) * TSTR + c;
  if (row >= 0) {
    const T* g = stage_addr(table, (int64_t)row * kHeadDim + c);
    lds_store8<T>(win, plane, e, g);
    lds_store8<T>(win, plane, e + 8, g + 8);
  } else {
    lds_zero8<NP>(win, plane, e);
    lds_zero8<NP>(win, plane, e + 8);
  }
}

// ---------------------------------------------------------------------------------------
// Wave products.  `lane` operands: Op<NP> x[4] for the wave's 32 lane-side rows (lane % 32
// = row, k = d chunk c: 16 c + 8 (lane / 32) .. + 7).
// ---------------------------------------------------------------------------------------
// acc[b] = Y[32 b + m] . X[n]  (C[m = other row][n = lane row]); Y is a 64-row LDS tile.
// With INIT the accumulator starts from vec[other row] (a per-other-row additive term) and
// the MFMA adds the products to it.
template <int NP, bool INIT = false>
__device__ __forceinline__ void other_dot_lane(f32x16 acc[2], const uint16_t* ytile,
                                               const Op<NP> xop[4], Op<NP> yop[2][4],
                                               const float* vec = nullptr) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    acc[b] = f32x16{};
    if constexpr (INIT) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = *(const f32x4*)(vec + 32 * b + 8 * q4 + 4 * kh);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[b][4 * q4 + i] = v4[i];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      yop[b][c] = op_from_lds<NP>(ytile, BOTH * TSTR, (32 * b + l32) * TSTR + 16 * c + 8 * kh);
      mma<NP>(acc[b], yop[b][c], xop[c]);
    }
  }
}

// The same product with the accumulators starting from an LDS vector indexed by the lane-side
// window t = n - y + 63 + w0 (a per-offset additive term, added before the products).
template <int NP>
__device__ __forceinline__ void other_dot_lane_offset(f32x16 acc[2], const uint16_t* ytile,
                                                      const Op<NP> xop[4], Op<NP> yop[2][4],
                                                      const float* vec, int w0) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int y = 32 * b + 8 * (r >> 2) + 4 * kh + (r & 3);
      acc[b][r] = vec[w0 + l32 - y + 63];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      yop[b][c] = op_from_lds<NP>(ytile, BOTH * TSTR, (32 * b + l32) * TSTR + 16 * c + 8 * kh);
      mma<NP>(acc[b], yop[b][c], xop[c]);
    }
  }
}

// The same product with every accumulator starting from one per-lane value (a lane-row term).
template <int NP>
__device__ __forceinline__ void other_dot_lane_from(f32x16 acc[2], const uint16_t* ytile,
                                                    const Op<NP> xop[4], Op<NP> yop[2][4],
                                                    float init) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[b][r] = init;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      yop[b][c] = op_from_lds<NP>(ytile, BOTH * TSTR, (32 * b + l32) * TSTR + 16 * c + 8 * kh);
      mma<NP>(acc[b], yop[b][c], xop[c]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Skew through a wave-private LDS buffer of 32 rows x 64 offsets: the 96-offset product
// block of a wave is written 64 columns at a time and read back along the diagonals.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void put_block(float* gs, const f32x16& g, int bb, int tbase) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int t = 32 * bb + 8 * q4 + 4 * kh - tbase;
    f32x4 v = {g[4 * q4], g[4 * q4 + 1], g[4 * q4 + 2], g[4 * q4 + 3]};
    *(f32x4*)(gs + l32 * GS2 + t) = v;
  }
}

// Physical row of window row x in a circular window rotated by xrot (a multiple of 64).
__device__ __forceinline__ int wrow(int x, int xrot) {
  const int p = x + xrot;
  return p >= WIN ? p - WIN : p;
}
// Physical row of the first row of an aligned block of 16 or 32 window rows (x0 a multiple of
// the block size, the same in every lane).  Such a block never wraps, since the rotation is a
// multiple of 64, so its rows stay consecutive and the wrap is decided once, on the scalar unit.
__device__ __forceinline__ int wrow_block(int x0, int xrot) {
  return __builtin_amdgcn_readfirstlane(wrow(x0, xrot));
}

// Row side, all three 32-offset blocks of products in registers (optionally + the per-row
// value kept in the window's padding, win_vec).  With ROT the window is circular: row x
// sits at physical row wrow(x, xrot).
template <int NP, bool ADDVEC, bool ROT = false>
__device__ __forceinline__ void row_products(f32x16 g[3], const uint16_t* win, int w0,
                                             const Op<NP> xop[4], int xrot = 0) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int bb = 0; bb < 3; ++bb) {
    g[bb] = f32x16{};
    const int pb = ROT ? wrow_block(w0 + 32 * bb, xrot) : w0 + 32 * bb;   // w0 % 32 == 0
    if constexpr (ADDVEC) {   // the MFMA accumulates on top of the per-row value
      const uint16_t* vb = win_vec4_base(win, pb, kh);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = *(const f32x4*)(vb + 2 * q4 * TSTR);
#pragma unroll
        for (int i = 0; i < 4; ++i) g[bb][4 * q4 + i] = v4[i];
      }
    }
    const int prow = pb + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      Op<NP> aop = op_from_lds<NP>(win, WIN * TSTR, prow * TSTR + 16 * c + 8 * kh);
      mma<NP>(g[bb], aop, xop[c]);
    }
  }
}

// s[b][r] += G[n][n - y + 63]: block b = 0 needs offsets 32..94, block 1 needs 0..62.
__device__ __forceinline__ void row_skew_add(f32x16 s[2], const f32x16 g[3], float* gs) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
  wave_lds_sync();
  put_block(gs, g[1], 1, 32);
  put_block(gs, g[2], 2, 32);
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int y = 8 * (r >> 2) + 4 * kh + (r & 3);
    s[0][r] += gs[l32 * GS2 + l32 - y + 63 - 32];
  }
  wave_lds_sync();
  put_block(gs, g[0], 0, 0);
  put_block(gs, g[1], 1, 0);
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int y = 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    s[1][r] += gs[l32 * GS2 + l32 - y + 63];
  }
}

// Column side for other block ob: products Win[w0 + t'] . Y[32 ob + n] for t' in
// [32 ob, 32 ob + 64), then s[ob][r] += H[y - 32 ob][y - n + 31].  With ROT the window is
// circular (row x at physical row wrow(x, xrot)).
// The other-side operands are re-read from the streamed tile (fewer live registers).
template <int NP, bool ADDVEC, bool ROT = false>
__device__ __forceinline__ void col_skew_add(f32x16 s[2], const uint16_t* win, int w0, int ob,
                                             const uint16_t* ytile, float* gs, int xrot = 0) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
  f32x16 h[2];
  int prow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int bb = ob + i;
    h[i] = f32x16{};
    const int pb = ROT ? wrow_block(w0 + 32 * bb, xrot) : w0 + 32 * bb;   // w0 % 32 == 0
    if constexpr (ADDVEC) {   // the MFMA accumulates on top of the per-row value
      // (addressed row by row: with win_vec4_base the T-XL key-side pass, at its register
      // limit, is scheduled worse; measured)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int x = pb + 8 * q4 + 4 * kh;
        const f32x4 v4 = *(const f32x4*)(win + (x >> 2) * TSTR + kHeadDim);
#pragma unroll
        for (int j = 0; j < 4; ++j) h[i][4 * q4 + j] = v4[j];
      }
    }
    prow[i] = pb + l32;
  }
  // (chunk-outer: each streamed-row operand is read once for both blocks; each block still
  // takes its chunks in ascending order)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    Op<NP> yop = op_from_lds<NP>(ytile, BOTH * TSTR, (32 * ob + l32) * TSTR + 16 * c + 8 * kh);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      Op<NP> aop = op_from_lds<NP>(win, WIN * TSTR, prow[i] * TSTR + 16 * c + 8 * kh);
      mma<NP>(h[i], aop, yop);
    }
  }
  wave_lds_sync();
  put_block(gs, h[0], ob, 32 * ob);
  put_block(gs, h[1], ob + 1, 32 * ob);
  wave_lds_sync();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int yy = 8 * (r >> 2) + 4 * kh + (r & 3);
    const int y = 32 * ob + yy;
    s[ob][r] += gs[yy * GS2 + y - l32 + 31 - 32 * ob];
  }
}

// Element-wise addition of an LDS vector indexed by the lane-side window t = n - y + 63 + w0.
__device__ __forceinline__ void add_offset_vec(f32x16 s[2], const float* vec, int w0) {
  const int lane = __lane_id();
  const int l32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int y = 32 * b + 8 * (r >> 2) + 4 * kh + (r & 3);
      s[b][r] += vec[w0 + l32 - y + 63];
    }
}

// Operand whose k index runs down 16 consecutive rows of an LDS tile (row-major, TSTR):
// 32x32x16 A/B layout with m/n = column col0 + (lane % 32) and k = rows row0 + (8 i + 4 kh
// + j) as the P / dS register permutation expects (slot j < 4: row0 + 4 kh + j, slot
// 4 + j: row0 + 8 + 4 kh + j).
template <int NP>
__device__ __forceinline__ Op<NP> op_rows_tr(const uint16_t* tile, int plane, int stride,
                                             int row0, int col0) {
  const int lane = __lane_id();
  const int g = lane >> 4, i = lane & 15;
  const int kh = g >> 1;
  const int col = col0 + 16 * (g & 1) + 4 * (i & 3);
  const int r = row0 + 4 * kh + (i >> 2);
  return op_tr_from_lds<NP>(tile, plane, r * stride + col, (r + 8) * stride + col);
}

// op_rows_tr over a circular window rotated by xrot (row0 a multiple of 16, the same in every
// lane: the 16 rows read form one block that does not wrap).
template <int NP>
__device__ __forceinline__ Op<NP> op_rows_tr_rot(const uint16_t* tile, int plane, int stride,
                                                 int row0, int col0, int xrot) {
  return op_rows_tr<NP>(tile, plane, stride, wrow_block(row0, xrot), col0);
}

// Operand from an fp32 register block in accumulator layout: 16 consecutive other-side
// rows 16 c .. 16 c + 15 of s[c / 2].
template <int NP>
__device__ __forceinline__ Op<NP> op_from_acc(const f32x16 s[2], int c) {
  float x[8];
  const f32x16& v = s[c >> 1];
  const int base = 8 * (c & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = v[base + i];
  return op_from_f32<NP>(x);
}

}  // namespace relpos
