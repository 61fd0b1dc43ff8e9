// Device-side building blocks shared by the gfx950 kernels: MFMA operand types, LDS
// access helpers (including the CDNA4 transpose read), wave-level exchanges and the index
// maps of the four relative-position mechanisms.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "relpos_kernels.h"

namespace relpos {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------------------
// bf16 conversions: the CDNA4 packed converter (v_cvt_pk_bf16_f32, round to nearest even)
// ---------------------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f2bf_bits(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xFFFFu);
}
__device__ __forceinline__ float bf_bits2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Split x into hi + lo with both parts bf16 (the three-product fp32 emulation).
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf_bits(x);
  lo = f2bf_bits(x - bf_bits2f(hi));
}

// ---------------------------------------------------------------------------------------
// MFMA operands.  NP = 1: plain bf16.  NP = 2: (hi, lo) bf16 planes of an fp32 value; the
// product hi*hi + hi*lo + lo*hi carries about 16 significant bits per factor.
// ---------------------------------------------------------------------------------------
template <int NP>
struct Op {
  bf16x8 p[NP];
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int NP>
__device__ __forceinline__ void mma(f32x16& acc, const Op<NP>& a, const Op<NP>& b) {
  acc = mfma32(a.p[0], b.p[0], acc);
  if constexpr (NP == 2) {
    acc = mfma32(a.p[0], b.p[1], acc);
    acc = mfma32(a.p[1], b.p[0], acc);
  }
}

__device__ __forceinline__ bf16x8 u4_to_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Build an operand from 8 fp32 values (k-order 0..7).
template <int NP>
__device__ __forceinline__ Op<NP> op_from_f32(const float* x) {
  Op<NP> o;
  if constexpr (NP == 1) {
    u32x4 v;
    v[0] = pack_bf16x2(x[0], x[1]);
    v[1] = pack_bf16x2(x[2], x[3]);
    v[2] = pack_bf16x2(x[4], x[5]);
    v[3] = pack_bf16x2(x[6], x[7]);
    o.p[0] = u4_to_bf8(v);
  } else {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t h0, l0, h1, l1;
      split_bf16(x[2 * i], h0, l0);
      split_bf16(x[2 * i + 1], h1, l1);
      h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    o.p[0] = u4_to_bf8(h);
    o.p[1] = u4_to_bf8(l);
  }
  return o;
}

// ---------------------------------------------------------------------------------------
// Global element access.  Tensors are bf16 (uint16_t bits) or fp32.
// ---------------------------------------------------------------------------------------
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int NP = 1;
  __device__ static __forceinline__ float to_f(uint16_t v) { return bf_bits2f(v); }
};
template <> struct Elem<float> {
  static constexpr int NP = 2;
  __device__ static __forceinline__ float to_f(float v) { return v; }
};

// Load 8 consecutive elements starting at p (16 B aligned for bf16, 32 B for fp32) as floats.
__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
  u32x4 v = *(const u32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __builtin_bit_cast(float, v[i] << 16);
    x[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  f32x4 a = *(const f32x4*)p;
  f32x4 b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}

// Operand straight from global memory (8 consecutive k elements).
template <typename T>
__device__ __forceinline__ Op<Elem<T>::NP> op_from_global(const T* p) {
  if constexpr (Elem<T>::NP == 1) {
    Op<1> o;
    o.p[0] = u4_to_bf8(*(const u32x4*)p);
    return o;
  } else {
    float x[8];
    load8(p, x);
    return op_from_f32<2>(x);
  }
}

// ---------------------------------------------------------------------------------------
// LDS tiles: NP planes of bf16, row-major with a padded row stride (in elements).
// ---------------------------------------------------------------------------------------
// Store 8 consecutive elements (from global, any T) into NP planes at element offset e.
template <typename T>
__device__ __forceinline__ void lds_store8(uint16_t* planes, int plane_elems, int e, const T* g) {
  if constexpr (Elem<T>::NP == 1) {
    *(u32x4*)(planes + e) = *(const u32x4*)g;
  } else {
    float x[8];
    load8(g, x);
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t h0, l0, h1, l1;
      split_bf16(x[2 * i], h0, l0);
      split_bf16(x[2 * i + 1], h1, l1);
      h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    *(u32x4*)(planes + e) = h;
    *(u32x4*)(planes + plane_elems + e) = l;
  }
}
template <int NP>
__device__ __forceinline__ void lds_zero8(uint16_t* planes, int plane_elems, int e) {
  u32x4 z = {0u, 0u, 0u, 0u};
  *(u32x4*)(planes + e) = z;
  if constexpr (NP == 2) *(u32x4*)(planes + plane_elems + e) = z;
}

// Operand read: 8 consecutive elements at element offset e.
template <int NP>
__device__ __forceinline__ Op<NP> op_from_lds(const uint16_t* planes, int plane_elems, int e) {
  Op<NP> o;
  o.p[0] = u4_to_bf8(*(const u32x4*)(planes + e));
  if constexpr (NP == 2) o.p[1] = u4_to_bf8(*(const u32x4*)(planes + plane_elems + e));
  return o;
}

// CDNA4 transpose read.  Within each group of 16 lanes, lane s points at 4 consecutive bf16;
// output lane i receives, in slot t, element (i % 4) of the 4 values lane (4 t + i / 4) of
// its group pointed at.  If source lane s of a group points at row (r0 + s / 4), columns
// c0 + 4 (s % 4) .. +3 of a row-major tile, output lane i receives column c0 + i at rows
// r0 .. r0 + 3: a 4 x 16 block read transposed.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  typedef LDS_AS s16x4 lds_s16x4;
  const lds_s16x4* lp = (const lds_s16x4*)(const LDS_AS uint16_t*)p;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lp);
}

// Operand whose k index runs down the rows of a row-major tile (stride in elements):
// lane l gets column col0 + (l % 32) ... for the 32x32x16 layout the caller passes, per
// lane, the element offset of row (krow0 + (l % 16) / 4) and column (c0 + 4 (l % 4)) for the
// first four k values and krow0 + 4 rows further for... see the call sites.
template <int NP>
__device__ __forceinline__ Op<NP> op_tr_from_lds(const uint16_t* planes, int plane_elems, int e0,
                                                 int e1) {
  Op<NP> o;
#pragma unroll
  for (int pl = 0; pl < NP; ++pl) {
    s16x4 a = lds_read_tr16(planes + pl * plane_elems + e0);
    s16x4 b = lds_read_tr16(planes + pl * plane_elems + e1);
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    s16x8 c;
    c[0] = a[0]; c[1] = a[1]; c[2] = a[2]; c[3] = a[3];
    c[4] = b[0]; c[5] = b[1]; c[6] = b[2]; c[7] = b[3];
    o.p[pl] = __builtin_bit_cast(bf16x8, c);
  }
  return o;
}

// ---------------------------------------------------------------------------------------
// Wave exchanges
// ---------------------------------------------------------------------------------------
// Value of the same lane in the other half-wave (lane ^ 32).
__device__ __forceinline__ float xhalf(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  // lanes 0..31 receive the upper half in r[1]; lanes 32..63 receive the lower half in r[0]
  uint32_t other = (__lane_id() < 32) ? r[1] : r[0];
  return __builtin_bit_cast(float, other);
}

// Order LDS traffic between lanes of one wave (wave-private buffers need no s_barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------
// Index maps (bit-exact; offsets delta = i - j)
// ---------------------------------------------------------------------------------------
// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value: every
// per-wave decision derived from it is then taken on the scalar unit.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// A wave-uniform pointer rebuilt from scalar registers where it is used (an opaque pair of
// SGPRs), so that the compiler does not keep it in, and spill it from, vector registers.
typedef __attribute__((address_space(1))) const char gchar;   // global memory
__device__ __forceinline__ gchar* scalar_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  int hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  asm volatile("" : "+s"(lo), "+s"(hi));
  return (gchar*)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ float load_f32(gchar* base, uint32_t byte_off) {
  return *(const __attribute__((address_space(1))) float*)(base + byte_off);
}

// max(a, b, c) as one v_maximum3_f32 (NaN-propagating; no canonicalisation of the inputs)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Sum of the 8 bf16 values of an operand register group, accumulated in fp32 on the dot unit.
__device__ __forceinline__ float sum_bf16x8(const bf16x8& v, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t word = u[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, word), one, acc, false);
  }
  return acc;
}

// Workgroups are dispatched round-robin over the chip's 8 XCDs (hardware id % 8), each with
// its own L2.  Renumbering so that every XCD runs one contiguous range of logical workgroups
// puts the blocks of one (batch, head) on the same L2, where they share K / V and table rows.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int hw_id, int nwg) {
  const int xcd = hw_id % kNumXcd, slot = hw_id / kNumXcd;
  const int per = nwg / kNumXcd, rem = nwg % kNumXcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// T5 bucket of offset delta = i - j, from the integer thresholds the host computed.
__device__ __forceinline__ int t5_bucket_dev(int delta, const T5Map& m) {
  int n = delta;
  int ret = 0;
  if (m.bidirectional) {
    if (n < 0) { ret = m.half; n = -n; }
  } else {
    n = n < 0 ? 0 : n;
  }
  if (n < m.max_exact) return ret + n;
  int t = 0;
#pragma unroll 1
  for (int e = 0; e < m.nthr; ++e) t += (n >= m.thr[e]) ? 1 : 0;
  return ret + m.max_exact + t;
}

// Table row of offset delta for the row-side table (Shaw w, T-XL r, DeBERTa Kr).  Returns -1
// when T-XL's table has no such row.
__device__ __forceinline__ int row_side_row(int mech, int delta, int span, int nrel, int txl_off) {
  if (mech == MECH_SHAW) return clampi(-delta, -span, span) + span;
  if (mech == MECH_DEBERTA) return clampi(delta + span, 0, 2 * span - 1);
  int r = delta + txl_off;
  return (r >= 0 && r < nrel) ? r : -1;
}
// DeBERTa p2c row of offset delta = i - j: clamp(j - i + k, 0, 2k - 1).
__device__ __forceinline__ int p2c_row(int delta, int span) { return clampi(-delta + span, 0, 2 * span - 1); }

__device__ __forceinline__ bool pair_allowed(int i, int j, int wl, int wr) {
  return (wl < 0 || i - j <= wl) && (wr < 0 || j - i <= wr);
}
// The same test without branches, for per-element use: wlx / wrx are the window bounds with
// "unbounded" (< 0) replaced by L, and rows / columns at or beyond L are excluded.
__device__ __forceinline__ bool pair_ok(int i, int j, int L, int wlx, int wrx) {
  return (i < L) & (j < L) & (i - j <= wlx) & (j - i <= wrx);
}

}  // namespace relpos
