// sv_common.h -- device helpers of libspecverify (gfx950): element access, keys, Philox, reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

// Host: whether device `dev` is a gfx950 (cached per device); `cus` receives its compute-unit count.
bool device_ok(int dev, int& cus);

constexpr int NT = 256;          // threads per workgroup (4 wave64s)
constexpr int NWAVE = NT / 64;
constexpr int MAXK = 8;          // largest number of drafts per batch row
constexpr int MAXROWS = 2 * MAXK + 1;

// ---------------------------------------------------------------------------------------------
// Element types.  A 16-byte vector holds 8 bf16 or 4 fp32 logits.
// ---------------------------------------------------------------------------------------------
struct BF16 {
  static constexpr int EPV = 8;       // elements per 16-byte vector
  static constexpr int KEYBITS = 16;  // bits of the order-preserving key
  __device__ static inline float get(const uint4& v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static inline float load1(const void* row, int x) {
    return __uint_as_float((uint32_t)((const uint16_t*)row)[x] << 16);
  }
  // the raw bits of one logit, and their value (a load whose result is only stored waits only there)
  __device__ static inline uint32_t load1_raw(const void* row, int x) { return ((const uint16_t*)row)[x]; }
  __device__ static inline float from_raw(uint32_t h) { return __uint_as_float(h << 16); }
};

struct F32 {
  static constexpr int EPV = 4;
  static constexpr int KEYBITS = 32;
  __device__ static inline float get(const uint4& v, int e) {
    return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
  }
  __device__ static inline float load1(const void* row, int x) { return ((const float*)row)[x]; }
  __device__ static inline uint32_t load1_raw(const void* row, int x) { return ((const uint32_t*)row)[x]; }
  __device__ static inline float from_raw(uint32_t h) { return __uint_as_float(h); }
};

// Order-preserving unsigned keys (larger value -> larger key; -0 and +0 share one key; key 0 never
// occurs for a bf16 value, so a threshold key of 0 can mean "keep everything").
//   fp32:  key32(f) = f >= 0 ? bits | 2^31 : ~bits                  (-0 canonicalised to +0 first)
//   bf16:  key16(h) = h | 0x8000 for h < 0x8000 (+0 -> 0x8000), (2^16 - h) mod 2^16 otherwise
//          (-0 -> 0x8000, the smallest negative -> 0x7fff, -inf 0xff80 -> 0x0080)
__device__ inline uint32_t key32(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline uint32_t key16(uint32_t h) { return (h & 0x8000u) ? ((0u - h) & 0xffffu) : (h | 0x8000u); }
__device__ inline uint32_t key16f(float f) { return key16(__float_as_uint(f) >> 16); }

// key16 of both bf16 halves of a 32-bit word at once (packed 16-bit operations).
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t key16x2(uint32_t w) {
  const s16x2 h = __builtin_bit_cast(s16x2, w);
  const uint32_t sgn = __builtin_bit_cast(uint32_t, (s16x2)(h >> (short)15));  // 0xffff in negative halves
  const uint32_t neg = __builtin_bit_cast(uint32_t, (u16x2)((u16x2)0 - __builtin_bit_cast(u16x2, w)));
  const uint32_t pos = w | 0x80008000u;
  return (neg & sgn) | (pos & ~sgn);
}
// Per-half difference a - b modulo 2^16.
__device__ inline uint32_t sub16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, (u16x2)(__builtin_bit_cast(u16x2, a) - __builtin_bit_cast(u16x2, b)));
}
// Per-half minimum.
__device__ inline uint32_t min16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

template <class E>
__device__ inline uint32_t key_of(float f) {
  return E::KEYBITS == 16 ? key16f(f) : key32(f);
}
// Value of a key (inverse of key_of); used for keys of values that occur, so never NaN.
__device__ inline float key16_value(uint32_t k) {
  const uint32_t h = (k & 0x8000u) ? (k & 0x7fffu) : ((0x10000u - k) & 0xffffu);
  return __uint_as_float(h << 16);
}
__device__ inline float key32_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
template <class E>
__device__ inline float key_value(uint32_t k) {
  return E::KEYBITS == 16 ? key16_value(k) : key32_value(k);
}

// NaN-propagating maximum (v_maximum3_f32 on gfx950): a NaN anywhere in a row reaches its maximum.
__device__ inline float nan_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// ---------------------------------------------------------------------------------------------
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  The multiplies map to v_mad_u64_u32.
// ---------------------------------------------------------------------------------------------
__device__ inline uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
    c.y = (uint32_t)p1;
    c.w = (uint32_t)p0;
    c.x = n0;
    c.z = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// a ^ b ^ k in one instruction (v_bitop3_b32, truth table 0x96), k from a scalar register.  Only for a k
// that is the same in every lane of the wave: the "s" operand takes lane 0's value.
__device__ __forceinline__ uint32_t xor3_uk(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// philox10 for a key that is uniform across the wave (the verify kernels' keys are kernel arguments).  The
// first two rounds stay plain code: counters whose words other than x are uniform keep half of those rounds
// on the scalar unit.  From the third round on every word differs per lane, and each new word's two xors
// fold into one three-input xor with the round key.
__device__ inline uint4 philox10_uk(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    uint32_t n0, n2;
    if (r < 2) {
      n0 = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
      n2 = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
    } else {
      n0 = xor3_uk((uint32_t)(p1 >> 32), c.y, k0);
      n2 = xor3_uk((uint32_t)(p0 >> 32), c.w, k1);
    }
    c.y = (uint32_t)p1;
    c.w = (uint32_t)p0;
    c.x = n0;
    c.z = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Two Philox-4x32-10 blocks under one key, rounds interleaved (two independent dependency chains).
__device__ inline void philox10x2(uint4& c0, uint4& c1, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a0 = (uint64_t)0xD2511F53u * c0.x, a1 = (uint64_t)0xD2511F53u * c1.x;
    const uint64_t b0 = (uint64_t)0xCD9E8D57u * c0.z, b1 = (uint64_t)0xCD9E8D57u * c1.z;
    const uint32_t n00 = (uint32_t)(b0 >> 32) ^ c0.y ^ k0, n01 = (uint32_t)(b1 >> 32) ^ c1.y ^ k0;
    const uint32_t n20 = (uint32_t)(a0 >> 32) ^ c0.w ^ k1, n21 = (uint32_t)(a1 >> 32) ^ c1.w ^ k1;
    c0.y = (uint32_t)b0;
    c1.y = (uint32_t)b1;
    c0.w = (uint32_t)a0;
    c1.w = (uint32_t)a1;
    c0.x = n00;
    c1.x = n01;
    c0.z = n20;
    c1.z = n21;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A workgroup barrier for LDS traffic only: this wave's LDS operations complete (lgkmcnt 0), then the
// barrier.  Unlike __syncthreads() it does not wait for global loads in flight (data prefetched for later
// work keeps streaming in across it); the signal fences keep the compiler from moving memory accesses
// across it.  Not for data handed over through global memory or LDS DMA.
__device__ __forceinline__ void lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Accept uniform: top 24 bits, exact in fp32.
__device__ inline float u24(uint32_t w) { return (float)(w >> 8) * 0x1p-24f; }

// Exponential variate of the Gumbel draw, in base-2 units: E2 = -log2(U), U = ((w>>9)+0.5) 2^-23.
// The Gumbel key ln w + G equals ln(w / E) with E = -ln U; E2 = E / ln 2 only rescales every key
// by the same factor, so argmax_x w(x) / E2(x) is the Gumbel-max draw.
__device__ inline float exp_race_E2(uint32_t w) {
  const float U = fmaf((float)(w >> 9), 0x1p-23f, 0x1p-24f);  // ((w >> 9) + 1/2) 2^-23, exact (one fma)
  return -__builtin_amdgcn_logf(U);
}

// ---------------------------------------------------------------------------------------------
// Wave / workgroup reductions and scans (fixed order: deterministic).
//
// Cross-lane moves without LDS: inside each row of 16 lanes, DPP moves -- quad permutes [1,0,3,2] and
// [2,3,0,1] (the partners lane ^ 1 and lane ^ 2), the half-row mirror (lane 7 - i within 8) and the row
// mirror (15 - i within 16); once a group's lanes hold equal partials, a mirror partner holds the same
// partial as lane ^ 4 / lane ^ 8 would.  Across the four rows, the rows' partials are read as scalars
// (lanes 0, 16, 32, 48) and combined as (r0 . r1) . (r2 . r3), the order of a butterfly.  Every lane gets
// the result.  Callers run with the whole wave active.
// ---------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov_f(float x) {
  return __uint_as_float(dpp_mov_u<CTRL>(__float_as_uint(x)));
}
__device__ __forceinline__ uint32_t row_u(uint32_t x, int r) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 16 * r); }
__device__ __forceinline__ float row_f(float x, int r) { return __uint_as_float(row_u(__float_as_uint(x), r)); }
constexpr int DPP_QX1 = 0xB1, DPP_QX2 = 0x4E, DPP_HMIRROR = 0x141, DPP_MIRROR = 0x140;

// One butterfly step inside the rows: combine with the partner of step 0..3 (x1, x2, half-row, row mirror).
#define SV_ROW_STEPS(STEP)  \
  STEP(DPP_QX1);            \
  STEP(DPP_QX2);            \
  STEP(DPP_HMIRROR);        \
  STEP(DPP_MIRROR)

__device__ inline float wave_sum(float v) {
#define SV_SUM_STEP(C) v += dpp_mov_f<C>(v)
  SV_ROW_STEPS(SV_SUM_STEP);
#undef SV_SUM_STEP
  return (row_f(v, 0) + row_f(v, 1)) + (row_f(v, 2) + row_f(v, 3));
}
__device__ inline uint32_t wave_or(uint32_t v) {
#define SV_OR_STEP(C) v |= dpp_mov_u<C>(v)
  SV_ROW_STEPS(SV_OR_STEP);
#undef SV_OR_STEP
  return (row_u(v, 0) | row_u(v, 1)) | (row_u(v, 2) | row_u(v, 3));
}
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
#define SV_SUMU_STEP(C) v += dpp_mov_u<C>(v)
  SV_ROW_STEPS(SV_SUMU_STEP);
#undef SV_SUMU_STEP
  return (row_u(v, 0) + row_u(v, 1)) + (row_u(v, 2) + row_u(v, 3));
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
#define SV_MAXU_STEP(C) v = max(v, dpp_mov_u<C>(v))
  SV_ROW_STEPS(SV_MAXU_STEP);
#undef SV_MAXU_STEP
  return max(max(row_u(v, 0), row_u(v, 1)), max(row_u(v, 2), row_u(v, 3)));
}
__device__ inline unsigned long long wave_sum_u64(unsigned long long v) {
#define SV_SUM64_STEP(C)                                                                                    \
  v += ((unsigned long long)dpp_mov_u<C>((uint32_t)(v >> 32)) << 32) | dpp_mov_u<C>((uint32_t)v)
  SV_ROW_STEPS(SV_SUM64_STEP);
#undef SV_SUM64_STEP
  auto row64 = [&](int r) { return ((unsigned long long)row_u((uint32_t)(v >> 32), r) << 32) | row_u((uint32_t)v, r); };
  return (row64(0) + row64(1)) + (row64(2) + row64(3));
}

__device__ inline float wave_nan_max(float v) {  // NaN-propagating
#define SV_NMAX_STEP(C) v = nan_max(v, dpp_mov_f<C>(v))
  SV_ROW_STEPS(SV_NMAX_STEP);
#undef SV_NMAX_STEP
  return nan_max(nan_max(row_f(v, 0), row_f(v, 1)), nan_max(row_f(v, 2), row_f(v, 3)));
}

// (max, lowest argmax) of a value; idx = INT32_MAX means "none".
__device__ inline void maxarg_combine(float& m, int& a, float m2, int a2) {
  if (m2 > m || (m2 == m && a2 < a)) {
    m = m2;
    a = a2;
  }
}
__device__ inline void wave_maxarg(float& m, int& a) {
#define SV_MAXARG_STEP(C) maxarg_combine(m, a, dpp_mov_f<C>(m), (int)dpp_mov_u<C>((uint32_t)a))
  SV_ROW_STEPS(SV_MAXARG_STEP);
#undef SV_MAXARG_STEP
  float m0 = row_f(m, 0), m2 = row_f(m, 2);
  int a0 = (int)row_u((uint32_t)a, 0), a2 = (int)row_u((uint32_t)a, 2);
  maxarg_combine(m0, a0, row_f(m, 1), (int)row_u((uint32_t)a, 1));
  maxarg_combine(m2, a2, row_f(m, 3), (int)row_u((uint32_t)a, 3));
  maxarg_combine(m0, a0, m2, a2);
  m = m0;
  a = a0;
}

// Combine two (max, sum of exp2((l - max) c)) pairs.
__device__ inline void lse_combine(float& m, float& s, float m2, float s2, float c) {
  if (m2 > m) {
    s = s2 + (m == -INFINITY ? 0.0f : s * fexp2((m - m2) * c));
    m = m2;
  } else if (m2 != -INFINITY) {
    s = s + s2 * fexp2((m2 - m) * c);
  }
}

// Inclusive scans in lane order: DPP row shifts by 1, 2, 4 and 8 lanes (lanes without a source add 0), then
// row 15's and row 31's totals broadcast into the rows above them.
template <int CTRL, int ROWM>
__device__ __forceinline__ uint32_t dpp_or0_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWM, 0xF, false);
}
#define SV_SCAN_STEPS(STEP) \
  STEP(0x111, 0xF);         \
  STEP(0x112, 0xF);         \
  STEP(0x114, 0xF);         \
  STEP(0x118, 0xF);         \
  STEP(0x142, 0xA);         \
  STEP(0x143, 0xC)
__device__ inline uint32_t wave_incl_scan_u32(uint32_t v) {
#define SV_SCAN32_STEP(C, R) v += dpp_or0_u<C, R>(v)
  SV_SCAN_STEPS(SV_SCAN32_STEP);
#undef SV_SCAN32_STEP
  return v;
}
__device__ inline unsigned long long wave_incl_scan_u64(unsigned long long v) {
#define SV_SCAN64_STEP(C, R) \
  v += ((unsigned long long)dpp_or0_u<C, R>((uint32_t)(v >> 32)) << 32) | dpp_or0_u<C, R>((uint32_t)v)
  SV_SCAN_STEPS(SV_SCAN64_STEP);
#undef SV_SCAN64_STEP
  return v;
}
__device__ inline double wave_incl_scan_f64(double v) {
#define SV_SCANF64_STEP(C, R)                                                                                \
  {                                                                                                          \
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);                                \
    v += __longlong_as_double((long long)(((unsigned long long)dpp_or0_u<C, R>((uint32_t)(b >> 32)) << 32) | \
                                          dpp_or0_u<C, R>((uint32_t)b)));                                    \
  }
  SV_SCAN_STEPS(SV_SCANF64_STEP);
#undef SV_SCANF64_STEP
  return v;
}
__device__ inline uint32_t wave_incl_scan(uint32_t v) { return wave_incl_scan_u32(v); }
__device__ inline unsigned long long wave_incl_scan(unsigned long long v) { return wave_incl_scan_u64(v); }
__device__ inline double wave_incl_scan(double v) { return wave_incl_scan_f64(v); }

// Lowest lane whose predicate holds (64 if none).
__device__ inline int first_lane(bool pred) {
  const unsigned long long m = __ballot(pred);
  return m ? __ffsll((long long)m) - 1 : 64;
}

// Inclusive scan over the workgroup in thread order (NT threads), 32-bit and 64-bit.
template <class T>
__device__ inline T block_inclusive_scan(T v, T* lds_tmp /* >= NWAVE */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  if (lane == 63) lds_tmp[wave] = v;
  __syncthreads();
  T add = 0;
  for (int w = 0; w < wave; ++w) add += lds_tmp[w];
  __syncthreads();
  return v + add;
}

}  // namespace sv
