// specverify.hip -- libspecverify: the speculative-decoding verify sampler for gfx950 (MI355X), and its
// C ABI (include/specverify.h).
//
// Method: AReno pull request "feat(engine): MTP training loss and speculative decoding for bailing_v3",
// section "What does this PR do?" (Phase 2: sampler-equivalent target distribution, exact chain
// rejection sampling, unchanged logprobs), its accept-probability table (alpha = sum min(p, q)), and
// its per-step optimisation table (Gumbel-max draws, no host synchronisation).
//
// One call enqueues three kernels on the caller's stream; no workgroup ever waits for another.  A
// merge across workgroups is done by the last one to arrive at a per-row counter (agent-scope
// atomics; partials travel through agent-scope atomic stores and loads, coherent across the XCDs'
// L2s without cache-wide write-back or invalidation).
//
//   K1 stats   grid (slices, logit rows).  Streams every logit once (16-byte loads): slice max,
//              lowest argmax, sum of exp2((l - max) * log2(e) / T), NaN/+inf flags; for rows with
//              top-k / top-p (bf16) also a count histogram of the 512 order-preserving codes below the
//              slice max and a 128-bin histogram of log2 value (counts, and masses relative to each
//              bin's top).  The last slice of a row merges: row max / argmax / normaliser, and the
//              exact kept threshold when it lies among the row's top 512 codes (per-code counts merged
//              exactly, masses = count x 2^40 fixed-point exp2 of the code's value: integer sums).
//              Otherwise it picks, from the merged log2-value histogram, a window of codes that must
//              hold the threshold.
//   K3 fine    grid (slices, logit rows), only rows with a pending window: exact per-code counts in
//              the window and the exact fixed-point mass above it; the last slice merges and sets the
//              threshold.  Rows this cannot settle (fp32 keys, a window too wide, a threshold outside
//              the window) take an exact whole-row MSD radix select instead.
//   K5 verify  grid (slices, batch rows).  Every slice evaluates the accept chain (p_i(x_i), q_i(x_i)
//              from the row statistics and two gathered logits, Philox accept uniforms), then re-reads
//              its slice of the draft-position rows: alpha partial sums for every position and the
//              Gumbel-max race candidate at the first rejected position (residual max(p - q, 0)) or at
//              position k (bonus from p_k).  The last slice of a batch row writes the outputs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "specverify.h"
#include "sv_common.h"

namespace sv {

constexpr int MODE_VERIFY = 0;
constexpr int MODE_SAMPLE = 1;  // plain sampler: k = 0, one logit row per batch row, stream tag 2
constexpr int MAXDEV = 64;
constexpr int VPT1 = 8;         // K1: 16-byte vectors per thread per slice
constexpr int VPT3 = 8;         // K3
constexpr int VPT5 = 4;         // K5
constexpr int WTOP = 512;       // K1: per-code window below the slice max
constexpr int NB = 128;         // K1: log2-value bins (2 per log2 unit)
constexpr float BR = 2.0f;      // bins per log2 unit
constexpr int WF = 2048;        // K3: widest per-code window

// RowInfo.state bits
constexpr uint32_t ST_BAD = 1u;      // NaN / +inf entries, or every entry -inf
constexpr uint32_t ST_FINE = 2u;     // threshold pending: fine pass over [clo, chi]
constexpr uint32_t ST_RADIX = 4u;    // threshold pending: whole-row radix select

struct StatPart {  // K1, per (logit row, slice)
  float m;         // slice max
  int32_t arg;     // lowest index of the slice max (INT_MAX if none)
  float s;         // sum of exp2((l - m) * c) over the slice
  uint32_t flags;  // bit 0: NaN or +inf seen
};

struct RowInfo {    // per logit row
  float m;          // row max
  int32_t arg;      // lowest argmax
  float Z;          // normaliser of the kept set: sum of exp2((l - m) * c) over kept entries
  uint32_t thr;     // smallest kept order-preserving key (0: everything kept)
  uint32_t state;   // ST_* bits
  uint32_t clo, chi;  // K3 window of keys [clo, chi]
  float Ztot;       // normaliser of the whole row
};

struct FinePart {  // K3, per (logit row, slice): count and fixed-point mass of the entries above chi
  unsigned long long above_mass;
  uint32_t above_cnt;
  uint32_t pad;
};

struct FinalPart {  // K5, per (batch row, slice)
  float alpha[MAXK];
  float key;        // best Gumbel race key w / E2 (0 = no candidate)
  int32_t idx;      // its vocabulary index (INT_MAX = none)
  uint32_t pad[2];
};

struct Params {
  const uint8_t* target;
  const uint8_t* draft;
  const int32_t* draft_tokens;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t B, k, V, rows, R;  // rows = 2k + 1 logit rows per batch row, R = B * rows
  int32_t S1, S3, S5, L1, L3, L5;
  int32_t mode;              // MODE_VERIFY or MODE_SAMPLE
  const int32_t* row_b;      // plain sampler: stream coordinate b of each row (NULL = row index)
  const int32_t* row_pos;    // plain sampler: stream coordinate i of each row (NULL = 0)
  uint32_t key0, key1, offset;
  int32_t* tokens;
  int32_t* accept_len;
  float* logprobs;
  float* alpha;
  uint32_t* cnt1;     // [R] K1 arrivals
  uint32_t* cnt3;     // [R] K3 arrivals
  uint32_t* cnt5;     // [B] K5 arrivals
  StatPart* st1;      // [R][S1]
  uint32_t* hw1;      // [R][S1][WTOP/2] packed 16-bit code counts
  uint32_t* hb1;      // [R][S1][NB/2 + NB + 1] packed 16-bit bin counts, bin masses, slice base bin
  RowInfo* rinfo;     // [R]
  FinePart* fp3;      // [R][S3]
  uint32_t* fc3;      // [R][S3][WF/2] packed 16-bit code counts
  FinalPart* fin5;    // [B][S5]
  unsigned long long* trace;  // K1 phase timestamps per (row, slice), instrumented builds only
};

// Phase timestamps of instrumented builds (compiled with -DSV_TRACE); no-ops otherwise.
#ifdef SV_TRACE
constexpr int TRACE_SLOTS = 8;
#define SV_TRACE_AT(idx, slot)                                                   \
  do {                                                                           \
    if (threadIdx.x == 0 && p.trace) p.trace[(size_t)(idx)*TRACE_SLOTS + (slot)] = wall_clock64(); \
  } while (0)
#else
constexpr int TRACE_SLOTS = 0;
#define SV_TRACE_AT(idx, slot) \
  do {                         \
  } while (0)
#endif

// ---- small helpers ------------------------------------------------------------------------------
__device__ inline const uint8_t* row_ptr(const Params& p, int b, int r, int esize) {
  const size_t V = (size_t)p.V;
  if (r <= p.k) return p.target + ((size_t)b * (p.k + 1) + r) * V * esize;
  return p.draft + ((size_t)b * p.k + (r - p.k - 1)) * V * esize;
}

__device__ inline unsigned long long fixmass(float e) {  // e in [0, 1] -> 2^40 fixed point
  return __float2ull_rn(e * 0x1p40f);
}

// bf16 value of a 16-bit order-preserving key (inverse of key32(f) >> 16)
__device__ inline float key16_value(uint32_t k16) {
  const uint32_t k32 = k16 << 16;
  const uint32_t u = (k32 & 0x80000000u) ? (k32 & 0x7fffffffu) : ~k32;
  return __uint_as_float(u & 0xffff0000u);
}

__device__ inline void st32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st64(void* p, unsigned long long v) {
  __hip_atomic_store((unsigned long long*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void stf(void* p, float v) { st32(p, __float_as_uint(v)); }
__device__ inline uint32_t ld32(const void* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned long long ld64(const void* p) {
  return __hip_atomic_load((const unsigned long long*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ldf(const void* p) { return __uint_as_float(ld32(p)); }
// Wait until this thread's outstanding memory operations (stores and atomics included) are done.
__device__ inline void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Arrive at a counter after this workgroup's partials are written; true in the last arriving one.
__device__ inline bool arrive_last(uint32_t* counter, uint32_t total, int* flag) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0) *flag = (atomicAdd(counter, 1u) == total - 1) ? 1 : 0;
  __syncthreads();
  return *flag != 0;
}

// Sampling parameters of a batch row.
struct RowParams {
  float T, P, c;
  int K;
  bool ok, greedy, trunc;
};
__device__ inline RowParams row_params(const Params& p, int b) {
  RowParams q;
  q.T = p.temperature[b];
  q.K = p.top_k[b];
  q.P = p.top_p[b];
  q.ok = !(__builtin_isnan(q.T) || __builtin_isinf(q.T) || q.T < 0.0f) && q.K >= 0 &&
         !(__builtin_isnan(q.P) || q.P <= 0.0f);
  q.greedy = q.T == 0.0f;
  q.c = q.greedy ? 0.0f : 1.4426950408889634f / q.T;
  q.trunc = q.ok && !q.greedy && ((q.K > 0 && q.K < p.V) || q.P < 1.0f);
  return q;
}

// Wave butterfly of (max, lowest argmax, sum of exp2((l - max) c), flags).
__device__ inline void wave_stats(float& m, int& a, float& s, uint32_t& fl, float c) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64);
    const int a2 = __shfl_xor(a, o, 64);
    const float s2 = __shfl_xor(s, o, 64);
    const uint32_t f2 = __shfl_xor(fl, o, 64);
    float mm = m, ss = s;
    lse_combine(mm, ss, m2, s2, c);
    maxarg_combine(m, a, m2, a2);
    s = ss;
    fl |= f2;
  }
}

struct RedSmem {
  float f[NWAVE], g[NWAVE];
  int32_t i[NWAVE];
  uint32_t u[NWAVE];
  unsigned long long scan64[NWAVE];
  uint32_t scan32[NWAVE];
  int32_t flag;
};

// Workgroup (max, argmax, sum, flags) into every thread.
__device__ void block_stats(RedSmem& rs, float& m, int& a, float& s, uint32_t& fl, float c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_stats(m, a, s, fl, c);
  if (lane == 0) {
    rs.f[wave] = m;
    rs.i[wave] = a;
    rs.g[wave] = s;
    rs.u[wave] = fl;
  }
  __syncthreads();
  m = rs.f[0];
  a = rs.i[0];
  s = rs.g[0];
  fl = rs.u[0];
  for (int w = 1; w < NWAVE; ++w) {
    float mm = m, ss = s;
    lse_combine(mm, ss, rs.f[w], rs.g[w], c);
    maxarg_combine(m, a, rs.f[w], rs.i[w]);
    s = ss;
    fl |= rs.u[w];
  }
  __syncthreads();
}

__device__ float block_max(RedSmem& rs, float m) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) rs.f[wave] = m;
  __syncthreads();
  m = rs.f[0];
  for (int w = 1; w < NWAVE; ++w) m = fmaxf(m, rs.f[w]);
  __syncthreads();
  return m;
}

__device__ void block_maxarg(RedSmem& rs, float& m, int& a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_maxarg(m, a);
  if (lane == 0) {
    rs.f[wave] = m;
    rs.i[wave] = a;
  }
  __syncthreads();
  m = rs.f[0];
  a = rs.i[0];
  for (int w = 1; w < NWAVE; ++w) maxarg_combine(m, a, rs.f[w], rs.i[w]);
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// Exact kept threshold of one whole row (top-k, then top-p on the top-k mass), by one workgroup.
// MSD radix select over order-preserving keys, 8-bit digits; per-digit LDS histograms of counts
// and of 2^40 fixed-point masses exp2((l - m) * c) (integer sums: order independent, deterministic).
// ---------------------------------------------------------------------------------------------
struct RadixSmem {
  uint32_t hcnt[256];
  unsigned long long hmass[256];
  uint32_t sel, sel_excl;
  unsigned long long sel_mexcl, sel_m;
};

template <class E>
__device__ void row_cutoff(RadixSmem& sm, RedSmem& rs, const uint8_t* row, int V, float m, float c, int K, float P,
                           uint32_t& thr_out, float& Z_out) {
  const int tid = threadIdx.x;
  const int nvec = V / E::EPV;
  const uint4* src = (const uint4*)row;
  constexpr int LEVELS = E::KEYBITS / 8;
  uint32_t thr = 0;
  unsigned long long zk = 0;
  bool have_zk = false;

  if (K > 0 && K < V) {
    uint32_t prefix = 0, need = (uint32_t)K;
    unsigned long long mabove = 0;
    for (int lev = 0; lev < LEVELS; ++lev) {
      const int shift = E::KEYBITS - 8 * (lev + 1);
      sm.hcnt[tid] = 0;
      sm.hmass[tid] = 0;
      __syncthreads();
      for (int j = tid; j < nvec; j += NT) {
        const uint4 v = src[j];
#pragma unroll
        for (int e = 0; e < E::EPV; ++e) {
          const float f = E::get(v, e);
          const uint32_t key = key_of<E>(f);
          if (lev == 0 || (key >> (shift + 8)) == prefix) {
            const uint32_t d = (key >> shift) & 255u;
            atomicAdd(&sm.hcnt[d], 1u);
            atomicAdd(&sm.hmass[d], fixmass(fexp2((f - m) * c)));
          }
        }
      }
      __syncthreads();
      const int d = 255 - tid;  // thread t scans bins in descending key order
      const uint32_t cnt = sm.hcnt[d];
      const unsigned long long ms = sm.hmass[d];
      const uint32_t incl = block_inclusive_scan<uint32_t>(cnt, rs.scan32);
      const unsigned long long minc = block_inclusive_scan<unsigned long long>(ms, rs.scan64);
      const uint32_t excl = incl - cnt;
      if (excl < need && need <= incl) {
        sm.sel = (uint32_t)d;
        sm.sel_excl = excl;
        sm.sel_mexcl = minc - ms;
        sm.sel_m = ms;
      }
      __syncthreads();
      need -= sm.sel_excl;
      mabove += sm.sel_mexcl;
      prefix = (prefix << 8) | sm.sel;
      if (lev == LEVELS - 1) zk = mabove + sm.sel_m;
      __syncthreads();
    }
    thr = prefix;
    have_zk = true;
  }

  if (P < 1.0f) {
    uint32_t prefix = 0;
    unsigned long long mabove = 0;
    double target = 0.0;
    for (int lev = 0; lev < LEVELS; ++lev) {
      const int shift = E::KEYBITS - 8 * (lev + 1);
      sm.hmass[tid] = 0;
      __syncthreads();
      for (int j = tid; j < nvec; j += NT) {
        const uint4 v = src[j];
#pragma unroll
        for (int e = 0; e < E::EPV; ++e) {
          const float f = E::get(v, e);
          const uint32_t key = key_of<E>(f);
          if (key >= thr && (lev == 0 || (key >> (shift + 8)) == prefix))
            atomicAdd(&sm.hmass[(key >> shift) & 255u], fixmass(fexp2((f - m) * c)));
        }
      }
      __syncthreads();
      const int d = 255 - tid;
      const unsigned long long ms = sm.hmass[d];
      const unsigned long long minc = block_inclusive_scan<unsigned long long>(ms, rs.scan64);
      if (lev == 0) {
        if (!have_zk) {
          if (tid == NT - 1) sm.sel_m = minc;  // total kept mass
          __syncthreads();
          zk = sm.sel_m;
          __syncthreads();
        }
        target = (double)P * (double)zk;
      }
      const unsigned long long mexcl = minc - ms;
      if ((double)(mabove + minc) >= target && (double)(mabove + mexcl) < target) {
        sm.sel = (uint32_t)d;
        sm.sel_mexcl = mexcl;
        sm.sel_m = ms;
      }
      __syncthreads();
      mabove += sm.sel_mexcl;
      prefix = (prefix << 8) | sm.sel;
      if (lev == LEVELS - 1) zk = mabove + sm.sel_m;
      __syncthreads();
    }
    thr = prefix;
  }
  thr_out = thr;
  Z_out = (float)((double)zk * 0x1p-40);
}

// ---------------------------------------------------------------------------------------------
// Threshold search over a descending run of per-code (count, mass) entries, 2 per thread:
// the first entry where the running count reaches K (top-k) and, within the kept prefix, the first
// where the running mass reaches P * Z_K (top-p).  Entries are indexed 0..n-1 from the top.
// ---------------------------------------------------------------------------------------------
struct SelState {
  int32_t sel_k, sel_p;
  unsigned long long zk, zp;
};

// cnt/mass[0..n) hold the entries (LDS); base_cnt / base_mass are the totals above entry 0; ztot_fixed is
// the whole row's mass (used when top-k is off).  Returns false if a threshold lies beyond the run.
__device__ bool select_run(const uint32_t* cnt, const unsigned long long* mass, SelState& ss, RedSmem& rs, int n,
                           uint32_t base_cnt, unsigned long long base_mass, double ztot_fixed, int K, float P, int V,
                           int& sel, unsigned long long& zsel) {
  const int tid = threadIdx.x;
  const bool useK = K > 0 && K < V;
  const bool useP = P < 1.0f;
  if (tid == 0) {
    ss.sel_k = -1;
    ss.sel_p = -1;
  }
  __syncthreads();
  unsigned long long zk = 0;
  int selk = -1;
  // chunks of 2 * NT entries, thread t owns entries 2t and 2t+1 of a chunk
  uint32_t ccarry = base_cnt;
  unsigned long long mcarry = base_mass;
  if (useK) {
    for (int c0 = 0; c0 < n; c0 += 2 * NT) {
      const int i0 = c0 + 2 * tid, i1 = i0 + 1;
      const uint32_t a0 = i0 < n ? cnt[i0] : 0u, a1 = i1 < n ? cnt[i1] : 0u;
      const unsigned long long b0 = i0 < n ? mass[i0] : 0ull, b1 = i1 < n ? mass[i1] : 0ull;
      const uint32_t ic = block_inclusive_scan<uint32_t>(a0 + a1, rs.scan32) + ccarry;
      const unsigned long long im = block_inclusive_scan<unsigned long long>(b0 + b1, rs.scan64) + mcarry;
      const uint32_t e0 = ic - a0 - a1;
      const unsigned long long f0 = im - b0 - b1;
      if (i0 < n && e0 < (uint32_t)K && e0 + a0 >= (uint32_t)K) {
        ss.sel_k = i0;
        ss.zk = f0 + b0;
      } else if (i1 < n && e0 + a0 < (uint32_t)K && ic >= (uint32_t)K) {
        ss.sel_k = i1;
        ss.zk = im;
      }
      if (tid == NT - 1) {
        rs.u[0] = ic;
        rs.scan64[0] = im;
      }
      __syncthreads();
      ccarry = rs.u[0];
      mcarry = rs.scan64[0];
      const int sk = ss.sel_k;
      __syncthreads();
      if (sk >= 0) break;
    }
    selk = ss.sel_k;
    if (selk < 0) return false;
    zk = ss.zk;
  }
  const double target = (double)P * (useK ? (double)zk : ztot_fixed);
  int selp = -1;
  unsigned long long zp = useK ? zk : 0ull;
  if (useP) {
    const int last = useK ? selk : n - 1;
    mcarry = base_mass;
    for (int c0 = 0; c0 <= last; c0 += 2 * NT) {
      const int i0 = c0 + 2 * tid, i1 = i0 + 1;
      const unsigned long long b0 = i0 <= last ? mass[i0] : 0ull, b1 = i1 <= last ? mass[i1] : 0ull;
      const unsigned long long im = block_inclusive_scan<unsigned long long>(b0 + b1, rs.scan64) + mcarry;
      const unsigned long long f0 = im - b0 - b1;
      if (i0 <= last && (double)f0 < target && (double)(f0 + b0) >= target) {
        ss.sel_p = i0;
        ss.zp = f0 + b0;
      } else if (i1 <= last && (double)(f0 + b0) < target && (double)im >= target) {
        ss.sel_p = i1;
        ss.zp = im;
      }
      if (tid == NT - 1) rs.scan64[0] = im;
      __syncthreads();
      mcarry = rs.scan64[0];
      const int sp = ss.sel_p;
      __syncthreads();
      if (sp >= 0) break;
    }
    selp = ss.sel_p;
    if (selp < 0) return false;
    zp = ss.zp;
  }
  sel = useP ? selp : selk;
  zsel = zp;
  return true;
}

// ---------------------------------------------------------------------------------------------
// K1: row statistics (every logit read once), merged by the last slice of each row.
// ---------------------------------------------------------------------------------------------
struct K1Smem {
  RedSmem rs;
  uint32_t hw[WTOP];   // per-code counts below the slice max
  uint32_t hbc[NB];    // log2-value bin counts
  float hbm[NB];       // bin masses relative to each bin's top
  uint4 st[64];        // staged slice statistics (merge), chunks of 64 slices
  uint32_t keyms[64];  // slice max keys (merge; bf16 rows have at most 64 slices)
  uint32_t scnt[WTOP];
  unsigned long long smass[WTOP];
  SelState ss;
  float bm[NB];        // merged bin masses relative to the row max
  uint32_t bc[NB];     // merged bin counts
  uint32_t win[4];
};

template <class E>
__device__ void k1_merge(const Params& p, K1Smem& sm, int r, const RowParams& q) {
  constexpr bool BF = E::KEYBITS == 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.S1;
  RowInfo* ri = p.rinfo + r;
  // row statistics: slice partials combined in slice order by wave 0
  float m = -INFINITY, sum = 0.0f;
  int a = INT_MAX;
  uint32_t fl = 0;
  for (int s0 = 0; s0 < S; s0 += 64) {
    if (tid < 64 && s0 + tid < S) {
      const StatPart* sp = p.st1 + (size_t)r * S + s0 + tid;
      sm.st[tid] = make_uint4(ld32(&sp->m), ld32(&sp->arg), ld32(&sp->s), ld32(&sp->flags));
      if (s0 == 0) sm.keyms[tid] = key32(__uint_as_float(sm.st[tid].x)) >> 16;
    }
    __syncthreads();
    if (wave == 0 && s0 + lane < S) {
      const uint4 v = sm.st[lane];
      float mm = m, ss = sum;
      lse_combine(mm, ss, __uint_as_float(v.x), __uint_as_float(v.z), q.c);
      maxarg_combine(m, a, __uint_as_float(v.x), (int)v.y);
      sum = ss;
      fl |= v.w;
    }
    __syncthreads();
  }
  if (wave == 0) wave_stats(m, a, sum, fl, q.c);
  if (tid == 0) {
    sm.rs.f[0] = m;
    sm.rs.i[0] = a;
    sm.rs.g[0] = sum;
    sm.rs.u[0] = fl;
  }
  __syncthreads();
  m = sm.rs.f[0];
  a = sm.rs.i[0];
  sum = sm.rs.g[0];
  fl = sm.rs.u[0];
  __syncthreads();
  const bool bad = fl != 0 || m == -INFINITY;
  uint32_t state = bad ? ST_BAD : 0u, thr = 0, clo = 0, chi = 0;
  float Zk = sum;
  if (!bad && q.trunc && !BF) state |= ST_RADIX;
  if (!bad && q.trunc && BF) {
    const uint32_t keym = key32(m) >> 16;
    // merged per-code counts of the row's top WTOP codes (exact: every slice's window reaches them)
    for (int co = tid; co < WTOP; co += NT) {
      uint32_t cnt = 0;
      for (int s = 0; s < S; ++s) {
        const int d = co - (int)(keym - sm.keyms[s]);
        if (d >= 0 && d < WTOP) {
          const uint32_t w = ld32(&p.hw1[((size_t)r * S + s) * (WTOP / 2) + (d >> 1)]);
          cnt += (d & 1) ? (w >> 16) : (w & 0xffffu);
        }
      }
      sm.scnt[co] = cnt;
      const float e = (cnt != 0 && (uint32_t)co <= keym) ? fexp2((key16_value(keym - (uint32_t)co) - m) * q.c) : 0.0f;
      sm.smass[co] = (unsigned long long)cnt * fixmass(e);
    }
    __syncthreads();
    int sel = -1;
    unsigned long long zsel = 0;
    const double ztot = (double)sum * 0x1p40;
    if (select_run(sm.scnt, sm.smass, sm.ss, sm.rs, WTOP, 0u, 0ull, ztot, q.K, q.P, p.V, sel, zsel)) {
      thr = keym - (uint32_t)sel;
      Zk = (float)((double)zsel * 0x1p-40);
    } else {
      // The threshold lies below the top codes: merge the log2-value bins and pick a key window.
      const float base_row = floorf(-m * q.c * BR);
      for (int j = tid; j < NB; j += NT) {
        sm.bc[j] = 0;
        sm.bm[j] = 0.0f;
      }
      __syncthreads();
      if (wave == 0) {
        for (int s = 0; s < S; ++s) {
          const uint32_t* hb = p.hb1 + ((size_t)r * S + s) * (NB / 2 + NB + 1);
          const float base_s = ldf(&hb[NB / 2 + NB]);
          for (int j = lane; j < NB; j += 64) {
            const float jrf = base_s + (float)j - base_row;  // row-relative bin
            if (jrf >= 0.0f && jrf < (float)NB) {
              const int jr = (int)jrf;
              const uint32_t w = ld32(&hb[j >> 1]);
              const uint32_t cnt = (j & 1) ? (w >> 16) : (w & 0xffffu);
              const float ms = ldf(&hb[NB / 2 + j]);
              sm.bc[jr] += cnt;
              // masses relative to the bin top 2^(-(base_s + j) / BR) -> relative to the row max
              sm.bm[jr] += ms * fexp2(-(base_s + (float)j) / BR - m * q.c);
            }
          }
        }
      }
      __syncthreads();
      if (tid == 0) {
        const bool useK = q.K > 0 && q.K < p.V;
        const bool useP = q.P < 1.0f;
        int jk = NB - 1, jlo, jhi;
        double zk_lo = 0.0, zk_hi = 0.0, ztot_est = 0.0;
        for (int j = 0; j < NB; ++j) ztot_est += sm.bm[j];
        if (useK) {
          uint32_t cc = 0;
          double mm = 0.0;
          for (int j = 0; j < NB; ++j) {
            if (cc + sm.bc[j] >= (uint32_t)q.K) {
              jk = j;
              zk_lo = mm;
              zk_hi = mm + sm.bm[j];
              break;
            }
            cc += sm.bc[j];
            mm += sm.bm[j];
          }
        }
        if (useP) {
          const double tlo = (double)q.P * (useK ? zk_lo : ztot_est), thi = (double)q.P * (useK ? zk_hi : ztot_est);
          double mm = 0.0;
          int plo = NB - 1, phi = NB - 1;
          bool got = false;
          for (int j = 0; j < NB; ++j) {
            mm += sm.bm[j];
            if (!got && mm >= tlo * 0.999) {
              plo = j;
              got = true;
            }
            if (mm >= thi * 1.001 || j == NB - 1) {
              phi = j;
              break;
            }
          }
          jlo = plo;
          jhi = useK ? jk : phi;
        } else {
          jlo = jk;
          jhi = jk;
        }
        // widen by two bins either side against bin-edge rounding and the estimated masses
        jlo = max(jlo - 2, 0);
        jhi = min(jhi + 2, NB - 1);
        // keys of the window: bins hold -l * c * BR in [base_row + j, base_row + j + 1)
        const float vhi = -(base_row + (float)jlo) / (BR * q.c);
        const float vlo = -(base_row + (float)(jhi + 1)) / (BR * q.c);
        uint32_t khi = key32(vhi) >> 16, klo = key32(vlo) >> 16;
        khi = min(khi + 2u, keym);
        klo = klo > 2u ? klo - 2u : 0u;
        if (jhi >= NB - 1 || khi < klo || khi - klo + 1 > (uint32_t)WF) {
          sm.win[0] = ST_RADIX;
        } else {
          sm.win[0] = ST_FINE;
          sm.win[1] = klo;
          sm.win[2] = khi;
        }
      }
      __syncthreads();
      state |= sm.win[0];
      clo = sm.win[1];
      chi = sm.win[2];
    }
  }
  if (tid == 0) {
    stf(&ri->m, m);
    st32(&ri->arg, (uint32_t)a);
    stf(&ri->Z, Zk);
    st32(&ri->thr, thr);
    st32(&ri->state, state);
    st32(&ri->clo, clo);
    st32(&ri->chi, chi);
    stf(&ri->Ztot, sum);
    atomicExch(&p.cnt1[r], 0u);
  }
}

template <class E, int VPT>
__global__ __launch_bounds__(NT) void k1_stats(Params p) {
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  constexpr bool BF = E::KEYBITS == 16;
  __shared__ K1Smem sm;
  const int tid = threadIdx.x;
  const int r = blockIdx.x / p.S1, s = blockIdx.x - r * p.S1;
  const int b = r / p.rows, i = r - b * p.rows;
  const RowParams q = row_params(p, b);
  const int x0 = s * p.L1;
  const int x1 = min(x0 + p.L1, p.V);
  const int nv = x0 < x1 ? (x1 - x0) / EPV : 0;
  const uint4* src = (const uint4*)(row_ptr(p, b, i, esize) + (size_t)x0 * esize);
  SV_TRACE_AT(blockIdx.x, 0);

  uint4 v[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j < nv) v[u] = src[j];
  }
  float m = -INFINITY, sum = 0.0f;
  int a = INT_MAX;
  uint32_t fl = 0;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j < nv) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float f = E::get(v[u], e);
        fl |= (__builtin_isnan(f) || f == INFINITY) ? 1u : 0u;
        if (f > m) {
          m = f;
          a = x0 + j * EPV + e;
        }
      }
    }
  }
  const bool hist = BF && q.trunc;
  float base_s = 0.0f;
  if (hist) {
    // histograms are relative to the slice max
    const float ms = block_max(sm.rs, m);
    for (int j = tid; j < WTOP; j += NT) sm.hw[j] = 0;
    for (int j = tid; j < NB; j += NT) {
      sm.hbc[j] = 0;
      sm.hbm[j] = 0.0f;
    }
    __syncthreads();
    if (ms != -INFINITY) {
      const uint32_t keyms = key32(ms) >> 16;
      base_s = floorf(-ms * q.c * BR);
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float f = E::get(v[u], e);
            if (f == -INFINITY) continue;
            sum += fexp2((f - ms) * q.c);
            const uint32_t d = keyms - key_of<E>(f);
            if (d < (uint32_t)WTOP) atomicAdd(&sm.hw[d], 1u);
            const float ta = f * q.c;
            const float bin = floorf(-ta * BR);
            const float jb = bin - base_s;
            if (jb >= 0.0f && jb < (float)NB) {
              atomicAdd(&sm.hbc[(int)jb], 1u);
              atomicAdd(&sm.hbm[(int)jb], fexp2(ta + bin / BR));
            }
          }
        }
      }
    }
    m = ms;  // the sums above are relative to the slice max
  } else if (!q.greedy && m != -INFINITY) {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int j = tid + u * NT;
      if (j < nv) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) sum += fexp2((E::get(v[u], e) - m) * q.c);
      }
    }
  }
  SV_TRACE_AT(blockIdx.x, 1);
  block_stats(sm.rs, m, a, sum, fl, q.c);
  StatPart* sp = p.st1 + (size_t)r * p.S1 + s;
  if (tid == 0) {
    stf(&sp->m, m);
    st32(&sp->arg, (uint32_t)a);
    stf(&sp->s, sum);
    st32(&sp->flags, fl);
  }
  if (hist) {
    uint32_t* hw = p.hw1 + ((size_t)r * p.S1 + s) * (WTOP / 2);
    for (int j = tid; j < WTOP / 2; j += NT) st32(&hw[j], sm.hw[2 * j] | (sm.hw[2 * j + 1] << 16));
    uint32_t* hb = p.hb1 + ((size_t)r * p.S1 + s) * (NB / 2 + NB + 1);
    for (int j = tid; j < NB / 2; j += NT) st32(&hb[j], sm.hbc[2 * j] | (sm.hbc[2 * j + 1] << 16));
    for (int j = tid; j < NB; j += NT) stf(&hb[NB / 2 + j], sm.hbm[j]);
    if (tid == 0) stf(&hb[NB / 2 + NB], base_s);
  }
  SV_TRACE_AT(blockIdx.x, 2);
  if (arrive_last(&p.cnt1[r], (uint32_t)p.S1, &sm.rs.flag)) {
    SV_TRACE_AT(blockIdx.x, 3);
    k1_merge<E>(p, sm, r, q);
    SV_TRACE_AT(blockIdx.x, 4);
  }
}

// ---------------------------------------------------------------------------------------------
// K3: exact per-code window (rows whose threshold lies below the top codes), or the radix select.
// ---------------------------------------------------------------------------------------------
struct K3Smem {
  RedSmem rs;
  uint32_t h[WF];
  uint32_t scnt[WF];
  unsigned long long smass[WF];
  SelState ss;
  RadixSmem rad;
  uint32_t state, clo, chi;
  float m, Ztot;
};

template <class E, int VPT>
__global__ __launch_bounds__(NT) void k3_fine(Params p) {
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  __shared__ K3Smem sm;
  const int tid = threadIdx.x;
  const int r = blockIdx.x / p.S3, s = blockIdx.x - r * p.S3;
  RowInfo* ri = p.rinfo + r;
  if (tid == 0) {
    sm.state = ri->state;
    sm.clo = ri->clo;
    sm.chi = ri->chi;
    sm.m = ri->m;
    sm.Ztot = ri->Ztot;
  }
  __syncthreads();
  const uint32_t state = sm.state;
  if (state & ST_BAD) return;
  if (!(state & (ST_FINE | ST_RADIX))) return;
  const int b = r / p.rows, i = r - b * p.rows;
  const RowParams q = row_params(p, b);
  const float m = sm.m;
  const uint8_t* row = row_ptr(p, b, i, esize);
  if (state & ST_RADIX) {
    if (s != 0) return;
    uint32_t thr;
    float Z;
    row_cutoff<E>(sm.rad, sm.rs, row, p.V, m, q.c, q.K, q.P, thr, Z);
    if (tid == 0) {
      ri->thr = thr;
      ri->Z = Z;
      ri->state = state & ~ST_RADIX;
    }
    return;
  }
  const uint32_t clo = sm.clo, chi = sm.chi;
  const int width = (int)(chi - clo + 1);
  for (int j = tid; j < width; j += NT) sm.h[j] = 0;
  __syncthreads();
  const int x0 = s * p.L3;
  const int x1 = min(x0 + p.L3, p.V);
  const int nv = x0 < x1 ? (x1 - x0) / EPV : 0;
  const uint4* src = (const uint4*)(row + (size_t)x0 * esize);
  uint4 v[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j < nv) v[u] = src[j];
  }
  uint32_t acnt = 0;
  unsigned long long amass = 0;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j < nv) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float f = E::get(v[u], e);
        const uint32_t key = key_of<E>(f);
        if (key > chi) {
          ++acnt;
          amass += fixmass(fexp2((f - m) * q.c));
        } else if (key >= clo) {
          atomicAdd(&sm.h[key - clo], 1u);
        }
      }
    }
  }
  // workgroup sums of the entries above the window
  const uint32_t tc = block_inclusive_scan<uint32_t>(acnt, sm.rs.scan32);
  const unsigned long long tm = block_inclusive_scan<unsigned long long>(amass, sm.rs.scan64);
  FinePart* fp = p.fp3 + (size_t)r * p.S3 + s;
  if (tid == NT - 1) {
    st64(&fp->above_mass, tm);
    st32(&fp->above_cnt, tc);
  }
  uint32_t* fc = p.fc3 + ((size_t)r * p.S3 + s) * (WF / 2);
  for (int j = tid; j < (width + 1) / 2; j += NT) {
    const uint32_t lo = sm.h[2 * j], hi = (2 * j + 1 < width) ? sm.h[2 * j + 1] : 0u;
    st32(&fc[j], lo | (hi << 16));
  }
  if (!arrive_last(&p.cnt3[r], (uint32_t)p.S3, &sm.rs.flag)) return;
  // merge: entries from the top of the window (key chi) downwards
  uint32_t above_c = 0;
  unsigned long long above_m = 0;
  for (int t = 0; t < p.S3; ++t) {
    above_c += ld32(&p.fp3[(size_t)r * p.S3 + t].above_cnt);
    above_m += ld64(&p.fp3[(size_t)r * p.S3 + t].above_mass);
  }
  for (int co = tid; co < width; co += NT) {
    const uint32_t key = chi - (uint32_t)co;
    const uint32_t d = key - clo;
    uint32_t cnt = 0;
    for (int t = 0; t < p.S3; ++t) {
      const uint32_t w = ld32(&p.fc3[((size_t)r * p.S3 + t) * (WF / 2) + (d >> 1)]);
      cnt += (d & 1) ? (w >> 16) : (w & 0xffffu);
    }
    sm.scnt[co] = cnt;
    sm.smass[co] = cnt ? (unsigned long long)cnt * fixmass(fexp2((key16_value(key) - m) * q.c)) : 0ull;
  }
  __syncthreads();
  int sel = -1;
  unsigned long long zsel = 0;
  const bool good = select_run(sm.scnt, sm.smass, sm.ss, sm.rs, width, above_c, above_m, (double)sm.Ztot * 0x1p40,
                               q.K, q.P, p.V, sel, zsel);
  uint32_t thr = 0;
  float Z = 0.0f;
  if (good) {
    thr = chi - (uint32_t)sel;
    Z = (float)((double)zsel * 0x1p-40);
  } else {
    row_cutoff<E>(sm.rad, sm.rs, row, p.V, m, q.c, q.K, q.P, thr, Z);
  }
  if (tid == 0) {
    ri->thr = thr;
    ri->Z = Z;
    ri->state = state & ~ST_FINE;
    atomicExch(&p.cnt3[r], 0u);
  }
}

// ---------------------------------------------------------------------------------------------
// K5: accept chain, alpha, residual / bonus draw, outputs.
// ---------------------------------------------------------------------------------------------
struct K5Smem {
  RedSmem rs;
  float m[MAXROWS], Z[MAXROWS], invZ[MAXROWS];
  int32_t arg[MAXROWS];
  uint32_t thr[MAXROWS], state[MAXROWS];
  float gath[2 * MAXK];
  float u[MAXK];
  float wacc[MAXK][NWAVE];
  float stage[64 * (MAXK + 2)];
  int32_t n, pick;
};

// Gumbel-max over w(x) = exp2((l - m) c) on the kept entries of one row (stream tag, b, position j).
template <class E>
__device__ void gumbel_row_partial(const uint4& v, int xbase, float m, float c, uint32_t thr, uint32_t tag,
                                   uint32_t b, uint32_t j, const Params& p, float& best, int& bidx) {
#pragma unroll
  for (int g = 0; g < E::EPV; g += 4) {
    const int x = xbase + g;
    const uint4 w4 = philox10(make_uint4((uint32_t)x >> 2, b, (tag << 24) | j, p.offset), p.key0, p.key1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = E::get(v, g + e);
      const float w = key_of<E>(f) >= thr ? fexp2((f - m) * c) : 0.0f;
      if (w > 0.0f) {
        const uint32_t word = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
        const float key = w / exp_race_E2(word);
        if (key > best) {
          best = key;
          bidx = x + e;
        }
      }
    }
  }
}

__device__ void write_sentinel(const Params& p, int b) {
  const int k = p.k, tid = threadIdx.x;
  if (p.mode == MODE_SAMPLE) {
    if (tid == 0) {
      p.tokens[b] = -1;
      p.logprobs[b] = __builtin_nanf("");
    }
    return;
  }
  if (tid <= k) {
    p.tokens[(size_t)b * (k + 1) + tid] = -1;
    p.logprobs[(size_t)b * (k + 1) + tid] = __builtin_nanf("");
  }
  if (tid < k) p.alpha[(size_t)b * k + tid] = __builtin_nanf("");
  if (tid == 0) p.accept_len[b] = 0;
}

template <class E>
__device__ void k5_finalize(const Params& p, K5Smem& sm, int b, bool ok, const RowParams& q) {
  const int k = p.k, S = p.S5;
  const int tid = threadIdx.x;
  constexpr int esize = 16 / E::EPV;
  if (!ok) return write_sentinel(p, b);
  if (q.greedy) {
    if (p.mode == MODE_SAMPLE) {
      if (tid == 0) {
        p.tokens[b] = sm.arg[0];
        p.logprobs[b] = 0.0f;
      }
      return;
    }
    int n = k;
    for (int i = 0; i < k; ++i)
      if (p.draft_tokens[(size_t)b * k + i] != sm.arg[i]) {
        n = i;
        break;
      }
    const int y = sm.arg[n];
    if (tid < k) p.alpha[(size_t)b * k + tid] = (sm.arg[tid] == sm.arg[k + 1 + tid]) ? 1.0f : 0.0f;
    if (tid <= k) {
      const int t = tid < n ? p.draft_tokens[(size_t)b * k + tid] : (tid == n ? y : -1);
      p.tokens[(size_t)b * (k + 1) + tid] = t;
      p.logprobs[(size_t)b * (k + 1) + tid] = 0.0f;
    }
    if (tid == 0) p.accept_len[b] = n + 1;
    return;
  }
  const int n = sm.n;
  const int W = k + 2;
  float asum = 0.0f;  // thread t < k: alpha_t summed in slice order
  float best = 0.0f;
  int bidx = INT_MAX;
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int cnt = min(64, S - s0);
    for (int e = tid; e < cnt * W; e += NT) {
      const int sl = e / W, f = e - sl * W;
      const FinalPart* fp = p.fin5 + (size_t)b * S + s0 + sl;
      sm.stage[e] = f < k ? ldf(&fp->alpha[f]) : (f == k ? ldf(&fp->key) : __uint_as_float(ld32(&fp->idx)));
    }
    __syncthreads();
    if (tid < k)
      for (int sl = 0; sl < cnt; ++sl) asum += sm.stage[sl * W + tid];
    if (tid == 0)
      for (int sl = 0; sl < cnt; ++sl) {
        const float key = sm.stage[sl * W + k];
        if (key > best) {
          best = key;
          bidx = (int)__float_as_uint(sm.stage[sl * W + k + 1]);
        }
      }
    __syncthreads();
  }
  if (tid < k) p.alpha[(size_t)b * k + tid] = asum;
  if (tid == 0) sm.pick = bidx;
  __syncthreads();
  int y = sm.pick;
  __syncthreads();
  if (y == INT_MAX && n < k) {
    // The residual mass vanished in fp32 (rounding only): draw from p_n over the whole row.
    const uint8_t* row = row_ptr(p, b, n, esize);
    float bb = 0.0f;
    int bi = INT_MAX;
    for (int j = tid; j < p.V / E::EPV; j += NT)
      gumbel_row_partial<E>(((const uint4*)row)[j], j * E::EPV, sm.m[n], q.c, sm.thr[n], 1u, (uint32_t)b, (uint32_t)n,
                            p, bb, bi);
    block_maxarg(sm.rs, bb, bi);
    y = bi;
  }
  if (y < 0 || y >= p.V) return write_sentinel(p, b);  // no candidate: not reachable for a valid row
  if (p.mode == MODE_SAMPLE) {
    if (tid == 0) {
      const float l = E::load1(row_ptr(p, b, 0, esize), y);
      p.tokens[b] = y;
      p.logprobs[b] = (l - sm.m[0]) / q.T - logf(sm.Z[0]);
    }
    return;
  }
  if (tid <= k) {
    int t = -1;
    float lp = 0.0f;
    if (tid <= n) {
      t = tid < n ? p.draft_tokens[(size_t)b * k + tid] : y;
      const float l = tid < n ? sm.gath[tid] : E::load1(row_ptr(p, b, tid, esize), t);
      lp = (l - sm.m[tid]) / q.T - logf(sm.Z[tid]);
    }
    p.tokens[(size_t)b * (k + 1) + tid] = t;
    p.logprobs[(size_t)b * (k + 1) + tid] = lp;
  }
  if (tid == 0) p.accept_len[b] = n + 1;
}

template <class E, int VPT>
__global__ __launch_bounds__(NT) void k5_verify(Params p) {
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  __shared__ K5Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.S5, s = blockIdx.x - b * p.S5;
  const int k = p.k, rows = p.rows;
  const RowParams q = row_params(p, b);
  bool ok = q.ok;
  for (int i = 0; i < k; ++i) {
    const int x = p.draft_tokens[(size_t)b * k + i];
    ok = ok && x >= 0 && x < p.V;
  }
  float gv = 0.0f;
  if (ok && !q.greedy && tid < 2 * k) {
    const int i = tid < k ? tid : tid - k;
    gv = E::load1(row_ptr(p, b, tid < k ? i : k + 1 + i, esize), p.draft_tokens[(size_t)b * k + i]);
  }
  if (tid < rows) {
    const RowInfo* ri = p.rinfo + (size_t)b * rows + tid;
    sm.m[tid] = ri->m;
    sm.arg[tid] = ri->arg;
    sm.Z[tid] = ri->Z;
    sm.invZ[tid] = 1.0f / ri->Z;
    sm.thr[tid] = ri->thr;
    sm.state[tid] = ri->state;
  }
  if (ok && !q.greedy && tid < k) {
    const uint4 w4 = philox10(make_uint4((uint32_t)tid >> 2, (uint32_t)b, 0u, p.offset), p.key0, p.key1);
    const int qq = tid & 3;
    sm.u[tid] = u24(qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w);
  }
  if (ok && !q.greedy && tid < 2 * k) sm.gath[tid] = gv;
  __syncthreads();
  for (int r = 0; r < rows; ++r) ok = ok && sm.state[r] == 0;
  if (ok && !q.greedy) {
    if (tid == 0) {
      int n = k;  // k = 0 in sample mode: the draw below is the sampler's
      for (int i = 0; i < k; ++i) {
        const float lt = sm.gath[i], ld = sm.gath[k + i];
        const float pt = key_of<E>(lt) >= sm.thr[i] ? fexp2((lt - sm.m[i]) * q.c) / sm.Z[i] : 0.0f;
        const float qd = key_of<E>(ld) >= sm.thr[k + 1 + i] ? fexp2((ld - sm.m[k + 1 + i]) * q.c) / sm.Z[k + 1 + i] : 0.0f;
        const bool accept = pt > 0.0f && (qd == 0.0f || sm.u[i] < pt / qd);
        if (!accept) {
          n = i;
          break;
        }
      }
      sm.n = n;
    }
    __syncthreads();
    const int n = sm.n;
    const int x0 = s * p.L5;
    const int x1 = min(x0 + p.L5, p.V);
    const int nv = x0 < x1 ? (x1 - x0) / EPV : 0;
    float best = 0.0f;
    int bidx = INT_MAX;
    for (int i = 0; i < k; ++i) {
      const uint4* vt = (const uint4*)(row_ptr(p, b, i, esize) + (size_t)x0 * esize);
      const uint4* vd = (const uint4*)(row_ptr(p, b, k + 1 + i, esize) + (size_t)x0 * esize);
      uint4 va[VPT], vb[VPT];
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) {
          va[u] = vt[j];
          vb[u] = vd[j];
        }
      }
      const float mt = sm.m[i], md = sm.m[k + 1 + i];
      const float it = sm.invZ[i], id = sm.invZ[k + 1 + i];
      const uint32_t tt = sm.thr[i], td = sm.thr[k + 1 + i];
      float acc = 0.0f;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) {
#pragma unroll
          for (int g = 0; g < EPV; g += 4) {
            float r4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lt = E::get(va[u], g + e), ld = E::get(vb[u], g + e);
              const float pt = key_of<E>(lt) >= tt ? fexp2((lt - mt) * q.c) * it : 0.0f;
              const float qd = key_of<E>(ld) >= td ? fexp2((ld - md) * q.c) * id : 0.0f;
              acc += fminf(pt, qd);
              r4[e] = pt - qd;
            }
            if (i == n) {
              const int x = x0 + j * EPV + g;
              const uint4 w4 = philox10(make_uint4((uint32_t)x >> 2, (uint32_t)b, (1u << 24) | (uint32_t)n, p.offset),
                                        p.key0, p.key1);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (r4[e] > 0.0f) {
                  const uint32_t word = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
                  const float key = r4[e] / exp_race_E2(word);
                  if (key > best) {
                    best = key;
                    bidx = x + e;
                  }
                }
              }
            }
          }
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) sm.wacc[i][wave] = acc;
    }
    if (n == k) {
      // bonus draw from p_k (verify stream), or the plain sampler's draw (its own stream)
      const bool smp = p.mode == MODE_SAMPLE;
      const uint32_t tag = smp ? 2u : 1u;
      const uint32_t sb = smp ? (uint32_t)(p.row_b ? p.row_b[b] : b) : (uint32_t)b;
      const uint32_t sj = smp ? (uint32_t)(p.row_pos ? p.row_pos[b] : 0) : (uint32_t)k;
      const uint4* vt = (const uint4*)(row_ptr(p, b, k, esize) + (size_t)x0 * esize);
      uint4 va[VPT];
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) va[u] = vt[j];
      }
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) gumbel_row_partial<E>(va[u], x0 + j * EPV, sm.m[k], q.c, sm.thr[k], tag, sb, sj, p, best, bidx);
      }
    }
    block_maxarg(sm.rs, best, bidx);  // its barriers also order the wacc writes before the reads below
    FinalPart* fp = p.fin5 + (size_t)b * p.S5 + s;
    if (tid < k) {
      float v = 0.0f;
      for (int w = 0; w < NWAVE; ++w) v += sm.wacc[tid][w];
      stf(&fp->alpha[tid], v);
    }
    if (tid == 0) {
      stf(&fp->key, best);
      st32(&fp->idx, (uint32_t)bidx);
    }
  }
  if (arrive_last(&p.cnt5[b], (uint32_t)p.S5, &sm.rs.flag)) {
    k5_finalize<E>(p, sm, b, ok, q);
    if (tid == 0) atomicExch(&p.cnt5[b], 0u);
  }
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
struct Geo {
  int rows, R, S1, S3, S5, L1, L3, L5, esize, EPV;
  size_t off_cnt1, off_cnt3, off_cnt5, off_st1, off_hw1, off_hb1, off_rinfo, off_fp3, off_fc3, off_fin5, off_trace,
      total;
};

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static bool make_geo(int32_t B, int32_t k, int32_t V, spec_dtype_t dtype, Geo& g) {
  if (B < 1 || B > (1 << 20) || k < 0 || k > MAXK || V < 8 || V > (1 << 20)) return false;
  if (dtype != SPEC_DTYPE_BF16 && dtype != SPEC_DTYPE_F32) return false;
  g.esize = dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  g.EPV = 16 / g.esize;
  if (V % g.EPV != 0) return false;
  g.rows = 2 * k + 1;
  if ((long long)B * g.rows > (1 << 24)) return false;  // grids stay below 2^31 workgroups
  g.R = B * g.rows;
  g.L1 = NT * g.EPV * VPT1;
  g.L3 = NT * g.EPV * VPT3;
  g.L5 = NT * g.EPV * VPT5;
  g.S1 = (V + g.L1 - 1) / g.L1;
  g.S3 = (V + g.L3 - 1) / g.L3;
  g.S5 = (V + g.L5 - 1) / g.L5;
  const size_t R = (size_t)g.R;
  size_t off = 256;
  auto take = [&](size_t& o, size_t bytes) {
    o = off;
    off = align_up(off + bytes, 256);
  };
  take(g.off_cnt1, R * 4);
  take(g.off_cnt3, R * 4);
  take(g.off_cnt5, (size_t)B * 4);
  take(g.off_st1, R * g.S1 * sizeof(StatPart));
  take(g.off_hw1, R * g.S1 * (WTOP / 2) * 4);
  take(g.off_hb1, R * g.S1 * (NB / 2 + NB + 1) * 4);
  take(g.off_rinfo, R * sizeof(RowInfo));
  take(g.off_fp3, R * g.S3 * sizeof(FinePart));
  take(g.off_fc3, R * g.S3 * (WF / 2) * 4);
  take(g.off_fin5, (size_t)B * g.S5 * sizeof(FinalPart));
  take(g.off_trace, R * g.S1 * TRACE_SLOTS * 8);
  g.total = off;
  return true;
}

struct DevInfo {
  int state;  // 0 unknown, 1 gfx950, 2 other
};
static DevInfo g_dev[MAXDEV];
static std::mutex g_mu;

static bool device_ok(int dev) {
  if (dev < 0 || dev >= MAXDEV) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_dev[dev].state == 0) {
    hipDeviceProp_t pr;
    if (hipGetDeviceProperties(&pr, dev) != hipSuccess) return false;
    g_dev[dev].state = (std::strncmp(pr.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  return g_dev[dev].state == 1;
}

template <class E>
static void enqueue(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL((k1_stats<E, VPT1>), dim3((unsigned)p.S1 * p.R), dim3(NT), 0, st, p);
  hipLaunchKernelGGL((k3_fine<E, VPT3>), dim3((unsigned)p.S3 * p.R), dim3(NT), 0, st, p);
  hipLaunchKernelGGL((k5_verify<E, VPT5>), dim3((unsigned)p.S5 * p.B), dim3(NT), 0, st, p);
}

static spec_status_t launch(Params& p, const Geo& g, spec_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!workspace || workspace_bytes < g.total || ((uintptr_t)workspace & 15)) return SPEC_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) return SPEC_ERR_UNSUPPORTED_DEVICE;
  p.rows = g.rows;
  p.R = g.R;
  p.S1 = g.S1;
  p.S3 = g.S3;
  p.S5 = g.S5;
  p.L1 = g.L1;
  p.L3 = g.L3;
  p.L5 = g.L5;
  uint8_t* ws = (uint8_t*)workspace;
  p.cnt1 = (uint32_t*)(ws + g.off_cnt1);
  p.cnt3 = (uint32_t*)(ws + g.off_cnt3);
  p.cnt5 = (uint32_t*)(ws + g.off_cnt5);
  p.st1 = (StatPart*)(ws + g.off_st1);
  p.hw1 = (uint32_t*)(ws + g.off_hw1);
  p.hb1 = (uint32_t*)(ws + g.off_hb1);
  p.rinfo = (RowInfo*)(ws + g.off_rinfo);
  p.fp3 = (FinePart*)(ws + g.off_fp3);
  p.fc3 = (uint32_t*)(ws + g.off_fc3);
  p.fin5 = (FinalPart*)(ws + g.off_fin5);
  p.trace = TRACE_SLOTS > 0 ? (unsigned long long*)(ws + g.off_trace) : nullptr;
  if (dtype == SPEC_DTYPE_BF16)
    enqueue<BF16>(p, (hipStream_t)stream);
  else
    enqueue<F32>(p, (hipStream_t)stream);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}

}  // namespace sv

using namespace sv;

extern "C" size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, spec_dtype_t dtype) {
  Geo g;
  if (k < 1 || !make_geo(B, k, V, dtype, g)) return 0;
  return g.total;
}

extern "C" const char* spec_verify_status_string(spec_status_t status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPEC_ERR_WORKSPACE: return "workspace missing or too small";
    case SPEC_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case SPEC_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

extern "C" spec_status_t spec_verify(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                     const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                                     const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed,
                                     uint64_t offset, int32_t* tokens, int32_t* accept_len, float* logprobs,
                                     float* alpha, void* workspace, size_t workspace_bytes, void* stream) {
  Geo g;
  if (k < 1 || !make_geo(B, k, V, dtype, g)) return SPEC_ERR_INVALID_ARGUMENT;
  if (offset >= (1ull << 32)) return SPEC_ERR_INVALID_ARGUMENT;
  if (!target_logits || !draft_logits || !draft_tokens || !temperature || !top_k || !top_p || !tokens ||
      !accept_len || !logprobs || !alpha)
    return SPEC_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)target_logits & 15) || ((uintptr_t)draft_logits & 15)) return SPEC_ERR_INVALID_ARGUMENT;
  Params p;
  std::memset(&p, 0, sizeof p);
  p.target = (const uint8_t*)target_logits;
  p.draft = (const uint8_t*)draft_logits;
  p.draft_tokens = draft_tokens;
  p.temperature = temperature;
  p.top_k = top_k;
  p.top_p = top_p;
  p.B = B;
  p.k = k;
  p.V = V;
  p.mode = MODE_VERIFY;
  p.key0 = (uint32_t)(seed & 0xffffffffu);
  p.key1 = (uint32_t)(seed >> 32);
  p.offset = (uint32_t)offset;
  p.tokens = tokens;
  p.accept_len = accept_len;
  p.logprobs = logprobs;
  p.alpha = alpha;
  return launch(p, g, dtype, workspace, workspace_bytes, stream);
}

extern "C" size_t spec_sample_workspace_size(int32_t R, int32_t V, spec_dtype_t dtype) {
  Geo g;
  if (!make_geo(R, 0, V, dtype, g)) return 0;
  return g.total;
}

extern "C" spec_status_t spec_sample(const void* logits, spec_dtype_t dtype, const float* temperature,
                                     const int32_t* top_k, const float* top_p, const int32_t* row_b,
                                     const int32_t* row_pos, int32_t R, int32_t V, uint64_t seed, uint64_t offset,
                                     int32_t* tokens, float* logprobs, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  Geo g;
  if (!make_geo(R, 0, V, dtype, g)) return SPEC_ERR_INVALID_ARGUMENT;
  if (offset >= (1ull << 32)) return SPEC_ERR_INVALID_ARGUMENT;
  if (!logits || !temperature || !top_k || !top_p || !tokens || !logprobs) return SPEC_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)logits & 15) return SPEC_ERR_INVALID_ARGUMENT;
  Params p;
  std::memset(&p, 0, sizeof p);
  p.target = (const uint8_t*)logits;
  p.draft = (const uint8_t*)logits;
  p.temperature = temperature;
  p.top_k = top_k;
  p.top_p = top_p;
  p.B = R;
  p.k = 0;
  p.V = V;
  p.mode = MODE_SAMPLE;
  p.row_b = row_b;
  p.row_pos = row_pos;
  p.key0 = (uint32_t)(seed & 0xffffffffu);
  p.key1 = (uint32_t)(seed >> 32);
  p.offset = (uint32_t)offset;
  p.tokens = tokens;
  p.logprobs = logprobs;
  return launch(p, g, dtype, workspace, workspace_bytes, stream);
}
