// specverify.hip -- libspecverify: the speculative-decoding verify sampler for gfx950 (MI355X), and its
// C ABI (include/specverify.h).
//
// Method: AReno pull request "feat(engine): MTP training loss and speculative decoding for bailing_v3",
// section "What does this PR do?" (Phase 2: sampler-equivalent target distribution, exact chain
// rejection sampling, unchanged logprobs), its accept-probability table (alpha = sum min(p, q)), and
// its per-step optimisation table (Gumbel-max draws, no host synchronisation).
//
// One call enqueues three kernels on the caller's stream; no workgroup ever waits for another.  Where
// workgroups of one kernel combine partials (K5, the tree kernel), the last one to arrive at a per-row
// counter does it (agent-scope atomics; partials travel through agent-scope atomic stores and loads,
// coherent across the XCDs' L2s without cache-wide write-back or invalidation).
//
//   K1 stats   items (logit row, slice of 18432 bf16 logits, 24576 on calls of many slices, 9216 fp32), all
//              slices of a row on one XCD.  Streams every logit once with
//              16-byte loads and keeps only what the row needs: NaN-propagating max (lowest argmax for
//              greedy rows); the sum of exp2((l - max) * log2(e) / T) for rows whose normaliser is the
//              whole row; for bf16 rows with top-k <= 64, a record of the slice's candidate logits; for
//              other truncated bf16 rows, exact per-code counts of the 512 order-preserving codes below
//              the slice max (keys of two logits at a time, packed 16-bit operations) and, for top-p-only
//              rows, counts in 1/8-log2-unit weight bins.
//   K1 rows    one workgroup per logit row, after every slice is done: row max / argmax / normaliser and,
//              for truncated rows, the kept threshold (one round trip for all partials).  From recorded
//              candidates or among the row's top 512 codes the threshold is exact (merged per-code counts,
//              masses = count x 2^40 fixed-point weight, integer sums).  Otherwise the weight bins bound
//              the cumulative mass, which gives a code window that must hold the threshold; the workgroup
//              counts that window exactly over the whole row (or lists its entries when the window
//              straddles logit 0).  Anything this cannot settle (fp32 keys, a failed self-check) takes an
//              exact MSD radix select.
//   K5 verify  items (batch row, slice).  Each evaluates the accept chain (p_i(x_i), q_i(x_i) from the
//              row statistics and two gathered logits, Philox accept uniforms), then re-reads its slice
//              of the draft-position rows, one position at a time: alpha partial sums for every position
//              and the Gumbel-max race candidate at the first rejected position (residual max(p - q, 0))
//              or at position k (bonus from p_k).  Logits below a row's kept threshold are skipped a wave
//              at a time.  Batch rows whose kept sets K1 recorded whole are finished from the records.
//              The last slice of a batch row writes the outputs.
//   k_tree     tree verification in place of K5 (see its comment).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "specverify.h"
#include "sv_common.h"

namespace sv {

constexpr int MODE_VERIFY = 0;
constexpr int MODE_SAMPLE = 1;  // plain sampler: k = 0, one logit row per batch row, stream tag 2
constexpr int MODE_TREE = 2;    // tree verification: N = rows = k + 1 target rows per batch row, no draft rows
constexpr int MAXN = 64;        // nodes per draft tree
constexpr int MAXDEV = 64;
constexpr int VPT1 = 9;         // K1: 16-byte vectors per thread per slice (18432 bf16 logits)
constexpr int VPT1W = 12;       // K1, bf16 calls of many slices (at least K1W_ITEMS of 24576 logits): wider slices
constexpr int K1W_ITEMS = 8192; //   (several rounds of the slice kernel's workgroup slots: its per-slice work dominates)
constexpr int VPT5 = 2;         // K5
constexpr int OCC1 = 7;         // K1 workgroups per CU (register budget of its launch bounds)
constexpr int FVPT = 2;         // whole-row passes of one workgroup: vectors per thread per step
constexpr int WTOP = 512;       // K1: exact per-code window below the slice max
constexpr int NBC = 256;        // K1: weight bins of top-p-only rows
constexpr float BRC = 8.0f;     // weight bins per log2 unit
constexpr int NCOPY = 4;        // K1: interleaved copies of each weight bin (lane & 3 picks one)
constexpr int WF = 2048;        // widest exact code window of the whole-row pass
constexpr int MAXS1 = 64;       // slices per bf16 row at the largest V
constexpr int MB = 8;           // merge: slices whose histogram words are loaded in one round trip
constexpr int HCW = NBC / 2 + 1;  // words per slice of packed bin counts + the slice's base bin
constexpr int NKERN = SPEC_MAX_KERNELS;  // kernels per call at most

constexpr int WC = 64;          // K1: candidate window (codes below the slice max) of truncated rows
constexpr int NC = 192;         // K1: candidates recorded per slice at most
constexpr int NFLAG = 192;      // K1: staged candidate-holding vectors per slice at most
constexpr int NFW = 64;         // K1 top-k slices: staged candidate-holding vectors per wave at most
constexpr int KMAX = 1024;
constexpr int KC = 64;          // bf16 top-k rows with K <= KC take their kept threshold from the candidates      // kept entries per row at most for the candidate (sparse) path of K5
constexpr int HT = 2048;        // K5 sparse path: hash table entries (power of two, > KMAX)

constexpr uint32_t ST_BAD = 1u;     // NaN / +inf entries, or every entry -inf
constexpr uint32_t ST_SPARSE = 2u;  // every kept entry is among the row's recorded candidates

struct StatPart {  // K1, per (logit row, slice)
  float m;         // slice max (NaN if the slice holds a NaN, for non-greedy rows)
  int32_t arg;     // lowest index of the slice max (greedy rows; INT_MAX otherwise)
  float s;         // sum of exp2((l - m) c) over the slice (rows that need the whole-row normaliser)
  uint32_t flags;  // bit 0: NaN or +inf seen
  float g;         // the row's logit at its draft token, if the token falls in this slice
  uint32_t floor;  // candidate rows: every finite logit of the slice with key >= floor was recorded
  float rmax, rsum;  // raw logprobs requested, target rows: the slice max and sum of exp(l - rmax)
};

struct RowInfo {    // per logit row
  float m;          // row max
  int32_t arg;      // lowest argmax (greedy rows)
  float Z;          // normaliser of the kept set: sum of exp2((l - m) c) over kept entries
  float lz;         // log2(Z)
  float fthr;       // smallest kept value (-inf: every entry kept)
  uint32_t state;   // ST_BAD
  float rlz;        // raw logprobs requested, target rows: log2 of the sum of exp(l - m) (no T, no truncation)
  float gath;       // logit at the draft token of this position (draft-position rows of a valid token)
};

struct FinalPart {  // K5, per (batch row, slice)
  float alpha[MAXK];
  float key;        // best Gumbel race key w / E2 (0 = no candidate)
  int32_t idx;      // its vocabulary index (INT_MAX = none)
  float val;        // its logit
  uint32_t pad;
};

struct Params {
  const uint8_t* target;
  const uint8_t* draft;
  const int32_t* draft_tokens;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t B, k, V, rows, R;  // rows = 2k + 1 logit rows per batch row, R = B * rows
  int32_t S1, S5, L1, L5;
  int32_t mode;              // MODE_VERIFY or MODE_SAMPLE
  const int32_t* row_b;      // plain sampler: stream coordinate b of each row (NULL = row index)
  const int32_t* row_pos;    // plain sampler: stream coordinate i of each row (NULL = 0)
  uint32_t key0, key1, offset;
  const int32_t* parent;     // tree mode: [B][N] parent of each node (the draft tokens are the nodes' tokens)
  int32_t* path;             // tree mode: [B][N] accepted node indices
  int32_t* tokens;
  int32_t* accept_len;
  float* logprobs;
  float* alpha;
  float* raw_logprobs;  // NULL, or [B][k+1] raw logprobs of the committed tokens
  uint32_t* cnt5;     // [B] K5 arrivals
  StatPart* st1;      // [R][S1]
  uint32_t* hw1;      // [R][S1][WTOP/2] packed 16-bit code counts
  uint32_t* hc1;      // [R][S1][HCW] packed 16-bit bin counts, then the slice's base bin (float)
  unsigned long long* cand1;  // [R][S1][NC] candidates of truncated rows: index << 16 | bf16 bits
  uint32_t* ncand1;   // [R][S1] candidates found per slice (may exceed NC: then the list is incomplete)
  RowInfo* rinfo;     // [R]
  FinalPart* fin5;    // [B][S5]
  unsigned long long* trace;   // K1 phase timestamps per item: instrumented builds only
  unsigned long long* trace5;  // K5 phase timestamps per item: instrumented builds only
};

// Phase timestamps of instrumented builds (compiled with -DSV_TRACE); no-ops otherwise.
#ifdef SV_TRACE
constexpr int TRACE_SLOTS = 8;
#define SV_TRACE_AT(p, item, slot)                                                                  \
  do {                                                                                             \
    if (threadIdx.x == 0 && (p).trace) (p).trace[(size_t)(item)*TRACE_SLOTS + (slot)] = wall_clock64(); \
  } while (0)
#define SV_TRACE5_AT(p, item, slot)                                                                 \
  do {                                                                                             \
    if (threadIdx.x == 0 && (p).trace5) (p).trace5[(size_t)(item)*TRACE_SLOTS + (slot)] = wall_clock64(); \
  } while (0)
#else
constexpr int TRACE_SLOTS = 0;
#define SV_TRACE_AT(p, item, slot) \
  do {                             \
  } while (0)
#define SV_TRACE5_AT(p, item, slot) \
  do {                              \
  } while (0)
#endif

// ---- small helpers ------------------------------------------------------------------------------
__device__ inline const uint8_t* row_ptr(const Params& p, int b, int r, int esize) {
  const size_t V = (size_t)p.V;
  if (r <= p.k) return p.target + ((size_t)b * (p.k + 1) + r) * V * esize;
  return p.draft + ((size_t)b * p.k + (r - p.k - 1)) * V * esize;
}

// Work item g -> (row r, slice s) for R rows of S slices.  Rows go in groups of 8, slice-major within
// a group: with a grid that is a multiple of 8 (workgroups are dealt to the 8 XCDs round robin) every
// slice of row 8q + x runs on XCD x.  Rows past the last full group map row-major.
__device__ inline void item_rs(int g, int R, int S, int& r, int& s) {
  const int full = (R & ~7) * S;
  if (g < full) {
    const int grp = g / (8 * S), rem = g - grp * 8 * S;
    s = rem >> 3;
    r = grp * 8 + (rem & 7);
  } else {
    const int h = g - full, q = h / S;
    r = (R & ~7) + q;
    s = h - q * S;
  }
}

__device__ inline unsigned long long fixmass(float e) {  // e in [0, 1] -> 2^40 fixed point
  return __float2ull_rn(e * 0x1p40f);
}

__device__ inline void st32(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void stf(void* p, float v) { st32(p, __float_as_uint(v)); }
// Plain stores, for partials read only by a later kernel (the kernel boundary makes them visible).
__device__ inline void pst32(void* p, uint32_t v) { *(uint32_t*)p = v; }
__device__ inline void pstf(void* p, float v) { *(float*)p = v; }
__device__ inline uint32_t ld32(const void* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  if (total == 1) return true;  // the only arrival: no round trip (the counter stays at 0)
  if (threadIdx.x == 0) *flag = (atomicAdd(counter, 1u) == total - 1) ? 1 : 0;
  __syncthreads();
  return *flag != 0;
}

// Sampling parameters of a batch row.
struct RowParams {
  float T, P, c;
  int K;
  bool ok, greedy, trunc, useK, useP;
  bool cand;  // top-k with K <= KC (bf16 rows: kept threshold selected from the recorded candidates)
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
  q.useK = q.ok && !q.greedy && q.K > 0 && q.K < p.V;
  q.useP = q.ok && !q.greedy && q.P < 1.0f;
  q.trunc = q.useK || q.useP;
  q.cand = q.useK && q.K <= KC;
  return q;
}

// Combine (max, lowest argmax, sum of exp2((l - max) c), flags) with a second such quadruple.
__device__ inline void stats_combine(float& m, int& a, float& s, uint32_t& fl, float m2, int a2, float s2, uint32_t f2,
                                     float c) {
  float mm = m, ss = s;
  lse_combine(mm, ss, m2, s2, c);
  maxarg_combine(m, a, m2, a2);
  s = ss;
  fl |= f2;
}
// Wave reduction of (max, lowest argmax, sum of exp2((l - max) c), flags) into every lane (DPP steps inside
// the rows, then the four rows' quadruples).
__device__ inline void wave_stats(float& m, int& a, float& s, uint32_t& fl, float c) {
#define SV_STATS_STEP(C) \
  stats_combine(m, a, s, fl, dpp_mov_f<C>(m), (int)dpp_mov_u<C>((uint32_t)a), dpp_mov_f<C>(s), dpp_mov_u<C>(fl), c)
  SV_ROW_STEPS(SV_STATS_STEP);
#undef SV_STATS_STEP
  float m0 = row_f(m, 0), s0 = row_f(s, 0), m2 = row_f(m, 2), s2 = row_f(s, 2);
  int a0 = (int)row_u((uint32_t)a, 0), a2 = (int)row_u((uint32_t)a, 2);
  uint32_t f0 = row_u(fl, 0), f2 = row_u(fl, 2);
  stats_combine(m0, a0, s0, f0, row_f(m, 1), (int)row_u((uint32_t)a, 1), row_f(s, 1), row_u(fl, 1), c);
  stats_combine(m2, a2, s2, f2, row_f(m, 3), (int)row_u((uint32_t)a, 3), row_f(s, 3), row_u(fl, 3), c);
  stats_combine(m0, a0, s0, f0, m2, a2, s2, f2, c);
  m = m0;
  a = a0;
  s = s0;
  fl = f0;
}

struct RedSmem {
  float f[NWAVE], g[NWAVE];
  int32_t i[NWAVE];
  uint32_t u[NWAVE];
  unsigned long long scan64[NWAVE];
  uint32_t scan32[NWAVE];
  double scand[NWAVE];
  int32_t flag;
};

// Workgroup (max, argmax, sum, flags) into every thread.
__device__ __forceinline__ void block_stats(RedSmem& rs, float& m, int& a, float& s, uint32_t& fl, float c) {
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

// Workgroup NaN-propagating max into every thread.
__device__ __forceinline__ float block_nan_max(RedSmem& rs, float m) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  m = wave_nan_max(m);
  if (lane == 0) rs.f[wave] = m;
  __syncthreads();
  m = rs.f[0];
  for (int w = 1; w < NWAVE; ++w) m = nan_max(m, rs.f[w]);
  __syncthreads();
  return m;
}

__device__ __forceinline__ void block_maxarg(RedSmem& rs, float& m, int& a) {
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

// Workgroup sum into every thread.
__device__ __forceinline__ uint32_t block_sum_u32(RedSmem& rs, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_u32(v);
  if (lane == 0) rs.u[wave] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < NWAVE; ++w) t += rs.u[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ uint32_t block_max_u32(RedSmem& rs, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_max_u32(v);
  if (lane == 0) rs.u[wave] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < NWAVE; ++w) t = max(t, rs.u[w]);
  __syncthreads();
  return t;
}

// Lowest thread index whose predicate holds, into every thread (NT if none).
__device__ __forceinline__ int block_first(RedSmem& rs, bool pred) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fl = first_lane(pred);
  if (lane == 0) rs.i[wave] = fl < 64 ? wave * 64 + fl : NT;
  __syncthreads();
  int r = NT;
  for (int w = 0; w < NWAVE; ++w) r = min(r, rs.i[w]);
  __syncthreads();
  return r;
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

// One digit histogram of the entries whose key is >= thr and matches `prefix` above the digit.
template <class E, bool COUNTS>
__device__ __forceinline__ void radix_hist(RadixSmem& sm, const uint4* src, int nvec, int lev, uint32_t prefix, uint32_t thr,
                           float m, float c) {
  const int tid = threadIdx.x;
  const int shift = E::KEYBITS - 8 * (lev + 1);
  for (int j0 = 0; j0 < nvec; j0 += NT * FVPT) {
    uint4 v[FVPT];
#pragma unroll
    for (int u = 0; u < FVPT; ++u) {
      const int j = j0 + tid + u * NT;
      if (j < nvec) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < FVPT; ++u) {
      const int j = j0 + tid + u * NT;
      if (j < nvec) {
#pragma unroll
        for (int e = 0; e < E::EPV; ++e) {
          const float f = E::get(v[u], e);
          const uint32_t key = key_of<E>(f);
          if (key >= thr && (lev == 0 || (key >> (shift + 8)) == prefix)) {
            const uint32_t d = (key >> shift) & 255u;
            if (COUNTS) atomicAdd(&sm.hcnt[d], 1u);
            atomicAdd(&sm.hmass[d], fixmass(fexp2((f - m) * c)));
          }
        }
      }
    }
  }
}

template <class E>
__device__ __forceinline__ void row_cutoff(RadixSmem& sm, RedSmem& rs, const uint8_t* row, int V, float m, float c, int K, float P,
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
      sm.hcnt[tid] = 0;
      sm.hmass[tid] = 0;
      __syncthreads();
      radix_hist<E, true>(sm, src, nvec, lev, prefix, 0u, m, c);
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
      sm.hmass[tid] = 0;
      __syncthreads();
      radix_hist<E, false>(sm, src, nvec, lev, prefix, thr, m, c);
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
// Threshold search over a descending run of bf16 codes: cnt[i] (LDS) counts code ktop - i, whose mass
// is cnt x 2^40-fixed-point exp2((value - m) c).  Finds the first entry where the running count reaches
// K (top-k) and, within the kept prefix, the first where the running mass reaches P * Z_K (top-p).
// base_cnt / base_mass are the totals above entry 0; ztot_fixed is the whole row's mass (used when
// top-k is off).  Returns false if a threshold lies outside the run: the caller then looks elsewhere.
// ---------------------------------------------------------------------------------------------
struct SelState {
  int32_t sel_k, sel_p;
  uint32_t ck;  // entries at or above the top-k cut
  unsigned long long zk, zp;
};

__device__ inline unsigned long long code_mass(uint32_t cnt, uint32_t code, float m, float c) {
  return cnt ? (unsigned long long)cnt * fixmass(fexp2((key16_value(code) - m) * c)) : 0ull;
}

// Entry i is code ktop - i, or codes[i] when a list of (descending) codes is given.
__device__ __forceinline__ bool select_run(const uint32_t* cnt, int n, uint32_t ktop, float m, float c, SelState& ss, RedSmem& rs,
                           uint32_t base_cnt, unsigned long long base_mass, double ztot_fixed, bool useK, int K,
                           bool useP, float P, int& sel, unsigned long long& zsel, const uint32_t* codes = nullptr) {
  const int tid = threadIdx.x;
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
      const uint32_t k0 = codes ? (i0 < n ? codes[i0] : 0u) : ktop - i0, k1 = codes ? (i1 < n ? codes[i1] : 0u) : ktop - i1;
      const unsigned long long b0 = code_mass(a0, k0, m, c), b1 = code_mass(a1, k1, m, c);
      const uint32_t ic = block_inclusive_scan<uint32_t>(a0 + a1, rs.scan32) + ccarry;
      const unsigned long long im = block_inclusive_scan<unsigned long long>(b0 + b1, rs.scan64) + mcarry;
      const uint32_t e0 = ic - a0 - a1;
      const unsigned long long f0 = im - b0 - b1;
      if (i0 < n && e0 < (uint32_t)K && e0 + a0 >= (uint32_t)K) {
        ss.sel_k = i0;
        ss.zk = f0 + b0;
        ss.ck = e0 + a0;
      } else if (i1 < n && e0 + a0 < (uint32_t)K && ic >= (uint32_t)K) {
        ss.sel_k = i1;
        ss.zk = im;
        ss.ck = ic;
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
      const uint32_t a0 = i0 <= last ? cnt[i0] : 0u, a1 = i1 <= last ? cnt[i1] : 0u;
      const uint32_t k0 = codes ? (i0 <= last ? codes[i0] : 0u) : ktop - i0;
      const uint32_t k1 = codes ? (i1 <= last ? codes[i1] : 0u) : ktop - i1;
      const unsigned long long b0 = code_mass(a0, k0, m, c), b1 = code_mass(a1, k1, m, c);
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

// Loads row r's candidate slots (slice s, entry e < count) with key >= thr: thread t takes slots t,
// t + NT, ... of the S x NC slot grid from base on; all of a thread's loads are issued before any is
// used.  Empty or filtered slots get index 0xffffffff.
template <int NSLOT>
__device__ inline void sparse_load(const Params& p, const uint32_t* ncs, int r, uint32_t thr, uint32_t (&xs)[NSLOT],
                                   float (&fs)[NSLOT], int base) {
  const int tid = threadIdx.x, S = p.S1;
  unsigned long long c[NSLOT];
#pragma unroll
  for (int t = 0; t < NSLOT; ++t) {
    const int g = base + tid + t * NT, sl = g / NC, e = g - sl * NC;
    c[t] = (sl < S && (uint32_t)e < min(ncs[sl], (uint32_t)NC))
               ? __hip_atomic_load(p.cand1 + ((size_t)r * S + sl) * NC + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : ~0ull;  // no slot (a recorded candidate has an index below 2^20)
  }
#pragma unroll
  for (int t = 0; t < NSLOT; ++t) {
    const float f = __uint_as_float((uint32_t)(c[t] & 0xffffu) << 16);
    const bool keep = c[t] != ~0ull && key16f(f) >= thr;
    xs[t] = keep ? (uint32_t)(c[t] >> 16) : 0xffffffffu;
    fs[t] = f;
  }
}

// Bit e set: entry e of a bf16 vector has key >= fe.
__device__ inline uint32_t cand_bits_ge(const uint4& v, uint32_t fe) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t k2 = key16x2(wv[q]);
    bits |= ((k2 & 0xffffu) >= fe ? 1u : 0u) << (2 * q);
    bits |= ((k2 >> 16) >= fe ? 1u : 0u) << (2 * q + 1);
  }
  return bits;
}

// ---------------------------------------------------------------------------------------------
// K1: row statistics (every logit read once) per slice, then one merge per row (k1_rows, its own kernel).
// ---------------------------------------------------------------------------------------------
struct K1Smem {
  RedSmem rs;
  SelState ss;
  uint32_t win[4];
  union {
    struct {                    // streaming phase; entries past WTOP / NBC absorb out-of-range
      uint32_t hw[WTOP + 64];   // logits, one per lane, so the atomics need no branch
      uint32_t hc[(NBC + 64) * NCOPY];  // bin j, copy q at j NCOPY + q: lanes that hit one bin
                                        // mostly hit different words (fewer same-address atomics)
      unsigned long long cand[NC];  // the slice's recorded candidates (index << 16 | bits): logits within WC
                                    // codes of the slice max, or at or above a top-k slice's floor
      uint32_t ncand;
      uint4 fvec[NWAVE * NFW];  // staged vectors that hold a candidate, and their vector indices
      uint32_t fidx[NWAVE * NFW];
      uint32_t nflag;
      uint32_t over;            // a wave could not stage all its candidate-holding vectors
      float wmax[NWAVE];        // per-wave slice max and candidate floor key (top-k slices)
      uint32_t wfloor[NWAVE];
    } st;
    struct {               // merge phase
      uint32_t keyms[MAXS1];  // slice max keys
      uint32_t ncs[MAXS1];    // slice candidate counts
      float cbs[MAXS1];       // slice base bins
      uint32_t bc[NBC];       // merged weight-bin counts (row-relative)
      uint32_t cnt[WF];       // merged per-code counts: the top codes, later the exact window
    } mg;
    RadixSmem rad;
  } u;
};

// Code window [klo, khi] that must hold the top-p threshold of a top-p-only row, from the merged
// weight-bin counts: bin j holds the entries with floor(-l c BRC) = A_m + j, A_m = floor(-m c BRC),
// so its weights exp2((l - m) c) lie in (2^(hi_j - 1/BRC), 2^hi_j], hi_j = -(A_m + j)/BRC - m c.
// With these bounds and Z (the row normaliser) the threshold bin lies between the first bin whose
// upper-bound cumulative mass can reach P Z and the first whose lower-bound cumulative mass must.
__device__ __forceinline__ bool coarse_window(K1Smem& sm, float m, float c, float P, float Ztot, int V, uint32_t keym, uint32_t& klo,
                              uint32_t& khi) {
  const int tid = threadIdx.x;  // NT == NBC: thread t owns bin t
  const float Am = floorf(-m * (c * BRC));
  const double mc = (double)m * (double)c;
  const double hi = -((double)Am + tid) / BRC - mc;
  const double wmax = exp2(fmin(hi, 0.0)), wmin = exp2(hi - 1.0 / BRC);
  const uint32_t n = sm.u.mg.bc[tid];
  const uint32_t nin = block_inclusive_scan<uint32_t>(n, sm.rs.scan32);
  const double U = block_inclusive_scan<double>((double)n * wmax, sm.rs.scand);
  const double L = block_inclusive_scan<double>((double)n * wmin, sm.rs.scand);
  if (tid == NT - 1) {
    sm.rs.scand[0] = U;
    sm.rs.u[0] = nin;
  }
  __syncthreads();
  const double Utot = sm.rs.scand[0];
  const uint32_t ntot = sm.rs.u[0];
  __syncthreads();
  const double wunder = exp2(fmin(-((double)Am + NBC) / BRC - mc, 0.0));
  const double Ubelow = Utot - U + (double)((uint32_t)V - ntot) * wunder;
  const double t = (double)P * (double)Ztot;
  const double slack = 1e-4;
  const int jlo = block_first(sm.rs, U >= t * (1.0 - slack));
  const int jhi = block_first(sm.rs, fmax(L, (double)Ztot * (1.0 - slack) - Ubelow) >= t * (1.0 + slack));
  if (jhi >= NBC || !(fabsf(Am) <= 0x1p22f)) return false;
  // one bin of slack either side (bin edges are computed in fp32), then the codes of those values
  const float vhi = -(Am + (float)(jlo - 1)) / (BRC * c);
  const float vlo = -(Am + (float)(jhi + 2)) / (BRC * c);
  const uint32_t kh = key32(vhi) >> 16, kl = key32(vlo) >> 16;  // within one code of key16 of those values
  khi = min(kh + 2u, keym);
  klo = kl > 2u ? kl - 2u : 0u;
  return khi >= klo;
}

// Exact per-code counts of [klo, khi] over the whole row by this workgroup (entry i counts code khi - i),
// plus the exact count and fixed-point mass above khi; then the threshold search over the window.
__device__ __forceinline__ bool window_pass(K1Smem& sm, const uint8_t* row, int V, float m, float c, uint32_t klo, uint32_t khi,
                            bool useK, int K, bool useP, float P, double ztot_fixed, uint32_t& thr, float& Z) {
  const int tid = threadIdx.x;
  const int width = (int)(khi - klo + 1);
  uint32_t* h = sm.u.mg.cnt;
  for (int j = tid; j < width; j += NT) h[j] = 0;
  __syncthreads();
  const uint4* src = (const uint4*)row;
  const int nvec = V / BF16::EPV;
  uint32_t acnt = 0;
  unsigned long long amass = 0;
  for (int j0 = 0; j0 < nvec; j0 += NT * FVPT) {
    uint4 v[FVPT];
#pragma unroll
    for (int u = 0; u < FVPT; ++u) {
      const int j = j0 + tid + u * NT;
      if (j < nvec) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < FVPT; ++u) {
      const int j = j0 + tid + u * NT;
      if (j < nvec) {
#pragma unroll
        for (int e = 0; e < BF16::EPV; ++e) {
          const float f = BF16::get(v[u], e);
          const uint32_t key = key16f(f);
          if (key > khi) {
            ++acnt;
            amass += fixmass(fexp2((f - m) * c));
          } else if (key >= klo) {
            atomicAdd(&h[khi - key], 1u);  // descending: entry i is code khi - i
          }
        }
      }
    }
  }
  const uint32_t tc = block_inclusive_scan<uint32_t>(acnt, sm.rs.scan32);
  const unsigned long long tm = block_inclusive_scan<unsigned long long>(amass, sm.rs.scan64);
  if (tid == NT - 1) {
    sm.win[0] = tc;
    sm.rs.scan64[0] = tm;
  }
  __syncthreads();
  const uint32_t above_c = sm.win[0];
  const unsigned long long above_m = sm.rs.scan64[0];
  __syncthreads();
  int sel = -1;
  unsigned long long zsel = 0;
  if (!select_run(h, width, khi, m, c, sm.ss, sm.rs, above_c, above_m, ztot_fixed, useK, K, useP, P, sel, zsel))
    return false;
  thr = khi - (uint32_t)sel;
  Z = (float)((double)zsel * 0x1p-40);
  return true;
}

// The same search for a window too wide to count per code: a window that straddles logit 0 is narrow in
// value but spans thousands of order-preserving codes (they are logarithmic in magnitude), while holding few
// entries.  Those entries (up to LCAP) are listed in LDS; their distinct codes, ranked in descending order,
// with their counts form the histogram the search runs on.  Codes without entries add no count and no mass,
// so the result equals counting every code.  More than LCAP entries: false (the caller takes the radix select).
constexpr int LCAP = 512;
__device__ __forceinline__ bool window_list_pass(K1Smem& sm, const uint8_t* row, int V, float m, float c, uint32_t klo,
                                 uint32_t khi, bool useK, int K, bool useP, float P, double ztot_fixed, uint32_t& thr,
                                 float& Z) {
  static_assert(4 * LCAP <= WF, "list, codes, counts and first-occurrence counts share the count array");
  const int tid = threadIdx.x;
  uint32_t* list = sm.u.mg.cnt;              // entry keys, in arrival order
  uint32_t* ucode = sm.u.mg.cnt + LCAP;      // distinct keys, descending
  uint32_t* ucnt = sm.u.mg.cnt + 2 * LCAP;   // their counts
  uint32_t* fcnt = sm.u.mg.cnt + 3 * LCAP;   // per entry: its key's count at the key's first occurrence, else 0
  if (tid == 0) sm.win[3] = 0;
  __syncthreads();
  const uint4* src = (const uint4*)row;
  const int nvec = V / BF16::EPV;
  uint32_t acnt = 0;
  unsigned long long amass = 0;
  for (int j0 = 0; j0 < nvec; j0 += NT * FVPT) {
    uint4 v[FVPT];
#pragma unroll
    for (int u = 0; u < FVPT; ++u) {
      const int j = j0 + tid + u * NT;
      if (j < nvec) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < FVPT; ++u) {
      const int j = j0 + tid + u * NT;
      if (j < nvec) {
#pragma unroll
        for (int e = 0; e < BF16::EPV; ++e) {
          const float f = BF16::get(v[u], e);
          const uint32_t key = key16f(f);
          if (key > khi) {
            ++acnt;
            amass += fixmass(fexp2((f - m) * c));
          } else if (key >= klo) {
            const uint32_t at = atomicAdd(&sm.win[3], 1u);
            if (at < (uint32_t)LCAP) list[at] = key;
          }
        }
      }
    }
  }
  const uint32_t tc = block_inclusive_scan<uint32_t>(acnt, sm.rs.scan32);
  const unsigned long long tm = block_inclusive_scan<unsigned long long>(amass, sm.rs.scan64);
  if (tid == NT - 1) {
    sm.win[0] = tc;
    sm.rs.scan64[0] = tm;
  }
  __syncthreads();
  const uint32_t above_c = sm.win[0];
  const unsigned long long above_m = sm.rs.scan64[0];
  const uint32_t nl = sm.win[3];
  __syncthreads();
  if (nl > (uint32_t)LCAP) return false;
  // first occurrences of each key with the key's count; then each one's rank among the distinct keys
  for (int e = tid; e < (int)nl; e += NT) {
    const uint32_t k = list[e];
    uint32_t count = 0;
    bool first = true;
    for (int o = 0; o < (int)nl; ++o) {
      count += list[o] == k ? 1u : 0u;
      first = first && !(list[o] == k && o < e);
    }
    fcnt[e] = first ? count : 0u;
  }
  __syncthreads();
  uint32_t nd = 0;
  for (int e = tid; e < (int)nl; e += NT) {
    if (fcnt[e] == 0u) continue;
    const uint32_t k = list[e];
    uint32_t rank = 0;
    for (int o = 0; o < (int)nl; ++o) rank += (fcnt[o] != 0u && list[o] > k) ? 1u : 0u;
    ucode[rank] = k;
    ucnt[rank] = fcnt[e];
    ++nd;
  }
  const uint32_t ndist = block_inclusive_scan<uint32_t>(nd, sm.rs.scan32);
  if (tid == NT - 1) sm.win[2] = ndist;
  __syncthreads();
  const int n = (int)sm.win[2];
  __syncthreads();
  int sel = -1;
  unsigned long long zsel = 0;
  if (!select_run(ucnt, n, khi, m, c, sm.ss, sm.rs, above_c, above_m, ztot_fixed, useK, K, useP, P, sel, zsel, ucode))
    return false;
  thr = ucode[sel];
  Z = (float)((double)zsel * 0x1p-40);
  return true;
}

// Merge of one row (the row-merge kernel, after all its slices are done).  The slice statistics and, for histogram rows,
// thread t's word of each slice's packed code counts are all loaded before any is used, so they cost
// one round trip for up to MB slices; the weight-bin counts are loaded only when the top codes do not
// hold the threshold.
// Kept threshold of a top-k row (K <= KC) from the recorded candidates.  Slice s recorded every finite
// logit with key >= floor_s, so with Fe = max(floor_s, key of the smallest finite value) the merged
// counts of the codes from the row max down to Fe are exact; the selection succeeds when the kept
// threshold lies among them.  A slice whose record overflowed is read again instead.  Also reports
// whether the row can take K5's candidate path.
__device__ __forceinline__ bool cand_select(const Params& p, K1Smem& sm, int r, const uint8_t* row, float m,
                                            const RowParams& q, uint32_t flo, uint32_t& thr, float& Z,
                                            bool& sparse) {
  const int tid = threadIdx.x, S = p.S1;
  const uint32_t kinf = key16f(-INFINITY);
  const uint32_t Fe = max(block_max_u32(sm.rs, tid < S ? flo : 0u), kinf + 1u);
  const uint32_t keym = key16f(m);
  const int nb = (int)(keym - Fe) + 1;  // m is finite, so keym >= Fe
  if (nb > WF) return false;
  uint32_t* cnt = sm.u.mg.cnt;
  for (int j = tid; j < nb; j += NT) cnt[j] = 0;
  // overflowed slices (S <= 64: wave 0 holds one lane per slice); their records are not used
  const bool ovf = tid < S && sm.u.mg.ncs[tid] > (uint32_t)NC;
  const unsigned long long om = __ballot(ovf);
  if (tid == 0) sm.win[2] = (uint32_t)om, sm.win[3] = (uint32_t)(om >> 32);
  if (ovf) sm.u.mg.ncs[tid] = 0;
  __syncthreads();
  const unsigned long long omask = ((unsigned long long)sm.win[3] << 32) | sm.win[2];
  for (int base = 0; base < S * NC; base += NT * 4) {
    uint32_t xs[4];
    float fs[4];
    sparse_load<4>(p, sm.u.mg.ncs, r, Fe, xs, fs, base);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (xs[t] != 0xffffffffu) atomicAdd(&cnt[keym - key16f(fs[t])], 1u);
  }
  for (unsigned long long om2 = omask; om2 != 0; om2 &= om2 - 1) {
    const int so = __ffsll((long long)om2) - 1;
    const int x0 = so * p.L1;
    const int nvs = min(p.L1, p.V - x0) / BF16::EPV;
    const uint4* src = (const uint4*)(row + (size_t)x0 * 2);
    for (int j0 = 0; j0 < nvs; j0 += NT * FVPT) {
      uint4 vv[FVPT];
#pragma unroll
      for (int u = 0; u < FVPT; ++u) {
        const int j = j0 + tid + u * NT;
        if (j < nvs) vv[u] = src[j];
      }
#pragma unroll
      for (int u = 0; u < FVPT; ++u) {
        const int j = j0 + tid + u * NT;
        if (j < nvs) {
          const uint32_t bits = cand_bits_ge(vv[u], Fe);
          if (bits) {
            const uint32_t wv[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll 1
            for (int e = 0; e < BF16::EPV; ++e)
              if (bits & (1u << e)) {
                const uint32_t w = (e >> 1) == 0 ? wv[0] : (e >> 1) == 1 ? wv[1] : (e >> 1) == 2 ? wv[2] : wv[3];
                atomicAdd(&cnt[keym - key16((e & 1) ? (w >> 16) : (w & 0xffffu))], 1u);
              }
          }
        }
      }
    }
  }
  __syncthreads();
  int sel = -1;
  unsigned long long zsel = 0;
  if (!select_run(cnt, nb, keym, m, q.c, sm.ss, sm.rs, 0u, 0ull, 0.0, q.useK, q.K, q.useP, q.P, sel, zsel))
    return false;
  thr = keym - (uint32_t)sel;
  Z = (float)((double)zsel * 0x1p-40);
  sparse = omask == 0 && sm.ss.ck <= (uint32_t)KMAX;  // top-p only shrinks the top-k set
  return true;
}

template <class E, bool RAW>
__device__ __forceinline__ void k1_merge(const Params& p, K1Smem& sm, int r, int b, int i, const RowParams& q) {
  constexpr bool BF = E::KEYBITS == 16;
  constexpr int esize = 16 / E::EPV;
  const int tid = threadIdx.x;
  const int S = p.S1;
  const bool cmode = BF && q.cand;
  const bool hist = BF && q.trunc && !cmode;
  const bool coarse = hist && !q.useK;
  float m = -INFINITY, sum = 0.0f;
  int a = INT_MAX;
  uint32_t fl = 0, flo = 0;
  // Every partial the merge needs is issued before any of them is used (one round trip): the logit at
  // the draft token of every slice is loaded, the one of the slice holding the token is kept.
  uint32_t gv = 0, ncv = 0;
  float cbv = 0.0f;
  if (tid < S) {
    const StatPart* sp = p.st1 + (size_t)r * S + tid;
    m = ldf(&sp->m);
    a = (int)ld32(&sp->arg);
    sum = ldf(&sp->s);
    fl = ld32(&sp->flags);
    gv = ld32(&sp->g);
    if (hist || cmode) ncv = ld32(&p.ncand1[(size_t)r * S + tid]);
    if (cmode) flo = ld32(&sp->floor);
    if (coarse) cbv = ldf(&p.hc1[((size_t)r * S + tid) * HCW + NBC / 2]);
  }
  uint32_t hwv[MB];
  if (hist) {
#pragma unroll
    for (int t = 0; t < MB; ++t) hwv[t] = t < S ? ld32(&p.hw1[((size_t)r * S + t) * (WTOP / 2) + tid]) : 0u;
  }
  int32_t xg = -1;  // this row's draft token (draft-position rows), loaded after the partials are in flight
  if (p.mode == MODE_VERIFY && i != p.k) xg = p.draft_tokens[(size_t)b * p.k + (i < p.k ? i : i - p.k - 1)];
  const int sg = (xg >= 0 && xg < p.V) ? xg / p.L1 : -1;  // slice holding it (-1: none or out of range)
  if (tid < S) {
    if (tid == sg) sm.win[1] = gv;
    if (hist || cmode) sm.u.mg.ncs[tid] = ncv;
    if (coarse) sm.u.mg.cbs[tid] = cbv;
  }
  if (hist) {
    sm.u.mg.cnt[tid] = 0;
    sm.u.mg.cnt[tid + NT] = 0;
  }
  if (coarse) sm.u.mg.bc[tid] = 0;
  if (hist && tid < S) sm.u.mg.keyms[tid] = key16f(m);
  block_stats(sm.rs, m, a, sum, fl, q.c);  // its barriers publish keyms / cbs and the cleared counts
  const bool bad = fl != 0 || !(m > -INFINITY) || m == INFINITY;
  float rlz = 0.0f;
  if constexpr (RAW) {
    if (p.mode == MODE_VERIFY && i <= p.k) {  // the row's raw normaliser, relative to its max
      float rm = -INFINITY, rsm = 0.0f;
      int ra = INT_MAX;
      uint32_t rf = 0;
      if (tid < S) {
        const StatPart* sp = p.st1 + (size_t)r * S + tid;
        rm = ldf(&sp->rmax);
        rsm = ldf(&sp->rsum);
      }
      block_stats(sm.rs, rm, ra, rsm, rf, 1.4426950408889634f);
      rlz = __builtin_amdgcn_logf(rsm) + (rm - m) * 1.4426950408889634f;
    }
  }
  uint32_t thr = 0;
  float Z = sum;
  bool sparse = false;
  if (!bad && q.trunc) {
    bool done = false;
    const double ztot = (double)sum * 0x1p40;
    if (cmode) {
      done = cand_select(p, sm, r, row_ptr(p, b, i, esize), m, q, flo, thr, Z, sparse);
    } else if (BF) {
      const uint32_t keym = key16f(m);
      // merged counts of the row's top WTOP codes: entry co is code keym - co.  Slice s's word tid holds
      // its codes keyms[s] - 2 tid and keyms[s] - 2 tid - 1, i.e. entries off + 2 tid (+1) with
      // off = keym - keyms[s] >= 0.
      uint32_t* cnt = sm.u.mg.cnt;
      for (int s0 = 0; s0 < S; s0 += MB) {
        if (s0 > 0) {
#pragma unroll
          for (int t = 0; t < MB; ++t)
            hwv[t] = s0 + t < S ? ld32(&p.hw1[((size_t)r * S + s0 + t) * (WTOP / 2) + tid]) : 0u;
        }
#pragma unroll
        for (int t = 0; t < MB; ++t) {
          const uint32_t w = hwv[t];
          if (w != 0) {
            const uint32_t co = (keym - sm.u.mg.keyms[s0 + t]) + 2u * tid;
            if (co < (uint32_t)WTOP && (w & 0xffffu)) atomicAdd(&cnt[co], w & 0xffffu);
            if (co + 1u < (uint32_t)WTOP && (w >> 16)) atomicAdd(&cnt[co + 1u], w >> 16);
          }
        }
      }
      __syncthreads();
      int sel = -1;
      unsigned long long zsel = 0;
      if (select_run(cnt, WTOP, keym, m, q.c, sm.ss, sm.rs, 0u, 0ull, ztot, q.useK, q.K, q.useP, q.P, sel, zsel)) {
        thr = keym - (uint32_t)sel;
        Z = (float)((double)zsel * 0x1p-40);
        done = true;
        // Candidate (sparse) path of K5: every slice recorded all its logits within WC codes of its max,
        // so it recorded every kept one if its max is within WC codes of the threshold; the kept set must
        // also be small.
        const uint32_t kept = block_sum_u32(sm.rs, (tid <= sel ? cnt[tid] : 0u) + (tid + NT <= sel ? cnt[tid + NT] : 0u));
        const bool slice_ok = tid >= S || (sm.u.mg.ncs[tid] <= (uint32_t)NC && sm.u.mg.keyms[tid] < thr + (uint32_t)WC);
        const bool all_slices = __syncthreads_and(slice_ok) != 0;
        sparse = kept <= (uint32_t)KMAX && all_slices;
      } else if (coarse) {
        // merged weight bins, row-relative: slice bin j is row bin cbs[s] + j - A_m
        const float Am = floorf(-m * (q.c * BRC));
        for (int s0 = 0; s0 < S; s0 += MB) {
          uint32_t hcv[MB];
#pragma unroll
          for (int t = 0; t < MB; ++t)
            hcv[t] = (s0 + t < S && tid < NBC / 2) ? ld32(&p.hc1[((size_t)r * S + s0 + t) * HCW + tid]) : 0u;
#pragma unroll
          for (int t = 0; t < MB; ++t) {
            const uint32_t w = hcv[t];
            if (w != 0) {
              const float jr = sm.u.mg.cbs[s0 + t] + (float)(2 * tid) - Am;
              if (jr >= 0.0f && jr < (float)NBC && (w & 0xffffu)) atomicAdd(&sm.u.mg.bc[(int)jr], w & 0xffffu);
              if (jr + 1.0f >= 0.0f && jr + 1.0f < (float)NBC && (w >> 16))
                atomicAdd(&sm.u.mg.bc[(int)jr + 1], w >> 16);
            }
          }
        }
        __syncthreads();
        uint32_t klo = 0, khi = 0;
        if (coarse_window(sm, m, q.c, q.P, sum, p.V, keym, klo, khi)) {
          if (khi - klo + 1u <= (uint32_t)WF)
            done = window_pass(sm, row_ptr(p, b, i, esize), p.V, m, q.c, klo, khi, q.useK, q.K, q.useP, q.P, ztot,
                               thr, Z);
          else
            done = window_list_pass(sm, row_ptr(p, b, i, esize), p.V, m, q.c, klo, khi, q.useK, q.K, q.useP, q.P,
                                    ztot, thr, Z);
        }
      }
    }
    if (!done) {
      __syncthreads();
      row_cutoff<E>(sm.u.rad, sm.rs, row_ptr(p, b, i, esize), p.V, m, q.c, q.K, q.P, thr, Z);
    }
  }
  if (tid == 0) {
    RowInfo* ri = p.rinfo + r;
    ri->m = m;
    ri->arg = a;
    ri->Z = Z;
    ri->lz = __builtin_amdgcn_logf(Z);
    ri->fthr = thr == 0 ? -INFINITY : key_value<E>(thr);
    ri->state = bad ? ST_BAD : (sparse ? ST_SPARSE : 0u);
    ri->rlz = rlz;
    ri->gath = sg >= 0 ? __uint_as_float(sm.win[1]) : 0.0f;
  }
}

// 16-byte vector u (runtime index) of a per-thread slice held in registers.
template <int VPT>
__device__ inline uint4 pick_vec(const uint4 (&v)[VPT], int u) {
  uint4 r = v[0];
#pragma unroll
  for (int t = 1; t < VPT; ++t)
    if (u == t) r = v[t];
  return r;
}

// Slots for a wave: every lane asks for cnt < 16 consecutive slots of an LDS counter; one atomic per
// wave reserves them all, and each lane gets its first slot (lanes in order).  All lanes of the wave
// must be active.
__device__ inline uint32_t wave_reserve(uint32_t* counter, uint32_t cnt) {
  uint32_t excl = 0, total = 0;
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    const unsigned long long mk = __ballot((cnt >> bit) & 1u);
    excl += __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u)) << bit;
    total += (uint32_t)__popcll(mk) << bit;
  }
  uint32_t base = 0;
  if (total != 0 && (threadIdx.x & 63) == 0) base = atomicAdd(counter, total);
  return __builtin_amdgcn_readfirstlane(base) + excl;
}

// Bit e set: entry e of a bf16 vector lies within WC codes of the slice max (keyms2: its key in both
// halves); key distances are taken as in the histogram pass.
__device__ inline uint32_t cand_bits(const uint4& v, uint32_t keyms2) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t d2 = sub16x2(keyms2, key16x2(wv[q]));
    bits |= ((d2 & 0xffffu) < (uint32_t)WC ? 1u : 0u) << (2 * q);
    bits |= ((d2 >> 16) < (uint32_t)WC ? 1u : 0u) << (2 * q + 1);
  }
  return bits;
}

// Histogram pass of a truncated bf16 slice (values held in registers), relative to the slice max ms:
// per-code counts of the WTOP codes below ms; top-p-only rows also add the normaliser sum and the
// weight-bin counts (bin floor(-l c BRC) - cbase).  Out-of-range entries go to a per-lane spare bin.
template <int VPT, bool TOPP_ONLY>
__device__ __forceinline__ void k1_hist(K1Smem& sm, const uint4 (&v)[VPT], int nv, int x0, float ms, float c, float cbase,
                        float& sum) {
  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t keyms = key16f(ms);
  const uint32_t keyms2 = keyms * 0x10001u;
  const uint32_t spare2 = (WTOP + lane) * 0x10001u;
  const uint32_t spare_c = NBC + lane;
  const uint32_t copy4 = (lane & (NCOPY - 1)) << 2;  // byte offset of this lane's copy of a bin
  uint8_t* const hcb = (uint8_t*)sm.u.st.hc;
  const float cb = c * BRC;
  const float nmc = -ms * c;
  uint32_t cmask = 0;  // bit u: vector u holds a candidate (an entry within WC codes of the slice max)
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j < nv) {
      const uint32_t wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      uint32_t dmin = 0xffffffffu;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t d2 = min16x2(sub16x2(keyms2, key16x2(wv[q])), spare2);
        atomicAdd(&sm.u.st.hw[d2 & 0xffffu], 1u);
        atomicAdd(&sm.u.st.hw[d2 >> 16], 1u);
        dmin = min16x2(dmin, d2);
        if (TOPP_ONLY) {
          const float f0 = __uint_as_float(wv[q] << 16), f1 = __uint_as_float(wv[q] & 0xffff0000u);
          sum += fexp2(fmaf(f0, c, nmc));
          sum += fexp2(fmaf(f1, c, nmc));
          const uint32_t j0 = min(__float2uint_rz(fmaf(f0, -cb, -cbase)), spare_c);
          const uint32_t j1 = min(__float2uint_rz(fmaf(f1, -cb, -cbase)), spare_c);
          atomicAdd((uint32_t*)(hcb + ((j0 * (NCOPY * 4)) | copy4)), 1u);
          atomicAdd((uint32_t*)(hcb + ((j1 * (NCOPY * 4)) | copy4)), 1u);
        }
      }
      if (min(dmin & 0xffffu, dmin >> 16) < (uint32_t)WC) cmask |= 1u << u;
    }
  }
  // Candidates: the logits within WC codes of the slice max (index and raw bits).  The vectors flagged
  // above are staged in LDS, then one thread per staged vector appends its candidates.  More than
  // NFLAG staged vectors, or more than NC candidates, leave ncand above NC: the slice then has no
  // usable candidate list.
  if (__ballot(cmask != 0) != 0) {
    uint32_t at = wave_reserve(&sm.u.st.nflag, (uint32_t)__popc(cmask));
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      if (cmask & (1u << u)) {
        if (at < (uint32_t)NFLAG) {
          sm.u.st.fvec[at] = v[u];
          sm.u.st.fidx[at] = (uint32_t)(tid + u * NT);
        }
        ++at;
      }
    }
  }
  __syncthreads();
  const uint32_t nflag = sm.u.st.nflag;
  if (nflag > (uint32_t)NFLAG) {
    if (tid == 0) sm.u.st.ncand = NC + 1;
  } else if ((uint32_t)(tid & ~63) < nflag) {  // waves holding a staged vector
    const bool mine = (uint32_t)tid < nflag;
    const uint4 vv = mine ? sm.u.st.fvec[tid] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t bits = mine ? cand_bits(vv, keyms2) : 0u;
    const int xb = x0 + (mine ? (int)sm.u.st.fidx[tid] : 0) * BF16::EPV;
    uint32_t c = wave_reserve(&sm.u.st.ncand, (uint32_t)__popc(bits));
    const uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < BF16::EPV; ++e) {
      if (bits & (1u << e)) {
        const uint32_t h = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffffu);
        if (c < (uint32_t)NC) sm.u.st.cand[c] = ((unsigned long long)(xb + e) << 16) | h;
        ++c;
      }
    }
  }
}

// Exclusive prefix over the lanes of a wave of per-lane counts cnt < 16, and their total.
__device__ inline uint32_t wave_excl_prefix(uint32_t cnt, uint32_t& total) {
  uint32_t excl = 0;
  total = 0;
#pragma unroll
  for (int bit = 0; bit < 4; ++bit) {
    const unsigned long long mk = __ballot((cnt >> bit) & 1u);
    excl += __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u)) << bit;
    total += (uint32_t)__popcll(mk) << bit;
  }
  return excl;
}

// Largest 16-bit key t with at least kth lanes of the wave holding a key >= t (the wave's kth largest
// key); bit by bit from the top, one ballot each.
__device__ inline uint32_t wave_kth_key(uint32_t key, int kth) {
  uint32_t t = 0;
#pragma unroll
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    if (__popcll(__ballot(key >= c)) >= (unsigned)kth) t = c;
  }
  return t;
}

// Candidates of a top-k slice: every logit with key >= fe, collected (index << 16 | bits) in LDS; the
// item writes them to the slice's record in one coalesced store.  vm holds the vector maxima.  Each wave stages its own vectors whose maximum
// reaches fe in its LDS region, then one lane per staged vector appends that vector's candidates, with
// one slot reservation per wave.  A wave with more than NFW such vectors sets `over`; more than NC
// candidates leave ncand above NC.  Either way the slice has no usable record.
template <int VPT>
__device__ __forceinline__ void k1_capture(const Params& p, K1Smem& sm, const uint4 (&v)[VPT], const float (&vm)[VPT],
                                           int x0, int r, int s, uint32_t fe) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float fcand = key16_value(fe);
  uint32_t cmask = 0;
#pragma unroll
  for (int u = 0; u < VPT; ++u) cmask |= (vm[u] >= fcand ? 1u : 0u) << u;
  uint32_t total;
  uint32_t at = wave_excl_prefix((uint32_t)__popc(cmask), total);
  if (total == 0) return;
  if (total > (uint32_t)NFW) {
    if (lane == 0) sm.u.st.over = 1;
    return;
  }
  uint4* fv = sm.u.st.fvec + wave * NFW;
  uint32_t* fi = sm.u.st.fidx + wave * NFW;
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    if (cmask & (1u << u)) {
      fv[at] = v[u];
      fi[at] = (uint32_t)(tid + u * NT);
      ++at;
    }
  }
  // the wave reads back what its lanes wrote: LDS operations of one wave complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const bool mine = (uint32_t)lane < total;
  const uint4 vv = mine ? fv[lane] : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t bits = mine ? cand_bits_ge(vv, fe) : 0u;
  const int xb = x0 + (mine ? (int)fi[lane] : 0) * BF16::EPV;
  uint32_t c = wave_reserve(&sm.u.st.ncand, (uint32_t)__popc(bits));
  const uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int e = 0; e < BF16::EPV; ++e) {
    if (bits & (1u << e)) {
      const uint32_t h = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffffu);
      if (c < (uint32_t)NC) sm.u.st.cand[c] = ((unsigned long long)(xb + e) << 16) | h;
      ++c;
    }
  }
}

// One K1 work item: slice s of logit row r.
template <class E, int VPT, bool RAW>
__device__ __forceinline__ void k1_item(const Params& p, K1Smem& sm, int item, int r, int s) {
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  constexpr bool BF = E::KEYBITS == 16;
  const int tid = threadIdx.x;
  const int b = r / p.rows, i = r - b * p.rows;
  const int x0 = s * p.L1;
  const int nv = min(p.L1, p.V - x0) / EPV;
  const uint4* src = (const uint4*)(row_ptr(p, b, i, esize) + (size_t)x0 * esize);
  SV_TRACE_AT(p, item, 0);

  // the slice's loads go out first: nothing in them waits for the sampling parameters
  uint4 v[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j < nv) v[u] = src[j];
  }
  const RowParams q = row_params(p, b);
  // draft-position rows also record their logit at the draft token (used by the accept chain)
  float gval = 0.0f;
  if (p.mode == MODE_VERIFY && i != p.k) {
    const int xg = p.draft_tokens[(size_t)b * p.k + (i < p.k ? i : i - p.k - 1)];
    if (tid == 0 && xg >= x0 && xg < x0 + nv * EPV) gval = E::load1(row_ptr(p, b, i, esize), xg);
  }
  float m = -INFINITY, sum = 0.0f;
  int a = INT_MAX;
  uint32_t fl = 0, flo = 0;
  if (q.greedy) {
    // lowest argmax; NaN never compares greater, so it is flagged separately
    bool nan = false;
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int j = tid + u * NT;
      if (j < nv) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float f = E::get(v[u], e);
          nan = nan | (f != f);  // bitwise: no branch per entry
          if (f > m) {
            m = f;
            a = x0 + j * EPV + e;
          }
        }
      }
    }
    fl = (nan || m == INFINITY) ? 1u : 0u;
  } else if (BF && q.cand) {
    // Top-k row with K <= KC: no histograms.  The slice records every logit at or above a floor: the
    // smallest over the waves of each wave's (KC / NWAVE)-th largest thread maximum.  At least KC
    // distinct logits reach it, so the slice's top KC logits are all recorded, and the merge selects
    // the kept threshold from the records.
    const int lane = tid & 63, wave = tid >> 6;
    float vm[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int j = tid + u * NT;
      vm[u] = -INFINITY;
      if (j < nv) {
        float x = E::get(v[u], 0);
#pragma unroll
        for (int e = 1; e < EPV; ++e) x = nan_max(x, E::get(v[u], e));
        vm[u] = x;
        m = nan_max(m, x);
      }
    }
    SV_TRACE_AT(p, item, 1);
    if (tid == 0) {
      sm.u.st.ncand = 0;
      sm.u.st.over = 0;
    }
    float wm = m;
    wm = wave_nan_max(wm);
    const uint32_t wf = wave_kth_key(key16f(m), KC / NWAVE);
    if (lane == 0) {
      sm.u.st.wmax[wave] = wm;
      sm.u.st.wfloor[wave] = wf;
    }
    __syncthreads();
    float ms = sm.u.st.wmax[0];
    uint32_t fk = sm.u.st.wfloor[0];
#pragma unroll
    for (int w = 1; w < NWAVE; ++w) {
      ms = nan_max(ms, sm.u.st.wmax[w]);
      fk = min(fk, sm.u.st.wfloor[w]);
    }
    const uint32_t kinf = key16f(-INFINITY);
    if (ms > -INFINITY && ms < INFINITY) {  // not NaN, +inf or an all -inf slice
      flo = max(fk, kinf);
      k1_capture<VPT>(p, sm, v, vm, x0, r, s, max(flo, kinf + 1u));
    }
    m = ms;
    if (!(m == m) || m == INFINITY) fl = 1u;
  } else {
    // NaN-propagating max: a NaN or +inf anywhere shows in the row max
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int j = tid + u * NT;
      if (j < nv) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) m = nan_max(m, E::get(v[u], e));
      }
    }
    SV_TRACE_AT(p, item, 1);
    if (!(BF && q.trunc)) {
      // the whole-row normaliser, unless top-k fixes the kept set (fp32 truncated rows: radix select)
      if (!q.useK && m > -INFINITY) {
        const float nmc = -m * q.c;  // exp2(l c - m c): one fma per logit
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          const int j = tid + u * NT;
          if (j < nv) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) sum += fexp2(fmaf(E::get(v[u], e), q.c, nmc));
          }
        }
      }
    } else if constexpr (BF) {
      // histograms relative to the slice max
      const bool topp_only = !q.useK;
      sm.u.st.hw[tid] = 0;
      sm.u.st.hw[tid + NT] = 0;
      if (topp_only) {
#pragma unroll
        for (int q = 0; q < NCOPY; ++q) sm.u.st.hc[tid + q * NT] = 0;  // the bins, not the spares
      }
      if (tid == 0) {
        sm.u.st.ncand = 0;
        sm.u.st.nflag = 0;
      }
      const float ms = block_nan_max(sm.rs, m);
      const float cbase = floorf(-ms * (q.c * BRC));
      if (ms > -INFINITY && ms < INFINITY) {  // not NaN, +inf or an all -inf slice
        if (topp_only)
          k1_hist<VPT, true>(sm, v, nv, x0, ms, q.c, cbase, sum);
        else
          k1_hist<VPT, false>(sm, v, nv, x0, ms, q.c, cbase, sum);
      }
      m = ms;  // the sums above are relative to the slice max
      __syncthreads();
      uint32_t* hw = p.hw1 + ((size_t)r * p.S1 + s) * (WTOP / 2);
      pst32(&hw[tid], sm.u.st.hw[2 * tid] | (sm.u.st.hw[2 * tid + 1] << 16));  // WTOP / 2 == NT
      const uint32_t nc = sm.u.st.ncand;
      if (tid < (int)min(nc, (uint32_t)NC)) {
        unsigned long long* cd = p.cand1 + ((size_t)r * p.S1 + s) * NC + tid;
        *cd = sm.u.st.cand[tid];
      }
      if (tid == 0) pst32(&p.ncand1[(size_t)r * p.S1 + s], nc);
      if (topp_only) {
        uint32_t* hc = p.hc1 + ((size_t)r * p.S1 + s) * HCW;
        if (tid < NBC / 2) {
          uint32_t c0 = 0, c1 = 0;
#pragma unroll
          for (int q = 0; q < NCOPY; ++q) {
            c0 += sm.u.st.hc[2 * tid * NCOPY + q];
            c1 += sm.u.st.hc[(2 * tid + 1) * NCOPY + q];
          }
          pst32(&hc[tid], c0 | (c1 << 16));
        }
        if (tid == 0) pstf(&hc[NBC / 2], cbase);
      }
    }
    if (!(m == m) || m == INFINITY) fl = 1u;
  }
  // raw logprobs: the sum of exp(l - slice max) of target rows, whatever the sampling parameters
  float rmax = -INFINITY, rsum = 0.0f;
  if constexpr (RAW) {
    if (p.mode == MODE_VERIFY && i <= p.k) {
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) {
#pragma unroll
          for (int e = 0; e < EPV; ++e) rmax = nan_max(rmax, E::get(v[u], e));
        }
      }
      if (rmax > -INFINITY) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          const int j = tid + u * NT;
          if (j < nv) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) rsum += fexp2((E::get(v[u], e) - rmax) * 1.4426950408889634f);
          }
        }
      }
      int ra = INT_MAX;
      uint32_t rf = 0;
      block_stats(sm.rs, rmax, ra, rsum, rf, 1.4426950408889634f);
    }
  }
  block_stats(sm.rs, m, a, sum, fl, q.c);
  if (tid == 0) {
    StatPart* sp = p.st1 + (size_t)r * p.S1 + s;
    if (RAW) {
      pstf(&sp->rmax, rmax);
      pstf(&sp->rsum, rsum);
    }
    pstf(&sp->m, m);
    pst32(&sp->arg, (uint32_t)a);
    pstf(&sp->s, sum);
    pst32(&sp->flags, fl);
    pstf(&sp->g, gval);
    pst32(&sp->floor, flo);
    if (BF && q.cand) pst32(&p.ncand1[(size_t)r * p.S1 + s], sm.u.st.over ? (uint32_t)NC + 1u : sm.u.st.ncand);
  }
  if (BF && q.cand) {  // the candidates collected in LDS (block_stats' barriers order them), coalesced
    const uint32_t nc = sm.u.st.ncand;
    if (tid < (int)min(nc, (uint32_t)NC)) p.cand1[((size_t)r * p.S1 + s) * NC + tid] = sm.u.st.cand[tid];
  }
  SV_TRACE_AT(p, item, 2);
}

// Wide slices with raw logprobs need more registers than seven workgroups per CU leave (they would spill).
template <class E, int VPT, bool RAW>
__global__ __launch_bounds__(NT, (RAW && VPT > VPT1) ? OCC1 - 1 : OCC1) void k1_stats(Params p) {
  __shared__ K1Smem sm;
  int r, s;
  item_rs(blockIdx.x, p.R, p.S1, r, s);
  k1_item<E, VPT, RAW>(p, sm, blockIdx.x, r, s);
}

// Row merges: one workgroup per logit row, launched after every slice has written its partials.  Kept
// apart from the slices so that long merges (top-p rows that count a code window over the whole row)
// neither hold slice slots nor pile up on one XCD: workgroups are handed to the XCDs in order, so one
// XCD full of long merges stalls the hand-out to all of them.
template <class E, bool RAW>
__global__ __launch_bounds__(NT) void k1_rows(Params p) {
  __shared__ K1Smem sm;
  const int r = blockIdx.x;
  const int b = r / p.rows, i = r - b * p.rows;
  const RowParams q = row_params(p, b);
  // Re-arm the batch row's arrival counter of the next kernel (K5 or the tree kernel): this kernel ends
  // before that one starts, so every call starts from zero whatever the workspace held.
  if (i == 0 && threadIdx.x == 0) p.cnt5[b] = 0u;
  SV_TRACE_AT(p, (size_t)r * p.S1, 3);
  k1_merge<E, RAW>(p, sm, r, b, i, q);
  SV_TRACE_AT(p, (size_t)r * p.S1, 7);
}

// ---------------------------------------------------------------------------------------------
// K5: accept chain, alpha, residual / bonus draw, outputs.
// ---------------------------------------------------------------------------------------------
struct K5Smem {
  RedSmem rs;
  float m[MAXROWS], Z[MAXROWS], lz[MAXROWS], fthr[MAXROWS], gath[MAXROWS], rlz[MAXROWS];
  int32_t arg[MAXROWS];
  uint32_t state[MAXROWS];
  int32_t tok[MAXK];
  float u[MAXK];
  float wacc[MAXK][NWAVE];
  int32_t n;
  // sparse path
  int32_t hidx[HT];
  float hlq[HT];
  uint32_t ncs[MAXS1], ncs2[MAXS1];  // candidate counts per slice: target row, draft row
  unsigned long long asum[NWAVE];
};

// p(x) = exp2((l - m) c - log2 Z) on the kept entries, 0 below the kept threshold.
__device__ inline float kept_p(float f, float m, float c, float lz, float fthr) {
  return f >= fthr ? fexp2(fmaf(f - m, c, -lz)) : 0.0f;
}

// Exponential-race key w / E2 with E2 = -log2 U (see exp_race_E2): a reciprocal and a product; keys
// are only compared with each other.
__device__ inline float race_key(float w, uint32_t word) { return w * __builtin_amdgcn_rcpf(exp_race_E2(word)); }

// Race candidate update: larger key wins, the lower index on an exact tie (selects, no branch).
__device__ inline void race_take(float& best, int& bidx, float& bval, float key, int idx, float val) {
  const bool take = (key > best) | ((key == best) & (idx < bidx));  // bitwise: no short-circuit branches
  best = take ? key : best;
  bidx = take ? idx : bidx;
  bval = take ? val : bval;
}

// Race key of weight w with stream word `word`, or -1 (never taken: keys of positive weights are positive)
// when w is 0: computed for every entry of a group, so that no entry branches.
__device__ inline float race_key_or_none(float w, uint32_t word) {
  return w > 0.0f ? race_key(w, word) : -1.0f;
}

// Workgroup race winner (key, index, logit) into every thread.
__device__ __forceinline__ void block_race(RedSmem& rs, float& best, int& bidx, float& bval) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#define SV_RACE_STEP(C) \
  race_take(best, bidx, bval, dpp_mov_f<C>(best), (int)dpp_mov_u<C>((uint32_t)bidx), dpp_mov_f<C>(bval))
  SV_ROW_STEPS(SV_RACE_STEP);
#undef SV_RACE_STEP
  {
    float b0 = row_f(best, 0), v0 = row_f(bval, 0), b2 = row_f(best, 2), v2 = row_f(bval, 2);
    int i0 = (int)row_u((uint32_t)bidx, 0), i2 = (int)row_u((uint32_t)bidx, 2);
    race_take(b0, i0, v0, row_f(best, 1), (int)row_u((uint32_t)bidx, 1), row_f(bval, 1));
    race_take(b2, i2, v2, row_f(best, 3), (int)row_u((uint32_t)bidx, 3), row_f(bval, 3));
    race_take(b0, i0, v0, b2, i2, v2);
    best = b0;
    bidx = i0;
    bval = v0;
  }
  if (lane == 0) {
    rs.f[wave] = best;
    rs.i[wave] = bidx;
    rs.g[wave] = bval;
  }
  __syncthreads();
  best = rs.f[0];
  bidx = rs.i[0];
  bval = rs.g[0];
  for (int w = 1; w < NWAVE; ++w) race_take(best, bidx, bval, rs.f[w], rs.i[w], rs.g[w]);
  __syncthreads();
}

// Gumbel-max candidates over w(x) = exp2((l - m) c) on the kept entries of one 16-byte vector
// (stream tag, b, position j).  Groups of four entries with no kept entry draw nothing.
template <class E>
__device__ __forceinline__ void gumbel_vec(const uint4& v, int xbase, float m, float c, float fthr, uint32_t tag, uint32_t b,
                           uint32_t j, const Params& p, float& best, int& bidx, float& bval) {
#pragma unroll
  for (int g = 0; g < E::EPV; g += 4) {
    float w[4];
    bool any = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float f = E::get(v, g + e);
      w[e] = f >= fthr ? fexp2((f - m) * c) : 0.0f;
      any = any | (w[e] > 0.0f);
    }
    if (any) {
      const int x = xbase + g;
      const uint4 w4 = philox10_uk(make_uint4((uint32_t)x >> 2, b, (tag << 24) | j, p.offset), p.key0, p.key1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (w[e] > 0.0f) {
          const uint32_t word = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
          race_take(best, bidx, bval, race_key(w[e], word), x + e, E::get(v, g + e));
        }
      }
    }
  }
}

// Raw logprob of a committed token with logit l at position i: ln of the softmax of the unprocessed row.
__device__ inline float raw_lp(const K5Smem& sm, int i, float l) {
  return (l - sm.m[i]) - sm.rlz[i] * 0.6931471805599453f;
}

__device__ __forceinline__ void write_sentinel(const Params& p, int b) {
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
    if (p.raw_logprobs) p.raw_logprobs[(size_t)b * (k + 1) + tid] = __builtin_nanf("");
  }
  if (tid < k) p.alpha[(size_t)b * k + tid] = __builtin_nanf("");
  if (tid == 0) p.accept_len[b] = 0;
}

template <class E>
__device__ __forceinline__ void k5_finalize(const Params& p, K5Smem& sm, int b, bool ok, const RowParams& q) {
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
      if (sm.tok[i] != sm.arg[i]) {
        n = i;
        break;
      }
    const int y = sm.arg[n];
    if (tid < k) p.alpha[(size_t)b * k + tid] = (sm.arg[tid] == sm.arg[k + 1 + tid]) ? 1.0f : 0.0f;
    if (tid <= k) {
      const int t = tid < n ? sm.tok[tid] : (tid == n ? y : -1);
      p.tokens[(size_t)b * (k + 1) + tid] = t;
      p.logprobs[(size_t)b * (k + 1) + tid] = 0.0f;
      if (p.raw_logprobs)  // the committed token of row n is its argmax, whose logit is the row max
        p.raw_logprobs[(size_t)b * (k + 1) + tid] =
            tid < n ? raw_lp(sm, tid, sm.gath[tid]) : (tid == n ? raw_lp(sm, n, sm.m[n]) : 0.0f);
    }
    if (tid == 0) p.accept_len[b] = n + 1;
    return;
  }
  const int n = sm.n;
  const int lane = tid & 63, wave = tid >> 6;
  // slice partials: thread t reads slices t, t + NT, ... (one round of loads when S <= NT)
  float best = 0.0f, bval = 0.0f;
  int bidx = INT_MAX;
  float al[MAXK];
#pragma unroll
  for (int i = 0; i < MAXK; ++i) al[i] = 0.0f;
  for (int sl = tid; sl < S; sl += NT) {
    const FinalPart* fp = p.fin5 + (size_t)b * S + sl;
    race_take(best, bidx, bval, ldf(&fp->key), (int)ld32(&fp->idx), ldf(&fp->val));
#pragma unroll
    for (int i = 0; i < MAXK; ++i)
      if (i < k) al[i] += ldf(&fp->alpha[i]);
  }
#pragma unroll
  for (int i = 0; i < MAXK; ++i) {
    if (i < k) {
      const float v = wave_sum(al[i]);
      if (lane == 0) sm.wacc[i][wave] = v;
    }
  }
  block_race(sm.rs, best, bidx, bval);  // also orders the wacc writes before the reads below
  if (tid < k) {
    float v = 0.0f;
    for (int w = 0; w < NWAVE; ++w) v += sm.wacc[tid][w];
    p.alpha[(size_t)b * k + tid] = v;
  }
  int y = bidx;
  float yv = bval;
  if (y == INT_MAX && n < k) {
    // The residual mass vanished in fp32 (rounding only): draw from p_n over the whole row.
    const uint4* row = (const uint4*)row_ptr(p, b, n, esize);
    float bb = 0.0f, bv = 0.0f;
    int bi = INT_MAX;
    for (int j = tid; j < p.V / E::EPV; j += NT)
      gumbel_vec<E>(row[j], j * E::EPV, sm.m[n], q.c, sm.fthr[n], 1u, (uint32_t)b, (uint32_t)n, p, bb, bi, bv);
    block_race(sm.rs, bb, bi, bv);
    y = bi;
    yv = bv;
  }
  if (y < 0 || y >= p.V) return write_sentinel(p, b);  // no candidate: not reachable for a valid row
  if (p.mode == MODE_SAMPLE) {
    if (tid == 0) {
      p.tokens[b] = y;
      p.logprobs[b] = (yv - sm.m[0]) / q.T - logf(sm.Z[0]);
    }
    return;
  }
  if (tid <= k) {
    int t = -1;
    float lp = 0.0f, rlp = 0.0f;
    if (tid <= n) {
      t = tid < n ? sm.tok[tid] : y;
      const float l = tid < n ? sm.gath[tid] : yv;
      lp = (l - sm.m[tid]) / q.T - logf(sm.Z[tid]);
      rlp = raw_lp(sm, tid, l);
    }
    p.tokens[(size_t)b * (k + 1) + tid] = t;
    p.logprobs[(size_t)b * (k + 1) + tid] = lp;
    if (p.raw_logprobs) p.raw_logprobs[(size_t)b * (k + 1) + tid] = rlp;
  }
  if (tid == 0) p.accept_len[b] = n + 1;
}

template <class E, int VPT>
__device__ inline void load_slice(const uint8_t* row, int x0, int nv, uint4 (&v)[VPT]) {
  constexpr int esize = 16 / E::EPV;
  const uint4* src = (const uint4*)(row + (size_t)x0 * esize);
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = threadIdx.x + u * NT;
    if (j < nv) v[u] = src[j];
  }
}

// Gumbel-max race over the 4-entry groups of a slice held in registers, one vector at a time (the
// Philox rounds of different groups are not interleaved, which keeps register use flat).  Weights:
// RESID: r(x) = max(p(x) - q(x), 0) of a target / draft pair; otherwise w(x) = exp2((l - m) c) on the
// kept entries of one row.  Either is 0 wherever the (target) logit is below the kept threshold tt, so
// a vector with no entry >= tt is skipped before any exp2.  Stream (tag, b, position j).  The winner's
// (target) logit rides along.  ALPHA (with RESID): also adds min(p, q) of every entry to acc -- the
// alpha partial sum of the position, from the same p and q.
template <class E, int VPT, bool RESID, bool ALPHA = false, bool TRUNC = true>
__device__ __forceinline__ void race_slice(const Params& p, const uint4 (&va)[VPT], const uint4 (&vb)[VPT], int x0, int nv, float c,
                           float mt, float lt, float tt, float md, float ld, float td, uint32_t tag, uint32_t sb,
                           uint32_t sj, float& best, int& bidx, float& bval, float* acc = nullptr) {
  constexpr int EPV = E::EPV;
  const int tid = threadIdx.x;
  // This thread's best so far.  Its entries come in increasing index order, so a strict compare keeps the
  // lowest index among equal keys; entries without weight are never taken, the start value -0.5 lies below
  // every real key (>= 0), and the caller's candidate is merged with the full tie rule at the end.  TRUNC
  // false: an untruncated batch row (thresholds -inf), whose entries need no kept test.
  float lb = -0.5f, lv = 0.0f;
  int li = INT_MAX;
#pragma unroll 1
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j >= nv) continue;
    const uint4 a = pick_vec<VPT>(va, u);
    if (TRUNC) {  // untruncated rows keep every entry (thresholds -inf): no test
      bool kept = false;
#pragma unroll
      for (int e = 0; e < EPV; ++e) kept = kept | (E::get(a, e) >= tt);  // bitwise: no branch per entry
      if (!kept) continue;
    }
    const uint4 bv = RESID ? pick_vec<VPT>(vb, u) : a;
#pragma unroll 1
    for (int g = 0; g < EPV; g += 4) {
      float w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ft = E::get(a, g + e);
        if (RESID) {
          const float fd = E::get(bv, g + e);
          const float pp = TRUNC ? kept_p(ft, mt, c, lt, tt) : fexp2(fmaf(ft - mt, c, -lt));
          const float qq = TRUNC ? kept_p(fd, md, c, ld, td) : fexp2(fmaf(fd - md, c, -ld));
          if (ALPHA) *acc += fminf(pp, qq);
          w[e] = pp - qq;
        } else {
          w[e] = (!TRUNC || ft >= tt) ? fexp2((ft - mt) * c) : 0.0f;
        }
      }
      // no positive weight in the group: no draw (the largest of the four, one compare)
      if (!(fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])) > 0.0f)) continue;
      const int x = x0 + j * EPV + g;
      const uint4 w4 = philox10_uk(make_uint4((uint32_t)x >> 2, sb, (tag << 24) | sj, p.offset), p.key0, p.key1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
        const float key = race_key(w[e], word);
        const bool take = (w[e] > 0.0f) & (key > lb);  // no weight: no candidate; a later index never wins a tie
        lb = take ? key : lb;
        li = take ? x + e : li;
        lv = take ? E::get(a, g + e) : lv;
      }
    }
  }
  race_take(best, bidx, bval, lb, li, lv);
}

// Alpha partial sum of draft position i over this slice (va / vb: its target / draft slices), and the
// residual race if i is the first rejected position.  Off the drawing position min(p, q) is taken on the
// log2 weights, so it costs one exp2; at it, the race computes p and q anyway and alpha takes their
// minimum.  TRUNC: the batch row is truncated (some entries have p = 0); then a vector without a kept
// target entry adds nothing and is skipped.
template <class E, int VPT, bool TRUNC>
__device__ __forceinline__ void k5_position(const Params& p, K5Smem& sm, int b, int i, int n, int x0, int nv, float c,
                            const uint4 (&va)[VPT], const uint4 (&vb)[VPT], float& best, int& bidx, float& bval) {
  constexpr int EPV = E::EPV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = p.k;
  const float mt = sm.m[i], md = sm.m[k + 1 + i];
  const float lt = sm.lz[i], ld = sm.lz[k + 1 + i];
  const float tt = sm.fthr[i], td = sm.fthr[k + 1 + i];
  float acc = 0.0f;
  if (i == n) {
    // the drawing position: alpha and the residual race in one pass over p and q
    race_slice<E, VPT, true, true, TRUNC>(p, va, vb, x0, nv, c, mt, lt, tt, md, ld, td, 1u, (uint32_t)b, (uint32_t)n, best,
                                   bidx, bval, &acc);
    acc = wave_sum(acc);
    if (lane == 0) sm.wacc[i][wave] = acc;
    return;
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    bool live = j < nv;
    if (TRUNC) {
      bool any = false;
#pragma unroll
      for (int e = 0; e < EPV; ++e) any = any | (E::get(va[u], e) >= tt);  // bitwise: no branch per entry
      live = live & any;
    }
    if (live) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float ft = E::get(va[u], e), fd = E::get(vb[u], e);
        float lp = fmaf(ft - mt, c, -lt), lq = fmaf(fd - md, c, -ld);  // log2 p, log2 q
        if (TRUNC) {
          lp = ft >= tt ? lp : -INFINITY;
          lq = fd >= td ? lq : -INFINITY;
        }
        acc += fexp2(fminf(lp, lq));
      }
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) sm.wacc[i][wave] = acc;
}

template <class E, int VPT, bool TRUNC>
__device__ __forceinline__ void k5_positions(const Params& p, K5Smem& sm, int b, int n, int x0, int nv, float c,
                                             uint4 (&a0)[VPT], uint4 (&b0)[VPT], float& best, int& bidx, float& bval) {
  constexpr int esize = 16 / E::EPV;
  const int k = p.k;
  for (int i = 0; i < k; ++i) {
    k5_position<E, VPT, TRUNC>(p, sm, b, i, n, x0, nv, c, a0, b0, best, bidx, bval);
    if (i + 1 < k) {
      load_slice<E, VPT>(row_ptr(p, b, i + 1, esize), x0, nv, a0);
      load_slice<E, VPT>(row_ptr(p, b, k + 2 + i, esize), x0, nv, b0);
    }
  }
}

// One K5 work item: slice s of batch row b.
// ---------------------------------------------------------------------------------------------
// K5 candidate (sparse) path: a truncated batch row whose every logit row kept at most KMAX entries,
// all of them among the candidates K1 recorded, is finished from those candidates, one workgroup per
// draft position: the same weights, accept chain, alpha and Philox race keys as the streaming path,
// without re-reading the rows.  bf16 rows only.
// ---------------------------------------------------------------------------------------------

__device__ inline uint32_t hslot(uint32_t x) { return (x * 2654435761u) >> (32 - 11); }  // HT == 2^11
__device__ inline uint32_t thr_key(float fthr) { return fthr == -INFINITY ? 0u : key16f(fthr); }

// Race over target candidates with weights exp2((l - m) c) (a plain draw from that row's kept set).
template <int NSLOT>
__device__ inline void sparse_plain_race(const Params& p, const uint32_t (&xs)[NSLOT], const float (&fs)[NSLOT],
                                         float m, float c, uint32_t tag, uint32_t sb, uint32_t sj, float& best,
                                         int& bidx, float& bval) {
#pragma unroll
  for (int t = 0; t < NSLOT; ++t) {
    if (xs[t] == 0xffffffffu) continue;
    const float w = fexp2((fs[t] - m) * c);
    if (w > 0.0f) {
      const uint4 w4 = philox10_uk(make_uint4(xs[t] >> 2, sb, (tag << 24) | sj, p.offset), p.key0, p.key1);
      const uint32_t qq = xs[t] & 3u;
      race_take(best, bidx, bval, race_key(w, qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w), (int)xs[t],
                fs[t]);
    }
  }
}

// Position i of a candidate-path batch row (one workgroup per position): alpha_i for i < k, and the
// token draw where this position is the one that draws (the first rejection n, or the bonus position
// k when every draft was accepted), with the row's outputs.
template <class E>
__device__ __forceinline__ void k5_sparse(const Params& p, K5Smem& sm, int b, int n, int i, const RowParams& q) {
  constexpr int NSLOT = 4;  // slots per thread per pass: NT * NSLOT = 1024 slots
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = p.k, S = p.S1;
  const int nslots = S * NC;
  const bool pair = i < k;
  const bool draw = pair ? i == n : n == k;
  if (!pair && !draw) return;
  const int rt = i, rd = k + 1 + i;
  const int Rt = b * p.rows + rt, Rd = b * p.rows + rd;
  // candidate counts of both rows in one round trip; the index -> log2 q table cleared meanwhile
  if (tid < S) sm.ncs[tid] = ld32(&p.ncand1[(size_t)Rt * S + tid]);
  if (pair && tid >= 64 && tid < 64 + S) sm.ncs2[tid - 64] = ld32(&p.ncand1[(size_t)Rd * S + tid - 64]);
  if (pair)
    for (int j = tid; j < HT; j += NT) sm.hidx[j] = -1;
  __syncthreads();
  const float mt = sm.m[rt], lt = sm.lz[rt];
  const uint32_t kt = thr_key(sm.fthr[rt]);
  uint32_t xt[NSLOT];
  float ft[NSLOT];
  sparse_load<NSLOT>(p, sm.ncs, Rt, kt, xt, ft, 0);  // first pass of the target row, in flight with the draft's
  if (pair) {
    const float md = sm.m[rd], ld = sm.lz[rd];
    const uint32_t kd = thr_key(sm.fthr[rd]);
    for (int base = 0; base < nslots; base += NT * NSLOT) {
      uint32_t xs[NSLOT];
      float fs[NSLOT];
      sparse_load<NSLOT>(p, sm.ncs2, Rd, kd, xs, fs, base);
#pragma unroll
      for (int t = 0; t < NSLOT; ++t) {
        if (xs[t] == 0xffffffffu) continue;
        uint32_t h = hslot(xs[t]);
        for (int probe = 0; probe < HT; ++probe) {  // bounded: the table holds at most KMAX < HT entries
          const int prev = atomicCAS(&sm.hidx[h], -1, (int)xs[t]);
          if (prev == -1 || prev == (int)xs[t]) {
            sm.hlq[h] = fmaf(fs[t] - md, q.c, -ld);
            break;
          }
          h = (h + 1) & (HT - 1);
        }
      }
    }
    __syncthreads();
  }
  // target kept entries: alpha (2^40 fixed point: the candidates' slot order varies from call to call,
  // and this sum does not depend on it) and the residual or bonus race
  float best = 0.0f, bval = 0.0f;
  int bidx = INT_MAX;
  unsigned long long acc = 0;
  const bool smp = p.mode == MODE_SAMPLE;
  const uint32_t tag = smp ? 2u : 1u;
  const uint32_t sb = smp ? (uint32_t)(p.row_b ? p.row_b[b] : b) : (uint32_t)b;
  const uint32_t sj = smp ? (uint32_t)(p.row_pos ? p.row_pos[b] : 0) : (uint32_t)i;
  for (int base = 0; base < nslots; base += NT * NSLOT) {
    if (base > 0) sparse_load<NSLOT>(p, sm.ncs, Rt, kt, xt, ft, base);
    if (!pair) {
      sparse_plain_race<NSLOT>(p, xt, ft, mt, q.c, tag, sb, sj, best, bidx, bval);
      continue;
    }
#pragma unroll
    for (int t = 0; t < NSLOT; ++t) {
      if (xt[t] == 0xffffffffu) continue;
      const uint32_t x = xt[t];
      const float lp = fmaf(ft[t] - mt, q.c, -lt);
      float lq = -INFINITY;
      uint32_t h = hslot(x);
      for (int probe = 0; probe < HT; ++probe) {
        const int v = sm.hidx[h];
        if (v == (int)x) {
          lq = sm.hlq[h];
          break;
        }
        if (v == -1) break;
        h = (h + 1) & (HT - 1);
      }
      acc += fixmass(fexp2(fminf(lp, lq)));
      if (draw) {
        const float w = fexp2(lp) - fexp2(lq);
        if (w > 0.0f) {
          const uint4 w4 = philox10_uk(make_uint4(x >> 2, sb, (tag << 24) | sj, p.offset), p.key0, p.key1);
          const uint32_t qq = x & 3u;
          race_take(best, bidx, bval, race_key(w, qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w), (int)x,
                    ft[t]);
        }
      }
    }
  }
  if (pair) {
    acc = wave_sum_u64(acc);
    if (lane == 0) sm.asum[wave] = acc;
    __syncthreads();
    if (tid == 0) {
      unsigned long long v = 0;
      for (int w = 0; w < NWAVE; ++w) v += sm.asum[w];
      p.alpha[(size_t)b * k + i] = (float)((double)v * 0x1p-40);
    }
  }
  if (!draw) return;
  block_race(sm.rs, best, bidx, bval);
  if (bidx == INT_MAX && pair) {
    // The residual mass vanished in fp32 (rounding only): draw from p_n (its kept entries).
    for (int base = 0; base < nslots; base += NT * NSLOT) {
      sparse_load<NSLOT>(p, sm.ncs, Rt, kt, xt, ft, base);
      sparse_plain_race<NSLOT>(p, xt, ft, mt, q.c, 1u, (uint32_t)b, (uint32_t)n, best, bidx, bval);
    }
    block_race(sm.rs, best, bidx, bval);
  }
  const int y = bidx;
  if (y < 0 || y >= p.V) return write_sentinel(p, b);  // no candidate: not reachable for a valid row
  if (smp) {
    if (tid == 0) {
      p.tokens[b] = y;
      p.logprobs[b] = (bval - sm.m[0]) / q.T - logf(sm.Z[0]);
    }
    return;
  }
  if (tid <= k) {
    int t = -1;
    float lp = 0.0f, rlp = 0.0f;
    if (tid <= n) {
      t = tid < n ? sm.tok[tid] : y;
      const float l = tid < n ? sm.gath[tid] : bval;
      lp = (l - sm.m[tid]) / q.T - logf(sm.Z[tid]);
      rlp = raw_lp(sm, tid, l);
    }
    p.tokens[(size_t)b * (k + 1) + tid] = t;
    p.logprobs[(size_t)b * (k + 1) + tid] = lp;
    if (p.raw_logprobs) p.raw_logprobs[(size_t)b * (k + 1) + tid] = rlp;
  }
  if (tid == 0) p.accept_len[b] = n + 1;
}

template <class E, int VPT>
__device__ __forceinline__ void k5_item(const Params& p, K5Smem& sm, int item, int b, int s) {
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  const int tid = threadIdx.x;
  SV_TRACE5_AT(p, item, 0);
  const int k = p.k, rows = p.rows;
  const int x0 = s * p.L5;
  const int nv = min(p.L5, p.V - x0) / EPV;
  // Everything independent is issued at once: the rows' statistics (with the logits at the draft
  // tokens) and the draft tokens into registers, then the first position's slices; the accept
  // uniforms are computed while they are in flight.  Truncated rows wait for their
  // statistics before loading slices: they may take the candidate path instead.  (Issuing the slices
  // of rows unlikely to take it at once as well measured no faster.)
  const RowParams q = row_params(p, b);
  RowInfo ri{};
  if (tid < rows) ri = p.rinfo[(size_t)b * rows + tid];
  int32_t tokv = 0;
  if (tid < k) tokv = p.draft_tokens[(size_t)b * k + tid];
  uint4 a0[VPT], b0[VPT];
  if (!q.greedy && !q.trunc && k > 0) {
    load_slice<E, VPT>(row_ptr(p, b, 0, esize), x0, nv, a0);
    load_slice<E, VPT>(row_ptr(p, b, k + 1, esize), x0, nv, b0);
  }
  if (tid < k) {
    const uint4 w4 = philox10_uk(make_uint4((uint32_t)tid >> 2, (uint32_t)b, 0u, p.offset), p.key0, p.key1);
    const int qq = tid & 3;
    sm.u[tid] = u24(qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w);
    sm.tok[tid] = tokv;
  }
  if (tid < rows) {
    sm.m[tid] = ri.m;
    sm.arg[tid] = ri.arg;
    sm.Z[tid] = ri.Z;
    sm.lz[tid] = ri.lz;
    sm.fthr[tid] = ri.fthr;
    sm.state[tid] = ri.state;
    sm.gath[tid] = ri.gath;
    if (p.raw_logprobs) sm.rlz[tid] = ri.rlz;
  }
  // Greedy rows need nothing but the row statistics: workgroup 0 of the batch row writes every output,
  // the others leave.  (Tested only after the loads above are issued, so that other rows do not wait
  // for the temperature before issuing them.)
  if (q.greedy && s != 0) return;
  __syncthreads();
  SV_TRACE5_AT(p, item, 1);
  bool ok = q.ok;
  for (int i = 0; i < k; ++i) ok = ok && sm.tok[i] >= 0 && sm.tok[i] < p.V;
  bool sparse = E::KEYBITS == 16 && q.trunc;
  for (int r = 0; r < rows; ++r) {
    ok = ok && (sm.state[r] & ST_BAD) == 0;
    sparse = sparse && (sm.state[r] & ST_SPARSE) != 0;
  }
  if (q.greedy) {  // workgroup 0 only (see above): no slice partials, no arrivals
    k5_finalize<E>(p, sm, b, ok, q);
    SV_TRACE5_AT(p, item, 7);
    return;
  }
  if (ok && sparse && s > k) {  // candidate-path row: this workgroup has no position to finish
    SV_TRACE5_AT(p, item, 7);
    return;
  }
  if (ok && q.trunc && !q.greedy && !sparse && k > 0) {  // truncated rows streamed after all
    load_slice<E, VPT>(row_ptr(p, b, 0, esize), x0, nv, a0);
    load_slice<E, VPT>(row_ptr(p, b, k + 1, esize), x0, nv, b0);
  }
  if (ok && !q.greedy) {
    // accept decisions of all positions at once (lane i of wave 0); n = the first rejection, else k
    // (k = 0 in sample mode: the draw below is the sampler's)
    if (tid < 64) {
      bool reject = false;
      if (tid < k) {
        const float pt = kept_p(sm.gath[tid], sm.m[tid], q.c, sm.lz[tid], sm.fthr[tid]);
        const float qd =
            kept_p(sm.gath[k + 1 + tid], sm.m[k + 1 + tid], q.c, sm.lz[k + 1 + tid], sm.fthr[k + 1 + tid]);
        reject = !(pt > 0.0f && (qd == 0.0f || sm.u[tid] < pt / qd));
      }
      const int fr = first_lane(reject);
      if (tid == 0) sm.n = fr < k ? fr : k;
    }
    __syncthreads();
    SV_TRACE5_AT(p, item, 2);
    const int n = sm.n;
    if constexpr (E::KEYBITS == 16) {
      if (sparse) {  // workgroup s finishes positions s, s + S5, ... from the candidates; no arrivals
        for (int pi = s; pi <= k; pi += p.S5) {
          k5_sparse<E>(p, sm, b, n, pi, q);
          __syncthreads();  // the shared tables are reused by the next position
        }
        if (s <= k) SV_TRACE5_AT(p, item, 3);
        SV_TRACE5_AT(p, item, 7);
        return;
      }
    }
    uint4 vc[VPT];
    if (n == k) load_slice<E, VPT>(row_ptr(p, b, k, esize), x0, nv, vc);
    float best = 0.0f, bval = 0.0f;
    int bidx = INT_MAX;
    if (q.trunc)
      k5_positions<E, VPT, true>(p, sm, b, n, x0, nv, q.c, a0, b0, best, bidx, bval);
    else
      k5_positions<E, VPT, false>(p, sm, b, n, x0, nv, q.c, a0, b0, best, bidx, bval);
    if (n == k) {
      // bonus draw from p_k (verify stream), or the plain sampler's draw (its own stream)
      const bool smp = p.mode == MODE_SAMPLE;
      const uint32_t tag = smp ? 2u : 1u;
      const uint32_t sb = smp ? (uint32_t)(p.row_b ? p.row_b[b] : b) : (uint32_t)b;
      const uint32_t sj = smp ? (uint32_t)(p.row_pos ? p.row_pos[b] : 0) : (uint32_t)k;
      if (q.trunc)
        race_slice<E, VPT, false>(p, vc, vc, x0, nv, q.c, sm.m[k], 0.0f, sm.fthr[k], 0.0f, 0.0f, 0.0f, tag, sb, sj, best,
                                  bidx, bval);
      else
        race_slice<E, VPT, false, false, false>(p, vc, vc, x0, nv, q.c, sm.m[k], 0.0f, sm.fthr[k], 0.0f, 0.0f, 0.0f, tag,
                                                sb, sj, best, bidx, bval);
    }
    SV_TRACE5_AT(p, item, 3);
    block_race(sm.rs, best, bidx, bval);  // its barriers also order the wacc writes before the reads below
    FinalPart* fp = p.fin5 + (size_t)b * p.S5 + s;
    if (tid < k) {
      float v = 0.0f;
      for (int w = 0; w < NWAVE; ++w) v += sm.wacc[tid][w];
      stf(&fp->alpha[tid], v);
    }
    if (tid == 0) {
      stf(&fp->key, best);
      st32(&fp->idx, (uint32_t)bidx);
      stf(&fp->val, bval);
    }
  }
  SV_TRACE5_AT(p, item, 4);
  if (arrive_last(&p.cnt5[b], (uint32_t)p.S5, &sm.rs.flag)) {
    SV_TRACE5_AT(p, item, 5);
    k5_finalize<E>(p, sm, b, ok, q);
    SV_TRACE5_AT(p, item, 6);
  }
  SV_TRACE5_AT(p, item, 7);
}

template <class E, int VPT, bool RAW>
__global__ __launch_bounds__(NT, RAW ? 4 : 5) void k5_verify(Params p) {
  __shared__ K5Smem sm;
  int b, s;
  // row-major items: workgroups go to the XCDs round-robin, so each batch row's slices spread over
  // all of them and a run of expensive rows does not pile onto one XCD
  b = blockIdx.x / p.S5;
  s = blockIdx.x - b * p.S5;
  if constexpr (!RAW) p.raw_logprobs = nullptr;  // every raw-output branch folds away
  k5_item<E, VPT>(p, sm, blockIdx.x, b, s);
}

// ---------------------------------------------------------------------------------------------
// Tree verification: one workgroup per (batch row, K5-sized slice).  Every workgroup checks the tree,
// gathers each node's token logit from its parent's row and walks the tree from the root out of LDS
// (one uniform per depth on the accept stream: the first child whose cumulative target mass exceeds it
// is accepted); then all slices race over the stopping node's row -- with its children's tokens removed
// after a rejection (weights p, as the chain's residual with a one-hot draft), or the plain bonus
// weights at a leaf -- and the last slice to arrive writes the outputs.  A chain of single children is
// therefore the chain verify step with one-hot draft rows, bit for bit.
// ---------------------------------------------------------------------------------------------
struct TreeSmem {
  RedSmem rs;
  float m[MAXN], Z[MAXN], lz[MAXN], fthr[MAXN], gl[MAXN], u[MAXN];
  int32_t arg[MAXN], par[MAXN], tok[MAXN], path[MAXN], ex[MAXN];
  uint32_t state[MAXN];
  int32_t nex, d, stop, leaf;
};

// Race over one slice of the stopping node's row after a rejection: weights kept_p on the kept entries,
// except the node's children's tokens (stream tag 1, position = depth).
template <class E, int VPT>
__device__ __forceinline__ void tree_resid_slice(const Params& p, const TreeSmem& sm, const uint4 (&va)[VPT], int x0, int nv,
                                                 float c, float mt, float lt, float tt, uint32_t sb, uint32_t sj,
                                                 float& best, int& bidx, float& bval) {
  constexpr int EPV = E::EPV;
  const int tid = threadIdx.x, nex = sm.nex;
  float lb = -0.5f, lv = 0.0f;  // this thread's best, as in race_slice: entries in increasing index order
  int li = INT_MAX;
#pragma unroll 1
  for (int u = 0; u < VPT; ++u) {
    const int j = tid + u * NT;
    if (j >= nv) continue;
    const uint4 a = pick_vec<VPT>(va, u);
    bool kept = false;
#pragma unroll
    for (int e = 0; e < EPV; ++e) kept = kept | (E::get(a, e) >= tt);  // bitwise: no branch per entry
    if (!kept) continue;
#pragma unroll 1
    for (int g = 0; g < EPV; g += 4) {
      const int x = x0 + j * EPV + g;
      float w[4];
      bool any = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = kept_p(E::get(a, g + e), mt, c, lt, tt);
        if (w[e] > 0.0f)
          for (int t = 0; t < nex; ++t)
            if (sm.ex[t] == x + e) w[e] = 0.0f;
        any = any | (w[e] > 0.0f);
      }
      if (!any) continue;
      const uint4 w4 = philox10_uk(make_uint4((uint32_t)x >> 2, sb, (1u << 24) | sj, p.offset), p.key0, p.key1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
        const float key = race_key_or_none(w[e], word);
        const bool take = key > lb;
        lb = take ? key : lb;
        li = take ? x + e : li;
        lv = take ? E::get(a, g + e) : lv;
      }
    }
  }
  race_take(best, bidx, bval, lb, li, lv);
}

__device__ __forceinline__ void tree_sentinel(const Params& p, int b) {
  const int N = p.rows, tid = threadIdx.x;
  if (tid < N) {
    p.tokens[(size_t)b * N + tid] = -1;
    p.path[(size_t)b * N + tid] = -1;
    p.logprobs[(size_t)b * N + tid] = __builtin_nanf("");
  }
  if (tid == 0) p.accept_len[b] = 0;
}

// Outputs of a batch row whose walk ended at depth d on node u with drawn token y (logit yv).
__device__ __forceinline__ void tree_emit(const Params& p, const TreeSmem& sm, int b, const RowParams& q, int y, float yv) {
  const int N = p.rows, tid = threadIdx.x, d = sm.d, u = sm.stop;
  if (tid < N) {
    int t = -1, pth = -1;
    float lp = 0.0f;
    if (tid < d) {
      const int node = sm.path[tid], row = tid == 0 ? 0 : sm.path[tid - 1];
      t = sm.tok[node];
      pth = node;
      if (!q.greedy) lp = (sm.gl[node] - sm.m[row]) / q.T - logf(sm.Z[row]);
    } else if (tid == d) {
      t = y;
      if (!q.greedy) lp = (yv - sm.m[u]) / q.T - logf(sm.Z[u]);
    }
    p.tokens[(size_t)b * N + tid] = t;
    p.path[(size_t)b * N + tid] = pth;
    p.logprobs[(size_t)b * N + tid] = lp;
  }
  if (tid == 0) p.accept_len[b] = d + 1;
}

template <class E, int VPT>
// At most 80 scalar registers in the compiler's total (the attribute's 82 gives 80, a few spilled to vector
// lanes): the hardware holds eight 256-thread workgroups per CU only up to that total, and the tree items are
// latency-bound (unconstrained, 92 scalars gave seven per CU and a 0.5 us slower kernel).
__global__ __launch_bounds__(NT) __attribute__((amdgpu_num_sgpr(82))) void k_tree(Params p) {
  __shared__ TreeSmem sm;
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  const int b = blockIdx.x / p.S5, s = blockIdx.x - b * p.S5;
  const int N = p.rows, tid = threadIdx.x;
  const RowParams q = row_params(p, b);
  if (tid < N) {
    const RowInfo* ri = p.rinfo + (size_t)b * N + tid;
    sm.m[tid] = ri->m;
    sm.arg[tid] = ri->arg;
    sm.Z[tid] = ri->Z;
    sm.lz[tid] = ri->lz;
    sm.fthr[tid] = ri->fthr;
    sm.state[tid] = ri->state;
    sm.par[tid] = p.parent[(size_t)b * N + tid];
    sm.tok[tid] = p.draft_tokens[(size_t)b * N + tid];
    const uint4 w4 = philox10_uk(make_uint4((uint32_t)tid >> 2, (uint32_t)b, 0u, p.offset), p.key0, p.key1);
    const int qq = tid & 3;
    sm.u[tid] = u24(qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w);
  }
  __syncthreads();
  // the tree: every node but the root has an earlier parent and a token in range; siblings differ
  bool bad = false;
  if (tid < N) {
    bad = (sm.state[tid] & ST_BAD) != 0;
    if (tid >= 1) {
      const int pa = sm.par[tid], tk = sm.tok[tid];
      bad = bad || pa < 0 || pa >= tid || tk < 0 || tk >= p.V;
      for (int j = 1; j < tid; ++j) bad = bad || (sm.par[j] == pa && sm.tok[j] == tk);
    }
  }
  const bool ok = q.ok && !__syncthreads_or(bad);
  if (!ok) {
    if (s == 0) tree_sentinel(p, b);
    return;
  }
  if (tid >= 1 && tid < N) sm.gl[tid] = E::load1(row_ptr(p, b, sm.par[tid], esize), sm.tok[tid]);
  __syncthreads();
  if (tid == 0) {
    int u = 0, d = 0, leaf = 0;
    for (;;) {
      int acc = -1;
      bool any = false;
      float S = 0.0f;
      for (int c = u + 1; c < N; ++c) {  // children have larger indices than their parent
        if (sm.par[c] != u) continue;
        any = true;
        if (q.greedy) {
          if (sm.tok[c] == sm.arg[u]) {
            acc = c;
            break;
          }
        } else {
          S += kept_p(sm.gl[c], sm.m[u], q.c, sm.lz[u], sm.fthr[u]);
          if (sm.u[d] < S) {
            acc = c;
            break;
          }
        }
      }
      if (!any) {
        leaf = 1;
        break;
      }
      if (acc < 0) break;
      sm.path[d++] = acc;
      u = acc;
    }
    int ne = 0;
    if (!leaf)
      for (int c = u + 1; c < N; ++c)
        if (sm.par[c] == u) sm.ex[ne++] = sm.tok[c];
    sm.nex = ne;
    sm.d = d;
    sm.stop = u;
    sm.leaf = leaf;
  }
  __syncthreads();
  const int u = sm.stop, d = sm.d;
  if (q.greedy) {
    if (s == 0) tree_emit(p, sm, b, q, sm.arg[u], sm.m[u]);
    return;
  }
  const int x0 = s * p.L5;
  const int nv = min(p.L5, p.V - x0) / EPV;
  uint4 v[VPT];
  load_slice<E, VPT>(row_ptr(p, b, u, esize), x0, nv, v);
  float best = 0.0f, bval = 0.0f;
  int bidx = INT_MAX;
  if (sm.leaf)
    race_slice<E, VPT, false>(p, v, v, x0, nv, q.c, sm.m[u], 0.0f, sm.fthr[u], 0.0f, 0.0f, 0.0f, 1u, (uint32_t)b,
                              (uint32_t)d, best, bidx, bval);
  else
    tree_resid_slice<E, VPT>(p, sm, v, x0, nv, q.c, sm.m[u], sm.lz[u], sm.fthr[u], (uint32_t)b, (uint32_t)d, best,
                             bidx, bval);
  block_race(sm.rs, best, bidx, bval);
  FinalPart* fp = p.fin5 + (size_t)b * p.S5 + s;
  if (tid == 0) {
    stf(&fp->key, best);
    st32(&fp->idx, (uint32_t)bidx);
    stf(&fp->val, bval);
  }
  if (!arrive_last(&p.cnt5[b], (uint32_t)p.S5, &sm.rs.flag)) return;
  best = 0.0f;
  bval = 0.0f;
  bidx = INT_MAX;
  for (int sl = tid; sl < p.S5; sl += NT) {
    const FinalPart* f = p.fin5 + (size_t)b * p.S5 + sl;
    race_take(best, bidx, bval, ldf(&f->key), (int)ld32(&f->idx), ldf(&f->val));
  }
  block_race(sm.rs, best, bidx, bval);
  if (bidx == INT_MAX) {
    // nothing left after removing the children (rounding only): draw from p_u over the whole row
    const uint4* row = (const uint4*)row_ptr(p, b, u, esize);
    for (int j = tid; j < p.V / EPV; j += NT)
      gumbel_vec<E>(row[j], j * EPV, sm.m[u], q.c, sm.fthr[u], 1u, (uint32_t)b, (uint32_t)d, p, best, bidx, bval);
    block_race(sm.rs, best, bidx, bval);
  }
  if (bidx < 0 || bidx >= p.V)
    tree_sentinel(p, b);  // no candidate: not reachable for a valid row
  else
    tree_emit(p, sm, b, q, bidx, bval);
}

#include "sv_resident.h"

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
constexpr int RMAXK = 4;      // the resident kernel serves k = 1..RMAXK
constexpr int RMAXWG = 1024;  // the largest resident grid the workspace is sized for (a GPU with <= 1024 CUs)
// The library's own choice takes the resident path only up to this many vectors per thread and row: none
// at present (measured on MI355X, the staged path is as fast or faster on every workload that fits: its
// single workgroup per CU has too few waves to hide the latency of its exchanges and reductions).
constexpr int RAUTO_NV = 0;

// Workspace of the resident kernel with S slices per batch row.
static size_t resident_bytes(int32_t B, int32_t k, int32_t S) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)(2 * k + 1), bs = (size_t)B * (size_t)S;
  return al(bs * rows * sizeof(RPart)) + al(bs * rows * RWIN * 4) + al(bs * sizeof(RFin)) + 2 * al(bs * 8) +
         (TRACE_SLOTS > 0 ? al(bs * 128) : 0) + 256;
}

// Slices per batch row the resident kernel would use on a GPU with `cus` compute units (one workgroup per
// CU): the smallest nv (vectors per thread per row) whose grid B x ceil(V / 4096 nv) fits; false if none.
static bool resident_plan(int32_t B, int32_t k, int32_t V, int cus, int& nv, int& S) {
  if (k < 1 || k > RMAXK) return false;
  for (nv = 1; nv <= rnv_max(k); ++nv) {
    const int L = RT * BF16::EPV * nv;
    S = (V + L - 1) / L;
    if ((long long)B * S <= (long long)cus) return true;
  }
  return false;
}

struct Geo {
  int rows, R, S1, S5, L1, L5, esize, EPV, vpt1;
  size_t off_cnt5, off_st1, off_hw1, off_hc1, off_cand1, off_ncand1, off_rinfo, off_fin5, off_trace, off_trace5,
      total;
};

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// tree_nodes > 0: tree verification with that many nodes (target rows) per batch row; k is ignored.
static bool make_geo(int32_t B, int32_t k, int32_t V, spec_dtype_t dtype, Geo& g, int32_t tree_nodes = 0) {
  if (tree_nodes > 0) {
    if (tree_nodes > MAXN) return false;
    k = 0;
  }
  if (B < 1 || B > (1 << 20) || k < 0 || k > MAXK || V < 1 || V > (1 << 20)) return false;
  if (dtype != SPEC_DTYPE_BF16 && dtype != SPEC_DTYPE_F32) return false;
  g.esize = dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  g.EPV = 16 / g.esize;
  if (V % g.EPV != 0) return false;  // whole 16-byte vectors per row: V >= 8 (bf16) or V >= 4 (fp32)
  g.rows = tree_nodes > 0 ? tree_nodes : 2 * k + 1;
  if ((long long)B * g.rows > (1 << 24)) return false;  // item counts stay below 2^31
  g.R = B * g.rows;
  // Wide slices only where K1 runs many rounds of items: there the per-slice work (histogram clears,
  // partials, candidate staging) and the number of partials each merge reads count for more than the tail of
  // the last round, which wider slices lengthen on calls of few rounds.
  g.vpt1 = VPT1;
  if (dtype == SPEC_DTYPE_BF16) {
    const long long sw = (V + NT * g.EPV * VPT1W - 1) / (NT * g.EPV * VPT1W);
    if ((long long)g.R * sw >= K1W_ITEMS) g.vpt1 = VPT1W;
  }
  g.L1 = NT * g.EPV * g.vpt1;
  g.L5 = NT * g.EPV * VPT5;
  g.S1 = (V + g.L1 - 1) / g.L1;
  g.S5 = (V + g.L5 - 1) / g.L5;
  const size_t R = (size_t)g.R;
  size_t off = 256;
  auto take = [&](size_t& o, size_t bytes) {
    o = off;
    off = align_up(off + bytes, 256);
  };
  take(g.off_cnt5, (size_t)B * 4);
  take(g.off_st1, R * g.S1 * sizeof(StatPart));
  const bool bf = dtype == SPEC_DTYPE_BF16;  // per-code and weight-bin partials: bf16 rows only
  take(g.off_hw1, bf ? R * g.S1 * (WTOP / 2) * 4 : 0);
  take(g.off_hc1, bf ? R * g.S1 * HCW * 4 : 0);
  take(g.off_cand1, bf ? R * g.S1 * NC * 8 : 0);
  take(g.off_ncand1, bf ? R * g.S1 * 4 : 0);
  take(g.off_rinfo, R * sizeof(RowInfo));
  take(g.off_fin5, (size_t)B * g.S5 * sizeof(FinalPart));
  take(g.off_trace, R * g.S1 * TRACE_SLOTS * 8);
  take(g.off_trace5, (size_t)B * g.S5 * TRACE_SLOTS * 8);
  g.total = off;
  // the resident kernel (bf16 verify, k <= RMAXK) lays out its own partials in the same workspace
  int nv = 0, S = 0;
  if (dtype == SPEC_DTYPE_BF16 && tree_nodes == 0 && k >= 1 && resident_plan(B, k, V, RMAXWG, nv, S))
    g.total = std::max(g.total, resident_bytes(B, k, std::max(S, 1)) + 256);
  return true;
}

struct DevInfo {
  int state;  // 0 unknown, 1 gfx950, 2 other
  int cus;    // compute units
  int rocc[RMAXK + 1];  // resident kernel: co-resident workgroups per CU (0 unknown, -1 unusable)
};
static DevInfo g_dev[MAXDEV];
static std::mutex g_mu;

bool device_ok(int dev, int& cus) {
  if (dev < 0 || dev >= MAXDEV) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_dev[dev].state == 0) {
    hipDeviceProp_t pr;
    if (hipGetDeviceProperties(&pr, dev) != hipSuccess) return false;
    g_dev[dev].state = (std::strncmp(pr.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev[dev].cus = pr.multiProcessorCount > 0 ? pr.multiProcessorCount : 256;
  }
  cus = g_dev[dev].cus;
  return g_dev[dev].state == 1;
}

// Per-call kernel timing (the timed entry points): events[2j] / events[2j+1] around kernel j; and the
// bound on the resident kernel's waits (0: the default).
struct Timing {
  hipEvent_t ev[2 * NKERN];
  int used;
  int path;  // SPEC_PATH_*
  uint64_t wait_limit;
};
static void prof_mark(Timing* t, int idx, hipStream_t st) {
  if (t && t->ev[idx]) (void)hipEventRecord(t->ev[idx], st);
}

template <class E>
static void enqueue(const Params& p, int cus, hipStream_t st, Timing* tm) {
  static_assert(WTOP / 2 == NT && NBC == NT, "K1 assumes one histogram word pair per thread");
  static_assert((NCOPY & (NCOPY - 1)) == 0 && NCOPY <= 64, "weight-bin copies: a power of two");
  (void)cus;
  const dim3 g1((unsigned)(p.R * p.S1)), gr((unsigned)p.R), g5((unsigned)(p.B * p.S5));
  const bool raw = p.raw_logprobs != nullptr;
  prof_mark(tm, 0, st);
  bool wide = false;  // the slice width the geometry chose (bf16 only)
  if constexpr (E::KEYBITS == 16) wide = p.L1 == NT * E::EPV * VPT1W;
  if constexpr (E::KEYBITS == 16) {
    if (wide && raw)
      hipLaunchKernelGGL((k1_stats<E, VPT1W, true>), g1, dim3(NT), 0, st, p);
    else if (wide)
      hipLaunchKernelGGL((k1_stats<E, VPT1W, false>), g1, dim3(NT), 0, st, p);
  }
  if (!wide && raw)
    hipLaunchKernelGGL((k1_stats<E, VPT1, true>), g1, dim3(NT), 0, st, p);
  else if (!wide)
    hipLaunchKernelGGL((k1_stats<E, VPT1, false>), g1, dim3(NT), 0, st, p);
  prof_mark(tm, 1, st);
  prof_mark(tm, 2, st);
  if (raw)
    hipLaunchKernelGGL((k1_rows<E, true>), gr, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((k1_rows<E, false>), gr, dim3(NT), 0, st, p);
  prof_mark(tm, 3, st);
  prof_mark(tm, 4, st);
  if (p.mode == MODE_TREE)
    hipLaunchKernelGGL((k_tree<E, VPT5>), g5, dim3(NT), 0, st, p);
  else if (raw)
    hipLaunchKernelGGL((k5_verify<E, VPT5, true>), g5, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((k5_verify<E, VPT5, false>), g5, dim3(NT), 0, st, p);
  prof_mark(tm, 5, st);
  if (tm) tm->used = NKERN;
}

template <int KK>
static int resident_occupancy() {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kr_verify<KK>, RT, 0) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return nb >= 1 ? nb : -1;
}

// Co-resident workgroups per CU of the resident kernel for k (cached per device); <= 0 if it cannot run.
static int resident_occ(int dev, int k) {
  std::lock_guard<std::mutex> lk(g_mu);
  int& o = g_dev[dev].rocc[k];
  if (o == 0) o = k == 1 ? resident_occupancy<1>() : k == 2 ? resident_occupancy<2>()
                  : k == 3 ? resident_occupancy<3>() : resident_occupancy<4>();
  return o;
}

// The resident kernel for this call, if its grid fits the device; false (nothing enqueued) otherwise, and
// also if the runtime refuses the cooperative launch.
static bool launch_resident(const Params& p, int dev, int cus, uint8_t* ws, size_t ws_bytes, hipStream_t st,
                            Timing* tm, uint64_t seed, bool forced) {
  int nv = 0, S = 0;
  if (p.mode != MODE_VERIFY || p.raw_logprobs || !resident_plan(p.B, p.k, p.V, cus, nv, S)) return false;
  if (!forced && nv > RAUTO_NV) return false;  // the staged path is faster for longer slices
  const int occ = resident_occ(dev, p.k);
  if (occ < 1 || (long long)p.B * S > (long long)occ * cus || resident_bytes(p.B, p.k, S) > ws_bytes) return false;
  RParams r;
  std::memset(&r, 0, sizeof r);
  r.target = p.target;
  r.draft = p.draft;
  r.draft_tokens = p.draft_tokens;
  r.temperature = p.temperature;
  r.top_k = p.top_k;
  r.top_p = p.top_p;
  r.B = p.B;
  r.k = p.k;
  r.V = p.V;
  r.S = S;
  r.nv = nv;
  r.L = RT * BF16::EPV * nv;
  r.key0 = p.key0;
  r.key1 = p.key1;
  r.offset = p.offset;
  r.salt = seed ^ ((uint64_t)p.offset << 32) ^ ((uint64_t)p.B * 0x100000001B3ull) ^ ((uint64_t)p.k << 56) ^
           ((uint64_t)p.V << 20);
  r.wait_limit = (tm && tm->wait_limit) ? tm->wait_limit : RWAIT_DEFAULT;
  r.tokens = p.tokens;
  r.accept_len = p.accept_len;
  r.logprobs = p.logprobs;
  r.alpha = p.alpha;
  const size_t bs = (size_t)p.B * S, rows = (size_t)(2 * p.k + 1);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  r.part = (RPart*)(ws + off);
  off += al(bs * rows * sizeof(RPart));
  r.win = (uint32_t*)(ws + off);
  off += al(bs * rows * RWIN * 4);
  r.fin = (RFin*)(ws + off);
  off += al(bs * sizeof(RFin));
  r.flag1 = (unsigned long long*)(ws + off);
  off += al(bs * 8);
  r.flag2 = (unsigned long long*)(ws + off);
  off += al(bs * 8);
  r.trace = TRACE_SLOTS > 0 ? (unsigned long long*)(ws + off) : nullptr;
  // An ordinary launch: its grid (one workgroup per CU at most, checked above against the occupancy of
  // this kernel) is resident at once on an otherwise idle device.  A cooperative launch would guarantee it
  // but costs ~20 us per call on this runtime; the bounded waits keep a stalled grid from hanging instead.
  prof_mark(tm, 0, st);
  if (p.k == 1)
    hipLaunchKernelGGL(kr_verify<1>, dim3((unsigned)bs), dim3(RT), 0, st, r);
  else if (p.k == 2)
    hipLaunchKernelGGL(kr_verify<2>, dim3((unsigned)bs), dim3(RT), 0, st, r);
  else if (p.k == 3)
    hipLaunchKernelGGL(kr_verify<3>, dim3((unsigned)bs), dim3(RT), 0, st, r);
  else
    hipLaunchKernelGGL(kr_verify<4>, dim3((unsigned)bs), dim3(RT), 0, st, r);
  prof_mark(tm, 1, st);
  if (tm) tm->used = 1;
  return true;
}

static spec_status_t launch(Params& p, const Geo& g, spec_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream, Timing* tm = nullptr, uint64_t seed = 0) {
  if (!workspace || workspace_bytes < g.total || ((uintptr_t)workspace & 15)) return SPEC_ERR_WORKSPACE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev, cus)) return SPEC_ERR_UNSUPPORTED_DEVICE;
  p.rows = g.rows;
  p.R = g.R;
  p.S1 = g.S1;
  p.S5 = g.S5;
  p.L1 = g.L1;
  p.L5 = g.L5;
  uint8_t* ws = (uint8_t*)workspace;
  p.cnt5 = (uint32_t*)(ws + g.off_cnt5);
  p.st1 = (StatPart*)(ws + g.off_st1);
  p.hw1 = (uint32_t*)(ws + g.off_hw1);
  p.hc1 = (uint32_t*)(ws + g.off_hc1);
  p.cand1 = (unsigned long long*)(ws + g.off_cand1);
  p.ncand1 = (uint32_t*)(ws + g.off_ncand1);
  p.rinfo = (RowInfo*)(ws + g.off_rinfo);
  p.fin5 = (FinalPart*)(ws + g.off_fin5);
  p.trace = TRACE_SLOTS > 0 ? (unsigned long long*)(ws + g.off_trace) : nullptr;
  p.trace5 = TRACE_SLOTS > 0 ? (unsigned long long*)(ws + g.off_trace5) : nullptr;
  // hipGetLastError reports the last error of any earlier runtime call of this thread (a caller's, too);
  // read it once before enqueueing so that the check after the launches is about them alone
  (void)hipGetLastError();
  const int path = tm ? tm->path : SPEC_PATH_AUTO;
  if (dtype == SPEC_DTYPE_BF16 && path != SPEC_PATH_STAGED &&
      launch_resident(p, dev, cus, ws, workspace_bytes, (hipStream_t)stream, tm, seed, path == SPEC_PATH_RESIDENT)) {
    if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
    return SPEC_OK;
  }
  if (dtype == SPEC_DTYPE_BF16)
    enqueue<BF16>(p, cus, (hipStream_t)stream, tm);
  else
    enqueue<F32>(p, cus, (hipStream_t)stream, tm);
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

static spec_status_t verify_impl(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                 const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                                 const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                                 int32_t* tokens, int32_t* accept_len, float* logprobs, float* raw_logprobs,
                                 float* alpha, void* workspace, size_t workspace_bytes, void* stream, Timing* tm) {
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
  p.raw_logprobs = raw_logprobs;
  p.alpha = alpha;
  return launch(p, g, dtype, workspace, workspace_bytes, stream, tm, seed);
}

extern "C" spec_status_t spec_verify(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                     const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                                     const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed,
                                     uint64_t offset, int32_t* tokens, int32_t* accept_len, float* logprobs,
                                     float* alpha, void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(target_logits, draft_logits, dtype, draft_tokens, temperature, top_k, top_p, B, k, V, seed,
                     offset, tokens, accept_len, logprobs, nullptr, alpha, workspace, workspace_bytes, stream, nullptr);
}

// Scratch of spec_verify_noalloc: file-scope static device memory, one copy per GPU.  Host code never
// uses the array's name as an address: its per-device address comes from hipGetSymbolAddress, looked
// up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[SPEC_NOALLOC_SCRATCH_BYTES];
static void* g_scratch[MAXDEV];

static void* scratch_address(int dev) {
  if (dev < 0 || dev >= MAXDEV) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

extern "C" spec_status_t spec_verify_noalloc(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                             const int32_t* draft_tokens, const float* temperature,
                                             const int32_t* top_k, const float* top_p, int32_t B, int32_t k,
                                             int32_t V, uint64_t seed, uint64_t offset, int32_t* tokens,
                                             int32_t* accept_len, float* logprobs, float* alpha, void* stream) {
  Geo g;
  if (k < 1 || !make_geo(B, k, V, dtype, g)) return SPEC_ERR_INVALID_ARGUMENT;
  if (g.total > SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev, cus)) return SPEC_ERR_UNSUPPORTED_DEVICE;
  void* ws = scratch_address(dev);
  if (!ws) return SPEC_ERR_LAUNCH;
  return verify_impl(target_logits, draft_logits, dtype, draft_tokens, temperature, top_k, top_p, B, k, V, seed,
                     offset, tokens, accept_len, logprobs, nullptr, alpha, ws, SPEC_NOALLOC_SCRATCH_BYTES, stream,
                     nullptr);
}

extern "C" spec_status_t spec_verify_raw(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                         const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                                         const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed,
                                         uint64_t offset, int32_t* tokens, int32_t* accept_len, float* logprobs,
                                         float* raw_logprobs, float* alpha, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  if (!raw_logprobs) return SPEC_ERR_INVALID_ARGUMENT;
  return verify_impl(target_logits, draft_logits, dtype, draft_tokens, temperature, top_k, top_p, B, k, V, seed,
                     offset, tokens, accept_len, logprobs, raw_logprobs, alpha, workspace, workspace_bytes, stream,
                     nullptr);
}

// Copies the caller's events into a per-call Timing (nothing outlives the call).
static bool timing_in(const spec_timing_t* t, Timing& tm) {
  if (!t) return false;
  for (int j = 0; j < 2 * NKERN; ++j) tm.ev[j] = t->events ? (hipEvent_t)t->events[j] : nullptr;
  tm.used = 0;
  if (t->path != SPEC_PATH_AUTO && t->path != SPEC_PATH_STAGED && t->path != SPEC_PATH_RESIDENT) return false;
  tm.path = t->path;
  tm.wait_limit = t->wait_limit;
  return true;
}

extern "C" spec_status_t spec_verify_timed(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                           const int32_t* draft_tokens, const float* temperature,
                                           const int32_t* top_k, const float* top_p, int32_t B, int32_t k, int32_t V,
                                           uint64_t seed, uint64_t offset, int32_t* tokens, int32_t* accept_len,
                                           float* logprobs, float* raw_logprobs, float* alpha, void* workspace,
                                           size_t workspace_bytes, void* stream, spec_timing_t* timing) {
  Timing tm;
  if (!timing_in(timing, tm)) return SPEC_ERR_INVALID_ARGUMENT;
  const spec_status_t st =
      verify_impl(target_logits, draft_logits, dtype, draft_tokens, temperature, top_k, top_p, B, k, V, seed, offset,
                  tokens, accept_len, logprobs, raw_logprobs, alpha, workspace, workspace_bytes, stream, &tm);
  timing->kernels = tm.used;
  return st;
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

extern "C" size_t spec_tree_verify_workspace_size(int32_t B, int32_t N, int32_t V, spec_dtype_t dtype) {
  Geo g;
  if (N < 1 || !make_geo(B, 0, V, dtype, g, N)) return 0;
  return g.total;
}

static spec_status_t tree_impl(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                               const int32_t* node_tokens, const float* temperature, const int32_t* top_k,
                               const float* top_p, int32_t B, int32_t N, int32_t V, uint64_t seed, uint64_t offset,
                               int32_t* tokens, int32_t* path, int32_t* accept_len, float* logprobs, void* workspace,
                               size_t workspace_bytes, void* stream, Timing* tm) {
  Geo g;
  if (N < 1 || !make_geo(B, 0, V, dtype, g, N)) return SPEC_ERR_INVALID_ARGUMENT;
  if (offset >= (1ull << 32)) return SPEC_ERR_INVALID_ARGUMENT;
  if (!target_logits || !parent || !node_tokens || !temperature || !top_k || !top_p || !tokens || !path ||
      !accept_len || !logprobs)
    return SPEC_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)target_logits & 15) return SPEC_ERR_INVALID_ARGUMENT;
  Params p;
  std::memset(&p, 0, sizeof p);
  p.target = (const uint8_t*)target_logits;
  p.draft = (const uint8_t*)target_logits;
  p.draft_tokens = node_tokens;
  p.parent = parent;
  p.path = path;
  p.temperature = temperature;
  p.top_k = top_k;
  p.top_p = top_p;
  p.B = B;
  p.k = N - 1;  // rows 0..N-1 of a batch row are all target rows
  p.V = V;
  p.mode = MODE_TREE;
  p.key0 = (uint32_t)(seed & 0xffffffffu);
  p.key1 = (uint32_t)(seed >> 32);
  p.offset = (uint32_t)offset;
  p.tokens = tokens;
  p.accept_len = accept_len;
  p.logprobs = logprobs;
  return launch(p, g, dtype, workspace, workspace_bytes, stream, tm);
}

extern "C" spec_status_t spec_tree_verify(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                                          const int32_t* node_tokens, const float* temperature, const int32_t* top_k,
                                          const float* top_p, int32_t B, int32_t N, int32_t V, uint64_t seed,
                                          uint64_t offset, int32_t* tokens, int32_t* path, int32_t* accept_len,
                                          float* logprobs, void* workspace, size_t workspace_bytes, void* stream) {
  return tree_impl(target_logits, dtype, parent, node_tokens, temperature, top_k, top_p, B, N, V, seed, offset, tokens,
                   path, accept_len, logprobs, workspace, workspace_bytes, stream, nullptr);
}

extern "C" spec_status_t spec_tree_verify_timed(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                                                const int32_t* node_tokens, const float* temperature,
                                                const int32_t* top_k, const float* top_p, int32_t B, int32_t N,
                                                int32_t V, uint64_t seed, uint64_t offset, int32_t* tokens,
                                                int32_t* path, int32_t* accept_len, float* logprobs, void* workspace,
                                                size_t workspace_bytes, void* stream, spec_timing_t* timing) {
  Timing tm;
  if (!timing_in(timing, tm)) return SPEC_ERR_INVALID_ARGUMENT;
  const spec_status_t st = tree_impl(target_logits, dtype, parent, node_tokens, temperature, top_k, top_p, B, N, V,
                                     seed, offset, tokens, path, accept_len, logprobs, workspace, workspace_bytes,
                                     stream, &tm);
  timing->kernels = tm.used;
  return st;
}
