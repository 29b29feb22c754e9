// specverify.hip -- libspecverify: the speculative-decoding verify sampler as one persistent HIP kernel
// for gfx950 (MI355X), plus its C ABI (include/specverify.h).
//
// Method: AReno pull request "feat(engine): MTP training loss and speculative decoding for bailing_v3",
// section "What does this PR do?" (Phase 2: sampler-equivalent target distribution, exact chain
// rejection sampling, unchanged logprobs), its accept-probability table (alpha = sum min(p, q)), and
// its per-step optimisation table (Gumbel-max draws, no host synchronisation).
//
// Work decomposition.  A batch row b owns 2k+1 logit rows (k+1 target, k draft).  Its vocabulary is
// cut into S slices of L entries; work item (b, s) is "slice s of all 2k+1 rows of b".  Workgroups
// take items from a device-wide counter in order, so the S items of one batch row are held by
// workgroups that are running at the same time; they form a cluster that meets at counting barriers
// (a per-batch-row arrival counter).  Because items are taken in order and a workgroup only waits for
// items taken before it could finish, any grid with at least S resident workgroups makes progress;
// every wait is bounded as well, and a wait that runs out marks the batch row as a sentinel row.
//
// Phases of an item (the slice stays in LDS between them, so each logit is read from HBM once):
//   A  load the slice of every row (16-byte loads, coalesced), per-slice max / lowest argmax /
//      sum of exp2((l - max) * log2(e) / T), NaN/+inf flags -> partials; barrier 1.
//   B  every member combines the S partials of each row in slice order (same result everywhere).
//      If top-k or top-p is on, row r's leader (member r mod S) finds the exact kept threshold of
//      the whole row by an MSD radix select on order-preserving keys with LDS histograms (counts and
//      fixed-point masses), then barrier 2.
//   C  every member evaluates the accept chain (p_i(x_i), q_i(x_i) from the row statistics and the
//      two gathered logits), then over its slice: alpha partial sums for every draft position and the
//      Gumbel-max candidate at the first rejected position (residual) or at position k (bonus).
//      The last member to arrive combines the partials and writes the batch row's outputs.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>

#include "specverify.h"
#include "sv_common.h"

namespace sv {

constexpr int MODE_VERIFY = 0;
constexpr int MODE_SAMPLE = 1;  // plain sampler: k = 0, one logit row per batch row, stream tag 2
constexpr uint32_t SPIN_LIMIT = 1u << 21;  // bounded waits (~2 s): a run-out marks the row invalid
constexpr int MAXDEV = 64;

struct StatPart {  // per (batch row, logit row, slice)
  float m;         // slice max
  int32_t arg;     // lowest index of the slice max (INT_MAX if none)
  float s;         // sum of exp2((l - m) * c) over the slice
  uint32_t flags;  // bit 0: NaN or +inf seen
};

struct CutRes {   // per (batch row, logit row): kept threshold
  uint32_t thr;   // smallest kept order-preserving key
  float Z;        // kept-set normaliser: sum of exp2((l - m) * c) over kept entries
  uint32_t pad[2];
};

struct FinalPart {  // per (batch row, slice)
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
  int32_t B, k, V, rows, S, L, total_items;
  int32_t mode;               // MODE_VERIFY or MODE_SAMPLE
  const int32_t* row_b;       // plain sampler: stream coordinate b of each row (NULL = row index)
  const int32_t* row_pos;     // plain sampler: stream coordinate i of each row (NULL = 0)
  uint32_t key0, key1, offset;
  int32_t* tokens;
  int32_t* accept_len;
  float* logprobs;
  float* alpha;
  uint32_t* ctrl;    // [0] next item, [1] exited workgroups
  uint32_t* arrive;  // [B] cluster arrival counters
  uint32_t* err;     // [B] wait run-out flags
  StatPart* stats;   // [B][rows][S]
  CutRes* cut;       // [B][rows]
  FinalPart* fin;    // [B][S]
};

struct Smem {
  float m[MAXROWS];
  int32_t arg[MAXROWS];
  float Z[MAXROWS];
  float invZ[MAXROWS];
  uint32_t thr[MAXROWS];
  uint32_t bad;
  int32_t item;
  int32_t pick;
  int32_t n;
  int32_t last;
  float red_f[NWAVE];
  float red_g[NWAVE];
  int32_t red_i[NWAVE];
  uint32_t red_u[NWAVE];
  uint32_t hcnt[256];
  unsigned long long hmass[256];
  unsigned long long scan64[NWAVE];
  uint32_t scan32[NWAVE];
  uint32_t sel, sel_excl;
  unsigned long long sel_mexcl, sel_m;
};

__device__ inline const uint8_t* row_ptr(const Params& p, int b, int r, int esize) {
  const size_t V = (size_t)p.V;
  if (r <= p.k) return p.target + ((size_t)b * (p.k + 1) + r) * V * esize;
  return p.draft + ((size_t)b * p.k + (r - p.k - 1)) * V * esize;
}

__device__ inline unsigned long long fixmass(float e) {  // e in [0, 1] -> 2^40 fixed point
  return __float2ull_rn(e * 0x1p40f);
}

// ---------------------------------------------------------------------------------------------
// Cluster barrier: release own writes, count the arrival, wait (bounded) for all S members.
// ---------------------------------------------------------------------------------------------
__device__ void cluster_barrier(const Params& p, int b, uint32_t target) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&p.arrive[b], 1u);
    uint32_t it = 0;
    while (__hip_atomic_load(&p.arrive[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++it > SPIN_LIMIT) {
        atomicOr(&p.err[b], 1u);
        break;
      }
    }
  }
  __syncthreads();
  __threadfence();
}

// ---------------------------------------------------------------------------------------------
// Workgroup reductions into thread 0 (fixed order).
// ---------------------------------------------------------------------------------------------
__device__ void block_stats(Smem& sm, float& m, int& a, float& s, uint32_t& fl, float c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
  if (lane == 0) {
    sm.red_f[wave] = m;
    sm.red_i[wave] = a;
    sm.red_g[wave] = s;
    sm.red_u[wave] = fl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < NWAVE; ++w) {
      float mm = m, ss = s;
      lse_combine(mm, ss, sm.red_f[w], sm.red_g[w], c);
      maxarg_combine(m, a, sm.red_f[w], sm.red_i[w]);
      s = ss;
      fl |= sm.red_u[w];
    }
  }
  __syncthreads();
}

__device__ float block_sum(Smem& sm, float v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) sm.red_f[wave] = v;
  __syncthreads();
  float r = 0.0f;
  if (threadIdx.x == 0)
    for (int w = 0; w < NWAVE; ++w) r += sm.red_f[w];
  __syncthreads();
  return r;
}

__device__ void block_maxarg(Smem& sm, float& m, int& a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_maxarg(m, a);
  if (lane == 0) {
    sm.red_f[wave] = m;
    sm.red_i[wave] = a;
  }
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < NWAVE; ++w) maxarg_combine(m, a, sm.red_f[w], sm.red_i[w]);
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// Exact kept threshold of one whole row (top-k, then top-p on the top-k mass), by one workgroup.
// MSD radix select over order-preserving keys, 8-bit digits; per-digit LDS histograms of counts
// and of 2^40 fixed-point masses exp2((l - m) * c) (integer sums: order independent, deterministic).
// ---------------------------------------------------------------------------------------------
template <class E>
__device__ void row_cutoff(Smem& sm, const uint8_t* row, int V, float m, float c, int K, float P,
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
      const uint32_t incl = block_inclusive_scan<uint32_t>(cnt, sm.scan32);
      const unsigned long long minc = block_inclusive_scan<unsigned long long>(ms, sm.scan64);
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
      const unsigned long long minc = block_inclusive_scan<unsigned long long>(ms, sm.scan64);
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

// Gumbel-max over w(x) = exp2((l - m) c) on the kept entries of one row (verify stream, position j).
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

// ---------------------------------------------------------------------------------------------
// Finalisation of a batch row by the last cluster member.
// ---------------------------------------------------------------------------------------------
template <class E>
__device__ void finalize(const Params& p, Smem& sm, int b, bool ok, bool greedy, float T) {
  const int k = p.k;
  const int tid = threadIdx.x;
  constexpr int esize = 16 / E::EPV;
  if (ok && p.err[b] != 0) ok = false;
  if (p.mode == MODE_SAMPLE) {
    if (tid != 0) return;
    if (!ok) {
      p.tokens[b] = -1;
      p.logprobs[b] = __builtin_nanf("");
      return;
    }
    if (greedy) {
      p.tokens[b] = sm.arg[0];
      p.logprobs[b] = 0.0f;
      return;
    }
    float best = 0.0f;
    int y = INT_MAX;
    for (int s = 0; s < p.S; ++s) {
      const FinalPart& f = p.fin[(size_t)b * p.S + s];
      if (f.key > best) {
        best = f.key;
        y = f.idx;
      }
    }
    if (y < 0 || y >= p.V) {  // no candidate: cannot happen for a valid row; report it as unusable
      p.tokens[b] = -1;
      p.logprobs[b] = __builtin_nanf("");
      return;
    }
    const float l = E::load1(row_ptr(p, b, 0, esize), y);
    p.tokens[b] = y;
    p.logprobs[b] = (l - sm.m[0]) / T - logf(sm.Z[0]);
    return;
  }
  if (!ok) {
    if (tid <= k) {
      p.tokens[(size_t)b * (k + 1) + tid] = -1;
      p.logprobs[(size_t)b * (k + 1) + tid] = __builtin_nanf("");
    }
    if (tid < k) p.alpha[(size_t)b * k + tid] = __builtin_nanf("");
    if (tid == 0) p.accept_len[b] = 0;
    return;
  }
  int n;
  int y;
  if (greedy) {
    n = k;
    for (int i = 0; i < k; ++i)
      if (p.draft_tokens[(size_t)b * k + i] != sm.arg[i]) {
        n = i;
        break;
      }
    y = sm.arg[n];
    if (tid < k) p.alpha[(size_t)b * k + tid] = (sm.arg[tid] == sm.arg[k + 1 + tid]) ? 1.0f : 0.0f;
    if (tid <= k) {
      const int t = tid < n ? p.draft_tokens[(size_t)b * k + tid] : (tid == n ? y : -1);
      p.tokens[(size_t)b * (k + 1) + tid] = t;
      p.logprobs[(size_t)b * (k + 1) + tid] = 0.0f;
    }
    if (tid == 0) p.accept_len[b] = n + 1;
    return;
  }
  n = sm.n;
  const float c = 1.4426950408889634f / T;
  // alpha: sum of slice partials in slice order
  if (tid < k) {
    float a = 0.0f;
    for (int s = 0; s < p.S; ++s) a += p.fin[(size_t)b * p.S + s].alpha[tid];
    p.alpha[(size_t)b * k + tid] = a;
  }
  if (tid == 0) {
    float best = 0.0f;
    int bidx = INT_MAX;
    for (int s = 0; s < p.S; ++s) {
      const FinalPart& f = p.fin[(size_t)b * p.S + s];
      if (f.key > best) {
        best = f.key;
        bidx = f.idx;
      }
    }
    sm.pick = bidx;
  }
  __syncthreads();
  y = sm.pick;
  __syncthreads();
  if (y == INT_MAX) {
    // Residual mass vanished in fp32 (rounding): draw from p_n instead, over the whole row.
    const uint8_t* row = row_ptr(p, b, n, esize);
    float best = 0.0f;
    int bidx = INT_MAX;
    for (int j = tid; j < p.V / E::EPV; j += NT)
      gumbel_row_partial<E>(((const uint4*)row)[j], j * E::EPV, sm.m[n], c, sm.thr[n], 1u, (uint32_t)b, (uint32_t)n,
                            p, best, bidx);
    block_maxarg(sm, best, bidx);
    if (tid == 0) sm.pick = bidx;
    __syncthreads();
    y = sm.pick;
    __syncthreads();
  }
  if (y < 0 || y >= p.V) {  // no candidate even over p_n: cannot happen for a valid row
    if (tid <= k) {
      p.tokens[(size_t)b * (k + 1) + tid] = -1;
      p.logprobs[(size_t)b * (k + 1) + tid] = __builtin_nanf("");
    }
    if (tid < k) p.alpha[(size_t)b * k + tid] = __builtin_nanf("");
    if (tid == 0) p.accept_len[b] = 0;
    return;
  }
  if (tid <= k) {
    int t = -1;
    float lp = 0.0f;
    if (tid <= n) {
      t = tid < n ? p.draft_tokens[(size_t)b * k + tid] : y;
      const float l = E::load1(row_ptr(p, b, tid, esize), t);
      lp = (l - sm.m[tid]) / T - logf(sm.Z[tid]);
    }
    p.tokens[(size_t)b * (k + 1) + tid] = t;
    p.logprobs[(size_t)b * (k + 1) + tid] = lp;
  }
  if (tid == 0) p.accept_len[b] = n + 1;
}

// ---------------------------------------------------------------------------------------------
// One work item (b, s).
// ---------------------------------------------------------------------------------------------
template <class E, int VPT>
__device__ void do_item(const Params& p, Smem& sm, uint4* slice, int b, int s) {
  constexpr int EPV = E::EPV;
  constexpr int esize = 16 / EPV;
  const int tid = threadIdx.x;
  const int k = p.k, rows = p.rows, S = p.S;
  const int nvL = p.L / EPV;

  const float T = p.temperature[b];
  const int K = p.top_k[b];
  const float P = p.top_p[b];
  bool ok = !(__builtin_isnan(T) || __builtin_isinf(T) || T < 0.0f) && K >= 0 && !(__builtin_isnan(P) || P <= 0.0f);
  for (int i = 0; i < k; ++i) {
    const int x = p.draft_tokens[(size_t)b * k + i];
    ok = ok && x >= 0 && x < p.V;
  }
  const bool greedy = (T == 0.0f);
  const float c = greedy ? 0.0f : 1.4426950408889634f / T;

  const int x0 = s * p.L;
  const int x1 = min(x0 + p.L, p.V);
  const int nv = x0 < x1 ? (x1 - x0) / EPV : 0;

  // ---- phase A: load the slice, per-slice statistics -------------------------------------
  if (ok) {
    uint4 cur[VPT], nxt[VPT];
    {
      const uint4* src = (const uint4*)(row_ptr(p, b, 0, esize) + (size_t)x0 * esize);
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) cur[u] = src[j];
      }
    }
    for (int r = 0; r < rows; ++r) {
      if (r + 1 < rows) {
        const uint4* src = (const uint4*)(row_ptr(p, b, r + 1, esize) + (size_t)x0 * esize);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          const int j = tid + u * NT;
          if (j < nv) nxt[u] = src[j];
        }
      }
      float m = -INFINITY, sum = 0.0f;
      int a = INT_MAX;
      uint32_t fl = 0;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        const int j = tid + u * NT;
        if (j < nv) {
          if (!greedy) slice[r * nvL + j] = cur[u];
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const float f = E::get(cur[u], e);
            fl |= (__builtin_isnan(f) || f == INFINITY) ? 1u : 0u;
            if (f > m) {
              m = f;
              a = x0 + j * EPV + e;
            }
          }
        }
      }
      if (!greedy && m != -INFINITY) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          const int j = tid + u * NT;
          if (j < nv) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) sum += fexp2((E::get(cur[u], e) - m) * c);
          }
        }
      }
      block_stats(sm, m, a, sum, fl, c);
      if (tid == 0) p.stats[((size_t)b * rows + r) * S + s] = StatPart{m, a, sum, fl};
      if (r + 1 < rows) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) cur[u] = nxt[u];
      }
    }
  }
  cluster_barrier(p, b, (uint32_t)S);

  // ---- phase B: row statistics, kept thresholds -------------------------------------------
  bool trunc = false;
  if (ok) {
    if (tid == 0) sm.bad = 0;
    for (int r = 0; r < rows; ++r) {
      float m = -INFINITY, sum = 0.0f;
      int a = INT_MAX;
      uint32_t fl = 0;
      for (int t = tid; t < S; t += NT) {
        const StatPart sp = p.stats[((size_t)b * rows + r) * S + t];
        float mm = m, ss = sum;
        lse_combine(mm, ss, sp.m, sp.s, c);
        maxarg_combine(m, a, sp.m, sp.arg);
        sum = ss;
        fl |= sp.flags;
      }
      block_stats(sm, m, a, sum, fl, c);
      if (tid == 0) {
        sm.m[r] = m;
        sm.arg[r] = a;
        sm.Z[r] = sum;
        sm.thr[r] = 0;
        if (fl != 0 || m == -INFINITY) sm.bad = 1;
      }
    }
    __syncthreads();
    ok = (sm.bad == 0);
    trunc = ok && !greedy && ((K > 0 && K < p.V) || P < 1.0f);
  }
  uint32_t nbar = 1;
  if (trunc) {
    for (int r = s; r < rows; r += S) {
      uint32_t thr;
      float Z;
      row_cutoff<E>(sm, row_ptr(p, b, r, esize), p.V, sm.m[r], c, K, P, thr, Z);
      if (tid == 0) p.cut[(size_t)b * rows + r] = CutRes{thr, Z, {0, 0}};
    }
    cluster_barrier(p, b, 2u * (uint32_t)S);
    nbar = 2;
    if (tid < rows) {
      const CutRes cr = p.cut[(size_t)b * rows + tid];
      sm.thr[tid] = cr.thr;
      sm.Z[tid] = cr.Z;
    }
    __syncthreads();
  }

  // ---- phase C: accept chain, alpha partials, Gumbel candidate ------------------------------
  if (ok && !greedy) {
    if (tid < rows) sm.invZ[tid] = 1.0f / sm.Z[tid];
    if (tid == 0) {
      int n = k;  // k = 0 in sample mode: the draw below is the sampler's
      for (int i = 0; i < k; ++i) {
        const int x = p.draft_tokens[(size_t)b * k + i];
        const float lt = E::load1(row_ptr(p, b, i, esize), x);
        const float ld = E::load1(row_ptr(p, b, k + 1 + i, esize), x);
        const float pt = key_of<E>(lt) >= sm.thr[i] ? fexp2((lt - sm.m[i]) * c) / sm.Z[i] : 0.0f;
        const float qd = key_of<E>(ld) >= sm.thr[k + 1 + i] ? fexp2((ld - sm.m[k + 1 + i]) * c) / sm.Z[k + 1 + i] : 0.0f;
        const uint4 w4 = philox10(make_uint4((uint32_t)i >> 2, (uint32_t)b, 0u, p.offset), p.key0, p.key1);
        const uint32_t w = (i & 3) == 0 ? w4.x : (i & 3) == 1 ? w4.y : (i & 3) == 2 ? w4.z : w4.w;
        const float u = u24(w);
        const bool accept = pt > 0.0f && (qd == 0.0f || u < pt / qd);
        if (!accept) {
          n = i;
          break;
        }
      }
      sm.n = n;
    }
    __syncthreads();
    const int n = sm.n;
    float best = 0.0f;
    int bidx = INT_MAX;
    for (int i = 0; i < k; ++i) {
      const uint4* vt = slice + i * nvL;
      const uint4* vd = slice + (k + 1 + i) * nvL;
      const float mt = sm.m[i], md = sm.m[k + 1 + i];
      const float it = sm.invZ[i], id = sm.invZ[k + 1 + i];
      const uint32_t tt = sm.thr[i], td = sm.thr[k + 1 + i];
      float acc = 0.0f;
      for (int j = tid; j < nv; j += NT) {
        const uint4 a = vt[j], d = vd[j];
#pragma unroll
        for (int g = 0; g < EPV; g += 4) {
          float r4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float lt = E::get(a, g + e), ld = E::get(d, g + e);
            const float pt = key_of<E>(lt) >= tt ? fexp2((lt - mt) * c) * it : 0.0f;
            const float qd = key_of<E>(ld) >= td ? fexp2((ld - md) * c) * id : 0.0f;
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
      acc = block_sum(sm, acc);
      if (tid == 0) p.fin[(size_t)b * S + s].alpha[i] = acc;
    }
    if (n == k) {
      // bonus draw from p_k (verify stream), or the plain sampler's draw (its own stream)
      const bool smp = p.mode == MODE_SAMPLE;
      const uint32_t tag = smp ? 2u : 1u;
      const uint32_t sb = smp ? (uint32_t)(p.row_b ? p.row_b[b] : b) : (uint32_t)b;
      const uint32_t sj = smp ? (uint32_t)(p.row_pos ? p.row_pos[b] : 0) : (uint32_t)k;
      const uint4* vt = slice + k * nvL;
      for (int j = tid; j < nv; j += NT)
        gumbel_row_partial<E>(vt[j], x0 + j * EPV, sm.m[k], c, sm.thr[k], tag, sb, sj, p, best, bidx);
    }
    block_maxarg(sm, best, bidx);
    if (tid == 0) {
      p.fin[(size_t)b * S + s].key = best;
      p.fin[(size_t)b * S + s].idx = bidx;
    }
  }

  // ---- final arrival; the last member writes the outputs -----------------------------------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t total = (nbar + 1) * (uint32_t)S;
    const uint32_t old = atomicAdd(&p.arrive[b], 1u);
    sm.last = (old == total - 1) ? 1 : 0;
  }
  __syncthreads();
  if (sm.last) {
    __threadfence();
    finalize<E>(p, sm, b, ok, greedy, T);
    __syncthreads();
    if (tid == 0) {
      atomicExch(&p.err[b], 0u);
      atomicExch(&p.arrive[b], 0u);
    }
  }
  __syncthreads();
}

template <class E, int VPT>
__global__ __launch_bounds__(NT) void verify_kernel(Params p) {
  extern __shared__ uint4 slice[];
  __shared__ Smem sm;
  for (;;) {
    if (threadIdx.x == 0) sm.item = (int32_t)atomicAdd(&p.ctrl[0], 1u);
    __syncthreads();
    const int item = sm.item;
    __syncthreads();
    if (item >= p.total_items) break;
    do_item<E, VPT>(p, sm, slice, item / p.S, item % p.S);
  }
  if (threadIdx.x == 0) {
    __threadfence();
    const uint32_t old = atomicAdd(&p.ctrl[1], 1u);
    if (old == gridDim.x - 1) {
      atomicExch(&p.ctrl[0], 0u);
      atomicExch(&p.ctrl[1], 0u);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------------------------
struct Geo {
  int rows, S, L, VPT, esize, EPV;
  size_t lds;
  size_t off_arrive, off_err, off_stats, off_cut, off_fin, total;
};

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static bool make_geo(int32_t B, int32_t k, int32_t V, spec_dtype_t dtype, Geo& g) {
  if (B < 1 || B > (1 << 20) || k < 0 || k > MAXK || V < 8 || V > (1 << 20)) return false;
  if (dtype != SPEC_DTYPE_BF16 && dtype != SPEC_DTYPE_F32) return false;
  g.esize = dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  g.EPV = 16 / g.esize;
  if (V % g.EPV != 0) return false;
  g.rows = 2 * k + 1;
  // Slice data in LDS takes rows * VPT * NT * 16 bytes.  Prefer <= 64 KiB (two items per CU), but
  // grow the slice (up to 4 vectors per thread and ~150 KiB) while a batch row would need more than
  // 32 slices: every member reads all S partials of every row, so exchange traffic grows with S^2.
  int vpt = (int)((64 * 1024) / ((size_t)g.rows * NT * 16));
  if (vpt < 1) vpt = 1;
  if (vpt > 4) vpt = 4;
  while (vpt < 4 && (V + NT * g.EPV * vpt - 1) / (NT * g.EPV * vpt) > 32 &&
         (size_t)g.rows * (vpt + 1) * NT * 16 <= 150 * 1024)
    ++vpt;
  const int Lmax = NT * g.EPV * vpt;
  g.S = (V + Lmax - 1) / Lmax;
  const int per = (V + g.S - 1) / g.S;
  g.L = (per + g.EPV - 1) / g.EPV * g.EPV;
  g.VPT = vpt;
  g.lds = (size_t)g.rows * (g.L / g.EPV) * 16;
  size_t off = 256;  // ctrl
  g.off_arrive = off;
  off = align_up(off + (size_t)B * 4, 256);
  g.off_err = off;
  off = align_up(off + (size_t)B * 4, 256);
  g.off_stats = off;
  off = align_up(off + (size_t)B * g.rows * g.S * sizeof(StatPart), 256);
  g.off_cut = off;
  off = align_up(off + (size_t)B * g.rows * sizeof(CutRes), 256);
  g.off_fin = off;
  off = align_up(off + (size_t)B * g.S * sizeof(FinalPart), 256);
  g.total = off;
  return true;
}

typedef void (*KernelFn)(Params);

template <class E>
static KernelFn pick(int vpt) {
  switch (vpt) {
    case 1: return verify_kernel<E, 1>;
    case 2: return verify_kernel<E, 2>;
    case 3: return verify_kernel<E, 3>;
    default: return verify_kernel<E, 4>;
  }
}

struct DevInfo {
  int state;  // 0 unknown, 1 gfx950, 2 other
  int cus;
};
static DevInfo g_dev[MAXDEV];
static std::mutex g_mu;

static bool device_ok(int dev, int* cus) {
  if (dev < 0 || dev >= MAXDEV) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_dev[dev].state == 0) {
    hipDeviceProp_t pr;
    if (hipGetDeviceProperties(&pr, dev) != hipSuccess) return false;
    g_dev[dev].state = (std::strncmp(pr.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev[dev].cus = pr.multiProcessorCount;
  }
  *cus = g_dev[dev].cus;
  return g_dev[dev].state == 1;
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

static spec_status_t launch(Params& p, const Geo& g, spec_dtype_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!workspace || workspace_bytes < g.total || ((uintptr_t)workspace & 15)) return SPEC_ERR_WORKSPACE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev, &cus)) return SPEC_ERR_UNSUPPORTED_DEVICE;
  p.rows = g.rows;
  p.S = g.S;
  p.L = g.L;
  p.total_items = p.B * g.S;
  uint8_t* ws = (uint8_t*)workspace;
  p.ctrl = (uint32_t*)ws;
  p.arrive = (uint32_t*)(ws + g.off_arrive);
  p.err = (uint32_t*)(ws + g.off_err);
  p.stats = (StatPart*)(ws + g.off_stats);
  p.cut = (CutRes*)(ws + g.off_cut);
  p.fin = (FinalPart*)(ws + g.off_fin);
  KernelFn fn = dtype == SPEC_DTYPE_BF16 ? pick<BF16>(g.VPT) : pick<F32>(g.VPT);
  if (g.lds > 64 * 1024 &&
      hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)g.lds) != hipSuccess)
    return SPEC_ERR_LAUNCH;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, NT, g.lds) != hipSuccess || per_cu < 1)
    return SPEC_ERR_LAUNCH;
  long long grid = (long long)per_cu * cus;
  if (grid > p.total_items) grid = p.total_items;
  if (grid < g.S) return SPEC_ERR_LAUNCH;  // a cluster must fit on the device at once
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(NT), g.lds, (hipStream_t)stream, p);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
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
