// sv_resident.h -- the resident verify kernel of libspecverify (gfx950): one launch per call, every logit
// read from HBM exactly once, for batches whose logits fit on chip.  Included by specverify.hip inside
// namespace sv (it uses that file's helpers: keys, Philox, code masses, race keys).
//
// Method: AReno pull request "feat(engine): MTP training loss and speculative decoding for bailing_v3",
// section "What does this PR do?" (Phase 2: sampler-equivalent target distribution, exact chain rejection
// sampling, unchanged logprobs), its accept-probability table (alpha = sum min(p, q)) and its per-step
// optimisation table (one-pass logprobs, Gumbel-max draws, no host synchronisation).
//
// Shape.  One workgroup of RT = 512 threads per compute unit (its LDS holds part of the data, so one fits);
// workgroup (b, s) owns columns [s L, min((s + 1) L, V)) of all 2k + 1 logit rows of batch row b, with
// L = 4096 nv (nv 16-byte vectors per thread per row).  Each thread's vectors are slots r NV + u (row r,
// vector u): the first RREG slots live in registers, the rest in LDS, filled by 16-byte LDS DMA loads
// (global_load_lds_dwordx4).  All loads are issued at once; the kernel then never touches the logits in
// HBM again.
//
//   phase 1   per row, as its data arrives: NaN-propagating slice max (lowest argmax on greedy rows), the
//             sum of exp2((l - max) c) where the normaliser is the whole row, and, on truncated rows, exact
//             counts of the 512 order-preserving codes below the slice max.  Partials and a flag go out.
//   merge     every workgroup of the batch row waits for the row's flags and merges the partials itself
//             (one wave per logit row, no further exchange): row max, argmax, normaliser and the kept
//             threshold (from the merged code counts; count x 2^40 fixed-point masses, integer sums).  A
//             threshold outside the merged window takes an exact MSD radix select over the row.
//   phase 2   the accept chain (gathered logits, Philox accept uniforms) gives n; each workgroup then adds
//             its columns' share of alpha_i = sum min(p_i, q_i) for every i < k and runs the Gumbel-max
//             race of position n (residual max(p_n - q_n, 0), or the bonus p_k) on its resident data.
//   finish    workgroup s = 0 of the batch row waits for the others' alpha partials and race winners and
//             writes the outputs.  Greedy and sentinel rows are written right after the merge.
//
// Cross-workgroup handoffs.  Partials are stored with agent-scope relaxed atomics, drained, and followed by
// a 64-bit flag holding this dispatch's tag (a hash of the queue address and the dispatch id, which every
// workgroup of one launch shares and no other launch has); readers poll the flags with agent-scope loads.
// A flag left by an earlier call, or workspace garbage, never equals the tag, so the workspace needs no
// initialisation and no counter is reset.  Every wait is bounded (wait_limit ticks of the 100 MHz clock):
// a workgroup that gives up abandons its batch row, whose outputs become a sentinel row, and exits, so the
// grid always drains.  The launch is cooperative: the runtime refuses it unless the grid is co-resident.
#pragma once

constexpr int RT = 512;           // threads per resident workgroup
constexpr int RWAVE = RT / 64;    // waves per resident workgroup
constexpr int RREG = 32;          // vector slots per thread held in registers (128 VGPRs)
constexpr int RWIN = WTOP / 2;    // packed words of one row-slice's code counts (2 x 16-bit)
// Rows cut by top-k with K <= RKNARROW count only the RWNARROW codes below each slice max (one octave of
// bf16 values for a positive max: where such a cut usually lies); other truncated rows count WTOP codes.
// The fewer logits fall in the window, the fewer LDS atomics phase 1 issues.
constexpr int RKNARROW = 256;
constexpr uint32_t RWNARROW = 128;
constexpr uint64_t RWAIT_DEFAULT = 20000000ull;  // 200 ms of the 100 MHz clock

// Vector slots per thread per logit row, by k (at most ~50 slots per thread: 32 in registers, the rest
// in LDS); slices are at most 4096 nv <= 61440 logits, so a code count fits 16 bits.
__host__ __device__ constexpr int rnv_max(int k) { return k == 1 ? 15 : k == 2 ? 10 : k == 3 ? 7 : 5; }

struct RPart {  // per (batch row, slice, logit row): slice statistics (exchange 1)
  float m;        // slice max (NaN-propagating)
  int32_t arg;    // lowest index of the slice max (greedy rows)
  float s;        // sum of exp2((l - m) c) over the slice (rows whose normaliser is the whole row)
  uint32_t flags; // bit 0: NaN or +inf seen
};

struct RFin {  // per (batch row, slice): alpha partials and the race candidate (exchange 2)
  float alpha[MAXK];
  float key;
  int32_t idx;
  float val;
  uint32_t pad;
};

struct RParams {
  const uint8_t* target;
  const uint8_t* draft;
  const int32_t* draft_tokens;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t B, k, V, S, nv, L;  // S slices of L = 4096 nv columns per batch row
  uint32_t key0, key1, offset;
  uint64_t salt;              // mixed into the dispatch tag (seed, offset and sizes of this call)
  uint64_t wait_limit;        // bound on each wait, in 100 MHz clock ticks
  int32_t* tokens;
  int32_t* accept_len;
  float* logprobs;
  float* alpha;
  RPart* part;                // [B][S][rows]
  uint32_t* win;              // [B][S][rows][RWIN]
  RFin* fin;                  // [B][S]
  unsigned long long* flag1;  // [B][S]
  unsigned long long* flag2;  // [B][S]
  unsigned long long* trace;  // [B S][16] phase timestamps: instrumented builds only
};

// Phase timestamps of instrumented builds (compiled with -DSV_TRACE); no-ops otherwise.
#ifdef SV_TRACE
#define RTRACE(p, slot)                                                                       \
  do {                                                                                        \
    if (threadIdx.x == 0 && (p).trace) (p).trace[(size_t)blockIdx.x * 16 + (slot)] = wall_clock64(); \
  } while (0)
#else
#define RTRACE(p, slot) \
  do {                  \
  } while (0)
#endif

// The dispatch id (the LLVM intrinsic has no clang builtin of its own).
extern "C" __device__ unsigned long long sv_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// This dispatch's tag: the queue address, the dispatch id (the queue's packet index) and the call's salt,
// mixed; never 0 and never one byte repeated eight times (uniform fills of the workspace).
__device__ inline unsigned long long dispatch_tag(uint64_t salt) {
  uint64_t h = (uint64_t)(uintptr_t)__builtin_amdgcn_queue_ptr() * 0x9E3779B97F4A7C15ull;
  h ^= sv_dispatch_id() + 0x632BE59BD9B4E019ull + (h << 6) + (h >> 2);
  h ^= salt * 0xC2B2AE3D27D4EB4Full;
  h ^= h >> 29;
  h *= 0xBF58476D1CE4E5B9ull;
  h ^= h >> 32;
  if ((h & 0xffull) * 0x0101010101010101ull == h) h ^= 0x5A00ull;
  return h;
}

__device__ inline void st64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline unsigned long long ld64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until at most N vector-memory operations of this wave are outstanding (the LDS DMA loads are not
// tracked by the compiler, so their consumers wait explicitly).  Fences keep memory operations on their side.
template <int N>
__device__ inline void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Threads 0..n-1 each poll one flag until it holds `tag`; true in every thread if all did within the limit.
__device__ inline bool wait_flags(const unsigned long long* flags, int n, unsigned long long tag, uint64_t limit) {
  bool ok = true;
  const int tid = threadIdx.x;
  if (tid < n) {
    const uint64_t t0 = (uint64_t)wall_clock64();
    while (ld64(&flags[tid]) != tag) {
      if ((uint64_t)wall_clock64() - t0 > limit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  return __syncthreads_and(ok) != 0;
}

struct RSmem {
  unsigned long long wq[2];
  float wf[RWAVE], wg[RWAVE];
  int32_t wi[RWAVE];
  uint32_t wu[RWAVE];
  float wacc[MAXK][RWAVE];
  // per logit row after the merge
  float m[MAXROWS], Z[MAXROWS], lz[MAXROWS], fthr[MAXROWS], gath[MAXROWS];
  int32_t arg[MAXROWS];
  uint32_t bad[MAXROWS], fb[MAXROWS];
  int32_t tok[MAXK];
  float u[MAXK];
  int32_t n;
  float rf[2][RWAVE];        // phase 1 reductions (two buffers, alternating)
  int32_t ri[2][RWAVE];
  uint32_t hist[2][WTOP];    // phase 1: code counts of a row (two arrays, by row parity; zero between uses)
};


// The LDS byte address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* q) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)q;
}

// Increment of an LDS counter (ds_add_u32, no return).  Written as an instruction of its own because the
// compiler cannot tell a counter array from the LDS DMA destination and would wait for every DMA load in
// flight before each atomic; the counters are read only after an lds_sync(), which waits for it.
__device__ __forceinline__ void lds_inc(uint32_t lds_byte_addr, uint32_t one) {
  asm volatile("ds_add_u32 %0, %1" : : "v"(lds_byte_addr), "v"(one) : "memory");
}
// A value the compiler cannot fold or rematerialise (kept in the register class it was made in).
__device__ __forceinline__ uint32_t opaque_v(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// ---- wave reductions on the DPP lane network (result in lane 63), and phase 1's workgroup reductions ----
// Steps: swap neighbours, swap pairs (quad permutes), mirror half rows, mirror rows (every lane then holds
// its 16-lane row's value), then rows 1 and 3 take lane 15 of the row before and rows 2 and 3 take lane 31.
template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, ROWM, 0xF, false));
}
template <int CTRL, int ROWM = 0xF>
__device__ __forceinline__ int dpp_i(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWM, 0xF, false);
}
__device__ __forceinline__ float dpp_wave_sum(float x) {
  x += dpp_f<0xB1>(0.0f, x);
  x += dpp_f<0x4E>(0.0f, x);
  x += dpp_f<0x141>(0.0f, x);
  x += dpp_f<0x140>(0.0f, x);
  x += dpp_f<0x142, 0xA>(0.0f, x);
  x += dpp_f<0x143, 0xC>(0.0f, x);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float dpp_wave_max(float x) {  // NaN-propagating
  x = nan_max(x, dpp_f<0xB1>(-INFINITY, x));
  x = nan_max(x, dpp_f<0x4E>(-INFINITY, x));
  x = nan_max(x, dpp_f<0x141>(-INFINITY, x));
  x = nan_max(x, dpp_f<0x140>(-INFINITY, x));
  x = nan_max(x, dpp_f<0x142, 0xA>(-INFINITY, x));
  x = nan_max(x, dpp_f<0x143, 0xC>(-INFINITY, x));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ int dpp_wave_imin(int x) {
  x = min(x, dpp_i<0xB1>(INT_MAX, x));
  x = min(x, dpp_i<0x4E>(INT_MAX, x));
  x = min(x, dpp_i<0x141>(INT_MAX, x));
  x = min(x, dpp_i<0x140>(INT_MAX, x));
  x = min(x, dpp_i<0x142, 0xA>(INT_MAX, x));
  x = min(x, dpp_i<0x143, 0xC>(INT_MAX, x));
  return __builtin_amdgcn_readlane(x, 63);
}

// Workgroup reductions with one barrier each: buffer `buf` of two, which consecutive reductions alternate
// (a wave writes buffer b again only after the barrier of the reduction in between, which every reader of
// b's previous contents has passed).
__device__ __forceinline__ float rblock_max2(RSmem& sm, float x, int buf) {
  x = dpp_wave_max(x);
  if ((threadIdx.x & 63) == 0) sm.rf[buf][threadIdx.x >> 6] = x;
  lds_sync();
  float m = sm.rf[buf][0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) m = nan_max(m, sm.rf[buf][w]);
  return m;
}
__device__ __forceinline__ float rblock_sum2(RSmem& sm, float x, int buf) {
  x = dpp_wave_sum(x);
  if ((threadIdx.x & 63) == 0) sm.rf[buf][threadIdx.x >> 6] = x;
  lds_sync();
  float t = sm.rf[buf][0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) t += sm.rf[buf][w];
  return t;
}
__device__ __forceinline__ int rblock_imin2(RSmem& sm, int x, int buf) {
  x = dpp_wave_imin(x);
  if ((threadIdx.x & 63) == 0) sm.ri[buf][threadIdx.x >> 6] = x;
  lds_sync();
  int t = sm.ri[buf][0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) t = min(t, sm.ri[buf][w]);
  return t;
}

// ---- 512-thread block reductions (fixed order: deterministic) ----
__device__ __forceinline__ float rblock_max(RSmem& sm, float m) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = nan_max(m, __shfl_xor(m, o, 64));
  if (lane == 0) sm.wf[wave] = m;
  lds_sync();
  m = sm.wf[0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) m = nan_max(m, sm.wf[w]);
  lds_sync();
  return m;
}

__device__ __forceinline__ void rblock_maxarg(RSmem& sm, float& m, int& a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  wave_maxarg(m, a);
  if (lane == 0) {
    sm.wf[wave] = m;
    sm.wi[wave] = a;
  }
  lds_sync();
  m = sm.wf[0];
  a = sm.wi[0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) maxarg_combine(m, a, sm.wf[w], sm.wi[w]);
  lds_sync();
}

__device__ __forceinline__ float rblock_sum(RSmem& sm, float v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) sm.wg[wave] = v;
  lds_sync();
  v = sm.wg[0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) v += sm.wg[w];
  lds_sync();
  return v;
}

// Workgroup (NaN-propagating max, sum of exp2((l - max) c)) of per-thread pairs, into every thread.
__device__ __forceinline__ void block_stats_r(RSmem& sm, float& m, float& sum, float c) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(sum, o, 64);
    float mm = m, ss = sum;
    lse_combine(mm, ss, m2, s2, c);
    m = nan_max(m, m2);
    sum = ss;
  }
  if (lane == 0) {
    sm.wf[wave] = m;
    sm.wg[wave] = sum;
  }
  lds_sync();
  m = sm.wf[0];
  sum = sm.wg[0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) {
    float mm = m, ss = sum;
    lse_combine(mm, ss, sm.wf[w], sm.wg[w], c);
    m = nan_max(m, sm.wf[w]);
    sum = ss;
  }
  lds_sync();
}

__device__ __forceinline__ uint32_t rblock_or(RSmem& sm, uint32_t v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool any = __ballot(v != 0) != 0ull;
  if (lane == 0) sm.wu[wave] = any ? 1u : 0u;
  lds_sync();
  uint32_t o = 0u;
#pragma unroll
  for (int w = 0; w < RWAVE; ++w) o |= sm.wu[w];
  lds_sync();
  return o;
}

__device__ __forceinline__ void rblock_race(RSmem& sm, float& best, int& bidx, float& bval) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float k2 = __shfl_xor(best, o, 64);
    const int i2 = __shfl_xor(bidx, o, 64);
    const float v2 = __shfl_xor(bval, o, 64);
    race_take(best, bidx, bval, k2, i2, v2);
  }
  if (lane == 0) {
    sm.wf[wave] = best;
    sm.wi[wave] = bidx;
    sm.wg[wave] = bval;
  }
  lds_sync();
  best = sm.wf[0];
  bidx = sm.wi[0];
  bval = sm.wg[0];
#pragma unroll
  for (int w = 1; w < RWAVE; ++w) race_take(best, bidx, bval, sm.wf[w], sm.wi[w], sm.wg[w]);
  lds_sync();
}

// ---- wave-level helpers of the merge ----
template <class T>
__device__ inline T wave_excl_scan(T v, T& total) {
  const T incl = wave_incl_scan(v);
  total = __shfl(incl, 63, 64);
  return incl - v;
}

// Kept threshold of one row from its merged code counts, by one wave: entry e of cnt (e < WTOP) counts code
// keym - e.  Lane l owns entries 8l .. 8l + 7.  The same selection as select_run: the first entry where the
// running count reaches K (top-k), then within the kept prefix the first where the running mass reaches
// P Z_K (or P Z with top-k off; ztot_fixed = Z in 2^40 fixed point).  Entries below lim are exact (every
// slice counted them); returns false if a threshold lies at entry lim or further down.
__device__ inline bool wave_select(const uint32_t* cnt, uint32_t keym, float m, float c, bool useK, int K, bool useP,
                                   float P, double ztot_fixed, int lim, uint32_t& thr, unsigned long long& zsel) {
  const int lane = threadIdx.x & 63;
  uint32_t ce[8];
  unsigned long long me[8];
  uint32_t csum = 0;
  unsigned long long msum = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ce[e] = cnt[8 * lane + e];
    me[e] = code_mass(ce[e], keym - (uint32_t)(8 * lane + e), m, c);
    csum += ce[e];
    msum += me[e];
  }
  uint32_t ctot;
  unsigned long long mtot;
  const uint32_t cex = wave_excl_scan<uint32_t>(csum, ctot);
  const unsigned long long mex = wave_excl_scan<unsigned long long>(msum, mtot);
  int selk = WTOP;  // entry of the top-k cut (WTOP: not in the window)
  unsigned long long zk = 0;
  if (useK) {
    int found = WTOP;
    unsigned long long zf = 0;
    uint32_t run = cex;
    unsigned long long mrun = mex;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (found == WTOP && run < (uint32_t)K && run + ce[e] >= (uint32_t)K) {
        found = 8 * lane + e;
        zf = mrun + me[e];
      }
      run += ce[e];
      mrun += me[e];
    }
    // the lowest lane that found it holds the cut
    const unsigned long long ball = __ballot(found < WTOP);
    if (!ball) return false;
    const int src = __ffsll((long long)ball) - 1;
    selk = __shfl(found, src, 64);
    zk = __shfl(zf, src, 64);
    if (selk >= lim) return false;  // past the codes every slice counted
  }
  int sel = selk;
  unsigned long long z = zk;
  if (useP) {
    const double target = (double)P * (useK ? (double)zk : ztot_fixed);
    int found = WTOP;
    unsigned long long zf = 0;
    unsigned long long mrun = mex;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int idx = 8 * lane + e;
      if (found == WTOP && idx <= selk && (double)mrun < target && (double)(mrun + me[e]) >= target) {
        found = idx;
        zf = mrun + me[e];
      }
      mrun += me[e];
    }
    const unsigned long long ball = __ballot(found < WTOP);
    if (!ball) return false;
    const int src = __ffsll((long long)ball) - 1;
    sel = __shfl(found, src, 64);
    z = __shfl(zf, src, 64);
    if (sel >= lim) return false;  // past the codes every slice counted
  }
  thr = keym - (uint32_t)sel;
  zsel = z;
  return true;
}


// Sampling parameters of batch row b (as row_params, for the resident kernel's arguments).
__device__ inline RowParams row_params_r(const RParams& p, int b) {
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
  q.cand = false;
  return q;
}

// Slot SL of this thread's resident vectors: a register, or its LDS entry (FIRST: the first read of an LDS
// slot, which waits for its DMA load -- loads were issued register slots first, then LDS slots in order, so
// NS - 1 - SL vector-memory operations may still be outstanding behind it).
template <int SL, int NREG, int NLDS, bool FIRST>
__device__ __forceinline__ uint4 slot(const uint4 (&v)[NREG], const uint4* ldsv, int tid) {
  if constexpr (SL < NREG) {
    return v[SL];
  } else {
    if constexpr (FIRST) vm_wait<NREG + NLDS - 1 - SL>();
    return ldsv[(SL - NREG) * RT + tid];
  }
}

// A workgroup-uniform condition in a scalar register (so branches on it are scalar, not exec-masked).
__device__ inline bool uni(bool c) { return __builtin_amdgcn_readfirstlane((int)c) != 0; }

// Compile-time loop: f(std::integral_constant<int, I>) for I = A .. B-1.
template <int A, int B, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (A < B) {
    f(std::integral_constant<int, A>{});
    static_for<A + 1, B>(f);
  }
}

// Exact kept threshold of one whole bf16 row by the whole workgroup, reading the row from memory: the MSD
// radix select of row_cutoff (8-bit digits; per-digit counts and 2^40 fixed-point masses, integer sums), with
// the digit scans done by wave 0.  scratch: LDS of at least 768 words, 8-byte aligned.
__device__ __forceinline__ void r_cutoff(RSmem& sm, uint32_t* scratch, const uint8_t* row, int V, float m, float c,
                                         int K, float P, uint32_t& thr_out, float& Z_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t* hcnt = scratch;
  unsigned long long* hmass = (unsigned long long*)(scratch + 256);
  const uint4* src = (const uint4*)row;
  const int nvec = V / 8;
  uint32_t thr = 0;
  unsigned long long zk = 0;
  bool have_zk = false;
  for (int pass = 0; pass < 2; ++pass) {
    const bool topk = pass == 0;
    if (topk && !(K > 0 && K < V)) continue;
    if (!topk && !(P < 1.0f)) continue;
    uint32_t prefix = 0, need = (uint32_t)K;
    unsigned long long mabove = 0;
    double target = 0.0;
    for (int lev = 0; lev < 2; ++lev) {
      const int shift = 8 - 8 * lev;
      for (int i = tid; i < 256; i += RT) {
        hcnt[i] = 0;
        hmass[i] = 0;
      }
      __syncthreads();
      for (int j = tid; j < nvec; j += RT) {
        const uint4 w = src[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = BF16::get(w, e);
          const uint32_t key = key16f(f);
          if (key >= (topk ? 0u : thr) && (lev == 0 || (key >> 8) == prefix)) {
            const uint32_t d = (key >> shift) & 255u;
            if (topk) atomicAdd(&hcnt[d], 1u);
            atomicAdd(&hmass[d], fixmass(fexp2((f - m) * c)));
          }
        }
      }
      __syncthreads();
      if (tid < 64) {
        // lane l scans digits 255 - 4l .. 252 - 4l (descending key order)
        uint32_t ce[4];
        unsigned long long me[4];
        uint32_t cs = 0;
        unsigned long long ms = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 255 - 4 * lane - e;
          ce[e] = hcnt[d];
          me[e] = hmass[d];
          cs += ce[e];
          ms += me[e];
        }
        uint32_t ctot;
        unsigned long long mtot;
        const uint32_t cex = wave_excl_scan<uint32_t>(cs, ctot);
        const unsigned long long mex = wave_excl_scan<unsigned long long>(ms, mtot);
        if (!topk && lev == 0) {
          if (!have_zk) zk = mtot;
          target = (double)P * (double)zk;
        }
        int found = -1;
        uint32_t fex = 0;
        unsigned long long fmx = 0, fm = 0;
        uint32_t run = cex;
        unsigned long long mrun = mex;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool hit = topk ? (found < 0 && run < need && run + ce[e] >= need)
                                : (found < 0 && (double)(mabove + mrun) < target &&
                                   (double)(mabove + mrun + me[e]) >= target);
          if (hit) {
            found = 255 - 4 * lane - e;
            fex = run;
            fmx = mrun;
            fm = me[e];
          }
          run += ce[e];
          mrun += me[e];
        }
        const unsigned long long ball = __ballot(found >= 0);
        if (lane == 0) sm.wu[0] = 0xffffffffu;
        if (ball) {
          const int src_lane = __ffsll((long long)ball) - 1;
          const int d = __shfl(found, src_lane, 64);
          const uint32_t e0 = __shfl(fex, src_lane, 64);
          const unsigned long long m0 = __shfl(fmx, src_lane, 64), m1 = __shfl(fm, src_lane, 64);
          if (lane == 0) {
            sm.wu[0] = (uint32_t)d;
            sm.wu[1] = e0;
            sm.wq[0] = m0;
            sm.wq[1] = m1;
          }
        }
      }
      __syncthreads();
      const uint32_t d = sm.wu[0];
      const uint32_t e0 = sm.wu[1];
      const unsigned long long m0 = sm.wq[0], m1 = sm.wq[1];
      __syncthreads();
      if (d == 0xffffffffu) {  // not reachable for a valid row (the counts and masses cover it)
        thr_out = thr;
        Z_out = (float)((double)(have_zk ? zk : 0ull) * 0x1p-40);
        return;
      }
      need -= e0;
      mabove += m0;
      prefix = (prefix << 8) | d;
      if (lev == 1) zk = mabove + m1;
    }
    thr = prefix;
    have_zk = true;
  }
  thr_out = thr;
  Z_out = (float)((double)zk * 0x1p-40);
}

// ---- the kernel ----
template <int KK>
struct RG {
  static constexpr int ROWS = 2 * KK + 1;
  static constexpr int NV = rnv_max(KK);
  static constexpr int NS = ROWS * NV;
  static constexpr int NREG = NS < RREG ? NS : RREG;
  static constexpr int NLDS = NS - NREG;
};

// A uniform global pointer as an opaque value in scalar registers.  Selecting between two kernel-argument
// fields by a runtime condition otherwise becomes a load through a select of their addresses, which puts the
// arguments in scratch memory; every later load then waits behind that scratch read.
__device__ __forceinline__ const uint8_t* gbase(const void* q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(const uint8_t __attribute__((address_space(1)))*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// A raw buffer resource over `bytes` bytes at `base` (word 3: the gfx9-family raw 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS DMA load of `size` bytes per lane (4 or 16) at byte offset `off` of the buffer into this wave's LDS
// block at `lds` (lane l writes lds + l * size).  Counted by vmcnt like any vector-memory load.
__device__ __forceinline__ void dma_lds(__amdgpu_buffer_rsrc_t rs, uint32_t off, void* lds, int size) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, 0);
}

// The 2k + 1 logit rows of one batch row (targets 0..k, then drafts), from two uniform bases.
struct RRows {
  const uint8_t* t;  // target row 0 of the batch row
  const uint8_t* d;  // draft row 0 of the batch row
  size_t rb;         // bytes per row
  int k;
  __device__ __forceinline__ const uint8_t* operator()(int r) const {
    const uint8_t* const tt = t;
    const uint8_t* const dd = d;
    return r <= k ? tt + (size_t)r * rb : dd + (size_t)(r - k - 1) * rb;
  }
};

__device__ inline void r_sentinel(const RParams& p, int b, int KK) {
  const int tid = threadIdx.x;
  const size_t ob = (size_t)b * (KK + 1);
  if (tid <= KK) {
    p.tokens[ob + tid] = -1;
    p.logprobs[ob + tid] = __builtin_nanf("");
  }
  if (tid < KK) p.alpha[(size_t)b * KK + tid] = __builtin_nanf("");
  if (tid == 0) p.accept_len[b] = 0;
}

// Philox-4x32-10 as philox10_uk (the key is uniform: kernel arguments), with the rounds in a loop: the
// resident kernel instantiates it at every vector slot of its unrolled loops, where ten inlined rounds would
// multiply the code size.
__device__ __forceinline__ uint4 philox10_loop(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll 1
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t n0 = xor3_uk((uint32_t)(p1 >> 32), c.y, k0);
    const uint32_t n2 = xor3_uk((uint32_t)(p0 >> 32), c.w, k1);
    c.y = (uint32_t)p1;
    c.w = (uint32_t)p0;
    c.x = n0;
    c.z = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Two Philox-4x32-10 blocks (counters c0, c1) under one uniform key, rounds interleaved: two independent
// chains.
__device__ __forceinline__ void philox10x2_loop(uint4& c0, uint4& c1, uint32_t k0, uint32_t k1) {
#pragma unroll 1
  for (int r = 0; r < 10; ++r) {
    const uint64_t a0 = (uint64_t)0xD2511F53u * c0.x, a1 = (uint64_t)0xD2511F53u * c1.x;
    const uint64_t b0 = (uint64_t)0xCD9E8D57u * c0.z, b1 = (uint64_t)0xCD9E8D57u * c1.z;
    const uint32_t n00 = xor3_uk((uint32_t)(b0 >> 32), c0.y, k0), n01 = xor3_uk((uint32_t)(b1 >> 32), c1.y, k0);
    const uint32_t n20 = xor3_uk((uint32_t)(a0 >> 32), c0.w, k1), n21 = xor3_uk((uint32_t)(a1 >> 32), c1.w, k1);
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

// Gumbel-max candidates of one 8-logit vector at x (a multiple of 8): weights wr, logits of the row drawn
// from in wa; the vector's two Philox blocks are computed together.
__device__ __forceinline__ void r_race8(const RParams& p, int b, int j_pos, int x, const float (&wr)[8],
                                        const uint4& wa, float& best, int& bidx, float& bval) {
  const uint32_t tagj = (1u << 24) | (uint32_t)j_pos;
  uint4 c0 = make_uint4((uint32_t)x >> 2, (uint32_t)b, tagj, p.offset);
  uint4 c1 = make_uint4(((uint32_t)x >> 2) + 1u, (uint32_t)b, tagj, p.offset);
  philox10x2_loop(c0, c1, p.key0, p.key1);
  const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) race_take(best, bidx, bval, race_key_or_none(wr[e], words[e]), x + e, BF16::get(wa, e));
}

// Gumbel-max candidates of one 4-logit group (weights wr, logits of the row drawn from at g of vector wa).
__device__ __forceinline__ void r_race4(const RParams& p, int b, int j_pos, int x, const float (&wr)[4],
                                        const uint4& wa, int g, float& best, int& bidx, float& bval) {
  const uint4 w4 = philox10_loop(make_uint4((uint32_t)x >> 2, (uint32_t)b, (1u << 24) | (uint32_t)j_pos, p.offset),
                                 p.key0, p.key1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (wr[e] > 0.0f) {
      const uint32_t word = e == 0 ? w4.x : e == 1 ? w4.y : e == 2 ? w4.z : w4.w;
      race_take(best, bidx, bval, race_key(wr[e], word), x + e, BF16::get(wa, g + e));
    }
  }
}

template <int KK>
__global__ __launch_bounds__(RT, 1) void kr_verify(RParams p) {
  using G = RG<KK>;
  constexpr int ROWS = G::ROWS, NV = G::NV, NREG = G::NREG, NLDS = G::NLDS;
  __shared__ uint4 ldsv[NLDS > 0 ? NLDS * RT : 1];
  __shared__ RSmem sm;
  __shared__ __align__(8) uint32_t cnt[ROWS][WTOP];  // merge: each row's merged code counts (one wave per row)
  __shared__ uint32_t gdma[64];                      // the draft-token logits' dwords (LDS DMA, wave 0)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / p.S, s = blockIdx.x - b * p.S;
  const int x0 = s * p.L;
  const int nvs = min(p.L, p.V - x0) / BF16::EPV;  // valid vectors of this slice
  const unsigned long long tag = dispatch_tag(p.salt);
  RRows rows;
  rows.rb = (size_t)p.V * 2;
  rows.k = KK;
  rows.t = gbase(p.target) + (size_t)b * (KK + 1) * rows.rb;
  rows.d = gbase(p.draft) + (size_t)b * KK * rows.rb;
  // sampling parameters and draft tokens first: tiny uniform loads, done before the slice's data arrives
  const RowParams q = row_params_r(p, b);
  int32_t tok[KK];
#pragma unroll
  for (int i = 0; i < KK; ++i) tok[i] = p.draft_tokens[(size_t)b * KK + i];
  // buffer resources over the batch row's target and draft rows, for the LDS DMA loads (buffer loads: the
  // global form of the LDS DMA load makes the compiler wait for every load in flight before any use)
  const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(rows.t, (uint32_t)((KK + 1) * rows.rb));
  const __amdgpu_buffer_rsrc_t rs_d = make_rsrc(rows.d, (uint32_t)(KK * rows.rb));
  RTRACE(p, 0);

  // ---- the slice's loads go out next (register slots, then the LDS slots' DMA loads, in slot order) ----
  uint4 v[NREG];
  static_for<0, NREG>([&](auto SI) {
    constexpr int sl = decltype(SI)::value;
    constexpr int r = sl / NV, u = sl - r * NV;
    // clamped, so that every lane loads a valid vector without a branch (every use masks lanes past nvs)
    const int j = min(tid + u * RT, max(nvs - 1, 0));
    v[sl] = ((const uint4*)(rows(r) + (size_t)x0 * 2))[j];
    if constexpr (u == NV - 1) __builtin_amdgcn_sched_barrier(0);  // rows in order: row 0's data lands first
  });
  __builtin_amdgcn_sched_barrier(0);
  static_for<NREG, NREG + NLDS>([&](auto SI) {
    constexpr int sl = decltype(SI)::value;
    constexpr int r = sl / NV, u = sl - r * NV;
    const int j = min(tid + u * RT, max(nvs - 1, 0));  // clamped: every lane loads a valid vector
    dma_lds(r <= KK ? rs_t : rs_d, (uint32_t)((r <= KK ? r : r - KK - 1) * rows.rb + (size_t)x0 * 2 + (size_t)j * 16),
            ldsv + (sl - NREG) * RT + (tid & ~63), 16);
    __builtin_amdgcn_sched_barrier(0);
  });
  bool gok = false;
  int gx = 0;
  if (tid < KK) {
    const uint4 w4 = philox10(make_uint4(0u, (uint32_t)b, 0u, p.offset), p.key0, p.key1);
    const int qq = tid & 3;
    sm.u[tid] = u24(qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w);
    int tv = 0;
#pragma unroll
    for (int i = 0; i < KK; ++i) tv = tid == i ? tok[i] : tv;
    sm.tok[tid] = tv;
  }
  // phase 1's code counts start at zero (the first row's max reduction orders this before their use)
  for (int i = tid; i < 2 * WTOP; i += RT) (&sm.hist[0][0])[i] = 0u;

  // ---- phase 1: per row statistics, as the data arrives ----
  const bool ok_u = uni(q.ok), greedy = uni(q.greedy), hist = uni(q.trunc), zrow = uni(!q.useK);
  const int nvu = p.nv;  // vector slots per row in use (the kernel is compiled for NV)
  int rbuf = 0;  // reduction buffer of the next phase-1 workgroup reduction
  // codes counted exactly per slice; the 64 entries above them are per-lane spares that take every logit
  // further down (branch-free counting), so their counts mean nothing
  const uint32_t wlim = (q.useK && q.K <= RKNARROW) ? RWNARROW : (uint32_t)(WTOP - 64);
  const uint32_t spare2 = (wlim + (uint32_t)lane) * 0x10001u;
  RPart* prt = p.part + ((size_t)b * p.S + s) * ROWS;
  uint32_t* win = p.win + ((size_t)b * p.S + s) * ROWS * RWIN;
  static_for<0, ROWS>([&](auto RI) {
    constexpr int r = decltype(RI)::value;
    constexpr int last = r * NV + NV - 1;  // the row's last slot
    // the row's LDS slots were DMA'd behind every earlier slot: wait for them once, before the row
    if constexpr (last >= NREG) vm_wait<NREG + NLDS - 1 - last>();
    if constexpr (r == ROWS - 1) {
      // the logits at the draft tokens (lane i < k: target row i, lane k + i: draft row i), which only the
      // accept chain reads, after the merge: an LDS DMA load each of the dword holding the logit, issued
      // once every slice load has landed and read after the row
      if (tid < 2 * KK) {
#pragma unroll
        for (int i = 0; i < KK; ++i) gx = (tid == i || tid == KK + i) ? tok[i] : gx;
        gok = gx >= 0 && gx < p.V;
        const int rg = tid < KK ? tid : tid + 1;
        const uint32_t off = (uint32_t)((rg <= KK ? rg : rg - KK - 1) * rows.rb) + (gok ? (uint32_t)(gx >> 1) * 4u : 0u);
        dma_lds(rg <= KK ? rs_t : rs_d, off, gdma, 4);
      }
    }
    RTRACE(p, 8 + (r < 5 ? r : 4));
    float m = -INFINITY, sum = 0.0f;
    int a = INT_MAX;
    if (ok_u) {
      // pass A: NaN-propagating max (four independent chains), then the workgroup max
      float mq[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      static_for<0, NV>([&](auto UI) {
        constexpr int u = decltype(UI)::value;
        if (u < nvu) {
          const uint4 w = slot<r * NV + u, NREG, NLDS, false>(v, ldsv, tid);
          float vm = nan_max(nan_max(nan_max(BF16::get(w, 0), BF16::get(w, 1)), nan_max(BF16::get(w, 2), BF16::get(w, 3))),
                             nan_max(nan_max(BF16::get(w, 4), BF16::get(w, 5)), nan_max(BF16::get(w, 6), BF16::get(w, 7))));
          mq[u & 3] = nan_max(mq[u & 3], tid + u * RT < nvs ? vm : -INFINITY);
        }
      });
      m = rblock_max2(sm, nan_max(nan_max(mq[0], mq[1]), nan_max(mq[2], mq[3])), rbuf);
      rbuf ^= 1;
      if (greedy) {
        // lowest index holding the max: per thread the first vector holding it, the first entry in it
        if (uni(m == m && m > -INFINITY)) {
          int ia = INT_MAX;
          static_for<0, NV>([&](auto UI) {
            constexpr int u = decltype(UI)::value;
            if (u < nvu) {
              const uint4 w = slot<r * NV + u, NREG, NLDS, false>(v, ldsv, tid);
              const int j = tid + u * RT;
              int e1 = INT_MAX;
#pragma unroll
              for (int e = 7; e >= 0; --e) e1 = BF16::get(w, e) == m ? e : e1;
              ia = (ia == INT_MAX && e1 != INT_MAX && j < nvs) ? x0 + 8 * j + e1 : ia;
            }
          });
          a = rblock_imin2(sm, ia, rbuf);
          rbuf ^= 1;
        }
      } else if (zrow && uni(m == m && m > -INFINITY)) {
        // pass A2 (rows whose normaliser is the whole row): sum of exp2((l - m) c) against the slice max
        const float nmc = -m * q.c;
        float sq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        static_for<0, NV>([&](auto UI) {
          constexpr int u = decltype(UI)::value;
          if (u < nvu) {
            const uint4 w = slot<r * NV + u, NREG, NLDS, false>(v, ldsv, tid);
            float ex[8];  // independent exponentials, then a tree (no result waits on the one before)
#pragma unroll
            for (int e = 0; e < 8; ++e) ex[e] = fexp2(fmaf(BF16::get(w, e), q.c, nmc));
            const float t = ((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7]));
            sq[u & 3] += tid + u * RT < nvs ? t : 0.0f;
          }
        });
        sum = rblock_sum2(sm, (sq[0] + sq[1]) + (sq[2] + sq[3]), rbuf);
        rbuf ^= 1;
      }
    }
    const bool nan = m != m || m == INFINITY;
    // pass B (truncated rows): exact counts of the wlim codes below the slice max; codes further down and
    // lanes past the slice's end go to the lane's spare entry.  Two count arrays, by row parity: each is
    // zeroed by its readers, and the barrier of the next row's use of the other one orders that before its
    // next use.
    if (hist) {
      uint32_t* const hc = sm.hist[r & 1];
      if (ok_u && uni(!nan && m > -INFINITY)) {
        const uint32_t keym = key16f(m);
        const uint32_t hbase = opaque_s(lds_addr(hc)), one = opaque_v(1u);
        // Slice max at least WTOP codes above +0 (the usual case): the window holds positive values only,
        // whose code distance to the max is the difference of their bf16 bits; a negative value's difference
        // (mod 2^16) exceeds the max's own bits, so it lands outside the window without its key.
        const bool posw = uni(__float_as_uint(m) >= ((uint32_t)WTOP << 16) && __float_as_uint(m) < 0x80000000u);
        const uint32_t mk2 = (posw ? (__float_as_uint(m) >> 16) : keym) * 0x10001u;
        static_for<0, NV>([&](auto UI) {
          constexpr int u = decltype(UI)::value;
          if (u < nvu) {
            const uint4 w = slot<r * NV + u, NREG, NLDS, false>(v, ldsv, tid);
            const bool valid = tid + u * RT < nvs;
            const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              uint32_t d2 = min16x2(sub16x2(mk2, posw ? wv[qd] : key16x2(wv[qd])), spare2);
              d2 = valid ? d2 : spare2;
              lds_inc(hbase + (d2 & 0xffffu) * 4u, one);
              lds_inc(hbase + (d2 >> 16) * 4u, one);
            }
          }
        });
      }
      lds_sync();
      if (tid < RWIN) {
        st32(&win[r * RWIN + tid], hc[2 * tid] | (hc[2 * tid + 1] << 16));
        hc[2 * tid] = 0u;
        hc[2 * tid + 1] = 0u;
      }
    }
    if (tid == 0) {
      stf(&prt[r].m, m);
      st32(&prt[r].arg, (uint32_t)a);
      stf(&prt[r].s, sum);
      st32(&prt[r].flags, nan ? 1u : 0u);
    }
    RTRACE(p, 13 + (r < 3 ? r : 2));
  });
  if (tid < 2 * KK) {
    vm_wait<0>();
    const uint32_t gw = gdma[tid];
    sm.gath[tid < KK ? tid : tid + 1] = gok ? __uint_as_float((gx & 1) ? (gw & 0xffff0000u) : (gw << 16)) : 0.0f;
  }

  // ---- exchange 1: partials out, flag, then every workgroup of the batch row merges them ----
  RTRACE(p, 1);
  drain();
  __syncthreads();
  if (tid == 0) st64(&p.flag1[(size_t)b * p.S + s], tag);
  const bool alive = wait_flags(p.flag1 + (size_t)b * p.S, p.S, tag, p.wait_limit);
  RTRACE(p, 2);
  if (alive) {
    for (int r = wave; r < ROWS; r += RWAVE) {
      // slice statistics, lane t reading slice t (64 slices per pass): the row max (NaN-propagating), its
      // lowest index on greedy rows, then the normaliser sum_t s_t exp2((m_t - max) c) (each slice's sum is
      // taken against its own max)
      float m = -INFINITY, sum = 0.0f;
      int a = INT_MAX;
      uint32_t fl = 0;
      for (int t0 = 0; t0 < p.S; t0 += 64) {
        const int t = t0 + lane;
        float mt = -INFINITY;
        uint32_t ft = 0;
        if (t < p.S) {
          const RPart* pp = p.part + ((size_t)b * p.S + t) * ROWS + r;
          mt = ldf(&pp->m);
          ft = ld32(&pp->flags);
        }
        m = nan_max(m, dpp_wave_max(mt));
        fl |= __ballot(ft != 0) != 0ull ? 1u : 0u;
      }
      if (m == m && m > -INFINITY) {
        for (int t0 = 0; t0 < p.S; t0 += 64) {
          const int t = t0 + lane;
          float term = 0.0f;
          int at = INT_MAX;
          if (t < p.S) {
            const RPart* pp = p.part + ((size_t)b * p.S + t) * ROWS + r;
            const float mt = ldf(&pp->m);
            if (q.greedy) {
              at = mt == m ? (int)ld32(&pp->arg) : INT_MAX;
            } else if (mt > -INFINITY) {
              term = ldf(&pp->s) * fexp2((mt - m) * q.c);
            }
          }
          if (q.greedy) a = min(a, dpp_wave_imin(at));
          else sum += dpp_wave_sum(term);
        }
      }
      const bool bad = !q.ok || fl != 0 || !(m > -INFINITY) || m == INFINITY;
      uint32_t thr = 0;
      float Z = sum;
      uint32_t fb = 0;
      if (!bad && q.trunc) {
        const uint32_t keym = key16f(m);
        uint32_t* c = cnt[r];
        for (int e = lane; e < WTOP; e += 64) c[e] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // every slice's window, CH slices at a time with all their loads in flight together
        constexpr int CH = 8;
        for (int t0 = 0; t0 < p.S; t0 += CH) {
          float mt[CH];
          uint32_t wv[CH][RWIN / 64];
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            const int t = min(t0 + h, p.S - 1);
            mt[h] = ldf(&p.part[((size_t)b * p.S + t) * ROWS + r].m);
            const uint32_t* wt = p.win + (((size_t)b * p.S + t) * ROWS + r) * RWIN;
#pragma unroll
            for (int i = 0; i < RWIN / 64; ++i) wv[h][i] = ld32(&wt[lane + 64 * i]);
          }
#pragma unroll
          for (int h = 0; h < CH; ++h) {
            if (t0 + h >= p.S || !(mt[h] > -INFINITY)) continue;  // an all -inf slice counted nothing
            const uint32_t off = keym - key16f(mt[h]);           // its window starts that many codes lower
            if (off >= (uint32_t)WTOP) continue;                 // entirely below the row's window
#pragma unroll
            for (int i = 0; i < RWIN / 64; ++i) {
              const uint32_t co = off + 2u * (uint32_t)(lane + 64 * i);
              if (co < (uint32_t)WTOP && (wv[h][i] & 0xffffu)) atomicAdd(&c[co], wv[h][i] & 0xffffu);
              if (co + 1u < (uint32_t)WTOP && (wv[h][i] >> 16)) atomicAdd(&c[co + 1u], wv[h][i] >> 16);
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        unsigned long long zsel = 0;
        if (wave_select(c, keym, m, q.c, q.useK, q.K, q.useP, q.P, (double)sum * 0x1p40, (int)wlim, thr, zsel))
          Z = (float)((double)zsel * 0x1p-40);
        else
          fb = 1;
      }
      if (lane == 0) {
        sm.m[r] = m;
        sm.arg[r] = a;
        sm.Z[r] = Z;
        sm.lz[r] = __builtin_amdgcn_logf(Z);
        sm.fthr[r] = thr == 0 ? -INFINITY : key16_value(thr);
        sm.bad[r] = bad ? 1u : 0u;
        sm.fb[r] = fb;
      }
    }
  }
  __syncthreads();
  RTRACE(p, 3);
  // thresholds the merged windows could not settle: an exact radix select over the row (rare: read again)
  if (alive) {
    for (int r = 0; r < ROWS; ++r) {
      if (!sm.fb[r]) continue;
      uint32_t thr = 0;
      float Z = 0.0f;
      r_cutoff(sm, &cnt[0][0], rows(r), p.V, sm.m[r], q.c, q.useK ? q.K : 0, q.useP ? q.P : 1.0f, thr, Z);
      if (tid == 0) {
        sm.Z[r] = Z;
        sm.lz[r] = __builtin_amdgcn_logf(Z);
        sm.fthr[r] = thr == 0 ? -INFINITY : key16_value(thr);
        sm.fb[r] = 0;
      }
      __syncthreads();
    }
  }
  bool ok = q.ok;
#pragma unroll
  for (int i = 0; i < KK; ++i) ok = ok && sm.tok[i] >= 0 && sm.tok[i] < p.V;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) ok = ok && sm.bad[r] == 0u;
  const size_t ob = (size_t)b * (KK + 1);
  if (!alive || !ok || q.greedy) {
    // sentinel, greedy or abandoned rows: workgroup 0 writes every output now; the others are done
    if (s != 0) return;
    if (!alive || !ok) return r_sentinel(p, b, KK);
    int n = KK;
#pragma unroll
    for (int i = KK - 1; i >= 0; --i)
      if (sm.tok[i] != sm.arg[i]) n = i;
    if (tid < KK) p.alpha[(size_t)b * KK + tid] = (sm.arg[tid] == sm.arg[KK + 1 + tid]) ? 1.0f : 0.0f;
    if (tid <= KK) {
      p.tokens[ob + tid] = tid < n ? sm.tok[tid] : (tid == n ? sm.arg[n] : -1);
      p.logprobs[ob + tid] = 0.0f;
    }
    if (tid == 0) p.accept_len[b] = n + 1;
    return;
  }

  // ---- accept chain (lane i of wave 0): n = the first rejection, else k ----
  if (tid < 64) {
    bool reject = false;
    if (tid < KK) {
      const float pt = kept_p(sm.gath[tid], sm.m[tid], q.c, sm.lz[tid], sm.fthr[tid]);
      const float qd =
          kept_p(sm.gath[KK + 1 + tid], sm.m[KK + 1 + tid], q.c, sm.lz[KK + 1 + tid], sm.fthr[KK + 1 + tid]);
      reject = !(pt > 0.0f && (qd == 0.0f || sm.u[tid] < pt / qd));
    }
    const int fr = first_lane(reject);
    if (tid == 0) sm.n = fr < KK ? fr : KK;
  }
  __syncthreads();
  const int n = sm.n;

  // ---- phase 2: alpha for every position, the race at position n, on the resident columns ----
  float best = 0.0f, bval = 0.0f;
  int bidx = INT_MAX;
  static_for<0, KK>([&](auto II) {
    constexpr int i = decltype(II)::value;
    constexpr int rt = i, rd = KK + 1 + i;
    const float mt = sm.m[rt], md = sm.m[rd], lt = sm.lz[rt], ld = sm.lz[rd], tt = sm.fthr[rt], td = sm.fthr[rd];
    const bool draw = i == n;
    float acc = 0.0f;
    static_for<0, NV>([&](auto UI) {
      constexpr int u = decltype(UI)::value;
      const uint4 wa = slot<rt * NV + u, NREG, NLDS, false>(v, ldsv, tid);
      const uint4 wb = slot<rd * NV + u, NREG, NLDS, false>(v, ldsv, tid);
      const int j = tid + u * RT;
      bool live = j < nvs;
      if (q.trunc) {
        bool any = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) any = any || BF16::get(wa, e) >= tt;
        live = live && any;
      }
      if (live) {
        float wr[8];
        bool anyw = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ft = BF16::get(wa, e), fd = BF16::get(wb, e);
          float lp = fmaf(ft - mt, q.c, -lt), lq = fmaf(fd - md, q.c, -ld);  // log2 p, log2 q
          if (q.trunc) {
            lp = ft >= tt ? lp : -INFINITY;
            lq = fd >= td ? lq : -INFINITY;
          }
          if (draw) {
            const float pe = fexp2(lp), qe = fexp2(lq);
            acc += fminf(pe, qe);
            wr[e] = pe - qe;
            anyw = anyw || wr[e] > 0.0f;
          } else {
            acc += fexp2(fminf(lp, lq));
            wr[e] = 0.0f;
          }
        }
        if (anyw) r_race8(p, b, n, x0 + 8 * j, wr, wa, best, bidx, bval);
      }
    });
    acc = wave_sum(acc);
    if (lane == 0) sm.wacc[i][wave] = acc;
  });
  if (n == KK) {  // every draft accepted: the bonus race on row k
    const float mt = sm.m[KK], tt = sm.fthr[KK];
    static_for<0, NV>([&](auto UI) {
      constexpr int u = decltype(UI)::value;
      const uint4 wa = slot<KK * NV + u, NREG, NLDS, false>(v, ldsv, tid);
      const int j = tid + u * RT;
      if (j < nvs) {
        float wr[8];
        bool anyw = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ft = BF16::get(wa, e);
          wr[e] = ft >= tt ? fexp2((ft - mt) * q.c) : 0.0f;
          anyw = anyw || wr[e] > 0.0f;
        }
        if (anyw) r_race8(p, b, KK, x0 + 8 * j, wr, wa, best, bidx, bval);
      }
    });
  }
  rblock_race(sm, best, bidx, bval);  // its barriers also publish the wacc entries
  RTRACE(p, 4);

  // ---- exchange 2: alpha partials and the race winner to workgroup 0 of the batch row ----
  if (s != 0) {
    RFin* fp = p.fin + (size_t)b * p.S + s;
    if (tid < KK) {
      float a = 0.0f;
#pragma unroll
      for (int w = 0; w < RWAVE; ++w) a += sm.wacc[tid][w];
      stf(&fp->alpha[tid], a);
    }
    if (tid == 0) {
      stf(&fp->key, best);
      st32(&fp->idx, (uint32_t)bidx);
      stf(&fp->val, bval);
    }
    drain();
    __syncthreads();
    if (tid == 0) st64(&p.flag2[(size_t)b * p.S + s], tag);
    RTRACE(p, 7);
    return;
  }
  // workgroup 0: its own partials stay local; the others' arrive behind flags 1..S-1
  if (!wait_flags(p.flag2 + (size_t)b * p.S + 1, p.S - 1, tag, p.wait_limit)) return r_sentinel(p, b, KK);
  RTRACE(p, 5);
  if (tid < 64) {
    // lane t < S holds slice t's partials (slice 0: this workgroup's); fixed-order sums over the slices
    float al[KK];
    float k2 = 0.0f, v2 = 0.0f;
    int i2 = INT_MAX;
#pragma unroll
    for (int i = 0; i < KK; ++i) al[i] = 0.0f;
    for (int t0 = 0; t0 < p.S; t0 += 64) {
      const int t = t0 + tid;
      if (t == 0) {
#pragma unroll
        for (int i = 0; i < KK; ++i) {
          float a = 0.0f;
#pragma unroll
          for (int w = 0; w < RWAVE; ++w) a += sm.wacc[i][w];
          al[i] += a;
        }
        race_take(k2, i2, v2, best, bidx, bval);
      } else if (t < p.S) {
        const RFin* fp = p.fin + (size_t)b * p.S + t;
#pragma unroll
        for (int i = 0; i < KK; ++i) al[i] += ldf(&fp->alpha[i]);
        race_take(k2, i2, v2, ldf(&fp->key), (int)ld32(&fp->idx), ldf(&fp->val));
      }
    }
#pragma unroll
    for (int i = 0; i < KK; ++i) al[i] = wave_sum(al[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float kk = __shfl_xor(k2, o, 64);
      const int ii = __shfl_xor(i2, o, 64);
      const float vv = __shfl_xor(v2, o, 64);
      race_take(k2, i2, v2, kk, ii, vv);
    }
    if (tid < KK) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < KK; ++i) a = tid == i ? al[i] : a;
      p.alpha[(size_t)b * KK + tid] = a;
    }
    if (tid == 0) {
      sm.wi[0] = i2;
      sm.wf[0] = v2;
    }
  }
  __syncthreads();
  int y = sm.wi[0];
  float yv = sm.wf[0];
  __syncthreads();
  if (y == INT_MAX && n < KK) {
    // The residual mass vanished in fp32 (rounding only): draw from p_n over the whole row (read again).
    const uint4* row = (const uint4*)rows(n);
    const float mn = sm.m[n], tn = sm.fthr[n];
    float bb = 0.0f, bv = 0.0f;
    int bi = INT_MAX;
    for (int j = tid; j < p.V / 8; j += RT) {
      const uint4 w = row[j];
#pragma unroll
      for (int g = 0; g < 8; g += 4) {
        float wr[4];
        bool anyw = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = BF16::get(w, g + e);
          wr[e] = f >= tn ? fexp2((f - mn) * q.c) : 0.0f;
          anyw = anyw || wr[e] > 0.0f;
        }
        if (anyw) r_race4(p, b, n, 8 * j + g, wr, w, g, bb, bi, bv);
      }
    }
    rblock_race(sm, bb, bi, bv);
    y = bi;
    yv = bv;
  }
  if (y < 0 || y >= p.V) return r_sentinel(p, b, KK);  // no candidate: not reachable for a valid row
  if (tid <= KK) {
    int t = -1;
    float lp = 0.0f;
    if (tid <= n) {
      t = tid < n ? sm.tok[tid] : y;
      const float l = tid < n ? sm.gath[tid] : yv;
      lp = (l - sm.m[tid]) / q.T - logf(sm.Z[tid]);
    }
    p.tokens[ob + tid] = t;
    p.logprobs[ob + tid] = lp;
  }
  if (tid == 0) p.accept_len[b] = n + 1;
  RTRACE(p, 7);
}
