// specverify_oracle.cpp -- plain CPU oracle of the speculative-decoding verify sampler.
//
// TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the benchmark's
// CPU-baseline leg, never by the product path.  Shares no code with the GPU library.
//
// Plain double-precision loops, std::sort as the only library primitive.  No blocking,
// fusion or reordering beyond what the definitions below state, so every step can be
// checked by eye against its source:
//   * AReno PR "feat(engine): MTP training loss and speculative decoding for bailing_v3",
//     section "What does this PR do?", Phase 2 paragraph: the verify step builds the
//     sampler-equivalent target distribution and runs exact chain rejection sampling so
//     that both the sampled distribution and the reported logprobs are those of plain
//     sampling.
//   * same page, accept-probability table: alpha = sum_x min(p, q); expected accept length.
//   * same page, per-step optimisation table: draws are Gumbel-max, without host syncs.
//   * same page, section "How was it tested?": sampler equivalence with and without
//     top-k/top-p; distribution preservation; exact under greedy.
// Where the page is silent, the reading taken is named in the comment (R-numbers refer to
// the list of readings in the design notes).
//
// Negative controls: building with -DORACLE_MUTANT=<n> plants one deliberate mistake
// (see the MUTANT switch comments); the test suite checks that its pins catch each one.

#include "specverify_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <utility>
#include <vector>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

namespace {

const double kInf = std::numeric_limits<double>::infinity();
const double kNaN = std::numeric_limits<double>::quiet_NaN();

// ---------------------------------------------------------------------------------------
// Philox-4x32-10 (Salmon et al., SC'11, section 5): two 32x32->64 multiplies per round,
// the high halves xored with the other counter words and the round key, the key bumped
// by the Weyl constants between rounds.
// ---------------------------------------------------------------------------------------
void philox_round(uint32_t c[4], const uint32_t key[2]) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
  const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  const uint32_t n0 = hi1 ^ c[1] ^ key[0];
  const uint32_t n1 = lo1;
  const uint32_t n2 = hi0 ^ c[3] ^ key[1];
  const uint32_t n3 = lo0;
  c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

void philox10(const uint32_t ctr[4], const uint32_t key_in[2], uint32_t out[4]) {
#if ORACLE_MUTANT == 11
  const int rounds = 9;  // MUTANT 11: one round short
#else
  const int rounds = 10;
#endif
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t key[2] = {key_in[0], key_in[1]};
  for (int r = 0; r < rounds; ++r) {
    if (r > 0) {
      key[0] += 0x9E3779B9u;
      key[1] += 0xBB67AE85u;
    }
    philox_round(c, key);
  }
  for (int j = 0; j < 4; ++j) out[j] = c[j];
}

uint32_t philox_word(uint64_t seed, uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t word) {
  const uint32_t ctr[4] = {c0, c1, c2, c3};
  const uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  philox10(ctr, key, out);
  return out[word & 3u];
}

// Accept uniform u(b, i) in [0, 1): the top 24 bits of the word, exact in float and double (R6).
double accept_uniform(uint64_t seed, uint32_t b, uint32_t i, uint32_t offset) {
  const uint32_t w = philox_word(seed, i >> 2, b, 0u, offset, i & 3u);
  return (double)(w >> 8) * 0x1p-24;
}

// Gumbel uniform U in (0, 1): the top 23 bits plus one half, exact in float and double (R13).
double gumbel_uniform(uint64_t seed, uint32_t tag, uint32_t b, uint32_t j, uint32_t x, uint32_t offset) {
  const uint32_t w = philox_word(seed, x >> 2, b, (tag << 24) | j, offset, x & 3u);
  return ((double)(w >> 9) + 0.5) * 0x1p-23;
}

double gumbel(uint64_t seed, uint32_t tag, uint32_t b, uint32_t j, uint32_t x, uint32_t offset) {
  const double U = gumbel_uniform(seed, tag, b, j, x, offset);
  return -std::log(-std::log(U));
}

// ---------------------------------------------------------------------------------------
// Input conversion: both maps are exact.
// ---------------------------------------------------------------------------------------
double bf16_to_double(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return (double)f;
}

void load_row(const void* base, int32_t dtype, size_t row, int32_t V, std::vector<double>& out) {
  out.resize((size_t)V);
  if (dtype == ORACLE_DTYPE_BF16) {
    const uint16_t* p = (const uint16_t*)base + row * (size_t)V;
    for (int32_t x = 0; x < V; ++x) out[(size_t)x] = bf16_to_double(p[x]);
  } else {
    const float* p = (const float*)base + row * (size_t)V;
    for (int32_t x = 0; x < V; ++x) out[(size_t)x] = (double)p[x];
  }
}

// A row is unusable if it holds NaN or +inf (R15).  -inf is a legal logit (probability 0).
bool row_has_nan_or_posinf(const std::vector<double>& l) {
  for (double v : l)
    if (std::isnan(v) || v == kInf) return true;
  return false;
}

// Sampling parameters are valid when T is finite and >= 0, top_k >= 0, and top_p > 0
// (top_p >= 1, including +inf, switches top-p off) (R3, R4).
bool params_valid(float T, int32_t K, float P) {
  if (std::isnan(T) || std::isinf(T) || T < 0.0f) return false;
  if (K < 0) return false;
  if (std::isnan(P) || P <= 0.0f) return false;
  return true;
}

// ---------------------------------------------------------------------------------------
// The sampler distribution of one row: temperature, then top-k, then top-p on the top-k
// renormalised mass, then renormalise (R1).  Ties at either threshold are kept whole (R2,
// R3).  T == 0 is greedy: a one-hot at the lowest-index maximum (R4).
// ---------------------------------------------------------------------------------------
struct RowDist {
  std::vector<double> p;  // the distribution
  double m = -kInf;       // row max
  int32_t argmax = -1;    // lowest-index maximum
  double Z = 0.0;         // kept-set normaliser of exp((l - m) / T)
  int32_t kept = 0;       // number of kept entries
  double thr = -kInf;     // smallest kept logit
  double topp_margin = kInf;
  double topp_at = kInf;    // |M(v)/Z_K - P| at the chosen value v
  double topp_prev = kInf;  // |M(v')/Z_K - P| at the next larger distinct value v' (+inf if none)
};

// topp_shift selects an alternative resolution of the top-p decision, for rows whose decision lies
// within rounding of the boundary: 0 = the definition; -1 = one distinct value lower than the chosen
// one (as if M(v) had fallen just short of P Z_K: one more value kept); +1 = the next larger distinct
// value (as if M(v') had reached P Z_K: one value fewer kept).  Either is a no-op where no such value
// exists.
bool row_dist(const std::vector<double>& l, double T, int32_t K, double P, RowDist& d, int topp_shift = 0) {
  const int32_t V = (int32_t)l.size();
  d.p.assign((size_t)V, 0.0);
  d.m = -kInf;
  d.argmax = -1;
  for (int32_t x = 0; x < V; ++x) {
#if ORACLE_MUTANT == 4
    if (l[(size_t)x] >= d.m && l[(size_t)x] > -kInf) {  // MUTANT 4: highest index wins ties
#else
    if (l[(size_t)x] > d.m) {  // strict: the first (lowest-index) maximum is kept
#endif
      d.m = l[(size_t)x];
      d.argmax = x;
    }
  }
  if (d.argmax < 0) return false;  // every entry is -inf: no distribution

  if (T == 0.0) {  // greedy
    d.p[(size_t)d.argmax] = 1.0;
    d.Z = 1.0;
    d.kept = 1;
    d.thr = d.m;
    return true;
  }

  std::vector<double> e((size_t)V);
  for (int32_t x = 0; x < V; ++x) {
#if ORACLE_MUTANT == 9
    e[(size_t)x] = std::exp((l[(size_t)x] - d.m) * T);  // MUTANT 9: temperature multiplies
#else
    e[(size_t)x] = std::exp((l[(size_t)x] - d.m) / T);
#endif
  }

  double thr = -kInf;
  if (K > 0 && K < V) {
    // K-th largest value, counting multiplicity.
    std::vector<double> s(l);
    std::sort(s.begin(), s.end(), [](double a, double b) { return a > b; });
#if ORACLE_MUTANT == 10
    thr = s[(size_t)K];  // MUTANT 10: keeps one more than K
#else
    thr = s[(size_t)K - 1];
#endif
  }

  if (P < 1.0) {
    // Kept set so far, sorted by value (descending); M(v) = mass of kept entries >= v.
    std::vector<std::pair<double, double>> kv;  // (logit, e)
    double ZK = 0.0;
    for (int32_t x = 0; x < V; ++x) {
      if (l[(size_t)x] >= thr) {
        kv.emplace_back(l[(size_t)x], e[(size_t)x]);
        ZK += e[(size_t)x];
      }
    }
    std::sort(kv.begin(), kv.end(), [](const std::pair<double, double>& a, const std::pair<double, double>& b) {
      return a.first > b.first;
    });
    const double target = P * ZK;
    double M = 0.0, prevM = -1.0;
    double chosen = -kInf, prevv = -kInf;
    size_t i = 0;
    while (i < kv.size()) {
      const double v = kv[i].first;
      while (i < kv.size() && kv[i].first == v) {
        M += kv[i].second;
        ++i;
      }
#if ORACLE_MUTANT == 3
      if (M > target) {  // MUTANT 3: strict inequality
#else
      if (M >= target) {  // smallest upper set holding at least P of the mass (R3)
#endif
        chosen = v;
        break;
      }
      prevM = M;
      prevv = v;
    }
    if (chosen == -kInf && !kv.empty()) chosen = kv.back().first;  // unreachable for P < 1
    d.topp_at = std::fabs(M / ZK - P);
    d.topp_prev = prevM >= 0.0 ? std::fabs(prevM / ZK - P) : kInf;
#if ORACLE_MUTANT == 28
    d.topp_margin = d.topp_at;  // MUTANT 28: the next larger value's distance is left out
#else
    d.topp_margin = std::min(d.topp_at, d.topp_prev);
#endif
    if (topp_shift < 0 && i < kv.size()) chosen = kv[i].first;  // the next lower distinct value
    if (topp_shift > 0 && prevv > -kInf) chosen = prevv;        // the next larger distinct value
    thr = std::max(thr, chosen);
  }

  double Z = 0.0;
  int32_t kept = 0;
  for (int32_t x = 0; x < V; ++x) {
#if ORACLE_MUTANT == 5
    Z += e[(size_t)x];  // MUTANT 5: no renormalisation after truncation
    if (l[(size_t)x] >= thr) ++kept;
#else
    if (l[(size_t)x] >= thr) {
      Z += e[(size_t)x];
      ++kept;
    }
#endif
  }
  for (int32_t x = 0; x < V; ++x)
    if (l[(size_t)x] >= thr) d.p[(size_t)x] = e[(size_t)x] / Z;
  d.Z = Z;
  d.kept = kept;
  d.thr = thr;
  return true;
}

// Gumbel-max over a weight vector w (entries <= 0 are excluded): argmax of ln w(x) + G(x),
// lowest index on exact key ties (R13).  Returns the index and the top-2 key gap (natural-log key
// units).  runner_up = true returns the index of the second-largest key instead (an alternative
// resolution of a draw whose gap lies within rounding); the winner if there is no second candidate.
int32_t gumbel_argmax(const std::vector<double>& w, uint64_t seed, uint32_t tag, uint32_t b, uint32_t j,
                      uint32_t offset, double* gap, bool runner_up = false) {
  double best = -kInf, second = -kInf;
  int32_t y = -1, y2 = -1;
  for (size_t x = 0; x < w.size(); ++x) {
    if (!(w[x] > 0.0)) continue;
#if ORACLE_MUTANT == 8
    const double key = std::log(w[x]) - gumbel(seed, tag, b, j, (uint32_t)x, offset);  // MUTANT 8
#else
    const double key = std::log(w[x]) + gumbel(seed, tag, b, j, (uint32_t)x, offset);
#endif
    if (key > best) {
      second = best;
      y2 = y;
      best = key;
      y = (int32_t)x;
    } else if (key > second) {
      second = key;
      y2 = (int32_t)x;
    }
  }
#if ORACLE_MUTANT == 27
  *gap = (second == -kInf) ? kInf : std::exp(best) - std::exp(second);  // MUTANT 27: gap of the exp'd keys
#else
  *gap = (second == -kInf) ? kInf : best - second;
#endif
#if ORACLE_MUTANT != 29
  if (runner_up && y2 >= 0) return y2;  // MUTANT 29 ignores the runner-up request
#endif
  return y;
}

// ---------------------------------------------------------------------------------------
// One batch row of the verify step.
// ---------------------------------------------------------------------------------------
struct VerifyArgs {
  const void* target;
  const void* draft;
  int32_t dtype;
  const int32_t* draft_tokens;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t B, k, V;
  uint64_t seed;
  uint32_t offset;
  int32_t* tokens;
  int32_t* accept_len;
  double* logprobs;
  double* alpha;
  double* diag;
  int32_t* dflags;
  const int32_t* alt;   // [B][4] alternative resolutions, or NULL (see oracle_spec_verify_ex)
  double* topp_rows;    // [B][2k+1][2] per-row top-p distances, or NULL
  double* accept_pos;   // [B][k] per-position accept distances, or NULL
};

void write_sentinel(const VerifyArgs& a, int32_t b) {
  const int32_t k = a.k;
  for (int32_t i = 0; i <= k; ++i) {
    a.tokens[(size_t)b * (k + 1) + i] = -1;
    a.logprobs[(size_t)b * (k + 1) + i] = kNaN;
  }
  for (int32_t i = 0; i < k; ++i) a.alpha[(size_t)b * k + i] = kNaN;
  a.accept_len[b] = 0;
  if (a.diag)
    for (int j = 0; j < 4; ++j) a.diag[(size_t)b * 4 + j] = kInf;
  if (a.dflags) a.dflags[b] = 2;
  if (a.topp_rows)
    for (int32_t j = 0; j < 2 * (2 * k + 1); ++j) a.topp_rows[(size_t)b * 2 * (2 * k + 1) + j] = kInf;
  if (a.accept_pos)
    for (int32_t i = 0; i < k; ++i) a.accept_pos[(size_t)b * k + i] = kInf;
}

void verify_row(const VerifyArgs& a, int32_t b) {
  const int32_t k = a.k, V = a.V;
  // alternative resolutions of this row's near-boundary decisions (all zero: the definition)
  const int32_t* alt = a.alt ? a.alt + (size_t)b * 4 : nullptr;
  const uint32_t topp_down = alt ? (uint32_t)alt[0] : 0u, topp_up = alt ? (uint32_t)alt[1] : 0u;
  const uint32_t flips = alt ? ((uint32_t)alt[2] & 0xffffu) : 0u;
  const bool runner_up = alt ? (((uint32_t)alt[2] >> 16) & 1u) != 0 : false;
  auto shift_of = [&](int32_t r) { return ((topp_down >> r) & 1u) ? -1 : (((topp_up >> r) & 1u) ? 1 : 0); };
  const float Tf = a.temperature[b];
  const int32_t K = a.top_k[b];
  const float Pf = a.top_p[b];
  if (!params_valid(Tf, K, Pf)) return write_sentinel(a, b);
  for (int32_t i = 0; i < k; ++i) {
    const int32_t x = a.draft_tokens[(size_t)b * k + i];
    if (x < 0 || x >= V) return write_sentinel(a, b);
  }
  const double T = (double)Tf, P = (double)Pf;

  // p_i for target positions i = 0..k, q_i for draft positions i = 0..k-1, each with the
  // batch row's own (T, top-k, top-p): the draft side is processed exactly like the target.
  std::vector<RowDist> p((size_t)k + 1), q((size_t)k);
  std::vector<double> l;
  double topp_margin = kInf;
  for (int32_t i = 0; i <= k; ++i) {
    load_row(a.target, a.dtype, (size_t)b * (k + 1) + i, V, l);
    if (row_has_nan_or_posinf(l) || !row_dist(l, T, K, P, p[(size_t)i], shift_of(i))) return write_sentinel(a, b);
    topp_margin = std::min(topp_margin, p[(size_t)i].topp_margin);
  }
  for (int32_t i = 0; i < k; ++i) {
    load_row(a.draft, a.dtype, (size_t)b * k + i, V, l);
    if (row_has_nan_or_posinf(l) || !row_dist(l, T, K, P, q[(size_t)i], shift_of(k + 1 + i)))
      return write_sentinel(a, b);
    topp_margin = std::min(topp_margin, q[(size_t)i].topp_margin);
  }
  if (a.topp_rows) {  // logit row r: targets 0..k, then drafts
    double* tr = a.topp_rows + (size_t)b * 2 * (2 * k + 1);
    for (int32_t r = 0; r <= 2 * k; ++r) {
      const RowDist& d = r <= k ? p[(size_t)r] : q[(size_t)(r - k - 1)];
      tr[2 * r] = d.topp_at;
      tr[2 * r + 1] = d.topp_prev;
    }
  }
  if (a.accept_pos)
    for (int32_t i = 0; i < k; ++i) a.accept_pos[(size_t)b * k + i] = kInf;

  // Chain rejection: accept draft x_i while the target allows it and u_i < p_i(x_i) / q_i(x_i);
  // a draft outside q's support is accepted whenever p_i(x_i) > 0 (R5).  Greedy rows reduce to
  // "accept iff x_i is the target argmax" because p and q are one-hot.
  int32_t n = k;
  double accept_margin = kInf;
  for (int32_t i = 0; i < k; ++i) {
    const int32_t x = a.draft_tokens[(size_t)b * k + i];
    const double pt = p[(size_t)i].p[(size_t)x];
    const double qd = q[(size_t)i].p[(size_t)x];
    const double u = accept_uniform(a.seed, (uint32_t)b, (uint32_t)i, a.offset);
#if ORACLE_MUTANT == 1
    bool accept = qd > 0.0 && (pt == 0.0 || u < qd / pt);  // MUTANT 1: p and q swapped
#else
    bool accept = pt > 0.0 && (qd == 0.0 || u < pt / qd);
#endif
    if ((flips >> i) & 1u) accept = !accept;  // alternative resolution of a near-boundary test
    if (T != 0.0 && pt > 0.0 && qd > 0.0) {
      const double dist = std::fabs(u - pt / qd);
      accept_margin = std::min(accept_margin, dist);
      if (a.accept_pos) a.accept_pos[(size_t)b * k + i] = dist;
    }
    if (!accept) {
      n = i;
      break;
    }
  }
#if ORACLE_MUTANT == 26
  for (int32_t i = n + 1; i < k; ++i) {  // MUTANT 26: tests past the first rejection count as well
    const int32_t x = a.draft_tokens[(size_t)b * k + i];
    const double pt = p[(size_t)i].p[(size_t)x], qd = q[(size_t)i].p[(size_t)x];
    const double u = accept_uniform(a.seed, (uint32_t)b, (uint32_t)i, a.offset);
    if (T != 0.0 && pt > 0.0 && qd > 0.0) accept_margin = std::min(accept_margin, std::fabs(u - pt / qd));
  }
#endif

  // The committed extra token: residual normalize(max(p_n - q_n, 0)) after a rejection,
  // the bonus from p_k when every draft is accepted.  Drawn by Gumbel-max (verify stream).
  int32_t y;
  double gap = kInf;
  double resid_mass = -1.0;
  int32_t flags = 0;
  if (T == 0.0) {
    y = p[(size_t)n].argmax;  // greedy: the residual of two one-hots is the target one-hot
  } else {
    std::vector<double> w((size_t)V);
    if (n < k) {
      resid_mass = 0.0;
      for (int32_t x = 0; x < V; ++x) {
#if ORACLE_MUTANT == 13
        w[(size_t)x] = std::fabs(p[(size_t)n].p[(size_t)x] - q[(size_t)n].p[(size_t)x]);  // MUTANT 13
#elif ORACLE_MUTANT == 2
        w[(size_t)x] = p[(size_t)n].p[(size_t)x];  // MUTANT 2: resample from the target
#else
        w[(size_t)x] = std::max(p[(size_t)n].p[(size_t)x] - q[(size_t)n].p[(size_t)x], 0.0);
#endif
        resid_mass += w[(size_t)x];
      }
      if (!(resid_mass > 0.0)) {  // reachable only through rounding: fall back to p_n (R7)
        w = p[(size_t)n].p;
        flags |= 1;
      }
    } else {
#if ORACLE_MUTANT == 12
      w = p[(size_t)k - 1].p;  // MUTANT 12: bonus drawn at the wrong position
#else
      w = p[(size_t)k].p;
#endif
    }
    y = gumbel_argmax(w, a.seed, 1u, (uint32_t)b, (uint32_t)n, a.offset, &gap, runner_up);
  }

  // Outputs (R8, R9, R10, R11).
  for (int32_t i = 0; i <= k; ++i) {
    const size_t o = (size_t)b * (k + 1) + i;
    if (i < n) {
      const int32_t x = a.draft_tokens[(size_t)b * k + i];
      a.tokens[o] = x;
      a.logprobs[o] = std::log(p[(size_t)i].p[(size_t)x]);
    } else if (i == n) {
      a.tokens[o] = y;
      a.logprobs[o] = std::log(p[(size_t)n].p[(size_t)y]);
    } else {
      a.tokens[o] = -1;
      a.logprobs[o] = 0.0;
    }
  }
#if ORACLE_MUTANT == 6
  a.accept_len[b] = n;  // MUTANT 6: the extra token is not counted
#else
  a.accept_len[b] = n + 1;
#endif
  for (int32_t i = 0; i < k; ++i) {
    double s = 0.0;
    for (int32_t x = 0; x < V; ++x) {
#if ORACLE_MUTANT == 7
      s += std::fabs(p[(size_t)i].p[(size_t)x] - q[(size_t)i].p[(size_t)x]);  // MUTANT 7
#else
      s += std::min(p[(size_t)i].p[(size_t)x], q[(size_t)i].p[(size_t)x]);
#endif
    }
#if ORACLE_MUTANT == 7
    s = 1.0 - s;
#endif
    a.alpha[(size_t)b * k + i] = s;
  }
  if (a.diag) {
    a.diag[(size_t)b * 4 + 0] = accept_margin;
    a.diag[(size_t)b * 4 + 1] = gap;
    a.diag[(size_t)b * 4 + 2] = topp_margin;
    a.diag[(size_t)b * 4 + 3] = resid_mass;
  }
  if (a.dflags) a.dflags[b] = flags | (n << 8);
}

// ---------------------------------------------------------------------------------------
// One batch row of tree verification.  The pages name only the draft-tree parameters (EAGLE top-k
// through SGLang's NEXTN passthrough, AReaL pull request "MTP training with speculative decoding
// rollout", its key-changes list); the rule below is the published recursive rejection for drafts
// that are distinct tokens chosen deterministically (top-k children), taken from outside the pages:
// at a node u with target distribution p_u and children c_1..c_m (node-index order), one uniform U
// (the accept stream at position = depth) accepts the first child j with U < p_u(t_1) + ... +
// p_u(t_j); if none is accepted the token is drawn from p_u with the children's tokens removed
// (renormalised), and at a leaf from p_u itself.  Every emitted token is then distributed exactly as
// p_u, so the committed sequence follows the target sampler.  A tree whose nodes each have one child
// is chain verification with one-hot draft distributions.
// ---------------------------------------------------------------------------------------
struct TreeArgs {
  const void* target;
  int32_t dtype;
  const int32_t* parent;
  const int32_t* node_tokens;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  int32_t B, N, V;
  uint64_t seed;
  uint32_t offset;
  int32_t* tokens;
  int32_t* path;
  int32_t* accept_len;
  double* logprobs;
  double* diag;
};

void tree_sentinel(const TreeArgs& a, int32_t b) {
  for (int32_t i = 0; i < a.N; ++i) {
    a.tokens[(size_t)b * a.N + i] = -1;
    a.path[(size_t)b * a.N + i] = -1;
    a.logprobs[(size_t)b * a.N + i] = kNaN;
  }
  a.accept_len[b] = 0;
  if (a.diag)
    for (int j = 0; j < 4; ++j) a.diag[(size_t)b * 4 + j] = kInf;
}

void tree_row(const TreeArgs& a, int32_t b) {
  const int32_t N = a.N, V = a.V;
  const int32_t* par = a.parent + (size_t)b * N;
  const int32_t* tok = a.node_tokens + (size_t)b * N;
  const float Tf = a.temperature[b];
  const int32_t K = a.top_k[b];
  const float Pf = a.top_p[b];
  if (!params_valid(Tf, K, Pf)) return tree_sentinel(a, b);
  // the tree: every node but the root has an earlier parent and a token in range; siblings differ
  std::vector<std::vector<int32_t>> children((size_t)N);
  for (int32_t i = 1; i < N; ++i) {
    if (par[i] < 0 || par[i] >= i || tok[i] < 0 || tok[i] >= V) return tree_sentinel(a, b);
    for (int32_t c : children[(size_t)par[i]])
      if (tok[c] == tok[i]) return tree_sentinel(a, b);
    children[(size_t)par[i]].push_back(i);
  }
  const double T = (double)Tf, P = (double)Pf;
  std::vector<RowDist> p((size_t)N);
  std::vector<double> l;
  double topp_margin = kInf;
  for (int32_t i = 0; i < N; ++i) {
    load_row(a.target, a.dtype, (size_t)b * N + i, V, l);
    if (row_has_nan_or_posinf(l) || !row_dist(l, T, K, P, p[(size_t)i])) return tree_sentinel(a, b);
    topp_margin = std::min(topp_margin, p[(size_t)i].topp_margin);
  }

  // walk from the root
  std::vector<int32_t> path;
  int32_t u = 0;
  bool leaf = false;
  double accept_margin = kInf;
  for (;;) {
    const std::vector<int32_t>& ch = children[(size_t)u];
    if (ch.empty()) {
      leaf = true;
      break;
    }
    const int32_t d = (int32_t)path.size();
#if ORACLE_MUTANT == 24
    const RowDist& pu = p[(size_t)(d == 0 ? 0 : par[u])];  // MUTANT 24: the parent's distribution
#else
    const RowDist& pu = p[(size_t)u];
#endif
    int32_t acc = -1;
    if (T == 0.0) {
      for (int32_t c : ch)
        if (tok[c] == pu.argmax) acc = c;
    } else {
      const double U = accept_uniform(a.seed, (uint32_t)b, (uint32_t)d, a.offset);
      double S = 0.0;
      for (int32_t c : ch) {
#if ORACLE_MUTANT == 23
        S = pu.p[(size_t)tok[c]];  // MUTANT 23: each child tested against its own mass alone
#else
        S += pu.p[(size_t)tok[c]];
#endif
        if (S > 0.0) accept_margin = std::min(accept_margin, std::fabs(U - S));
        if (U < S) {
          acc = c;
          break;
        }
      }
    }
    if (acc < 0) break;
    path.push_back(acc);
    u = acc;
  }
  const int32_t d = (int32_t)path.size();

  // the committed extra token at the stopping node u
  int32_t y;
  double gap = kInf;
  if (T == 0.0) {
    y = p[(size_t)u].argmax;
  } else {
    std::vector<double> w = p[(size_t)u].p;
    if (!leaf) {
      double mass = 0.0;
#if ORACLE_MUTANT != 22
      for (int32_t c : children[(size_t)u]) w[(size_t)tok[c]] = 0.0;  // MUTANT 22 keeps the rejected children
#endif
      for (double v : w) mass += v;
      if (!(mass > 0.0)) w = p[(size_t)u].p;  // reachable only through rounding (as R7)
    }
#if ORACLE_MUTANT == 25
    y = gumbel_argmax(w, a.seed, 1u, (uint32_t)b, (uint32_t)d + 1u, a.offset, &gap);  // MUTANT 25: one depth late
#else
    y = gumbel_argmax(w, a.seed, 1u, (uint32_t)b, (uint32_t)d, a.offset, &gap);
#endif
  }

  for (int32_t i = 0; i < N; ++i) {
    const size_t o = (size_t)b * N + i;
    if (i < d) {
      const int32_t row = i == 0 ? 0 : path[(size_t)i - 1];
      a.tokens[o] = tok[path[(size_t)i]];
      a.path[o] = path[(size_t)i];
      a.logprobs[o] = std::log(p[(size_t)row].p[(size_t)tok[path[(size_t)i]]]);
    } else if (i == d) {
      a.tokens[o] = y;
      a.path[o] = -1;
      a.logprobs[o] = std::log(p[(size_t)u].p[(size_t)y]);
    } else {
      a.tokens[o] = -1;
      a.path[o] = -1;
      a.logprobs[o] = 0.0;
    }
  }
  a.accept_len[b] = d + 1;
  if (a.diag) {
    a.diag[(size_t)b * 4 + 0] = accept_margin;
    a.diag[(size_t)b * 4 + 1] = gap;
    a.diag[(size_t)b * 4 + 2] = topp_margin;
    a.diag[(size_t)b * 4 + 3] = (double)u;
  }
}

template <class F>
void parallel_rows(int32_t n_rows, int32_t num_threads, F f) {
  int32_t nt = num_threads > 0 ? num_threads : (int32_t)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > n_rows) nt = n_rows;
  if (nt <= 1) {
    for (int32_t r = 0; r < n_rows; ++r) f(r);
    return;
  }
  std::vector<std::thread> pool;
  for (int32_t t = 0; t < nt; ++t)
    pool.emplace_back([=]() {
      for (int32_t r = t; r < n_rows; r += nt) f(r);
    });
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) { philox10(ctr, key, out); }

double oracle_accept_uniform(uint64_t seed, uint32_t b, uint32_t i, uint32_t offset) {
  return accept_uniform(seed, b, i, offset);
}

double oracle_gumbel_uniform(uint64_t seed, uint32_t tag, uint32_t b, uint32_t j, uint32_t x, uint32_t offset) {
  return gumbel_uniform(seed, tag, b, j, x, offset);
}

int oracle_row_probs(const double* logits, int32_t V, double T, int32_t K, double P, double* probs, double* info) {
  std::vector<double> l(logits, logits + V);
  RowDist d;
  if (!row_dist(l, T, K, P, d)) return 1;
  std::copy(d.p.begin(), d.p.end(), probs);
  if (info) {
    info[0] = d.m;
    info[1] = (double)d.argmax;
    info[2] = d.Z;
    info[3] = (double)d.kept;
    info[4] = d.thr;
    info[5] = d.topp_margin;
    info[6] = d.topp_at;
    info[7] = d.topp_prev;
  }
  return 0;
}

int oracle_spec_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                       const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                       const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                       int32_t* tokens, int32_t* accept_len, double* logprobs, double* alpha, double* diag,
                       int32_t* dflags, int32_t num_threads) {
  if (B < 1 || k < 1 || V < 1 || offset >= (1ull << 32)) return 1;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_F32) return 1;
  VerifyArgs a{target_logits, draft_logits, dtype, draft_tokens, temperature, top_k, top_p, B, k, V,
               seed, (uint32_t)offset, tokens, accept_len, logprobs, alpha, diag, dflags, nullptr, nullptr,
               nullptr};
  parallel_rows(B, num_threads, [&](int32_t b) { verify_row(a, b); });
  return 0;
}

int oracle_spec_verify_ex(const void* target_logits, const void* draft_logits, int32_t dtype,
                          const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                          const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                          int32_t* tokens, int32_t* accept_len, double* logprobs, double* alpha, double* diag,
                          int32_t* dflags, const int32_t* alt, double* topp_rows, double* accept_pos,
                          int32_t num_threads) {
  if (B < 1 || k < 1 || V < 1 || offset >= (1ull << 32)) return 1;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_F32) return 1;
  VerifyArgs a{target_logits, draft_logits, dtype, draft_tokens, temperature, top_k, top_p, B, k, V,
               seed, (uint32_t)offset, tokens, accept_len, logprobs, alpha, diag, dflags, alt, topp_rows,
               accept_pos};
  std::vector<int32_t> rows;  // with alternatives: only the rows asked for
  for (int32_t b = 0; b < B; ++b)
    if (!alt || alt[(size_t)b * 4 + 3] != 0) rows.push_back(b);
  if (rows.empty()) return 0;
  parallel_rows((int32_t)rows.size(), num_threads, [&](int32_t j) { verify_row(a, rows[(size_t)j]); });
  return 0;
}

// The raw logprob of each committed token: the natural-log softmax of its position's unprocessed target
// logits (no temperature, no truncation), the other reading of the logprobs that plain sampling reports
// (AReno pull request "feat(engine): MTP training loss and speculative decoding for bailing_v3", section
// "What does this PR do?", Phase-2 paragraph: speculative decoding leaves them unchanged).  Slots after
// the committed ones are 0; sentinel rows (accept_len 0) are NaN.
int oracle_raw_logprobs(const void* target_logits, int32_t dtype, const int32_t* tokens, const int32_t* accept_len,
                        int32_t B, int32_t k, int32_t V, const float* temperature, double* out,
                        int32_t num_threads) {
  if (B < 1 || k < 0 || V < 1) return 1;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_F32) return 1;
  parallel_rows(B, num_threads, [&](int32_t b) {
    const int32_t committed = accept_len[b];
    std::vector<double> l;
    for (int32_t i = 0; i <= k; ++i) {
      const size_t o = (size_t)b * (k + 1) + i;
      if (committed == 0) {
        out[o] = kNaN;
        continue;
      }
      if (i >= committed) {
        out[o] = 0.0;
        continue;
      }
      load_row(target_logits, dtype, (size_t)b * (k + 1) + i, V, l);
#if ORACLE_MUTANT == 15
      for (double& v : l) v /= (double)temperature[b];  // MUTANT 15: the temperature is applied
#else
      (void)temperature;
#endif
      double m = -kInf;
      for (int32_t x = 0; x < V; ++x) m = std::max(m, l[(size_t)x]);
      double s = 0.0;
      for (int32_t x = 0; x < V; ++x) s += std::exp(l[(size_t)x] - m);
      const int32_t y = tokens[o];
#if ORACLE_MUTANT == 14
      out[o] = (l[(size_t)y] - m) / std::log(2.0) - std::log2(s);  // MUTANT 14: base-2 logarithm
#else
      out[o] = (l[(size_t)y] - m) - std::log(s);
#endif
    }
  });
  return 0;
}

// The commit step after verify (AReno pull request above, section "What does this PR do?": the Phase-2
// paragraph's recurrent and conv caches stacked across layers with one shared verify-state buffer, and
// the per-step table's commit row; InfiniLM pull request "add mtp draft models for speculative
// decoding", the state-consistency row of its mechanism table).  The verify forward is fed k+1 tokens
// per row (the last committed token, then the k drafts) and leaves, for every layer l, row b and fed
// position j, the state after position j in verify_state[l][b][j] (row_bytes bytes).  With n drafts
// accepted, accept_len = n + 1 tokens were consumed (the last committed token and the n drafts; the
// drawn token is fed at the next step), so the committed state is the one after position accept_len-1:
//   state_cache[l][state_slot[b]] = verify_state[l][b][accept_len[b] - 1]   for every layer l,
//   seq_len[b] += accept_len[b]  (keys and values of the rejected positions lie past the new length).
// A row with accept_len outside 1..k+1 (0 marks a row whose inputs were unusable) or a slot outside
// 0..num_slots-1 keeps its state and length; status[b] (may be NULL) is 0 for a committed row, 1 for
// a bad accept_len, 2 for a bad slot.  seq_len may be NULL.  Plain byte copies, row by row.
int oracle_commit(const void* verify_state, void* state_cache, const int32_t* state_slot,
                  const int32_t* accept_len, int32_t* seq_len, int32_t* status, int32_t L, int32_t B, int32_t k,
                  int32_t num_slots, int64_t row_bytes) {
  if (L < 1 || B < 1 || k < 0 || num_slots < 1 || row_bytes < 1) return 1;
  const uint8_t* src = (const uint8_t*)verify_state;
  uint8_t* dst = (uint8_t*)state_cache;
  const size_t rb = (size_t)row_bytes;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t a = accept_len[b];
    const int32_t slot = state_slot[b];
    int32_t st = 0;
    if (a < 1 || a > k + 1) st = 1;
    else if (slot < 0 || slot >= num_slots) st = 2;
    if (status) status[b] = st;
    if (st != 0) continue;
#if ORACLE_MUTANT == 16
    const int32_t j = a < k + 1 ? a : k;  // MUTANT 16: the state after the drawn token's position
#else
    const int32_t j = a - 1;
#endif
    for (int32_t l = 0; l < L; ++l) {
#if ORACLE_MUTANT == 17
      const size_t from = (((size_t)b * L + l) * (size_t)(k + 1) + (size_t)j) * rb;  // MUTANT 17: [B][L] order
#else
      const size_t from = (((size_t)l * B + b) * (size_t)(k + 1) + (size_t)j) * rb;
#endif
#if ORACLE_MUTANT == 19
      const size_t to = ((size_t)l * (size_t)num_slots + (size_t)b) * rb;  // MUTANT 19: slot map ignored
#else
      const size_t to = ((size_t)l * (size_t)num_slots + (size_t)slot) * rb;
#endif
      std::memcpy(dst + to, src + from, rb);
    }
#if ORACLE_MUTANT == 18
    if (seq_len) seq_len[b] += a - 1;  // MUTANT 18: length grows by the accepted drafts only
#else
    if (seq_len) seq_len[b] += a;
#endif
  }
  return 0;
}

// The commit step by slot numbers (InfiniLM pull request "add mtp draft models for speculative decoding",
// the state-consistency row of its mechanism table: verify writes to a scratch slot and a full accept
// swaps slot numbers instead of copying).  Here the verify forward writes the state after fed position j
// of row b into pool slot pos_slot[b][j], so any accept length is a swap: the row's committed slot
// becomes pos_slot[b][accept_len - 1], and the slot it held takes that place among the row's scratch
// slots.  seq_len and status as in oracle_commit.  No state byte moves.
int oracle_commit_slots(int32_t* state_slot, int32_t* pos_slot, const int32_t* accept_len, int32_t* seq_len,
                        int32_t* status, int32_t B, int32_t k, int32_t num_slots) {
  if (B < 1 || k < 0 || num_slots < 1) return 1;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t a = accept_len[b];
    int32_t st = 0;
    if (a < 1 || a > k + 1) st = 1;
    else {
      const int32_t cur = state_slot[b];
      const int32_t nxt = pos_slot[(size_t)b * (size_t)(k + 1) + (size_t)(a - 1)];
      if (cur < 0 || cur >= num_slots || nxt < 0 || nxt >= num_slots) st = 2;
    }
    if (status) status[b] = st;
    if (st != 0) continue;
#if ORACLE_MUTANT == 20
    const size_t j = (size_t)b * (size_t)(k + 1) + (size_t)(a < k + 1 ? a : k);  // MUTANT 20: one position late
#else
    const size_t j = (size_t)b * (size_t)(k + 1) + (size_t)(a - 1);
#endif
    const int32_t held = state_slot[b];
    state_slot[b] = pos_slot[j];
#if ORACLE_MUTANT != 21
    pos_slot[j] = held;  // MUTANT 21 leaves the old slot out of the scratch set
#endif
    if (seq_len) seq_len[b] += a;
  }
  return 0;
}

int oracle_tree_verify(const void* target_logits, int32_t dtype, const int32_t* parent, const int32_t* node_tokens,
                       const float* temperature, const int32_t* top_k, const float* top_p, int32_t B, int32_t N,
                       int32_t V, uint64_t seed, uint64_t offset, int32_t* tokens, int32_t* path, int32_t* accept_len,
                       double* logprobs, double* diag, int32_t num_threads) {
  if (B < 1 || N < 1 || V < 1 || offset >= (1ull << 32)) return 1;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_F32) return 1;
  TreeArgs a{target_logits, dtype, parent, node_tokens, temperature, top_k, top_p, B, N, V, seed, (uint32_t)offset,
             tokens, path, accept_len, logprobs, diag};
  parallel_rows(B, num_threads, [&](int32_t b) { tree_row(a, b); });
  return 0;
}

int oracle_sample(const void* logits, int32_t dtype, const float* temperature, const int32_t* top_k,
                  const float* top_p, const int32_t* row_b, const int32_t* row_pos, int32_t R, int32_t V,
                  uint64_t seed, uint64_t offset, int32_t* tokens, double* logprobs, double* gap,
                  int32_t num_threads) {
  if (R < 1 || V < 1 || offset >= (1ull << 32)) return 1;
  if (dtype != ORACLE_DTYPE_BF16 && dtype != ORACLE_DTYPE_F32) return 1;
  parallel_rows(R, num_threads, [&](int32_t r) {
    std::vector<double> l;
    load_row(logits, dtype, (size_t)r, V, l);
    RowDist d;
    double g = kInf;
    if (!params_valid(temperature[r], top_k[r], top_p[r]) || row_has_nan_or_posinf(l) ||
        !row_dist(l, (double)temperature[r], top_k[r], (double)top_p[r], d)) {
      tokens[r] = -1;
      logprobs[r] = kNaN;
      if (gap) gap[r] = kInf;
      return;
    }
    int32_t y;
    if (temperature[r] == 0.0f) {
      y = d.argmax;
    } else {
      y = gumbel_argmax(d.p, seed, 2u, (uint32_t)row_b[r], (uint32_t)row_pos[r], (uint32_t)offset, &g);
    }
    tokens[r] = y;
    logprobs[r] = std::log(d.p[(size_t)y]);
    if (gap) gap[r] = g;
  });
  return 0;
}

}  // extern "C"
