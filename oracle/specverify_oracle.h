/*
 * specverify_oracle.h -- plain CPU oracle for the speculative-decoding verify sampler.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the correctness reference for the GPU
 * library; only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the GPU path.
 *
 * Everything is computed in IEEE double precision from exactly converted inputs
 * (bf16 -> double and fp32 -> double are exact), with plain loops and std::sort.
 *
 * What is computed follows the AReno pull request "feat(engine): MTP training loss and
 * speculative decoding for bailing_v3" (page section "What does this PR do?", Phase 2:
 * a sampler-equivalent target distribution, exact chain rejection sampling, unchanged
 * logprobs; accept-probability table: alpha = sum of min(p, q); step-time table:
 * Gumbel-max draws instead of multinomial).  Points the page leaves open are resolved
 * by the readings listed in the repository design notes; each function below names
 * the reading it takes.
 *
 * Counter-based random numbers: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3", SC'11), with the stream layout:
 *   key  = (seed & 0xffffffff, seed >> 32)
 *   accept uniform u(b,i):           ctr = (i>>2, b, 0,               offset), word i&3,
 *                                    u = (w >> 8) * 2^-24
 *   verify Gumbel uniform U(b,j,x):  ctr = (x>>2, b, (1<<24) | j,     offset), word x&3,
 *                                    U = ((w >> 9) + 0.5) * 2^-23,  G = -ln(-ln U)
 *   plain-sampler uniform U(b,i,x):  ctr = (x>>2, b, (2<<24) | i,     offset), word x&3,
 *                                    same map as the verify Gumbel uniform.
 */
#ifndef SPECVERIFY_ORACLE_H
#define SPECVERIFY_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes of the logit arrays: 0 = bf16 (raw 16-bit patterns), 1 = fp32 */
#define ORACLE_DTYPE_BF16 0
#define ORACLE_DTYPE_F32 1

/* Philox-4x32-10 block function: out = philox(ctr, key). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The stream values defined in the header comment. */
double oracle_accept_uniform(uint64_t seed, uint32_t b, uint32_t i, uint32_t offset);
double oracle_gumbel_uniform(uint64_t seed, uint32_t tag, uint32_t b, uint32_t j, uint32_t x, uint32_t offset);

/*
 * Sampler distribution of one logit row (temperature, top-k, top-p as in plain sampling).
 *   logits : V doubles (may contain -inf; NaN/+inf are the caller's concern)
 *   T      : temperature; 0 = greedy (one-hot at the lowest-index maximum)
 *   K      : top-k; 0 or >= V = off
 *   P      : top-p; >= 1 = off
 *   probs  : out, V doubles, the distribution (zeros outside the kept set)
 *   info   : out (may be NULL), 8 doubles:
 *            [0] row max m, [1] lowest argmax, [2] kept-set normaliser Z (sum of exp((l-m)/T) over kept),
 *            [3] number of kept entries, [4] kept threshold value (smallest kept logit),
 *            [5] top-p decision margin (min distance of M(v)/Z_K to P at the chosen value and the next
 *                larger distinct value; +inf if top-p is off or T == 0),
 *            [6] the distance at the chosen value, [7] the distance at the next larger distinct value
 * Returns 0 on success, nonzero if the row is invalid (all -inf).
 */
int oracle_row_probs(const double* logits, int32_t V, double T, int32_t K, double P, double* probs, double* info);

/*
 * Full verify step, host arrays.  Argument order and meaning follow the GPU library's
 * spec_verify(); outputs are in double so that comparisons see the oracle's own values.
 *   target_logits [B, k+1, V], draft_logits [B, k, V] (dtype as above)
 *   draft_tokens [B, k]; temperature/top_k/top_p [B]
 *   tokens [B, k+1]  (committed tokens, -1 padding)      accept_len [B] (n_accepted + 1; 0 = invalid row)
 *   logprobs [B, k+1] (ln p_i of the committed token at position i, 0 padding)
 *   alpha [B, k]      (sum_x min(p_i(x), q_i(x)))
 *   diag [B, 4] (may be NULL): [0] accept margin = min |u_i - p_i/q_i| over evaluated tests with p,q > 0,
 *                              [1] Gumbel top-2 gap at the sampled position (natural-log key units),
 *                              [2] top-p decision margin, min over the row's 2k+1 distributions,
 *                              [3] residual mass sum max(p_n - q_n, 0) at the rejection position (-1 if none)
 *     (+inf where not applicable)
 *   dflags [B] (may be NULL): bit0 = residual fell back to p_n, bit1 = invalid (sentinel) row,
 *                             bits 8.. = number of accepted drafts n
 *   num_threads: worker threads over batch rows (0 = hardware concurrency)
 * Invalid rows get accept_len 0, tokens -1, logprobs NaN, alpha NaN.
 * Returns 0, or 1 for bad scalar arguments (nothing written).
 */
int oracle_spec_verify(const void* target_logits, const void* draft_logits, int32_t dtype,
                       const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                       const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                       int32_t* tokens, int32_t* accept_len, double* logprobs, double* alpha, double* diag,
                       int32_t* dflags, int32_t num_threads);

/*
 * The verify step with per-decision diagnostics and alternative resolutions, for the parity check of
 * rows whose outcome a correct rounding could change (the margin rows).  Arguments as in
 * oracle_spec_verify, plus (each may be NULL):
 *   alt [B, 4]: row b is computed only if alt[b][3] != 0 (other rows' outputs are left untouched);
 *               alt[b][0] bit r: logit row r (targets 0..k, then drafts k+1..2k) keeps one more distinct
 *               value than its top-p threshold (as if M(v) had fallen just short of P Z_K);
 *               alt[b][1] bit r: logit row r's top-p threshold moves to the next larger distinct value
 *               (as if that value's M had reached P Z_K);
 *               alt[b][2] bits 0..k-1: the accept test at that position is decided the other way;
 *               alt[b][2] bit 16: the draw takes the runner-up of the Gumbel race.
 *   topp_rows [B, 2k+1, 2] out: per logit row, |M(v)/Z_K - P| at the chosen top-p value and at the next
 *               larger distinct value (+inf where top-p is off, T == 0, or no such value).
 *   accept_pos [B, k] out: |u_i - p_i(x_i)/q_i(x_i)| for each evaluated accept test with p, q > 0 and
 *               T > 0 (+inf for tests not evaluated).
 */
int oracle_spec_verify_ex(const void* target_logits, const void* draft_logits, int32_t dtype,
                          const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                          const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                          int32_t* tokens, int32_t* accept_len, double* logprobs, double* alpha, double* diag,
                          int32_t* dflags, const int32_t* alt, double* topp_rows, double* accept_pos,
                          int32_t num_threads);

/*
 * Plain (non-speculative) sampler over R independent logit rows [R, V]: Gumbel-max over the
 * sampler distribution with the plain-sampler stream, row r using stream coordinates
 * (b = row_b[r], i = row_pos[r]).  Greedy rows take the lowest-index maximum.
 *   tokens [R] out; logprobs [R] out (ln of the sampler probability of the token);
 *   gap [R] out (may be NULL): Gumbel top-2 gap (+inf for greedy or a single candidate).
 * Invalid rows (bad parameters, NaN/+inf, all -inf) get token -1, logprob NaN.
 */
int oracle_sample(const void* logits, int32_t dtype, const float* temperature, const int32_t* top_k,
                  const float* top_p, const int32_t* row_b, const int32_t* row_pos, int32_t R, int32_t V,
                  uint64_t seed, uint64_t offset, int32_t* tokens, double* logprobs, double* gap,
                  int32_t num_threads);

/*
 * Commit step: for every row b with 1 <= accept_len[b] <= k+1 and 0 <= state_slot[b] < num_slots,
 *   state_cache[l][state_slot[b]][:] = verify_state[l][b][accept_len[b]-1][:]  (all L layers)
 *   seq_len[b] += accept_len[b]                                                  (seq_len may be NULL)
 *   verify_state [L, B, k+1, row_bytes], state_cache [L, num_slots, row_bytes] (raw bytes)
 *   status [B] out (may be NULL): 0 committed, 1 accept_len out of range, 2 slot out of range
 * Other rows are left as they are.  Returns 0, or 1 for bad scalar arguments (nothing written).
 */
int oracle_commit(const void* verify_state, void* state_cache, const int32_t* state_slot,
                  const int32_t* accept_len, int32_t* seq_len, int32_t* status, int32_t L, int32_t B, int32_t k,
                  int32_t num_slots, int64_t row_bytes);

/*
 * Commit step by slot numbers: for every row b with 1 <= accept_len[b] <= k+1 whose current slot
 * state_slot[b] and accepted-position slot pos_slot[b][accept_len[b]-1] both lie in 0..num_slots-1,
 *   swap(state_slot[b], pos_slot[b][accept_len[b]-1]);  seq_len[b] += accept_len[b]  (seq_len may be NULL)
 *   state_slot [B] in/out, pos_slot [B, k+1] in/out; status [B] out (may be NULL): 0 committed,
 *   1 accept_len out of range, 2 a slot out of range.  Other rows are left as they are.
 * Returns 0, or 1 for bad scalar arguments (nothing written).
 */
int oracle_commit_slots(int32_t* state_slot, int32_t* pos_slot, const int32_t* accept_len, int32_t* seq_len,
                        int32_t* status, int32_t B, int32_t k, int32_t num_slots);

/*
 * Tree verification (recursive rejection for deterministic, distinct draft children):
 *   target_logits [B, N, V] (row i: the target distribution after node i; node 0 is the root, the last
 *   committed token); parent [B, N] (parent[b][i] < i for i >= 1; entry 0 ignored); node_tokens [B, N]
 *   (the draft token of node i >= 1; siblings must differ); temperature/top_k/top_p [B].
 *   tokens [B, N] out: the accepted nodes' tokens, then the drawn token, then -1
 *   path [B, N] out: the accepted node indices (root excluded), then -1
 *   accept_len [B] out: accepted nodes + 1 (0 = unusable row)
 *   logprobs [B, N] out: ln p of each committed token under the distribution it was drawn from, 0 after
 *   diag [B, 4] (may be NULL): [0] min |U - S_j| over evaluated children with S_j > 0, [1] Gumbel top-2
 *   gap of the final draw, [2] top-p margin over the N rows, [3] the stopping node.
 * Unusable rows (bad parameters, a bad tree, NaN/+inf or all -inf in any of the N rows) get
 * accept_len 0, tokens and path -1, logprobs NaN.  Returns 0, or 1 for bad scalar arguments.
 */
int oracle_tree_verify(const void* target_logits, int32_t dtype, const int32_t* parent, const int32_t* node_tokens,
                       const float* temperature, const int32_t* top_k, const float* top_p, int32_t B, int32_t N,
                       int32_t V, uint64_t seed, uint64_t offset, int32_t* tokens, int32_t* path, int32_t* accept_len,
                       double* logprobs, double* diag, int32_t num_threads);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_ORACLE_H */
