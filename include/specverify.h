/*
 * specverify.h -- C ABI of libspecverify, the MI355X (gfx950) speculative-decoding verify sampler.
 *
 * What the library computes (AReno pull request "feat(engine): MTP training loss and speculative
 * decoding for bailing_v3", section "What does this PR do?", Phase 2 paragraph; its accept-probability
 * table; its per-step optimisation table):
 *
 *   For every batch row b, the k+1 target logit rows and the k draft logit rows are turned into the
 *   distributions plain sampling would draw from (temperature, then top-k, then top-p on the top-k
 *   renormalised mass, ties at a threshold kept whole; temperature 0 = greedy one-hot at the
 *   lowest-index maximum): p_0..p_k (target) and q_0..q_{k-1} (draft).  Draft x_i is accepted while
 *   p_i(x_i) > 0 and (q_i(x_i) == 0 or u_i < p_i(x_i) / q_i(x_i)); at the first rejection n one token
 *   is drawn from normalize(max(p_n - q_n, 0)), and when all k are accepted a bonus token is drawn
 *   from p_k.  Draws are Gumbel-max (argmax of ln w(x) + G(x), lowest index on exact ties) on a
 *   Philox-4x32-10 stream.  Reported are the committed tokens, their count, ln p_i of each committed
 *   token, and alpha_i = sum_x min(p_i(x), q_i(x)) for every draft position.
 *
 * Random stream (Philox-4x32-10 of Salmon et al., SC'11; key = (seed & 0xffffffff, seed >> 32)):
 *   accept uniform u(b,i):        counter (i>>2, b, 0, offset), word i&3, u = (w>>8) * 2^-24
 *   verify Gumbel U(b,j,x):       counter (x>>2, b, (1<<24)|j, offset), word x&3, U = ((w>>9)+0.5) * 2^-23
 *   plain-sampler Gumbel U(b,i,x): counter (x>>2, b, (2<<24)|i, offset), word x&3, same map
 * b is the batch row index within the call.  Replaying a call with the same (seed, offset) reproduces
 * its outputs bit for bit; callers advance `offset` between calls.
 *
 * Memory and streams.  Every pointer except `stream` is a device pointer owned by the caller.  The
 * library allocates nothing per call and keeps no per-call state outside the caller's workspace.  A
 * call only enqueues work on `stream` (a hipStream_t; NULL = the default stream) and returns without
 * synchronising, so it can be captured in a HIP graph.  Outputs are valid once the stream reaches the
 * enqueued work.  Calls that share one workspace must be ordered on one stream.
 *
 * Errors.  Scalar, pointer and size problems detectable on the host return a status and enqueue
 * nothing.  Problems found in the data (a draft token outside [0, V), a NaN or +inf logit in any of
 * a batch row's 2k+1 rows, a row that is entirely -inf, a temperature that is NaN, negative or
 * infinite, top_k < 0, top_p <= 0 or NaN) turn that batch row into a sentinel row: accept_len 0,
 * tokens -1, logprobs NaN, alpha NaN.  -inf logits are legal and mean probability 0.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPEC_DTYPE_BF16 = 0, SPEC_DTYPE_F32 = 1 } spec_dtype_t;

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARGUMENT = 1,   /* bad scalar, null or misaligned pointer, offset >= 2^32 */
  SPEC_ERR_WORKSPACE = 2,          /* workspace null or smaller than spec_verify_workspace_size() */
  SPEC_ERR_UNSUPPORTED_DEVICE = 3, /* the current device is not a gfx950 */
  SPEC_ERR_LAUNCH = 4              /* the HIP runtime refused the launch */
} spec_status_t;

/*
 * Bytes of device workspace spec_verify() needs for these sizes (0 if the sizes are invalid).
 * The workspace needs no initialisation and may hold anything: every call writes each workspace byte it
 * reads (partials, arrival counters, flags) before reading it, in stream order.  Calls that share one
 * workspace must not overlap (order them on one stream).
 */
size_t spec_verify_workspace_size(int32_t B, int32_t k, int32_t V, spec_dtype_t dtype);

/*
 * The verify step (see the top of this file for the method).
 *
 *   target_logits  [B, k+1, V] row-major, contiguous, dtype; 16-byte aligned
 *   draft_logits   [B, k,   V] row-major, contiguous, dtype; 16-byte aligned
 *   dtype          SPEC_DTYPE_BF16 (V % 8 == 0) or SPEC_DTYPE_F32 (V % 4 == 0)
 *   draft_tokens   int32 [B, k]
 *   temperature    float [B]   0 = greedy (top_k/top_p ignored)
 *   top_k          int32 [B]   0 or >= V = off
 *   top_p          float [B]   >= 1 (including +inf) = off
 *   B, k, V        1 <= B <= 2^20, 1 <= k <= 8, 1 <= V <= 2^20 (with V % 8 == 0 for bf16 and
 *                  V % 4 == 0 for fp32, so V >= 8 for bf16 and V >= 4 for fp32)
 *   seed, offset   Philox key and counter word 3; offset < 2^32
 *   tokens         out int32 [B, k+1]  x_0..x_{n-1}, the drawn token, then -1
 *   accept_len     out int32 [B]       n + 1 (committed tokens, 1..k+1), 0 for a sentinel row
 *   logprobs       out float [B, k+1]  ln p_i(tokens[b,i]) for i <= n, 0 after
 *   alpha          out float [B, k]    sum_x min(p_i(x), q_i(x)) for every i < k
 *   workspace      device scratch of at least spec_verify_workspace_size() bytes (see there)
 *   stream         hipStream_t or NULL
 * Every output element is written by every successful call.
 */
spec_status_t spec_verify(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                          const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                          const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                          int32_t* tokens, int32_t* accept_len, float* logprobs, float* alpha, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * The verify step for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): spec_verify's arguments and outputs without the
 * workspace.  The library keeps one scratch array of SPEC_NOALLOC_SCRATCH_BYTES per GPU in its own static
 * device memory (held by every GPU the library is loaded on, until the process ends) and runs the same
 * kernels on it; nothing is allocated or freed by the call.
 *   Sizes whose spec_verify_workspace_size() exceeds SPEC_NOALLOC_SCRATCH_BYTES: SPEC_ERR_WORKSPACE,
 *   nothing enqueued.  The scratch array's device address is looked up once per GPU, on the first call
 *   with that GPU current (SPEC_ERR_LAUNCH if that fails).
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (on different streams,
 *   from different threads, or in graphs replayed concurrently) race and give wrong results; order them.
 *   The array needs no clearing: each call sets up every byte it reads.
 */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

spec_status_t spec_verify_noalloc(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                  const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                                  const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed,
                                  uint64_t offset, int32_t* tokens, int32_t* accept_len, float* logprobs,
                                  float* alpha, void* stream);

/*
 * The verify step with raw logprobs as well: spec_verify's arguments and outputs, plus
 *
 *   raw_logprobs   out float [B, k+1]  for i <= n: ln softmax of target row i's unprocessed logits (no
 *                                     temperature, no truncation) at tokens[b,i]; 0 after; NaN for a
 *                                     sentinel row
 *
 * This is the other reading of "the reported logprobs" that speculative decoding leaves unchanged (AReno
 * pull request above, section "What does this PR do?", Phase-2 paragraph): the model's own log-probability
 * of each committed token rather than its log-probability under the sampler distribution.  Greedy rows
 * get a finite value too.  It costs an extra exp per target logit in the statistics kernel.
 * raw_logprobs must not be NULL (SPEC_ERR_INVALID_ARGUMENT); the workspace is spec_verify's.
 */
spec_status_t spec_verify_raw(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                              const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                              const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                              int32_t* tokens, int32_t* accept_len, float* logprobs, float* raw_logprobs,
                              float* alpha, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Plain (non-speculative) sampler: one token per logit row from the same sampler distribution
 * (temperature, top-k, top-p as above) by Gumbel-max on the plain-sampler stream.  This is the step
 * either side of verify: it draws the draft tokens from q, and it is what "sampler-equivalent" refers
 * to (AReno pull request above, section "How was it tested?": sampler equivalence with and without
 * top-k/top-p).
 *
 *   logits        [R, V] row-major, contiguous, dtype; 16-byte aligned
 *   temperature   float [R]; top_k int32 [R]; top_p float [R] (meaning as in spec_verify)
 *   row_b, row_pos  int32 [R] stream coordinates (b, i) of each row; NULL = (row index, 0)
 *   R, V          1 <= R <= 2^20, 1 <= V <= 2^20 (V % 8 == 0 for bf16, V % 4 == 0 for fp32)
 *   tokens        out int32 [R]   the drawn token (-1 for a row with unusable inputs)
 *   logprobs      out float [R]   ln of its sampler probability (0 for greedy rows, NaN if unusable)
 *   workspace     at least spec_sample_workspace_size(R, V, dtype) bytes, same rules as spec_verify
 */
size_t spec_sample_workspace_size(int32_t R, int32_t V, spec_dtype_t dtype);

spec_status_t spec_sample(const void* logits, spec_dtype_t dtype, const float* temperature, const int32_t* top_k,
                          const float* top_p, const int32_t* row_b, const int32_t* row_pos, int32_t R, int32_t V,
                          uint64_t seed, uint64_t offset, int32_t* tokens, float* logprobs, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * Tree verification: verify a draft tree per batch row instead of a chain.  The pages name only the
 * draft-tree parameters (EAGLE top-k, passed through to SGLang's NEXTN speculative decoding: AReaL pull
 * request "MTP training with speculative decoding rollout", its key-changes list); the rule is the
 * published recursive rejection for draft children that are distinct tokens chosen deterministically
 * (top-k of the draft), which keeps the committed sequence distributed exactly as target sampling:
 *
 *   Start at the root (node 0: the last committed token).  At a node u with children c_1..c_m (in node
 *   index order) and sampler distribution p_u (temperature, top-k, top-p as in spec_verify), draw one
 *   uniform U (the accept stream of spec_verify at position = depth) and accept the first child j with
 *   U < p_u(t_{c_1}) + ... + p_u(t_{c_j}); continue at that child.  If no child is accepted, draw the
 *   committed extra token from p_u with the children's tokens removed; at a leaf, draw it from p_u.
 *   Draws are Gumbel-max on spec_verify's draw stream at position = depth.  Greedy rows (T = 0) follow
 *   the child whose token is the row's lowest-index argmax and end on the argmax.
 *
 * A tree whose nodes each have one child gives spec_verify's tokens and accept lengths for draft rows
 * that are one-hot at the draft tokens (0 there, -inf elsewhere), and its logprobs up to the rounding of
 * the fp32 normaliser sums (which spec_verify may add up in another order).
 *
 *   target_logits  [B, N, V] contiguous, dtype, 16-byte aligned: row i is the target's logits after node i
 *   parent         int32 [B, N]  parent[b][i] in 0..i-1 for i >= 1 (entry 0 ignored)
 *   node_tokens    int32 [B, N]  draft token of node i >= 1 (entry 0 ignored); siblings must differ
 *   temperature, top_k, top_p   [B] as in spec_verify
 *   B, N, V        1 <= B <= 2^20, 1 <= N <= 64, B * N <= 2^24, V as in spec_verify
 *   tokens         out int32 [B, N]  the accepted nodes' tokens, then the drawn token, then -1
 *   path           out int32 [B, N]  the accepted node indices (root excluded), then -1
 *   accept_len     out int32 [B]     accepted nodes + 1 (committed tokens); 0 for an unusable row
 *   logprobs       out float [B, N]  ln p of each committed token under the distribution it was drawn from
 *                                    (0 for greedy rows), 0 after
 *   workspace      at least spec_tree_verify_workspace_size(B, N, V, dtype) bytes, same rules as spec_verify
 * A row is unusable (accept_len 0, tokens and path -1, logprobs NaN) if its parameters are invalid, its
 * tree breaks the rules above, or any of its N logit rows holds NaN or +inf or is entirely -inf.
 */
size_t spec_tree_verify_workspace_size(int32_t B, int32_t N, int32_t V, spec_dtype_t dtype);

spec_status_t spec_tree_verify(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                               const int32_t* node_tokens, const float* temperature, const int32_t* top_k,
                               const float* top_p, int32_t B, int32_t N, int32_t V, uint64_t seed, uint64_t offset,
                               int32_t* tokens, int32_t* path, int32_t* accept_len, float* logprobs, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Commit step: after verify, make each batch row's cached model state the state after its last consumed
 * token (AReno pull request above, section "What does this PR do?": the Phase-2 paragraph keeps the
 * recurrent and conv caches stacked across layers with one verify-state buffer, and its per-step table
 * commits them in a few kernels; InfiniLM pull request "add mtp draft models for speculative decoding",
 * the state-consistency row of its mechanism table: verify reads the committed state and writes elsewhere,
 * and only (k, accepted count) decide what becomes committed).
 *
 * The verify forward is fed k+1 tokens per row (the last committed token, then the k drafts) and writes,
 * for every layer l, row b and fed position j, the state after position j into verify_state[l][b][j].
 * With accept_len = n + 1 (n drafts accepted), the last committed token and the n drafts were consumed
 * and the drawn token will be fed at the next step, so the state after position accept_len - 1 is the
 * one to keep.  For every row b with 1 <= accept_len[b] <= k+1 and 0 <= state_slot[b] < num_slots:
 *
 *   state_cache[l][state_slot[b]][:] = verify_state[l][b][accept_len[b] - 1][:]  for every tensor, layer
 *   seq_len[b] += accept_len[b]
 *
 * Keys and values of full-attention layers need no copy: verify wrote all k+1 positions in place, and
 * the ones past the new seq_len are overwritten by the next step, so seq_len is their whole commit.
 * Other rows (accept_len 0 marks a sentinel row of spec_verify) keep their state and length.
 *
 *   tensors     HOST array of n_tensors descriptors (read during the call only); each names one stateful
 *               tensor stacked across its layers:
 *                 verify_state  device [layers, B, k+1, row_bytes] bytes (any dtype; copied bit for bit)
 *                 state_cache   device [layers, num_slots, row_bytes] bytes
 *                 row_bytes     one layer's state of one row, >= 1; layers >= 1; layers * B < 2^31
 *               n_tensors 0 .. SPEC_COMMIT_MAX_TENSORS (0: only seq_len / status, e.g. a model whose
 *               layers all keep keys and values)
 *   state_slot  device int32 [B]   cache slot of each row (rows committed in one call need distinct slots)
 *   accept_len  device int32 [B]   spec_verify's accept_len
 *   seq_len     device int32 [B] in/out, may be NULL
 *   status      device int32 [B] out, may be NULL: 0 committed, 1 accept_len outside 1..k+1,
 *               2 slot outside 0..num_slots-1 (checked in that order)
 *   B           1 .. 2^20;  k  0 .. 255;  num_slots >= 1
 * No verify_state range may overlap any state_cache range, and state_cache ranges must not overlap
 * each other (SPEC_ERR_INVALID_ARGUMENT).  Copies are fastest with row_bytes a multiple of 16 and
 * 16-byte aligned tensors; any size and alignment is accepted.  Enqueues one kernel on `stream` and
 * returns without synchronising; needs no workspace.
 */
#define SPEC_COMMIT_MAX_TENSORS 8

typedef struct {
  const void* verify_state;
  void* state_cache;
  int64_t row_bytes;
  int32_t layers;
} spec_state_tensor_t;

spec_status_t spec_commit(const spec_state_tensor_t* tensors, int32_t n_tensors, const int32_t* state_slot,
                          const int32_t* accept_len, int32_t* seq_len, int32_t* status, int32_t B, int32_t k,
                          int32_t num_slots, void* stream);

/*
 * Commit step by slot numbers: the same commit without moving state bytes, for callers whose verify
 * forward writes each fed position's state into a slot of a shared pool (InfiniLM pull request above, the
 * state-consistency row of its mechanism table: verify writes a scratch slot and a full accept swaps slot
 * numbers; keeping one scratch slot per fed position makes every accept length a swap, so a partial
 * accept needs no replay).  Row b's committed state lives in pool slot state_slot[b] and the verify
 * forward wrote the state after fed position j into pool slot pos_slot[b][j].  For every row with
 * 1 <= accept_len[b] <= k+1 whose state_slot[b] and pos_slot[b][accept_len[b]-1] both lie in
 * 0..num_slots-1:
 *
 *   swap(state_slot[b], pos_slot[b][accept_len[b] - 1]);   seq_len[b] += accept_len[b]
 *
 * so the accepted position's slot becomes the committed one and the previous committed slot joins the
 * row's scratch slots for the next verify.  The pool itself is not touched (the caller owns it).
 *
 *   state_slot  device int32 [B] in/out
 *   pos_slot    device int32 [B, k+1] in/out
 *   accept_len  device int32 [B]   spec_verify's accept_len
 *   seq_len     device int32 [B] in/out, may be NULL
 *   status      device int32 [B] out, may be NULL: 0 committed, 1 accept_len outside 1..k+1,
 *               2 a slot outside 0..num_slots-1 (the row is then left as it is)
 *   B           1 .. 2^20;  k  0 .. 255;  num_slots >= 1
 * None of the five arrays may overlap another (SPEC_ERR_INVALID_ARGUMENT).  Enqueues one kernel on
 * `stream` and returns without synchronising; needs no workspace.
 */
spec_status_t spec_commit_slots(int32_t* state_slot, int32_t* pos_slot, const int32_t* accept_len, int32_t* seq_len,
                                int32_t* status, int32_t B, int32_t k, int32_t num_slots, void* stream);

/* A static, human-readable name of a status code. */
const char* spec_verify_status_string(spec_status_t status);

/*
 * Per-kernel timing of one call, for benchmarks.  The timed entry points take the arguments of the call
 * they time (spec_verify_timed: spec_verify's, plus raw_logprobs, which may be NULL for the plain verify
 * step and otherwise makes it spec_verify_raw; spec_tree_verify_timed: spec_tree_verify's) and one
 * spec_timing_t.  They enqueue exactly the same kernels, and in addition record, on `stream`,
 * events[2j] just before kernel j and events[2j+1] just after it, for each of the kernels the call
 * launches; `kernels` receives how many that is (1 .. SPEC_MAX_KERNELS; which kernels depends on the
 * sizes and the device).  hipEventElapsedTime(events[2j], events[2j+1]) is then kernel j's duration.
 *
 *   events      HOST array of 2 * SPEC_MAX_KERNELS hipEvent_t handles, created by the caller with timing
 *               enabled, or NULL (no events recorded); read during the call only.  Entries past
 *               2 * kernels are not recorded.
 *   kernels     out: kernels this call launched (1: the one-launch resident path; 2 or 3: the staged path)
 *   path        in: SPEC_PATH_AUTO (the library chooses), SPEC_PATH_STAGED (slice statistics, row merges and
 *               the verify kernel as separate launches) or SPEC_PATH_RESIDENT (one launch that holds the
 *               logits on chip; bf16 verify calls whose grid fits the device, otherwise the staged path is
 *               taken, and `kernels` tells which ran).  Every path computes the same results up to fp32
 *               rounding order.  Other values are SPEC_ERR_INVALID_ARGUMENT.
 *   wait_limit  0 for the default, or a bound (in ticks of the GPU's 100 MHz clock) on each wait of a
 *               workgroup for its batch row's other workgroups in the one-launch path (the grid is
 *               co-resident, so the waits always end; the bound only keeps a stalled grid from hanging: a
 *               workgroup that gives up turns its batch row into a sentinel row and exits).  Tests use a
 *               tiny bound to exercise that path from the host.
 * Nothing is kept between calls: the timing applies to this call alone.  A NULL timing pointer is
 * SPEC_ERR_INVALID_ARGUMENT.
 */
#define SPEC_MAX_KERNELS 3
#define SPEC_PATH_AUTO 0
#define SPEC_PATH_STAGED 1
#define SPEC_PATH_RESIDENT 2

typedef struct {
  void* const* events;
  int32_t kernels;
  int32_t path;
  uint64_t wait_limit;
} spec_timing_t;

spec_status_t spec_verify_timed(const void* target_logits, const void* draft_logits, spec_dtype_t dtype,
                                const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                                const float* top_p, int32_t B, int32_t k, int32_t V, uint64_t seed, uint64_t offset,
                                int32_t* tokens, int32_t* accept_len, float* logprobs, float* raw_logprobs,
                                float* alpha, void* workspace, size_t workspace_bytes, void* stream,
                                spec_timing_t* timing);

spec_status_t spec_tree_verify_timed(const void* target_logits, spec_dtype_t dtype, const int32_t* parent,
                                     const int32_t* node_tokens, const float* temperature, const int32_t* top_k,
                                     const float* top_p, int32_t B, int32_t N, int32_t V, uint64_t seed,
                                     uint64_t offset, int32_t* tokens, int32_t* path, int32_t* accept_len,
                                     float* logprobs, void* workspace, size_t workspace_bytes, void* stream,
                                     spec_timing_t* timing);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
