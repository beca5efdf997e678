/*
 * dspark.h -- C ABI of the DSpark draft-sample-verify hot path for MI355X (gfx950).
 *
 * Pages this follows:
 *   [P1] "DSpark 的实现和测评"              (vLLM's DSpark speculator, walked through)
 *   [P2] "推测解码：从零到DSpark"            (summary of the DSpark paper)
 *   [P3] "xserv/docs/25-speculative-methods-comparison.md"
 *
 * One round of the path:
 *   dspark_draft_logits   stage 1: base logits of all N draft positions  [P1 §2.2, §4]
 *   dspark_markov_sample  stage 2: N-step low-rank Markov Gumbel-max loop [P1 §2.2, §3, §5; P2 §4]
 *   dspark_admit          stage 4: survival by chain rule, pooled top-K    [P2 §6, §7]
 *   dspark_verify         stage 3: lossless rejection-sampling verify      [P2 §2; P3 §2]
 *   dspark_markov_sample_deferred / dspark_verify_deferred
 *                         stages 2 and 3 without storing every processed draft row
 *   dspark_context_kv     the step before the path: draft KV cache of new context
 *                         tokens from the target's hidden states [P1 §4]
 *
 * Conventions shared by every call
 *   Memory     Every pointer argument is device memory (HBM) unless stated otherwise.
 *              The caller owns all buffers; the library never allocates, frees or
 *              reads device memory on the host.  Buffers touched with 16-byte
 *              vector accesses must be 16-byte aligned (stated per argument).
 *   Streams    `stream` is a hipStream_t (NULL = the default stream).  Every call
 *              only enqueues kernels on it and returns; buffers must stay alive
 *              until the stream has passed them.  Nothing synchronises.
 *   Workspace  Calls that need scratch take (workspace, workspace_bytes); the size
 *              comes from the matching *_workspace_size query.  Contents need no
 *              initialisation and are undefined afterwards.  One workspace must
 *              not be used by two calls in flight at once.
 *   Errors     Arguments are validated on the host before any launch; a failed
 *              check returns DSPARK_ERR_INVALID / _UNSUPPORTED / _WORKSPACE and
 *              enqueues nothing.  A failed launch returns DSPARK_ERR_HIP.  Faults
 *              inside kernels surface at the caller's next synchronisation.  The
 *              message of the last failure on the calling host thread is in
 *              dspark_last_error().  No C++ exception crosses this boundary.
 *   Threads    Calls are reentrant.  Global state: the thread-local error message,
 *              and per device 64 sets of grid-barrier counters (4.2 KB each, device
 *              memory, zero when the library loads) for the few-request Markov
 *              kernel: each dspark_markov_sample call with B <= 16 takes the next
 *              set, and every launch leaves its set zero again, so 64 or more such
 *              launches must not be in flight at once.  The same holds, with 64
 *              sets of 34 KB of tickets, for dspark_verify with logits input and
 *              B <= 16 (statistics and acceptance in one launch).
 *   Sampling   All randomness is Philox4x32-10 (Salmon et al., SC'11) with
 *                key = (seed & 0xffffffff, seed >> 32),
 *                counter = (index >> 2, position, request_id, tag), word index & 3,
 *              and uniform u = ((word >> 8) | 1) * 2^-24 in (0, 1).
 *              tag 0: Gumbel noise of stage 2 (index = draft-vocabulary index);
 *              tag 1: acceptance uniform of stage 3 (index 0);
 *              tag 2: residual resample race; tag 3: bonus race (index = target id).
 *   Temperature  T > 0 divides logits; T == 0 is greedy (argmax, no noise).
 *   Ties       Every argmax over a vocabulary goes to the smallest target id.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_ABI_VERSION 6

typedef enum dspark_status {
  DSPARK_OK = 0,
  DSPARK_ERR_INVALID = 1,      /* null/misaligned pointer, bad size or flag          */
  DSPARK_ERR_UNSUPPORTED = 2,  /* valid request beyond this build's limits           */
  DSPARK_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the size query   */
  DSPARK_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed         */
} dspark_status;

enum { DSPARK_INPUT_LOGITS = 0, DSPARK_INPUT_PROBS = 1 };

/* Limits of this build (DSPARK_ERR_UNSUPPORTED beyond them). */
#define DSPARK_MAX_N 64          /* draft positions per request                      */
#define DSPARK_MAX_RANK 256      /* Markov rank r                                    */
#define DSPARK_MAX_B 65535       /* requests                                          */
#define DSPARK_MAX_ADMIT 16384   /* B * N of one admission call                       */

/* ABI version of the loaded library (== DSPARK_ABI_VERSION of its header). */
int dspark_abi_version(void);

/* Message of the last failed call on this host thread ("" if none).  Host memory
 * owned by the library, valid until the next call on the same thread. */
const char* dspark_last_error(void);

/* ---------------------------------------------------------------- random numbers
 * Raw Philox4x32-10 blocks, for checking the generator bit for bit.
 *   counters  [n, 4] uint32, device, 16-byte aligned: (c0, c1, c2, c3) per block
 *   seed      64-bit key (low word = key0)
 *   out       [n, 4] uint32, device, 16-byte aligned: the four output words
 *   n         number of blocks, >= 0 (0 enqueues nothing)
 */
dspark_status dspark_philox_blocks(const uint32_t* counters, uint64_t seed, uint32_t* out,
                                   int64_t n, void* stream);

/* Exponential variates of the stage-3 race: out[v] = -plog2(u(seed, v, position,
 * request_id, tag)) for v < n, where plog2 is the portable float32 log2 (IEEE
 * add/multiply/divide only: u = m * 2^e with m in [sqrt2/2, sqrt2), s = (m-1)/(m+1),
 * log2 u = e + s * (c1 + z(c3 + z(c5 + z(c7 + z c9)))), z = s*s, c_k = fp32(2/(k ln 2))).
 *   out  [n] float32, device.  n >= 0. */
dspark_status dspark_race_exponentials(uint64_t seed, uint32_t position, uint32_t request_id,
                                       uint32_t tag, float* out, int64_t n, void* stream);

/* ---------------------------------------------------------------- stage 1
 * Draft base logits for every draft position at once [P1 §2.2 (compute_draft_logits),
 * §4 step 2]:  logits[m, j] = sum_h hidden[m, h] * lm_head[j, h]   (fp32 accumulation).
 *   hidden   [M, H] bf16 bits, row m = b*N + i (backbone hidden state of position i
 *            of request b), device, 16-byte aligned
 *   lm_head  [Vd, H] bf16 bits, one row per draft token (the Hugging Face lm_head
 *            layout), device, 16-byte aligned
 *   logits   [M, Vd] float32, device
 *   M >= 0 (0 enqueues nothing), H > 0 with H % 8 == 0, Vd > 0.
 */
dspark_status dspark_draft_logits(const uint16_t* hidden, const uint16_t* lm_head, float* logits,
                                  int M, int H, int Vd, void* stream);

/* ---------------------------------------------------------------- stage 2
 * Sequential low-rank Markov sampling [P1 §2.2 (_sample_sequential), §3
 * (DSparkMarkovHead), §5 (reduced vocabulary); P2 §4].  For request b, with
 * prev = anchor[b], for i = 0 .. N-1:
 *     e      = w1[prev, :]                         (r values)
 *     bias_j = sum_k w2[j, k] * e_k                (j < Vd)
 *     l_j    = logits[b, i, j] + bias_j            (written back in place, fp32)
 *     x      = t(argmax_j key_j),   t(j) = j + d2t[j]  (t(j) = j without d2t)
 *              key_j = l_j / T_b + Gumbel(u(seed, j, i, request_id[b], 0))   (T_b > 0)
 *              key_j = l_j                                                    (T_b == 0)
 *     draft_tokens[b, i] = x;   log_z[b, i] = log sum_j exp(l_j / T_b)  (T_b == 0: max_j l_j)
 *     prev = x
 *   logits       [B, N, Vd] float32, device, 16-byte aligned.  In: base logits (stage 1
 *                output).  Out: processed logits l (untempered), what verify reads.
 *   w1           [V, r] bf16 bits, device, 16-byte aligned: markov_w1, indexed by target id
 *   w2           [Vd, r] bf16 bits, device, 16-byte aligned: markov_w2, one row per draft token
 *   d2t          [Vd] int64 offsets (target id = j + d2t[j]), device, or NULL iff Vd == V.
 *                Must map [0, Vd) injectively into [0, V) (not checked on the device).
 *   anchor       [B] int32 target ids in [0, V), device
 *   temperature  [B] float32 >= 0, device
 *   request_id   [B] uint32, device (Philox counter word 2)
 *   draft_tokens [B, N] int32 out, device (target ids)
 *   log_z        [B, N] float32 out, device
 *   1 <= B <= DSPARK_MAX_B, 1 <= N <= DSPARK_MAX_N, V % 4 == 0, Vd % 4 == 0, Vd <= V,
 *   8 <= r <= DSPARK_MAX_RANK with r % 8 == 0.
 *   workspace    >= dspark_markov_workspace_size(B, N, Vd, r) bytes, device, 16-byte aligned.
 */
size_t dspark_markov_workspace_size(int B, int N, int Vd, int r);
dspark_status dspark_markov_sample(float* logits, const uint16_t* w1, const uint16_t* w2,
                                   const int64_t* d2t, const int32_t* anchor,
                                   const float* temperature, const uint32_t* request_id,
                                   uint64_t seed, int32_t* draft_tokens, float* log_z,
                                   int B, int N, int V, int Vd, int r,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Give-up check of the few-request kernel (B <= 16).  That kernel synchronises its
 * workgroups with grid barriers whose waits are bounded (about 0.1 s), so a launch
 * whose workgroups cannot all become resident never hangs the device.  A wait that
 * runs out sets a sticky per-device error word; the launch then stops consuming
 * data of other workgroups and writes draft_tokens = -1 and log_z = NaN for every
 * position, as does every later launch until the word is cleared.
 * dspark_markov_check synchronises `stream`, reads the word, and if it is set
 * clears it (and the library's barrier counters) and returns DSPARK_ERR_HIP with a
 * message; otherwise DSPARK_OK.  It is the one call that waits and reads device
 * memory on the host. */
dspark_status dspark_markov_check(void* stream);

/* Test hooks of the few-request kernel (process-wide; not for production use):
 *   0 normal; 1 every vocabulary slice is run by a single workgroup (the fallback
 *   when not every workgroup becomes resident); 2 every grid barrier reports a
 *   give-up after it has completed (exercises the error path without ever reading
 *   data that was not published).  Other values: DSPARK_ERR_INVALID. */
dspark_status dspark_markov_test_mode(int mode);

/* Inverse of the reduced-vocabulary map [P3 §3.2 (d2t)]: inv_map[v] = j if
 * v == j + d2t[j], else -1.
 *   d2t [Vd] int64, device (injective into [0, V), not checked on the device);
 *   inv_map [V] int32 out, device.  0 < Vd <= V. */
dspark_status dspark_build_inverse_map(const int64_t* d2t, int Vd, int V, int32_t* inv_map,
                                       void* stream);

/* ---------------------------------------------------------------- stage 3
 * Lossless rejection-sampling verification [P2 §2; greedy case P3 §2].  Request b
 * with L = verify_len[b] (N when verify_len is NULL), x_k = draft_tokens[b, k]:
 *   for k < L: u_k = u(seed, 0, k, request_id[b], 1); accept x_k iff
 *              (double)u_k * p_d[k](x_k) < (double)p_t[k](x_k);
 *   first rejection at k:  y = race sample (tag 2, position k) of
 *              r_v = max(0, p_t[k](v) - p_d[k](v))  (float32 subtraction);
 *              if every r_v == 0, of p_t[k] itself (same uniforms);
 *   all L accepted:        y = race sample (tag 3, position L) of p_t[L].
 *   Race sample of weights r: argmax_v r_v / E_v with E_v the variates of
 *   dspark_race_exponentials, compared exactly as r_a*E_b vs r_b*E_a in double,
 *   ties to the smaller v.
 *   Outputs: accepted[b] = number of accepted draft tokens a;
 *            out_tokens[b, :] = x_0 .. x_{a-1}, y, then -1 up to column N;
 *            accept_prob[b, k] (optional) = sum_v min(p_t[k](v), p_d[k](v)), the
 *            probability that position k is accepted, i.e. one minus the total
 *            variation distance [P2 §2], for k < L; NaN for k >= L (those target
 *            rows are not read).  It costs one extra pass over rows k < L of both
 *            sides; NULL skips it.
 * input_kind DSPARK_INPUT_PROBS: target = p_t [B, N+1, V] float32 probabilities,
 *            draft = p_d [B, N, Vd] float32 probabilities; draft_log_z and
 *            temperature are ignored (may be NULL).  Given the same float32 arrays
 *            the result is bit-identical to the rule above.
 * input_kind DSPARK_INPUT_LOGITS: target = target logits [B, N+1, V] float32,
 *            draft = processed draft logits [B, N, Vd] (stage 2 output), draft_log_z
 *            = stage 2's log_z [B, N] (required); p_t = softmax(target / T),
 *            p_d(j) = exp(draft_j / T - log_z), both evaluated in float32 on the GPU.
 *            T == 0: p_t is the point mass on the target row's argmax and p_d the
 *            point mass on x_k (no randomness is used).
 *   target, draft  device, 16-byte aligned.  Only rows k <= L of the target and the
 *            entries needed of draft rows k < L are read.
 *   draft_tokens [B, N] int32 target ids, device.
 *   inv_map  [V] int32 (dspark_build_inverse_map), device; NULL iff Vd == V.
 *   verify_len [B] int32 in [0, N], device, or NULL (= N); dspark_admit's admit_len fits.
 *   temperature [B] float32 >= 0 (logits mode), request_id [B] uint32, device.
 *   accepted [B] int32 out; out_tokens [B, N+1] int32 out; accept_prob [B, N] float32
 *            out or NULL; device.
 *   1 <= B <= DSPARK_MAX_B, 1 <= N <= DSPARK_MAX_N, V % 4 == 0, Vd % 4 == 0, Vd <= V.
 *   workspace >= dspark_verify_workspace_size(B, N, V) bytes, device, 16-byte aligned.
 */
size_t dspark_verify_workspace_size(int B, int N, int V);
dspark_status dspark_verify(int input_kind, const float* target, const float* draft,
                            const float* draft_log_z, const int32_t* draft_tokens,
                            const int32_t* inv_map, const int32_t* verify_len,
                            const float* temperature, const uint32_t* request_id, uint64_t seed,
                            int32_t* accepted, int32_t* out_tokens, float* accept_prob,
                            int B, int N, int V, int Vd,
                            void* workspace, size_t workspace_bytes, void* stream);

/* dspark_verify without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments (minus workspace), checks, kernels and results as
 * dspark_verify.  The scratch is a static device array of the library,
 * dspark_verify_noalloc_max_bytes() bytes (4 MiB) per device, held until the process
 * ends; a shape whose dspark_verify_workspace_size(B, N, V) exceeds it returns
 * DSPARK_ERR_UNSUPPORTED and enqueues nothing.  The call allocates nothing.  Every
 * call on one device shares that device's array, so two calls that overlap on one
 * device (two streams, or two host threads) race and give undefined results; calls
 * on different devices do not interact. */
size_t dspark_verify_noalloc_max_bytes(void);
dspark_status dspark_verify_noalloc(int input_kind, const float* target, const float* draft,
                                    const float* draft_log_z, const int32_t* draft_tokens,
                                    const int32_t* inv_map, const int32_t* verify_len,
                                    const float* temperature, const uint32_t* request_id, uint64_t seed,
                                    int32_t* accepted, int32_t* out_tokens, float* accept_prob,
                                    int B, int N, int V, int Vd, void* stream);

/* ---------------------------------------------------------------- stage 3, coupled
 * Gumbel-coupled verification [P1 §5: the target verifies with the same Gumbel seed
 * the draft sampled with, so the output distribution is unchanged].  No draft
 * probabilities are used; the draft tokens must come from dspark_markov_sample with
 * the same seed and request ids.  Request b with L = verify_len[b] (N when NULL):
 *   row k <= L:  y_k = argmax_v l_t[k](v) / T + G_k(v) (T == 0: argmax l_t[k]),
 *                ties to the smaller v, where G_k(v) is the Gumbel variate stage 2
 *                drew for the draft entry j that is target id v (u(seed, j, k,
 *                request_id[b], 0)), and u(seed, v, k, request_id[b], 4) for an id
 *                outside the draft vocabulary;
 *   a = the first k < L with y_k != x_k, else L;
 *   accepted[b] = a; out_tokens[b, :] = x_0 .. x_{a-1}, y_a, then -1 up to column N.
 * Every emitted token is a Gumbel-max draw from softmax(l_t / T).  Keys are formed
 * in float32 in base-2 units, as stage 2 forms them (the same argmax up to rounding).
 *   target_logits [B, N+1, V] float32, device, 16-byte aligned; rows k <= L are read.
 *   draft_tokens [B, N] int32 target ids; inv_map [V] int32 (16-byte aligned),
 *            NULL iff Vd == V; verify_len [B] int32 in [0, N] or NULL;
 *   temperature [B] float32 >= 0; request_id [B] uint32; accepted [B] int32 out;
 *   out_tokens [B, N+1] int32 out; all device.
 *   1 <= B <= DSPARK_MAX_B, 1 <= N <= DSPARK_MAX_N, V % 4 == 0, 1 <= Vd <= V.
 *   workspace >= dspark_verify_coupled_workspace_size(B, N, V) bytes, device, 16-byte aligned.
 */
size_t dspark_verify_coupled_workspace_size(int B, int N, int V);
dspark_status dspark_verify_coupled(const float* target_logits, const int32_t* draft_tokens,
                                    const int32_t* inv_map, const int32_t* verify_len,
                                    const float* temperature, const uint32_t* request_id,
                                    uint64_t seed, int32_t* accepted, int32_t* out_tokens,
                                    int B, int N, int V, int Vd,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- stage 4
 * Confidence-scheduled admission [P2 §6 (chain rule, pooled greedy sort), §7 (K fixed
 * ahead, sort at the last moment, non-anticipation)]:
 *   survival[b, 0] = c[b, 0];  survival[b, k] = survival[b, k-1] * c[b, k]  (float32);
 *   all B*N (b, k) ordered by survival descending, then k ascending, then b ascending;
 *   the first min(K, B*N) admitted; admit_len[b] = admitted positions of request b.
 *   With c in [0, 1] every request's admitted set is a prefix, and whether (b, k) is
 *   admitted never depends on c[b, j > k].
 *   cond_accept [B, N] float32 in [0, 1], device; survival [B, N] float32 out, device;
 *   admit_len [B] int32 out, device.  1 <= B, 1 <= N <= DSPARK_MAX_N,
 *   B * N <= DSPARK_MAX_ADMIT, K >= 0.  Runs as one workgroup; no workspace.
 */
dspark_status dspark_admit(const float* cond_accept, int B, int N, int K, float* survival,
                           int32_t* admit_len, void* stream);

/* ---------------------------------------------------------------- confidence head, fused
 * Conditional acceptance probability of each draft position [P2 §6: a linear
 * projection of the backbone hidden state plus the Markov embedding, calibrated by
 * temperature scaling per position]:
 *   c[b, k] = 1 / (1 + exp(-(w_h . h[b*N + k] + w_e . W1[x_{k-1}] + conf_bias) / tau[k]))
 * with x_{-1} = anchor[b] (the token stage 2 starts from); its output is
 * dspark_admit's cond_accept.  It runs inside the two stages that already read its
 * inputs, with no launch of its own:
 *   dspark_draft_logits_conf   stage 1 with w_h as one more LM-head row: logits as
 *              dspark_draft_logits, plus h_dot[m] = w_h . hidden[m] (fp32 accumulation).
 *              w_h [H] bf16, device, 16-byte aligned; h_dot [M] float32 out, device.
 *   dspark_markov_sample_conf  stage 2 as dspark_markov_sample, plus c_out [B, N]:
 *              each step forms w_e . W1[previous token] from the W1 row it gathers.
 *              h_dot [B*N] float32 (from dspark_draft_logits_conf), w_e [r] bf16
 *              (16-byte aligned), conf_bias finite, tau [N] float32 > 0, c_out [B, N]
 *              float32 out; all device.  On a barrier give-up (dspark_markov_check)
 *              c_out is NaN like log_z.
 * Float32 arithmetic.  Other arguments, limits and errors as the plain calls. */
dspark_status dspark_draft_logits_conf(const uint16_t* hidden, const uint16_t* lm_head, const uint16_t* w_h,
                                       float* logits, float* h_dot, int M, int H, int Vd, void* stream);
dspark_status dspark_markov_sample_conf(float* logits, const uint16_t* w1, const uint16_t* w2,
                                        const int64_t* d2t, const int32_t* anchor,
                                        const float* temperature, const uint32_t* request_id,
                                        uint64_t seed, int32_t* draft_tokens, float* log_z,
                                        const float* h_dot, const uint16_t* w_e, float conf_bias,
                                        const float* tau, float* c_out,
                                        int B, int N, int V, int Vd, int r,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- deferred draft rows
 * Stages 2 and 3 without storing the processed draft logits of every position.  The
 * verification rule above [P2 §2] reads, per request, p_d of the drafted token at each
 * verified position and one whole processed draft row: the residual at the first
 * rejection (none when every position is accepted, or at T == 0).  The other N - 1
 * rows stage 2 would store are never read.
 *   dspark_markov_sample_deferred  stage 2 as dspark_markov_sample_conf (the five
 *              confidence arguments h_dot, w_e, tau, c_out all given or all NULL:
 *              no confidence, conf_bias ignored), except that logits keeps the base
 *              logits (nothing is written to it) and win_logit [B, N] float32 (device,
 *              out) receives l at each drafted token: win_logit[b, i] is the value
 *              dspark_markov_sample would have stored at logits[b, i, draft_tokens[b, i]].
 *              No target map: Vd == V (else DSPARK_ERR_UNSUPPORTED).  Always the
 *              per-step kernels (never the few-request kernel); the workspace is
 *              dspark_markov_workspace_size(B, N, Vd, r).
 *   dspark_verify_deferred  dspark_verify in logits mode on those outputs: draft_base
 *              [B, N, V] float32 = the base logits stage 2 kept (device, 16-byte
 *              aligned), draft_log_z, win_logit and draft_tokens from stage 2, anchor
 *              [B] and w1, w2, r as given to stage 2.  p_d of the drafted token at k is
 *              taken from win_logit; the processed row of each request's first
 *              rejection is recomputed in place in draft_base, with the same chunks,
 *              fragments and MFMA sequence as stage 2, so it equals what stage 2 would
 *              have stored bit for bit; every other row of draft_base is left as it
 *              is.  accepted and out_tokens then equal dspark_verify's on the processed
 *              logits bit for bit.  No inverse map, no acceptance probabilities.
 *              workspace >= dspark_verify_deferred_workspace_size(B, N, V) bytes.
 * Other arguments, limits and errors as dspark_markov_sample_conf / dspark_verify. */
dspark_status dspark_markov_sample_deferred(float* logits, const uint16_t* w1, const uint16_t* w2,
                                            const int32_t* anchor, const float* temperature,
                                            const uint32_t* request_id, uint64_t seed,
                                            int32_t* draft_tokens, float* log_z, float* win_logit,
                                            const float* h_dot, const uint16_t* w_e, float conf_bias,
                                            const float* tau, float* c_out,
                                            int B, int N, int V, int Vd, int r,
                                            void* workspace, size_t workspace_bytes, void* stream);
size_t dspark_verify_deferred_workspace_size(int B, int N, int V);
dspark_status dspark_verify_deferred(const float* target, float* draft_base, const float* draft_log_z,
                                     const float* win_logit, const int32_t* draft_tokens,
                                     const int32_t* anchor, const uint16_t* w1, const uint16_t* w2, int r,
                                     const int32_t* verify_len, const float* temperature,
                                     const uint32_t* request_id, uint64_t seed,
                                     int32_t* accepted, int32_t* out_tokens, int B, int N, int V,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- context-KV precompute
 * The draft KV cache of M = num_ctx new context tokens, filled from the target's
 * intermediate hidden states in one pass instead of a layer-by-layer target forward
 * [P1 §4 (Context KV 预计算); P2 §3 (KV injection)]:
 *   ctx    = aux . fc_w^T + fc_b                       [M, H_d]   (fc_b may be NULL)
 *   normed = bf16(ctx / sqrt(mean_j ctx_j^2 + eps) * hnorm_w)      the fused GEMM's operand
 *   all_kv = normed . kv_w^T + kv_b                    [M, L*2*nkv*hd], rows of kv_w
 *            ordered (layer, K/V, head, dim), one GEMM for every layer
 *   for every layer l and head h, token m at slot s = slots[m]:
 *     k = all_kv[m, l, 0, h, :] / sqrt(mean k^2 + eps) * knorm_w[l, :]    (grouped RMSNorm)
 *     k = rotate-half RoPE: for i < hd/2 the pair (k_i, k_{i+hd/2}) rotated by
 *         angle positions[m] * rope_theta^(-2i/hd)                          (fused RoPE)
 *     k_cache[l, s, h, :] = bf16(k);   v_cache[l, s, h, :] = bf16(all_kv[m, l, 1, h, :])
 *   aux [M, H_in], fc_w [H_d, H_in], fc_b [H_d] or NULL, hnorm_w [H_d], kv_w
 *   [L*2*nkv*hd, H_d], kv_b [L*2*nkv*hd], knorm_w [L, hd]: bf16 bits, device, each
 *   16-byte aligned.  positions [M] int32, slots [M] int64, device; a slot outside
 *   [0, num_slots) is skipped (nothing written for that token).  k_cache, v_cache
 *   [L, num_slots, nkv, hd] bf16 bits, device, 16-byte aligned, written in place
 *   (other slots untouched).
 *   Products accumulate in float32 on MFMA (the draft-logit kernels), norms and RoPE in
 *   float32 with the angles formed in double.  H_in % 8 == 0, H_d % 8 == 0, hd even,
 *   2 <= hd <= 256, eps >= 0, rope_theta > 0; num_ctx == 0 enqueues nothing.
 *   workspace >= dspark_context_kv_workspace_size(num_ctx, H_d, L, nkv, hd) bytes,
 *   device, 16-byte aligned. */
size_t dspark_context_kv_workspace_size(int num_ctx, int H_d, int L, int nkv, int hd);
dspark_status dspark_context_kv(const uint16_t* aux, const uint16_t* fc_w, const uint16_t* fc_b,
                                const uint16_t* hnorm_w, const uint16_t* kv_w, const uint16_t* kv_b,
                                const uint16_t* knorm_w, const int32_t* positions, const int64_t* slots,
                                uint16_t* k_cache, uint16_t* v_cache, int num_ctx, int H_in, int H_d,
                                int L, int nkv, int hd, int64_t num_slots, float eps, float rope_theta,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- end of a round
 * The next round's anchors ["DSpark 的实现和测评" §2.1: the anchor of a request is the
 * token its previous step verified]: anchor[b] = out_tokens[b, accepted[b]], the
 * correction or bonus token dspark_verify / dspark_verify_coupled emitted last, and,
 * when emitted is not NULL, emitted[b] += accepted[b] + 1 (tokens emitted this round),
 * for a multi-round driver that measures tokens per round.
 *   accepted [B] int32 in [0, N] (clamped), out_tokens [B, N+1] int32, anchor [B]
 *   int32 out, emitted [B] int64 in/out or NULL; device.  1 <= B <= DSPARK_MAX_B,
 *   1 <= N <= DSPARK_MAX_N. */
dspark_status dspark_advance(const int32_t* accepted, const int32_t* out_tokens, int32_t* anchor,
                             int64_t* emitted, int B, int N, void* stream);

/* ---------------------------------------------------------------- verification budget
 * Throughput-optimal budget K [P2 §6 (maximise expected tokens per batch times SPS at
 * that batch size; pool all requests' candidates, admit by survival), §7 (the SPS
 * curve is jagged: scan every K; K is fixed from earlier scores)]:
 *   objective(K) = (B + S_K) * sps[B + K], S_K = sum of the K largest survival values
 *   (fp64), for K = 0 .. min(B*N, S-1-B); *k_out = the smallest K with the largest
 *   objective, *objective_out = that objective (optional).
 * Readings: a batch holds B + K tokens (each request's current position plus its
 * admitted drafts) and yields B + S_K tokens in expectation.  The prefix sums are
 * taken in a parallel order, so K can differ from a sequential sum only where two
 * objectives agree to about 1e-15 relative.
 *   survival [B, N] float32 (dspark_admit's output of an earlier round), device;
 *   sps [S] float32 steps per second at a batch of n tokens, n = 0 .. S-1, device;
 *   k_out [1] int32, objective_out [1] double or NULL, device.
 *   B * N <= DSPARK_MAX_ADMIT, S >= B + 1.
 */
dspark_status dspark_choose_k(const float* survival, int B, int N, const float* sps, int S,
                              int32_t* k_out, double* objective_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
