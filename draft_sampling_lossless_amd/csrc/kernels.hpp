// Host-side launchers of the DSpark kernels (called by the C ABI layer after it
// has validated every argument).  Each enqueues on `stream` and returns the
// launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// ---- random numbers
hipError_t launch_philox_blocks(const uint32_t* counters, uint64_t seed, uint32_t* out, int64_t n,
                                hipStream_t stream);
hipError_t launch_race_exponentials(uint64_t seed, uint32_t position, uint32_t request_id, uint32_t tag,
                                    float* out, int64_t n, hipStream_t stream);

// ---- stage 1
// wx (optional, [H] bf16): one more LM-head row; its output column goes to xout [M]
hipError_t launch_draft_logits(const uint16_t* hidden, const uint16_t* lm_head, float* logits, int M, int H,
                               int Vd, const uint16_t* wx, float* xout, hipStream_t stream);

// ---- stage 2
// Confidence head fused into the Markov loop (all null/unused when out == nullptr):
// c[b, k] = sigmoid((hdot[b*N + k] + we . W1[x_{k-1}] + bias) / tau[k]), x_{-1} = anchor
struct ConfArgs {
  const float* hdot = nullptr;    // [B*N] w_h . hidden (the draft-logit product's extra column)
  const uint16_t* we = nullptr;   // [r] bf16
  float bias = 0.0f;
  const float* tau = nullptr;     // [N]
  float* out = nullptr;           // [B, N]
};

// Few requests: one cooperative launch (markov_few.hip).
struct FewPlan {
  bool use;            // B <= 16 and the per-workgroup W2 slice fits in LDS
  int grid, ch;        // workgroups (at most one per CU), 64-wide vocabulary chunks per workgroup
  int cap;             // survivors per step whose weight rows phase C can hold in LDS
  size_t lds;          // dynamic LDS bytes
  int gmax;            // workgroup count the workspace layout is sized for
  size_t off_norms, off_n1, off_rec, off_fstep, off_partF, off_partD, off_rows, bytes;
};
FewPlan plan_markov_few(int B, int N, int Vd, int r, int cus);
hipError_t launch_markov_few(const FewPlan& p, float* logits, const uint16_t* w1, const uint16_t* w2,
                             const int64_t* d2t, const int32_t* anchor, const float* temperature,
                             const uint32_t* request_id, uint64_t seed, int32_t* draft_tokens, float* log_z, int B,
                             int N, int V, int Vd, int r, void* workspace, const ConfArgs& conf, hipStream_t stream);

struct MarkovPlan {
  int chunks_per_wg;   // 64-wide vocabulary chunks per workgroup, at most (per-step path)
  int vslices;         // workgroups per request tile; workgroup v takes chunks v, v + vslices, ...
  int btiles;          // 64-request tiles
  size_t tgt_offset;   // workspace offset of the int32 target-id table (reduced vocabulary)
  size_t spill_offset; // workspace offset of the spill row (stores of entries that do not exist)
  size_t lw_offset;    // workspace offset of the partials' winner logits (kept base logits)
  size_t partial_bytes;  // workspace bytes (the larger need of the two paths)
  FewPlan few;
};
// cus: compute units of the device (0: upper bound for workspace sizing, no HIP calls)
MarkovPlan plan_markov(int B, int N, int Vd, int r, int cus);
hipError_t launch_markov_sample(float* logits, const uint16_t* w1, const uint16_t* w2, const int64_t* d2t,
                                const int32_t* anchor, const float* temperature, const uint32_t* request_id,
                                uint64_t seed, int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd,
                                int r, void* workspace, const ConfArgs& conf, float* win, hipStream_t stream);
// processed logits of one row per request (rows[b], -1: none), recomputed in place from
// the base logits there with the previous token prev[b], exactly as the sampling pass
// forms them; spill: markov_replay_spill_bytes(Vd) bytes of scratch
size_t markov_replay_spill_bytes(int Vd);
hipError_t launch_markov_replay(float* logits, const uint16_t* w1, const uint16_t* w2, const int32_t* rows,
                                const int32_t* prev, const float* temperature, const uint32_t* request_id, int B,
                                int N, int V, int Vd, int r, float* spill, hipStream_t stream);
// few-request kernel: test hooks (0 normal, 1 single workgroup, 2 forced barrier give-up)
// and the host-side check of the device's sticky give-up word (synchronises `stream`;
// on a give-up also resets the counter sets)
void set_markov_test_mode(int mode);
hipError_t markov_check(hipStream_t stream, bool* gave_up);
hipError_t launch_build_inverse_map(const int64_t* d2t, int Vd, int V, int32_t* inv_map, hipStream_t stream);

// ---- stage 3
struct VerifyPlan {
  int stat_chunks;     // chunks per target row in the row-statistics pass
  int stat_chunk;      // elements per chunk (multiple of 4)
  int sample_chunks;   // chunks per sampling row
  int sample_chunk;
  size_t stats_bytes, jobs_bytes, race_bytes, total_bytes;
};
VerifyPlan plan_verify(int B, int N, int V);
hipError_t launch_verify(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                         const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                         const float* temperature, const uint32_t* request_id, uint64_t seed, int32_t* accepted,
                         int32_t* out_tokens, float* accept_prob, int B, int N, int V, int Vd, void* workspace,
                         hipStream_t stream);
// Logits mode on kept base logits (stage 2 run with win != nullptr): p_d of each drafted
// token comes from win, and the processed row of each request's first rejection is
// recomputed in place in draft_base before the sampling pass reads it.  No inverse map
// (Vd == V), no acceptance probabilities.  workspace: plan_verify(B, N, V).total_bytes
// + verify_deferred_extra_bytes(B, V).
struct DeferredArgs {
  const float* win = nullptr;       // [B, N] processed logit of each drafted token
  const int32_t* anchor = nullptr;  // [B] token before position 0
  const uint16_t* w1 = nullptr;     // [V, r] bf16
  const uint16_t* w2 = nullptr;     // [Vd, r] bf16
  int r = 0;
};
size_t verify_deferred_extra_bytes(int B, int V);
hipError_t launch_verify_deferred(const float* target, float* draft_base, const float* draft_log_z,
                                  const int32_t* draft_tokens, const int32_t* verify_len, const float* temperature,
                                  const uint32_t* request_id, uint64_t seed, int32_t* accepted, int32_t* out_tokens,
                                  int B, int N, int V, const DeferredArgs& d, void* workspace, hipStream_t stream);
// ---- context-KV precompute (the step before the path)
// The fused K/V product's epilogue: per output row (token) and 128-wide head block, the
// bias, then for K blocks the RMSNorm over the head and rotate-half RoPE, then bf16 into
// the caches at the token's slot.  Column n of the product is (layer, K/V, head, dim)
// with head blocks of 128.
struct KvEpilogue {
  const uint16_t* kv_b = nullptr;     // [L*2*nkv*128] bf16
  const uint16_t* knorm_w = nullptr;  // [L, 128] bf16
  const float* rope = nullptr;        // [M, 128]: cos of the 64 angles, then their sin
  const int64_t* slots = nullptr;     // [M]; a slot outside [0, num_slots) is skipped
  uint16_t* kc = nullptr;             // [L, num_slots, nkv, 128] bf16
  uint16_t* vc = nullptr;
  int nkv = 0;
  int64_t num_slots = 0;
  float eps = 0.0f;
};
// whether the K/V product of M tokens over H_d runs with the fused epilogue (head size 128,
// the 256 x 256 tiling)
bool kv_product_fused(int M, int Hd, int hd);
hipError_t launch_kv_product(const uint16_t* normed, const uint16_t* kv_w, int M, int Hd, int ncols,
                             const KvEpilogue& ep, hipStream_t stream);
size_t context_kv_workspace_bytes(int M, int Hd, int L, int nkv, int hd);
hipError_t launch_context_kv(const uint16_t* aux, const uint16_t* fc_w, const uint16_t* fc_b, const uint16_t* hnorm_w,
                             const uint16_t* kv_w, const uint16_t* kv_b, const uint16_t* knorm_w,
                             const int32_t* positions, const int64_t* slots, uint16_t* k_cache, uint16_t* v_cache,
                             int M, int H_in, int Hd, int L, int nkv, int hd, int64_t num_slots, float eps,
                             float theta, void* workspace, hipStream_t stream);
// launch_verify with the library's static per-device scratch array as workspace
constexpr size_t kVerifyScratchBytes = (size_t)4 << 20;
hipError_t launch_verify_noalloc(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                                 const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                                 const float* temperature, const uint32_t* request_id, uint64_t seed,
                                 int32_t* accepted, int32_t* out_tokens, float* accept_prob, int B, int N, int V,
                                 int Vd, hipStream_t stream);

// ---- Gumbel-coupled verification
size_t coupled_workspace_bytes(int B, int N, int V);
hipError_t launch_verify_coupled(const float* target, const int32_t* draft_tokens, const int32_t* inv_map,
                                 const int32_t* verify_len, const float* temperature, const uint32_t* request_id,
                                 uint64_t seed, int32_t* accepted, int32_t* out_tokens, int B, int N, int V,
                                 void* workspace, hipStream_t stream);

// ---- end of a round: next anchors, emitted-token counts
hipError_t launch_advance(const int32_t* accepted, const int32_t* out_tokens, int32_t* anchor, int64_t* emitted,
                          int B, int N, hipStream_t stream);

// ---- verification budget
hipError_t launch_choose_k(const float* survival, int B, int N, const float* sps, int S, int32_t* k_out,
                           double* obj_out, hipStream_t stream);

// ---- stage 4
hipError_t launch_admit(const float* cond_accept, int B, int N, int K, float* survival, int32_t* admit_len,
                        hipStream_t stream);

}  // namespace dspark
