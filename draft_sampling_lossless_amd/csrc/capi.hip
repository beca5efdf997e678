// C ABI of the DSpark hot path: argument validation on the host, then the
// kernel launchers.  Nothing here allocates, frees or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "dspark.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512];

dspark_status fail(dspark_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

dspark_status ok() {
  g_err[0] = '\0';
  return DSPARK_OK;
}

dspark_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSPARK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, st, ...)            \
  do {                                    \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p, name)                                                          \
  do {                                                                                \
    if (!(p)) return fail(DSPARK_ERR_INVALID, "%s must not be NULL", name);          \
  } while (0)

#define REQUIRE_PTR16(p, name)                                                               \
  do {                                                                                       \
    if (!(p)) return fail(DSPARK_ERR_INVALID, "%s must not be NULL", name);                 \
    if (!aligned16(p)) return fail(DSPARK_ERR_INVALID, "%s must be 16-byte aligned", name); \
  } while (0)

}  // namespace

extern "C" {

int dspark_abi_version(void) { return DSPARK_ABI_VERSION; }

const char* dspark_last_error(void) { return g_err; }

dspark_status dspark_philox_blocks(const uint32_t* counters, uint64_t seed, uint32_t* out, int64_t n,
                                   void* stream) {
  REQUIRE(n >= 0, DSPARK_ERR_INVALID, "n must be >= 0 (got %lld)", (long long)n);
  if (n == 0) return ok();
  REQUIRE(n <= ((int64_t)1 << 38), DSPARK_ERR_UNSUPPORTED, "n too large");
  REQUIRE_PTR16(counters, "counters");
  REQUIRE_PTR16(out, "out");
  return hip_status(dspark::launch_philox_blocks(counters, seed, out, n, (hipStream_t)stream), "philox_blocks");
}

dspark_status dspark_race_exponentials(uint64_t seed, uint32_t position, uint32_t request_id, uint32_t tag,
                                       float* out, int64_t n, void* stream) {
  REQUIRE(n >= 0, DSPARK_ERR_INVALID, "n must be >= 0 (got %lld)", (long long)n);
  if (n == 0) return ok();
  REQUIRE(n <= ((int64_t)1 << 38), DSPARK_ERR_UNSUPPORTED, "n too large");
  REQUIRE_PTR(out, "out");
  return hip_status(dspark::launch_race_exponentials(seed, position, request_id, tag, out, n, (hipStream_t)stream),
                    "race_exponentials");
}

dspark_status dspark_draft_logits(const uint16_t* hidden, const uint16_t* lm_head, float* logits, int M, int H,
                                  int Vd, void* stream) {
  REQUIRE(M >= 0, DSPARK_ERR_INVALID, "M must be >= 0 (got %d)", M);
  REQUIRE(H > 0 && H % 8 == 0, DSPARK_ERR_INVALID, "H must be a positive multiple of 8 (got %d)", H);
  REQUIRE(Vd > 0, DSPARK_ERR_INVALID, "Vd must be > 0 (got %d)", Vd);
  if (M == 0) return ok();
  REQUIRE((int64_t)M * Vd < ((int64_t)1 << 40), DSPARK_ERR_UNSUPPORTED, "M * Vd too large");
  REQUIRE_PTR16(hidden, "hidden");
  REQUIRE_PTR16(lm_head, "lm_head");
  REQUIRE_PTR(logits, "logits");
  return hip_status(dspark::launch_draft_logits(hidden, lm_head, logits, M, H, Vd, nullptr, nullptr,
                                                (hipStream_t)stream),
                    "draft_logits");
}

dspark_status dspark_draft_logits_conf(const uint16_t* hidden, const uint16_t* lm_head, const uint16_t* w_h,
                                       float* logits, float* h_dot, int M, int H, int Vd, void* stream) {
  REQUIRE(M >= 0, DSPARK_ERR_INVALID, "M must be >= 0 (got %d)", M);
  REQUIRE(H > 0 && H % 8 == 0, DSPARK_ERR_INVALID, "H must be a positive multiple of 8 (got %d)", H);
  REQUIRE(Vd > 0, DSPARK_ERR_INVALID, "Vd must be > 0 (got %d)", Vd);
  if (M == 0) return ok();
  REQUIRE((int64_t)M * (Vd + 1) < ((int64_t)1 << 40), DSPARK_ERR_UNSUPPORTED, "M * Vd too large");
  REQUIRE_PTR16(hidden, "hidden");
  REQUIRE_PTR16(lm_head, "lm_head");
  REQUIRE_PTR16(w_h, "w_h");
  REQUIRE_PTR(logits, "logits");
  REQUIRE_PTR(h_dot, "h_dot");
  return hip_status(dspark::launch_draft_logits(hidden, lm_head, logits, M, H, Vd, w_h, h_dot, (hipStream_t)stream),
                    "draft_logits_conf");
}

size_t dspark_markov_workspace_size(int B, int N, int Vd, int r) {
  if (B <= 0 || N <= 0 || Vd <= 0 || r <= 0) return 0;
  return dspark::plan_markov(B, N, Vd, r, 0).partial_bytes;
}

}  // extern "C"

namespace {
dspark_status markov_checked(float* logits, const uint16_t* w1, const uint16_t* w2, const int64_t* d2t,
                             const int32_t* anchor, const float* temperature, const uint32_t* request_id,
                             uint64_t seed, int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd, int r,
                             void* workspace, size_t workspace_bytes, const dspark::ConfArgs& conf, float* win,
                             void* stream) {
  REQUIRE(B >= 1, DSPARK_ERR_INVALID, "B must be >= 1 (got %d)", B);
  REQUIRE(B <= DSPARK_MAX_B, DSPARK_ERR_UNSUPPORTED, "B must be <= %d (got %d)", DSPARK_MAX_B, B);
  REQUIRE(N >= 1, DSPARK_ERR_INVALID, "N must be >= 1 (got %d)", N);
  REQUIRE(N <= DSPARK_MAX_N, DSPARK_ERR_UNSUPPORTED, "N must be <= %d (got %d)", DSPARK_MAX_N, N);
  REQUIRE(V > 0 && V % 4 == 0, DSPARK_ERR_INVALID, "V must be a positive multiple of 4 (got %d)", V);
  REQUIRE(Vd > 0 && Vd % 4 == 0, DSPARK_ERR_INVALID, "Vd must be a positive multiple of 4 (got %d)", Vd);
  REQUIRE(Vd <= V, DSPARK_ERR_INVALID, "Vd (%d) must be <= V (%d)", Vd, V);
  REQUIRE(r >= 8 && r % 8 == 0, DSPARK_ERR_INVALID, "r must be a positive multiple of 8 (got %d)", r);
  REQUIRE(r <= DSPARK_MAX_RANK, DSPARK_ERR_UNSUPPORTED, "r must be <= %d (got %d)", DSPARK_MAX_RANK, r);
  REQUIRE((int64_t)B * N * Vd < ((int64_t)1 << 40), DSPARK_ERR_UNSUPPORTED, "B * N * Vd too large");
  REQUIRE_PTR16(logits, "logits");
  REQUIRE_PTR16(w1, "w1");
  REQUIRE_PTR16(w2, "w2");
  if (Vd != V) REQUIRE_PTR16(d2t, "d2t (required when Vd != V)");
  else if (d2t) REQUIRE(aligned16(d2t), DSPARK_ERR_INVALID, "d2t must be 16-byte aligned");
  REQUIRE_PTR(anchor, "anchor");
  REQUIRE_PTR(temperature, "temperature");
  REQUIRE_PTR(request_id, "request_id");
  REQUIRE_PTR(draft_tokens, "draft_tokens");
  REQUIRE_PTR(log_z, "log_z");
  const size_t need = dspark_markov_workspace_size(B, N, Vd, r);
  REQUIRE(workspace != nullptr, DSPARK_ERR_WORKSPACE, "workspace must not be NULL (%zu bytes needed)", need);
  REQUIRE(aligned16(workspace), DSPARK_ERR_INVALID, "workspace must be 16-byte aligned");
  REQUIRE(workspace_bytes >= need, DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
          need);
  return hip_status(dspark::launch_markov_sample(logits, w1, w2, d2t, anchor, temperature, request_id, seed,
                                                 draft_tokens, log_z, B, N, V, Vd, r, workspace, conf, win,
                                                 (hipStream_t)stream),
                    win ? "markov_sample_deferred" : conf.out ? "markov_sample_conf" : "markov_sample");
}
}  // namespace

extern "C" {

dspark_status dspark_markov_sample(float* logits, const uint16_t* w1, const uint16_t* w2, const int64_t* d2t,
                                   const int32_t* anchor, const float* temperature, const uint32_t* request_id,
                                   uint64_t seed, int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd,
                                   int r, void* workspace, size_t workspace_bytes, void* stream) {
  return markov_checked(logits, w1, w2, d2t, anchor, temperature, request_id, seed, draft_tokens, log_z, B, N, V, Vd,
                        r, workspace, workspace_bytes, dspark::ConfArgs{}, nullptr, stream);
}

dspark_status dspark_markov_sample_conf(float* logits, const uint16_t* w1, const uint16_t* w2, const int64_t* d2t,
                                        const int32_t* anchor, const float* temperature,
                                        const uint32_t* request_id, uint64_t seed, int32_t* draft_tokens,
                                        float* log_z, const float* h_dot, const uint16_t* w_e, float conf_bias,
                                        const float* tau, float* c_out, int B, int N, int V, int Vd, int r,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE_PTR(h_dot, "h_dot");
  REQUIRE_PTR16(w_e, "w_e");
  REQUIRE_PTR(tau, "tau");
  REQUIRE_PTR(c_out, "c_out");
  REQUIRE(std::isfinite(conf_bias), DSPARK_ERR_INVALID, "conf_bias must be finite");
  dspark::ConfArgs conf;
  conf.hdot = h_dot;
  conf.we = w_e;
  conf.bias = conf_bias;
  conf.tau = tau;
  conf.out = c_out;
  return markov_checked(logits, w1, w2, d2t, anchor, temperature, request_id, seed, draft_tokens, log_z, B, N, V, Vd,
                        r, workspace, workspace_bytes, conf, nullptr, stream);
}

dspark_status dspark_markov_sample_deferred(float* logits, const uint16_t* w1, const uint16_t* w2,
                                            const int32_t* anchor, const float* temperature,
                                            const uint32_t* request_id, uint64_t seed, int32_t* draft_tokens,
                                            float* log_z, float* win_logit, const float* h_dot, const uint16_t* w_e,
                                            float conf_bias, const float* tau, float* c_out, int B, int N, int V,
                                            int Vd, int r, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(Vd == V, DSPARK_ERR_UNSUPPORTED, "markov_sample_deferred: no target map (Vd must equal V; got Vd=%d, V=%d)",
          Vd, V);
  REQUIRE_PTR(win_logit, "win_logit");
  dspark::ConfArgs conf;
  const bool with_conf = h_dot || w_e || tau || c_out;
  if (with_conf) {
    REQUIRE_PTR(h_dot, "h_dot (the confidence arguments are all given or all NULL)");
    REQUIRE_PTR16(w_e, "w_e (the confidence arguments are all given or all NULL)");
    REQUIRE_PTR(tau, "tau (the confidence arguments are all given or all NULL)");
    REQUIRE_PTR(c_out, "c_out (the confidence arguments are all given or all NULL)");
    REQUIRE(std::isfinite(conf_bias), DSPARK_ERR_INVALID, "conf_bias must be finite");
    conf.hdot = h_dot;
    conf.we = w_e;
    conf.bias = conf_bias;
    conf.tau = tau;
    conf.out = c_out;
  }
  return markov_checked(logits, w1, w2, nullptr, anchor, temperature, request_id, seed, draft_tokens, log_z, B, N, V,
                        Vd, r, workspace, workspace_bytes, conf, win_logit, stream);
}

dspark_status dspark_markov_check(void* stream) {
  bool gave_up = false;
  const hipError_t e = dspark::markov_check((hipStream_t)stream, &gave_up);
  if (e != hipSuccess) return hip_status(e, "markov_check");
  if (gave_up)
    return fail(DSPARK_ERR_HIP,
                "markov_sample: a grid barrier of the few-request kernel gave up waiting (not every workgroup "
                "became resident); the draft tokens and log Z of the launches since the previous check are "
                "invalid (-1 / NaN)");
  return ok();
}

dspark_status dspark_markov_test_mode(int mode) {
  REQUIRE(mode >= 0 && mode <= 2, DSPARK_ERR_INVALID, "mode must be 0, 1 or 2 (got %d)", mode);
  dspark::set_markov_test_mode(mode);
  return ok();
}

dspark_status dspark_build_inverse_map(const int64_t* d2t, int Vd, int V, int32_t* inv_map, void* stream) {
  REQUIRE(Vd > 0 && V > 0 && Vd <= V, DSPARK_ERR_INVALID, "need 0 < Vd <= V (got Vd=%d, V=%d)", Vd, V);
  REQUIRE_PTR(d2t, "d2t");
  REQUIRE_PTR(inv_map, "inv_map");
  return hip_status(dspark::launch_build_inverse_map(d2t, Vd, V, inv_map, (hipStream_t)stream),
                    "build_inverse_map");
}

size_t dspark_verify_workspace_size(int B, int N, int V) {
  if (B <= 0 || N <= 0 || V <= 0) return 0;
  return dspark::plan_verify(B, N, V).total_bytes;
}

}  // extern "C"

namespace {
// the argument checks of dspark_verify and dspark_verify_noalloc (everything but the workspace)
dspark_status verify_args(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                          const int32_t* draft_tokens, const int32_t* inv_map, const float* temperature,
                          const uint32_t* request_id, const int32_t* accepted, const int32_t* out_tokens, int B, int N,
                          int V, int Vd) {
  REQUIRE(input_kind == DSPARK_INPUT_LOGITS || input_kind == DSPARK_INPUT_PROBS, DSPARK_ERR_INVALID,
          "input_kind must be DSPARK_INPUT_LOGITS or DSPARK_INPUT_PROBS (got %d)", input_kind);
  REQUIRE(B >= 1, DSPARK_ERR_INVALID, "B must be >= 1 (got %d)", B);
  REQUIRE(B <= DSPARK_MAX_B, DSPARK_ERR_UNSUPPORTED, "B must be <= %d (got %d)", DSPARK_MAX_B, B);
  REQUIRE(N >= 1, DSPARK_ERR_INVALID, "N must be >= 1 (got %d)", N);
  REQUIRE(N <= DSPARK_MAX_N, DSPARK_ERR_UNSUPPORTED, "N must be <= %d (got %d)", DSPARK_MAX_N, N);
  REQUIRE(V > 0 && V % 4 == 0, DSPARK_ERR_INVALID, "V must be a positive multiple of 4 (got %d)", V);
  REQUIRE(Vd > 0 && Vd % 4 == 0, DSPARK_ERR_INVALID, "Vd must be a positive multiple of 4 (got %d)", Vd);
  REQUIRE(Vd <= V, DSPARK_ERR_INVALID, "Vd (%d) must be <= V (%d)", Vd, V);
  REQUIRE((int64_t)B * (N + 1) * V < ((int64_t)1 << 40), DSPARK_ERR_UNSUPPORTED, "B * (N+1) * V too large");
  REQUIRE_PTR16(target, "target");
  REQUIRE_PTR16(draft, "draft");
  REQUIRE_PTR(draft_tokens, "draft_tokens");
  if (Vd != V) REQUIRE_PTR(inv_map, "inv_map (required when Vd != V)");
  REQUIRE_PTR(request_id, "request_id");
  REQUIRE_PTR(accepted, "accepted");
  REQUIRE_PTR(out_tokens, "out_tokens");
  if (input_kind == DSPARK_INPUT_LOGITS) {
    REQUIRE_PTR(temperature, "temperature (required for logits input)");
    REQUIRE_PTR(draft_log_z, "draft_log_z (required for logits input)");
  }
  return ok();
}
}  // namespace

extern "C" {

dspark_status dspark_verify(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                            const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                            const float* temperature, const uint32_t* request_id, uint64_t seed, int32_t* accepted,
                            int32_t* out_tokens, float* accept_prob, int B, int N, int V, int Vd, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const dspark_status st = verify_args(input_kind, target, draft, draft_log_z, draft_tokens, inv_map, temperature,
                                       request_id, accepted, out_tokens, B, N, V, Vd);
  if (st != DSPARK_OK) return st;
  const size_t need = dspark_verify_workspace_size(B, N, V);
  REQUIRE(workspace != nullptr, DSPARK_ERR_WORKSPACE, "workspace must not be NULL (%zu bytes needed)", need);
  REQUIRE(aligned16(workspace), DSPARK_ERR_INVALID, "workspace must be 16-byte aligned");
  REQUIRE(workspace_bytes >= need, DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
          need);
  return hip_status(dspark::launch_verify(input_kind, target, draft, draft_log_z, draft_tokens, inv_map, verify_len,
                                          temperature, request_id, seed, accepted, out_tokens, accept_prob, B, N,
                                          V, Vd, workspace, (hipStream_t)stream),
                    "verify");
}

size_t dspark_verify_deferred_workspace_size(int B, int N, int V) {
  if (B <= 0 || N <= 0 || V <= 0) return 0;
  return dspark::plan_verify(B, N, V).total_bytes + dspark::verify_deferred_extra_bytes(B, V);
}

dspark_status dspark_verify_deferred(const float* target, float* draft_base, const float* draft_log_z,
                                     const float* win_logit, const int32_t* draft_tokens, const int32_t* anchor,
                                     const uint16_t* w1, const uint16_t* w2, int r, const int32_t* verify_len,
                                     const float* temperature, const uint32_t* request_id, uint64_t seed,
                                     int32_t* accepted, int32_t* out_tokens, int B, int N, int V, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const dspark_status st = verify_args(DSPARK_INPUT_LOGITS, target, draft_base, draft_log_z, draft_tokens, nullptr,
                                       temperature, request_id, accepted, out_tokens, B, N, V, V);
  if (st != DSPARK_OK) return st;
  REQUIRE_PTR(win_logit, "win_logit");
  REQUIRE_PTR(anchor, "anchor");
  REQUIRE_PTR16(w1, "w1");
  REQUIRE_PTR16(w2, "w2");
  REQUIRE(r >= 8 && r % 8 == 0, DSPARK_ERR_INVALID, "r must be a positive multiple of 8 (got %d)", r);
  REQUIRE(r <= DSPARK_MAX_RANK, DSPARK_ERR_UNSUPPORTED, "r must be <= %d (got %d)", DSPARK_MAX_RANK, r);
  const size_t need = dspark_verify_deferred_workspace_size(B, N, V);
  REQUIRE(workspace != nullptr, DSPARK_ERR_WORKSPACE, "workspace must not be NULL (%zu bytes needed)", need);
  REQUIRE(aligned16(workspace), DSPARK_ERR_INVALID, "workspace must be 16-byte aligned");
  REQUIRE(workspace_bytes >= need, DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
          need);
  dspark::DeferredArgs d;
  d.win = win_logit;
  d.anchor = anchor;
  d.w1 = w1;
  d.w2 = w2;
  d.r = r;
  return hip_status(dspark::launch_verify_deferred(target, draft_base, draft_log_z, draft_tokens, verify_len,
                                                   temperature, request_id, seed, accepted, out_tokens, B, N, V, d,
                                                   workspace, (hipStream_t)stream),
                    "verify_deferred");
}

size_t dspark_context_kv_workspace_size(int num_ctx, int H_d, int L, int nkv, int hd) {
  if (num_ctx <= 0 || H_d <= 0 || L <= 0 || nkv <= 0 || hd <= 0) return 0;
  return dspark::context_kv_workspace_bytes(num_ctx, H_d, L, nkv, hd);
}

dspark_status dspark_context_kv(const uint16_t* aux, const uint16_t* fc_w, const uint16_t* fc_b,
                                const uint16_t* hnorm_w, const uint16_t* kv_w, const uint16_t* kv_b,
                                const uint16_t* knorm_w, const int32_t* positions, const int64_t* slots,
                                uint16_t* k_cache, uint16_t* v_cache, int num_ctx, int H_in, int H_d, int L,
                                int nkv, int hd, int64_t num_slots, float eps, float rope_theta, void* workspace,
                                size_t workspace_bytes, void* stream) {
  REQUIRE(num_ctx >= 0, DSPARK_ERR_INVALID, "num_ctx must be >= 0 (got %d)", num_ctx);
  REQUIRE(H_in > 0 && H_in % 8 == 0, DSPARK_ERR_INVALID, "H_in must be a positive multiple of 8 (got %d)", H_in);
  REQUIRE(H_d > 0 && H_d % 8 == 0, DSPARK_ERR_INVALID, "H_d must be a positive multiple of 8 (got %d)", H_d);
  REQUIRE(L >= 1 && nkv >= 1, DSPARK_ERR_INVALID, "L and nkv must be >= 1 (got %d, %d)", L, nkv);
  REQUIRE(hd >= 2 && hd % 2 == 0, DSPARK_ERR_INVALID, "hd must be even and >= 2 (got %d)", hd);
  REQUIRE(hd <= 256, DSPARK_ERR_UNSUPPORTED, "hd must be <= 256 (got %d)", hd);
  REQUIRE((L * 2 * nkv * hd) % 8 == 0, DSPARK_ERR_INVALID, "L * 2 * nkv * hd must be a multiple of 8");
  REQUIRE(num_slots >= 1, DSPARK_ERR_INVALID, "num_slots must be >= 1");
  REQUIRE(eps >= 0.0f && std::isfinite(eps), DSPARK_ERR_INVALID, "eps must be finite and >= 0");
  REQUIRE(rope_theta > 0.0f && std::isfinite(rope_theta), DSPARK_ERR_INVALID, "rope_theta must be finite and > 0");
  if (num_ctx == 0) return ok();
  REQUIRE((int64_t)num_ctx * L * 2 * nkv * hd < ((int64_t)1 << 40), DSPARK_ERR_UNSUPPORTED, "num_ctx too large");
  REQUIRE_PTR16(aux, "aux");
  REQUIRE_PTR16(fc_w, "fc_w");
  if (fc_b) REQUIRE(aligned16(fc_b), DSPARK_ERR_INVALID, "fc_b must be 16-byte aligned");
  REQUIRE_PTR16(hnorm_w, "hnorm_w");
  REQUIRE_PTR16(kv_w, "kv_w");
  REQUIRE_PTR16(kv_b, "kv_b");
  REQUIRE_PTR16(knorm_w, "knorm_w");
  REQUIRE_PTR(positions, "positions");
  REQUIRE_PTR(slots, "slots");
  REQUIRE_PTR16(k_cache, "k_cache");
  REQUIRE_PTR16(v_cache, "v_cache");
  const size_t need = dspark_context_kv_workspace_size(num_ctx, H_d, L, nkv, hd);
  REQUIRE(workspace != nullptr, DSPARK_ERR_WORKSPACE, "workspace must not be NULL (%zu bytes needed)", need);
  REQUIRE(aligned16(workspace), DSPARK_ERR_INVALID, "workspace must be 16-byte aligned");
  REQUIRE(workspace_bytes >= need, DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
          need);
  return hip_status(dspark::launch_context_kv(aux, fc_w, fc_b, hnorm_w, kv_w, kv_b, knorm_w, positions, slots,
                                              k_cache, v_cache, num_ctx, H_in, H_d, L, nkv, hd, num_slots, eps,
                                              rope_theta, workspace, (hipStream_t)stream),
                    "context_kv");
}

size_t dspark_verify_noalloc_max_bytes(void) { return dspark::kVerifyScratchBytes; }

dspark_status dspark_verify_noalloc(int input_kind, const float* target, const float* draft,
                                    const float* draft_log_z, const int32_t* draft_tokens, const int32_t* inv_map,
                                    const int32_t* verify_len, const float* temperature, const uint32_t* request_id,
                                    uint64_t seed, int32_t* accepted, int32_t* out_tokens, float* accept_prob, int B,
                                    int N, int V, int Vd, void* stream) {
  const dspark_status st = verify_args(input_kind, target, draft, draft_log_z, draft_tokens, inv_map, temperature,
                                       request_id, accepted, out_tokens, B, N, V, Vd);
  if (st != DSPARK_OK) return st;
  const size_t need = dspark_verify_workspace_size(B, N, V);
  REQUIRE(need <= dspark::kVerifyScratchBytes, DSPARK_ERR_UNSUPPORTED,
          "verify_noalloc: this shape needs %zu bytes of scratch, above the static %zu (use dspark_verify with a "
          "workspace)", need, dspark::kVerifyScratchBytes);
  return hip_status(dspark::launch_verify_noalloc(input_kind, target, draft, draft_log_z, draft_tokens, inv_map,
                                                  verify_len, temperature, request_id, seed, accepted, out_tokens,
                                                  accept_prob, B, N, V, Vd, (hipStream_t)stream),
                    "verify_noalloc");
}

size_t dspark_verify_coupled_workspace_size(int B, int N, int V) {
  if (B <= 0 || N <= 0 || V <= 0) return 0;
  return dspark::coupled_workspace_bytes(B, N, V);
}

dspark_status dspark_verify_coupled(const float* target_logits, const int32_t* draft_tokens, const int32_t* inv_map,
                                    const int32_t* verify_len, const float* temperature, const uint32_t* request_id,
                                    uint64_t seed, int32_t* accepted, int32_t* out_tokens, int B, int N, int V, int Vd,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(B >= 1, DSPARK_ERR_INVALID, "B must be >= 1 (got %d)", B);
  REQUIRE(B <= DSPARK_MAX_B, DSPARK_ERR_UNSUPPORTED, "B must be <= %d (got %d)", DSPARK_MAX_B, B);
  REQUIRE(N >= 1, DSPARK_ERR_INVALID, "N must be >= 1 (got %d)", N);
  REQUIRE(N <= DSPARK_MAX_N, DSPARK_ERR_UNSUPPORTED, "N must be <= %d (got %d)", DSPARK_MAX_N, N);
  REQUIRE(V > 0 && V % 4 == 0, DSPARK_ERR_INVALID, "V must be a positive multiple of 4 (got %d)", V);
  REQUIRE(Vd > 0 && Vd <= V, DSPARK_ERR_INVALID, "Vd must be in [1, V] (got %d)", Vd);
  REQUIRE((int64_t)B * (N + 1) * V < ((int64_t)1 << 40), DSPARK_ERR_UNSUPPORTED, "B * (N+1) * V too large");
  REQUIRE_PTR16(target_logits, "target_logits");
  REQUIRE_PTR(draft_tokens, "draft_tokens");
  if (Vd != V) REQUIRE_PTR16(inv_map, "inv_map (required when Vd != V)");
  REQUIRE_PTR(temperature, "temperature");
  REQUIRE_PTR(request_id, "request_id");
  REQUIRE_PTR(accepted, "accepted");
  REQUIRE_PTR(out_tokens, "out_tokens");
  const size_t need = dspark_verify_coupled_workspace_size(B, N, V);
  REQUIRE(workspace != nullptr, DSPARK_ERR_WORKSPACE, "workspace must not be NULL (%zu bytes needed)", need);
  REQUIRE(aligned16(workspace), DSPARK_ERR_INVALID, "workspace must be 16-byte aligned");
  REQUIRE(workspace_bytes >= need, DSPARK_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", workspace_bytes,
          need);
  return hip_status(dspark::launch_verify_coupled(target_logits, draft_tokens, Vd != V ? inv_map : nullptr,
                                                  verify_len, temperature, request_id, seed, accepted, out_tokens,
                                                  B, N, V, workspace, (hipStream_t)stream),
                    "verify_coupled");
}

dspark_status dspark_admit(const float* cond_accept, int B, int N, int K, float* survival, int32_t* admit_len,
                           void* stream) {
  REQUIRE(B >= 1, DSPARK_ERR_INVALID, "B must be >= 1 (got %d)", B);
  REQUIRE(N >= 1, DSPARK_ERR_INVALID, "N must be >= 1 (got %d)", N);
  REQUIRE(N <= DSPARK_MAX_N, DSPARK_ERR_UNSUPPORTED, "N must be <= %d (got %d)", DSPARK_MAX_N, N);
  REQUIRE(B <= DSPARK_MAX_B, DSPARK_ERR_UNSUPPORTED, "B must be <= %d (got %d)", DSPARK_MAX_B, B);
  REQUIRE((int64_t)B * N <= DSPARK_MAX_ADMIT, DSPARK_ERR_UNSUPPORTED, "B * N must be <= %d (got %lld)",
          DSPARK_MAX_ADMIT, (long long)B * N);
  REQUIRE(K >= 0, DSPARK_ERR_INVALID, "K must be >= 0 (got %d)", K);
  REQUIRE_PTR(cond_accept, "cond_accept");
  REQUIRE_PTR(survival, "survival");
  REQUIRE_PTR(admit_len, "admit_len");
  return hip_status(dspark::launch_admit(cond_accept, B, N, K, survival, admit_len, (hipStream_t)stream), "admit");
}

dspark_status dspark_advance(const int32_t* accepted, const int32_t* out_tokens, int32_t* anchor, int64_t* emitted,
                             int B, int N, void* stream) {
  REQUIRE(B >= 1, DSPARK_ERR_INVALID, "B must be >= 1 (got %d)", B);
  REQUIRE(B <= DSPARK_MAX_B, DSPARK_ERR_UNSUPPORTED, "B must be <= %d (got %d)", DSPARK_MAX_B, B);
  REQUIRE(N >= 1, DSPARK_ERR_INVALID, "N must be >= 1 (got %d)", N);
  REQUIRE(N <= DSPARK_MAX_N, DSPARK_ERR_UNSUPPORTED, "N must be <= %d (got %d)", DSPARK_MAX_N, N);
  REQUIRE_PTR(accepted, "accepted");
  REQUIRE_PTR(out_tokens, "out_tokens");
  REQUIRE_PTR(anchor, "anchor");
  return hip_status(dspark::launch_advance(accepted, out_tokens, anchor, emitted, B, N, (hipStream_t)stream),
                    "advance");
}

dspark_status dspark_choose_k(const float* survival, int B, int N, const float* sps, int S, int32_t* k_out,
                              double* objective_out, void* stream) {
  REQUIRE(B >= 1, DSPARK_ERR_INVALID, "B must be >= 1 (got %d)", B);
  REQUIRE(N >= 1, DSPARK_ERR_INVALID, "N must be >= 1 (got %d)", N);
  REQUIRE(N <= DSPARK_MAX_N, DSPARK_ERR_UNSUPPORTED, "N must be <= %d (got %d)", DSPARK_MAX_N, N);
  REQUIRE(B <= DSPARK_MAX_B, DSPARK_ERR_UNSUPPORTED, "B must be <= %d (got %d)", DSPARK_MAX_B, B);
  REQUIRE((int64_t)B * N <= DSPARK_MAX_ADMIT, DSPARK_ERR_UNSUPPORTED, "B * N must be <= %d (got %lld)",
          DSPARK_MAX_ADMIT, (long long)B * N);
  REQUIRE(S >= B + 1, DSPARK_ERR_INVALID, "the SPS table must cover a batch of B tokens: S >= B + 1 (got S=%d, B=%d)",
          S, B);
  REQUIRE_PTR(survival, "survival");
  REQUIRE_PTR(sps, "sps");
  REQUIRE_PTR(k_out, "k_out");
  return hip_status(dspark::launch_choose_k(survival, B, N, sps, S, k_out, objective_out, (hipStream_t)stream),
                    "choose_k");
}

}  // extern "C"
