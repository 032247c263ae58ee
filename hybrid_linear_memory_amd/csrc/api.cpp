// C-ABI layer of libarl2: host-side validation, workspace carving and
// dispatch to the HIP kernels. Every check runs before anything is enqueued;
// on error nothing is launched and the detail text is kept per thread.
//
// The pass-level calls follow "Attend Locally, Remember Linearly" technical
// summary §2.2: a denoising read takes the state as const; only the clean
// pass (or arl2_commit) writes the next state, into a separate buffer.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "../../include/arl2.h"
#include "arl2_internal.h"

namespace {

thread_local std::string g_err;

arl2_status fail(arl2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

arl2_status ok() {
  g_err.clear();
  return ARL2_OK;
}

arl2_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ARL2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

arl2_status check_shape(const arl2_shape* sh, arl2::Dims* d) {
  if (!sh) return fail(ARL2_E_NULL, "shape is NULL");
  if (sh->act_dtype != ARL2_F32 && sh->act_dtype != ARL2_BF16)
    return fail(ARL2_E_DTYPE, "act_dtype %d is neither ARL2_F32 (0) nor ARL2_BF16 (1)",
                sh->act_dtype);
  if (sh->B < 1 || sh->H < 1 || sh->T < 1)
    return fail(ARL2_E_SHAPE, "B, H, T must be >= 1 (got %d, %d, %d)", sh->B, sh->H, sh->T);
  const bool bf16 = sh->act_dtype == ARL2_BF16;
  if (sh->D != 16 && sh->D != 32 && sh->D != 64 && sh->D != 128)
    return fail(ARL2_E_SHAPE, "D must be one of 16, 32, 64, 128 (got %d)", sh->D);
  const double elems = (double)sh->B * sh->H * sh->T * sh->D;
  if (elems >= 2147483648.0)
    return fail(ARL2_E_SHAPE, "B*H*T*D = %.0f exceeds 2^31 - 1", elems);
  if (!(sh->softmax_scale >= 0.f) || isinf(sh->softmax_scale))
    return fail(ARL2_E_SHAPE, "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(D))");
  d->B = sh->B;
  d->H = sh->H;
  d->T = sh->T;
  d->D = sh->D;
  d->bf16 = bf16;
  d->scale = sh->softmax_scale > 0.f ? sh->softmax_scale : 1.0f / sqrtf((float)sh->D);
  return ARL2_OK;
}

// The token-level and training calls run bf16 activations at D = 128 only
// (their smaller-D kernels are float32).
arl2_status require_d128_for_bf16(const arl2::Dims& d, const char* what) {
  if (d.bf16 && d.D != 128)
    return fail(ARL2_E_SHAPE, "%s with bf16 activations needs D = 128 (got %d)", what, d.D);
  return ARL2_OK;
}

#define REQUIRE_PTR(p)                                                          \
  do {                                                                          \
    if (!(p)) return fail(ARL2_E_NULL, "argument '%s' is NULL", #p);            \
    if (!aligned16(p)) return fail(ARL2_E_LAYOUT, "argument '%s' is not 16-byte aligned", #p); \
  } while (0)

#define OPTIONAL_PTR(p)                                                         \
  do {                                                                          \
    if ((p) && !aligned16(p))                                                   \
      return fail(ARL2_E_LAYOUT, "argument '%s' is not 16-byte aligned", #p);   \
  } while (0)

size_t state_bytes(const arl2::Dims& d) { return (size_t)d.B * d.H * d.D * d.D * sizeof(float); }
size_t phi_bytes(const arl2::Dims& d) { return (size_t)d.H * d.D * d.D * (d.bf16 ? 2 : 4); }
size_t commit_ws(const arl2::Dims& d) {
  return arl2::use_mfma(d) ? arl2::mfma_state_commit_ws_bytes(d)
                           : arl2::generic_state_commit_ws_bytes(d);
}

size_t ws_read(const arl2::Dims& d) {
  return arl2::use_mfma(d) ? arl2::round_up(arl2::mfma_read_ws_bytes(d), 256)
                           : 2 * arl2::round_up(arl2::act_bytes(d), 256);
}
size_t prepared_bytes(const arl2::Dims& d) {
  return (size_t)d.B * d.H * d.D * d.D * (arl2::use_mfma(d) ? 2 : 4);
}
size_t ws_read_prepared(const arl2::Dims& d) {
  return arl2::use_mfma(d) ? arl2::mfma_read_prepared_ws_bytes(d)
                           : arl2::round_up(arl2::act_bytes(d), 256);
}
size_t ws_commit(const arl2::Dims& d) {
  if (arl2::use_mfma(d)) return arl2::round_up(arl2::mfma_commit_ws_bytes(d), 256);
  return 2 * arl2::round_up(arl2::act_bytes(d), 256) + arl2::round_up(commit_ws(d), 256);
}
// bf16: the commit partials of the one-launch clean pass; otherwise the read
// and the commit run one after the other in the same workspace.
size_t ws_clean_pass_prepared(const arl2::Dims& d) {
  return arl2::use_mfma(d) ? arl2::round_up(arl2::mfma_clean_commit_ws_bytes(d), 256)
                           : std::max(ws_read_prepared(d), ws_commit(d));
}

// Token-level access: Q', K', V', an o_intra buffer, then the scan's own.
size_t ws_token(const arl2::Dims& d) {
  return 4 * arl2::round_up(arl2::act_bytes(d), 256) +
         arl2::round_up(arl2::token_level_scan_ws_bytes(d), 256);
}

arl2_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return ARL2_OK;
  if (!ws) return fail(ARL2_E_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned16(ws)) return fail(ARL2_E_LAYOUT, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(ARL2_E_WORKSPACE, "workspace has %zu bytes, %zu are needed", ws_bytes, need);
  return ARL2_OK;
}

// ---------------------------------------------------------------- dispatch
hipError_t run_feature_map(const arl2::Dims& d, const void* x, const void* phi, void* out,
                           bool norm, hipStream_t s) {
  return arl2::use_mfma(d) ? arl2::mfma_feature_map(d, x, phi, out, norm, s)
                           : arl2::generic_feature_map(d, x, phi, out, norm, s);
}
hipError_t run_attention(const arl2::Dims& d, const void* q, const void* k, const void* v,
                         void* o, int64_t n_kv, int64_t cap, hipStream_t s) {
  return arl2::use_mfma(d) ? arl2::mfma_attention(d, q, k, v, o, n_kv, cap, s)
                           : arl2::generic_attention(d, q, k, v, o, n_kv, cap, s);
}
hipError_t run_inter_read(const arl2::Dims& d, const void* qp, const float* S, const void* oi,
                          void* o, void* oe, hipStream_t s) {
  return arl2::use_mfma(d) ? arl2::mfma_inter_read(d, qp, S, oi, o, oe, s)
                           : arl2::generic_inter_read(d, qp, S, oi, o, oe, s);
}
hipError_t run_state_commit(const arl2::Dims& d, const void* kp, const void* vp,
                            const float* beta, const float* alpha, const float* Sp, float* Sn,
                            void* ws, hipStream_t s) {
  return arl2::use_mfma(d) ? arl2::mfma_state_commit(d, kp, vp, beta, alpha, Sp, Sn, ws, s)
                           : arl2::generic_state_commit(d, kp, vp, beta, alpha, Sp, Sn, ws, s);
}

// Read = feature map of Q, intra attention, inter read + combine. The bf16
// D = 128 path fuses them: M = Phi_q S per head, then attention with the
// epilogue O = O_intra + Q M.
arl2_status do_read(const arl2::Dims& d, const void* q, const void* k, const void* v,
                    const void* phi_q, const float* S, void* o, void* o_intra, void* o_inter,
                    void* ws, hipStream_t s) {
  if (arl2::use_mfma(d))
    return hip_status(arl2::mfma_read(d, q, k, v, phi_q, S, o, o_intra, o_inter, ws, s),
                      "fused read");
  const size_t ab = arl2::round_up(arl2::act_bytes(d), 256);
  char* w = static_cast<char*>(ws);
  void* q_prime = w;
  void* oi = o_intra ? o_intra : (void*)(w + ab);
  hipError_t e = run_feature_map(d, q, phi_q, q_prime, false, s);
  if (e != hipSuccess) return hip_status(e, "feature map (phi_q)");
  e = run_attention(d, q, k, v, oi, d.T, d.T, s);
  if (e != hipSuccess) return hip_status(e, "intra-frame attention");
  e = run_inter_read(d, q_prime, S, oi, o, o_inter, s);
  if (e != hipSuccess) return hip_status(e, "inter-frame read");
  return ok();
}

arl2_status do_commit(const arl2::Dims& d, const void* k, const void* v, const void* phi_k,
                      const void* phi_v, const float* beta, const float* alpha,
                      const float* S_prev, float* S_next, void* ws, hipStream_t s) {
  if (arl2::use_mfma(d))
    return hip_status(arl2::mfma_commit(d, k, v, phi_k, phi_v, beta, alpha, S_prev, S_next, ws, s),
                      "fused commit");
  const size_t ab = arl2::round_up(arl2::act_bytes(d), 256);
  char* w = static_cast<char*>(ws);
  void* kp = w;
  void* vp = w + ab;
  void* cws = w + 2 * ab;
  hipError_t e = run_feature_map(d, k, phi_k, kp, true, s);
  if (e != hipSuccess) return hip_status(e, "feature map (phi_k)");
  e = run_feature_map(d, v, phi_v, vp, false, s);
  if (e != hipSuccess) return hip_status(e, "feature map (phi_v)");
  e = run_state_commit(d, kp, vp, beta, alpha, S_prev, S_next, cws, s);
  if (e != hipSuccess) return hip_status(e, "state commit");
  return ok();
}

// One pass under token-level access; alpha and S_next null for a read.
arl2_status do_token(const arl2::Dims& d, const void* q, const void* k, const void* v,
                     const void* phi_q, const void* phi_k, const void* phi_v, const float* beta,
                     const float* alpha, const float* S_prev, float* S_next, void* o,
                     void* o_intra, void* o_inter, void* ws, hipStream_t s) {
  const size_t ab = arl2::round_up(arl2::act_bytes(d), 256);
  char* w = static_cast<char*>(ws);
  void* qp = w;
  void* kp = w + ab;
  void* vp = w + 2 * ab;
  void* oi = o_intra ? o_intra : (void*)(w + 3 * ab);
  hipError_t e;
  if (arl2::use_mfma(d)) {
    const arl2::FeatureMapJob jobs[3] = {
        {q, phi_q, qp, false}, {k, phi_k, kp, true}, {v, phi_v, vp, false}};
    e = arl2::mfma_feature_maps(d, jobs, 3, s);
    if (e != hipSuccess) return hip_status(e, "feature maps");
  } else {
    e = run_feature_map(d, q, phi_q, qp, false, s);
    if (e != hipSuccess) return hip_status(e, "feature map (phi_q)");
    e = run_feature_map(d, k, phi_k, kp, true, s);
    if (e != hipSuccess) return hip_status(e, "feature map (phi_k)");
    e = run_feature_map(d, v, phi_v, vp, false, s);
    if (e != hipSuccess) return hip_status(e, "feature map (phi_v)");
  }
  e = run_attention(d, q, k, v, oi, d.T, d.T, s);
  if (e != hipSuccess) return hip_status(e, "intra-frame attention");
  e = arl2::token_level_scan(d, qp, kp, vp, beta, S_prev, alpha, S_next, oi, o, o_inter,
                             w + 4 * ab, s);
  return hip_status(e, "token-level scan");
}

// Validation shared by the two token-level entry points.
arl2_status check_token(const arl2::Dims& d, const void* q, const void* k, const void* v,
                        const void* phi_q, const void* phi_k, const void* phi_v,
                        const float* beta, const float* alpha, const float* S_prev,
                        float* S_next, void* o, void* o_intra, void* o_inter, void* ws,
                        size_t ws_bytes) {
  arl2_status st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_q);
  REQUIRE_PTR(phi_k);
  REQUIRE_PTR(phi_v);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(S_prev);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  OPTIONAL_PTR(o_inter);
  const size_t need = ws_token(d);
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d), sb = (size_t)d.B * d.H * d.D * d.D * sizeof(float);
  const Range outs[4] = {{o, ab}, {o_intra, ab}, {o_inter, ab}, {S_next, S_next ? sb : 0}};
  const Range ins[10] = {{q, ab},
                         {k, ab},
                         {v, ab},
                         {phi_q, phi_bytes(d)},
                         {phi_k, phi_bytes(d)},
                         {phi_v, phi_bytes(d)},
                         {S_prev, sb},
                         {ws, need},
                         {beta, (size_t)d.B * d.H * d.T * 4},
                         {alpha, alpha ? (size_t)d.B * d.H * 4 : 0}};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ARL2_E_ALIAS, "an output overlaps an input or the workspace");
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(ARL2_E_ALIAS, "two outputs overlap");
  return ARL2_OK;
}

arl2_status check_disjoint(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(ARL2_E_ALIAS, "an output overlaps an input or the workspace");
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return fail(ARL2_E_ALIAS, "two outputs overlap");
  }
  return ARL2_OK;
}

arl2_status check_state_pair(const arl2::Dims& d, const float* S_prev, const float* S_next) {
  if (overlap({S_prev, state_bytes(d)}, {S_next, state_bytes(d)}))
    return fail(ARL2_E_ALIAS, "S_prev and S_next overlap; the state must be double-buffered");
  return ARL2_OK;
}

}  // namespace

extern "C" {

int32_t arl2_abi_version(void) { return ARL2_ABI_VERSION; }

const char* arl2_last_error(void) { return g_err.c_str(); }

const char* arl2_status_string(arl2_status st) {
  switch (st) {
    case ARL2_OK: return "ARL2_OK";
    case ARL2_E_NULL: return "ARL2_E_NULL";
    case ARL2_E_SHAPE: return "ARL2_E_SHAPE";
    case ARL2_E_DTYPE: return "ARL2_E_DTYPE";
    case ARL2_E_LAYOUT: return "ARL2_E_LAYOUT";
    case ARL2_E_ALIAS: return "ARL2_E_ALIAS";
    case ARL2_E_WORKSPACE: return "ARL2_E_WORKSPACE";
    case ARL2_E_HIP: return "ARL2_E_HIP";
  }
  return "ARL2_E_UNKNOWN";
}

size_t arl2_workspace_bytes(const arl2_shape* shape, int32_t op) {
  arl2::Dims d;
  if (check_shape(shape, &d) != ARL2_OK) return 0;
  switch (op) {
    case ARL2_OP_READ: return ws_read(d);
    case ARL2_OP_COMMIT: return ws_commit(d);
    case ARL2_OP_CLEAN_PASS: return std::max(ws_read(d), ws_commit(d));
    case ARL2_OP_STATE_COMMIT: return commit_ws(d);
    case ARL2_OP_READ_PREPARED: return ws_read_prepared(d);
    case ARL2_OP_CLEAN_PASS_PREPARED: return ws_clean_pass_prepared(d);
    case ARL2_OP_TOKEN_LEVEL: return ws_token(d);
    case ARL2_OP_INTRA_ATTN_BACKWARD: return arl2::attn_backward_ws_bytes(d);
    case ARL2_OP_READ_BACKWARD: return arl2::read_backward_ws_bytes(d);
    case ARL2_OP_COMMIT_BACKWARD: return arl2::commit_backward_ws_bytes(d);
    default: return 0;
  }
}

arl2_status arl2_feature_map(const arl2_shape* shape, const void* x, const void* phi, void* x_out,
                             int32_t normalize_rows, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(x);
  REQUIRE_PTR(phi);
  REQUIRE_PTR(x_out);
  const size_t ab = arl2::act_bytes(d);
  if (overlap({x, ab}, {x_out, ab}) || overlap({phi, phi_bytes(d)}, {x_out, ab}))
    return fail(ARL2_E_ALIAS, "x_out overlaps an input");
  return hip_status(run_feature_map(d, x, phi, x_out, normalize_rows != 0, (hipStream_t)stream),
                    "feature map");
}

arl2_status arl2_intra_attn(const arl2_shape* shape, const void* q, const void* k, const void* v,
                            void* o_intra, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o_intra);
  const size_t ab = arl2::act_bytes(d);
  if (overlap({q, ab}, {o_intra, ab}) || overlap({k, ab}, {o_intra, ab}) ||
      overlap({v, ab}, {o_intra, ab}))
    return fail(ARL2_E_ALIAS, "o_intra overlaps an input");
  return hip_status(run_attention(d, q, k, v, o_intra, d.T, d.T, (hipStream_t)stream),
                    "intra-frame attention");
}

arl2_status arl2_intra_attn_lse(const arl2_shape* shape, const void* q, const void* k,
                                const void* v, void* o_intra, float* lse, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if ((st = require_d128_for_bf16(d, "arl2_intra_attn_lse")) != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o_intra);
  REQUIRE_PTR(lse);
  const size_t ab = arl2::act_bytes(d);
  const size_t lb = (size_t)d.B * d.H * d.T * sizeof(float);
  const Range outs[2] = {{o_intra, ab}, {lse, lb}};
  const Range ins[3] = {{q, ab}, {k, ab}, {v, ab}};
  if ((st = check_disjoint(outs, 2, ins, 3)) != ARL2_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (arl2::use_mfma(d))
    return hip_status(arl2::mfma_attention_lse(d, q, k, v, o_intra, lse, s),
                      "intra-frame attention");
  hipError_t e = run_attention(d, q, k, v, o_intra, d.T, d.T, s);
  if (e != hipSuccess) return hip_status(e, "intra-frame attention");
  return hip_status(arl2::attn_lse_f32(d, q, k, lse, s), "row log-sum-exp");
}

arl2_status arl2_inter_read(const arl2_shape* shape, const void* q_prime, const float* S,
                            const void* o_intra, void* o, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q_prime);
  REQUIRE_PTR(S);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  const size_t ab = arl2::act_bytes(d);
  if (overlap({q_prime, ab}, {o, ab}) || overlap({S, state_bytes(d)}, {o, ab}))
    return fail(ARL2_E_ALIAS, "o overlaps q_prime or S");
  if (o_intra && o_intra != o && overlap({o_intra, ab}, {o, ab}))
    return fail(ARL2_E_ALIAS, "o partially overlaps o_intra (only o == o_intra is allowed)");
  return hip_status(run_inter_read(d, q_prime, S, o_intra, o, nullptr, (hipStream_t)stream),
                    "inter-frame read");
}

arl2_status arl2_state_commit(const arl2_shape* shape, const void* k_prime, const void* v_prime,
                              const float* beta, const float* alpha, const float* S_prev,
                              float* S_next, void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(k_prime);
  REQUIRE_PTR(v_prime);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S_prev);
  REQUIRE_PTR(S_next);
  if ((st = check_state_pair(d, S_prev, S_next)) != ARL2_OK) return st;
  if ((st = check_ws(ws, ws_bytes, commit_ws(d))) != ARL2_OK) return st;
  {
    const size_t ab = arl2::act_bytes(d);
    const Range outs[1] = {{S_next, state_bytes(d)}};
    const Range ins[6] = {{k_prime, ab},
                          {v_prime, ab},
                          {beta, (size_t)d.B * d.H * d.T * 4},
                          {alpha, (size_t)d.B * d.H * 4},
                          {S_prev, state_bytes(d)},
                          {ws, commit_ws(d)}};
    if ((st = check_disjoint(outs, 1, ins, 6)) != ARL2_OK) return st;
  }
  return hip_status(run_state_commit(d, k_prime, v_prime, beta, alpha, S_prev, S_next, ws,
                                     (hipStream_t)stream),
                    "state commit");
}

arl2_status arl2_read(const arl2_shape* shape, const void* q, const void* k, const void* v,
                      const void* phi_q, const float* S, void* o, void* o_intra, void* o_inter,
                      void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_q);
  REQUIRE_PTR(S);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  OPTIONAL_PTR(o_inter);
  if ((st = check_ws(ws, ws_bytes, ws_read(d))) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d);
  const Range outs[3] = {{o, ab}, {o_intra, ab}, {o_inter, ab}};
  const Range ins[6] = {{q, ab}, {k, ab}, {v, ab}, {phi_q, phi_bytes(d)}, {S, state_bytes(d)},
                        {ws, ws_read(d)}};
  for (const Range& a : outs) {
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ARL2_E_ALIAS, "an output overlaps an input or the workspace");
  }
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2]))
    return fail(ARL2_E_ALIAS, "outputs o, o_intra, o_inter overlap");
  return do_read(d, q, k, v, phi_q, S, o, o_intra, o_inter, ws, (hipStream_t)stream);
}

arl2_status arl2_read_noalloc(const arl2_shape* shape, const void* q, const void* k,
                              const void* v, const void* phi_q, const float* S, void* o,
                              void* o_intra, void* o_inter, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_q);
  REQUIRE_PTR(S);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  OPTIONAL_PTR(o_inter);
  const size_t ab = arl2::act_bytes(d);
  const Range outs[3] = {{o, ab}, {o_intra, ab}, {o_inter, ab}};
  const Range ins[5] = {{q, ab}, {k, ab}, {v, ab}, {phi_q, phi_bytes(d)}, {S, state_bytes(d)}};
  if ((st = check_disjoint(outs, 3, ins, 5)) != ARL2_OK) return st;
  // bf16 at D = 128: the map M^T = (Phi_q S)^T, then the fused read on the
  // plain grid (one workgroup per 128 queries of a head, no split-key
  // workspace); other shapes: Q' and o_intra as in arl2_read
  const bool mf = arl2::use_mfma(d);
  const size_t need = mf ? arl2::round_up(prepared_bytes(d), 256) : ws_read(d);
  const size_t have = arl2::noalloc_scratch_bytes();
  if (need > have)
    return fail(ARL2_E_WORKSPACE,
                "arl2_read_noalloc needs %zu bytes of scratch for this shape; the library's "
                "fixed scratch holds %zu (use arl2_read with a workspace)",
                need, have);
  void* scratch_ptr = nullptr;
  if ((st = hip_status(arl2::noalloc_scratch(&scratch_ptr), "scratch address")) != ARL2_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  if (!mf) return do_read(d, q, k, v, phi_q, S, o, o_intra, o_inter, scratch_ptr, s);
  hipError_t e = arl2::mfma_read_prepare(d, phi_q, S, scratch_ptr, s);
  if (e != hipSuccess) return hip_status(e, "read preparation");
  return hip_status(arl2::mfma_read_prepared(d, q, k, v, scratch_ptr, o, o_intra, o_inter,
                                             nullptr, 0, s),
                    "prepared read");
}

size_t arl2_prepared_bytes(const arl2_shape* shape) {
  arl2::Dims d;
  if (check_shape(shape, &d) != ARL2_OK) return 0;
  return prepared_bytes(d);
}

arl2_status arl2_read_prepare(const arl2_shape* shape, const void* phi_q, const float* S,
                              void* prepared, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(phi_q);
  REQUIRE_PTR(S);
  REQUIRE_PTR(prepared);
  const size_t pb = prepared_bytes(d);
  if (overlap({prepared, pb}, {S, state_bytes(d)}) || overlap({prepared, pb}, {phi_q, phi_bytes(d)}))
    return fail(ARL2_E_ALIAS, "prepared overlaps phi_q or S");
  hipStream_t s = (hipStream_t)stream;
  return hip_status(arl2::use_mfma(d)
                        ? arl2::mfma_read_prepare(d, phi_q, S, prepared, s)
                        : arl2::generic_read_prepare(d, phi_q, S, static_cast<float*>(prepared), s),
                    "read preparation");
}

arl2_status arl2_read_prepared(const arl2_shape* shape, const void* q, const void* k,
                               const void* v, const void* prepared, void* o, void* o_intra,
                               void* o_inter, void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(prepared);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  OPTIONAL_PTR(o_inter);
  const size_t need = ws_read_prepared(d);
  // bf16: the workspace is optional (without it the read runs on the plain grid)
  if ((ws || !arl2::use_mfma(d)) && (st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d);
  const Range outs[3] = {{o, ab}, {o_intra, ab}, {o_inter, ab}};
  const Range ins[5] = {{q, ab}, {k, ab}, {v, ab}, {prepared, prepared_bytes(d)}, {ws, need}};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ARL2_E_ALIAS, "an output overlaps an input or the workspace");
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2]))
    return fail(ARL2_E_ALIAS, "outputs o, o_intra, o_inter overlap");
  hipStream_t s = (hipStream_t)stream;
  if (arl2::use_mfma(d))
    return hip_status(arl2::mfma_read_prepared(d, q, k, v, prepared, o, o_intra, o_inter, ws,
                                               ws ? ws_bytes : 0, s),
                      "prepared read");
  void* oi = o_intra ? o_intra : ws;
  hipError_t e = run_attention(d, q, k, v, oi, d.T, d.T, s);
  if (e != hipSuccess) return hip_status(e, "intra-frame attention");
  // the inter read with the prepared map: o = o_intra + Q M
  e = arl2::generic_inter_read(d, q, static_cast<const float*>(prepared), oi, o, o_inter, s);
  return hip_status(e, "inter-frame read");
}

arl2_status arl2_commit(const arl2_shape* shape, const void* k, const void* v, const void* phi_k,
                        const void* phi_v, const float* beta, const float* alpha,
                        const float* S_prev, float* S_next, void* ws, size_t ws_bytes,
                        void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_k);
  REQUIRE_PTR(phi_v);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S_prev);
  REQUIRE_PTR(S_next);
  if ((st = check_state_pair(d, S_prev, S_next)) != ARL2_OK) return st;
  if ((st = check_ws(ws, ws_bytes, ws_commit(d))) != ARL2_OK) return st;
  {
    const size_t ab = arl2::act_bytes(d);
    const Range outs[1] = {{S_next, state_bytes(d)}};
    const Range ins[8] = {{k, ab},
                          {v, ab},
                          {phi_k, phi_bytes(d)},
                          {phi_v, phi_bytes(d)},
                          {beta, (size_t)d.B * d.H * d.T * 4},
                          {alpha, (size_t)d.B * d.H * 4},
                          {S_prev, state_bytes(d)},
                          {ws, ws_commit(d)}};
    if ((st = check_disjoint(outs, 1, ins, 8)) != ARL2_OK) return st;
  }
  return do_commit(d, k, v, phi_k, phi_v, beta, alpha, S_prev, S_next, ws, (hipStream_t)stream);
}

arl2_status arl2_clean_pass(const arl2_shape* shape, const void* q, const void* k, const void* v,
                            const void* phi_q, const void* phi_k, const void* phi_v,
                            const float* beta, const float* alpha, const float* S_prev,
                            float* S_next, void* o, void* o_intra, void* o_inter, void* ws,
                            size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_q);
  REQUIRE_PTR(phi_k);
  REQUIRE_PTR(phi_v);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S_prev);
  REQUIRE_PTR(S_next);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  OPTIONAL_PTR(o_inter);
  if ((st = check_state_pair(d, S_prev, S_next)) != ARL2_OK) return st;
  const size_t need = std::max(ws_read(d), ws_commit(d));
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d);
  const Range outs[4] = {{o, ab}, {o_intra, ab}, {o_inter, ab}, {S_next, state_bytes(d)}};
  const Range ins[10] = {{q, ab},
                         {k, ab},
                         {v, ab},
                         {phi_q, phi_bytes(d)},
                         {phi_k, phi_bytes(d)},
                         {phi_v, phi_bytes(d)},
                         {S_prev, state_bytes(d)},
                         {ws, need},
                         {beta, (size_t)d.B * d.H * d.T * 4},
                         {alpha, (size_t)d.B * d.H * 4}};
  if ((st = check_disjoint(outs, 4, ins, 10)) != ARL2_OK) return st;
  st = do_read(d, q, k, v, phi_q, S_prev, o, o_intra, o_inter, ws, (hipStream_t)stream);
  if (st != ARL2_OK) return st;
  return do_commit(d, k, v, phi_k, phi_v, beta, alpha, S_prev, S_next, ws, (hipStream_t)stream);
}

arl2_status arl2_clean_pass_prepared(const arl2_shape* shape, const void* q, const void* k,
                                     const void* v, const void* prepared, const void* phi_q,
                                     const void* phi_k, const void* phi_v, const float* beta,
                                     const float* alpha, const float* S_prev, float* S_next,
                                     void* prepared_next, void* o, void* o_intra, void* o_inter,
                                     void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(prepared);
  REQUIRE_PTR(phi_k);
  REQUIRE_PTR(phi_v);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S_prev);
  REQUIRE_PTR(S_next);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(o_intra);
  OPTIONAL_PTR(o_inter);
  OPTIONAL_PTR(prepared_next);
  if (prepared_next) REQUIRE_PTR(phi_q);
  if ((st = check_state_pair(d, S_prev, S_next)) != ARL2_OK) return st;
  const size_t need = ws_clean_pass_prepared(d);
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d);
  const size_t pb = prepared_bytes(d);
  const Range outs[5] = {{o, ab}, {o_intra, ab}, {o_inter, ab}, {S_next, state_bytes(d)},
                         {prepared_next, pb}};
  const Range ins[11] = {{q, ab},
                         {k, ab},
                         {v, ab},
                         {prepared, pb},
                         {phi_q, prepared_next ? phi_bytes(d) : 0},
                         {phi_k, phi_bytes(d)},
                         {phi_v, phi_bytes(d)},
                         {S_prev, state_bytes(d)},
                         {ws, need},
                         {beta, (size_t)d.B * d.H * d.T * 4},
                         {alpha, (size_t)d.B * d.H * 4}};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ARL2_E_ALIAS, "an output overlaps an input or the workspace");
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return fail(ARL2_E_ALIAS, "two outputs overlap");
  hipStream_t s = (hipStream_t)stream;
  if (arl2::use_mfma(d))
    return hip_status(arl2::mfma_clean_pass_prepared(d, q, k, v, prepared, phi_q, phi_k, phi_v,
                                                     beta, alpha, S_prev, S_next, prepared_next,
                                                     o, o_intra, o_inter, ws, s),
                      "clean pass");
  st = arl2_read_prepared(shape, q, k, v, prepared, o, o_intra, o_inter, ws, ws_bytes, stream);
  if (st != ARL2_OK) return st;
  st = do_commit(d, k, v, phi_k, phi_v, beta, alpha, S_prev, S_next, ws, s);
  if (st != ARL2_OK || !prepared_next) return st;
  return hip_status(
      arl2::generic_read_prepare(d, phi_q, S_next, static_cast<float*>(prepared_next), s),
      "read preparation");
}

arl2_status arl2_token_read(const arl2_shape* shape, const void* q, const void* k, const void* v,
                            const void* phi_q, const void* phi_k, const void* phi_v,
                            const float* beta, const float* S, void* o, void* o_intra,
                            void* o_inter, void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if ((st = require_d128_for_bf16(d, "token-level access")) != ARL2_OK) return st;
  st = check_token(d, q, k, v, phi_q, phi_k, phi_v, beta, nullptr, S, nullptr, o, o_intra,
                   o_inter, ws, ws_bytes);
  if (st != ARL2_OK) return st;
  return do_token(d, q, k, v, phi_q, phi_k, phi_v, beta, nullptr, S, nullptr, o, o_intra,
                  o_inter, ws, (hipStream_t)stream);
}

arl2_status arl2_token_clean_pass(const arl2_shape* shape, const void* q, const void* k,
                                  const void* v, const void* phi_q, const void* phi_k,
                                  const void* phi_v, const float* beta, const float* alpha,
                                  const float* S_prev, float* S_next, void* o, void* o_intra,
                                  void* o_inter, void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if ((st = require_d128_for_bf16(d, "token-level access")) != ARL2_OK) return st;
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S_next);
  if ((st = check_state_pair(d, S_prev, S_next)) != ARL2_OK) return st;
  st = check_token(d, q, k, v, phi_q, phi_k, phi_v, beta, alpha, S_prev, S_next, o, o_intra,
                   o_inter, ws, ws_bytes);
  if (st != ARL2_OK) return st;
  return do_token(d, q, k, v, phi_q, phi_k, phi_v, beta, alpha, S_prev, S_next, o, o_intra,
                  o_inter, ws, (hipStream_t)stream);
}

// ------------------------------------------------------------- training side

arl2_status arl2_intra_attn_backward(const arl2_shape* shape, const void* q, const void* k,
                                     const void* v, const void* o_intra, const float* lse,
                                     const void* d_o, void* dq, void* dk, void* dv,
                                     int32_t accumulate, void* ws, size_t ws_bytes,
                                     void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if ((st = require_d128_for_bf16(d, "the attention backward")) != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o_intra);
  REQUIRE_PTR(d_o);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  const size_t need = arl2::attn_backward_ws_bytes(d);
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d);
  OPTIONAL_PTR(lse);
  const size_t lb = (size_t)d.B * d.H * d.T * sizeof(float);
  const Range outs[3] = {{dq, ab}, {dk, ab}, {dv, ab}};
  const Range ins[7] = {{q, ab},   {k, ab},    {v, ab},  {o_intra, ab},
                        {d_o, ab}, {ws, need}, {lse, lb}};
  if ((st = check_disjoint(outs, 3, ins, 7)) != ARL2_OK) return st;
  if (overlap({lse, lb}, {ws, need})) return fail(ARL2_E_ALIAS, "lse overlaps the workspace");
  return hip_status(arl2::attn_backward(d, q, k, v, o_intra, lse, d_o, dq, dk, dv,
                                        accumulate != 0, ws, (hipStream_t)stream),
                    "attention backward");
}

arl2_status arl2_read_backward(const arl2_shape* shape, const void* q, const void* k,
                               const void* v, const void* phi_q, const float* S,
                               const void* o_intra, const float* lse, const void* d_o, void* dq,
                               void* dk, void* dv, float* dphi_q, float* dS, int32_t accumulate,
                               void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if ((st = require_d128_for_bf16(d, "the read backward")) != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_q);
  REQUIRE_PTR(S);
  REQUIRE_PTR(o_intra);
  REQUIRE_PTR(d_o);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  REQUIRE_PTR(dphi_q);
  REQUIRE_PTR(dS);
  const size_t need = arl2::read_backward_ws_bytes(d);
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d);
  const size_t pb = (size_t)d.H * d.D * d.D * 4;
  OPTIONAL_PTR(lse);
  const size_t lb = (size_t)d.B * d.H * d.T * sizeof(float);
  const Range outs[5] = {{dq, ab}, {dk, ab}, {dv, ab}, {dphi_q, pb}, {dS, state_bytes(d)}};
  const Range ins[9] = {{q, ab},       {k, ab},   {v, ab},   {phi_q, phi_bytes(d)},
                        {S, state_bytes(d)}, {o_intra, ab}, {d_o, ab}, {ws, need}, {lse, lb}};
  if ((st = check_disjoint(outs, 5, ins, 9)) != ARL2_OK) return st;
  if (overlap({lse, lb}, {ws, need})) return fail(ARL2_E_ALIAS, "lse overlaps the workspace");
  return hip_status(arl2::read_backward(d, q, k, v, phi_q, S, o_intra, lse, d_o, dq, dk, dv,
                                        dphi_q, dS, accumulate != 0, ws, (hipStream_t)stream),
                    "read backward");
}

arl2_status arl2_commit_backward(const arl2_shape* shape, const void* k, const void* v,
                                 const void* phi_k, const void* phi_v, const float* beta,
                                 const float* alpha, const float* S_prev, const float* dS_next,
                                 void* dk, void* dv, float* dphi_k, float* dphi_v, float* dbeta,
                                 float* dalpha, float* dS_prev, int32_t accumulate, void* ws,
                                 size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if ((st = require_d128_for_bf16(d, "the commit backward")) != ARL2_OK) return st;
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_k);
  REQUIRE_PTR(phi_v);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S_prev);
  REQUIRE_PTR(dS_next);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  REQUIRE_PTR(dphi_k);
  REQUIRE_PTR(dphi_v);
  REQUIRE_PTR(dbeta);
  REQUIRE_PTR(dalpha);
  REQUIRE_PTR(dS_prev);
  const size_t need = arl2::commit_backward_ws_bytes(d);
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d), sb = state_bytes(d);
  const size_t pb = (size_t)d.H * d.D * d.D * 4;
  const size_t bb = (size_t)d.B * d.H * d.T * 4, gb = (size_t)d.B * d.H * 4;
  const Range outs[7] = {{dk, ab},     {dv, ab},     {dphi_k, pb}, {dphi_v, pb},
                         {dbeta, bb},  {dalpha, gb}, {dS_prev, sb}};
  const Range ins[9] = {{k, ab},          {v, ab},       {phi_k, phi_bytes(d)},
                        {phi_v, phi_bytes(d)}, {beta, bb}, {alpha, gb},
                        {S_prev, sb},     {dS_next, sb}, {ws, need}};
  if ((st = check_disjoint(outs, 7, ins, 9)) != ARL2_OK) return st;
  return hip_status(arl2::commit_backward(d, k, v, phi_k, phi_v, beta, alpha, S_prev, dS_next, dk,
                                          dv, dphi_k, dphi_v, dbeta, dalpha, dS_prev,
                                          accumulate != 0, ws, (hipStream_t)stream),
                    "commit backward");
}

arl2_status arl2_state_scan(const arl2_shape* shape, int32_t n_frames, const void* k,
                            const void* v, const void* phi_k, const void* phi_v,
                            const float* beta, const float* alpha, const float* S0,
                            float* states, void* ws, size_t ws_bytes, void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  if (n_frames < 1) return fail(ARL2_E_SHAPE, "n_frames must be >= 1 (got %d)", n_frames);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(phi_k);
  REQUIRE_PTR(phi_v);
  REQUIRE_PTR(beta);
  REQUIRE_PTR(alpha);
  REQUIRE_PTR(S0);
  REQUIRE_PTR(states);
  const size_t need = ws_commit(d);
  if ((st = check_ws(ws, ws_bytes, need)) != ARL2_OK) return st;
  const size_t ab = arl2::act_bytes(d), sb = state_bytes(d);
  const size_t F = (size_t)n_frames;
  const Range outs[1] = {{states, (F + 1) * sb}};
  const Range ins[8] = {{k, F * ab},
                        {v, F * ab},
                        {phi_k, phi_bytes(d)},
                        {phi_v, phi_bytes(d)},
                        {beta, F * d.B * d.H * d.T * 4},
                        {alpha, F * d.B * d.H * 4},
                        {S0, sb},
                        {ws, need}};
  if ((st = check_disjoint(outs, 1, ins, 8)) != ARL2_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const size_t sn = sb / 4;
  if ((st = hip_status(arl2::copy_state(S0, states, sn, s), "state copy")) != ARL2_OK) return st;
  for (size_t f = 0; f < F; ++f) {
    st = do_commit(d, static_cast<const char*>(k) + f * ab, static_cast<const char*>(v) + f * ab,
                   phi_k, phi_v, beta + f * d.B * d.H * d.T, alpha + f * d.B * d.H,
                   states + f * sn, states + (f + 1) * sn, ws, s);
    if (st != ARL2_OK) return st;
  }
  return ok();
}

arl2_status arl2_fullkv_attn(const arl2_shape* shape, const void* q, const void* k_cache,
                             const void* v_cache, int64_t n_kv, int64_t kv_capacity, void* o,
                             void* stream) {
  arl2::Dims d;
  arl2_status st = check_shape(shape, &d);
  if (st != ARL2_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(o);
  if (n_kv < 1 || n_kv > kv_capacity)
    return fail(ARL2_E_SHAPE, "need 1 <= n_kv <= kv_capacity (got %lld, %lld)", (long long)n_kv,
                (long long)kv_capacity);
  const double cache_elems = (double)d.B * d.H * (double)kv_capacity * d.D;
  if (cache_elems >= 2147483648.0 * 64.0 || n_kv >= 2147483647LL)
    return fail(ARL2_E_SHAPE, "KV cache too large");
  const size_t ab = arl2::act_bytes(d);
  const size_t cb = (size_t)cache_elems * (d.bf16 ? 2 : 4);
  if (overlap({o, ab}, {q, ab}) || overlap({o, ab}, {k_cache, cb}) || overlap({o, ab}, {v_cache, cb}))
    return fail(ARL2_E_ALIAS, "o overlaps an input");
  return hip_status(run_attention(d, q, k_cache, v_cache, o, n_kv, kv_capacity, (hipStream_t)stream),
                    "full-KV attention");
}

}  // extern "C"
