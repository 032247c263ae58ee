// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace arl2 {

// Validated problem size, as the launchers see it.
struct Dims {
  int B, H, T, D;
  bool bf16;     // activations and Phi maps in bfloat16 (else float32)
  float scale;   // softmax temperature, already resolved (never 0)
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline size_t act_bytes(const Dims& d) {
  return (size_t)d.B * d.H * d.T * d.D * (d.bf16 ? 2 : 4);
}

// Generic (scalar-FMA) implementations, any supported D, either dtype. The
// MFMA implementations take over for bf16 at D = 128.
hipError_t generic_feature_map(const Dims& d, const void* x, const void* phi,
                               void* out, bool normalize, hipStream_t s);
hipError_t generic_attention(const Dims& d, const void* q, const void* k,
                             const void* v, void* o, int64_t n_kv,
                             int64_t kv_cap, hipStream_t s);
hipError_t generic_inter_read(const Dims& d, const void* q_prime,
                              const float* S, const void* o_intra, void* o,
                              void* o_inter, hipStream_t s);
size_t generic_state_commit_ws_bytes(const Dims& d);
hipError_t generic_state_commit(const Dims& d, const void* k_prime,
                                const void* v_prime, const float* beta,
                                const float* alpha, const float* S_prev,
                                float* S_next, void* ws, hipStream_t s);

// Up to three feature maps of one shape in one launch.
struct FeatureMapJob {
  const void* x;
  const void* phi;
  void* out;
  bool normalize;
  float* norms = nullptr;   // first job only, with normalize: each row's norm before the floor
};
hipError_t mfma_feature_maps(const Dims& d, const FeatureMapJob* jobs, int n_jobs, hipStream_t s);
hipError_t mfma_feature_map(const Dims& d, const void* x, const void* phi,
                            void* out, bool normalize, hipStream_t s);
hipError_t mfma_attention(const Dims& d, const void* q, const void* k,
                          const void* v, void* o, int64_t n_kv, int64_t kv_cap,
                          hipStream_t s);
// Intra-frame attention that also writes each row's log-sum-exp of the
// scaled scores (natural log, fp32 [B, H, T]).
hipError_t mfma_attention_lse(const Dims& d, const void* q, const void* k, const void* v,
                              void* o, float* lse, hipStream_t s);
hipError_t mfma_inter_read(const Dims& d, const void* q_prime, const float* S,
                           const void* o_intra, void* o, void* o_inter,
                           hipStream_t s);
// Fused read (bf16, D = 128): M = Phi_q S per head into `ws`, then the
// attention kernel with the epilogue O = O_intra + Q M (the split read's
// workspace follows M).
size_t mfma_read_ws_bytes(const Dims& d);
// Prepared reads: M^T = (Phi_q S)^T once per frame, then attention + Q M.
hipError_t mfma_read_prepare(const Dims& d, const void* phi_q, const float* S, void* mt,
                             hipStream_t s);
// With a workspace of mfma_read_prepared_ws_bytes (0: never used for this
// shape), shapes whose grid would leave compute units idle split key ranges
// over one workgroup per compute unit; ws may be null (plain grid).
size_t mfma_read_prepared_ws_bytes(const Dims& d);
hipError_t mfma_read_prepared(const Dims& d, const void* q, const void* k, const void* v,
                              const void* mt, void* o, void* o_intra, void* o_inter, void* ws,
                              size_t ws_bytes, hipStream_t s);
// Clean pass from a prepared map in one launch: the fused read's workgroups
// plus the column-split commit's (four per (b, h), no workspace), which also
// form the map of S_next into mt_next when mt_next is given (phi_q then
// required). The workspace argument is unused.
hipError_t mfma_clean_pass_prepared(const Dims& d, const void* q, const void* k, const void* v,
                                    const void* mt, const void* phi_q, const void* phi_k,
                                    const void* phi_v, const float* beta, const float* alpha,
                                    const float* S_prev, float* S_next, void* mt_next, void* o,
                                    void* o_intra, void* o_inter, void* ws, hipStream_t s);
// float32 / generic: M = Phi_q S (fp32, row-major per head).
hipError_t generic_read_prepare(const Dims& d, const void* phi_q, const float* S, float* m,
                                hipStream_t s);
hipError_t mfma_read(const Dims& d, const void* q, const void* k, const void* v,
                     const void* phi_q, const float* S, void* o, void* o_intra, void* o_inter,
                     void* ws, hipStream_t s);
// Fused commit (bf16, D = 128) from the raw K, V: feature maps, row norm and
// the gated delta update in one launch, one workgroup per (b, h, 32 state
// columns, token part); the workspace holds each part's fp32 sum and one
// counter per column block (mfma_commit_ws_bytes; the clean pass, whose commit
// takes two token parts, needs mfma_clean_commit_ws_bytes).
size_t mfma_commit_ws_bytes(const Dims& d);
size_t mfma_clean_commit_ws_bytes(const Dims& d);
hipError_t mfma_commit(const Dims& d, const void* k, const void* v, const void* phi_k,
                       const void* phi_v, const float* beta, const float* alpha,
                       const float* S_prev, float* S_next, void* ws, hipStream_t s);
size_t mfma_state_commit_ws_bytes(const Dims& d);
hipError_t mfma_state_commit(const Dims& d, const void* k_prime,
                             const void* v_prime, const float* beta,
                             const float* alpha, const float* S_prev,
                             float* S_next, void* ws, hipStream_t s);

// Token-level access (the ablated alternative to frame-level access): from
// mapped Q', K', V' and o_intra, o = o_intra + o_inter with token t reading the
// state updated by the frame's earlier tokens from S_prev; with S_next given,
// the end state S_T commits S_next = alpha S_prev + (S_T - S_prev).
size_t token_level_scan_ws_bytes(const Dims& d);
hipError_t token_level_scan(const Dims& d, const void* q_prime, const void* k_prime,
                            const void* v_prime, const float* beta, const float* S_prev,
                            const float* alpha, float* S_next, const void* o_intra, void* o,
                            void* o_inter, void* ws, hipStream_t s);

// Training side: exact derivatives of the read and of the commit (accumulate:
// add every gradient to its output instead of overwriting it).
size_t attn_backward_ws_bytes(const Dims& d);
size_t read_backward_ws_bytes(const Dims& d);
size_t commit_backward_ws_bytes(const Dims& d);
// lse: the rows' log-sum-exp from the forward (natural log), or null to
// compute it here.
hipError_t attn_backward(const Dims& d, const void* q, const void* k, const void* v,
                         const void* o_intra, const float* lse, const void* d_o, void* dq,
                         void* dk, void* dv, bool accumulate, void* ws, hipStream_t s);
hipError_t read_backward(const Dims& d, const void* q, const void* k, const void* v,
                         const void* phi_q, const float* S, const void* o_intra, const float* lse,
                         const void* d_o, void* dq, void* dk, void* dv, float* dphi_q, float* dS,
                         bool accumulate, void* ws, hipStream_t s);
// float32 shapes: the rows' log-sum-exp of scale Q K^T (natural log).
hipError_t attn_lse_f32(const Dims& d, const void* q, const void* k, float* lse, hipStream_t s);
hipError_t commit_backward(const Dims& d, const void* k, const void* v, const void* phi_k,
                           const void* phi_v, const float* beta, const float* alpha,
                           const float* S_prev, const float* dS_next, void* dk, void* dv,
                           float* dphi_k, float* dphi_v, float* dbeta, float* dalpha,
                           float* dS_prev, bool accumulate, void* ws, hipStream_t s);
hipError_t copy_state(const float* src, float* dst, size_t n, hipStream_t s);

// The library's fixed device scratch (noalloc.hip): its size, and the device
// address of the current device's copy (looked up on first use per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

inline bool use_mfma(const Dims& d) { return d.bf16 && d.D == 128; }

}  // namespace arl2
