/*
 * arl2.h - C ABI of the ARL2 hybrid attention step on MI355X (gfx950).
 *
 * The step follows "Attend Locally, Remember Linearly: Linear Attention as
 * Cross-Frame Memory for Autoregressive Video Diffusion" (Li, Shah, Shang),
 * technical summary on gist.science (Chinese, Portuguese and French versions):
 *
 *   §2.1 Hybrid attention decomposition
 *        intra-frame branch: bidirectional softmax over the frame's T tokens
 *          with the frozen Q, K, V (no mask);
 *        inter-frame branch: per-head grouped 1x1 feature maps
 *          Q' = Q Phi_q[h], K' = rownorm(K Phi_k[h]), V' = V Phi_v[h];
 *          read   O_inter = Q' S_{N-1};
 *          update S_N = alpha_N S_{N-1} + K'^T diag(beta_N) (V' - K' S_{N-1}).
 *   §2.2 Memory state management
 *        frame-level access: every token of frame N reads the same S_{N-1};
 *        clean-pass update: denoising reads never write S; S is written once
 *          per frame, after the frame's clean pass.
 *
 * The printed update lacks the transpose on the first K'; the row-vector read
 * Q'S fixes it as written above. The residual uses the undecayed S_{N-1} as
 * printed; alpha is one scalar per (video, head, frame), beta one per (video,
 * head, token); K' rows are normalised as x / max(||x||_2, 1e-12) after
 * Phi_k; O = O_intra + O_inter.
 *
 * Conventions shared by every entry point
 *   - Activations Q, K, V, Q', K', V', O are contiguous [B, H, T, D] tensors
 *     of the shape's act_dtype (float32 or bfloat16), D contiguous.
 *   - Phi maps are contiguous [H, D_in, D_out] of act_dtype: X' = X Phi[h].
 *   - The state S is always float32, contiguous [B, H, D_k, D_v], D_v
 *     contiguous.
 *   - beta is float32 [B, H, T]; alpha is float32 [B, H].
 *   - Every pointer is a device pointer, 16-byte aligned, owned by the
 *     caller. The library allocates no memory. Scratch memory comes from the
 *     caller's workspace (ws, ws_bytes), sized by arl2_workspace_bytes().
 *     Its only state between calls is a process-wide host counter that gives
 *     each call of the split-key read and of the attention backward's split
 *     a distinct tag for its workspace block counters (so that a workspace
 *     needs no clearing); results never depend on the counter's value.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued asynchronously on it; stream order alone makes a
 *     read of frame N+1 see the S_N written by frame N's commit.
 *   - Each call validates every argument on the host first; on error nothing
 *     is enqueued and a status other than ARL2_OK is returned, with detail
 *     text available from arl2_last_error() on the calling thread.
 *     ARL2_E_HIP reports a launch failure (hipGetLastError after launch).
 *   - Supported shapes: act_dtype ARL2_F32 or ARL2_BF16 with D in
 *     {16, 32, 64, 128}; any T >= 1, B >= 1, H >= 1 with B*H*T*D < 2^31.
 *     bf16 at D = 128 runs on the MFMA kernels, other shapes on plain
 *     per-thread kernels. Token-level access and the training calls (from
 *     arl2_intra_attn_lse on) take bf16 only at D = 128 (ARL2_E_SHAPE
 *     otherwise).
 *   - Results are deterministic: no floating-point atomics, fixed reduction
 *     order, so identical inputs give bit-identical outputs.
 */
#ifndef ARL2_H
#define ARL2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARL2_ABI_VERSION 2

typedef enum arl2_status {
  ARL2_OK = 0,
  ARL2_E_NULL = 1,      /* a required pointer is NULL                        */
  ARL2_E_SHAPE = 2,     /* B, H, T, D out of range or unsupported            */
  ARL2_E_DTYPE = 3,     /* act_dtype not ARL2_F32 / ARL2_BF16                */
  ARL2_E_LAYOUT = 4,    /* a pointer is not 16-byte aligned                  */
  ARL2_E_ALIAS = 5,     /* S_prev and S_next overlap, or an output aliases   */
  ARL2_E_WORKSPACE = 6, /* workspace NULL or smaller than required           */
  ARL2_E_HIP = 7        /* the HIP runtime reported an error                 */
} arl2_status;

typedef enum arl2_dtype { ARL2_F32 = 0, ARL2_BF16 = 1 } arl2_dtype;

typedef struct arl2_shape {
  int32_t B;            /* videos (independent streams)                      */
  int32_t H;            /* heads                                             */
  int32_t T;            /* tokens per frame                                  */
  int32_t D;            /* head dimension (d_k = d_v = D)                    */
  int32_t act_dtype;    /* arl2_dtype of activations and Phi maps            */
  float softmax_scale;  /* intra-frame softmax temperature; 0 => 1/sqrt(D)   */
} arl2_shape;

/* Operations whose workspace size arl2_workspace_bytes() reports. */
typedef enum arl2_op {
  ARL2_OP_READ = 0,
  ARL2_OP_CLEAN_PASS = 1,
  ARL2_OP_COMMIT = 2,
  ARL2_OP_STATE_COMMIT = 3,
  ARL2_OP_READ_PREPARED = 4,
  ARL2_OP_CLEAN_PASS_PREPARED = 5,
  ARL2_OP_TOKEN_LEVEL = 6,
  ARL2_OP_INTRA_ATTN_BACKWARD = 7,
  ARL2_OP_READ_BACKWARD = 8,
  ARL2_OP_COMMIT_BACKWARD = 9
} arl2_op;

/* ------------------------------------------------------------------------
 * Steps of the hybrid attention layer, one entry point each.
 * ------------------------------------------------------------------------ */

/* Per-head grouped 1x1 feature map (§2.1, "adaptation" of Q, K, V):
 *   x_out[b,h,t,:] = x[b,h,t,:] Phi[h]          (Phi [H, D_in, D_out])
 * and, when normalize_rows != 0, each output row is divided by
 * max(||row||_2, 1e-12) (the key map). x and x_out are [B,H,T,D] act_dtype
 * and must not overlap. */
arl2_status arl2_feature_map(const arl2_shape* shape, const void* x,
                             const void* phi, void* x_out,
                             int32_t normalize_rows, void* stream);

/* Intra-frame branch (§2.1): per (b,h), the bidirectional softmax over the
 * frame's T tokens, no mask:
 *   o_intra = softmax(Q K^T * scale) V
 * q, k, v, o_intra are [B,H,T,D] act_dtype; o_intra must not overlap the
 * inputs. Accumulation in float32. */
arl2_status arl2_intra_attn(const arl2_shape* shape, const void* q,
                            const void* k, const void* v, void* o_intra,
                            void* stream);

/* Inter-frame read (§2.1 output equation, §2.2 frame-level access):
 *   o = o_intra + Q' S            (o = Q' S when o_intra is NULL)
 * q_prime, o_intra and o are [B,H,T,D] act_dtype; S is float32 [B,H,D,D]
 * and is only read. o may equal o_intra (in-place add); it must not overlap
 * q_prime or S. */
arl2_status arl2_inter_read(const arl2_shape* shape, const void* q_prime,
                            const float* S, const void* o_intra, void* o,
                            void* stream);

/* State commit (§2.1 update equation), from already mapped K', V':
 *   R      = V' - K' S_prev
 *   S_next = alpha * S_prev + K'^T diag(beta) R
 * k_prime, v_prime [B,H,T,D] act_dtype (K' rows expected unit length),
 * beta float32 [B,H,T], alpha float32 [B,H], S_prev and S_next float32
 * [B,H,D,D]. S_prev and S_next must not overlap (ARL2_E_ALIAS): the state is
 * double-buffered and S_prev is left untouched. Needs
 * arl2_workspace_bytes(shape, ARL2_OP_STATE_COMMIT) bytes of workspace. */
arl2_status arl2_state_commit(const arl2_shape* shape, const void* k_prime,
                              const void* v_prime, const float* beta,
                              const float* alpha, const float* S_prev,
                              float* S_next, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * The pass-level API: denoising reads versus the clean-pass commit (§2.2).
 * ------------------------------------------------------------------------ */

/* Denoising-step read: Q' = Q Phi_q[h], o_intra = softmax(QK^T*scale)V,
 * o = o_intra + Q' S. S is const: a read never writes the state.
 * o_intra and o_inter are optional extra outputs (NULL to skip) holding the
 * two branches separately. Needs arl2_workspace_bytes(shape, ARL2_OP_READ)
 * (bf16: the map of arl2_read_prepare, then the split read's workspace of
 * arl2_read_prepared when the shape takes it). */
arl2_status arl2_read(const arl2_shape* shape, const void* q, const void* k,
                      const void* v, const void* phi_q, const float* S,
                      void* o, void* o_intra, void* o_inter, void* ws,
                      size_t ws_bytes, void* stream);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): arl2_read without
 * a workspace argument. Same meaning, arguments and errors as arl2_read; its
 * scratch memory (the map M = Phi_q S on bf16 D = 128 shapes, where the read
 * then always runs on the plain grid; Q' and o_intra on other shapes) is a
 * fixed device array inside the library, ARL2_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on a GPU until the process ends. A shape that
 * needs more (bf16 D = 128: B*H*D*D*2 bytes; other shapes: 2*B*H*T*D*elem
 * bytes, each rounded up to 256) returns ARL2_E_WORKSPACE before anything is
 * enqueued. The call itself allocates nothing. Every call on one GPU uses
 * that GPU's one array (each call rewrites all it reads, so no state carries
 * over): calls that overlap in time on one GPU (different streams, or
 * different host threads) race on it and must be serialised by the caller. */
#define ARL2_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
arl2_status arl2_read_noalloc(const arl2_shape* shape, const void* q,
                              const void* k, const void* v,
                              const void* phi_q, const float* S, void* o,
                              void* o_intra, void* o_inter, void* stream);

/* Read preparation. Every token and every pass of a frame reads the same
 * S_{N-1} (frame-level access, §2.2), and Q' S = Q (Phi_q S), so the map
 * M = Phi_q[h] S[b,h] (D x D per head) can be formed once per frame, after the
 * commit that produced S, and reused by all of the frame's reads.
 * arl2_read_prepare writes M into `prepared` (caller-owned device memory of
 * arl2_prepared_bytes(shape) bytes; its layout is private to the library:
 * bf16 M^T for bf16 shapes, fp32 M for float32 shapes). S is only read. */
size_t arl2_prepared_bytes(const arl2_shape* shape);
arl2_status arl2_read_prepare(const arl2_shape* shape, const void* phi_q,
                              const float* S, void* prepared, void* stream);

/* Denoising-step read from a prepared map: o = softmax(Q K^T * scale) V + Q M,
 * identical in meaning to arl2_read with the (Phi_q, S) the map was prepared
 * from. o_intra / o_inter are optional extra outputs.
 * Workspace: float32 shapes need arl2_workspace_bytes(shape,
 * ARL2_OP_READ_PREPARED) bytes. For bf16 shapes it is optional: with ws NULL
 * the read runs one workgroup per 128 queries of a head; with a workspace of
 * at least that many bytes (a non-NULL ws smaller than that is
 * ARL2_E_WORKSPACE), shapes whose query blocks would leave many compute units
 * idle (too few blocks, or a last round of blocks that fills few units) and
 * whose frames are long enough (the size is 0 for other shapes) split each
 * block's keys over several workgroups and merge their partial softmax
 * results in key order. Results of the two agree to fp32 rounding order; each is
 * deterministic. The workspace needs no clearing (its block counters carry a
 * per-call tag and are left at zero); calls that share a workspace must not
 * overlap in time. */
arl2_status arl2_read_prepared(const arl2_shape* shape, const void* q,
                               const void* k, const void* v,
                               const void* prepared, void* o, void* o_intra,
                               void* o_inter, void* ws, size_t ws_bytes,
                               void* stream);

/* Commit only (the clean pass's state write without its read):
 * K' = rownorm(K Phi_k[h]), V' = V Phi_v[h], then arl2_state_commit.
 * Needs arl2_workspace_bytes(shape, ARL2_OP_COMMIT). On bf16 shapes (D = 128)
 * one launch: each (video, head, 32 state columns) is split over 2 to 8 token
 * parts (at most as many as fill 256 compute units, then the fewest that give
 * each wave the same number of 32-token slices; 4 at 1 video x 12 heads x 1560
 * tokens) whose fp32 products the last part to finish adds in part order, so
 * results are deterministic. The workspace holds those products and one
 * counter per column block; the counters carry a per-call tag and are left at
 * zero, so the workspace needs no clearing, and calls that share a workspace
 * must not overlap in time. */
arl2_status arl2_commit(const arl2_shape* shape, const void* k, const void* v,
                        const void* phi_k, const void* phi_v,
                        const float* beta, const float* alpha,
                        const float* S_prev, float* S_next, void* ws,
                        size_t ws_bytes, void* stream);

/* Clean pass: the read of arl2_read against S_prev, then the commit of
 * arl2_commit from the same K, V into S_next. Needs
 * arl2_workspace_bytes(shape, ARL2_OP_CLEAN_PASS). */
arl2_status arl2_clean_pass(const arl2_shape* shape, const void* q,
                            const void* k, const void* v, const void* phi_q,
                            const void* phi_k, const void* phi_v,
                            const float* beta, const float* alpha,
                            const float* S_prev, float* S_next, void* o,
                            void* o_intra, void* o_inter, void* ws,
                            size_t ws_bytes, void* stream);

/* Clean pass from a prepared map (§2.2: the frame's last pass reads S_{N-1}
 * like every other pass, then writes S_N once): o = softmax(Q K^T * scale) V +
 * Q M with the map M of S_prev in `prepared` (arl2_read_prepare), and S_next
 * from K, V, beta, alpha and S_prev as in arl2_commit. When prepared_next is
 * not NULL it also receives the map of S_next (what arl2_read_prepare(phi_q,
 * S_next) would write; phi_q is then required), ready for the next frame's
 * reads; it must be a different buffer from `prepared`. On bf16 shapes (D =
 * 128) the read and the commit run in one launch, the commit (as in
 * arl2_commit, also forming the next map) on the compute units the read leaves
 * idle. Needs arl2_workspace_bytes(shape,
 * ARL2_OP_CLEAN_PASS_PREPARED) bytes of workspace. Outputs must not overlap
 * each other, the inputs or the workspace. */
arl2_status arl2_clean_pass_prepared(const arl2_shape* shape, const void* q,
                                     const void* k, const void* v,
                                     const void* prepared, const void* phi_q,
                                     const void* phi_k, const void* phi_v,
                                     const float* beta, const float* alpha,
                                     const float* S_prev, float* S_next,
                                     void* prepared_next, void* o, void* o_intra,
                                     void* o_inter, void* ws, size_t ws_bytes,
                                     void* stream);

/* ------------------------------------------------------------------------
 * Token-level access: the alternative to frame-level access that the
 * summary's ablation (§4) compares against and finds worse. The pages do not
 * define it further; these calls take the plainest reading: within a pass,
 * token t reads the state left by the frame's earlier tokens, starting from
 * S_{N-1},
 *   o_inter_t = q'_t S_{t-1},
 *   S_t = S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1})   (S_0 = S_{N-1}),
 * and o = o_intra + o_inter with o_intra the intra-frame softmax as in
 * arl2_read. A read discards S_T; the clean pass commits
 *   S_next = alpha * S_prev + (S_T - S_prev)
 * (the frame's gate applied once, as in the frame-level update). With T = 1
 * both calls equal their frame-level counterparts. On bf16 shapes the scan runs
 * in chunks of 64 tokens (the closed form of the recurrence over a chunk,
 * formed by a triangular solve); the state is carried in float32 and enters
 * the chunk products as bfloat16. Both calls need arl2_workspace_bytes(shape,
 * ARL2_OP_TOKEN_LEVEL) bytes of workspace; outputs must not overlap each
 * other, the inputs or the workspace.
 * ------------------------------------------------------------------------ */

/* Denoising-step read under token-level access. S (float32 [B,H,D,D]) is
 * only read. o_intra / o_inter are optional extra outputs. */
arl2_status arl2_token_read(const arl2_shape* shape, const void* q,
                            const void* k, const void* v, const void* phi_q,
                            const void* phi_k, const void* phi_v,
                            const float* beta, const float* S, void* o,
                            void* o_intra, void* o_inter, void* ws,
                            size_t ws_bytes, void* stream);

/* Clean pass under token-level access: the read above against S_prev, and
 * the commit of its end state into S_next (which must not overlap S_prev). */
arl2_status arl2_token_clean_pass(const arl2_shape* shape, const void* q,
                                  const void* k, const void* v,
                                  const void* phi_q, const void* phi_k,
                                  const void* phi_v, const float* beta,
                                  const float* alpha, const float* S_prev,
                                  float* S_next, void* o, void* o_intra,
                                  void* o_inter, void* ws, size_t ws_bytes,
                                  void* stream);

/* ------------------------------------------------------------------------
 * Training side. The summary's two-stage distillation (§2.3) fine-tunes the
 * hybrid model end to end and prints no backward pass; these calls compute
 * the exact derivatives of the forward step defined above.
 *   Gradient outputs: activation gradients act_dtype [B,H,T,D]; map gradients
 *   float32 [H,D,D], summed over the B videos and the tokens; state gradients
 *   float32 [B,H,D,D]; dbeta float32 [B,H,T]; dalpha float32 [B,H].
 *   accumulate != 0 adds every gradient to what its output holds (so passes
 *   and frames sum in place); 0 overwrites. Outputs must not overlap each
 *   other, the inputs or the workspace. Reductions run in a fixed order:
 *   identical inputs give bit-identical gradients.
 * ------------------------------------------------------------------------ */

/* Intra-frame attention for training: arl2_intra_attn's o_intra, and lse =
 * each row's log-sum-exp of the scaled scores, lse[b,h,t] = log sum_j
 * exp(scale q_t . k_j) (natural log, float32 [B,H,T], caller-owned), which the
 * backward calls below take so as not to recompute Q K^T for it. */
arl2_status arl2_intra_attn_lse(const arl2_shape* shape, const void* q,
                                const void* k, const void* v, void* o_intra,
                                float* lse, void* stream);

/* Backward of the intra-frame softmax (arl2_intra_attn): from the forward's
 * o_intra and d_o = dL/dO_intra,
 *   P = softmax(Q K^T * scale), dV = P^T dO, dP = dO V^T,
 *   dZ = P * (dP - rowsum(dO * O_intra)), dQ = scale dZ K, dK = scale dZ^T Q.
 * lse: NULL, or the rows' log-sum-exp from arl2_intra_attn_lse on the same
 * q and k (then P = exp(scale Q K^T - lse) without a pass to find it).
 * Needs arl2_workspace_bytes(shape, ARL2_OP_INTRA_ATTN_BACKWARD). On shapes
 * with fewer than 512 blocks of 128 rows (bf16, d = 128) the workspace also
 * holds per-key-block partial sums and counters: it needs no clearing (the
 * counters carry a per-call tag and are left at zero), and calls that share a
 * workspace must not run concurrently. */
arl2_status arl2_intra_attn_backward(const arl2_shape* shape, const void* q,
                                     const void* k, const void* v,
                                     const void* o_intra, const float* lse,
                                     const void* d_o, void* dq, void* dk,
                                     void* dv, int32_t accumulate, void* ws,
                                     size_t ws_bytes, void* stream);

/* Backward of a read, O = softmax(Q K^T * scale) V + (Q Phi_q) S, from the
 * read's o_intra and d_o = dL/dO: dq, dk, dv, dphi_q and dS, with
 *   dQ += dO (Phi_q S)^T, dS = (Q Phi_q)^T dO, dPhi_q = sum_b Q^T dO S^T.
 * lse as in arl2_intra_attn_backward (NULL or from arl2_intra_attn_lse).
 * Needs arl2_workspace_bytes(shape, ARL2_OP_READ_BACKWARD) (with the same
 * sharing rule as arl2_intra_attn_backward's). */
arl2_status arl2_read_backward(const arl2_shape* shape, const void* q,
                               const void* k, const void* v, const void* phi_q,
                               const float* S, const void* o_intra,
                               const float* lse, const void* d_o, void* dq,
                               void* dk, void* dv, float* dphi_q, float* dS,
                               int32_t accumulate, void* ws, size_t ws_bytes,
                               void* stream);

/* Backward of the commit (arl2_commit) from dS_next = dL/dS_next = G, with
 * K' = rownorm(K Phi_k), V' = V Phi_v, R = V' - K' S_prev:
 *   dalpha = <S_prev, G>, dS_prev = alpha G - K'^T diag(beta) K' G,
 *   dbeta = rowsum((K' G) * R), dV' = diag(beta) K' G,
 *   dK' = diag(beta) (R G^T - K' G S_prev^T),
 * then through the row normalisation and the maps (dK, dV, dPhi_k, dPhi_v).
 * Needs arl2_workspace_bytes(shape, ARL2_OP_COMMIT_BACKWARD). */
arl2_status arl2_commit_backward(const arl2_shape* shape, const void* k,
                                 const void* v, const void* phi_k,
                                 const void* phi_v, const float* beta,
                                 const float* alpha, const float* S_prev,
                                 const float* dS_next, void* dk, void* dv,
                                 float* dphi_k, float* dphi_v, float* dbeta,
                                 float* dalpha, float* dS_prev,
                                 int32_t accumulate, void* ws, size_t ws_bytes,
                                 void* stream);

/* Clean-state scan (the clean states ahead of the reads, as training with
 * clean frames needs them): the states S_0..S_F that n_frames frames' clean
 * passes commit, arl2_commit frame after frame, no reads. k, v:
 * [n_frames,B,H,T,D] act_dtype; beta [n_frames,B,H,T]; alpha [n_frames,B,H];
 * S0 [B,H,D,D]; states [n_frames+1,B,H,D,D] float32 receives S0 then every
 * committed state. Needs arl2_workspace_bytes(shape, ARL2_OP_COMMIT). */
arl2_status arl2_state_scan(const arl2_shape* shape, int32_t n_frames,
                            const void* k, const void* v, const void* phi_k,
                            const void* phi_v, const float* beta,
                            const float* alpha, const float* S0, float* states,
                            void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Comparator: the cross-frame softmax over a growing KV cache that the
 * recurrent state replaces (§1 of the summary: the cache grows with every
 * generated block).
 * ------------------------------------------------------------------------ */

/* o[b,h,t,:] = softmax(q[b,h,t,:] K_c^T * scale) V_c over the first n_kv
 * cached tokens of head (b,h). q, o: [B,H,T,D] act_dtype; k_cache, v_cache:
 * [B,H,kv_capacity,D] act_dtype; 1 <= n_kv <= kv_capacity. The caller appends
 * each frame's keys and values to the cache. */
arl2_status arl2_fullkv_attn(const arl2_shape* shape, const void* q,
                             const void* k_cache, const void* v_cache,
                             int64_t n_kv, int64_t kv_capacity, void* o,
                             void* stream);

/* ------------------------------------------------------------------------
 * Support calls.
 * ------------------------------------------------------------------------ */

/* Workspace bytes needed by `op` (an arl2_op) for this shape; 0 for an
 * invalid shape or op. */
size_t arl2_workspace_bytes(const arl2_shape* shape, int32_t op);

/* Static text naming a status code. */
const char* arl2_status_string(arl2_status status);

/* Detail text of the last error on the calling thread ("" if none). */
const char* arl2_last_error(void);

/* ARL2_ABI_VERSION of the built library. */
int32_t arl2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ARL2_H */
