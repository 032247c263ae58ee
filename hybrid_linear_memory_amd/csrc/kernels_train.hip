// Training-side kernels: the backward of the read and of the commit, and the
// clean-state scan over frames. The summary's two-stage distillation (§2.3)
// fine-tunes the hybrid model end to end; these compute the exact derivatives
// of the forward step:
//   read    O = softmax(Q K^T * scale) V + (Q Phi_q) S
//   commit  S_next = alpha S + K'^T diag(beta) (V' - K' S),
//           K' = rownorm(K Phi_k), V' = V Phi_v.
//
// Building blocks (bf16 on MFMA at d = 128; plain float32 loops otherwise):
//   nt_gemm   Y = X Bt^T per (b, h) with an elementwise epilogue
//   xty       C = X^T Y summed over tokens (and over videos for the maps'
//             gradients), in fixed-order chunk partials
//   row steps (the row normalisation, beta and the norm's backward): in the
//             epilogues of the products that feed them on MFMA, row kernels
//             on the float path
//   attention backward: per-row log-sum-exp and dO.O, then dK, dV (one
//             workgroup per key block; on small grids two, over the query
//             halves, the second adding the first's sums) and dQ (one per
//             query block), each recomputing the scores; no atomic
//             accumulation, so the gradients are deterministic.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "arl2_internal.h"
#include "mfma_common.h"

namespace arl2 {
namespace {

constexpr float kNormFloor = 1e-12f;          // row-norm floor of the key map

__device__ __forceinline__ float4 ld4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

template <typename Tx>
__device__ __forceinline__ float ldf(const Tx* p, size_t i) { return (float)p[i]; }
template <typename Tx>
__device__ __forceinline__ void stf(Tx* p, size_t i, float x) { p[i] = (Tx)x; }

// ---------------------------------------------------------------------------
// Epilogue of the GEMM-shaped steps: y = (z ? z - acc : acc), written to y32
// (float) and / or yx (activation type), added to what is there when
// accumulate is set.
// ---------------------------------------------------------------------------
struct Epi {
  const void* z;        // activation type, or float when z_f32
  int z_f32;
  float* y32;
  void* yx;
  int accumulate;
};

template <typename Tx>
__device__ __forceinline__ void epilogue(const Epi& ep, size_t idx, float acc) {
  float y = acc;
  if (ep.z) y = (ep.z_f32 ? static_cast<const float*>(ep.z)[idx]
                          : ldf(static_cast<const Tx*>(ep.z), idx)) - y;
  if (ep.y32) ep.y32[idx] = ep.accumulate ? ep.y32[idx] + y : y;
  if (ep.yx) {
    Tx* yx = static_cast<Tx*>(ep.yx);
    stf(yx, idx, ep.accumulate ? ldf(yx, idx) + y : y);
  }
}

// ---------------------------------------------------------------------------
// float32 building blocks (any D <= 128)
// ---------------------------------------------------------------------------

// Y[g][t][n] = sum_k X[gx][t][k] * B(n, k), B(n, k) = bt[gb][n][k] (or
// bt[gb][k][n] when bt_trans); gx = x_per_head ? g % H : g, same for gb.
__global__ void nt_gemm_f32_k(const float* __restrict__ x, const float* __restrict__ bt,
                              Epi ep, int rows, int D, int H, int x_per_head,
                              int bt_per_head, int bt_trans, long n_out) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_out) return;
  const int n = (int)(idx % D);
  const long gr = idx / D;
  const int t = (int)(gr % rows);
  const long g = gr / rows;
  const float* xr = x + ((x_per_head ? g % H : g) * rows + t) * (long)D;
  const float* bm = bt + (bt_per_head ? g % H : g) * (long)D * D;
  float acc = 0.f;
  for (int k = 0; k < D; ++k) acc = fmaf(xr[k], bt_trans ? bm[(long)k * D + n] : bm[(long)n * D + k], acc);
  epilogue<float>(ep, idx, acc);
}

// C[go][e][v] = base + delta * sum_{b} sum_t X[g][t][e] Y[g][t][v] with
// g = b * H + h over all b when sum_b (go = h), else g = go alone;
// base = gamma[go] * base_mat[go][e][v] when base_mat is given; added to C
// when accumulate.
__global__ void xty_f32_k(const float* __restrict__ x, const float* __restrict__ y,
                          float* __restrict__ out, const float* __restrict__ base_mat,
                          const float* __restrict__ gamma, float delta, int accumulate, int T,
                          int D, int B, int H, int sum_b, long n_out) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_out) return;
  const int v = (int)(idx % D);
  const int e = (int)((idx / D) % D);
  const long go = idx / ((long)D * D);
  float acc = 0.f;
  const int nb = sum_b ? B : 1;
  for (int b = 0; b < nb; ++b) {
    const long g = sum_b ? (long)b * H + go : go;
    const float* xg = x + g * (long)T * D;
    const float* yg = y + g * (long)T * D;
    for (int t = 0; t < T; ++t) acc = fmaf(xg[(long)t * D + e], yg[(long)t * D + v], acc);
  }
  float r = delta * acc;
  if (base_mat) r += gamma[go] * base_mat[idx];
  out[idx] = accumulate ? out[idx] + r : r;
}

// Per query row: lse = max + log(sum exp(s - max)) of s = scale q.k over the
// frame's keys, and dsum = dO . O_intra.
__global__ void attn_pre_f32_k(const float* __restrict__ q, const float* __restrict__ k,
                               const float* __restrict__ o, const float* __restrict__ d_o,
                               float* __restrict__ lse, float* __restrict__ dsum, int T, int D,
                               float scale, long n_rows) {
  const long r = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const long g = r / T;
  if (q) {                       // (without q: dsum only, lse given)
    const float* qr = q + r * D;
    const float* kg = k + g * (long)T * D;
    float m = -INFINITY;
    for (int j = 0; j < T; ++j) {
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(qr[e], kg[(long)j * D + e], s);
      m = fmaxf(m, s * scale);
    }
    float l = 0.f;
    for (int j = 0; j < T; ++j) {
      float s = 0.f;
      for (int e = 0; e < D; ++e) s = fmaf(qr[e], kg[(long)j * D + e], s);
      l += expf(s * scale - m);
    }
    lse[r] = m + logf(l);
  }
  if (d_o) {                     // (without d_o: lse only)
    float dd = 0.f;
    for (int e = 0; e < D; ++e) dd = fmaf(d_o[r * D + e], o[r * D + e], dd);
    dsum[r] = dd;
  }
}

// P_ij = exp(scale q_i.k_j - lse_i), dS_ij = P_ij (dO_i.v_j - dsum_i).
__device__ __forceinline__ void attn_pd_f32(const float* qi, const float* kj, const float* doi,
                                            const float* vj, int D, float scale, float lse_i,
                                            float dsum_i, float* p, float* ds) {
  float s = 0.f, dp = 0.f;
  for (int e = 0; e < D; ++e) {
    s = fmaf(qi[e], kj[e], s);
    dp = fmaf(doi[e], vj[e], dp);
  }
  *p = expf(s * scale - lse_i);
  *ds = *p * (dp - dsum_i);
}

// dQ[i][e] = scale sum_j dS_ij K[j][e]   (one thread per element)
__global__ void attn_dq_f32_k(const float* __restrict__ q, const float* __restrict__ k,
                              const float* __restrict__ v, const float* __restrict__ d_o,
                              const float* __restrict__ lse, const float* __restrict__ dsum,
                              float* __restrict__ dq, int T, int D, float scale, int accumulate,
                              long n_out) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_out) return;
  const int e = (int)(idx % D);
  const long r = idx / D;
  const long g = r / T;
  const float* kg = k + g * (long)T * D;
  const float* vg = v + g * (long)T * D;
  float acc = 0.f;
  for (int j = 0; j < T; ++j) {
    float p, ds;
    attn_pd_f32(q + r * D, kg + (long)j * D, d_o + r * D, vg + (long)j * D, D, scale, lse[r],
                dsum[r], &p, &ds);
    acc = fmaf(ds, kg[(long)j * D + e], acc);
  }
  acc *= scale;
  dq[idx] = accumulate ? dq[idx] + acc : acc;
}

// dK[j][e] = scale sum_i dS_ij Q[i][e], dV[j][e] = sum_i P_ij dO[i][e]
__global__ void attn_dkdv_f32_k(const float* __restrict__ q, const float* __restrict__ k,
                                const float* __restrict__ v, const float* __restrict__ d_o,
                                const float* __restrict__ lse, const float* __restrict__ dsum,
                                float* __restrict__ dk, float* __restrict__ dv, int T, int D,
                                float scale, int accumulate, long n_out) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_out) return;
  const int e = (int)(idx % D);
  const long rj = idx / D;
  const long g = rj / T;
  const long r0 = g * T;
  float ak = 0.f, av = 0.f;
  for (int i = 0; i < T; ++i) {
    float p, ds;
    attn_pd_f32(q + (r0 + i) * D, k + rj * D, d_o + (r0 + i) * D, v + rj * D, D, scale,
                lse[r0 + i], dsum[r0 + i], &p, &ds);
    ak = fmaf(ds, q[(r0 + i) * D + e], ak);
    av = fmaf(p, d_o[(r0 + i) * D + e], av);
  }
  ak *= scale;
  dk[idx] = accumulate ? dk[idx] + ak : ak;
  dv[idx] = accumulate ? dv[idx] + av : av;
}

// ---------------------------------------------------------------------------
// Row kernels (either activation type): one wave per row, lane l holding
// elements l and l + 64 (D <= 128), 4 rows per workgroup of 256.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// out = x / max(||x||, floor) and the raw norm
template <typename Tx>
__global__ void __launch_bounds__(256)
rownorm_k(const Tx* __restrict__ x, Tx* __restrict__ out, float* __restrict__ nrm, int D,
          long n_rows) {
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= n_rows) return;
  const bool h0 = l < D, h1 = l + 64 < D;
  const float a0 = h0 ? ldf(x, r * D + l) : 0.f, a1 = h1 ? ldf(x, r * D + l + 64) : 0.f;
  const float n = sqrtf(wave_sum(a0 * a0 + a1 * a1));
  const float inv = 1.f / fmaxf(n, kNormFloor);
  if (h0) stf(out, r * D + l, a0 * inv);
  if (h1) stf(out, r * D + l + 64, a1 * inv);
  if (l == 0) nrm[r] = n;
}

// dbeta_t (+)= sum_v KG[t][v] R[t][v];  dV'[t][v] = beta_t KG[t][v]
template <typename Tx>
__global__ void __launch_bounds__(256)
commit_rows1_k(const float* __restrict__ kg, const float* __restrict__ rr,
               const float* __restrict__ beta, float* __restrict__ dbeta, Tx* __restrict__ dvp,
               int D, int accumulate, long n_rows) {
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= n_rows) return;
  const bool h0 = l < D, h1 = l + 64 < D;
  const float b = beta[r];
  const float x0 = h0 ? kg[r * D + l] : 0.f, x1 = h1 ? kg[r * D + l + 64] : 0.f;
  const float y0 = h0 ? rr[r * D + l] : 0.f, y1 = h1 ? rr[r * D + l + 64] : 0.f;
  const float acc = wave_sum(x0 * y0 + x1 * y1);
  if (h0) stf(dvp, r * D + l, b * x0);
  if (h1) stf(dvp, r * D + l + 64, b * x1);
  if (l == 0) dbeta[r] = accumulate ? dbeta[r] + acc : acc;
}

// dK~ = (dK' - K' (K'.dK')) / n with dK' = beta_t dKraw (dK' / floor below it)
template <typename Tx>
__global__ void __launch_bounds__(256)
commit_rows2_k(const float* __restrict__ dkraw, const Tx* __restrict__ kp,
               const float* __restrict__ nrm, const float* __restrict__ beta,
               Tx* __restrict__ dkt, int D, long n_rows) {
  const long r = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= n_rows) return;
  const bool h0 = l < D, h1 = l + 64 < D;
  const float b = beta[r], n = nrm[r];
  const float d0 = h0 ? dkraw[r * D + l] : 0.f, d1 = h1 ? dkraw[r * D + l + 64] : 0.f;
  const float k0 = h0 ? ldf(kp, r * D + l) : 0.f, k1 = h1 ? ldf(kp, r * D + l + 64) : 0.f;
  const float dot = wave_sum(k0 * d0 + k1 * d1);
  const bool above = n > kNormFloor;
  const float inv = above ? 1.f / n : 1.f / kNormFloor;
  const float pr = above ? dot : 0.f;
  if (h0) stf(dkt, r * D + l, b * (d0 - k0 * pr) * inv);
  if (h1) stf(dkt, r * D + l + 64, b * (d1 - k1 * pr) * inv);
}

// dalpha[g] (+)= <S[g], G[g]>  (one workgroup of 256 per (b, h), fixed order)
__device__ __forceinline__ void dalpha_block(long g, const float* __restrict__ S,
                                             const float* __restrict__ G,
                                             float* __restrict__ dalpha, int DD, int accumulate) {
  __shared__ float red[4];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = threadIdx.x * 4; i < DD; i += 256 * 4 * 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = i + u * 256 * 4;
      if (j < DD) {
        const float4 a = *reinterpret_cast<const float4*>(S + g * DD + j);
        const float4 c = *reinterpret_cast<const float4*>(G + g * DD + j);
        acc[u] = fmaf(a.x, c.x, fmaf(a.y, c.y, fmaf(a.z, c.z, fmaf(a.w, c.w, acc[u]))));
      }
    }
  }
  const float w = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    dalpha[g] = accumulate ? dalpha[g] + t : t;
  }
}

__global__ void __launch_bounds__(256)
dalpha_k(const float* __restrict__ S, const float* __restrict__ G, float* __restrict__ dalpha,
         int DD, int accumulate) {
  dalpha_block(blockIdx.x, S, G, dalpha, DD, accumulate);
}

// bf16 copies of a float [n][128][128] matrix set, row-major and transposed;
// threads from n_out take a second set (m1, mb1, mtb1) when the grid covers it
// (workgroups from n_cast_blocks on: dalpha_block over (m0, m1) when dalpha
// is given, one per matrix)
__global__ void __launch_bounds__(256)
to_bf16_pair_k(const float* __restrict__ m0, __bf16* __restrict__ mb0,
               __bf16* __restrict__ mtb0, const float* __restrict__ m1,
               __bf16* __restrict__ mb1, __bf16* __restrict__ mtb1, long n_out,
               float* __restrict__ dalpha = nullptr, long n_cast_blocks = 0,
               int accumulate = 0) {
  if (dalpha && (long)blockIdx.x >= n_cast_blocks) {
    dalpha_block((long)blockIdx.x - n_cast_blocks, m0, m1, dalpha, HD * HD, accumulate);
    return;
  }
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const bool second = idx >= n_out;
  if (second) idx -= n_out;
  if (idx >= n_out) return;
  const float* m = second ? m1 : m0;
  __bf16* mb = second ? mb1 : mb0;
  __bf16* mtb = second ? mtb1 : mtb0;
  const int c = (int)(idx % HD), r = (int)((idx / HD) % HD);
  const long g = idx / (HD * HD);
  const __bf16 x = (__bf16)m[idx];
  if (mb) mb[idx] = x;
  if (mtb) mtb[g * HD * HD + (long)c * HD + r] = x;
}

__global__ void copy_f32_k(const float* __restrict__ a, float* __restrict__ b, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) b[i] = a[i];
}

// ---------------------------------------------------------------------------
// bf16 MFMA building blocks (d = 128)
// ---------------------------------------------------------------------------

// One problem of a batched Y = X Bt^T launch: with x2 set, Y = X Bt^T -
// X2 Bt2^T (both products in fp32, then one subtraction).
struct NtProb {
  const __bf16* x;
  const __bf16* bt;
  const __bf16* x2;
  const __bf16* bt2;
  Epi ep;
  int x_per_head, bt_per_head;
};
struct NtBatch {
  NtProb p0, p1;
};

// Y = X Bt^T: one workgroup of 4 waves per 32 rows of one g; wave w computes
// the 32 x 32 tile of columns 32 w.., operands straight from memory (the rows
// of X are shared through L1, Bt, 32 KB, stays in L2). Workgroups from
// per_prob on take the batch's second problem (same shapes).
__device__ __forceinline__ f32x16 nt_tile(const __bf16* x, const __bf16* bt, int x_per_head,
                                          int bt_per_head, long g, int H, int rows, int row0,
                                          int lane, int wave) {
  const int n = lane & 31, h2 = lane >> 5;
  const __bf16* xg = x + (x_per_head ? g % H : g) * (long)rows * HD;
  const __bf16* bg = bt + (bt_per_head ? g % H : g) * (long)HD * HD;
  const __bf16* xr = xg + (long)min(row0 + n, rows - 1) * HD + 8 * h2;
  const __bf16* br = bg + (long)(32 * wave + n) * HD + 8 * h2;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    a[kc] = ld8(xr + 16 * kc);
    b[kc] = ld8(br + 16 * kc);
  }
  f32x16 acc = zero16();
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) acc = mfma32(a[kc], b[kc], acc);
  return acc;
}

__global__ void __launch_bounds__(256)
nt_gemm_mfma_k(NtBatch nb, int rows, int H, int n_rblk, long per_prob) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const bool second = (long)blockIdx.x >= per_prob;
  const long bid = second ? (long)blockIdx.x - per_prob : (long)blockIdx.x;
  const NtProb& P = second ? nb.p1 : nb.p0;
  const long g = bid / n_rblk;
  const int row0 = (int)(bid % n_rblk) * 32;
  f32x16 acc = nt_tile(P.x, P.bt, P.x_per_head, P.bt_per_head, g, H, rows, row0, lane, wave);
  if (P.x2)
    acc = acc - nt_tile(P.x2, P.bt2, P.x_per_head, P.bt_per_head, g, H, rows, row0, lane, wave);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
    if (row < rows) epilogue<__bf16>(P.ep, ((size_t)g * rows + row) * HD + 32 * wave + n, acc[r]);
  }
}

// The commit backward's row steps fused into the products that feed them. A
// workgroup holds 32 whole rows (4 waves x 32 columns), so the per-row sums
// go through LDS: value v[r] of lane (n, h2) of wave w sits at row
// 8 (r / 4) + 4 h2 + r % 4 and column 32 w + n (the accumulator's order).
constexpr int RS_LD = 132;                     // row stride of the reduction tile (floats)

// Row sums of the 32 x 128 tile, in a fixed order (8 runs of 16 columns, then
// a pairwise tree over the runs); every lane receives its 16 rows' sums.
__device__ __forceinline__ void tile_row_sums(const float (&v)[16], float (&sum)[16], float* red,
                                              float* rs) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) red[(8 * (r >> 2) + 4 * h2 + (r & 3)) * RS_LD + 32 * wave + n] = v[r];
  __syncthreads();
  const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) a += red[row * RS_LD + 16 * part + j];
  a += __shfl_xor(a, 1);
  a += __shfl_xor(a, 2);
  a += __shfl_xor(a, 4);
  if (part == 0) rs[row] = a;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 16; ++r) sum[r] = rs[8 * (r >> 2) + 4 * h2 + (r & 3)];
}

// Per 32 rows of one g: R = V' - K'S and K'G (both products in the workgroup),
// then dbeta_t (+)= sum_v K'G[t][v] R[t][v] and dV' = beta K'G; R, K'G and dV'
// leave as bf16 (the operands of the next products).
__global__ void __launch_bounds__(256)
commit_resid_rows_k(const __bf16* __restrict__ kp, const __bf16* __restrict__ st,
                    const __bf16* __restrict__ gt, const __bf16* __restrict__ vp,
                    const float* __restrict__ beta, __bf16* __restrict__ rx,
                    __bf16* __restrict__ kgx, __bf16* __restrict__ dvx,
                    float* __restrict__ dbeta, int T, int H, int n_rblk, int accumulate) {
  __shared__ float red[32 * RS_LD];
  __shared__ float rs[32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const long g = blockIdx.x / n_rblk;
  const int row0 = (int)(blockIdx.x % n_rblk) * 32;
  const f32x16 as = nt_tile(kp, st, 0, 0, g, H, T, row0, lane, wave);
  const f32x16 ag = nt_tile(kp, gt, 0, 0, g, H, T, row0, lane, wave);
  float prod[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
    prod[r] = 0.f;
    if (row < T) {
      const size_t idx = ((size_t)g * T + row) * HD + 32 * wave + n;
      const float R = (float)vp[idx] - as[r];
      const float kg = ag[r];
      prod[r] = kg * R;
      rx[idx] = (__bf16)R;
      kgx[idx] = (__bf16)kg;
      dvx[idx] = (__bf16)(beta[(size_t)g * T + row] * kg);
    }
  }
  float sum[16];
  tile_row_sums(prod, sum, red, rs);
  const int t = threadIdx.x;
  if (t < 32 && row0 + t < T) {
    const size_t i = (size_t)g * T + row0 + t;
    dbeta[i] = accumulate ? dbeta[i] + rs[t] : rs[t];
  }
}

// Per 32 rows of one g: dKraw = R G^T - K'G S^T, then through beta and the row
// normalisation K' = K~ / max(||K~||, floor): dK~ = beta (dKraw - K' (K'.dKraw))
// / ||K~|| above the floor, beta dKraw / floor below it (bf16 out).
__global__ void __launch_bounds__(256)
commit_dkt_rows_k(const __bf16* __restrict__ rx, const __bf16* __restrict__ gb,
                  const __bf16* __restrict__ kgx, const __bf16* __restrict__ sb,
                  const __bf16* __restrict__ kp, const float* __restrict__ nrm,
                  const float* __restrict__ beta, __bf16* __restrict__ dkt, int T, int H,
                  int n_rblk) {
  __shared__ float red[32 * RS_LD];
  __shared__ float rs[32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const long g = blockIdx.x / n_rblk;
  const int row0 = (int)(blockIdx.x % n_rblk) * 32;
  const f32x16 d = nt_tile(rx, gb, 0, 0, g, H, T, row0, lane, wave) -
                   nt_tile(kgx, sb, 0, 0, g, H, T, row0, lane, wave);
  float kv[16], prod[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
    kv[r] = row < T ? (float)kp[((size_t)g * T + row) * HD + 32 * wave + n] : 0.f;
    prod[r] = kv[r] * d[r];
  }
  float dot[16];
  tile_row_sums(prod, dot, red, rs);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = row0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
    if (row < T) {
      const size_t i = (size_t)g * T + row;
      const float nr = nrm[i];
      const bool above = nr > kNormFloor;
      const float inv = above ? 1.f / nr : 1.f / kNormFloor;
      const float pr = above ? dot[r] : 0.f;
      dkt[i * HD + 32 * wave + n] = (__bf16)(beta[i] * (d[r] - kv[r] * pr) * inv);
    }
  }
}

// bf16 chunk of `rows` x 128 into LDS under the swz_v swizzle, zero past `valid`
__device__ __forceinline__ void stage_tr(char* dst, const __bf16* src, int rows, int valid) {
  for (int idx = threadIdx.x; idx < rows * 16; idx += blockDim.x) {
    const int r = idx >> 4, p = idx & 15;
    uint4 val = {0u, 0u, 0u, 0u};
    if (r < valid) val = *reinterpret_cast<const uint4*>(src + (size_t)r * HD + 8 * p);
    *reinterpret_cast<uint4*>(dst + r * 256 + ((p ^ swz_v(r)) << 4)) = val;
  }
}

constexpr int XTY_SUB = 64;                   // tokens staged at a time

// Partial X^T Y over one chunk of `chunk` tokens of one g, for one 64 x 64
// quadrant (qe, qv) of the 128 x 128 result: wave w computes the 32 x 32 tile
// (2 qe + w / 2, 2 qv + w % 2), stored in MFMA accumulator order:
// part[(g * nch + ch) * 16 + tile][lane][16], tile = 4 te + tv.
// Up to three X^T Y problems of one shape per launch: workgroups
// [j per_prob, (j + 1) per_prob) take problem j, whose partials follow the
// previous problem's (part + j * per_prob * 4096 floats).
struct XtyBatch {
  const __bf16* x0;
  const __bf16* y0;
  const __bf16* x1;
  const __bf16* y1;
  const __bf16* x2;
  const __bf16* y2;
};

__global__ void __launch_bounds__(256)
xty_part_mfma_k(XtyBatch xb, float* __restrict__ part_all, int T, int chunk, int nch,
                long per_prob) {
  __shared__ __attribute__((aligned(16))) char lx[XTY_SUB * 256];
  __shared__ __attribute__((aligned(16))) char ly[XTY_SUB * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = (int)((long)blockIdx.x / per_prob);
  const long bid = (long)blockIdx.x - j * per_prob;
  const __bf16* x = j == 0 ? xb.x0 : j == 1 ? xb.x1 : xb.x2;
  const __bf16* y = j == 0 ? xb.y0 : j == 1 ? xb.y1 : xb.y2;
  float* part = part_all + (size_t)j * per_prob * 4096;
  const int quad = (int)(bid & 3);
  const long gc = bid >> 2;
  const long g = gc / nch;
  const int ch = gc % nch;
  const int te = 2 * (quad >> 1) + (wave >> 1), tv = 2 * (quad & 1) + (wave & 1);
  f32x16 acc = zero16();
  for (int s0 = ch * chunk; s0 < min(T, (ch + 1) * chunk); s0 += XTY_SUB) {
    const int valid = min(XTY_SUB, T - s0);
    stage_tr(lx, x + ((size_t)g * T + s0) * HD, XTY_SUB, valid);
    stage_tr(ly, y + ((size_t)g * T + s0) * HD, XTY_SUB, valid);
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < XTY_SUB / 16; ++kc)
      acc = mfma32(tr_op(lx, 16 * kc, 8, 32 * te, lane), tr_op(ly, 16 * kc, 8, 32 * tv, lane), acc);
    __syncthreads();
  }
  float* p = part + (((size_t)g * nch + ch) * 16 + 4 * te + tv) * 1024 + lane * 16;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    *reinterpret_cast<float4*>(p + 4 * q4) =
        make_float4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
}

// out[go][e][v] (+)= gamma[go] base[go][e][v] + delta * sum_b sum_ch part:
// one thread per (go, tile, lane, 4 registers), chunks summed in order with
// the loads of 4 chunks issued ahead of their sums.
struct XtyRed {
  float* out;
  const float* base_mat;
  const float* gamma;
  float delta;
  int sum_b;
  long n_thr;                     // go count x 4096
};
struct XtyRedBatch {
  XtyRed r0, r1, r2;
};

__global__ void __launch_bounds__(256)
xty_reduce_mfma_k(const float* __restrict__ part_all, XtyRedBatch rb, int accumulate, int nch,
                  int B, int H, long part_stride) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  int j = 0;
  if (idx >= rb.r0.n_thr) {
    idx -= rb.r0.n_thr;
    j = 1;
    if (idx >= rb.r1.n_thr) {
      idx -= rb.r1.n_thr;
      j = 2;
    }
  }
  const XtyRed& R = j == 0 ? rb.r0 : j == 1 ? rb.r1 : rb.r2;
  if (idx >= R.n_thr) return;
  const float* part = part_all + (size_t)j * part_stride;
  float* out = R.out;
  const float* base_mat = R.base_mat;
  const float* gamma = R.gamma;
  const float delta = R.delta;
  const int sum_b = R.sum_b;
  const int q4 = (int)(idx & 3);
  const int lane = (int)((idx >> 2) & 63);
  const int tile = (int)((idx >> 8) & 15);
  const long go = idx >> 12;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int nb = sum_b ? B : 1;
  const size_t inner = ((size_t)tile * 1024 + lane * 16 + 4 * q4);
  for (int b = 0; b < nb; ++b) {
    const long g = sum_b ? (long)b * H + go : go;
    const float* pg = part + (size_t)g * nch * 16 * 1024 + inner;
    for (int c0 = 0; c0 < nch; c0 += 4) {
      float4 xs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u < nch) xs[u] = *reinterpret_cast<const float4*>(pg + (size_t)(c0 + u) * 16 * 1024);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u < nch) {
          acc.x += xs[u].x; acc.y += xs[u].y; acc.z += xs[u].z; acc.w += xs[u].w;
        }
    }
  }
  const int n = lane & 31, h2 = lane >> 5;
  const int v = 32 * (tile & 3) + n;
  const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * q4 + u;
    const int e = 32 * (tile >> 2) + 8 * (r >> 2) + 4 * h2 + (r & 3);
    const size_t o = (size_t)go * HD * HD + (size_t)e * HD + v;
    float val = delta * a4[u];
    if (base_mat) val += gamma[go] * base_mat[o];
    out[o] = accumulate ? out[o] + val : val;
  }
}

// ---------------------------------------------------------------------------
// Attention backward, bf16 MFMA (d = 128). The exponent base is 2: with
// c = scale log2(e), P_ij = exp2(c q_i.k_j - lse2_i), lse2 in log2 units.
// ---------------------------------------------------------------------------
constexpr int AB_STAGE = 64;                  // keys (or queries) staged per step

// Chunk swizzle of the staged attention tiles: 16-byte chunk p of row r sits at
// p ^ swz_b(r). Bits 3:2 follow r % 4 and bits 1:0 follow (r / 4) % 4, so both
// ways the kernels read a tile are free of bank conflicts: a row read (16
// consecutive rows, one chunk each) meets 16 distinct positions, and a
// transposing read (4 consecutive rows, 4 aligned chunks each) meets 4
// disjoint groups of positions.
__device__ __forceinline__ int swz_b(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Operand reads from a staged tile. A operands by transposing reads follow an
// MFMA accumulator's register order in their contraction slots: lane (n, h2)
// receives M[r0 + 4 h2 + u][c0 + n] for u = 0..3 and M[r0 + 8 + 4 h2 + u - 4]
// [c0 + n] for u = 4..7, the rows that registers 8 kc .. 8 kc + 7 of a 32 x 32
// accumulator hold (r0 = 32 t + 16 kc). Row operands take 8 consecutive columns
// 16 kc + 8 h2 .. of row r0 + n.
// Per-lane byte offsets of the transposing reads and of the row operands, for a
// tile origin r0 that is a multiple of 16 (swz_b then depends on the lane
// alone, and r0 * 256 folds into the reads' immediate offsets). Made opaque so
// that each stays one register instead of being re-derived per read.
struct TileOffsets {
  int tr[4][2];                                  // transposing reads, by column tile
  int row[8];                                    // row operand, by 16-column step kc
};

__device__ __forceinline__ TileOffsets tile_offsets(int lane) {
  TileOffsets t;
  const int G = lane >> 4;
  const int s = lane & 15, c = s >> 2, j = s & 3;
  const int rb = 4 * (G >> 1) + c;
#pragma unroll
  for (int te = 0; te < 4; ++te) {
    const int col = 32 * te + 16 * (G & 1) + 4 * j;
    const int c16 = col >> 3, sub = (col & 7) * 2;
    t.tr[te][0] = rb * 256 + ((c16 ^ swz_b(rb)) << 4) + sub;
    t.tr[te][1] = (rb + 8) * 256 + ((c16 ^ swz_b(rb + 8)) << 4) + sub;
    asm volatile("" : "+v"(t.tr[te][0]), "+v"(t.tr[te][1]));
  }
  const int n = lane & 31, h2 = lane >> 5;
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    t.row[kc] = n * 256 + (((2 * kc + h2) ^ swz_b(n)) << 4);
    asm volatile("" : "+v"(t.row[kc]));
  }
  return t;
}

__device__ __forceinline__ bf16x8 tr_op_at(const char* base, int r0, const TileOffsets& t, int te) {
  return __builtin_shufflevector(tr_read(base + r0 * 256 + t.tr[te][0]),
                                 tr_read(base + r0 * 256 + t.tr[te][1]), 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 row_op_at(const char* base, int r0, const TileOffsets& t, int kc) {
  return *reinterpret_cast<const bf16x8*>(base + r0 * 256 + t.row[kc]);
}

// registers 8 kc .. 8 kc + 7 of an accumulator as a bf16 operand
__device__ __forceinline__ bf16x8 acc_op(const float* a, int kc) {
  bf16x8 r;
#pragma unroll
  for (int u = 0; u < 8; ++u) r[u] = (__bf16)a[8 * kc + u];
  return r;
}

// Tiles of 64 rows x 256 bytes move from memory to LDS by buffer-load DMA,
// two buffers per operand: while a stage computes from one, the next stage's
// rows land in the other. Each of the NW waves moves 64 / NW rows as 1 KB
// pieces; lane l's 16 bytes land at byte 16 l of its piece, so the lane loads
// the logical chunk that the swz_v swizzle puts there. Rows past the buffer
// resource's range (the frame's end) arrive as zeros.
// Byte offset that lane l loads for a piece whose first row is a multiple of
// 4 with (first row / 4) % 4 = q: row (l / 16) of the piece, logical chunk
// (l % 16) ^ swz_b(row).
__device__ __forceinline__ int dma_lane_off(int lane, int q) {
  return (lane >> 4) * 256 + (((lane & 15) ^ ((lane >> 4) << 2) ^ q) << 4);
}

struct DmaOffsets {
  int o[4];                                      // by q = piece % 4
};

__device__ __forceinline__ DmaOffsets dma_offsets(int lane) {
  DmaOffsets d;
#pragma unroll
  for (int q = 0; q < 4; ++q) d.o[q] = dma_lane_off(lane, q);
  return d;
}

template <int NW>
__device__ __forceinline__ void dma_tile64(char* dst, __amdgpu_buffer_rsrc_t src, int row0,
                                           const DmaOffsets& lo, int wave) {
  constexpr int PIECES = 16 / NW;               // 1 KB pieces per wave (a multiple of 4)
#pragma unroll
  for (int ii = 0; ii < PIECES; ++ii)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src, (lds_void_t*)(dst + wave * PIECES * 1024 + ii * 1024), 16, lo.o[ii & 3],
        row0 * 256 + wave * PIECES * 1024 + ii * 1024, 0, 0);
}

// s_waitcnt for the vector-memory counter only: wait until at most n (< 64)
// of this wave's vector-memory operations are outstanding (the count's low
// four bits in [3:0], its high two in [15:14]; expcnt and lgkmcnt at their
// maxima, i.e. not waited for).
#define VMCNT_WAIT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

// Per query row: lse2 = log2 sum_j exp2(c q.k_j) and dsum = dO . O_intra. One
// workgroup of NW waves per 32 NW queries; wave w holds queries 32 w.. as the
// columns of S^T = K Q^T (a lane's running max and sum cover half the keys;
// the halves combine at the end).
template <int NW>
__global__ void __launch_bounds__(64 * NW)
attn_pre_mfma_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                const __bf16* __restrict__ o, const __bf16* __restrict__ d_o,
                float* __restrict__ lse2, float* __restrict__ dsum, int T, float c, int n_qblk) {
  __shared__ __attribute__((aligned(16))) char lk0[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lk1[AB_STAGE * 256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h2 = lane >> 5;
  const long g = blockIdx.x / n_qblk;
  const int i = (blockIdx.x % n_qblk) * (32 * NW) + 32 * wave + n;   // this lane's query
  const size_t gbase = (size_t)g * T;
  const __bf16* qr = q + (gbase + min(i, T - 1)) * HD + 8 * h2;
  bf16x8 qb[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) qb[kc] = ld8(qr + 16 * kc);
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + gbase * HD, (uint32_t)T * 256);
  const DmaOffsets loff = dma_offsets(lane);
  const TileOffsets to = tile_offsets(lane);
  const int n_st = (T + AB_STAGE - 1) / AB_STAGE;
  float m = -INFINITY, l = 0.f;
  auto compute = [&](const char* lk, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < AB_STAGE / 32; ++sub) {
      f32x16 acc = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) acc = mfma32(row_op_at(lk, 32 * sub, to, kc), qb[kc], acc);
      float sv[16], mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3);
        sv[r] = j < T ? acc[r] * c : -INFINITY;
        mt = fmaxf(mt, sv[r]);
      }
      const float mn = fmaxf(m, mt);
      if (mn > -INFINITY) {
        float add = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) add += __builtin_amdgcn_exp2f(sv[r] - mn);
        l = l * exp2f(m - mn) + add;
        m = mn;
      }
    }
  };
  dma_tile64<NW>(lk0, rk, 0, loff, wave);
  for (int st = 0;;) {
    dma_tile64<NW>(lk1, rk, min(st + 1, n_st - 1) * AB_STAGE, loff, wave);
    VMCNT_WAIT(16 / NW);
    __builtin_amdgcn_s_barrier();
    compute(lk0, st * AB_STAGE);
    __builtin_amdgcn_s_barrier();
    if (++st >= n_st) break;
    dma_tile64<NW>(lk0, rk, min(st + 1, n_st - 1) * AB_STAGE, loff, wave);
    VMCNT_WAIT(16 / NW);
    __builtin_amdgcn_s_barrier();
    compute(lk1, st * AB_STAGE);
    __builtin_amdgcn_s_barrier();
    if (++st >= n_st) break;
  }
  VMCNT_WAIT(0);
  const float mo = swap_halves(m), lo = swap_halves(l);
  const float M = fmaxf(m, mo);
  const float L = (m > -INFINITY ? l * exp2f(m - M) : 0.f) + (mo > -INFINITY ? lo * exp2f(mo - M) : 0.f);
  // dO . O over this lane's half of the features, then both halves
  const __bf16* dr = d_o + (gbase + min(i, T - 1)) * HD + 64 * h2;
  const __bf16* orr = o + (gbase + min(i, T - 1)) * HD + 64 * h2;
  float dd = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const bf16x8 x = ld8(dr + 8 * u), y = ld8(orr + 8 * u);
#pragma unroll
    for (int e = 0; e < 8; ++e) dd = fmaf((float)x[e], (float)y[e], dd);
  }
  dd += swap_halves(dd);
  if (h2 == 0 && i < T) {
    lse2[gbase + i] = M + log2f(L);
    dsum[gbase + i] = dd;
  }
}

// dQ = scale sum_j dS_ij K_j (+ dO M^T when m_rows is given: the inter-frame
// branch with M = Phi_q S, bf16 row-major [e][v]). One workgroup of NW waves
// per 32 NW queries; wave w accumulates dQ^T for queries 32 w.. (lane = query,
// registers = features), key and value tiles staged in LDS.
// (Workgroup `blk` of the dQ grid; the LDS arrays are the kernel's and reach
// here as parameters, so that, once inlined, every access names its array.)
template <int NW>
__device__ __forceinline__ void attn_dq_block(
    int blk, char* lk0, char* lk1, char* lv0, char* lv1, const __bf16* __restrict__ q,
    const __bf16* __restrict__ k, const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
    const float* __restrict__ lse2, const float* __restrict__ dsum,
    const __bf16* __restrict__ m_rows, __bf16* __restrict__ dq, int T, float c, float scale,
    int n_qblk, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h2 = lane >> 5;
  const long g = blk / n_qblk;
  const int i = (blk % n_qblk) * (32 * NW) + 32 * wave + n;
  const size_t gbase = (size_t)g * T;
  const size_t qrow = gbase + min(i, T - 1);
  bf16x8 qb[8], ob[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    qb[kc] = ld8(q + qrow * HD + 16 * kc + 8 * h2);
    ob[kc] = ld8(d_o + qrow * HD + 16 * kc + 8 * h2);
  }
  const float li = lse2[qrow], di = dsum[qrow];
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(k + gbase * HD, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(v + gbase * HD, (uint32_t)T * 256);
  const DmaOffsets loff = dma_offsets(lane);
  const TileOffsets to = tile_offsets(lane);
  const int n_st = (T + AB_STAGE - 1) / AB_STAGE;
  f32x16 dacc[4] = {zero16(), zero16(), zero16(), zero16()};
  auto compute = [&](const char* lk, const char* lv, int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < AB_STAGE / 32; ++sub) {
      f32x16 st = zero16(), dp = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        st = mfma32(row_op_at(lk, 32 * sub, to, kc), qb[kc], st);
        dp = mfma32(row_op_at(lv, 32 * sub, to, kc), ob[kc], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const float e = __builtin_amdgcn_exp2f(st[r] * c - li);
        ds[r] = (j < T ? e : 0.f) * (dp[r] - di);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const bf16x8 b = acc_op(ds, kc);
#pragma unroll
        for (int te = 0; te < 4; ++te)
          dacc[te] = mfma32(tr_op_at(lk, 32 * sub + 16 * kc, to, te), b, dacc[te]);
      }
    }
  };
  auto issue = [&](char* lk, char* lv, int st) __attribute__((always_inline)) {
    dma_tile64<NW>(lk, rk, st * AB_STAGE, loff, wave);
    dma_tile64<NW>(lv, rv, st * AB_STAGE, loff, wave);
  };
  issue(lk0, lv0, 0);
  for (int st = 0;;) {
    issue(lk1, lv1, min(st + 1, n_st - 1));
    VMCNT_WAIT(32 / NW);
    __builtin_amdgcn_s_barrier();
    compute(lk0, lv0, st * AB_STAGE);
    __builtin_amdgcn_s_barrier();
    if (++st >= n_st) break;
    issue(lk0, lv0, min(st + 1, n_st - 1));
    VMCNT_WAIT(32 / NW);
    __builtin_amdgcn_s_barrier();
    compute(lk1, lv1, st * AB_STAGE);
    __builtin_amdgcn_s_barrier();
    if (++st >= n_st) break;
  }
  VMCNT_WAIT(0);
#pragma unroll
  for (int te = 0; te < 4; ++te) dacc[te] *= scale;
  if (m_rows) {
    const __bf16* mg = m_rows + (size_t)g * HD * HD;
#pragma unroll
    for (int te = 0; te < 4; ++te) {
      const __bf16* mr = mg + (size_t)(32 * te + n) * HD + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) dacc[te] = mfma32(ld8(mr + 16 * kc), ob[kc], dacc[te]);
    }
  }
  if (i < T) {
    __bf16* out = dq + (gbase + i) * HD;
#pragma unroll
    for (int te = 0; te < 4; ++te) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4* p4 = reinterpret_cast<bf16x4*>(out + 32 * te + 8 * rg + 4 * h2);
        bf16x4 w, old;
        if (accumulate) old = *p4;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          w[u] = (__bf16)(dacc[te][4 * rg + u] + (accumulate ? (float)old[u] : 0.f));
        *p4 = w;
      }
    }
  }
}

template <int NW>
__global__ void __launch_bounds__(64 * NW)
attn_dq_mfma_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
               const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
               const float* __restrict__ lse2, const float* __restrict__ dsum,
               const __bf16* __restrict__ m_rows, __bf16* __restrict__ dq, int T, float c,
               float scale, int n_qblk, int accumulate) {
  __shared__ __attribute__((aligned(16))) char lk0[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lk1[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lv0[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lv1[AB_STAGE * 256];
  attn_dq_block<NW>(blockIdx.x, lk0, lk1, lv0, lv1, q, k, v, d_o, lse2, dsum, m_rows, dq, T, c,
                    scale, n_qblk, accumulate);
}

// A key block's dK and dV summed over two halves of the queries, each half a
// workgroup of its own: both publish their fp32 sums (kacc, then vacc, in
// 16-byte pieces, lane-interleaved) in their slot with device-scope (sc1)
// stores, wait for them to complete and count their arrival on the block's
// counter; the second to arrive adds the other's sums to its own (a + b, the
// same value whichever half is second) and writes dK and dV.
struct PairSplit {
  float* slots;                  // 2 per key block (slot 2 blk + half), NW * 8192 floats each
  unsigned long long* ctr;       // one per key block
  unsigned long long tag;        // this call's tag (bit 63 set, so never 0)
};
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCoherentAux = 16;   // cache policy bits of the slot accesses: device scope (sc1)

// dK = scale sum_i dS_ij Q_i and dV = sum_i P_ij dO_i. One workgroup of NW
// waves per 32 NW keys; wave w holds keys 32 w.. as the columns of S = Q K^T and
// accumulates dK^T and dV^T (lane = key, registers = features); query, dO,
// lse2 and dsum tiles staged in LDS (waves 0 and 1 move lse2 and dsum; any
// further waves move lse2 once more into a spare slot, so that every wave
// issues the same number of transfers per stage). With a PairSplit (half 0
// or 1), the workgroup covers that half of the query stages.
template <int NW>
__device__ __forceinline__ void attn_dkdv_block(
    int blk, int half, char* lq0, char* lq1, char* lo0, char* lo1, float* lr0, float* lr1,
    int* flag, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
    const float* __restrict__ lse2, const float* __restrict__ dsum, __bf16* __restrict__ dk,
    __bf16* __restrict__ dv, int T, float c, float scale, int n_kblk, int accumulate,
    const PairSplit* ps) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, h2 = lane >> 5;
  const long g = blk / n_kblk;
  const int j = (blk % n_kblk) * (32 * NW) + 32 * wave + n;   // this lane's key
  const size_t gbase = (size_t)g * T;
  const size_t krow = gbase + min(j, T - 1);
  bf16x8 kb[8], vb[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    kb[kc] = ld8(k + krow * HD + 16 * kc + 8 * h2);
    vb[kc] = ld8(v + krow * HD + 16 * kc + 8 * h2);
  }
  f32x16 kacc[4] = {zero16(), zero16(), zero16(), zero16()};
  f32x16 vacc[4] = {zero16(), zero16(), zero16(), zero16()};
  const bool key_ok = j < T;
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(q + gbase * HD, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(d_o + gbase * HD, (uint32_t)T * 256);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(wave == 1 ? dsum + gbase : lse2 + gbase,
                                                (uint32_t)T * 4);
  const DmaOffsets loff = dma_offsets(lane);
  const TileOffsets to = tile_offsets(lane);
  const int n_st = (T + AB_STAGE - 1) / AB_STAGE;
  auto compute = [&](const char* lq, const char* lo, const float* lr, int i0)
                     __attribute__((always_inline)) {
    const float* ll = lr;
    const float* ld = lr + AB_STAGE;
#pragma unroll
    for (int sub = 0; sub < AB_STAGE / 32; ++sub) {
      f32x16 sc = zero16(), dp = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        sc = mfma32(row_op_at(lq, 32 * sub, to, kc), kb[kc], sc);
        dp = mfma32(row_op_at(lo, 32 * sub, to, kc), vb[kc], dp);
      }
      // lse2 and dsum of this lane's 16 query rows: 4 runs of 4 consecutive rows
      float lv[16], dv4[16];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 a = ld4(ll + 32 * sub + 8 * rg + 4 * h2);
        const float4 b = ld4(ld + 32 * sub + 8 * rg + 4 * h2);
        lv[4 * rg] = a.x; lv[4 * rg + 1] = a.y; lv[4 * rg + 2] = a.z; lv[4 * rg + 3] = a.w;
        dv4[4 * rg] = b.x; dv4[4 * rg + 1] = b.y; dv4[4 * rg + 2] = b.z; dv4[4 * rg + 3] = b.w;
      }
      float pv[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const float e = __builtin_amdgcn_exp2f(sc[r] * c - lv[r]);
        const bool ok = key_ok & (i0 + il < T);
        const float p = ok ? e : 0.f;
        pv[r] = p;
        ds[r] = p * (dp[r] - dv4[r]);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const bf16x8 pb = acc_op(pv, kc), db = acc_op(ds, kc);
#pragma unroll
        for (int te = 0; te < 4; ++te) {
          vacc[te] = mfma32(tr_op_at(lo, 32 * sub + 16 * kc, to, te), pb, vacc[te]);
          kacc[te] = mfma32(tr_op_at(lq, 32 * sub + 16 * kc, to, te), db, kacc[te]);
        }
      }
    }
  };
  auto issue = [&](char* lq, char* lo, float* lr, int st) __attribute__((always_inline)) {
    dma_tile64<NW>(lq, rq, st * AB_STAGE, loff, wave);
    dma_tile64<NW>(lo, ro, st * AB_STAGE, loff, wave);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(lr + wave * AB_STAGE), 4,
                                             lane * 4, st * AB_STAGE * 4, 0, 0);
  };
  // query stages [s_begin, s_end): all, or this half's (the host splits only
  // frames of at least 4 stages, so both halves are non-empty)
  const int s_mid = n_st / 2;
  const int s_begin = ps && half ? s_mid : 0;
  const int s_end = ps && !half ? s_mid : n_st;
  issue(lq0, lo0, lr0, s_begin);
  for (int st = s_begin;;) {
    issue(lq1, lo1, lr1, min(st + 1, s_end - 1));
    VMCNT_WAIT(32 / NW + 1);
    __builtin_amdgcn_s_barrier();
    compute(lq0, lo0, lr0, st * AB_STAGE);
    __builtin_amdgcn_s_barrier();
    if (++st >= s_end) break;
    issue(lq0, lo0, lr0, min(st + 1, s_end - 1));
    VMCNT_WAIT(32 / NW + 1);
    __builtin_amdgcn_s_barrier();
    compute(lq1, lo1, lr1, st * AB_STAGE);
    __builtin_amdgcn_s_barrier();
    if (++st >= s_end) break;
  }
  VMCNT_WAIT(0);
  if (ps) {
    constexpr int kSlotFloats = NW * 8192;
    const __amdgpu_buffer_rsrc_t mine =
        buffer_rsrc(ps->slots + (size_t)(2 * blk + half) * kSlotFloats, kSlotFloats * 4);
#pragma unroll
    for (int gp = 0; gp < 32; ++gp) {
      const f32x16& a = gp < 16 ? kacc[gp >> 2] : vacc[(gp >> 2) & 3];
      const f32x4 x = {a[4 * (gp & 3)], a[4 * (gp & 3) + 1], a[4 * (gp & 3) + 2],
                       a[4 * (gp & 3) + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), mine,
                                             ((wave * 32 + gp) * 64 + lane) * 16, 0,
                                             kCoherentAux);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) *flag = pair_arrive(ps->ctr + blk, ps->tag) ? 1 : 0;
    __syncthreads();
    if (*flag == 0) return;
    const __amdgpu_buffer_rsrc_t other =
        buffer_rsrc(ps->slots + (size_t)(2 * blk + 1 - half) * kSlotFloats, kSlotFloats * 4);
    f32x4 od[32];
#pragma unroll
    for (int gp = 0; gp < 32; ++gp)
      od[gp] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             other, ((wave * 32 + gp) * 64 + lane) * 16, 0,
                                             kCoherentAux));
#pragma unroll
    for (int gp = 0; gp < 32; ++gp)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (gp < 16)
          kacc[gp >> 2][4 * (gp & 3) + e] += od[gp][e];
        else
          vacc[(gp >> 2) & 3][4 * (gp & 3) + e] += od[gp][e];
      }
  }
  if (key_ok) {
    __bf16* ok = dk + (gbase + j) * HD;
    __bf16* ov = dv + (gbase + j) * HD;
#pragma unroll
    for (int te = 0; te < 4; ++te) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4* pk = reinterpret_cast<bf16x4*>(ok + 32 * te + 8 * rg + 4 * h2);
        bf16x4* pv4 = reinterpret_cast<bf16x4*>(ov + 32 * te + 8 * rg + 4 * h2);
        bf16x4 wk, wv, okd, ovd;
        if (accumulate) {
          okd = *pk;
          ovd = *pv4;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wk[u] = (__bf16)(scale * kacc[te][4 * rg + u] + (accumulate ? (float)okd[u] : 0.f));
          wv[u] = (__bf16)(vacc[te][4 * rg + u] + (accumulate ? (float)ovd[u] : 0.f));
        }
        *pk = wk;
        *pv4 = wv;
      }
    }
  }
}

template <int NW>
__global__ void __launch_bounds__(64 * NW)
attn_dkdv_mfma_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                 const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
                 const float* __restrict__ lse2, const float* __restrict__ dsum,
                 __bf16* __restrict__ dk, __bf16* __restrict__ dv, int T, float c, float scale,
                 int n_kblk, int accumulate) {
  __shared__ __attribute__((aligned(16))) char lq0[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lq1[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lo0[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char lo1[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) float lr0[4 * AB_STAGE];   // lse2, dsum, spare x2
  __shared__ __attribute__((aligned(16))) float lr1[4 * AB_STAGE];
  attn_dkdv_block<NW>(blockIdx.x, 0, lq0, lq1, lo0, lo1, lr0, lr1, nullptr, q, k, v, d_o, lse2,
                      dsum, dk, dv, T, c, scale, n_kblk, accumulate, nullptr);
}

// dQ and dK/dV in one grid, for shapes whose separate grids would each leave
// most SIMDs idle (both kernels hold one wave per SIMD): the n_dq dQ
// workgroups first (the longer ones), then the dK/dV workgroups, two per key
// block (query halves) when a PairSplit is given. The two share one set of
// LDS arrays.
template <int NW>
__global__ void __launch_bounds__(64 * NW)
attn_dqdkdv_mfma_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                   const __bf16* __restrict__ v, const __bf16* __restrict__ d_o,
                   const float* __restrict__ lse2, const float* __restrict__ dsum,
                   const __bf16* __restrict__ m_rows, __bf16* __restrict__ dq,
                   __bf16* __restrict__ dk, __bf16* __restrict__ dv, int T, float c, float scale,
                   int n_blk, int n_dq, int accumulate, PairSplit split) {
  __shared__ __attribute__((aligned(16))) char l0[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char l1[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char l2[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) char l3[AB_STAGE * 256];
  __shared__ __attribute__((aligned(16))) float lr0[4 * AB_STAGE];
  __shared__ __attribute__((aligned(16))) float lr1[4 * AB_STAGE];
  __shared__ int flag;
  const int b = blockIdx.x;
  if (b < n_dq) {
    attn_dq_block<NW>(b, l0, l1, l2, l3, q, k, v, d_o, lse2, dsum, m_rows, dq, T, c, scale,
                      n_blk, accumulate);
  } else if (split.slots) {
    const int u = b - n_dq;
    attn_dkdv_block<NW>(u >> 1, u & 1, l0, l1, l2, l3, lr0, lr1, &flag, q, k, v, d_o, lse2,
                        dsum, dk, dv, T, c, scale, n_blk, accumulate, &split);
  } else {
    attn_dkdv_block<NW>(b - n_dq, 0, l0, l1, l2, l3, lr0, lr1, &flag, q, k, v, d_o, lse2, dsum,
                        dk, dv, T, c, scale, n_blk, accumulate, nullptr);
  }
}

}  // namespace

// ===========================================================================
// Host side
// ===========================================================================
namespace {

inline unsigned blocks(long n, int per) { return (unsigned)((n + per - 1) / per); }

Epi make_epi(const void* z, bool z_f32, float* y32, void* yx, bool accumulate) {
  Epi e;
  e.z = z;
  e.z_f32 = z_f32 ? 1 : 0;
  e.y32 = y32;
  e.yx = yx;
  e.accumulate = accumulate ? 1 : 0;
  return e;
}

NtProb nt_prob(const void* x, bool x_per_head, const void* bt, bool bt_per_head, const Epi& ep,
               const void* x2 = nullptr, const void* bt2 = nullptr) {
  NtProb p;
  p.x = static_cast<const __bf16*>(x);
  p.bt = static_cast<const __bf16*>(bt);
  p.x2 = static_cast<const __bf16*>(x2);
  p.bt2 = static_cast<const __bf16*>(bt2);
  p.ep = ep;
  p.x_per_head = x_per_head ? 1 : 0;
  p.bt_per_head = bt_per_head ? 1 : 0;
  return p;
}

// bf16 MFMA: one or two independent Y = X B^T problems of `rows` rows per g in
// one launch.
hipError_t nt_gemm_batch(const Dims& d, int rows, const NtProb& p0, const NtProb* p1,
                         hipStream_t s) {
  const long n_g = (long)d.B * d.H;
  const int n_rblk = (rows + 31) / 32;
  const long per = n_g * n_rblk;
  const NtBatch nb{p0, p1 ? *p1 : p0};
  nt_gemm_mfma_k<<<(unsigned)(per * (p1 ? 2 : 1)), 256, 0, s>>>(nb, rows, d.H, n_rblk, per);
  return hipGetLastError();
}

// Y = X B^T per g over n_g = B*H matrices of `rows` rows; bt_trans (float32
// only) reads B^T from a row-major B instead.
hipError_t nt_gemm(const Dims& d, const void* x, int rows, bool x_per_head, const void* bt,
                   bool bt_per_head, bool bt_trans, const Epi& ep, hipStream_t s) {
  const long n_g = (long)d.B * d.H;
  if (use_mfma(d)) {
    if (bt_trans) return hipErrorInvalidValue;
    return nt_gemm_batch(d, rows, nt_prob(x, x_per_head, bt, bt_per_head, ep), nullptr, s);
  } else {
    const long n_out = n_g * rows * d.D;
    nt_gemm_f32_k<<<blocks(n_out, 256), 256, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(bt), ep, rows, d.D, d.H,
        x_per_head ? 1 : 0, bt_per_head ? 1 : 0, bt_trans ? 1 : 0, n_out);
  }
  return hipGetLastError();
}

// Tokens per partial of the X^T Y reduction: a multiple of 64 chosen so that
// the partial workgroups (four quadrants per chunk) number about two per
// compute unit.
int xty_chunk(const Dims& d) {
  const long n_g = (long)d.B * d.H;
  const long sub = (d.T + XTY_SUB - 1) / XTY_SUB;
  const long want = std::max(1L, std::min(sub, (512 + 4 * n_g - 1) / (4 * n_g)));
  return (int)(((sub + want - 1) / want) * XTY_SUB);
}

size_t xty_ws_bytes(const Dims& d) {
  if (!use_mfma(d)) return 0;
  const long nch = (d.T + xty_chunk(d) - 1) / xty_chunk(d);
  return (size_t)d.B * d.H * nch * HD * HD * sizeof(float);
}

// One X^T Y reduction: out (+)= gamma * base + delta * sum_t X^T Y, per
// (b, h) or summed over b into per-head outputs.
struct XtyJob {
  const void* x;
  const void* y;
  float* out;
  bool sum_b;
  const float* base_mat;
  const float* gamma;
  float delta;
};

hipError_t xty(const Dims& d, const void* x, const void* y, float* out, bool sum_b,
               const float* base_mat, const float* gamma, float delta, bool accumulate, void* ws,
               hipStream_t s);

// Up to three reductions of one shape in two launches (bf16 MFMA; ws holds
// n_jobs x xty_ws_bytes); float32 runs them one after the other.
hipError_t xty_batch(const Dims& d, const XtyJob* jobs, int n_jobs, bool accumulate, void* ws,
                     hipStream_t s) {
  if (!use_mfma(d)) {
    for (int j = 0; j < n_jobs; ++j) {
      const XtyJob& J = jobs[j];
      hipError_t e = xty(d, J.x, J.y, J.out, J.sum_b, J.base_mat, J.gamma, J.delta, accumulate,
                         ws, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int chunk = xty_chunk(d);
  const int nch = (d.T + chunk - 1) / chunk;
  const long per = (long)d.B * d.H * nch * 4;
  auto bx = [&](int j) { return static_cast<const __bf16*>(jobs[j < n_jobs ? j : 0].x); };
  auto by = [&](int j) { return static_cast<const __bf16*>(jobs[j < n_jobs ? j : 0].y); };
  const XtyBatch xb{bx(0), by(0), bx(1), by(1), bx(2), by(2)};
  float* part = static_cast<float*>(ws);
  xty_part_mfma_k<<<(unsigned)(per * n_jobs), 256, 0, s>>>(xb, part, d.T, chunk, nch, per);
  XtyRed r[3];
  long total = 0;
  for (int j = 0; j < 3; ++j) {
    if (j < n_jobs) {
      const XtyJob& J = jobs[j];
      r[j] = XtyRed{J.out, J.base_mat, J.gamma, J.delta, J.sum_b ? 1 : 0,
                    (J.sum_b ? (long)d.H : (long)d.B * d.H) * 4096};
    } else {
      r[j] = XtyRed{nullptr, nullptr, nullptr, 0.f, 0, 0};
    }
    total += r[j].n_thr;
  }
  xty_reduce_mfma_k<<<blocks(total, 256), 256, 0, s>>>(part, XtyRedBatch{r[0], r[1], r[2]},
                                                       accumulate ? 1 : 0, nch, d.B, d.H,
                                                       per * 4096);
  return hipGetLastError();
}

// out (+)= gamma * base + delta * sum_t X^T Y, per (b, h) or summed over b
// into per-head outputs.
hipError_t xty(const Dims& d, const void* x, const void* y, float* out, bool sum_b,
               const float* base_mat, const float* gamma, float delta, bool accumulate, void* ws,
               hipStream_t s) {
  const long n_go = sum_b ? d.H : (long)d.B * d.H;
  if (use_mfma(d)) {
    const XtyJob job{x, y, out, sum_b, base_mat, gamma, delta};
    return xty_batch(d, &job, 1, accumulate, ws, s);
  } else {
    const long n_out = n_go * d.D * d.D;
    xty_f32_k<<<blocks(n_out, 256), 256, 0, s>>>(
        static_cast<const float*>(x), static_cast<const float*>(y), out, base_mat, gamma, delta,
        accumulate ? 1 : 0, d.T, d.D, d.B, d.H, sum_b ? 1 : 0, n_out);
  }
  return hipGetLastError();
}

// Scratch carved from the caller's workspace in a fixed order; with a null
// base it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename P>
  P* take(size_t bytes) {
    off = round_up(off, 256);
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

size_t act_elem(const Dims& d) { return d.bf16 ? 2 : 4; }
size_t mat_count(const Dims& d) { return (size_t)d.B * d.H * d.D * d.D; }
size_t row_count(const Dims& d) { return (size_t)d.B * d.H * d.T; }

hipError_t feature_map_any(const Dims& d, const void* x, const void* phi, void* out, bool norm,
                           hipStream_t s) {
  return use_mfma(d) ? mfma_feature_map(d, x, phi, out, norm, s)
                     : generic_feature_map(d, x, phi, out, norm, s);
}

// With the rows' log-sum-exp given (natural log, from the forward): lse2 =
// lse log2(e) and dsum = dO . O_intra, 16 rows per workgroup (16 lanes of 8
// features per row).
__global__ void __launch_bounds__(256)
attn_dsum_mfma_k(const __bf16* __restrict__ o, const __bf16* __restrict__ d_o,
                 const float* __restrict__ lse_in, float* __restrict__ lse2,
                 float* __restrict__ dsum, long n_rows) {
  const long r = (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int p = threadIdx.x & 15;
  float dd = 0.f;
  if (r < n_rows) {
    const bf16x8 x = ld8(d_o + r * HD + 8 * p), y = ld8(o + r * HD + 8 * p);
#pragma unroll
    for (int e = 0; e < 8; ++e) dd = fmaf((float)x[e], (float)y[e], dd);
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) dd += __shfl_xor(dd, w, 16);
  if (r < n_rows && p == 0) {
    dsum[r] = dd;
    lse2[r] = lse_in[r] * kLog2e;
  }
}

// lse, dsum, then dQ (with the inter term dO M^T on bf16 shapes when m_rows is
// given), dK and dV.
hipError_t attn_backward_steps(const Dims& d, const void* q, const void* k, const void* v,
                               const void* o_intra, const void* d_o, void* dq, void* dk, void* dv,
                               const void* m_rows, bool accumulate, Carve& c, hipStream_t s,
                               const float* lse_in = nullptr) {
  const long n_rows = (long)row_count(d);
  float* lse = c.take<float>(n_rows * sizeof(float));
  float* dsum = c.take<float>(n_rows * sizeof(float));
  // One-grid dQ + dK/dV (2-wave workgroups of 64 rows) on shapes with fewer
  // than 512 blocks of 128 rows; its dK/dV split over query halves from 4
  // query stages up, with two fp32 slots and a counter per key block.
  const long n_g = (long)d.B * d.H;
  const bool small_grid = use_mfma(d) && n_g * ((d.T + 127) / 128) < 512;
  const long n_kb = n_g * ((d.T + 63) / 64);
  const bool split = small_grid && (d.T + AB_STAGE - 1) / AB_STAGE >= 4;
  PairSplit ps{nullptr, nullptr, 0};
  if (split) {
    ps.slots = c.take<float>((size_t)2 * n_kb * 2 * 8192 * sizeof(float));
    ps.ctr = c.take<unsigned long long>((size_t)n_kb * sizeof(unsigned long long));
  }
  if (!c.base) return hipSuccess;
  const int acc = accumulate ? 1 : 0;
  if (lse_in && use_mfma(d))
    attn_dsum_mfma_k<<<blocks(n_rows, 16), 256, 0, s>>>(
        static_cast<const __bf16*>(o_intra), static_cast<const __bf16*>(d_o), lse_in, lse, dsum,
        n_rows);
  if (use_mfma(d)) {
    const float cl = d.scale * kLog2e;
    const __bf16* qb = static_cast<const __bf16*>(q);
    const __bf16* kb = static_cast<const __bf16*>(k);
    const __bf16* vb = static_cast<const __bf16*>(v);
    const __bf16* ob = static_cast<const __bf16*>(d_o);
    const __bf16* oi = static_cast<const __bf16*>(o_intra);
    const __bf16* mr = static_cast<const __bf16*>(m_rows);
    // dQ and dK/dV: 4-wave workgroups (128 rows) when they fill the chip twice
    // over, else 2-wave ones (64 rows) for twice as many, in one grid; the row
    // statistics always in 4-wave workgroups
    if (!small_grid) {
      const int nb = (d.T + 127) / 128;
      const unsigned grid = (unsigned)(n_g * nb);
      if (!lse_in) attn_pre_mfma_k<4><<<grid, 256, 0, s>>>(qb, kb, oi, ob, lse, dsum, d.T, cl, nb);
      attn_dq_mfma_k<4><<<grid, 256, 0, s>>>(qb, kb, vb, ob, lse, dsum, mr,
                                             static_cast<__bf16*>(dq), d.T, cl, d.scale, nb, acc);
      attn_dkdv_mfma_k<4><<<grid, 256, 0, s>>>(qb, kb, vb, ob, lse, dsum,
                                               static_cast<__bf16*>(dk), static_cast<__bf16*>(dv),
                                               d.T, cl, d.scale, nb, acc);
    } else {
      const int nb = (d.T + 63) / 64;
      const unsigned grid = (unsigned)(n_g * nb);
      const int nb4 = (d.T + 127) / 128;
      if (!lse_in)
        attn_pre_mfma_k<4><<<(unsigned)(n_g * nb4), 256, 0, s>>>(qb, kb, oi, ob, lse, dsum, d.T,
                                                                cl, nb4);
      if (split) {
        static std::atomic<unsigned long long> g_pair_tag{0};
        ps.tag = (++g_pair_tag) | (1ull << 63);
      }
      const unsigned grid2 = grid + (split ? 2u : 1u) * grid;
      attn_dqdkdv_mfma_k<2><<<grid2, 128, 0, s>>>(
          qb, kb, vb, ob, lse, dsum, mr, static_cast<__bf16*>(dq), static_cast<__bf16*>(dk),
          static_cast<__bf16*>(dv), d.T, cl, d.scale, nb, (int)grid, acc, ps);
    }
  } else {
    const float* qf = static_cast<const float*>(q);
    const float* kf = static_cast<const float*>(k);
    const float* vf = static_cast<const float*>(v);
    const float* of = static_cast<const float*>(d_o);
    const long n_el = n_rows * d.D;
    if (lse_in) lse = const_cast<float*>(lse_in);     // read only below
    attn_pre_f32_k<<<blocks(n_rows, 128), 128, 0, s>>>(lse_in ? nullptr : qf, kf,
                                                       static_cast<const float*>(o_intra), of,
                                                       lse, dsum, d.T, d.D, d.scale, n_rows);
    attn_dq_f32_k<<<blocks(n_el, 128), 128, 0, s>>>(qf, kf, vf, of, lse, dsum,
                                                    static_cast<float*>(dq), d.T, d.D, d.scale,
                                                    acc, n_el);
    attn_dkdv_f32_k<<<blocks(n_el, 128), 128, 0, s>>>(qf, kf, vf, of, lse, dsum,
                                                      static_cast<float*>(dk),
                                                      static_cast<float*>(dv), d.T, d.D, d.scale,
                                                      acc, n_el);
  }
  return hipGetLastError();
}

hipError_t read_backward_steps(const Dims& d, const void* q, const void* k, const void* v,
                               const void* phi_q, const float* S, const void* o_intra,
                               const void* d_o, void* dq, void* dk, void* dv, float* dphi_q,
                               float* dS, bool accumulate, Carve& c, hipStream_t s,
                               const float* lse_in = nullptr) {
  const size_t ab = act_bytes(d);
  const bool mf = use_mfma(d);
  __bf16* Sb = mf ? c.take<__bf16>(mat_count(d) * 2) : nullptr;
  __bf16* Stb = mf ? c.take<__bf16>(mat_count(d) * 2) : nullptr;
  void* Mm = c.take<char>(mat_count(d) * (mf ? 2 : 4));     // M = Phi_q S per (b, h)
  void* qp = c.take<char>(ab);
  void* dqp = c.take<char>(ab);
  void* part = c.take<char>(2 * xty_ws_bytes(d));
  hipError_t e;
  if (c.base) {
    if (mf) {
      to_bf16_pair_k<<<blocks((long)mat_count(d), 256), 256, 0, s>>>(
          S, Sb, Stb, nullptr, nullptr, nullptr, (long)mat_count(d));
      // M[e][v] = sum_d Phi_q[e][d] S[d][v]: rows of Phi_q against S^T
      e = nt_gemm(d, phi_q, HD, true, Stb, false, false, make_epi(nullptr, false, nullptr, Mm, false), s);
    } else {
      e = nt_gemm(d, phi_q, d.D, true, S, false, true,
                  make_epi(nullptr, false, static_cast<float*>(Mm), nullptr, false), s);
    }
    if (e != hipSuccess) return e;
  }
  e = attn_backward_steps(d, q, k, v, o_intra, d_o, dq, dk, dv, mf ? Mm : nullptr, accumulate, c, s,
                          lse_in);
  if (e != hipSuccess || !c.base) return e;
  if (!mf) {
    // dQ += dO M^T
    e = nt_gemm(d, d_o, d.T, false, Mm, false, false, make_epi(nullptr, false, nullptr, dq, true), s);
    if (e != hipSuccess) return e;
  }
  // Q' = Q Phi_q, dQ' = dO S^T; then dS (+)= Q'^T dO and dPhi_q (+)= sum_b Q^T dQ'
  if ((e = feature_map_any(d, q, phi_q, qp, false, s)) != hipSuccess) return e;
  e = nt_gemm(d, d_o, d.T, false, mf ? (const void*)Sb : (const void*)S, false, false,
              make_epi(nullptr, false, nullptr, dqp, false), s);
  if (e != hipSuccess) return e;
  const XtyJob jobs[2] = {{qp, d_o, dS, false, nullptr, nullptr, 1.f},
                          {q, dqp, dphi_q, true, nullptr, nullptr, 1.f}};
  return xty_batch(d, jobs, 2, accumulate, part, s);
}

hipError_t commit_backward_steps(const Dims& d, const void* k, const void* v, const void* phi_k,
                                 const void* phi_v, const float* beta, const float* alpha,
                                 const float* S, const float* G, void* dk, void* dv,
                                 float* dphi_k, float* dphi_v, float* dbeta, float* dalpha,
                                 float* dS_prev, bool accumulate, Carve& c, hipStream_t s) {
  const size_t ab = act_bytes(d);
  const size_t fb = row_count(d) * d.D * sizeof(float);
  const bool mf = use_mfma(d);
  void* kt = mf ? nullptr : c.take<char>(ab);   // K Phi_k (the MFMA map normalises in place)
  void* kp = c.take<char>(ab);            // K'
  float* nrm = c.take<float>(row_count(d) * sizeof(float));
  void* vp = c.take<char>(ab);            // V'
  // (the fp32 intermediates only on the float path: the MFMA path keeps them
  // in the workgroups that form them)
  float* r32 = mf ? nullptr : c.take<float>(fb);    // R = V' - K'S
  void* rx = c.take<char>(ab);
  float* kg32 = mf ? nullptr : c.take<float>(fb);   // K'G
  void* kgx = c.take<char>(ab);
  void* dvx = c.take<char>(ab);           // dV'
  float* dkr = mf ? nullptr : c.take<float>(fb);    // R G^T - K'G S^T
  void* dktx = c.take<char>(ab);          // dK~
  __bf16* Sb = mf ? c.take<__bf16>(mat_count(d) * 2) : nullptr;
  __bf16* Stb = mf ? c.take<__bf16>(mat_count(d) * 2) : nullptr;
  __bf16* Gb = mf ? c.take<__bf16>(mat_count(d) * 2) : nullptr;
  __bf16* Gtb = mf ? c.take<__bf16>(mat_count(d) * 2) : nullptr;
  void* part = c.take<char>(3 * xty_ws_bytes(d));
  if (!c.base) return hipSuccess;
  const long n_rows = (long)row_count(d);
  const int acc = accumulate ? 1 : 0;
  hipError_t e;
  if (mf) {
    // K' = rownorm(K Phi_k) with its rows' norms, and V' = V Phi_v, in one launch
    const FeatureMapJob jobs[2] = {{k, phi_k, kp, true, nrm}, {v, phi_v, vp, false}};
    if ((e = mfma_feature_maps(d, jobs, 2, s)) != hipSuccess) return e;
  } else {
    if ((e = feature_map_any(d, k, phi_k, kt, false, s)) != hipSuccess) return e;
    if ((e = feature_map_any(d, v, phi_v, vp, false, s)) != hipSuccess) return e;
  }
  if (mf) {
    // bf16 copies of S and G, and dalpha = <S, G> per (b, h), in one launch
    const long cast_blocks = blocks(2 * (long)mat_count(d), 256);
    to_bf16_pair_k<<<(unsigned)(cast_blocks + (long)d.B * d.H), 256, 0, s>>>(
        S, Sb, Stb, G, Gb, Gtb, (long)mat_count(d), dalpha, cast_blocks, acc);
  } else {
    rownorm_k<float><<<blocks(n_rows, 4), 256, 0, s>>>(static_cast<const float*>(kt),
                                                         static_cast<float*>(kp), nrm, d.D, n_rows);
  }
  const int n_rblk = (d.T + 31) / 32;
  const unsigned row_grid = (unsigned)((long)d.B * d.H * n_rblk);
  if (mf) {
    // R = V' - K'S and K'G, then dbeta and dV' = beta K'G, in one launch
    commit_resid_rows_k<<<row_grid, 256, 0, s>>>(
        static_cast<const __bf16*>(kp), Stb, Gtb, static_cast<const __bf16*>(vp), beta,
        static_cast<__bf16*>(rx), static_cast<__bf16*>(kgx), static_cast<__bf16*>(dvx), dbeta,
        d.T, d.H, n_rblk, acc);
    // dKraw = R G^T - K'G S^T and dK~ through beta and the row normalisation
    commit_dkt_rows_k<<<row_grid, 256, 0, s>>>(
        static_cast<const __bf16*>(rx), Gb, static_cast<const __bf16*>(kgx), Sb,
        static_cast<const __bf16*>(kp), nrm, beta, static_cast<__bf16*>(dktx), d.T, d.H, n_rblk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    // R = V' - K' S ;  K'G
    e = nt_gemm(d, kp, d.T, false, S, false, true, make_epi(vp, false, r32, rx, false), s);
    if (e != hipSuccess) return e;
    e = nt_gemm(d, kp, d.T, false, G, false, true, make_epi(nullptr, false, kg32, kgx, false), s);
    if (e != hipSuccess) return e;
    // dbeta, dV' = beta K'G
    commit_rows1_k<float><<<blocks(n_rows, 4), 256, 0, s>>>(kg32, r32, beta, dbeta,
                                                              static_cast<float*>(dvx), d.D, acc,
                                                              n_rows);
    // dKraw = R G^T - K'G S^T
    e = nt_gemm(d, rx, d.T, false, G, false, false, make_epi(nullptr, false, dkr, nullptr, false), s);
    if (e != hipSuccess) return e;
    e = nt_gemm(d, kgx, d.T, false, S, false, false, make_epi(dkr, true, dkr, nullptr, false), s);
    if (e != hipSuccess) return e;
    // dK~ through beta and the row normalisation
    commit_rows2_k<float><<<blocks(n_rows, 4), 256, 0, s>>>(
        dkr, static_cast<const float*>(kp), nrm, beta, static_cast<float*>(dktx), d.D, n_rows);
  }
  // dK = dK~ Phi_k^T, dV = dV' Phi_v^T
  if (mf) {
    const NtProb p1 = nt_prob(dvx, false, phi_v, true,
                              make_epi(nullptr, false, nullptr, dv, accumulate));
    e = nt_gemm_batch(d, d.T, nt_prob(dktx, false, phi_k, true,
                                      make_epi(nullptr, false, nullptr, dk, accumulate)),
                      &p1, s);
  } else {
    e = nt_gemm(d, dktx, d.T, false, phi_k, true, false, make_epi(nullptr, false, nullptr, dk, accumulate), s);
    if (e != hipSuccess) return e;
    e = nt_gemm(d, dvx, d.T, false, phi_v, true, false, make_epi(nullptr, false, nullptr, dv, accumulate), s);
  }
  if (e != hipSuccess) return e;
  // dPhi_k = sum_b K^T dK~, dPhi_v = sum_b V^T dV', dS_prev = alpha G - K'^T dV'
  const XtyJob jobs[3] = {{k, dktx, dphi_k, true, nullptr, nullptr, 1.f},
                          {v, dvx, dphi_v, true, nullptr, nullptr, 1.f},
                          {kp, dvx, dS_prev, false, G, alpha, -1.f}};
  if ((e = xty_batch(d, jobs, 3, accumulate, part, s)) != hipSuccess) return e;
  if (!mf) dalpha_k<<<(unsigned)((long)d.B * d.H), 256, 0, s>>>(S, G, dalpha, d.D * d.D, acc);
  return hipGetLastError();
}

}  // namespace

size_t attn_backward_ws_bytes(const Dims& d) {
  Carve c(nullptr);
  (void)attn_backward_steps(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, false, c, nullptr);
  return c.off;
}
size_t read_backward_ws_bytes(const Dims& d) {
  Carve c(nullptr);
  (void)read_backward_steps(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, nullptr, nullptr, nullptr, false, c, nullptr);
  return c.off;
}
size_t commit_backward_ws_bytes(const Dims& d) {
  Carve c(nullptr);
  (void)commit_backward_steps(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false, c,
                        nullptr);
  return c.off;
}

hipError_t attn_backward(const Dims& d, const void* q, const void* k, const void* v,
                         const void* o_intra, const float* lse, const void* d_o, void* dq,
                         void* dk, void* dv, bool accumulate, void* ws, hipStream_t s) {
  Carve c(ws);
  return attn_backward_steps(d, q, k, v, o_intra, d_o, dq, dk, dv, nullptr, accumulate, c, s, lse);
}

hipError_t attn_lse_f32(const Dims& d, const void* q, const void* k, float* lse, hipStream_t s) {
  const long n_rows = (long)row_count(d);
  attn_pre_f32_k<<<blocks(n_rows, 128), 128, 0, s>>>(static_cast<const float*>(q),
                                                     static_cast<const float*>(k), nullptr,
                                                     nullptr, lse, nullptr, d.T, d.D, d.scale,
                                                     n_rows);
  return hipGetLastError();
}

hipError_t read_backward(const Dims& d, const void* q, const void* k, const void* v,
                         const void* phi_q, const float* S, const void* o_intra, const float* lse,
                         const void* d_o, void* dq, void* dk, void* dv, float* dphi_q, float* dS,
                         bool accumulate, void* ws, hipStream_t s) {
  Carve c(ws);
  return read_backward_steps(d, q, k, v, phi_q, S, o_intra, d_o, dq, dk, dv, dphi_q, dS,
                             accumulate, c, s, lse);
}

hipError_t commit_backward(const Dims& d, const void* k, const void* v, const void* phi_k,
                           const void* phi_v, const float* beta, const float* alpha,
                           const float* S_prev, const float* dS_next, void* dk, void* dv,
                           float* dphi_k, float* dphi_v, float* dbeta, float* dalpha,
                           float* dS_prev, bool accumulate, void* ws, hipStream_t s) {
  Carve c(ws);
  return commit_backward_steps(d, k, v, phi_k, phi_v, beta, alpha, S_prev, dS_next, dk, dv,
                               dphi_k, dphi_v, dbeta, dalpha, dS_prev, accumulate, c, s);
}

hipError_t copy_state(const float* src, float* dst, size_t n, hipStream_t s) {
  copy_f32_k<<<blocks((long)n, 256), 256, 0, s>>>(src, dst, (long)n);
  return hipGetLastError();
}

}  // namespace arl2
