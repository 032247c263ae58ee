// Scalar-FMA kernels of the ARL2 hybrid attention step, for any supported
// head dimension (16, 32, 64, 128) and either activation type (float32 or
// bfloat16), always accumulating in float32. They carry the float32
// workloads; bf16 at D = 128 runs on the MFMA kernels instead.
//
// Step definitions: "Attend Locally, Remember Linearly" technical summary,
// §2.1 (feature maps, intra-frame softmax, read O_inter = Q'S, gated delta
// update) and §2.2 (frame-level access, clean-pass update).
#include <math.h>

#include "arl2_internal.h"

namespace arl2 {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld(const __bf16* p, size_t i) { return (float)p[i]; }
__device__ __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(__bf16* p, size_t i, float v) { p[i] = (__bf16)v; }

// ---------------------------------------------------------------------------
// a1: out[row, j] = sum_i x[row, i] * phi[h, i, j]; optional row L2 norm.
// Block: 256 threads = R rows x D columns.
template <typename TI, int D>
__global__ void __launch_bounds__(256)
feature_map_k(const TI* __restrict__ x, const TI* __restrict__ phi,
              TI* __restrict__ out, int H, int T, long rows, int normalize) {
  constexpr int R = 256 / D;
  __shared__ float xs[R][D];
  __shared__ float sq[R][D];
  const int j = threadIdx.x % D;
  const int r = threadIdx.x / D;
  const long row = (long)blockIdx.x * R + r;
  const bool valid = row < rows;
  const int h = valid ? (int)((row / T) % H) : 0;
  xs[r][j] = valid ? ld(x, (size_t)row * D + j) : 0.f;
  __syncthreads();
  float acc = 0.f;
  const TI* ph = phi + (size_t)h * D * D + j;
#pragma unroll 8
  for (int i = 0; i < D; ++i) acc = fmaf(xs[r][i], ld(ph, (size_t)i * D), acc);
  if (normalize) {
    sq[r][j] = acc * acc;
    __syncthreads();
    float ss = 0.f;
    for (int i = 0; i < D; ++i) ss += sq[r][i];   // same fixed order in every thread
    acc = acc / fmaxf(sqrtf(ss), 1e-12f);
  }
  if (valid) st(out, (size_t)row * D + j, acc);
}

// ---------------------------------------------------------------------------
// a2 / comparator: one thread per query row, keys staged through LDS in
// tiles of KT; online softmax in the log2 domain with the scale folded into q.
template <typename TI, int D>
__global__ void __launch_bounds__(64)
attention_k(const TI* __restrict__ q, const TI* __restrict__ k,
            const TI* __restrict__ v, TI* __restrict__ o, int T, int n_kv,
            long kv_cap, float scale_log2) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const long bh = blockIdx.y;
  const int t = blockIdx.x * 64 + threadIdx.x;
  const bool valid = t < T;
  const TI* kh = k + (size_t)bh * kv_cap * D;
  const TI* vh = v + (size_t)bh * kv_cap * D;
  float qr[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = valid ? ld(q, ((size_t)bh * T + t) * D + d) * scale_log2 : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k0 = 0; k0 < n_kv; k0 += KT) {
    __syncthreads();
    for (int e = threadIdx.x; e < KT * D; e += 64) {
      const int kk = e / D, dd = e % D, key = k0 + kk;
      ks[kk][dd] = key < n_kv ? ld(kh, (size_t)key * D + dd) : 0.f;
      vs[kk][dd] = key < n_kv ? ld(vh, (size_t)key * D + dd) : 0.f;
    }
    __syncthreads();
    const int nk = min(KT, n_kv - k0);
    float s[KT];
    float mt = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(qr[d], ks[kk][d], dot);
      s[kk] = kk < nk ? dot : -INFINITY;
      mt = fmaxf(mt, s[kk]);
    }
    const float mn = fmaxf(m, mt);
    const float corr = exp2f(m - mn);          // 0 on the first tile
    l *= corr;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= corr;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) {
      const float p = exp2f(s[kk] - mn);       // 0 for masked keys
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[kk][d], acc[d]);
    }
    m = mn;
  }
  if (valid) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) st(o, ((size_t)bh * T + t) * D + d, acc[d] * inv);
  }
}

// ---------------------------------------------------------------------------
// a3 + a4: o[row, j] = o_intra[row, j] + sum_i q'[row, i] S[bh, i, j]
template <typename TI, int D>
__global__ void __launch_bounds__(256)
inter_read_k(const TI* __restrict__ qp, const float* __restrict__ S,
             const TI* o_intra, TI* o, TI* __restrict__ o_inter, int T,
             long rows) {
  constexpr int R = 256 / D;
  __shared__ float xs[R][D];
  const int j = threadIdx.x % D;
  const int r = threadIdx.x / D;
  const long row = (long)blockIdx.x * R + r;
  const bool valid = row < rows;
  const long bh = valid ? row / T : 0;
  xs[r][j] = valid ? ld(qp, (size_t)row * D + j) : 0.f;
  __syncthreads();
  if (!valid) return;
  const float* Sh = S + (size_t)bh * D * D + j;
  float acc = 0.f;
#pragma unroll 8
  for (int i = 0; i < D; ++i) acc = fmaf(xs[r][i], Sh[(size_t)i * D], acc);
  const size_t idx = (size_t)row * D + j;
  if (o_inter) st(o_inter, idx, acc);
  const float base = o_intra ? ld(o_intra, idx) : 0.f;
  st(o, idx, base + acc);
}

// ---------------------------------------------------------------------------
// a5, part 1: W[row, j] = beta[row] * (v'[row, j] - sum_i k'[row, i] S[bh, i, j])
template <typename TI, int D>
__global__ void __launch_bounds__(256)
commit_residual_k(const TI* __restrict__ kp, const TI* __restrict__ vp,
                  const float* __restrict__ beta, const float* __restrict__ S,
                  float* __restrict__ W, int T, long rows) {
  constexpr int R = 256 / D;
  __shared__ float xs[R][D];
  const int j = threadIdx.x % D;
  const int r = threadIdx.x / D;
  const long row = (long)blockIdx.x * R + r;
  const bool valid = row < rows;
  const long bh = valid ? row / T : 0;
  xs[r][j] = valid ? ld(kp, (size_t)row * D + j) : 0.f;
  __syncthreads();
  if (!valid) return;
  const float* Sh = S + (size_t)bh * D * D + j;
  float pred = 0.f;
#pragma unroll 8
  for (int i = 0; i < D; ++i) pred = fmaf(xs[r][i], Sh[(size_t)i * D], pred);
  const size_t idx = (size_t)row * D + j;
  W[idx] = beta[row] * (ld(vp, idx) - pred);
}

// a5, part 2: S_next[bh, i, j] = alpha[bh] S_prev[bh, i, j] + sum_t k'[t, i] W[t, j],
// summed over t in order.
template <typename TI, int D>
__global__ void __launch_bounds__(256)
commit_update_k(const TI* __restrict__ kp, const float* __restrict__ W,
                const float* __restrict__ alpha, const float* __restrict__ S_prev,
                float* __restrict__ S_next, int T, long n_state) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n_state) return;
  const long bh = e / (D * D);
  const int i = (int)((e / D) % D);
  const int j = (int)(e % D);
  const TI* kh = kp + (size_t)bh * T * D + i;
  const float* wh = W + (size_t)bh * T * D + j;
  float acc = 0.f;
  for (int t = 0; t < T; ++t) acc = fmaf(ld(kh, (size_t)t * D), wh[(size_t)t * D], acc);
  S_next[e] = fmaf(alpha[bh], S_prev[e], acc);
}

// M[bh, i, j] = sum_k phi[h, i, k] S[bh, k, j]  (k summed in order)
template <typename TI>
__global__ void __launch_bounds__(256)
read_prepare_k(const TI* __restrict__ phi, const float* __restrict__ S, float* __restrict__ M,
               int H, int D, long n) {
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const long bh = e / ((long)D * D);
  const int i = (int)((e / D) % D);
  const int j = (int)(e % D);
  const TI* ph = phi + ((size_t)(bh % H) * D + i) * D;
  const float* Sh = S + (size_t)bh * D * D + j;
  float acc = 0.f;
  for (int k = 0; k < D; ++k) acc = fmaf(ld(ph, k), Sh[(size_t)k * D], acc);
  M[e] = acc;
}

template <typename TI>
hipError_t feature_map_d(const Dims& d, const void* x, const void* phi, void* out,
                         bool norm, hipStream_t s) {
  const long rows = (long)d.B * d.H * d.T;
  const int R = 256 / d.D;
  const dim3 grid((unsigned)((rows + R - 1) / R));
  auto* X = static_cast<const TI*>(x);
  auto* P = static_cast<const TI*>(phi);
  auto* O = static_cast<TI*>(out);
  switch (d.D) {
    case 16: feature_map_k<TI, 16><<<grid, 256, 0, s>>>(X, P, O, d.H, d.T, rows, norm); break;
    case 32: feature_map_k<TI, 32><<<grid, 256, 0, s>>>(X, P, O, d.H, d.T, rows, norm); break;
    case 64: feature_map_k<TI, 64><<<grid, 256, 0, s>>>(X, P, O, d.H, d.T, rows, norm); break;
    case 128: feature_map_k<TI, 128><<<grid, 256, 0, s>>>(X, P, O, d.H, d.T, rows, norm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TI>
hipError_t attention_d(const Dims& d, const void* q, const void* k, const void* v,
                       void* o, int64_t n_kv, int64_t kv_cap, hipStream_t s) {
  const dim3 grid((unsigned)((d.T + 63) / 64), (unsigned)(d.B * d.H));
  const float sl2 = d.scale * kLog2e;
  auto* Q = static_cast<const TI*>(q);
  auto* K = static_cast<const TI*>(k);
  auto* V = static_cast<const TI*>(v);
  auto* O = static_cast<TI*>(o);
  const int nk = (int)n_kv;
  switch (d.D) {
    case 16: attention_k<TI, 16><<<grid, 64, 0, s>>>(Q, K, V, O, d.T, nk, kv_cap, sl2); break;
    case 32: attention_k<TI, 32><<<grid, 64, 0, s>>>(Q, K, V, O, d.T, nk, kv_cap, sl2); break;
    case 64: attention_k<TI, 64><<<grid, 64, 0, s>>>(Q, K, V, O, d.T, nk, kv_cap, sl2); break;
    case 128: attention_k<TI, 128><<<grid, 64, 0, s>>>(Q, K, V, O, d.T, nk, kv_cap, sl2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TI>
hipError_t inter_read_d(const Dims& d, const void* qp, const float* S, const void* oi,
                        void* o, void* oe, hipStream_t s) {
  const long rows = (long)d.B * d.H * d.T;
  const int R = 256 / d.D;
  const dim3 grid((unsigned)((rows + R - 1) / R));
  auto* Q = static_cast<const TI*>(qp);
  auto* OI = static_cast<const TI*>(oi);
  auto* O = static_cast<TI*>(o);
  auto* OE = static_cast<TI*>(oe);
  switch (d.D) {
    case 16: inter_read_k<TI, 16><<<grid, 256, 0, s>>>(Q, S, OI, O, OE, d.T, rows); break;
    case 32: inter_read_k<TI, 32><<<grid, 256, 0, s>>>(Q, S, OI, O, OE, d.T, rows); break;
    case 64: inter_read_k<TI, 64><<<grid, 256, 0, s>>>(Q, S, OI, O, OE, d.T, rows); break;
    case 128: inter_read_k<TI, 128><<<grid, 256, 0, s>>>(Q, S, OI, O, OE, d.T, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename TI, int D>
hipError_t state_commit_dd(const Dims& d, const void* kp, const void* vp, const float* beta,
                           const float* alpha, const float* Sp, float* Sn, void* ws,
                           hipStream_t s) {
  const long rows = (long)d.B * d.H * d.T;
  constexpr int R = 256 / D;
  float* W = static_cast<float*>(ws);
  auto* KP = static_cast<const TI*>(kp);
  auto* VP = static_cast<const TI*>(vp);
  commit_residual_k<TI, D><<<(unsigned)((rows + R - 1) / R), 256, 0, s>>>(KP, VP, beta, Sp, W,
                                                                        d.T, rows);
  const long n_state = (long)d.B * d.H * D * D;
  commit_update_k<TI, D><<<(unsigned)((n_state + 255) / 256), 256, 0, s>>>(KP, W, alpha, Sp, Sn,
                                                                         d.T, n_state);
  return hipGetLastError();
}

template <typename TI>
hipError_t state_commit_d(const Dims& d, const void* kp, const void* vp, const float* beta,
                          const float* alpha, const float* Sp, float* Sn, void* ws,
                          hipStream_t s) {
  switch (d.D) {
    case 16: return state_commit_dd<TI, 16>(d, kp, vp, beta, alpha, Sp, Sn, ws, s);
    case 32: return state_commit_dd<TI, 32>(d, kp, vp, beta, alpha, Sp, Sn, ws, s);
    case 64: return state_commit_dd<TI, 64>(d, kp, vp, beta, alpha, Sp, Sn, ws, s);
    case 128: return state_commit_dd<TI, 128>(d, kp, vp, beta, alpha, Sp, Sn, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t generic_feature_map(const Dims& d, const void* x, const void* phi, void* out,
                               bool normalize, hipStream_t s) {
  return d.bf16 ? feature_map_d<__bf16>(d, x, phi, out, normalize, s)
                : feature_map_d<float>(d, x, phi, out, normalize, s);
}

hipError_t generic_attention(const Dims& d, const void* q, const void* k, const void* v,
                             void* o, int64_t n_kv, int64_t kv_cap, hipStream_t s) {
  return d.bf16 ? attention_d<__bf16>(d, q, k, v, o, n_kv, kv_cap, s)
                : attention_d<float>(d, q, k, v, o, n_kv, kv_cap, s);
}

hipError_t generic_inter_read(const Dims& d, const void* q_prime, const float* S,
                              const void* o_intra, void* o, void* o_inter, hipStream_t s) {
  return d.bf16 ? inter_read_d<__bf16>(d, q_prime, S, o_intra, o, o_inter, s)
                : inter_read_d<float>(d, q_prime, S, o_intra, o, o_inter, s);
}

hipError_t generic_read_prepare(const Dims& d, const void* phi_q, const float* S, float* m,
                                hipStream_t s) {
  const long n = (long)d.B * d.H * d.D * d.D;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (d.bf16)
    read_prepare_k<__bf16><<<grid, 256, 0, s>>>(static_cast<const __bf16*>(phi_q), S, m, d.H, d.D, n);
  else
    read_prepare_k<float><<<grid, 256, 0, s>>>(static_cast<const float*>(phi_q), S, m, d.H, d.D, n);
  return hipGetLastError();
}

size_t generic_state_commit_ws_bytes(const Dims& d) {
  return (size_t)d.B * d.H * d.T * d.D * sizeof(float);
}

hipError_t generic_state_commit(const Dims& d, const void* k_prime, const void* v_prime,
                                const float* beta, const float* alpha, const float* S_prev,
                                float* S_next, void* ws, hipStream_t s) {
  return d.bf16 ? state_commit_d<__bf16>(d, k_prime, v_prime, beta, alpha, S_prev, S_next, ws, s)
                : state_commit_d<float>(d, k_prime, v_prime, beta, alpha, S_prev, S_next, ws, s);
}

}  // namespace arl2
