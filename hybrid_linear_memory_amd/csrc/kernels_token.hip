// Token-level access: the alternative to frame-level access that the
// "Attend Locally, Remember Linearly" technical summary ablates (§4: token-level
// access degrades quality). Within a pass, token t reads the state left by the
// frame's earlier tokens, starting from S_{N-1}:
//   o_inter_t = q'_t S_{t-1},   S_t = S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1}),
// and the clean pass commits S_N = alpha S_{N-1} + (S_T - S_{N-1}).
//
// bf16, d = 128: the recurrence runs in chunks of TC tokens in closed form.
// With A = I + tril(diag(beta) K' K'^T, -1) over a chunk, W = A^-1 diag(beta) K'
// and U = A^-1 diag(beta) V' do not depend on the state, so every chunk forms
// them at once (tl_chunk_k, by forward substitution); a sequential pass over
// the chunks (tl_scan_k) then carries the state:
//   X = U - W S,  O_inter = Q' S + tril(Q' K'^T, -1) X,  S <- S + K'^T X.
// float32 (any supported d): one workgroup per (b, h) walks the tokens
// (tl_seq_k).
#include <math.h>

#include "arl2_internal.h"
#include "mfma_common.h"

namespace arl2 {
namespace {

constexpr int TC = 64;                      // tokens per chunk
constexpr int AP = TC + 4;                  // padded row of A in LDS (fp32, 16-byte rows)
constexpr int XP = TC + 8;                  // padded row of X^T in LDS (bf16)
constexpr int SP = HD + 8;                  // padded row of S^T in LDS (bf16)

// Row-read swizzled bf16 chunk of `rows` x 128 (256-byte rows) into LDS: chunk
// p of row r at (p ^ swz) where swz is swz_r (row reads) or swz_v (transposing
// reads); rows past `valid` are zero.
template <bool TR>
__device__ __forceinline__ void stage_rows(char* dst, const __bf16* src, int rows, int valid) {
  for (int idx = threadIdx.x; idx < rows * 16; idx += blockDim.x) {
    const int r = idx >> 4, p = idx & 15;
    uint4 val = {0u, 0u, 0u, 0u};
    if (r < valid) val = *reinterpret_cast<const uint4*>(src + (size_t)r * HD + 8 * p);
    *reinterpret_cast<uint4*>(dst + r * 256 + ((p ^ (TR ? swz_v(r) : swz_r(r))) << 4)) = val;
  }
}

__device__ __forceinline__ bf16x8 row_op(const char* base, int row, int kc, int h2) {
  return *reinterpret_cast<const bf16x8*>(base + row * 256 + (((2 * kc + h2) ^ swz_r(row)) << 4));
}

__device__ __forceinline__ bf16x8 f32_to_bf16x8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  bf16x8 r;
  r[0] = (__bf16)a.x; r[1] = (__bf16)a.y; r[2] = (__bf16)a.z; r[3] = (__bf16)a.w;
  r[4] = (__bf16)b.x; r[5] = (__bf16)b.y; r[6] = (__bf16)b.z; r[7] = (__bf16)b.w;
  return r;
}

// ---------------------------------------------------------------------------
// Chunk preparation. One workgroup (4 waves) per (b, h, chunk):
//   A = I + tril(diag(beta) K'K'^T, -1) into LDS, Pq = tril(Q'K'^T, -1) out,
//   W = A^-1 diag(beta) K' and U = A^-1 diag(beta) V' out (fp32), solved by
//   forward substitution: thread c < 128 owns column c of W, thread 128 + c
//   column c of U, with the column in registers.
// Workspace layout per (bh, chunk): W [TC][128], U [TC][128], Pq [TC][TC].
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
tl_chunk_k(const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
           const __bf16* __restrict__ vp, const float* __restrict__ beta,
           float* __restrict__ w_out, float* __restrict__ u_out, float* __restrict__ pq_out,
           int T, int n_ch) {
  __shared__ __attribute__((aligned(16))) char lk[TC * 256];
  __shared__ __attribute__((aligned(16))) char lq[TC * 256];
  __shared__ float la[TC * AP];
  __shared__ float lb[TC];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const long bh = blockIdx.x / n_ch;
  const int ch = blockIdx.x % n_ch;
  const int t0 = ch * TC;
  const int valid = min(TC, T - t0);
  const size_t row0 = (size_t)bh * T + t0;
  stage_rows<false>(lk, kp + row0 * HD, TC, valid);
  stage_rows<false>(lq, qp + row0 * HD, TC, valid);
  if (tid < TC) lb[tid] = tid < valid ? beta[row0 + tid] : 0.f;
  __syncthreads();

  // wave w: 32 x 32 tile (ti, tj) of K'K'^T and of Q'K'^T
  const int ti = wave >> 1, tj = wave & 1;
  f32x16 g = zero16(), pq = zero16();
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    const bf16x8 b = row_op(lk, 32 * tj + n, kc, h2);
    g = mfma32(row_op(lk, 32 * ti + n, kc, h2), b, g);
    pq = mfma32(row_op(lq, 32 * ti + n, kc, h2), b, pq);
  }
  const size_t cbase = (size_t)bh * n_ch + ch;
  float* pq_c = pq_out + cbase * TC * TC;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = 32 * ti + 8 * (r >> 2) + 4 * h2 + (r & 3), j = 32 * tj + n;
    la[i * AP + j] = i > j ? lb[i] * g[r] : 0.f;
    pq_c[i * TC + j] = i > j ? pq[r] : 0.f;
  }
  __syncthreads();

  // forward substitution, one column per thread: x = diag(beta) rhs first
  // (all loads in flight at once), then x_i -= sum_{j<i} A_ij x_j in order
  const int c = tid & 127;
  const bool is_u = tid >= 128;
  float x[TC];
#pragma unroll
  for (int i = 0; i < TC; ++i) {
    float rhs;
    if (is_u) {
      rhs = i < valid ? (float)vp[(row0 + i) * HD + c] : 0.f;
    } else {
      const __bf16* kr = reinterpret_cast<const __bf16*>(
          lk + i * 256 + (((c >> 3) ^ swz_r(i)) << 4));
      rhs = (float)kr[c & 7];
    }
    x[i] = lb[i] * rhs;
  }
#pragma unroll
  for (int i = 1; i < TC; ++i) {
    float acc = x[i];
#pragma unroll
    for (int j = 0; j < i; ++j) acc = fmaf(-la[i * AP + j], x[j], acc);
    x[i] = acc;
    // keep each row's LDS reads next to their use (bounds register pressure)
    __builtin_amdgcn_sched_barrier(0);
  }
  float* out = (is_u ? u_out : w_out) + cbase * TC * HD + c;
#pragma unroll
  for (int i = 0; i < TC; ++i) out[(size_t)i * HD] = x[i];
}

// ---------------------------------------------------------------------------
// Sequential pass over the chunks. One workgroup (4 waves) per (b, h, 32-column
// block cb of the state). Wave w holds state rows [32w, 32w + 32) of the block
// as an MFMA accumulator; per chunk:
//   X = U - W S (waves 0-1: tokens [32w, 32w + 32)),
//   O_inter = Q' S + Pq X (waves 0-1), o = o_intra + O_inter,
//   S += K'^T X (all waves; K' staged for transposing reads).
// The state reaches the B operands as S^T in bf16 through LDS, X as X^T.
// With S_next given, the end state commits S_next = alpha S_prev + (S_T - S_prev).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
tl_scan_k(const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
          const float* __restrict__ w_in, const float* __restrict__ u_in,
          const float* __restrict__ pq_in, const float* __restrict__ S_prev,
          const float* __restrict__ alpha, float* __restrict__ S_next,
          const __bf16* __restrict__ o_intra, __bf16* __restrict__ o,
          __bf16* __restrict__ o_inter, int T, int n_ch) {
  __shared__ __attribute__((aligned(16))) char lk[TC * 256];
  __shared__ __attribute__((aligned(16))) __bf16 st[32 * SP];
  __shared__ __attribute__((aligned(16))) __bf16 xt[32 * XP];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const long bh = blockIdx.x >> 2;
  const int cb = blockIdx.x & 3;
  const int col = 32 * cb + n;                       // this lane's state column
  const float* Sp = S_prev + (size_t)bh * HD * HD;
  // state rows 32 w + 8 (r / 4) + 4 h2 + r % 4 of column `col`
  f32x16 sacc;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    sacc[r] = Sp[(size_t)(32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HD + col];

  for (int ch = 0; ch < n_ch; ++ch) {
    const int t0 = ch * TC;
    const int valid = min(TC, T - t0);
    const size_t row0 = (size_t)bh * T + t0;
    const size_t cbase = (size_t)bh * n_ch + ch;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      st[n * SP + 32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3)] = (__bf16)sacc[r];
    stage_rows<true>(lk, kp + row0 * HD, TC, valid);
    __syncthreads();

    f32x16 xacc;
    if (wave < 2) {
      // X = U - W S for tokens [32 wave, 32 wave + 32) of the chunk
      const float* wr = w_in + (cbase * TC + 32 * wave + n) * HD + 8 * h2;
      f32x16 ws = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        ws = mfma32(f32_to_bf16x8(wr + 16 * kc),
                    *reinterpret_cast<const bf16x8*>(st + n * SP + 16 * kc + 8 * h2), ws);
      const float* ur = u_in + cbase * TC * HD + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = 32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3);
        xacc[r] = ur[(size_t)tk * HD] - ws[r];
        xt[n * XP + tk] = (__bf16)xacc[r];
      }
    }
    __syncthreads();

    if (wave < 2) {
      // O_inter = Q' S + Pq X for tokens [32 wave, 32 wave + 32)
      const __bf16* qr = qp + (row0 + min(32 * wave + n, valid - 1)) * HD + 8 * h2;
      f32x16 oi = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        oi = mfma32(ld8(qr + 16 * kc),
                    *reinterpret_cast<const bf16x8*>(st + n * SP + 16 * kc + 8 * h2), oi);
      const float* pr = pq_in + (cbase * TC + 32 * wave + n) * TC + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < TC / 16; ++kc)
        oi = mfma32(f32_to_bf16x8(pr + 16 * kc),
                    *reinterpret_cast<const bf16x8*>(xt + n * XP + 16 * kc + 8 * h2), oi);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = 32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (tk < valid) {
          const size_t e = (row0 + tk) * HD + col;
          const float inter = oi[r];
          o[e] = (__bf16)((float)o_intra[e] + inter);
          if (o_inter) o_inter[e] = (__bf16)inter;
        }
      }
    }
    // S += K'^T X: A = K'^T rows (state rows 32 wave + n) by transposing reads
#pragma unroll
    for (int kc = 0; kc < TC / 16; ++kc)
      sacc = mfma32(tr_op(lk, 16 * kc, 8, 32 * wave, lane),
                    *reinterpret_cast<const bf16x8*>(xt + n * XP + 16 * kc + 8 * h2), sacc);
    __syncthreads();
  }
  if (S_next) {
    const float a = alpha[bh];
    float* Sn = S_next + (size_t)bh * HD * HD;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const size_t e = (size_t)(32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HD + col;
      const float sp = Sp[e];
      Sn[e] = fmaf(a, sp, sacc[r] - sp);
    }
  }
}

// ---------------------------------------------------------------------------
// float32, any d <= 128: one workgroup per (b, h), thread j owns column j of
// the state (in LDS); the tokens are walked in order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(128)
tl_seq_k(const float* __restrict__ qp, const float* __restrict__ kp, const float* __restrict__ vp,
         const float* __restrict__ beta, const float* __restrict__ S_prev,
         const float* __restrict__ alpha, float* __restrict__ S_next,
         const float* __restrict__ o_intra, float* __restrict__ o, float* __restrict__ o_inter,
         int T, int D) {
  extern __shared__ float ls[];                      // [D][D]
  const int j = threadIdx.x;
  const long bh = blockIdx.x;
  const float* Sp = S_prev + (size_t)bh * D * D;
  if (j < D)
    for (int i = 0; i < D; ++i) ls[i * D + j] = Sp[(size_t)i * D + j];
  __syncthreads();
  if (j >= D) return;
  for (int t = 0; t < T; ++t) {
    const size_t row = ((size_t)bh * T + t) * D;
    float oj = 0.f, pred = 0.f;
    for (int i = 0; i < D; ++i) {
      const float s = ls[i * D + j];
      oj = fmaf(qp[row + i], s, oj);
      pred = fmaf(kp[row + i], s, pred);
    }
    o[row + j] = o_intra[row + j] + oj;
    if (o_inter) o_inter[row + j] = oj;
    const float u = beta[(size_t)bh * T + t] * (vp[row + j] - pred);
    for (int i = 0; i < D; ++i) ls[i * D + j] = fmaf(kp[row + i], u, ls[i * D + j]);
  }
  if (S_next) {
    const float a = alpha[bh];
    for (int i = 0; i < D; ++i) {
      const float sp = Sp[(size_t)i * D + j];
      S_next[(size_t)bh * D * D + (size_t)i * D + j] = fmaf(a, sp, ls[i * D + j] - sp);
    }
  }
}

int n_chunks(const Dims& d) { return (d.T + TC - 1) / TC; }

}  // namespace

size_t token_level_scan_ws_bytes(const Dims& d) {
  if (!(d.bf16 && d.D == HD)) return 0;
  const size_t nc = (size_t)d.B * d.H * n_chunks(d);
  return nc * TC * (2 * HD + TC) * sizeof(float);
}

hipError_t token_level_scan(const Dims& d, const void* q_prime, const void* k_prime,
                            const void* v_prime, const float* beta, const float* S_prev,
                            const float* alpha, float* S_next, const void* o_intra, void* o,
                            void* o_inter, void* ws, hipStream_t s) {
  const long n_bh = (long)d.B * d.H;
  if (d.bf16 && d.D == HD) {
    const int nc = n_chunks(d);
    float* w = static_cast<float*>(ws);
    float* u = w + (size_t)n_bh * nc * TC * HD;
    float* pq = u + (size_t)n_bh * nc * TC * HD;
    tl_chunk_k<<<(unsigned)(n_bh * nc), 256, 0, s>>>(
        static_cast<const __bf16*>(q_prime), static_cast<const __bf16*>(k_prime),
        static_cast<const __bf16*>(v_prime), beta, w, u, pq, d.T, nc);
    tl_scan_k<<<(unsigned)(n_bh * 4), 256, 0, s>>>(
        static_cast<const __bf16*>(q_prime), static_cast<const __bf16*>(k_prime), w, u, pq,
        S_prev, alpha, S_next, static_cast<const __bf16*>(o_intra), static_cast<__bf16*>(o),
        static_cast<__bf16*>(o_inter), d.T, nc);
    return hipGetLastError();
  }
  if (d.bf16) return hipErrorInvalidValue;            // bf16 runs at d = 128 only
  tl_seq_k<<<(unsigned)n_bh, 128, (size_t)d.D * d.D * sizeof(float), s>>>(
      static_cast<const float*>(q_prime), static_cast<const float*>(k_prime),
      static_cast<const float*>(v_prime), beta, S_prev, alpha, S_next,
      static_cast<const float*>(o_intra), static_cast<float*>(o), static_cast<float*>(o_inter),
      d.T, d.D);
  return hipGetLastError();
}

}  // namespace arl2
