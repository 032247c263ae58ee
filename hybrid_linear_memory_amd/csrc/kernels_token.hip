// Token-level access: the alternative to frame-level access that the
// "Attend Locally, Remember Linearly" technical summary ablates (§4: token-level
// access degrades quality). Within a pass, token t reads the state left by the
// frame's earlier tokens, starting from S_{N-1}:
//   o_inter_t = q'_t S_{t-1},   S_t = S_{t-1} + beta_t k'_t^T (v'_t - k'_t S_{t-1}),
// and the clean pass commits S_N = alpha S_{N-1} + (S_T - S_{N-1}).
//
// bf16, d = 128: the recurrence runs in chunks of TC tokens in closed form.
// Over a chunk, A X = diag(beta) (V' - K' S) with A = I + tril(diag(beta) K'K'^T, -1)
// gives every token's update x_t at once; with T = A^-1 (unit lower triangular),
// W = T diag(beta) K' and U = T diag(beta) V' do not depend on the state, so
// every chunk forms them in parallel (tl_chunk_k); a sequential pass over the
// chunks (tl_scan_k) then carries the state:
//   X = U - W S,  O_inter = Q' S + tril(Q' K'^T, -1) X,  S <- S + K'^T X.
// float32 (any supported d): one workgroup per (b, h) walks the tokens
// (tl_seq_k).
#include <math.h>

#include "arl2_internal.h"
#include "mfma_common.h"

namespace arl2 {
namespace {

constexpr int TC = 64;                      // tokens per chunk
constexpr int AP = TC + 4;                  // fp32 row of A / T in LDS (16-byte rows)
constexpr int LP = TC + 8;                  // bf16 row of T diag(beta) in LDS (144 bytes)
constexpr int XP = TC + 8;                  // bf16 row of X^T in LDS
constexpr int SP = HD + 8;                  // bf16 row of S^T in LDS

// bf16 chunk of `rows` x 128 (256-byte rows) into LDS under the swz_v chunk
// swizzle (chunk p of row r at p ^ swz_v(r)); rows past `valid` are zero.
__device__ __forceinline__ void stage_rows(char* dst, const __bf16* src, int rows, int valid) {
  for (int idx = threadIdx.x; idx < rows * 16; idx += blockDim.x) {
    const int r = idx >> 4, p = idx & 15;
    uint4 val = {0u, 0u, 0u, 0u};
    if (r < valid) val = *reinterpret_cast<const uint4*>(src + (size_t)r * HD + 8 * p);
    *reinterpret_cast<uint4*>(dst + r * 256 + ((p ^ swz_v(r)) << 4)) = val;
  }
}

// Row operand (8 consecutive columns 16 kc + 8 h2 ..) from a swz_v-staged chunk.
__device__ __forceinline__ bf16x8 row_op(const char* base, int row, int kc, int h2) {
  return *reinterpret_cast<const bf16x8*>(base + row * 256 + (((2 * kc + h2) ^ swz_v(row)) << 4));
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float4 fma4(float a, float4 b, float4 c) {
  return make_float4(fmaf(a, b.x, c.x), fmaf(a, b.y, c.y), fmaf(a, b.z, c.z), fmaf(a, b.w, c.w));
}

// ---------------------------------------------------------------------------
// Chunk preparation. One workgroup (4 waves) per (b, h, chunk):
//   Pq = tril(Q'K'^T, -1) (bf16, out) and A = tril(diag(beta) K'K'^T, -1) (fp32,
//   LDS) on MFMA; T = (I + A)^-1 in fp32 by blocks: the four 16 x 16 diagonal
//   blocks by forward substitution, then two doublings, each forming the
//   off-diagonal block of a 2 x 2 blocking as  T_10 = -T_11 A_10 T_00;
//   W = T diag(beta) K' (bf16, out) and U = T diag(beta) V' (fp32, out) on MFMA,
//   the A operand T diag(beta) formed from T in registers and split into a
//   bf16 high and low part, so that both products carry fp32-level accuracy.
// Q' rows and the V' chunk are loaded into registers at the start; V' goes to
// LDS (over the doubling scratch) once T is done. About 50 KB of LDS.
// Workspace per (bh, chunk): W bf16 [TC][128] row-major; U fp32 as eight 32 x 32
// tiles (token tile ti, feature tile tf) each in MFMA accumulator order (lane
// l's 16 values, rows 8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32,
// contiguous), the order in which the scan consumes them; Pq bf16 [TC][TC].
// Tokens past the frame's end have beta = 0 and zero K', so their rows of W and
// U are zero and they leave the state alone.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
tl_chunk_k(const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
           const __bf16* __restrict__ vp, const float* __restrict__ beta,
           __bf16* __restrict__ w_out, float* __restrict__ u_out, __bf16* __restrict__ pq_out,
           int T, int n_ch) {
  __shared__ __attribute__((aligned(16))) char lk[TC * 256];
  __shared__ __attribute__((aligned(16))) char lv[TC * 256];   // doubling scratch, then V'
  __shared__ __attribute__((aligned(16))) float la[TC * AP];
  __shared__ float lb[TC];
  float* ly = reinterpret_cast<float*>(lv);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const long bh = blockIdx.x / n_ch;
  const int ch = blockIdx.x % n_ch;
  const int t0 = ch * TC;
  const int valid = min(TC, T - t0);
  const size_t row0 = (size_t)bh * T + t0;
  const size_t cbase = (size_t)bh * n_ch + ch;
  const int ti = wave == 0 ? 0 : 1, tj = wave == 2 ? 1 : 0;   // G / Pq tile of waves 0-2
  bf16x8 qa[8];
  if (wave < 3) {
    const __bf16* qr = qp + (row0 + min(32 * ti + n, valid - 1)) * HD + 8 * h2;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qa[kc] = ld8(qr + 16 * kc);
  }
  uint4 vr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 256 * e, r = idx >> 4, p = idx & 15;
    vr[e] = r < valid ? *reinterpret_cast<const uint4*>(vp + (row0 + r) * HD + 8 * p)
                      : make_uint4(0u, 0u, 0u, 0u);
  }
  stage_rows(lk, kp + row0 * HD, TC, valid);
  if (tid < TC) lb[tid] = tid < valid ? beta[row0 + tid] : 0.f;
  __syncthreads();

  // G = K'K'^T and Q'K'^T on the lower 32 x 32 tiles (0,0), (1,0), (1,1);
  // the upper tile of Pq is zero
  __bf16* pq_c = pq_out + cbase * TC * TC;
  if (wave < 3) {
    f32x16 g = zero16(), pq = zero16();
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8 b = row_op(lk, 32 * tj + n, kc, h2);
      g = mfma32(row_op(lk, 32 * ti + n, kc, h2), b, g);
      pq = mfma32(qa[kc], b, pq);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * ti + 8 * (r >> 2) + 4 * h2 + (r & 3), j = 32 * tj + n;
      la[i * AP + j] = i > j ? lb[i] * g[r] : 0.f;
      pq_c[i * TC + j] = (__bf16)(i > j ? pq[r] : 0.f);
    }
  } else {
    for (int e = lane; e < 32 * 32; e += 64) pq_c[(e >> 5) * TC + 32 + (e & 31)] = (__bf16)0.f;
  }
  __syncthreads();

  // T on the 16 x 16 diagonal blocks: lane (b, c) solves column c of block b
  if (wave == 0) {
    const int b = lane >> 4, c = lane & 15;
    float* ab = la + 16 * b * AP + 16 * b;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc = fmaf(ab[r * AP + j], t[j], acc);
      t[r] = r == c ? 1.f : -acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) ab[r * AP + c] = t[r];
  }
  __syncthreads();

  // 32 x 32 diagonal blocks: T_10 = -T_11 (A_10 T_00) with 16 x 16 blocks, for
  // the block pairs at rows / columns 0 and 32
  const int p2 = tid >> 6, r2 = (tid >> 2) & 15, c2 = 4 * (tid & 3);
  if (tid < 128) {
    const int o0 = 32 * p2;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      y = fma4(la[(o0 + 16 + r2) * AP + o0 + k], ld4(la + (o0 + k) * AP + o0 + c2), y);
    st4(ly + p2 * 256 + r2 * 16 + c2, y);
  }
  __syncthreads();
  if (tid < 128) {
    const int o0 = 32 * p2;
    float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      z = fma4(la[(o0 + 16 + r2) * AP + o0 + 16 + k], ld4(ly + p2 * 256 + k * 16 + c2), z);
    st4(la + (o0 + 16 + r2) * AP + o0 + c2, make_float4(-z.x, -z.y, -z.z, -z.w));
  }
  __syncthreads();

  // the whole 64 x 64: T_10 = -T_11 (A_10 T_00) with 32 x 32 blocks
  const int r3 = tid >> 3, c3 = 4 * (tid & 7);
  {
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 32; ++k) y = fma4(la[(32 + r3) * AP + k], ld4(la + k * AP + c3), y);
    st4(ly + r3 * 32 + c3, y);
  }
  __syncthreads();
  {
    float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < 32; ++k) z = fma4(la[(32 + r3) * AP + 32 + k], ld4(ly + k * 32 + c3), z);
    st4(la + (32 + r3) * AP + c3, make_float4(-z.x, -z.y, -z.z, -z.w));
  }
  __syncthreads();
  // V' over the scratch (its last reads were before the barrier above)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = tid + 256 * e, r = idx >> 4, p = idx & 15;
    *reinterpret_cast<uint4*>(lv + r * 256 + ((p ^ swz_v(r)) << 4)) = vr[e];
  }
  __syncthreads();

  // W (waves 0-1) and U (waves 2-3): wave covers feature tiles 2 (wave & 1) + {0, 1}
  const bool is_u = wave >= 2;
  const char* src = is_u ? lv : lk;
  __bf16* w_c = w_out + cbase * TC * HD;
  float* u_c = u_out + cbase * TC * HD;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
    f32x16 acc[2] = {zero16(), zero16()};
    const int t = 32 * tr + n;                    // this lane's row of T diag(beta)
#pragma unroll
    for (int kc = 0; kc < 2 + 2 * tr; ++kc) {
      // A operand: (T diag(beta))[t][16 kc + 8 h2 + u], zero above the diagonal
      const int j0 = 16 * kc + 8 * h2;
      const float4 x0 = ld4(la + t * AP + j0), x1 = ld4(la + t * AP + j0 + 4);
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 hi, lo;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float val = j0 + u <= t ? xv[u] * lb[j0 + u] : 0.f;
        hi[u] = (__bf16)val;
        lo[u] = (__bf16)(val - (float)hi[u]);
      }
#pragma unroll
      for (int tfi = 0; tfi < 2; ++tfi) {
        const bf16x8 b = tr_op(src, 16 * kc, 8, 32 * (2 * (wave & 1) + tfi), lane);
        acc[tfi] = mfma32(hi, b, acc[tfi]);
        acc[tfi] = mfma32(lo, b, acc[tfi]);
      }
    }
#pragma unroll
    for (int tfi = 0; tfi < 2; ++tfi) {
      const int tf = 2 * (wave & 1) + tfi;
      if (is_u) {
        // U tile (tr, tf) in accumulator order: lane-contiguous 16 floats
        float* ut = u_c + ((tr * 4 + tf) * 64 + lane) * 16;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          st4(ut + 4 * q4, make_float4(acc[tfi][4 * q4], acc[tfi][4 * q4 + 1],
                                       acc[tfi][4 * q4 + 2], acc[tfi][4 * q4 + 3]));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          w_c[(32 * tr + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HD + 32 * tf + n] =
              (__bf16)acc[tfi][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sequential pass over the chunks. One workgroup (4 waves) per (b, h, 32-column
// block cb of the state); the four blocks of a head share an XCD (and its L2).
// Wave w holds state rows [32w, 32w + 32) of the block as an MFMA accumulator.
// Per chunk, after the state S^T (bf16) is in LDS:
//   A: waves 0-1 form X = U - W S for tokens [32w, 32w + 32) (X^T to LDS),
//      waves 2-3 form Q' S for tokens [32(w-2), ..);
//   B: waves 2-3 add tril(Q'K'^T, -1) X and write o = o_intra + O_inter,
//      all waves add K'^T X to their state rows (K' staged for transposing
//      reads).
// The next chunk's operands (K' staging, W and U, or Q', Pq and o_intra) are
// loaded into registers while the current chunk computes, each as soon as its
// register is free. With S_next given,
// the end state commits S_next = alpha S_prev + (S_T - S_prev).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
tl_scan_k(const __bf16* __restrict__ qp, const __bf16* __restrict__ kp,
          const __bf16* __restrict__ w_in, const float* __restrict__ u_in,
          const __bf16* __restrict__ pq_in, const float* __restrict__ S_prev,
          const float* __restrict__ alpha, float* __restrict__ S_next,
          const __bf16* __restrict__ o_intra, __bf16* __restrict__ o,
          __bf16* __restrict__ o_inter, int T, int n_ch) {
  __shared__ __attribute__((aligned(16))) char lk0[TC * 256];
  __shared__ __attribute__((aligned(16))) char lk1[TC * 256];
  __shared__ __attribute__((aligned(16))) __bf16 st[32 * SP];
  __shared__ __attribute__((aligned(16))) __bf16 xt[32 * XP];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const long bh = logical >> 2;
  const int cb = logical & 3;
  const int col = 32 * cb + n;                       // this lane's state column
  const bool xw = wave < 2;                          // X waves (else O waves)
  const int rw = 32 * (wave & 1);                    // the wave's token rows in a chunk
  const float* Sp = S_prev + (size_t)bh * HD * HD;
  // state rows 32 w + 8 (r / 4) + 4 h2 + r % 4 of column `col`
  f32x16 sacc;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    sacc[r] = Sp[(size_t)(32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HD + col];

  // Each role runs its own straight-line loop (two barriers per chunk in both),
  // so that every wait for a prefetched operand counts exactly the loads
  // issued after it. Operands: am = W rows (X waves) or Q' rows (O waves);
  // um = U (X waves) or o_intra (O waves) at the accumulator's positions;
  // pm = Pq rows (O waves); kn = this thread's share of the next K' chunk (the
  // last chunk reloads itself). Global rows past the frame's end lie outside
  // the buffers' ranges: they read as zero and are not written.
  const uint32_t head_bytes = (uint32_t)T * HD * 2;
  const size_t head_off = (size_t)bh * T * HD;
  const __amdgpu_buffer_rsrc_t r_k = buffer_rsrc(kp + head_off, head_bytes);
  bf16x8 am[8];
  float um[16];
  uint4 kn[4];
  auto load_k = [&](int c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e, r = idx >> 4, p = idx & 15;
      kn[e] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(r_k, ((c * TC + r) * HD + 8 * p) * 2, 0, 0));
    }
  };
  auto store_k = [&](char* dst) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e, r = idx >> 4, p = idx & 15;
      *reinterpret_cast<uint4*>(dst + r * 256 + ((p ^ swz_v(r)) << 4)) = kn[e];
    }
  };
  auto state_to_lds = [&]() {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      st[n * SP + 32 * wave + 8 * (r >> 2) + 4 * h2 + (r & 3)] = (__bf16)sacc[r];
  };
  auto x_op = [&](int kc) {
    return *reinterpret_cast<const bf16x8*>(xt + n * XP + 16 * kc + 8 * h2);
  };
  auto update_state = [&](const char* lkc) {   // S += K'^T X
#pragma unroll
    for (int kc = 0; kc < TC / 16; ++kc)
      sacc = mfma32(tr_op(lkc, 16 * kc, 8, 32 * wave, lane), x_op(kc), sacc);
  };

  load_k(0);
  store_k(lk0);
  // Two sets of the operands that phase A needs, alternating between chunks
  // (the loop body covers a pair of chunks): each step first issues the next
  // chunk's loads into the other set, so they have a whole chunk of work to
  // arrive; phase B operands (Pq, o_intra) come at the start of their own step.
  if (xw) {
    bf16x8 am2[8];
    float um2[16];
    auto load_wu = [&](int c, bf16x8 (&a)[8], float (&u)[16]) {
      const size_t cbase = (size_t)bh * n_ch + c;
      const __bf16* wr = w_in + (cbase * TC + rw + n) * HD + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) a[kc] = ld8(wr + 16 * kc);
      const float* ut = u_in + cbase * TC * HD + (((wave & 1) * 4 + cb) * 64 + lane) * 16;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = ld4(ut + 4 * q4);
        u[4 * q4] = x.x;
        u[4 * q4 + 1] = x.y;
        u[4 * q4 + 2] = x.z;
        u[4 * q4 + 3] = x.w;
      }
    };
    auto step = [&](int c, bf16x8 (&a)[8], float (&u)[16], bf16x8 (&a_nx)[8],
                    float (&u_nx)[16]) {
      const int cn = min(c + 1, n_ch - 1);
      state_to_lds();
      load_k(cn);
      load_wu(cn, a_nx, u_nx);
      __syncthreads();
      f32x16 acc = zero16();                       // W S
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        acc = mfma32(a[kc], *reinterpret_cast<const bf16x8*>(st + n * SP + 16 * kc + 8 * h2), acc);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xt[n * XP + rw + 8 * (r >> 2) + 4 * h2 + (r & 3)] = (__bf16)(u[r] - acc[r]);
      __syncthreads();
      update_state((c & 1) ? lk1 : lk0);
      store_k((c & 1) ? lk0 : lk1);
    };
    load_wu(0, am, um);
    int c = 0;
    for (; c + 1 < n_ch; c += 2) {
      step(c, am, um, am2, um2);
      step(c + 1, am2, um2, am, um);
    }
    if (c < n_ch) step(c, am, um, am2, um2);
  } else {
    const __amdgpu_buffer_rsrc_t r_oi = buffer_rsrc(o_intra + head_off, head_bytes);
    const __amdgpu_buffer_rsrc_t r_o = buffer_rsrc(o + head_off, head_bytes);
    // without o_inter, a buffer of no bytes: its stores are dropped
    const __amdgpu_buffer_rsrc_t r_oe =
        o_inter ? buffer_rsrc(o_inter + head_off, head_bytes) : buffer_rsrc(o, 0);
    auto row_off = [](int r) { return (8 * (r >> 2) + (r & 3)) * HD * 2; };
    bf16x8 am2[8], pm[4];
    uint32_t oi[16];                               // o_intra, raw bf16 bits
    auto load_q = [&](int c, bf16x8 (&a)[8]) {
      const int valid = min(TC, T - c * TC);
      const __bf16* qr = qp + ((size_t)bh * T + c * TC + min(rw + n, valid - 1)) * HD + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) a[kc] = ld8(qr + 16 * kc);
    };
    // phase B operands of chunk c, loaded at the start of its own step
    auto load_pb = [&](int c) {
      const __bf16* pr = pq_in + (((size_t)bh * n_ch + c) * TC + rw + n) * TC + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) pm[kc] = ld8(pr + 16 * kc);
      const int vo = ((c * TC + rw + 4 * h2) * HD + col) * 2;
#pragma unroll
      for (int r = 0; r < 16; ++r) oi[r] = __builtin_amdgcn_raw_buffer_load_b16(r_oi, vo, row_off(r), 0);
    };
    auto step = [&](int c, bf16x8 (&a)[8], bf16x8 (&a_nx)[8]) {
      const int cn = min(c + 1, n_ch - 1);
      state_to_lds();
      load_k(cn);
      load_q(cn, a_nx);
      load_pb(c);
      __syncthreads();
      f32x16 acc = zero16();                       // Q' S
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        acc = mfma32(a[kc], *reinterpret_cast<const bf16x8*>(st + n * SP + 16 * kc + 8 * h2), acc);
      __syncthreads();
#pragma unroll
      for (int kc = 0; kc < TC / 16; ++kc) acc = mfma32(pm[kc], x_op(kc), acc);   // + Pq X
      const int vo = ((c * TC + rw + 4 * h2) * HD + col) * 2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float o_in = __builtin_bit_cast(float, oi[r] << 16);
        __builtin_amdgcn_raw_buffer_store_b16(
            __builtin_bit_cast(unsigned short, (__bf16)(o_in + acc[r])), r_o, vo, row_off(r), 0);
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)acc[r]),
                                              r_oe, vo, row_off(r), 0);
      }
      update_state((c & 1) ? lk1 : lk0);
      store_k((c & 1) ? lk0 : lk1);
    };
    load_q(0, am);
    int c = 0;
    for (; c + 1 < n_ch; c += 2) {
      step(c, am, am2);
      step(c + 1, am2, am);
    }
    if (c < n_ch) step(c, am, am2);
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
  return nc * TC * (HD * (sizeof(__bf16) + sizeof(float)) + TC * sizeof(__bf16));
}

hipError_t token_level_scan(const Dims& d, const void* q_prime, const void* k_prime,
                            const void* v_prime, const float* beta, const float* S_prev,
                            const float* alpha, float* S_next, const void* o_intra, void* o,
                            void* o_inter, void* ws, hipStream_t s) {
  const long n_bh = (long)d.B * d.H;
  if (d.bf16 && d.D == HD) {
    const int nc = n_chunks(d);
    __bf16* w = static_cast<__bf16*>(ws);
    float* u = reinterpret_cast<float*>(w + (size_t)n_bh * nc * TC * HD);
    __bf16* pq = reinterpret_cast<__bf16*>(u + (size_t)n_bh * nc * TC * HD);
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
