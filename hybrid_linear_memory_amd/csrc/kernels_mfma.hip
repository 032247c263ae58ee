// bf16 MFMA kernels of the ARL2 hybrid attention step at head dimension 128,
// for gfx950 (CDNA4): v_mfma_f32_32x32x16_bf16 tiles, fp32 accumulation,
// LDS-staged K / V / state tiles.
//
// Step definitions: "Attend Locally, Remember Linearly" technical summary,
// §2.1 (feature maps Q' = Q Phi_q, K' = rownorm(K Phi_k), V' = V Phi_v;
// intra-frame bidirectional softmax; read O_inter = Q' S_{N-1}; update
// S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1})) and §2.2
// (frame-level access: one S_{N-1} for the whole frame).
//
// MFMA operand layout used throughout (32x32x16, wave64): for C = A * B with
// A [32 x 16] and B [16 x 32], lane l supplies row (l % 32) of A and column
// (l % 32) of B, each as 8 consecutive k-slots starting at 8 * (l / 32); the
// result C [32 x 32] lands as lane l = column (l % 32), register r = row
// 8 * (r / 4) + 4 * (l / 32) + (r % 4). Every contraction below is arranged
// so that the contracted index is contiguous in memory for both operands, and
// so that an accumulator's register index runs over the index the next
// contraction sums over (softmax P and the commit's residual never leave
// registers).
#include <math.h>

#include "arl2_internal.h"

namespace arl2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 128;                 // head dimension
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int u = 0; u < 8; ++u) z[u] = (__bf16)0.f;
  return z;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int u = 0; u < 16; ++u) z[u] = 0.f;
  return z;
}

// Value of x held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// Row of a 32-row A-operand tile that lane slot m loads so that accumulator
// register r of lanes with half h2 holds row 16 * h2 + r of the tile.
__device__ __forceinline__ int perm32(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Map a linear block id so that consecutive logical blocks share an XCD
// (blocks are dealt round-robin over the 8 XCDs of the chip).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  constexpr int X = 8;
  const int per = nblk / X, rem = nblk % X;
  const int xcd = bid % X, idx = bid / X;
  // XCDs below `rem` own per + 1 logical blocks.
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}

// ===========================================================================
// Intra-frame softmax attention (and the full-KV comparator).
//
// One workgroup = 4 waves = 128 query rows of one (b, h); each wave owns 32
// queries. Keys stream through LDS in tiles of 64 (K row-major, V transposed),
// double-buffered. Scores are computed transposed, S^T = K Q^T, so that each
// lane holds one query's scores: the row max and sum need one cross-half
// exchange, and P^T feeds O^T = V^T P^T directly from registers.
// ===========================================================================
constexpr int AQ = 128;               // queries per workgroup
constexpr int AKT = 64;               // keys per tile
constexpr int AKS = HD + 8;           // K row stride in LDS (bf16)
constexpr int AVS = AKT + 8;          // V^T row stride in LDS (bf16)
constexpr int AKBUF = AKT * AKS;
constexpr int AVBUF = HD * AVS;
constexpr int ASTAGE = AKBUF + AVBUF;

struct KVRegs {
  uint4 k[4];
  uint4 v[4];
};

__device__ __forceinline__ void attn_load_tile(KVRegs& r, const __bf16* kh, const __bf16* vh,
                                               int k0, int n_kv, int tid) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;
    const int row = c >> 4, col = (c & 15) * 8;
    const int key = k0 + row;
    r.k[it] = key < n_kv ? *reinterpret_cast<const uint4*>(kh + (size_t)key * HD + col)
                         : make_uint4(0, 0, 0, 0);
  }
  const int kg = tid & 15, dg = tid >> 4;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int key = k0 + 4 * kg + rr;
    r.v[rr] = key < n_kv ? *reinterpret_cast<const uint4*>(vh + (size_t)key * HD + 8 * dg)
                         : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

// Element e (0..7) of 8 packed bf16 held as uint4.
__device__ __forceinline__ uint32_t elem(const uint4& x, int e) {
  const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  return (e & 1) ? hi16(w) : lo16(w);
}

__device__ __forceinline__ void attn_store_tile(const KVRegs& r, __bf16* stage, int tid) {
  __bf16* Ks = stage;
  __bf16* Vt = stage + AKBUF;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int c = tid + 256 * it;
    const int row = c >> 4, col = (c & 15) * 8;
    *reinterpret_cast<uint4*>(Ks + row * AKS + col) = r.k[it];
  }
  const int kg = tid & 15, dg = tid >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint2 w;
    w.x = elem(r.v[0], e) | (elem(r.v[1], e) << 16);
    w.y = elem(r.v[2], e) | (elem(r.v[3], e) << 16);
    *reinterpret_cast<uint2*>(Vt + (8 * dg + e) * AVS + 4 * kg) = w;
  }
}

__global__ void __launch_bounds__(256)
attn_mfma_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
            const __bf16* __restrict__ v, __bf16* __restrict__ o, int T, int n_kv,
            long kv_cap, float sl2, int n_qblk) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[2 * ASTAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const long bh = blk / n_qblk;
  const int qblk = blk % n_qblk;
  const int t = qblk * AQ + wave * 32 + n;
  const __bf16* kh = k + (size_t)bh * kv_cap * HD;
  const __bf16* vh = v + (size_t)bh * kv_cap * HD;

  // Q^T as the B operand of S^T = K Q^T: column n = query t, k = head dim.
  bf16x8 qreg[8];
  {
    const __bf16* qrow = q + ((size_t)bh * T + t) * HD + 8 * h2;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) qreg[kc] = t < T ? ld8(qrow + 16 * kc) : zero8();
  }

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (n_kv + AKT - 1) / AKT;
  KVRegs regs;
  attn_load_tile(regs, kh, vh, 0, n_kv, tid);
  attn_store_tile(regs, lds, tid);
  __syncthreads();

  const int krow = perm32(n);
  for (int kt = 0; kt < n_tiles; ++kt) {
    const int k0 = kt * AKT;
    if (kt + 1 < n_tiles) attn_load_tile(regs, kh, vh, k0 + AKT, n_kv, tid);
    const __bf16* Ks = lds + (kt & 1) * ASTAGE;
    const __bf16* Vt = Ks + AKBUF;

    // S^T tile: keys x queries, two 32-key halves.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
      const __bf16* kp = Ks + (kb * 32 + krow) * AKS + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) s[kb] = mfma32(ld8(kp + 16 * kc), qreg[kc], s[kb]);
    }
    if (k0 + AKT > n_kv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (k0 + kb * 32 + 16 * h2 + r >= n_kv) s[kb][r] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m_run, mt);
    const float corr = exp2f((m_run - m_new) * sl2);
    const float mc = m_new * sl2;
    m_run = m_new;

    bf16x8 pb[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(s[kb][r], sl2, -mc));
        lsum += p;
        pb[kb][r >> 3][r & 7] = (__bf16)p;
      }
    l_run = fmaf(l_run, corr, lsum);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= corr;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const __bf16* vp = Vt + (32 * db + n) * AVS + 16 * h2;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
          acc[db] = mfma32(ld8(vp + kb * 32 + 8 * cc), pb[kb][cc], acc[db]);
    }

    if (kt + 1 < n_tiles) attn_store_tile(regs, lds + ((kt + 1) & 1) * ASTAGE, tid);
    __syncthreads();
  }

  const float l_tot = l_run + swap_halves(l_run);
  const float inv = 1.f / l_tot;
  if (t < T) {
    __bf16* orow = o + ((size_t)bh * T + t) * HD + 4 * h2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)(acc[db][4 * jj + i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * jj) = w;
      }
  }
}

// ===========================================================================
// Row maps Y = X M per head: the feature maps (M = Phi[h], bf16, optional
// row normalisation) and the inter-frame read (M = S[b,h], fp32 staged as
// bf16, epilogue O = O_intra + Y).
//
// One workgroup = 4 waves; M^T is staged once in LDS; each wave computes
// Y^T = M^T X^T for 32 rows at a time (lane = one row, registers = 64 of its
// 128 outputs), so the row norm is an in-lane sum plus one exchange.
// ===========================================================================
constexpr int MS = HD + 8;            // M^T row stride in LDS (bf16)
constexpr int MAP_ROWS = 128;         // rows per workgroup

enum MapMode { MAP_PHI = 0, MAP_STATE = 1 };

template <int MODE>
__global__ void __launch_bounds__(256)
rowmap_mfma_k(const __bf16* __restrict__ x, const void* __restrict__ mat,
              const __bf16* o_intra, __bf16* out, __bf16* __restrict__ o_inter, int H,
              int T, int n_rblk, int normalize) {
  __shared__ __attribute__((aligned(16))) __bf16 MT[HD * MS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const long bh = blk / n_rblk;
  const int rblk = blk % n_rblk;

  // Stage M^T: MT[j][i] = M[i][j], written as bf16 pairs (i, i+1).
  if (MODE == MAP_PHI) {
    const __bf16* M = static_cast<const __bf16*>(mat) + (size_t)(bh % H) * HD * HD;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int u = tid + 256 * it;          // 64 row pairs x 16 column chunks
      const int ip = u >> 4, jc = (u & 15) * 8;
      const uint4 r0 = *reinterpret_cast<const uint4*>(M + (size_t)(2 * ip) * HD + jc);
      const uint4 r1 = *reinterpret_cast<const uint4*>(M + (size_t)(2 * ip + 1) * HD + jc);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t*>(MT + (jc + e) * MS + 2 * ip) = elem(r0, e) | (elem(r1, e) << 16);
    }
  } else {
    const float* M = static_cast<const float*>(mat) + (size_t)bh * HD * HD;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int u = tid + 256 * it;          // 64 row pairs x 32 column quads
      const int ip = u >> 5, jc = (u & 31) * 4;
      const float4 r0 = *reinterpret_cast<const float4*>(M + (size_t)(2 * ip) * HD + jc);
      const float4 r1 = *reinterpret_cast<const float4*>(M + (size_t)(2 * ip + 1) * HD + jc);
      const float a0[4] = {r0.x, r0.y, r0.z, r0.w};
      const float a1[4] = {r1.x, r1.y, r1.z, r1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 pair[2] = {(__bf16)a0[e], (__bf16)a1[e]};
        *reinterpret_cast<uint32_t*>(MT + (jc + e) * MS + 2 * ip) =
            *reinterpret_cast<const uint32_t*>(pair);
      }
    }
  }
  __syncthreads();

  const int t = rblk * MAP_ROWS + wave * 32 + n;
  if (rblk * MAP_ROWS + wave * 32 >= T) return;   // whole wave past the end
  const size_t row = (size_t)bh * T + t;
  bf16x8 xr[8];
  {
    const __bf16* xp = x + row * HD + 8 * h2;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) xr[kc] = t < T ? ld8(xp + 16 * kc) : zero8();
  }
  f32x16 acc[4];
#pragma unroll
  for (int ob = 0; ob < 4; ++ob) {
    acc[ob] = zero16();
    const __bf16* mp = MT + (32 * ob + n) * MS + 8 * h2;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) acc[ob] = mfma32(ld8(mp + 16 * kc), xr[kc], acc[ob]);
  }
  if (MODE == MAP_PHI && normalize) {
    float ss = 0.f;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss = fmaf(acc[ob][r], acc[ob][r], ss);
    ss += swap_halves(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int ob = 0; ob < 4; ++ob)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ob][r] *= inv;
  }
  if (t >= T) return;
#pragma unroll
  for (int ob = 0; ob < 4; ++ob)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const size_t off = row * HD + 32 * ob + 8 * jj + 4 * h2;
      bf16x4 w;
      if (MODE == MAP_STATE) {
        if (o_inter) {
#pragma unroll
          for (int i = 0; i < 4; ++i) w[i] = (__bf16)acc[ob][4 * jj + i];
          *reinterpret_cast<bf16x4*>(o_inter + off) = w;
        }
        bf16x4 base;
        if (o_intra) {
          base = *reinterpret_cast<const bf16x4*>(o_intra + off);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) base[i] = (__bf16)0.f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)((float)base[i] + acc[ob][4 * jj + i]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = (__bf16)acc[ob][4 * jj + i];
      }
      *reinterpret_cast<bf16x4*>(out + off) = w;
    }
}

// ===========================================================================
// State commit.
//
// One workgroup = 4 waves per (b, h, token chunk); wave w owns state columns
// [32w, 32w + 32). Per 32-token slice:
//   P^ = K' S_prev[:, cols]          (A = K' rows from LDS, B = S column block
//                                     held in registers as bf16)
//   W  = beta * (V' - P^)            (registers, fp32, then bf16)
//   U[:, cols] += K'^T W             (A = K'^T from LDS, B = W from registers)
// With one chunk the workgroup writes S_next = alpha S_prev + U; otherwise it
// writes U to a partial slot and a second kernel adds the partials in chunk
// order (fixed order, no atomics).
// ===========================================================================
constexpr int CT = 32;                // tokens per slice
constexpr int CKS = HD + 8;           // K' row stride (bf16)
constexpr int CTS = CT + 8;           // K'^T / V'^T row stride (bf16)
constexpr int C_KN = CT * CKS;
constexpr int C_KT = HD * CTS;
constexpr int C_STAGE = C_KN + 2 * C_KT;

__global__ void __launch_bounds__(256)
commit_mfma_k(const __bf16* __restrict__ kp, const __bf16* __restrict__ vp,
              const float* __restrict__ beta, const float* __restrict__ alpha,
              const float* __restrict__ S_prev, float* __restrict__ S_next,
              float* __restrict__ partial, int T, int chunk_tokens, int n_chunks,
              long n_bh) {
  __shared__ __attribute__((aligned(16))) __bf16 lds[C_STAGE];
  __shared__ float bsh[CT];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const long bh = blk / n_chunks;
  const int chunk = blk % n_chunks;
  const int t_begin = chunk * chunk_tokens;
  const int t_end = min(T, t_begin + chunk_tokens);
  const int col = 32 * wave + n;

  const float* Sp = S_prev + (size_t)bh * HD * HD;
  // S[:, col] as the B operand (k = state row).
  bf16x8 sreg[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
#pragma unroll
    for (int u = 0; u < 8; ++u) sreg[kc][u] = (__bf16)Sp[(size_t)(16 * kc + 8 * h2 + u) * HD + col];

  f32x16 uacc[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) uacc[ib] = zero16();

  __bf16* Kn = lds;
  __bf16* Kt = lds + C_KN;
  __bf16* Vt = Kt + C_KT;
  const __bf16* kh = kp + (size_t)bh * T * HD;
  const __bf16* vh = vp + (size_t)bh * T * HD;
  const float* bt = beta + (size_t)bh * T;
  const int krow = perm32(n);

  for (int t0 = t_begin; t0 < t_end; t0 += CT) {
    __syncthreads();
    {
      // threads 0..127 stage K' (natural + transposed), 128..255 stage V'^T:
      // unit = 4 tokens x 8 dims.
      const int u = tid & 127;
      const int tg = u & 7, dg = u >> 3;
      const __bf16* src = tid < 128 ? kh : vh;
      uint4 r[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int tok = t0 + 4 * tg + rr;
        r[rr] = tok < t_end ? *reinterpret_cast<const uint4*>(src + (size_t)tok * HD + 8 * dg)
                            : make_uint4(0, 0, 0, 0);
      }
      __bf16* dstT = tid < 128 ? Kt : Vt;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w;
        w.x = elem(r[0], e) | (elem(r[1], e) << 16);
        w.y = elem(r[2], e) | (elem(r[3], e) << 16);
        *reinterpret_cast<uint2*>(dstT + (8 * dg + e) * CTS + 4 * tg) = w;
      }
      if (tid < 128) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<uint4*>(Kn + (4 * tg + rr) * CKS + 8 * dg) = r[rr];
      }
      if (tid < CT) bsh[tid] = t0 + tid < t_end ? bt[t0 + tid] : 0.f;
    }
    __syncthreads();

    // P^ for 32 tokens x this wave's 32 columns; register r <-> token 16*h2 + r.
    f32x16 p = zero16();
    {
      const __bf16* kr = Kn + krow * CKS + 8 * h2;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) p = mfma32(ld8(kr + 16 * kc), sreg[kc], p);
    }
    bf16x8 wb[2];
    {
      const bf16x8 v0 = ld8(Vt + col * CTS + 16 * h2);
      const bf16x8 v1 = ld8(Vt + col * CTS + 16 * h2 + 8);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float vv = r < 8 ? (float)v0[r] : (float)v1[r - 8];
        const float w = bsh[16 * h2 + r] * (vv - p[r]);
        wb[r >> 3][r & 7] = (__bf16)w;
      }
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const __bf16* ka = Kt + (32 * ib + n) * CTS + 16 * h2;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) uacc[ib] = mfma32(ld8(ka + 8 * cc), wb[cc], uacc[ib]);
    }
  }

  // uacc[ib][r] = U[row 32*ib + 8*(r/4) + 4*h2 + (r%4)][col]
  if (n_chunks == 1) {
    const float a = alpha[bh];
    float* Sn = S_next + (size_t)bh * HD * HD;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const size_t e = (size_t)(32 * ib + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HD + col;
        Sn[e] = fmaf(a, Sp[e], uacc[ib][r]);
      }
  } else {
    float* P = partial + ((size_t)chunk * n_bh + bh) * HD * HD;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const size_t e = (size_t)(32 * ib + 8 * (r >> 2) + 4 * h2 + (r & 3)) * HD + col;
        P[e] = uacc[ib][r];
      }
  }
}

// S_next = alpha S_prev + sum over chunks (in chunk order) of the partials.
__global__ void __launch_bounds__(256)
commit_reduce_k(const float* __restrict__ partial, const float* __restrict__ alpha,
                const float* __restrict__ S_prev, float* __restrict__ S_next, int n_chunks,
                long n_bh) {
  const long q4 = (long)blockIdx.x * 256 + threadIdx.x;     // float4 index
  const long total4 = n_bh * HD * HD / 4;
  if (q4 >= total4) return;
  const long bh = q4 / (HD * HD / 4);
  const size_t stride4 = (size_t)n_bh * HD * HD / 4;
  const float4* P = reinterpret_cast<const float4*>(partial) + q4;
  float4 acc = P[0];
  for (int c = 1; c < n_chunks; ++c) {
    const float4 x = P[(size_t)c * stride4];
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  const float a = alpha[bh];
  const float4 s = reinterpret_cast<const float4*>(S_prev)[q4];
  float4 r;
  r.x = fmaf(a, s.x, acc.x);
  r.y = fmaf(a, s.y, acc.y);
  r.z = fmaf(a, s.z, acc.z);
  r.w = fmaf(a, s.w, acc.w);
  reinterpret_cast<float4*>(S_next)[q4] = r;
}

void commit_split(const Dims& d, int* chunk_tokens, int* n_chunks) {
  const long bh = (long)d.B * d.H;
  const int max_chunks = (d.T + 127) / 128;
  long want = (512 + bh - 1) / bh;
  int c = (int)std::min<long>(std::max<long>(want, 1), max_chunks);
  int ct = (d.T + c - 1) / c;
  ct = (ct + CT - 1) / CT * CT;
  *chunk_tokens = ct;
  *n_chunks = (d.T + ct - 1) / ct;
}

}  // namespace

hipError_t mfma_attention(const Dims& d, const void* q, const void* k, const void* v, void* o,
                          int64_t n_kv, int64_t kv_cap, hipStream_t s) {
  const int n_qblk = (d.T + AQ - 1) / AQ;
  const long nblk = (long)d.B * d.H * n_qblk;
  attn_mfma_k<<<(unsigned)nblk, 256, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), d.T, (int)n_kv, (long)kv_cap, d.scale * kLog2e, n_qblk);
  return hipGetLastError();
}

hipError_t mfma_feature_map(const Dims& d, const void* x, const void* phi, void* out,
                            bool normalize, hipStream_t s) {
  const int n_rblk = (d.T + MAP_ROWS - 1) / MAP_ROWS;
  const long nblk = (long)d.B * d.H * n_rblk;
  rowmap_mfma_k<MAP_PHI><<<(unsigned)nblk, 256, 0, s>>>(
      static_cast<const __bf16*>(x), phi, nullptr, static_cast<__bf16*>(out), nullptr, d.H, d.T,
      n_rblk, normalize ? 1 : 0);
  return hipGetLastError();
}

hipError_t mfma_inter_read(const Dims& d, const void* q_prime, const float* S,
                           const void* o_intra, void* o, void* o_inter, hipStream_t s) {
  const int n_rblk = (d.T + MAP_ROWS - 1) / MAP_ROWS;
  const long nblk = (long)d.B * d.H * n_rblk;
  rowmap_mfma_k<MAP_STATE><<<(unsigned)nblk, 256, 0, s>>>(
      static_cast<const __bf16*>(q_prime), S, static_cast<const __bf16*>(o_intra),
      static_cast<__bf16*>(o), static_cast<__bf16*>(o_inter), d.H, d.T, n_rblk, 0);
  return hipGetLastError();
}

size_t mfma_state_commit_ws_bytes(const Dims& d) {
  int ct, nc;
  commit_split(d, &ct, &nc);
  return nc > 1 ? (size_t)nc * d.B * d.H * HD * HD * sizeof(float) : 0;
}

hipError_t mfma_state_commit(const Dims& d, const void* k_prime, const void* v_prime,
                             const float* beta, const float* alpha, const float* S_prev,
                             float* S_next, void* ws, hipStream_t s) {
  int ct, nc;
  commit_split(d, &ct, &nc);
  const long n_bh = (long)d.B * d.H;
  float* partial = static_cast<float*>(ws);
  commit_mfma_k<<<(unsigned)(n_bh * nc), 256, 0, s>>>(
      static_cast<const __bf16*>(k_prime), static_cast<const __bf16*>(v_prime), beta, alpha,
      S_prev, S_next, partial, d.T, ct, nc, n_bh);
  if (nc > 1) {
    const long total4 = n_bh * HD * HD / 4;
    commit_reduce_k<<<(unsigned)((total4 + 255) / 256), 256, 0, s>>>(partial, alpha, S_prev,
                                                                     S_next, nc, n_bh);
  }
  return hipGetLastError();
}

}  // namespace arl2
