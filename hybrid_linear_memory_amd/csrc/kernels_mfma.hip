// bf16 MFMA kernels of the ARL2 hybrid attention step at head dimension 128,
// for gfx950 (CDNA4): v_mfma_f32_32x32x16_bf16 tiles, fp32 accumulation,
// LDS-staged K / V / state tiles.
//
// Step definitions: "Attend Locally, Remember Linearly" technical summary,
// §2.1 (feature maps Q' = Q Phi_q, K' = rownorm(K Phi_k), V' = V Phi_v;
// intra-frame bidirectional softmax; read O_inter = Q' S_{N-1}; update
// S_N = alpha S_{N-1} + K'^T diag(beta) (V' - K' S_{N-1})) and §2.2
// (frame-level access: one S_{N-1} for the whole frame). The MFMA operand
// layout is described in mfma_common.h.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "arl2_internal.h"
#include "mfma_common.h"

namespace arl2 {
namespace {

// ===========================================================================
// Intra-frame softmax attention (and the full-KV comparator).
//
// One workgroup = 8 waves = 128 query rows of one (b, h). The keys are dealt
// to two streams (even and odd tiles of 64 keys); waves 0-3 run stream A and
// waves 4-7 stream B, each wave owning 32 queries, so every SIMD holds one
// wave of each stream and interleaves the softmax of one with the matrix
// products of the other. The two streams' partial results are merged through
// LDS at the end.
//
// Tiles reach LDS by direct global->LDS loads (no staging registers), stored
// unpadded with an XOR swizzle of their 16-byte chunks so that the operand
// reads are free of bank conflicts: K is read as the A operand of
// S^T = K Q^T with plain 16-byte reads, V stays row-major and is read as the
// A operand of O^T = V^T P^T with transposing reads (ds_read_b64_tr_b16). Each
// lane therefore holds one query's scores, the row max and sum need a single
// cross-half exchange, and P^T feeds the second product straight from
// registers.
//
// Exponents are taken against a reference maximum fixed for the pass (the
// first tile's row maximum), so the accumulators are never rescaled inside the
// loop and later tiles need no row maximum at all. Each p is at most the
// lane's running sum l; if some l ends above 2^64 (a later tile exceeding the
// reference by more than 64 in log2 units, never for bounded inputs), the
// workgroup finds the exact row maxima in a scores-only pass and redoes the
// pass against them. Row sums add the bf16-rounded p that enter P V, so the
// normalised weights sum to one.
// ===========================================================================
constexpr int AQ = 128;                     // queries per workgroup
constexpr int AKT = 64;                     // keys per tile
constexpr int TILE_B = AKT * HD * 2;        // one 64 x 128 bf16 tile (16 KB)
constexpr float kRedoSum = 18446744073709551616.0f;   // 2^64: largest accepted l
constexpr float kLn2 = 0.6931471805599453f;
// LDS: the tiles of parity p (local tile index & 1) sit in arrays of their
// own: lk[p] = [stream A K, stream B K] of parity p and lv[p] = [stream A V,
// stream B V] of parity 1-p (each stream's V tiles are loaded one iteration
// after its K tiles; in split-key segments stream A's V tiles are of parity p,
// loaded with its K tiles). At an iteration of parity p every read is from lk[p] /
// lv[p] and every load in flight targets lk[1-p] / lv[1-p]: distinct objects,
// which lets the compiler see that the reads need not wait for the prefetch.
constexpr int AKV = 2 * TILE_B;


// Quarter-tile load by one wave of a stream: rows [16 q, 16 q + 16) (four
// 4-row instructions; qoff = 4096 q) of the 64 x 128 bf16 tile at byte offset
// `tile_off` of the buffer `src` into `dst`, 16-byte chunk p of row r holding
// global chunk p ^ swz(r). `off` holds the lane's byte offsets within 4 rows
// (K: by instruction parity; V: one). Rows past the end of the buffer (a tail
// tile past the last key) arrive as zeros: their scores are masked and their
// values meet p = 0.
template <bool IS_V>
__device__ __forceinline__ void tile_row4(char* dst, __amdgpu_buffer_rsrc_t src, int tile_off,
                                          int qoff, const int (&off)[2], int ii) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)(dst + qoff + ii * 1024), 16,
                                           IS_V ? off[0] : off[ii & 1],
                                           tile_off + qoff + ii * 1024, 0, 0);
}
template <bool IS_V>
__device__ __forceinline__ void tile_quarter(char* dst, __amdgpu_buffer_rsrc_t src, int tile_off,
                                             int qoff, const int (&off)[2]) {
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) tile_row4<IS_V>(dst, src, tile_off, qoff, off, ii);
}


// Per-lane LDS byte offsets of the operand reads within a tile.
//   K (A of S^T = K Q^T): lane row kb*32 + perm32(n), 16-byte chunk 2*kc + h2;
//     kb adds 32 rows (8192 bytes), the swizzle does not depend on kb.
//   V (A of O^T = V^T P^T, transposing read): source row
//     kb*32 + 16*(G>>1) + 8*cc + 4*half + c and column 32*db + 16*(G&1) + 4*j,
//     G = lane/16, c = (lane%16)/4, j = lane%4; kb, cc, half add 8192, 2048,
//     1024 bytes, the swizzle depends only on c.
struct AttnOffsets {
  int k[8];
  int v[4];
};

// The V tiles sit above the first 64 KB of LDS, beyond the reach of a read's
// 16-bit immediate offset, so the V offsets carry a 64 KB bias (kVBias) that
// the reads subtract again: the compiler then folds the rest of each address
// into the immediate instead of forming one register per read. The offsets are
// made opaque so that they stay one register each.
constexpr int kVBias = 65536;

__device__ __forceinline__ AttnOffsets attn_offsets(int lane) {
  AttnOffsets o;
  const int n = lane & 31, h2 = lane >> 5;
  const int krow = perm32(n);
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) o.k[kc] = krow * 256 + (((2 * kc + h2) ^ swz_k(krow)) << 4);
  const int G = lane >> 4, s = lane & 15, c = s >> 2, j = s & 3;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    o.v[db] = (16 * (G >> 1) + c) * 256 + ((4 * (db ^ c) + 2 * (G & 1) + (j >> 1)) << 4) +
              (j & 1) * 8 + kVBias;
    asm volatile("" : "+v"(o.v[db]));
  }
  return o;
}

// S^T: s[kb][r] = q . k[kb*32 + 16*h2 + r]
__device__ __forceinline__ void attn_qk(f32x16 (&s)[2], const char* Kb, const AttnOffsets& off,
                                        const bf16x8 (&qreg)[8]) {
  s[0] = zero16();
  s[1] = zero16();
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + kb * 8192 + off.k[kc]);
      s[kb] = mfma32(a, qreg[kc], s[kb]);
    }
  // keep only a few operand reads in flight ahead of their products
  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
  for (int i = 0; i < 13; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
}

// The same products with the caller's next-tile loads spread over them: after
// every second product, issue(n) sends load instruction n (n < n_ld, at most
// 8), so that the loads leave one at a time while the matrix unit works
// instead of in one burst that holds the wave. The order is fixed step by
// step (K operand reads three products ahead).
template <int N_LD, typename Issue>
__device__ __forceinline__ void attn_qk_ld(f32x16 (&s)[2], const char* Kb,
                                           const AttnOffsets& off, const bf16x8 (&qreg)[8],
                                           Issue&& issue) {
  bf16x8 ka[4];
  auto kread = [&](int i) __attribute__((always_inline)) {
    ka[i & 3] = *reinterpret_cast<const bf16x8*>(Kb + (i & 1) * 8192 + off.k[i >> 1]);
  };
  kread(0);
  kread(1);
  kread(2);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + 3 < 16) kread(i + 3);
    const int kc = i >> 1, kb = i & 1;
    s[kb] = mfma32(ka[i & 3], qreg[kc], kc == 0 ? zero16() : s[kb]);
    if ((i & 1) && (i >> 1) < N_LD) issue(i >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ __forceinline__ void attn_mask(f32x16 (&s)[2], int valid, int lane) {
  // key kb*32 + 16*h2 + r is past the end when the constant kb*32 + r reaches
  // lim (one register, no per-key index registers)
  const int lim = valid - 16 * (lane >> 5);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kb * 32 + r >= lim) s[kb][r] = -INFINITY;
}

__device__ __forceinline__ float attn_tile_max(const f32x16 (&s)[2]) {
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, s[kb][r]);
  return halves_max(m);
}

// p = 2^((s - m_ref) * sl2) rounded to bf16, and the row sums of the rounded
// p in fp32.
__device__ __forceinline__ void attn_softmax(bf16x8 (&pb)[2][2], float& l, float m_ref,
                                             const f32x16 (&s)[2], float sl2) {
  const float mc = m_ref * sl2;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      pb[kb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -mc));
  // row sums of the rounded p, two at a time (dot with (1, 1))
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const bf16x8 x = pb[kb][cc];
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), ones, ls1, false);
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), ones, ls1, false);
    }
  l += ls0 + ls1;
}

// O^T += V^T P^T: four independent accumulation chains advance together.
__device__ __forceinline__ void attn_pv(f32x16 (&acc)[4], const bf16x8 (&pb)[2][2],
                                        const char* Vb, const AttnOffsets& off) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const char* a = Vb + (off.v[db] - kVBias) + kb * 8192 + cc * 2048;
        const bf16x8 va = __builtin_shufflevector(tr_read(a), tr_read(a + 1024), 0, 1, 2, 3, 4,
                                                  5, 6, 7);
        acc[db] = mfma32(va, pb[kb][cc], acc[db]);
      }
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
  for (int i = 0; i < 13; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
}

__device__ __forceinline__ void attn_softmax_pv(f32x16 (&acc)[4], float& l, float m_ref,
                                                const f32x16 (&s)[2], const char* Vb,
                                                const AttnOffsets& off, float sl2) {
  bf16x8 pb[2][2];
  attn_softmax(pb, l, m_ref, s, sl2);
  attn_pv(acc, pb, Vb, off);
}

// Split key ranges ("stream-K"): when a shape's query blocks are too few to
// fill the chip, the key tiles of all query blocks are laid end to end and
// dealt evenly to one workgroup per compute unit, so a workgroup may hold the
// end of one query block's keys and the start of the next's (a segment each).
// A segment that is not a whole block publishes its unnormalised output, its
// reference maximum and its row sums in a slot of the workspace; the last of a
// block's segments to arrive (a per-block counter) merges them in key order.
// No workgroup waits for another.
constexpr int kSkSlotFloats = 8 * 2048 + 2 * 512;   // output, then (maximum, sum) pairs
constexpr int kSkStatOff = 8 * 2048 * 4;              // byte offset of the pairs
constexpr int kCoherent = 16;                         // cache policy: device scope (sc1)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct SkSeg {
  float* slots;                  // [2 * grid] slots of kSkSlotFloats
  unsigned long long* ctr;       // one counter per query block
  unsigned long long tag;        // this call's tag, in bits 16..63
  int nseg, iseg;                // the block's segment count, this segment's index
  int my_slot;                   // this segment's slot
  int wf, first_local;           // workgroup of the block's first segment, its slot parity
  __device__ int slot_of(int i) const { return i == 0 ? 2 * wf + first_local : 2 * (wf + i); }
};

// Counts one arrival at a block's counter; true for the block's last segment.
// The counter holds (tag << 16 | count) while a call is under way and is left
// at 0 by the last arrival; a value from another call (or any other content of
// the workspace) carries a different tag and counts as 0, so the workspace
// needs no clearing between calls. The first exchange assumes the 0 that a
// completed call leaves (no load first); a failed exchange returns the actual
// content, and each failure means another arrival succeeded, so the loop ends
// after at most nseg + 1 attempts.
__device__ __forceinline__ bool sk_arrive(unsigned long long* ctr, unsigned long long tag,
                                          int nseg) {
  unsigned long long old = 0;
  for (;;) {
    const unsigned c = (old >> 16) == (tag >> 16) ? (unsigned)(old & 0xFFFFu) : 0u;
    const bool last = (int)c + 1 == nseg;
    const unsigned long long nw = last ? 0ull : (tag | (c + 1u));
    if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return last;
  }
}

// With INTER (the fused read), the epilogue adds the inter-frame branch
// O_inter = Q M, M = Phi_q S (given transposed in `mt`, bf16 [B, H, D_v,
// D_in]); the two branches can also be written separately to o_intra /
// o_inter.
// One workgroup (logical block `blk`) of the attention; the LDS arrays are the
// kernel's (see AKV) and reach here as parameters so that, once inlined, every
// access still names its own array.
template <bool INTER, bool SK = false, bool LSE = false>
__device__ __forceinline__ void attn_block(
    int blk, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
    const __bf16* __restrict__ v, __bf16* __restrict__ o, int T, int n_kv, long kv_cap,
    float sl2, int n_qblk, const __bf16* __restrict__ mt, __bf16* __restrict__ o_intra,
    __bf16* __restrict__ o_inter, char* lk0, char* lk1, char* lv0, char* lv1,
    float (*mlx)[2][64], int& redo_flag, int t0 = 0, int nt = -1,
    const SkSeg* sk = nullptr, int* sk_last = nullptr, float* __restrict__ lse = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h2 = lane >> 5;
  const long bh = blk / n_qblk;
  const int qblk = blk % n_qblk;
  const int stream = wave >> 2;
  const int t = qblk * AQ + (wave & 3) * 32 + n;

  // The block's Q rows go to LDS (lk1, whose first use is the first
  // iteration's loads) by direct loads of whole 256-byte rows, wave w taking
  // rows [16 w, 16 w + 16) under the swz_r swizzle (rows past T arrive as
  // zeros); each wave takes its operand registers from there once they have
  // landed (run_pass, mode 0).
  bf16x8 qreg[8];
  {
    const int n_rows = min(AQ, T - qblk * AQ);
    const __amdgpu_buffer_rsrc_t qr =
        buffer_rsrc(q + ((size_t)bh * T + (size_t)qblk * AQ) * HD, (uint32_t)n_rows * HD * 2);
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      const int r = 16 * wave + 4 * qi + (lane >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (lds_void_t*)(lk1 + (16 * wave + 4 * qi) * 256),
                                               16, r * 256 + (((lane & 15) ^ swz_r(r)) << 4), 0,
                                               0, 0);
    }
  }
  auto read_q = [&]() __attribute__((always_inline)) {
    const int ql = (wave & 3) * 32 + n;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      qreg[kc] = *reinterpret_cast<const bf16x8*>(lk1 + ql * 256 +
                                                 (((2 * kc + h2) ^ swz_r(ql)) << 4));
  };
  const AttnOffsets off = attn_offsets(lane);

  // stream s owns global tiles s, s + 2, s + 4, ...: local tile j -> 2j + s.
  // Wave 4s + w loads rows [16w, 16w + 16) of the stream's K and V tiles.
  // this workgroup's key tiles: [t0, t0 + n_tiles) (all of them unless SK)
  const int n_tiles = SK ? nt : (n_kv + AKT - 1) / AKT;
  if (!SK) t0 = 0;
  const int my_cnt = (n_tiles - stream + 1) / 2;
  const uint32_t kv_bytes = (uint32_t)n_kv * (HD * 2);
  const __amdgpu_buffer_rsrc_t k_src = buffer_rsrc(k + (size_t)bh * kv_cap * HD, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_src = buffer_rsrc(v + (size_t)bh * kv_cap * HD, kv_bytes);
  int k_off[2], v_off[2];
  {
    const int p = lane & 15, L4 = lane >> 4;
    // rows 16 (wave & 1) + 4 e + L4 carry the K swizzle of instruction parity e
#pragma unroll
    for (int e = 0; e < 2; ++e)
      k_off[e] = L4 * 256 + ((p ^ swz_k(16 * (wave & 1) + 4 * e + L4)) << 4);
    v_off[0] = v_off[1] = L4 * 256 + ((p ^ swz_v(L4)) << 4);
  }
  auto load_k = [&](char* dst, int j) __attribute__((always_inline)) {
    int qoff = (wave & 3) * 4096;       // opaque: offsets formed in place
    asm volatile("" : "+s"(qoff));
    tile_quarter<false>(dst, k_src, (t0 + 2 * j + stream) * TILE_B, qoff, k_off);
  };
  auto load_v = [&](char* dst, int j) __attribute__((always_inline)) {
    int qoff = (wave & 3) * 4096;
    asm volatile("" : "+s"(qoff));
    tile_quarter<true>(dst, v_src, (t0 + 2 * j + stream) * TILE_B, qoff, v_off);
  };
  // instruction ii (0-3) of load_k / load_v
  auto load_k1 = [&](char* dst, int j, int ii) __attribute__((always_inline)) {
    int qoff = (wave & 3) * 4096;
    asm volatile("" : "+s"(qoff));
    tile_row4<false>(dst, k_src, (t0 + 2 * j + stream) * TILE_B, qoff, k_off, ii);
  };
  auto load_v1 = [&](char* dst, int j, int ii) __attribute__((always_inline)) {
    int qoff = (wave & 3) * 4096;
    asm volatile("" : "+s"(qoff));
    tile_row4<true>(dst, v_src, (t0 + 2 * j + stream) * TILE_B, qoff, v_off, ii);
  };
  // M^T (the inter-frame map, 32 KB) is loaded during the last iteration into
  // the K buffers that iteration leaves idle (rows under the swz_r swizzle),
  // wave w taking rows [16w, 16w + 16).
  const char* m_src = INTER ? reinterpret_cast<const char*>(mt + (size_t)bh * HD * HD) : nullptr;
  auto load_m = [&](char* dst) __attribute__((always_inline)) {
    if (!INTER) return;
    // (offsets formed here, not hoisted out of the loop into live registers)
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const __amdgpu_buffer_rsrc_t mr = buffer_rsrc(m_src, HD * HD * 2);
#pragma unroll
    for (int qi = 0; qi < 4; ++qi) {
      const int r = 16 * wave + 4 * qi + (lo >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(mr, (lds_void_t*)(dst + (16 * wave + 4 * qi) * 256),
                                               16, r * 256 + (((lo & 15) ^ swz_r(r)) << 4), 0, 0,
                                               0);
    }
  };
  // Every wave's loads of the current tile have landed once its own have
  // (vmcnt) and all waves have reached the barrier.
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070);     // vmcnt(0) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  };

  // The two streams run half an iteration apart so that the two waves sharing
  // a SIMD alternate between matrix products and the softmax, each wave's
  // products forming one block per iteration: after barrier it, stream A
  // computes P V of its tile it-1 (P kept in registers) and the scores of its
  // tile it, then their softmax; stream B first takes the softmax of its tile
  // it-1 (scores kept in registers), then P V of that tile and the scores of
  // its tile it. So while one wave of a SIMD runs its softmax the other runs
  // its products. Tile j's V sits in the V buffers of parity j + 1 for both
  // streams (loaded during iteration j, read during iteration j + 1).
  // (Split-key segments keep the earlier order of stream A, which finishes
  // each of its tiles within its iteration: their short key ranges would pay
  // the extra iteration once per segment. There tile j's V of stream A sits in
  // the V buffers of parity j.)
  const int n_iter = SK ? max((n_tiles + 1) / 2, n_tiles / 2 + 1)
                        : (n_tiles + 1) / 2 + 1;   // same for every wave
  f32x16 acc[4];
  float l = 0.f, m_ref = -INFINITY;
  // One pass over the keys. Mode 0: reference maximum from the stream's first
  // tile; returns whether the sums call for a redo. Mode 1: scores only, exact
  // row maxima into m_ref. Mode 2: the pass against the exact maxima. Written
  // as a lambda called per mode (rather than a loop) so that the rarely taken
  // later modes do not extend live ranges in the first.
  auto run_pass = [&](const int mode) -> bool {
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = zero16();
    l = 0.f;
    if (mode == 1) m_ref = -INFINITY;
    if (tid == 0) redo_flag = 0;
    f32x16 s[2];
    bf16x8 pa[2][2];      // stream A: P of its previous tile
    auto scores_tail = [&](int j) __attribute__((always_inline)) {
      const int valid = n_kv - (t0 + 2 * j + stream) * AKT;
      if (valid < AKT) attn_mask(s, valid, lane);
      if (mode == 1) m_ref = fmaxf(m_ref, attn_tile_max(s));
      if (mode == 0 && j == 0) m_ref = attn_tile_max(s);
    };
    // the scores of local tile j with load instructions spread over them
    auto scores_ld = [&](int j, const char* Kb, auto n_ld, auto&& issue)
        __attribute__((always_inline)) {
      attn_qk_ld<decltype(n_ld)::value>(s, Kb, off, qreg, issue);
      scores_tail(j);
    };
    auto scores = [&](int j, const char* Kb) __attribute__((always_inline)) {
      attn_qk(s, Kb, off, qreg);
      const int valid = n_kv - (t0 + 2 * j + stream) * AKT;
      if (valid < AKT) attn_mask(s, valid, lane);
      if (mode == 1) m_ref = fmaxf(m_ref, attn_tile_max(s));
      if (mode == 0 && j == 0) m_ref = attn_tile_max(s);
    };
    // Iteration it of parity p: kc / vc = lk[p] / lv[p] (read), kn / vn =
    // lk[1-p] / lv[1-p] (loaded).
    auto step_a = [&](int it, char* kc, char* vc, char* kn, char* vn)
        __attribute__((always_inline)) {
      sync();
      if (it == n_iter - 1) load_m(kn);
      if constexpr (SK) {
        // (split-key segments: the loads in one burst measured faster)
        if (it + 1 < my_cnt) {
          load_k(kn, it + 1);
          load_v(vn, it + 1);
        }
        if (it < my_cnt) scores(it, kc);
        if (mode != 1 && it < my_cnt) attn_softmax_pv(acc, l, m_ref, s, vc, off, sl2);
      } else {
        if (mode != 1 && it >= 1 && it <= my_cnt) attn_pv(acc, pa, vc, off);
        if (it < my_cnt) {
          if (it + 1 < my_cnt)
            scores_ld(it, kc, std::integral_constant<int, 8>(), [&](int n2) {
              if (n2 < 4) load_k1(kn, it + 1, n2);
              else load_v1(vn, it, n2 - 4);
            });
          else
            scores_ld(it, kc, std::integral_constant<int, 4>(),
                      [&](int n2) { load_v1(vn, it, n2); });
          if (mode != 1) attn_softmax(pa, l, m_ref, s, sl2);
        }
      }
    };
    auto step_b = [&](int it, char* kc, char* vc, char* kn, char* vn)
        __attribute__((always_inline)) {
      sync();
      if (it == n_iter - 1) load_m(kn);
      if constexpr (!SK) {
        // the V tile this stream needs next iteration, right after the barrier
        // (its buffer is free since then), a full iteration ahead of its wait
        if (it < my_cnt) load_v(vn + TILE_B, it);
      }
      if (mode != 1 && it >= 1 && it <= my_cnt)
        attn_softmax_pv(acc, l, m_ref, s, vc + TILE_B, off, sl2);
      if constexpr (SK) {
        if (it < my_cnt) load_v(vn + TILE_B, it);
        if (it + 1 < my_cnt) load_k(kn + TILE_B, it + 1);
        if (it < my_cnt) scores(it, kc + TILE_B);
      } else if (it + 1 < my_cnt) {
        scores_ld(it, kc + TILE_B, std::integral_constant<int, 4>(),
                  [&](int n2) { load_k1(kn + TILE_B, it + 1, n2); });
      } else if (it < my_cnt) {
        scores(it, kc + TILE_B);
      }
    };
    if (stream == 0) {
      if (my_cnt > 0) load_k(lk0, 0);
      if (SK && my_cnt > 0) load_v(lv0, 0);
      if (mode == 0) {
        // Q landed for every wave (the 4 or 8 tile loads just issued may still fly)
        if (SK && my_cnt > 0) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        else if (my_cnt > 0) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        read_q();
      }
      for (int it = 0; it < n_iter; it += 2) {
        step_a(it, lk0, lv0, lk1, lv1);
        if (it + 1 < n_iter) step_a(it + 1, lk1, lv1, lk0, lv0);
      }
    } else {
      if (my_cnt > 0) load_k(lk0 + TILE_B, 0);
      if (mode == 0) {
        if (my_cnt > 0) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        read_q();
      }
      // Stream B's chain (softmax, P V, scores) is the longer one after each
      // barrier: its instructions go first when both waves of a SIMD can issue.
      __builtin_amdgcn_s_setprio(2);
      for (int it = 0; it < n_iter; it += 2) {
        step_b(it, lk0, lv0, lk1, lv1);
        if (it + 1 < n_iter) step_b(it + 1, lk1, lv1, lk0, lv0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    if (mode == 0 && __any(l > kRedoSum)) redo_flag = 1;     // every writer stores 1
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int redo = redo_flag;
    __syncthreads();                     // everyone has read the flag
    return mode == 0 && redo != 0;
  };
  if (run_pass(0)) {
    run_pass(1);
    run_pass(2);
  }

  // Stream A finalises output columns 0-63 (blocks 0-1) and stream B columns
  // 64-127 (blocks 2-3); the two waves of a pair swap the other half of their
  // accumulators through LDS. The inter-frame branch of a wave's columns,
  // O_inter^T = M^T Q^T, is computed by the wave that writes them, from M^T in
  // the K buffers of parity n_iter & 1.
  f32x16 oi[2];
  if (INTER) {
    const char* mb = (n_iter & 1) ? lk1 : lk0;
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const int row = 32 * (2 * stream + b2) + n;
      oi[b2] = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(mb + row * 256 + (((2 * kc + h2) ^ swz_r(row)) << 4));
        oi[b2] = mfma32(a, qreg[kc], oi[b2]);
      }
    }
  }
  float* ex_w = reinterpret_cast<float*>(stream == 0 ? lv0 : lv1) + (wave & 3) * (32 * 64);
  const float* ex_r =
      reinterpret_cast<const float*>(stream == 0 ? lv1 : lv0) + (wave & 3) * (32 * 64);
  // (selected whole, so that the accumulators are never indexed at run time)
  const f32x16 give[2] = {stream == 0 ? acc[2] : acc[0], stream == 0 ? acc[3] : acc[1]};
  const f32x16 keep[2] = {stream == 0 ? acc[0] : acc[2], stream == 0 ? acc[1] : acc[3]};
#pragma unroll
  for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
    for (int r = 0; r < 16; ++r) ex_w[(b2 * 16 + r) * 64 + lane] = give[b2][r];
  mlx[wave][0][lane] = m_ref;
  mlx[wave][1][lane] = l;
  __syncthreads();
  const float mb = mlx[wave ^ 4][0][lane];
  const float lb = mlx[wave ^ 4][1][lane];
  const float m = fmaxf(m_ref, mb);
  const float fa = __builtin_amdgcn_exp2f((m_ref - m) * sl2);
  const float fb = __builtin_amdgcn_exp2f((mb - m) * sl2);
  const float lsum = halves_sum(l * fa + lb * fb);
  // Writes this wave's 32 queries x 64 output columns: intra(b2, r) is the
  // normalised softmax branch of accumulator register r of column block b2.
  // Each requested output goes through LDS (the K buffers are idle now): the
  // workgroup's 128 x 128 bf16 tile, row-major with 16-byte chunks under the
  // swz_r swizzle, then whole rows to memory (each store instruction writes
  // four 256-byte rows, where a lane's registers hold 8-byte pieces of 32).
  auto store = [&](auto intra_of) __attribute__((always_inline)) {
    char* st = lk0;
    const int ql = (wave & 3) * 32 + n;
    const size_t row0 = (size_t)bh * T + (size_t)qblk * AQ;
    const int n_rows = min(AQ, T - qblk * AQ);
#pragma unroll
    for (int kind = 0; kind < 3; ++kind) {
      __bf16* out = kind == 0 ? o : kind == 1 ? o_intra : o_inter;
      if (!out) continue;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        const int db = 2 * stream + b2;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 w;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * jj + i;
            const float intra = kind == 2 ? 0.f : intra_of(b2, r);
            const float inter = INTER && kind != 1 ? oi[b2][r] : 0.f;
            w[i] = (__bf16)(intra + inter);
          }
          const int c = 4 * db + jj;          // 16-byte chunk of the row
          *reinterpret_cast<bf16x4*>(st + ql * 256 + ((c ^ swz_r(ql)) << 4) + 8 * h2) = w;
        }
      }
      __syncthreads();
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const int g = tid + 512 * k2, r = g >> 4, c = g & 15;
        if (r < n_rows)
          *reinterpret_cast<bf16x8*>(out + (row0 + r) * HD + 8 * c) =
              *reinterpret_cast<const bf16x8*>(st + r * 256 + ((c ^ swz_r(r)) << 4));
      }
      __syncthreads();                    // the tile is read before the next output
    }
  };
  if (SK && sk->nseg > 1) {
    // A part of the query block's keys: publish the unnormalised output, the
    // reference maximum and the row sum; the segment that arrives last merges
    // every segment's results, in key order, and writes the output. Slots are
    // written and read with the device-scope coherence bit (what agent-scope
    // atomic accesses compile to: coherent across the XCDs' L2 caches without
    // writing back or invalidating them); each wave waits for its stores to
    // complete before the workgroup counts its arrival, and the last arrival
    // reads the slots only after that.
    f32x4 c[8];
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b2 = g >> 2, r = 4 * (g & 3) + e;
        c[g][e] = keep[b2][r] * fa + ex_r[(b2 * 16 + r) * 64 + lane] * fb;
      }
    const __amdgpu_buffer_rsrc_t mine =
        buffer_rsrc(sk->slots + (size_t)sk->my_slot * kSkSlotFloats, kSkSlotFloats * 4);
#pragma unroll
    for (int g = 0; g < 8; ++g)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c[g]), mine,
                                             ((wave * 8 + g) * 64 + lane) * 16, 0, kCoherent);
    const f32x2 ml = {m, lsum};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), mine,
                                          kSkStatOff + (wave * 64 + lane) * 8, 0, kCoherent);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) *sk_last = sk_arrive(sk->ctr + blk, sk->tag, sk->nseg) ? 1 : 0;
    __syncthreads();
    if (*sk_last == 0) return;
    // The other segments (at most two: the host plans only grids whose
    // workgroup ranges cover at least half a block), all loads issued before
    // the first use (an index past nseg reads an empty range: zeros, no access).
    f32x2 om[2];
    f32x4 od[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = j < sk->iseg ? j : j + 1;
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc(sk->slots + (size_t)sk->slot_of(i < sk->nseg ? i : 0) * kSkSlotFloats,
                      i < sk->nseg ? kSkSlotFloats * 4 : 0);
      om[j] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                            rs, kSkStatOff + (wave * 64 + lane) * 8, 0, kCoherent));
#pragma unroll
      for (int g = 0; g < 8; ++g)
        od[j][g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, ((wave * 8 + g) * 64 + lane) * 16, 0,
                                                 kCoherent));
    }
    float mx = m;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j + 1 < sk->nseg) mx = fmaxf(mx, om[j][0]);
    f32x4 acc2[8];
    float lt = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) acc2[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    // key order: segment i is this one (i == iseg) or other j = i - (i > iseg)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= sk->nseg) break;
      const bool own = i == sk->iseg;
      const bool j1 = i > sk->iseg ? i - 1 == 1 : i == 1;
      const float mi = own ? m : (j1 ? om[1][0] : om[0][0]);
      const float li = own ? lsum : (j1 ? om[1][1] : om[0][1]);
      const float wi = __builtin_amdgcn_exp2f((mi - mx) * sl2);
      lt += wi * li;
#pragma unroll
      for (int g = 0; g < 8; ++g) acc2[g] += wi * (own ? c[g] : (j1 ? od[1][g] : od[0][g]));
    }
    const float inv = 1.f / lt;
    store([&](int b2, int r) __attribute__((always_inline)) {
      return acc2[b2 * 4 + (r >> 2)][r & 3] * inv;
    });
    return;
  }
  // with LSE: the row's log-sum-exp of the scaled scores (natural log): the
  // weights are 2^((s - m) sl2) / lsum, so log sum_j e^(scale s_j) =
  // (m sl2 + log2(lsum)) ln 2
  if (LSE && stream == 0 && h2 == 0 && t < T)
    lse[(size_t)bh * T + t] = (m * sl2 + log2f(lsum)) * kLn2;
  const float inv = 1.f / lsum;
  store([&](int b2, int r) __attribute__((always_inline)) {
    return (keep[b2][r] * fa + ex_r[(b2 * 16 + r) * 64 + lane] * fb) * inv;
  });
}

// L2 warm-up by a workgroup on an otherwise idle compute unit: block i of the
// role (i = 0, 1, ...; blocks are dealt to the XCDs round-robin, so it runs on
// XCD i % 8) reads, tile by tile in the order the attention consumes them, the
// K and V of the heads whose attention workgroups the XCD holds (the logical
// blocks xcd_remap gives it), so that their tile loads find L2 warm. The data
// lands in this workgroup's own LDS and is discarded.
__device__ __forceinline__ void attn_l2_warm(int i, int per_xcd, int n_attn, int n_qblk,
                                             const __bf16* k, const __bf16* v, int n_kv,
                                             long kv_cap, char* scratch) {
  constexpr int X = 8;
  const int x = i % X, part = i / X;
  const int per = n_attn / X, rem = n_attn % X;
  const int first = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  const int cnt = per + (x < rem ? 1 : 0);
  if (cnt == 0) return;
  const int h0 = first / n_qblk, nh = (first + cnt - 1) / n_qblk - h0 + 1;
  const int n_tiles = (n_kv + AKT - 1) / AKT;
  const long units = (long)n_tiles * nh * 2;          // (tile, head, K or V), tile-major
  const long u0 = units * part / per_xcd, u1 = units * (part + 1) / per_xcd;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t kv_bytes = (uint32_t)n_kv * (HD * 2);
  for (long u = u0; u < u1; ++u) {
    const int g = (int)(u / (2 * nh));
    const int hh = (int)(u % (2 * nh)) >> 1;
    const __bf16* base = ((u & 1) ? v : k) + (size_t)(h0 + hh) * kv_cap * HD;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base, kv_bytes);
    // 16 KB tile: two 1 KB pieces per wave
#pragma unroll
    for (int c = 0; c < 2; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(scratch + wave * 1024), 16,
                                               lane * 16, g * TILE_B + (2 * wave + c) * 1024, 0,
                                               0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Blocks [0, n_attn): attention workgroups; blocks from n_attn_pad (n_attn
// rounded up to the XCD count): the L2 warm-up role (when the grid leaves
// compute units idle).
template <bool INTER, bool LSE = false>
__global__ void __launch_bounds__(512, 1)
attn_mfma_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
            const __bf16* __restrict__ v, __bf16* __restrict__ o, int T, int n_kv,
            long kv_cap, float sl2, int n_qblk, const __bf16* __restrict__ mt,
            __bf16* __restrict__ o_intra, __bf16* __restrict__ o_inter, int n_attn,
            int n_attn_pad, float* __restrict__ lse = nullptr) {
  __shared__ __attribute__((aligned(1024))) char lk0[AKV];
  __shared__ __attribute__((aligned(1024))) char lk1[AKV];
  __shared__ __attribute__((aligned(1024))) char lv0[AKV];
  __shared__ __attribute__((aligned(1024))) char lv1[AKV];
  __shared__ float mlx[8][2][64];
  __shared__ int redo_flag;
  const int b = blockIdx.x;
  if (b < n_attn)
    attn_block<INTER, false, LSE>(xcd_remap(b, n_attn), q, k, v, o, T, n_kv, kv_cap, sl2,
                                  n_qblk, mt, o_intra, o_inter, lk0, lk1, lv0, lv1, mlx,
                                  redo_flag, 0, -1, nullptr, nullptr, lse);
  else if (b >= n_attn_pad)
    attn_l2_warm(b - n_attn_pad, ((int)gridDim.x - n_attn_pad) / 8, n_attn, n_qblk, k, v, n_kv,
                 kv_cap, lk0);
}

// Split-key attention grid: one workgroup per compute unit (gridDim.x = G).
// Block qb's tiles sit at [qb L + pad, (qb + 1) L) of a line of n_blk L slots
// (L = tiles per block + pad); workgroup w takes [w V / G, (w + 1) V / G),
// V = n_blk L. The pad slots before each block make a workgroup that crosses
// a block boundary (and pays a second ramp and a merge) take fewer tiles. A
// workgroup's segments between its first and its last are whole blocks, so
// only those two can be partial: two slots per workgroup.
__device__ __forceinline__ int sk_wg_of(long x, long V, int G) {
  return (int)(((x + 1) * G - 1) / V);
}

template <bool INTER>
__global__ void __launch_bounds__(512, 1)
attn_sk_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
          const __bf16* __restrict__ v, __bf16* __restrict__ o, int T, float sl2, int n_qblk,
          const __bf16* __restrict__ mt, __bf16* __restrict__ o_intra,
          __bf16* __restrict__ o_inter, int n_blk, int pad, float* __restrict__ slots,
          unsigned long long* __restrict__ ctr, unsigned long long tag) {
  __shared__ __attribute__((aligned(1024))) char lk0[AKV];
  __shared__ __attribute__((aligned(1024))) char lk1[AKV];
  __shared__ __attribute__((aligned(1024))) char lv0[AKV];
  __shared__ __attribute__((aligned(1024))) char lv1[AKV];
  __shared__ float mlx[8][2][64];
  __shared__ int redo_flag;
  __shared__ int sk_last;
  const int G = (int)gridDim.x;
  const int w = xcd_remap(blockIdx.x, G);
  const int n_tiles = (T + AKT - 1) / AKT;
  const long L = n_tiles + pad, V = (long)n_blk * L;
  const long v0 = (long)w * V / G, v1 = (long)(w + 1) * V / G;
  int local = 0;        // segments of this workgroup so far
  for (int qb = (int)(v0 / L); qb < n_blk && (long)qb * L < v1; ++qb) {
    const long rs = (long)qb * L + pad;
    const long a = v0 > rs ? v0 : rs;
    const long b = v1 < rs + n_tiles ? v1 : rs + n_tiles;
    if (a >= b) continue;
    SkSeg sg;
    sg.slots = slots;
    sg.ctr = ctr;
    sg.tag = tag;
    sg.wf = sk_wg_of(rs, V, G);
    sg.nseg = sk_wg_of(rs + n_tiles - 1, V, G) - sg.wf + 1;
    sg.iseg = w - sg.wf;
    sg.first_local = (long)sg.wf * V / G < (long)qb * L ? 1 : 0;
    sg.my_slot = 2 * w + (local > 0 ? 1 : 0);    // only a first or a last segment is partial
    if (local > 0) __syncthreads();      // the previous segment's LDS reads are done
    attn_block<INTER, true>(qb, q, k, v, o, T, T, T, sl2, n_qblk, mt, o_intra, o_inter, lk0,
                            lk1, lv0, lv1, mlx, redo_flag, (int)(a - rs), (int)(b - a), &sg,
                            &sk_last);
    ++local;
  }
}

// ===========================================================================
// Read preparation for the fused read: M = Phi_q[h] S[b,h] (the inter-frame
// read Q' S = Q (Phi_q S) folded into one D x D map per head), stored
// transposed in bf16 so that the attention epilogue reads it as an MFMA A
// operand. One workgroup per (b, h, 32-column block of M); wave w computes
// rows [32w, 32w + 32).
// ===========================================================================
__global__ void __launch_bounds__(256)
read_prep_k(const __bf16* __restrict__ phi, const float* __restrict__ S,
            __bf16* __restrict__ mt, int H) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  const long bh = blockIdx.x >> 2;
  const int jb = blockIdx.x & 3;
  const int j = 32 * jb + n;
  const float* Sh = S + (size_t)bh * HD * HD;
  const __bf16* P = phi + (size_t)(bh % H) * HD * HD + (size_t)(32 * wave + n) * HD + 8 * h2;
  f32x16 acc = zero16();
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    bf16x8 b;
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = (__bf16)Sh[(size_t)(16 * kc + 8 * h2 + u) * HD + j];
    acc = mfma32(ld8(P + 16 * kc), b, acc);
  }
  // acc[r] = M[i = 32w + 8(r/4) + 4h2 + r%4][j]  ->  MT[j][i]
  __bf16* out = mt + (size_t)bh * HD * HD + (size_t)j * HD + 32 * wave + 4 * h2;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    bf16x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (__bf16)acc[4 * jj + i];
    *reinterpret_cast<bf16x4*>(out + 8 * jj) = w;
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

// Feature maps of up to three inputs of one shape in one launch (the
// token-level pass's Q', K', V'; the commit backward's K' with its rows'
// norms, and V'): workgroups [j per_prob, (j + 1) per_prob) map input j;
// input 0 is the kernel's x / mat / out / normalize / norms.
struct MapMore {
  const __bf16* x1;
  const void* m1;
  __bf16* o1;
  int n1;
  const __bf16* x2;
  const void* m2;
  __bf16* o2;
  int n2;
};

template <int MODE>
__global__ void __launch_bounds__(256)
rowmap_mfma_k(const __bf16* __restrict__ x, const void* __restrict__ mat,
              const __bf16* o_intra, __bf16* out, __bf16* __restrict__ o_inter, int H,
              int T, int n_rblk, int normalize, MapMore more = MapMore{}, int per_prob = 0,
              float* __restrict__ norms = nullptr) {
  __shared__ __attribute__((aligned(16))) __bf16 MT[HD * MS];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h2 = lane >> 5;
  int bid = blockIdx.x, nb = gridDim.x;
  if (MODE == MAP_PHI && per_prob > 0) {
    const int j = bid / per_prob;
    bid -= j * per_prob;
    nb = per_prob;
    if (j > 0) norms = nullptr;    // (the norms belong to input 0)
    if (j == 1) {
      x = more.x1;
      mat = more.m1;
      out = more.o1;
      normalize = more.n1;
    } else if (j == 2) {
      x = more.x2;
      mat = more.m2;
      out = more.o2;
      normalize = more.n2;
    }
  }
  const int blk = xcd_remap(bid, nb);
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
    const float nr = sqrtf(ss);
    if (norms && h2 == 0 && t < T) norms[row] = nr;
    const float inv = 1.f / fmaxf(nr, 1e-12f);
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

// Wave-wide DMA of `n_inst` x 4 rows (256-byte rows) starting at row r_begin of
// a row-major bf16 matrix into LDS under chunk swizzle `swz` (rows past
// `rows_valid` are clamped to the last valid row).
template <int SWZ>
__device__ __forceinline__ void rows_load(char* dst, const char* src, int r_begin, int n_inst,
                                          int rows_valid, int lane) {
  const int p = lane & 15;
  for (int i = 0; i < n_inst; ++i) {
    const int r = r_begin + 4 * i + (lane >> 4);
    const int sw = SWZ == 0 ? swz_k(r) : SWZ == 1 ? swz_v(r) : swz_r(r);
    const int rc = min(r, rows_valid - 1);
    const char* g = src + (size_t)rc * 256 + ((p ^ sw) << 4);
    __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)(dst + (r_begin + 4 * i) * 256),
                                     16, 0, 0);
  }
}

// ===========================================================================
// Column-split commit from the clean pass's raw K and V: the feature maps
// K' = rownorm(K Phi_k), V' = V Phi_v and the gated delta update, one
// workgroup (8 waves) per (b, h, 32-column block `cb` of the state) over all of
// the frame's tokens. A column block of the update needs only the same
// columns of S and V':
//   S_N[:, cols] = alpha S_{N-1}[:, cols] + K'^T diag(beta) (V'[:, cols] - K' S_{N-1}[:, cols]),
// so no workgroup needs another's results: the workgroup writes S_N[:, cols]
// and, when asked, the next frame's map for those columns,
// M^T[cols, :] = (Phi_q S_N[:, cols])^T. K' rows need all of K~ = K Phi_k (the
// row norm), so each of a head's four workgroups forms the whole of K~; they
// sit on one XCD and share the K and V reads in its L2.
//
// Wave w takes the 32-token slices w, w + 8, ... Per slice (all in registers
// except one transposition of K' through the wave's own LDS buffer):
//   K~^T = Phi_k^T K^T  (A = Phi_k^T by transposing LDS reads, B = K rows
//                        straight from global memory; lane = token, so the
//                        row norm is an in-lane sum and one half exchange)
//   V'   = V Phi_v[:, cols] (A = V rows from global memory, B from LDS)
//   P^   = K' S[:, cols]    (A = K' from the K~^T registers, B = S held in
//                        registers with its rows in the order those registers
//                        give the contraction index)
//   W    = beta (V' - P^);  U[:, cols] += K'^T W  (A = K' transposed via LDS)
// Tokens are loaded in the perm32 order, so that the accumulators of P^ and V'
// hold W in the register order that U's contraction takes. At the end the
// eight per-wave sums of U are added in wave order through LDS.
// ===========================================================================
constexpr int CC_WAVES = 8;
constexpr int CC_SLICE = 32;                    // tokens per slice
constexpr int CC_KP_B = CC_SLICE * HD * 2;      // one wave's K' slice (8 KB)
constexpr int CC_RED_B = HD * 32 * 4;           // one wave's U column block (16 KB)
constexpr int CC_ST_LD = HD + 8;                // row of the transposed S_N block (bf16)
constexpr int CC_OPS_B = 8 * 64 * 16;           // one fixed B operand in lane order (8 KB)
static_assert(4 * CC_KP_B <= AKV && 2 * CC_RED_B <= AKV && HD * HD * 2 <= AKV &&
                  2 * CC_OPS_B + CC_WAVES * 128 <= AKV,
              "column-split commit regions fit the arrays");

// The LDS arrays l0..l3 (32 KB each): Phi_k; the fixed B operands (Phi_v and
// S columns); the K' buffers of waves 0-3 and of waves 4-7; then the per-wave
// U sums (two waves per array).
// Token parts: the frame's 32-token slices are split into n_parts parts (two
// in the clean pass, up to eight in the commit alone), one workgroup each
// (logical block (n_parts bh + part) 4 + cb of column block 4 bh + cb; part p
// takes slices [ceil(p n / n_parts), ceil((p + 1) n / n_parts)) of the n).
// Each publishes its fp32 sum U_p[:, cols] (16 KB, lane order e = tid + 512 i)
// in its slot of the workspace with device-scope stores, waits for them to
// complete and counts its arrival on the column block's counter (two parts:
// pair_arrive, one exchange; more: commit_arrive, a compare-and-swap loop);
// the last to arrive loads the others' sums with device-scope loads and
// finishes the column block with U = U_0 + U_1 + ... in part order (the same
// sum whichever part arrives last). Device-scope accesses are served at the
// point where the XCDs' L2 caches are coherent, so no part can see a stale
// copy of a slot.
struct CommitPair {
  float* slots;                  // [4 B H][n_parts][4096] floats
  unsigned long long* ctr;       // one per (b, h, column block)
  unsigned long long tag;        // this call's tag, in bits 16..63 (never 0)
  int n_parts;                   // 2..8
};

// Counts one arrival at a column block's counter; true for the last of the
// n_parts parts. The counter holds (tag | count) while a call is under way and
// is left at 0 by the last arrival; a value carrying another tag (a completed
// call leaves 0; a fresh workspace holds anything) counts as no arrival, so
// the workspace needs no clearing between calls. The first exchange assumes
// the 0 that a completed call leaves (no load first); a failed exchange
// returns the actual content, and each failure means another arrival
// succeeded, so the loop ends after at most n_parts + 1 attempts.
__device__ __forceinline__ bool commit_arrive(unsigned long long* ctr, unsigned long long tag,
                                              int n_parts) {
  unsigned long long old = 0;
  for (;;) {
    const unsigned c = (old >> 16) == (tag >> 16) ? (unsigned)(old & 0xFFFFu) : 0u;
    const bool last = (int)c + 1 == n_parts;
    const unsigned long long nw = last ? 0ull : (tag | (c + 1u));
    if (__hip_atomic_compare_exchange_strong(ctr, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return last;
  }
}
constexpr int kScopeDevice = 16;   // cache policy bits: device scope (sc1)

// The last part's merge: every other part's sum (device-scope loads, all in
// flight at once), then U = U_0 + U_1 + ... in part order, this part's own
// sum (sv, lane order e = tid + 512 i) taking its place.
template <int NP>
__device__ __forceinline__ void commit_merge(float (&sv)[8], const float* cslots, int part,
                                             int tid) {
  float pv[NP][8];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const __amdgpu_buffer_rsrc_t other = buffer_rsrc(cslots + (size_t)j * 4096, 4096 * 4);
    if (j == part) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pv[j][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               other, (tid + 512 * i) * 4, 0, kScopeDevice));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float acc = part == 0 ? sv[i] : pv[0][i];
#pragma unroll
    for (int j = 1; j < NP; ++j) acc += j == part ? sv[i] : pv[j][i];
    sv[i] = acc;
  }
}

__device__ __forceinline__ void commit_col_block(
    int blk, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ phi_k, const __bf16* __restrict__ phi_v,
    const __bf16* __restrict__ phi_q, const float* __restrict__ beta,
    const float* __restrict__ alpha, const float* __restrict__ S_prev,
    float* __restrict__ S_next, __bf16* __restrict__ mt_next, int H, int T, char* l0, char* l1,
    char* l2, char* l3, const CommitPair* pair, int* flag) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h2 = lane >> 5;
  // logical block (n_parts bh + part) 4 + cb: the four column blocks that
  // read the same token part of K and V are consecutive, so the XCD-aware
  // block order keeps them on one XCD (one L2 fetch of that part)
  const int n_parts = pair ? pair->n_parts : 1;
  const int part = pair ? (blk >> 2) % n_parts : 0;
  const int cblk = pair ? (blk / (4 * n_parts)) * 4 + (blk & 3) : blk;   // 4 bh + cb
  const long bh = cblk >> 2;
  const int cb = cblk & 3;
  const int h = (int)(bh % H);
  const int col = 32 * cb + n;

  // Phi_k into l0 (waves 0-3, 32 rows each), row-major under the swz_v
  // swizzle for the transposing reads. The two B operands that stay fixed over
  // the frame go to l1 in MFMA lane order (16 bytes per lane and step, read
  // back without conflicts): Phi_v[:, cols] for V' = V Phi_v[:, cols], step kc
  // giving lane (c, h2) Phi_v[16 kc + 8 h2 + u][32 cb + c]; and S_{N-1}[:, cols]
  // for P^ = K' S, step j giving lane (c, h2) S[d][32 cb + c] with
  // d = 32 (j / 2) + 16 (j % 2) + 8 (u / 4) + 4 h2 + u % 4, the K~ columns that
  // the K~^T registers of block j / 2, registers 8 (j % 2) .. + 7 hold.
  if (wave < 4)
    rows_load<1>(l0, reinterpret_cast<const char*>(phi_k + (size_t)h * HD * HD), 32 * wave, 8,
                 HD, lane);
  const float* Sp = S_prev + (size_t)bh * HD * HD;
  {
    const int st = tid >> 6, sl_lane = tid & 63;
    const int c = 32 * cb + (sl_lane & 31), g2 = sl_lane >> 5;
    const __bf16* pv = phi_v + (size_t)h * HD * HD;
    bf16x8 a, b;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = pv[(size_t)(16 * st + 8 * g2 + u) * HD + c];
      const int d = 32 * (st >> 1) + 16 * (st & 1) + 8 * (u >> 2) + 4 * g2 + (u & 3);
      b[u] = (__bf16)Sp[(size_t)d * HD + c];
    }
    *reinterpret_cast<bf16x8*>(l1 + tid * 16) = a;
    *reinterpret_cast<bf16x8*>(l1 + CC_OPS_B + tid * 16) = b;
  }
  const uint32_t act_b = (uint32_t)T * (HD * 2);
  const __amdgpu_buffer_rsrc_t k_src = buffer_rsrc(k + (size_t)bh * T * HD, act_b);
  const __amdgpu_buffer_rsrc_t v_src = buffer_rsrc(v + (size_t)bh * T * HD, act_b);
  const __amdgpu_buffer_rsrc_t b_src = buffer_rsrc(beta + (size_t)bh * T, (uint32_t)T * 4);
  char* kpb = (wave < 4 ? l2 : l3) + (wave & 3) * CC_KP_B;
  const int krow = perm32(n);
  const char* pv_op = l1 + lane * 16;                 // + kc * 1024
  const char* s_op = l1 + CC_OPS_B + lane * 16;       // + j * 1024
  float* bslot = reinterpret_cast<float*>(l1 + 2 * CC_OPS_B + wave * 128);

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();                                      // maps and operands are in LDS

  f32x16 uacc[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) uacc[ib] = zero16();
  const int n_all = (T + CC_SLICE - 1) / CC_SLICE;
  const int s_begin = (part * n_all + n_parts - 1) / n_parts;
  const int n_slices = ((part + 1) * n_all + n_parts - 1) / n_parts;   // end of the range
  // Operands of slice sl: lane n holds token 32 sl + perm32(n) of K and V,
  // lane n < 32 the beta of token 32 sl + n, each a load of its own (rows past
  // T read as zeros; a slice past the last reads zeros only). The next slice's
  // are loaded while the current one computes; beta passes through the wave's
  // LDS slot, from which lane (c, h2) reads those of tokens 32 sl + 16 h2 + r.
  bf16x8 kop[8], vop[8];
  float bnext;
  auto load_slice = [&](int sl) __attribute__((always_inline)) {
    bnext = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                          b_src, (sl * CC_SLICE + n) * 4, 0, 0));
    const int roff = (sl * CC_SLICE + krow) * (HD * 2) + 16 * h2;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      kop[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               k_src, roff + 32 * kc, 0, 0));
      vop[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                               v_src, roff + 32 * kc, 0, 0));
    }
  };
  load_slice(s_begin + wave);
  for (int sl = s_begin + wave; sl < n_slices; sl += CC_WAVES) {
    if (h2 == 0) bslot[n] = bnext;
    // K~^T: kt[b][r] = K~[token][32 b + 8 (r / 4) + 4 h2 + r % 4]
    f32x16 kt[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      kt[b] = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        kt[b] = mfma32(tr_op(l0, 16 * kc, 8, 32 * b, lane), kop[kc], kt[b]);
    }
    // V'[:, cols]: vp[r] = V'[token 16 h2 + r][col]
    f32x16 vp = zero16();
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      vp = mfma32(vop[kc], *reinterpret_cast<const bf16x8*>(pv_op + kc * 1024), vp);
    load_slice(sl + CC_WAVES);

    float ss = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) ss = fmaf(kt[b][r], kt[b][r], ss);
    ss = halves_sum(ss);
    const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
    bf16x8 kp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u) kp[j][u] = (__bf16)(kt[j >> 1][8 * (j & 1) + u] * inv);

    // K' rows into this wave's buffer (row = token within the slice, swz_v)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const bf16x4 w4 = {kp[2 * b + (jj >> 1)][4 * (jj & 1)],
                           kp[2 * b + (jj >> 1)][4 * (jj & 1) + 1],
                           kp[2 * b + (jj >> 1)][4 * (jj & 1) + 2],
                           kp[2 * b + (jj >> 1)][4 * (jj & 1) + 3]};
        *reinterpret_cast<bf16x4*>(kpb + krow * 256 + (((4 * b + jj) ^ swz_v(krow)) << 4) +
                                   8 * h2) = w4;
      }
    // P^ = K' S[:, col]: p[r] = P^[token 16 h2 + r][col]
    f32x16 p = zero16();
#pragma unroll
    for (int j = 0; j < 8; ++j)
      p = mfma32(kp[j], *reinterpret_cast<const bf16x8*>(s_op + j * 1024), p);
    // the wave's own LDS writes (beta, K') are done before its reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    f32x4 bq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) bq[i] = *reinterpret_cast<const f32x4*>(bslot + 16 * h2 + 4 * i);
    bf16x8 wb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wb[r >> 3][r & 7] = (__bf16)(bq[r >> 2][r & 3] * (vp[r] - p[r]));
    // U[:, col] += K'^T W (A = K'^T: tokens 8 cc + 16 h2 + u, as W's registers)
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        uacc[ib] = mfma32(tr_op(kpb, 8 * cc, 16, 32 * ib, lane), wb[cc], uacc[ib]);
    // the next slice's K' writes follow this slice's reads in LDS order
  }

  // Sum of the eight per-wave U blocks, in wave order, through LDS:
  // red_w[d][c] (fp32, 32 columns per row), uacc[ib][r] = U[32 ib + 8 (r / 4) +
  // 4 h2 + r % 4][col]
  __syncthreads();                                      // every wave is done with l0-l3
  {
    char* arr = wave < 2 ? l0 : wave < 4 ? l1 : wave < 6 ? l2 : l3;
    float* red = reinterpret_cast<float*>(arr + (wave & 1) * CC_RED_B);
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        red[(32 * ib + 8 * (r >> 2) + 4 * h2 + (r & 3)) * 32 + n] = uacc[ib][r];
  }
  __syncthreads();
  float sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = tid + 512 * i;                        // (d, c) = (e / 32, e % 32)
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < CC_WAVES; ++w) {
      const char* arr = w < 2 ? l0 : w < 4 ? l1 : w < 6 ? l2 : l3;
      const float x = reinterpret_cast<const float*>(arr + (w & 1) * CC_RED_B)[e];
      acc = w == 0 ? x : acc + x;
    }
    sv[i] = acc;
  }
  if (pair) {
    float* cslots = pair->slots + (size_t)cblk * n_parts * 4096;
    const __amdgpu_buffer_rsrc_t mine = buffer_rsrc(cslots + (size_t)part * 4096, 4096 * 4);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, sv[i]), mine,
                                            (tid + 512 * i) * 4, 0, kScopeDevice);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      *flag = (n_parts == 2 ? pair_arrive(pair->ctr + cblk, pair->tag)
                            : commit_arrive(pair->ctr + cblk, pair->tag, n_parts))
                  ? 1
                  : 0;
    __syncthreads();
    if (*flag == 0) return;
    switch (n_parts) {
      case 2: commit_merge<2>(sv, cslots, part, tid); break;
      case 3: commit_merge<3>(sv, cslots, part, tid); break;
      case 4: commit_merge<4>(sv, cslots, part, tid); break;
      case 5: commit_merge<5>(sv, cslots, part, tid); break;
      case 6: commit_merge<6>(sv, cslots, part, tid); break;
      case 7: commit_merge<7>(sv, cslots, part, tid); break;
      default: commit_merge<8>(sv, cslots, part, tid); break;
    }
  }
  const float a = alpha[bh];
  float* Sn = S_next + (size_t)bh * HD * HD;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = tid + 512 * i;
    const size_t g = (size_t)(e >> 5) * HD + 32 * cb + (e & 31);
    sv[i] = fmaf(a, Sp[g], sv[i]);
    Sn[g] = sv[i];
  }
  if (!mt_next) return;
  // The next frame's map for these columns, as read_prep_k forms it: the block
  // S_N[:, cols] goes through LDS transposed (bf16) as the B operand of
  // M = Phi_q S_N; wave ib < 4 computes rows [32 ib, 32 ib + 32) of M.
  __syncthreads();                                      // every U sum is read
  __bf16* st = reinterpret_cast<__bf16*>(l0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = tid + 512 * i;
    st[(e & 31) * CC_ST_LD + (e >> 5)] = (__bf16)sv[i];
  }
  __syncthreads();
  if (wave >= 4) return;
  const __bf16* P = phi_q + (size_t)h * HD * HD + (size_t)(32 * wave + n) * HD + 8 * h2;
  f32x16 acc = zero16();
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    acc = mfma32(ld8(P + 16 * kc),
                 *reinterpret_cast<const bf16x8*>(st + n * CC_ST_LD + 16 * kc + 8 * h2), acc);
  // acc[r] = M[i = 32 wave + 8 (r / 4) + 4 h2 + r % 4][j = col]  ->  M^T[j][i]
  __bf16* out = mt_next + (size_t)bh * HD * HD + (size_t)col * HD + 32 * wave + 4 * h2;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    bf16x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (__bf16)acc[4 * jj + i];
    *reinterpret_cast<bf16x4*>(out + 8 * jj) = w;
  }
}

__global__ void __launch_bounds__(512, 1)
commit_col_k(const __bf16* __restrict__ k, const __bf16* __restrict__ v,
             const __bf16* __restrict__ phi_k, const __bf16* __restrict__ phi_v,
             const __bf16* __restrict__ phi_q, const float* __restrict__ beta,
             const float* __restrict__ alpha, const float* __restrict__ S_prev,
             float* __restrict__ S_next, __bf16* __restrict__ mt_next, int H, int T,
             CommitPair pair) {
  __shared__ __attribute__((aligned(1024))) char l0[AKV];
  __shared__ __attribute__((aligned(1024))) char l1[AKV];
  __shared__ __attribute__((aligned(1024))) char l2[AKV];
  __shared__ __attribute__((aligned(1024))) char l3[AKV];
  __shared__ int flag;
  commit_col_block(xcd_remap(blockIdx.x, gridDim.x), k, v, phi_k, phi_v, phi_q, beta, alpha,
                   S_prev, S_next, mt_next, H, T, l0, l1, l2, l3, &pair, &flag);
}

// The clean pass of the prepared read in one launch: blocks [0, n_attn) are
// the fused read's workgroups (dispatched first, they take their compute units
// first), the next n_commit blocks (from n_attn_pad) the column-split commit's
// eight workgroups per (b, h) (four column blocks x two token halves), which
// run on the compute units the read leaves idle, reuse its LDS arrays, and
// also write the next frame's map when mt_next is given; then n_warm blocks of the attention's L2 warm-up role
// (short-lived, on whatever compute units remain). n_attn_pad and
// n_commit_pad are multiples of 8, so each role's blocks are dealt
// round-robin over the XCDs from XCD 0.
__global__ void __launch_bounds__(512, 1)
clean_fused_k(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
              const __bf16* __restrict__ v, __bf16* __restrict__ o, int T, float sl2,
              int n_qblk, const __bf16* __restrict__ mt, __bf16* __restrict__ o_intra,
              __bf16* __restrict__ o_inter, int n_attn, int n_attn_pad, int n_commit,
              int n_commit_pad, int n_warm, const __bf16* __restrict__ phi_k,
              const __bf16* __restrict__ phi_v, const __bf16* __restrict__ phi_q,
              const float* __restrict__ beta, const float* __restrict__ alpha,
              const float* __restrict__ S_prev, float* __restrict__ S_next,
              __bf16* __restrict__ mt_next, int H, CommitPair pair) {
  __shared__ __attribute__((aligned(1024))) char lk0[AKV];
  __shared__ __attribute__((aligned(1024))) char lk1[AKV];
  __shared__ __attribute__((aligned(1024))) char lv0[AKV];
  __shared__ __attribute__((aligned(1024))) char lv1[AKV];
  __shared__ float mlx[8][2][64];
  __shared__ int redo_flag;
  __shared__ int flag;
  const int b = blockIdx.x;
  if (b < n_attn_pad) {
    if (b < n_attn)
      attn_block<true>(xcd_remap(b, n_attn), q, k, v, o, T, T, T, sl2, n_qblk, mt, o_intra,
                       o_inter, lk0, lk1, lv0, lv1, mlx, redo_flag);
  } else if (b < n_attn_pad + n_commit_pad) {
    const int c = b - n_attn_pad;
    if (c < n_commit)
      commit_col_block(xcd_remap(c, n_commit), k, v, phi_k, phi_v, phi_q, beta, alpha, S_prev,
                       S_next, mt_next, H, T, lk0, lk1, lv0, lv1, &pair, &flag);
  } else {
    attn_l2_warm(b - n_attn_pad - n_commit_pad, n_warm / 8, n_attn, n_qblk, k, v, T, T, lk0);
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
  // chunks in order; the loads of 8 chunks are issued before their sums
  for (int c0 = 1; c0 < n_chunks; c0 += 8) {
    float4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < n_chunks) x[u] = P[(size_t)(c0 + u) * stride4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < n_chunks) {
        acc.x += x[u].x; acc.y += x[u].y; acc.z += x[u].z; acc.w += x[u].w;
      }
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

// Grid of the attention: its workgroups, then (when they leave compute units
// idle, and the heads' K and V are short enough to stay in L2 until used: up to
// kWarmMaxKeys keys) up to 8 L2 warm-up workgroups per XCD.
constexpr long kWarmMaxKeys = 4096;
static void attn_grid(long n_attn, long n_kv, long* n_pad, long* total) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 0;
  *n_pad = (n_attn + 7) / 8 * 8;
  const long per_xcd =
      n_kv <= kWarmMaxKeys ? std::min<long>(8, std::max<long>(0, n_cu - *n_pad) / 8) : 0;
  *total = per_xcd > 0 ? *n_pad + 8 * per_xcd : n_attn;
}

hipError_t mfma_attention(const Dims& d, const void* q, const void* k, const void* v, void* o,
                          int64_t n_kv, int64_t kv_cap, hipStream_t s) {
  const int n_qblk = (d.T + AQ - 1) / AQ;
  const long nblk = (long)d.B * d.H * n_qblk;
  long n_pad, total;
  attn_grid(nblk, n_kv, &n_pad, &total);
  attn_mfma_k<false><<<(unsigned)total, 512, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), d.T, (int)n_kv, (long)kv_cap, d.scale * kLog2e, n_qblk, nullptr,
      nullptr, nullptr, (int)nblk, (int)n_pad);
  return hipGetLastError();
}

// Split-key fused read (attn_sk_k): used when the plain grid (one workgroup
// per 128 queries of a head) leaves compute units idle and the longest split
// workgroup is estimated to finish at least 10% before a whole query block
// does. Measured on MI355X: a segment boundary costs about 12 key tiles, so
// the split pays off for long frames with few heads (4 x 4096 tokens: 60 ->
// 45 us; 1 x 16384: 233 -> 134 us) and where the plain grid's last round is
// mostly idle (40 heads x 1560: 83 -> 76 us; 12 heads x 3600: 116 -> 102 us),
// and not at 12 heads x 1560 tokens (25 tiles per block) nor with the chip
// full.
constexpr int kSkMaxGrid = 256;
constexpr int kSkPad = 2;
constexpr int kSkBoundaryTiles = 12;
struct SkPlan {
  bool use;
  int G, pad;
};
static SkPlan sk_plan(const Dims& d, int n_cu) {
  SkPlan p{false, 0, kSkPad};
  const int n_tiles = (d.T + AKT - 1) / AKT;
  const long n_blk = (long)d.B * d.H * ((d.T + AQ - 1) / AQ);
  const int G = std::min(n_cu, kSkMaxGrid);
  if (G <= 0 || n_tiles < 4) return p;
  const long L = n_tiles + p.pad, V = n_blk * L;
  // each workgroup's range covers at least half a block, so a block meets at
  // most three workgroups (the merge reads at most two other segments at once)
  if (V < G || V / G < (L + 1) / 2) return p;
  // key tiles on the longest workgroup's path: one whole block per round of
  // the plain grid (one workgroup per compute unit at a time); on the split
  // grid its range plus the cost of its segment boundaries (publishing a
  // partial, the counter, the merge: about kSkBoundaryTiles)
  const long plain = (n_blk + G - 1) / G * n_tiles;
  p.use = 10 * ((V + G - 1) / G + kSkBoundaryTiles) < 9 * plain;
  p.G = G;
  return p;
}
static long sk_ctr_bytes(const Dims& d) {
  return (long)round_up((size_t)d.B * d.H * ((d.T + AQ - 1) / AQ) * 8, 256);
}

size_t mfma_read_prepared_ws_bytes(const Dims& d) {
  if (!sk_plan(d, kSkMaxGrid).use) return 0;
  return (size_t)sk_ctr_bytes(d) + (size_t)2 * kSkMaxGrid * kSkSlotFloats * sizeof(float);
}

hipError_t mfma_attention_lse(const Dims& d, const void* q, const void* k, const void* v,
                              void* o, float* lse, hipStream_t s) {
  const int n_qblk = (d.T + AQ - 1) / AQ;
  const long nblk = (long)d.B * d.H * n_qblk;
  long n_pad, total;
  attn_grid(nblk, d.T, &n_pad, &total);
  attn_mfma_k<false, true><<<(unsigned)total, 512, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), d.T, d.T, (long)d.T, d.scale * kLog2e, n_qblk, nullptr, nullptr,
      nullptr, (int)nblk, (int)n_pad, lse);
  return hipGetLastError();
}

size_t mfma_read_ws_bytes(const Dims& d) {
  return round_up((size_t)d.B * d.H * HD * HD * 2, 256) + mfma_read_prepared_ws_bytes(d);
}

// Per-call tags of the split read's block counters (48 bits, never 0).
static std::atomic<unsigned long long> g_sk_tag{0};

hipError_t mfma_read_prepare(const Dims& d, const void* phi_q, const float* S, void* mt,
                             hipStream_t s) {
  read_prep_k<<<(unsigned)(d.B * d.H * 4), 256, 0, s>>>(static_cast<const __bf16*>(phi_q), S,
                                                       static_cast<__bf16*>(mt), d.H);
  return hipGetLastError();
}

hipError_t mfma_read_prepared(const Dims& d, const void* q, const void* k, const void* v,
                              const void* mt, void* o, void* o_intra, void* o_inter, void* ws,
                              size_t ws_bytes, hipStream_t s) {
  const int n_qblk = (d.T + AQ - 1) / AQ;
  const long nblk = (long)d.B * d.H * n_qblk;
  const size_t sk_need = mfma_read_prepared_ws_bytes(d);
  if (ws && sk_need > 0 && ws_bytes >= sk_need) {
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n_cu = 0;
    const SkPlan p = sk_plan(d, n_cu);
    if (p.use) {
      unsigned long long tag = 0;
      while (tag == 0) tag = (++g_sk_tag) & 0xFFFFFFFFFFFFull;
      char* w = static_cast<char*>(ws);
      attn_sk_k<true><<<(unsigned)p.G, 512, 0, s>>>(
          static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
          static_cast<const __bf16*>(v), static_cast<__bf16*>(o), d.T, d.scale * kLog2e, n_qblk,
          static_cast<const __bf16*>(mt), static_cast<__bf16*>(o_intra),
          static_cast<__bf16*>(o_inter), (int)nblk, p.pad,
          reinterpret_cast<float*>(w + sk_ctr_bytes(d)),
          reinterpret_cast<unsigned long long*>(w), tag << 16);
      return hipGetLastError();
    }
  }
  long n_pad, total;
  attn_grid(nblk, d.T, &n_pad, &total);
  attn_mfma_k<true><<<(unsigned)total, 512, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), d.T, d.T, (long)d.T, d.scale * kLog2e, n_qblk,
      static_cast<const __bf16*>(mt), static_cast<__bf16*>(o_intra),
      static_cast<__bf16*>(o_inter), (int)nblk, (int)n_pad);
  return hipGetLastError();
}

// The commit's token-split workspace: n_parts slots per column block, then one
// counter per column block; each call gets its own tag.
static CommitPair commit_pair(const Dims& d, void* ws, int n_parts) {
  static std::atomic<unsigned long long> g_commit_tag{0};
  const size_t n_cb = (size_t)4 * d.B * d.H;
  char* w = static_cast<char*>(ws);
  unsigned long long tag = 0;
  while (tag == 0) tag = (++g_commit_tag) & 0xFFFFFFFFFFFFull;
  return CommitPair{reinterpret_cast<float*>(w),
                    reinterpret_cast<unsigned long long*>(w + n_cb * n_parts * 4096 * sizeof(float)),
                    tag << 16, n_parts};
}

hipError_t mfma_clean_pass_prepared(const Dims& d, const void* q, const void* k, const void* v,
                                    const void* mt, const void* phi_q, const void* phi_k,
                                    const void* phi_v, const float* beta, const float* alpha,
                                    const float* S_prev, float* S_next, void* mt_next, void* o,
                                    void* o_intra, void* o_inter, void* ws, hipStream_t s) {
  const long n_bh = (long)d.B * d.H;
  const int n_qblk = (d.T + AQ - 1) / AQ;
  const long n_attn = n_bh * n_qblk;
  const long n_pad = (n_attn + 7) / 8 * 8;
  const long n_commit = 8 * n_bh, n_commit_pad = (n_commit + 7) / 8 * 8;
  // the L2 warm-up role on the compute units that the read and the commit
  // leave idle (up to 8 per XCD), for frames short enough to stay in L2
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    n_cu = 0;
  const long n_warm =
      d.T <= kWarmMaxKeys ? 8 * std::min<long>(8, std::max<long>(0, n_cu - n_pad - n_commit_pad) / 8)
                          : 0;
  clean_fused_k<<<(unsigned)(n_pad + n_commit_pad + n_warm), 512, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<__bf16*>(o), d.T, d.scale * kLog2e, n_qblk, static_cast<const __bf16*>(mt),
      static_cast<__bf16*>(o_intra), static_cast<__bf16*>(o_inter), (int)n_attn, (int)n_pad,
      (int)n_commit, (int)n_commit_pad, (int)n_warm, static_cast<const __bf16*>(phi_k),
      static_cast<const __bf16*>(phi_v), static_cast<const __bf16*>(phi_q), beta, alpha, S_prev,
      S_next, static_cast<__bf16*>(mt_next), d.H, commit_pair(d, ws, 2));
  return hipGetLastError();
}

hipError_t mfma_read(const Dims& d, const void* q, const void* k, const void* v,
                     const void* phi_q, const float* S, void* o, void* o_intra, void* o_inter,
                     void* ws, hipStream_t s) {
  hipError_t e = mfma_read_prepare(d, phi_q, S, ws, s);
  if (e != hipSuccess) return e;
  const size_t mb = round_up((size_t)d.B * d.H * HD * HD * 2, 256);
  return mfma_read_prepared(d, q, k, v, ws, o, o_intra, o_inter, static_cast<char*>(ws) + mb,
                            mfma_read_prepared_ws_bytes(d), s);
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

hipError_t mfma_feature_maps(const Dims& d, const FeatureMapJob* jobs, int n_jobs, hipStream_t s) {
  if (n_jobs < 1 || n_jobs > 3) return hipErrorInvalidValue;
  for (int j = 1; j < n_jobs; ++j)
    if (jobs[j].norms) return hipErrorInvalidValue;
  if (jobs[0].norms && !jobs[0].normalize) return hipErrorInvalidValue;
  if (n_jobs == 1 && !jobs[0].norms)
    return mfma_feature_map(d, jobs[0].x, jobs[0].phi, jobs[0].out, jobs[0].normalize, s);
  const int n_rblk = (d.T + MAP_ROWS - 1) / MAP_ROWS;
  const long nblk = (long)d.B * d.H * n_rblk;
  const FeatureMapJob& j1 = jobs[1];
  const FeatureMapJob& j2 = jobs[n_jobs > 2 ? 2 : 1];
  const MapMore more{static_cast<const __bf16*>(j1.x), j1.phi, static_cast<__bf16*>(j1.out),
                     j1.normalize ? 1 : 0, static_cast<const __bf16*>(j2.x), j2.phi,
                     static_cast<__bf16*>(j2.out), j2.normalize ? 1 : 0};
  rowmap_mfma_k<MAP_PHI><<<(unsigned)(nblk * n_jobs), 256, 0, s>>>(
      static_cast<const __bf16*>(jobs[0].x), jobs[0].phi, nullptr,
      static_cast<__bf16*>(jobs[0].out), nullptr, d.H, d.T, n_rblk, jobs[0].normalize ? 1 : 0,
      more, (int)nblk, jobs[0].norms);
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

// Token parts of the commit alone: at most as many as fill 256 compute units
// with the 4 B H column blocks (at least two, at most eight), each part at
// least eight 32-token slices (one per wave) when the frame has them; then the
// fewest parts that give each wave the same number of slices (fewer sums to
// publish and merge for the same time).
static int commit_parts(const Dims& d) {
  const long n_cb = 4L * d.B * d.H;
  const int n_all = (d.T + CC_SLICE - 1) / CC_SLICE;
  long p = std::min<long>(256 / n_cb, n_all / CC_WAVES);
  p = std::max<long>(2, std::min<long>(8, p));
  auto rounds = [&](long q) { return ((n_all + q - 1) / q + CC_WAVES - 1) / CC_WAVES; };
  const long r = rounds(p);
  while (p > 2 && rounds(p - 1) == r) --p;
  return (int)p;
}

size_t mfma_commit_ws_bytes(const Dims& d) {
  const size_t n_cb = (size_t)4 * d.B * d.H;
  return n_cb * commit_parts(d) * 4096 * sizeof(float) + round_up(n_cb * 8, 256);
}

size_t mfma_clean_commit_ws_bytes(const Dims& d) {
  const size_t n_cb = (size_t)4 * d.B * d.H;
  return n_cb * 2 * 4096 * sizeof(float) + round_up(n_cb * 8, 256);
}

hipError_t mfma_commit(const Dims& d, const void* k, const void* v, const void* phi_k,
                       const void* phi_v, const float* beta, const float* alpha,
                       const float* S_prev, float* S_next, void* ws, hipStream_t s) {
  const int n_parts = commit_parts(d);
  commit_col_k<<<(unsigned)(4L * n_parts * d.B * d.H), 512, 0, s>>>(
      static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<const __bf16*>(phi_k), static_cast<const __bf16*>(phi_v), nullptr, beta, alpha,
      S_prev, S_next, nullptr, d.H, d.T, commit_pair(d, ws, n_parts));
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
