// Shared device helpers of the bf16 MFMA kernels (gfx950, wave64): vector
// types, the 32x32x16 bf16 MFMA, operand loads, LDS chunk swizzles and the
// transposing LDS read. Included by each kernel translation unit; everything
// here has internal linkage.
//
// MFMA operand layout used throughout (32x32x16, wave64): for C = A * B with
// A [32 x 16] and B [16 x 32], lane l supplies row (l % 32) of A and column
// (l % 32) of B, each as 8 consecutive k-slots starting at 8 * (l / 32); the
// result C [32 x 32] lands as lane l = column (l % 32), register r = row
// 8 * (r / 4) + 4 * (l / 32) + (r % 4). The kernels arrange every contraction
// so that the contracted index is contiguous in memory for both operands, and
// so that an accumulator's register index runs over the index the next
// contraction sums over (softmax P and the commit's residual never leave
// registers).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

// Element e (0..7) of 8 packed bf16 held as uint4.
__device__ __forceinline__ uint32_t elem(const uint4& x, int e) {
  const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  return (e & 1) ? hi16(w) : lo16(w);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz_k(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 2; }
__device__ __forceinline__ int swz_r(int r) { return r & 15; }

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled dwords).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Transposing read of 4 bf16 at a byte address in LDS.
__device__ __forceinline__ bf16x4 tr_read(const char* a) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)a);
  return __builtin_bit_cast(bf16x4, r);
}

// MFMA operand by two transposing reads from a row-major bf16 matrix in LDS
// with 256-byte rows stored under the swz_v chunk swizzle: lane (n = lane % 32,
// h2 = lane / 32) receives M[r0 + hoff*h2 + u][c0 + n] for u = 0..7.
// r0 and hoff must be multiples of 4.
__device__ __forceinline__ bf16x8 tr_op(const char* base, int r0, int hoff, int c0, int lane) {
  const int G = lane >> 4;
  const int s = lane & 15, c = s >> 2, j = s & 3;
  const int col = c0 + 16 * (G & 1) + 4 * j;
  const int c16 = col >> 3, sub = (col & 7) * 2;
  const int rb = r0 + hoff * (G >> 1) + c;
  const char* a0 = base + rb * 256 + ((c16 ^ swz_v(rb)) << 4) + sub;
  const char* a1 = base + (rb + 4) * 256 + ((c16 ^ swz_v(rb + 4)) << 4) + sub;
  return __builtin_shufflevector(tr_read(a0), tr_read(a1), 0, 1, 2, 3, 4, 5, 6, 7);
}

// max / sum of x over lanes l and l ^ 32.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two-party arrival on a per-pair counter in a workspace: false for the first
// of a pair, true for the second, which leaves the counter at 0 again. The
// first leaves this call's tag there (per-call, bit 63 set, so never 0); any
// other content (0 after a completed call, or whatever a fresh workspace holds)
// counts as no arrival, so the workspace needs no clearing between calls. The
// exchange is a device-scope atomic: both parties see one modification order.
__device__ __forceinline__ bool pair_arrive(unsigned long long* ctr, unsigned long long tag) {
  const unsigned long long old =
      __hip_atomic_exchange(ctr, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (old != tag) return false;
  __hip_atomic_store(ctr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

}  // namespace
}  // namespace arl2
