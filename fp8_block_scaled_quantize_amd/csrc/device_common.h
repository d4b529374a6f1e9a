// Device helpers shared by the quantizer and GEMM kernels (gfx950 only).
//
// E4M3 encoding, bf16 unpacking, the per-group scale and the per-element
// quotient. The numeric rule is the one the C ABI documents: s = fl32(amax/448)
// (1.0 for an all-zero group), q = E4M3_RNE(fl32(x / s)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bsq {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------- E4M3 --
// Every quotient the quantizers produce has |q| < 449 (a bf16 amax over its
// correctly rounded fp32 scale amax/448; the ratio only leaves
// [447.99997, 448.00003] when the scale is subnormal), and nearest-even
// rounding sends everything in [448, 464) to 448. Clamping to +-448 first
// therefore never changes the result; it only keeps the hardware converter
// out of its overflow range. med3 keeps the sign of zero.
__device__ __forceinline__ float clamp448(float q) {
  return __builtin_amdgcn_fmed3f(q, 448.0f, -448.0f);
}

// Four fp32 values -> four E4M3 bytes (value a in the lowest byte).
// v_cvt_pk_fp8_f32 on gfx950 converts to OCP E4M3 with round-to-nearest-even.
// This form clamps first and takes any |v| <= 464.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), v, true);
  return (uint32_t)v;
}

// The same for quotients, which always have |q| < 449: on gfx950 the
// converter gives, for every fp32 v with |v| < 449 (both signs, checked
// exhaustively on the GPU), the byte it gives for clamp448(v), so the clamp
// (two VALU operations per element) is left out.
__device__ __forceinline__ uint32_t e4m3x4_q(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// ------------------------------------------------------- group division --
// Per-group constants. The element quotient is computed as one correctly
// rounded fp32 division would give it, without a division per element:
//   r = fl32(1/sc), q0 = fl32(x*r), d = fma(q0, sc, -x), q = fma(-d, r, q0)
// (Markstein's correction step with a correctly rounded reciprocal; d is the
// exact residual with its sign flipped, which keeps q = -0 for x = -0, as the
// division gives). When the group's amax is below 2^-64 the scale may be
// subnormal and 1/s overflow, so both x and s are multiplied by 2^64 first
// (exact, same real quotient). The equivalence to IEEE x/s, down to the sign
// of zero, was checked exhaustively over every pair of bf16 values with
// |x| <= amax.
struct GroupDiv {
  float sc;     // scale used in the residual (s, or s * 2^64)
  float r;      // fl32(1 / sc)
  float xmul;   // 1 or 2^64, applied to x
};

__device__ __forceinline__ float group_scale(float amax) {
  // IEEE division; the library is built with correctly rounded fp32 divide.
  return amax == 0.0f ? 1.0f : amax / 448.0f;
}

__device__ __forceinline__ GroupDiv group_div(float amax, float s) {
  GroupDiv g;
  const bool tiny = amax < 0x1p-64f;
  g.xmul = tiny ? 0x1p64f : 1.0f;
  g.sc = s * g.xmul;
  g.r = 1.0f / g.sc;
  return g;
}

// True on every lane when some lane of the wavefront holds a tiny group
// (xmul != 1): the pre-scaling multiply runs only then, so the branch is
// uniform and the common case skips it (x * 1 is x, so either way the
// quotient is the same).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float quotient(float x, float sc, float r) {
  const float q0 = x * r;
  const float d = __builtin_fmaf(q0, sc, -x);
  return __builtin_fmaf(-d, r, q0);
}

// ------------------------------------------------------------ DPP max --
// Cross-lane max within aligned lane groups using DPP moves.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;     // reverse within each 8-lane half row
constexpr int DPP_ROW_MIRROR = 0x140;      // reverse within each 16-lane row

// Max over each aligned group of 8 lanes (all 8 lanes get the result).
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  return v;
}

// Max over each aligned group of 16 lanes.
__device__ __forceinline__ float max16(float v) {
  v = max8(v);
  return fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
}

// Max over the whole 64-lane wavefront.
__device__ __forceinline__ float max64(float v) {
  v = max16(v);
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Asynchronous global -> LDS copies ("LDS DMA"): every lane of the wavefront
// sends SIZE bytes from (sbase + voff) to LDS byte address lds + SIZE * lane.
// sbase and lds are wavefront-uniform (SGPR pair / M0), voff is a per-lane
// 32-bit offset. Written as inline assembly so the compiler neither keeps
// 64-bit per-lane pointers live nor inserts waits for these copies before
// unrelated LDS reads; the kernel waits for them itself (a vmcnt wait before
// each barrier). The s_nop is the wait state a copy needs after M0 is written.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint64_t uniform_ptr(const void* ptr) {
  const uint64_t v = (uint64_t)(uintptr_t)ptr;
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
}
// LDS byte address of a __shared__ object (wavefront-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(lds_void*)lds);
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds), "v"(voff), "s"(uniform_ptr(sbase)) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds), "v"(voff), "s"(uniform_ptr(sbase)) : "memory", "m0");
}
// Wait until at most N vector-memory operations of this wavefront are in
// flight (they complete in order), leaving LDS and export counters alone.
template <int N>
__device__ __forceinline__ void wait_dma_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace fp8bsq
