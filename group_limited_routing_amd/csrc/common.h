// Shared device helpers for the gfx950 kernels of the Beam MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace beam {

constexpr int kWave = 64;
constexpr int kExperts = 256;   // the block is built for Beam's 256 experts
constexpr int kChunk = 256;     // tokens per permutation chunk (one workgroup)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(8 * sizeof(int32_t)))) int32_t i32x8;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits with the gfx950 conversion instruction: round to nearest
// even, NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values -> packed bf16 pair (lo in the low half), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16x16x32 bf16 MFMA, fp32 accumulate. Operand layout (per lane l of 64):
// A: row l%16, eight k values; B: column l%16, eight k values; the products
// pair element i of A's lane group l/16 with element i of B's lane group l/16.
// C: column l%16, rows 4*(l/16) + 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x4 fp32 MFMA: A row l%16 / B column l%16, k slot l/16; C as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16x128 fp8 (OCP E4M3 on both operands) MFMA, fp32 accumulate. Each
// lane holds 32 one-byte values of its row (A) or column (B); the E8M0 block
// scales are 0x7F = 2^0, so this is the unscaled product.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

// 16x16x128 MFMA with an E4M3 first operand (unit scale) and an OCP MXFP4
// second operand: lane l holds 32 E2M1 codes (16 bytes, two per byte, low
// nibble first, in the first four registers of b) of column l % 16 and
// reduction elements 32 (l / 16) .. + 31, and bscale (low byte) is the E8M0
// scale of exactly those 32 elements.
__device__ __forceinline__ f32x4 mfma_fp8_fp4(i32x8 a, i32x8 b, int bscale, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 0x7f7f7f7f, 0, bscale);
}

// The same instruction with the operands the other way round: the MXFP4
// weights (with their per-lane E8M0 scales) as the first operand, E4M3 as
// the second, so the output holds weight rows along its row dimension.
__device__ __forceinline__ f32x4 mfma_fp4_fp8(i32x8 a, i32x8 b, int ascale, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, ascale, 0, 0x7f7f7f7f);
}

// fp32 -> OCP E4M3 code, round to nearest even, finite overflow saturates to
// +-448, NaN -> 0x7F. Written from the format: bias 7, 3 mantissa bits,
// subnormal spacing 2^-9, no infinity, largest finite 1.75 * 2^8.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448 (and +-inf): saturate
  if (a < 0x3c800000u) {                       // below 2^-6: multiples of 2^-9
    const float q = rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
    return sign | (uint32_t)q;                  // q == 8 is the code of 2^-6
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);   // RNE to 3 mantissa bits
  const uint32_t e = (r >> 23) - 120u;                   // rebias 127 -> 7
  const uint32_t code = (e << 3) | ((r >> 20) & 7u);
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes lds_base + 16 l (lds_base must be the same for the whole wave).
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(gsrc, lds_base, 16, 0, 0);
#endif
}

// The same with the non-temporal cache policy (the NT bit): for weights
// that each workgroup streams once, so they do not displace reused lines.
__device__ __forceinline__ void dma16_nt(const void* gsrc, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(gsrc, lds_base, 16, 0, 2);
#endif
}

// 16 bytes from global memory with the non-temporal hint (streamed weights).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Wait until at most N vector-memory operations of this wave are pending
// (gfx9 s_waitcnt encoding: vmcnt bits [3:0] and [15:14]; expcnt and
// lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
#endif
}

// Wait until all LDS/scalar-memory operations of this wave have completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0xc07f);
#endif
}

// Workgroup barrier without the memory fence of __syncthreads (the fence
// would wait for every pending global->LDS load, not just the needed ones).
__device__ __forceinline__ void barrier_only() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_barrier();
#endif
}

__device__ __forceinline__ float sigmoid_f32(float z) {
  return 1.0f / (1.0f + expf(-z));
}

// silu(v) = v * sigmoid(v) in fp32 with the hardware base-2 exponential and
// reciprocal (about one ulp each); the tails give v and -0 as they should.
__device__ __forceinline__ float silu_f32(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

}  // namespace beam
