// Device helpers shared by the routed-MoE kernels (gfx950, wave64).
//
// Format encoders are written from the public definitions: OCP Microscaling
// v1.0 (E2M1 elements, E8M0 scales, scale exponent floor(log2 amax) - 2) and
// the OCP 8-bit float spec (E4M3FN: bias 7, max 448, no infinities).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- memory
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }

// Workgroup barrier that orders LDS only: the fences are limited to the
// local address space, so the barrier does not wait for the wave's global
// loads still in flight (a plain __syncthreads() waits for all of them).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ----------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

// Maximum / minimum over the wave of a 32-bit value, uniform result. Each
// 16-lane row reduces with DPP (quad permutes, half-row and row mirrors),
// then the four row results are read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Order-preserving unsigned key of a float (-0 counts as +0; NaN unsupported).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ----------------------------------------------------------------- E2M1 / MX
// E2M1 codes of a (bits 0-3) and b (bits 4-7): the nearest E2M1 value
// (0, .5, 1, 1.5, 2, 3, 4, 6), ties to the even code, 6 above 6, the sign
// kept (also on zero), by the hardware conversion v_cvt_scalef32_pk_fp4_f32
// with a unit scale. Every caller converts scaled elements v * 2^-X of a
// block with X = floor(log2 amax) - 2, which lie below 8 in magnitude; over
// every fp32 of magnitude below 8, of either sign, the instruction returns
// exactly that code (tests/test_gpu_mfma_probe.py compares it with a
// reference encoder on all of them).
__device__ __forceinline__ uint32_t e2m1_pack2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// E8M0 scale byte of a 32-block from the largest |bf16| bit pattern of the block.
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t amax_bits16) {
  if (amax_bits16 == 0) return 0;
  int ex = (int)(amax_bits16 >> 7);
  int fl;  // floor(log2 amax)
  if (ex == 0) fl = -133 + (31 - __clz(amax_bits16 & 0x7F));
  else fl = ex - 127;
  int c = fl - 2 + 127;
  return (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
}

// E8M0 scale byte of a 32-block from the largest |fp32| bit pattern of the
// block: floor(log2 amax) - 2 + 127, clamped to [0, 254]; 0 for a zero block.
__device__ __forceinline__ uint32_t mx_scale_code_f32(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  const int ex = (int)(amax_bits >> 23);
  const int fl = ex != 0 ? ex - 127 : -149 + (31 - __clz(amax_bits));  // subnormal: mantissa * 2^-149
  const int c = fl - 2 + 127;
  return (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
}

// ----------------------------------------------------------------- E4M3FN
// E4M3 codes of a and b (bytes 0 and 1): the nearest E4M3 value, ties to the
// even code, the sign kept (also on zero), by the hardware conversion
// v_cvt_pk_fp8_f32. Every caller converts quotients v / s with s =
// fl32(amax / 448) and |v| <= amax, which lie below 464 in magnitude; over
// every fp32 of magnitude below 464, of either sign, the instruction returns
// exactly the nearest-even code (tests/test_gpu_mfma_probe.py compares it
// with a reference encoder on all of them). It does not saturate above 464.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// E4M3 value times 2^9 as base-128 digits. Every E4M3 value is an integer
// multiple of 2^-9 (the subnormal step) of magnitude <= 448, so v * 2^9 is an
// integer below 2^18: v * 2^9 = d0 + 2^7 d1 + 2^14 d2 with the value's sign
// on every digit, |d0|, |d1| <= 127, |d2| <= 14. Returns d0, d1, d2 as int8
// in bytes 0, 1, 2. Products of such digits summed by the int8 MFMA are exact
// integers, which makes E4M3 x E4M3 block sums exact.
__device__ __forceinline__ uint32_t e4m3_digits(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t mag = e ? ((8u | m) << (e - 1)) : m;
  uint32_t u0 = mag & 127u, u1 = (mag >> 7) & 127u, u2 = mag >> 14;
  if (c & 0x80u) {
    u0 = (0u - u0) & 255u;
    u1 = (0u - u1) & 255u;
    u2 = (0u - u2) & 255u;
  }
  return u0 | (u1 << 8) | (u2 << 16);
}

// Four E4M3 codes (a dword, first code in the low byte) -> their digit planes:
// byte q of plane p is digit p of code q.
__device__ __forceinline__ void e4m3x4_digits(uint32_t w, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
  p0 = p1 = p2 = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t d = e4m3_digits((w >> (8 * q)) & 255u);
    p0 |= (d & 255u) << (8 * q);
    p1 |= ((d >> 8) & 255u) << (8 * q);
    p2 |= (d >> 16) << (8 * q);
  }
}

// Operand layout of the shared-expert GEMMs ("digit rows"): a row of K E4M3
// values is stored as [K/128][3][128] int8: for each 128-block, digit plane 0,
// then 1, then 2 of its 128 values (e4m3_digits), so a row's block is one
// contiguous 384-byte run.
constexpr int kShDigitBlock = 3 * 128;

// 8 E4M3 codes (lo, hi: first code in the low byte) of elements off..off+7 of
// a 128-block -> their digits at `blk` (the block's 384-byte run).
__device__ __forceinline__ void store_digits8(uint8_t* blk, int off, uint32_t lo, uint32_t hi) {
  uint32_t a0, a1, a2, b0, b1, b2;
  e4m3x4_digits(lo, a0, a1, a2);
  e4m3x4_digits(hi, b0, b1, b2);
  *reinterpret_cast<uint2*>(blk + off) = make_uint2(a0, b0);
  *reinterpret_cast<uint2*>(blk + 128 + off) = make_uint2(a1, b1);
  *reinterpret_cast<uint2*>(blk + 256 + off) = make_uint2(a2, b2);
}

// 2 E4M3 codes (low byte first) of elements off, off+1 -> their digits.
__device__ __forceinline__ void store_digits2(uint8_t* blk, int off, uint32_t c01) {
  uint32_t p0, p1, p2;
  e4m3x4_digits(c01, p0, p1, p2);
  *reinterpret_cast<uint16_t*>(blk + off) = (uint16_t)p0;
  *reinterpret_cast<uint16_t*>(blk + 128 + off) = (uint16_t)p1;
  *reinterpret_cast<uint16_t*>(blk + 256 + off) = (uint16_t)p2;
}

// E4M3 code -> bf16 bits (every E4M3 value is exact in bf16).
__host__ __device__ constexpr uint16_t e4m3_to_bf16_bits(uint32_t c) {
  uint32_t s = (c & 0x80u) << 8;
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if ((c & 0x7Fu) == 0x7Fu) return (uint16_t)(s | 0x7FC0u);  // NaN
  if (e == 0) {
    if (m == 0) return (uint16_t)s;
    // m * 2^-9: normalise the 3-bit mantissa
    int p = m >= 4 ? 2 : (m >= 2 ? 1 : 0);
    uint32_t be = (uint32_t)(p - 9 + 127);
    uint32_t bm = ((m << (7 - p)) & 0x7Fu);
    return (uint16_t)(s | (be << 7) | bm);
  }
  return (uint16_t)(s | ((e - 7u + 127u) << 7) | (m << 4));
}

// ----------------------------------------------------------------- bf16
// Correctly rounded double -> bf16 (nearest, ties to even): truncate to
// binary32, make the result sticky-odd when bits were dropped (round to odd
// keeps enough information: 24 bits > 8 + 2), then round binary32 to bf16.
__device__ __forceinline__ uint32_t bf16_rne_from_double(double v) {
  float f = __double2float_rz(v);
  uint32_t u = __float_as_uint(f);
  if ((double)f != v) u |= 1u;
  u = u + 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ----------------------------------------------------------------- MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1. Lane l holds row
// (A) / column (B) l%16 and the 32 consecutive K elements 32*(l/16).. of that
// row in 16 bytes; its E8M0 scale byte covers exactly those 32 elements.
// D: lane l, element i = D[4*(l/16)+i][l%16].
__device__ __forceinline__ v4f mfma_fp4(uint4 a, uint4 b, v4f c, uint32_t sa, uint32_t sb) {
  v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// v_mfma_i32_16x16x64_i8: lane l holds row (A) / column (B) l%16 and 16
// int8 K elements; A and B take the same K bytes from a lane, so the exact
// int32 dot products do not depend on the order the unit reads them in.
// D: lane l, element i = D[4*(l/16)+i][l%16].
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i mfma_i8(uint4 a, uint4 b, v4i c) {
  const v4i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  const v4i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: lane l holds row/column l%16 and K elements
// 8*(l/16)..+8. Products are exact and the sum is exact whenever it is
// representable in binary32.
__device__ __forceinline__ v4f mfma_bf16(v8s a, v8s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two E2M1 codes (one byte, selected by SEL) -> two bf16 multiplied by scale.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16(uint32_t src, float scale) {
  bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scale, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// Four packed bf16 pairs as the 8-element bf16 MFMA operand.
__device__ __forceinline__ v8s as_v8s(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
  v8s r;
  r[0] = (short)(d0 & 0xFFFF); r[1] = (short)(d0 >> 16);
  r[2] = (short)(d1 & 0xFFFF); r[3] = (short)(d1 >> 16);
  r[4] = (short)(d2 & 0xFFFF); r[5] = (short)(d2 >> 16);
  r[6] = (short)(d3 & 0xFFFF); r[7] = (short)(d3 >> 16);
  return r;
}

// Two E4M3 bytes of w (the low or the high half) widened to bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ float e8m0_to_float(uint32_t s) {
  return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

// SiLU(g) * u in float64, one rounding to binary32.
__device__ __forceinline__ float silu_mul(float g, float u) {
  double gd = (double)g;
  return (float)((gd / (1.0 + exp(-gd))) * (double)u);
}

}  // namespace qmoe
