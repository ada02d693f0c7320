// Characterization probes of the MFMA arithmetic the routed down relies on
// (test infrastructure, not part of the library): one 16x16 tile, one wave.
//
// qmoe_probe_dot128: D[m][n] of a 16 x 128 (E4M3 codes, A) times 128 x 16
// (B given as bf16-exact values: E2M1 codes here) product, computed
//   (1) by the scaled FP8 x FP4 MFMA v_mfma_scale_f32_16x16x128_f8f6f4
//       (unit scales), and
//   (2) by four bf16 MFMAs v_mfma_f32_16x16x32_bf16 on the operands widened
//       to bf16 (exact),
// with the same values. The probes are built so that B is the same in every
// K position of a column, so neither result depends on how the MFMA spreads
// K over lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));

__global__ void probe_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ bq, float* __restrict__ d8,
                             float* __restrict__ d16) {
  const int l = threadIdx.x, r = l & 15, g = l >> 4;
  // (1) A: lane l holds row r, bytes 32 g .. 32 g + 31 of its 128 (a K
  // permutation the hardware fixes; B is constant along K, so it does not
  // matter); B: lane l holds column r, 32 E2M1 codes (16 bytes)
  v8i A, B;
  const uint32_t* pa = reinterpret_cast<const uint32_t*>(a + r * 128 + 32 * g);
  const uint32_t* pb = reinterpret_cast<const uint32_t*>(bq + r * 64 + 16 * g);
  for (int i = 0; i < 8; ++i) A[i] = (int)pa[i];
  for (int i = 0; i < 4; ++i) B[i] = (int)pb[i];
  for (int i = 4; i < 8; ++i) B[i] = 0;
  v4f D = {0.f, 0.f, 0.f, 0.f};
  D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, D, 0, 4, 0, 127, 0, 127);
  for (int i = 0; i < 4; ++i) d8[(4 * g + i) * 16 + r] = D[i];
  // (2) the same values widened to bf16, four K-steps of 32
  v4f E = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < 4; ++q) {
    v8s fa, fb;
    for (int e = 0; e < 8; ++e) {
      const int k = 32 * q + 8 * g + e;
      const uint32_t ca = a[r * 128 + k];
      const uint32_t nib = (bq[r * 64 + k / 2] >> (4 * (k & 1))) & 15u;
      const __bf16 va = (__bf16)(float)__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(ca, 1.0f, false)[0];
      const __bf16 vb = (__bf16)(float)__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(nib, 1.0f, 0)[0];
      fa[e] = __builtin_bit_cast(short, va);
      fb[e] = __builtin_bit_cast(short, vb);
    }
    E = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, E, 0, 0, 0);
  }
  for (int i = 0; i < 4; ++i) d16[(4 * g + i) * 16 + r] = E[i];
}

extern "C" int qmoe_probe_dot128(const void* a, const void* b, void* d8, void* d16, void* stream) {
  hipLaunchKernelGGL(probe_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a, (const uint8_t*)b,
                     (float*)d8, (float*)d16);
  return (int)hipGetLastError();
}
