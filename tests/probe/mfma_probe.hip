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
//
// qmoe_probe_e4m3_cvt: the hardware fp32 -> E4M3 conversion the quantizers
// use (v_cvt_pk_fp8_f32) against a reference encoder written from the
// format's definition (qmoe_probe_e4m3_ref, also callable on the host), on
// every fp32 of magnitude below 464, of both signs.
//
// qmoe_probe_e2m1_cvt: the same for the hardware fp32 -> E2M1 conversion
// (v_cvt_scalef32_pk_fp4_f32 with a unit scale; the first operand in the low
// nibble) against qmoe_probe_e2m1_ref, on every fp32 of magnitude below 8.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

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

// E4M3FN value of a non-negative code 0..126: k 2^-9 below code 8, else
// (1 + m/8) 2^(e-7) with exponent field e and mantissa field m.
__host__ __device__ inline double e4m3_ref_value(uint32_t c) {
  if (c < 8) return (double)c / 512.0;
  const int e = (int)(c >> 3) - 7;
  double v = 1.0 + (double)(c & 7u) / 8.0;
  for (int i = 0; i < e; ++i) v *= 2.0;
  for (int i = 0; i > e; --i) v *= 0.5;
  return v;
}

// The nearest E4M3 value to |v| (ties to the even code, 448 above 448), the
// sign bit of v kept: a binary search over the ascending non-negative codes.
__host__ __device__ inline uint32_t e4m3_ref(float v) {
  const double a = fabs((double)v);
  uint32_t bits;
  memcpy(&bits, &v, 4);
  const uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t lo = 0, hi = 126;  // the largest code whose value is <= a
  if (a >= 448.0) return 126u | sign;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (e4m3_ref_value(mid) <= a) lo = mid; else hi = mid;
  }
  if (e4m3_ref_value(hi) <= a) lo = hi;
  uint32_t c = lo;
  if (lo < 126) {
    const double dlo = a - e4m3_ref_value(lo), dhi = e4m3_ref_value(lo + 1) - a;
    if (dhi < dlo || (dhi == dlo && (lo & 1u))) c = lo + 1;
  }
  return c | sign;
}

constexpr uint32_t kCvtEnd = 0x43E80000u;  // bits of 464.0f

// thread t: the non-negative bit patterns t, t + n, ... below kCvtEnd, each
// with both signs; counts[t] mismatches, first[2t] the first one's bits and
// first[2t+1] its codes (hardware | reference << 16)
__global__ void e4m3_cvt_kernel(uint32_t* __restrict__ counts, uint32_t* __restrict__ first, int n) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (uint32_t)n) return;
  uint32_t bad = 0, fb = 0xFFFFFFFFu, fc = 0;
  for (uint32_t b = t; b < kCvtEnd; b += (uint32_t)n) {
    const float v = __uint_as_float(b);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, -v, 0, false) & 0xFFFFu;
    const uint32_t ref = e4m3_ref(v) | (e4m3_ref(-v) << 8);
    if (hw != ref) {
      if (!bad) fb = b, fc = hw | (ref << 16);
      ++bad;
    }
  }
  counts[t] = bad;
  first[2 * t] = fb;
  first[2 * t + 1] = fc;
}

extern "C" int qmoe_probe_e4m3_cvt(void* counts, void* first, int n, void* stream) {
  if (n <= 0 || n % 256) return -1;
  hipLaunchKernelGGL(e4m3_cvt_kernel, dim3(n / 256), dim3(256), 0, (hipStream_t)stream, (uint32_t*)counts,
                     (uint32_t*)first, n);
  return (int)hipGetLastError();
}

extern "C" uint32_t qmoe_probe_e4m3_ref(float v) { return e4m3_ref(v); }

// The nearest E2M1 magnitude to |v| among 0, .5, 1, 1.5, 2, 3, 4, 6 (ties to
// the even code, 6 above 6), the sign bit of v in bit 3: a scan of the
// ascending grid.
__host__ __device__ inline uint32_t e2m1_ref(float v) {
  const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double a = fabs((double)v);
  uint32_t bits;
  memcpy(&bits, &v, 4);
  uint32_t c = 7;
  for (uint32_t i = 0; i < 7; ++i) {
    const double mid = (grid[i] + grid[i + 1]) / 2;
    if (a < mid || (a == mid && (i & 1u) == 0)) {
      c = i;
      break;
    }
  }
  return c | ((bits >> 28) & 8u);
}

constexpr uint32_t kFp4CvtEnd = 0x41000000u;  // bits of 8.0f

// thread t: the non-negative bit patterns t, t + n, ... below kFp4CvtEnd, each
// with both signs (v in the low nibble, -v in the high one); counts[t]
// mismatches, first[2t] the first one's bits and first[2t+1] its codes
// (hardware | reference << 16)
__global__ void e2m1_cvt_kernel(uint32_t* __restrict__ counts, uint32_t* __restrict__ first, int n) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (uint32_t)n) return;
  uint32_t bad = 0, fb = 0xFFFFFFFFu, fc = 0;
  for (uint32_t b = t; b < kFp4CvtEnd; b += (uint32_t)n) {
    const float v = __uint_as_float(b);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, -v, 1.0f, 0) & 0xFFu;
    const uint32_t ref = e2m1_ref(v) | (e2m1_ref(-v) << 4);
    if (hw != ref) {
      if (!bad) fb = b, fc = hw | (ref << 16);
      ++bad;
    }
  }
  counts[t] = bad;
  first[2 * t] = fb;
  first[2 * t + 1] = fc;
}

extern "C" int qmoe_probe_e2m1_cvt(void* counts, void* first, int n, void* stream) {
  if (n <= 0 || n % 256) return -1;
  hipLaunchKernelGGL(e2m1_cvt_kernel, dim3(n / 256), dim3(256), 0, (hipStream_t)stream, (uint32_t*)counts,
                     (uint32_t*)first, n);
  return (int)hipGetLastError();
}

extern "C" uint32_t qmoe_probe_e2m1_ref(float v) { return e2m1_ref(v); }
