// Block-FP8 shared expert (E4M3 weights, one fp32 scale per 128x128 block),
// added to the routed output before the bf16 rounding with weight 1.
//
// "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing" (Summary: the
// shared experts keep the base model's block-FP8 configuration) and "feat(
// glm52 mono): serve a BF16-attention checkpoint" (group-128 FP8
// activations): x is quantized per token per 128 channels to E4M3 with an
// fp32 scale (the same rule as the mid blocks), gate/up and down run on the
// FP8 codes widened to bf16, every 128-block partial is scaled by the
// activation scale times the weight block scale in float64, and h is
// quantized like the routed mid.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

struct E4m3Bf16TableS {
  uint16_t v[256];
  constexpr E4m3Bf16TableS() : v() {
    for (int c = 0; c < 256; ++c) v[c] = e4m3_to_bf16_bits((uint32_t)c);
  }
};
__constant__ E4m3Bf16TableS kE4m3Bf16S = E4m3Bf16TableS();

__device__ __forceinline__ v8s e4m3x8_bf16(uint32_t lo, uint32_t hi, const uint16_t* tab) {
  v8s r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (short)tab[(lo >> (8 * i)) & 0xFFu];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[4 + i] = (short)tab[(hi >> (8 * i)) & 0xFFu];
  return r;
}

// x bf16 [M, H] -> E4M3 [M, H] + fp32 scale per 128; one wave per block.
__global__ __launch_bounds__(256) void sh_quant_x_kernel(const uint16_t* __restrict__ x, int M, int H,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int nb = H / 128;
  const int total = M * nb;
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < total; wv += gridDim.x * 4) {
    const int t = wv / nb, b = wv % nb;
    const size_t base = (size_t)t * H + b * 128 + 2 * lane;
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(x + base);
    const float v0 = __uint_as_float(pair << 16), v1 = __uint_as_float(pair & 0xFFFF0000u);
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float sc = __fdiv_rn(amax, 448.0f);
    uint32_t c0 = 0, c1 = 0;
    if (sc > 0.f) {
      c0 = e4m3_code(__fdiv_rn(v0, sc));
      c1 = e4m3_code(__fdiv_rn(v1, sc));
    }
    *reinterpret_cast<uint16_t*>(q + base) = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) s[(size_t)t * nb + b] = sc;
  }
}

// out[t, o] = fl32( sum_kb a_scale[t, kb] * w_scale[o/128, kb] * (a_kb . w_kb) )
// for a 16x16 tile per wave; a [rows, K] E4M3 with fp32 scales per 128 along
// K, w [N, K] E4M3 with fp32 scales per 128x128. With GATED, the tile's
// columns o and o + N/2 are gate and up and the output is SiLU(g) * u.
template <bool GATED>
__global__ __launch_bounds__(256) void sh_linear_kernel(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                        const uint8_t* __restrict__ w, const float* __restrict__ ws,
                                                        int rows, int K, int N, float* __restrict__ out) {
  __shared__ uint16_t tab[256];
  tab[threadIdx.x] = kE4m3Bf16S.v[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int n_out = GATED ? N / 2 : N;
  const int tiles_n = n_out / 16, tiles_m = (rows + 15) / 16;
  const int nkb = K / 128;
  const int kbw = K / 128;  // weight scale row length
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < tiles_m * tiles_n; wv += gridDim.x * 4) {
    const int tm = wv / tiles_n, tn = wv % tiles_n;
    const int row = tm * 16 + r;
    const bool rv = row < rows;
    const int o = tn * 16 + r;  // this lane's weight row (B column)
    const uint8_t* pa = a + (size_t)(rv ? row : 0) * K;
    const uint8_t* pg = w + (size_t)o * K;
    const uint8_t* pu = w + (size_t)(o + n_out) * K;
    double accg[4] = {0, 0, 0, 0}, accu[4] = {0, 0, 0, 0};
    for (int kb = 0; kb < nkb; ++kb) {
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
      if (rv) {
        a0 = ld16(pa + kb * 128 + g * 32);
        a1 = ld16(pa + kb * 128 + g * 32 + 16);
      }
      const v8s A0 = e4m3x8_bf16(a0.x, a0.y, tab), A1 = e4m3x8_bf16(a0.z, a0.w, tab);
      const v8s A2 = e4m3x8_bf16(a1.x, a1.y, tab), A3 = e4m3x8_bf16(a1.z, a1.w, tab);
      v4f P = {0, 0, 0, 0}, Q = {0, 0, 0, 0};
      {
        const uint4 b0 = ld16(pg + kb * 128 + g * 32), b1 = ld16(pg + kb * 128 + g * 32 + 16);
        P = mfma_bf16(A0, e4m3x8_bf16(b0.x, b0.y, tab), P);
        P = mfma_bf16(A1, e4m3x8_bf16(b0.z, b0.w, tab), P);
        P = mfma_bf16(A2, e4m3x8_bf16(b1.x, b1.y, tab), P);
        P = mfma_bf16(A3, e4m3x8_bf16(b1.z, b1.w, tab), P);
      }
      if (GATED) {
        const uint4 b0 = ld16(pu + kb * 128 + g * 32), b1 = ld16(pu + kb * 128 + g * 32 + 16);
        Q = mfma_bf16(A0, e4m3x8_bf16(b0.x, b0.y, tab), Q);
        Q = mfma_bf16(A1, e4m3x8_bf16(b0.z, b0.w, tab), Q);
        Q = mfma_bf16(A2, e4m3x8_bf16(b1.x, b1.y, tab), Q);
        Q = mfma_bf16(A3, e4m3x8_bf16(b1.z, b1.w, tab), Q);
      }
      // D rows 4g+i (activations), column r (weights)
      const double wsg = (double)ws[(size_t)(o / 128) * kbw + kb];
      const double wsu = GATED ? (double)ws[(size_t)((o + n_out) / 128) * kbw + kb] : 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = tm * 16 + 4 * g + i;
        const double sa = m < rows ? (double)as[(size_t)m * nkb + kb] : 0.0;
        accg[i] += (sa * wsg) * (double)P[i];
        if (GATED) accu[i] += (sa * wsu) * (double)Q[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm * 16 + 4 * g + i;
      if (m < rows) {
        float v = (float)accg[i];
        if (GATED) v = silu_mul(v, (float)accu[i]);
        out[(size_t)m * n_out + o] = v;
      }
    }
  }
}

// h fp32 [rows, I] -> E4M3 + fp32 scale per 128 (same rule as the routed mid)
__global__ __launch_bounds__(256) void sh_act_quant_kernel(const float* __restrict__ h, int rows, int I,
                                                           uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int nb = I / 128;
  const int total = rows * nb;
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < total; wv += gridDim.x * 4) {
    const int row = wv / nb, b = wv % nb;
    const size_t base = (size_t)row * I + b * 128 + 2 * lane;
    const float2 v = *reinterpret_cast<const float2*>(h + base);
    const float amax = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
    const float sc = __fdiv_rn(amax, 448.0f);
    uint32_t c0 = 0, c1 = 0;
    if (sc > 0.f) {
      c0 = e4m3_code(__fdiv_rn(v.x, sc));
      c1 = e4m3_code(__fdiv_rn(v.y, sc));
    }
    *reinterpret_cast<uint16_t*>(q + base) = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) s[(size_t)row * nb + b] = sc;
  }
}

hipError_t launch_shared(const moe_plan* p, const CallArgs& a, Ev ev) {
  if (p->s.shared_I == 0) return hipSuccess;
  const int M = (int)a.M, H = (int)p->s.H, Is = (int)p->s.shared_I;
  auto blocks_for = [](int64_t waves, int64_t cap) { return (int)std::min<int64_t>((waves + 3) / 4, cap); };
  hipError_t e = launch_k(sh_quant_x_kernel, dim3(blocks_for((int64_t)M * (H / 128), 8192)), dim3(256), 0, a.stream,
                          Ev{ev.start, nullptr}, reinterpret_cast<const uint16_t*>(a.x), M, H,
                          wsp<uint8_t>(p, p->L.sh_xq), wsp<float>(p, p->L.sh_xs));
  if (e != hipSuccess) return e;
  const int64_t t1 = (int64_t)((M + 15) / 16) * (Is / 16);
  e = launch_k(sh_linear_kernel<true>, dim3(blocks_for(t1, 8192)), dim3(256), 0, a.stream, Ev{},
               wsp<uint8_t>(p, p->L.sh_xq), wsp<float>(p, p->L.sh_xs), reinterpret_cast<const uint8_t*>(p->ws13),
               p->ss13, M, H, 2 * Is, wsp<float>(p, p->X.sh_h));
  if (e != hipSuccess) return e;
  e = launch_k(sh_act_quant_kernel, dim3(blocks_for((int64_t)M * (Is / 128), 8192)), dim3(256), 0, a.stream, Ev{},
               wsp<float>(p, p->X.sh_h), M, Is, wsp<uint8_t>(p, p->L.sh_hq), wsp<float>(p, p->L.sh_hs));
  if (e != hipSuccess) return e;
  const int64_t t2 = (int64_t)((M + 15) / 16) * (H / 16);
  return launch_k(sh_linear_kernel<false>, dim3(blocks_for(t2, 8192)), dim3(256), 0, a.stream, Ev{nullptr, ev.stop},
                  wsp<uint8_t>(p, p->L.sh_hq), wsp<float>(p, p->L.sh_hs), reinterpret_cast<const uint8_t*>(p->ws2),
                  p->ss2, M, Is, H, wsp<float>(p, p->L.sh_y));
}

}  // namespace qmoe
