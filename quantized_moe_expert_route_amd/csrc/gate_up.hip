// gate/up grouped GEMM on MXFP4 (scaled FP4 MFMA), SiLU(gate) * up, and the
// one-time per-128 FP8 E4M3 quantization of mid.
//
// gate/up: "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing"
// (Summary: SiLU activation after the usual expert selection) and the pages'
// MXFP4 (A4W4) arm. Mid: "glm53: FP8 mid hand-off, early split rows, ..."
// (Modifications table, row "mid as FP8 once": each 128-element mid block is
// quantized to FP8 once with its scale, and the down GEMM reads those bytes).
//
// Work item = (tile of up to 16 sorted rows of one expert, 16 columns of I).
// A workgroup of 4 waves computes the gate and the up columns of the item,
// each wave a quarter of the K super-steps; the four partial sums are added
// in wave order through LDS. Within a 512-element super-step, lane group g
// (lanes 16g..16g+15) loads 64 contiguous bytes of its row: the MX blocks
// 4g..4g+3, fed to four MFMAs as block 4g+j in step j. A and B use the same
// assignment, so every MFMA pairs matching K, and each lane's one scale byte
// per step covers exactly its 32 elements.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

__global__ __launch_bounds__(256) void gate_up_m16_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ s13, const int* __restrict__ sorted_entry,
    const int4* __restrict__ tiles, const int* __restrict__ meta, float* __restrict__ hout, int H,
    int I, int k) {
  __shared__ v4f red[2][4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n_it = I / 16;
  const int n_work = meta[0] * n_it;
  const size_t Hb = (size_t)H / 2, Hs = (size_t)H / 32;
  const int nss = H / 512;
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int4 tl = tiles[w / n_it];
    const int it = w % n_it;
    const int e = tl.x, r0 = tl.y, r1 = tl.z;
    const bool rv = r0 + r < r1;
    const int tok = rv ? sorted_entry[r0 + r] / k : 0;
    const uint8_t* pa = xq + (size_t)tok * Hb;
    const uint8_t* psa = xs + (size_t)tok * Hs;
    const size_t grow = (size_t)e * 2 * I + (size_t)it * 16 + r;
    const uint8_t* pg = w13 + grow * Hb;
    const uint8_t* psg = s13 + grow * Hs;
    const uint8_t* pu = pg + (size_t)I * Hb;
    const uint8_t* psu = psg + (size_t)I * Hs;
    v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    for (int ss = wave; ss < nss; ss += 4) {
      const int boff = ss * 256 + g * 64;
      const int soff = ss * 16 + g * 4;
      uint4 a[4], bg[4], bu[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] = rv ? ld16(pa + boff + 16 * j) : make_uint4(0, 0, 0, 0);
        bg[j] = ld16(pg + boff + 16 * j);
        bu[j] = ld16(pu + boff + 16 * j);
      }
      const uint32_t sa = rv ? ld4(psa + soff) : 0x7F7F7F7Fu;
      const uint32_t sg = ld4(psg + soff);
      const uint32_t su = ld4(psu + soff);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t xa = (sa >> (8 * j)) & 0xFFu;
        accg = mfma_fp4(a[j], bg[j], accg, xa, (sg >> (8 * j)) & 0xFFu);
        accu = mfma_fp4(a[j], bu[j], accu, xa, (su >> (8 * j)) & 0xFFu);
      }
    }
    red[0][wave][lane] = accg;
    red[1][wave][lane] = accu;
    __syncthreads();
    {
      // thread -> (row m, column n) of the 16x16 item
      const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
      const int l = n + 16 * (m >> 2), i = m & 3;
      const float G = ((red[0][0][l][i] + red[0][1][l][i]) + red[0][2][l][i]) + red[0][3][l][i];
      const float U = ((red[1][0][l][i] + red[1][1][l][i]) + red[1][2][l][i]) + red[1][3][l][i];
      if (r0 + m < r1) hout[(size_t)(r0 + m) * I + it * 16 + n] = silu_mul(G, U);
    }
    __syncthreads();
  }
}

// One wave per (row, 128-block): s = fl32(amax / 448), q = E4M3(fl32(h / s)).
__global__ __launch_bounds__(256) void act_quant_kernel(const float* __restrict__ h, int rows, int I,
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

hipError_t launch_gate_up(const moe_plan* p, const CallArgs& a) {
  const int I = (int)p->s.I;
  const int64_t n = a.M * p->s.top_k;
  const int64_t t16 = (n + std::min<int64_t>(p->s.E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows;
  const int64_t work_max = t16 * (I / 16);
  const int blocks = (int)std::min<int64_t>(work_max, 2048);
  hipLaunchKernelGGL(gate_up_m16_kernel, dim3(blocks), dim3(256), 0, a.stream,
                     wsp<uint8_t>(p, p->L.xq), wsp<uint8_t>(p, p->L.xs),
                     reinterpret_cast<const uint8_t*>(a.w13), reinterpret_cast<const uint8_t*>(a.s13),
                     wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles), wsp<int>(p, p->X.meta),
                     wsp<float>(p, p->X.h), (int)p->s.H, I, (int)p->s.top_k);
  return hipGetLastError();
}

hipError_t launch_act_quant(const moe_plan* p, const CallArgs& a) {
  const int rows = (int)(a.M * p->s.top_k);
  const int I = (int)p->s.I;
  const int64_t waves = (int64_t)rows * (I / 128);
  const int blocks = (int)std::min<int64_t>((waves + 3) / 4, 8192);
  hipLaunchKernelGGL(act_quant_kernel, dim3(blocks), dim3(256), 0, a.stream, wsp<float>(p, p->X.h), rows, I,
                     wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids));
  return hipGetLastError();
}

}  // namespace qmoe
