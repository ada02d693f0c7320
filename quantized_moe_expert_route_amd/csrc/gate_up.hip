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
// each wave a quarter of the K super-steps (4 K-steps of 128); the four
// partial sums are added in wave order through LDS. In K-step ks lane
// 16 g + r supplies row r's MX block 4 ks + g (16 bytes and one scale byte),
// for x and for the weights alike, so every MFMA pairs matching K. The
// weights come packed (moe_pack_w13): a K-step of the item's 16 gate (or up)
// rows is 1 KB contiguous in lane order, and a row block's scales of a
// super-step are one dword per lane.
#include "common.h"
#include "internal.h"
#include "shared_small.h"

#include <algorithm>

namespace qmoe {

constexpr int kSS = 3;  // super-steps (512 K each) whose loads a wave keeps in flight

// One wave quantizes rows [r0, r1) of mid block b: s = fl32(amax / 448),
// q = E4M3(fl32(h / s)); 128 values = 2 per lane.
__device__ __forceinline__ void quant_mid_rows(const float* __restrict__ h, int r0, int r1, int row_step, int I, int b,
                                               uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int nb = I / 128;
  for (int row = r0; row < r1; row += row_step) {
    const size_t base = (size_t)row * I + b * 128 + 2 * lane;
    const float2 v = *reinterpret_cast<const float2*>(h + base);
    const float amax = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
    const float sc = __fdiv_rn(amax, 448.0f);
    const uint32_t c01 = sc > 0.f ? e4m3_pack2(__fdiv_rn(v.x, sc), __fdiv_rn(v.y, sc)) : 0u;
    *reinterpret_cast<uint16_t*>(q + base) = (uint16_t)c01;
    if (lane == 0) s[(size_t)row * nb + b] = sc;
  }
}

__global__ __launch_bounds__(256) void gate_up_m16_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const uint8_t* __restrict__ w13p,
    const uint8_t* __restrict__ s13p, const int* __restrict__ sorted_entry,
    const int4* __restrict__ tiles, const int* __restrict__ meta, float* __restrict__ hout, int H,
    int I, int k) {
  __shared__ v4f red[2][4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n_it = I / 16;
  // The first item's tile is read beside meta (the grid never exceeds the
  // tile array's bound, so the read is in bounds; it is used only when the
  // item exists): one memory round trip fewer before the weights move.
  int4 tl = tiles[blockIdx.x / n_it];
  int n_tiles = meta[0];
  asm volatile("" : "+s"(n_tiles), "+s"(tl.x), "+s"(tl.y), "+s"(tl.z));  // both loads in flight together
  const int n_work = n_tiles * n_it;
  const size_t Hb = (size_t)H / 2, Hs = (size_t)H / 32;
  const int nss = H / 512, nks = H / 128;
  const size_t nrb = (size_t)I / 8;  // 16-row blocks of an expert's 2I rows
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    if (w != (int)blockIdx.x) tl = tiles[w / n_it];
    const int it = w % n_it;
    const int e = tl.x, r0 = tl.y, r1 = tl.z;
    const bool rv = r0 + r < r1;
    // the row's entry is waited for only after the first weight loads are
    // out (the empty asm keeps its use inside the loop, behind them)
    int se = sorted_entry[min(r0 + r, r1 - 1)];
    const uint8_t* pa = xq;   // the row's token's x: + 64 ks (set once the entry is in)
    const uint8_t* psa = xs;  // its scales: + 16 ss: byte 4 j + g is K-step 4 ss + j
    const size_t rbg = (size_t)e * nrb + it, rbu = rbg + I / 16;
    const uint8_t* pg = w13p + rbg * nks * 1024 + 16 * lane;  // + 1024 ks
    const uint8_t* pu = w13p + rbu * nks * 1024 + 16 * lane;
    const uint8_t* psg = s13p + rbg * nss * 256 + 4 * lane;  // + 256 ss: byte j is K-step 4 ss + j
    const uint8_t* psu = s13p + rbu * nss * 256 + 4 * lane;
    v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    // wave w owns the contiguous super-steps [w*per, (w+1)*per); all loads of
    // up to kSS of them are in flight before the first MFMA
    const int per = (nss + 3) / 4;
    const int ss_end = min(nss, (wave + 1) * per);
    for (int ss0 = wave * per; ss0 < ss_end; ss0 += kSS) {
      uint4 a[kSS][4], bg[kSS][4], bu[kSS][4], sa[kSS];
      uint32_t sg[kSS], su[kSS];
#pragma unroll
      for (int q = 0; q < kSS; ++q) {
        const int ss = min(ss0 + q, ss_end - 1);  // clamped: a duplicate step is loaded but not used
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bg[q][j] = ld16(pg + (size_t)(4 * ss + j) * 1024);
          bu[q][j] = ld16(pu + (size_t)(4 * ss + j) * 1024);
        }
        sg[q] = ld4(psg + 256 * ss);
        su[q] = ld4(psu + 256 * ss);
        if (q == 0) {
          asm volatile("" : "+v"(se));
          const size_t tok = rv ? (size_t)(se / k) : 0;
          pa = xq + tok * Hb + 16 * g;
          psa = xs + tok * Hs;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) a[q][j] = rv ? ld16(pa + (4 * ss + j) * 64) : make_uint4(0, 0, 0, 0);
        sa[q] = rv ? ld16(psa + 16 * ss) : make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
      }
#pragma unroll
      for (int q = 0; q < kSS; ++q) {
        if (ss0 + q < ss_end) {
          const uint32_t xw[4] = {sa[q].x, sa[q].y, sa[q].z, sa[q].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t xa = (xw[j] >> (8 * g)) & 0xFFu;
            accg = mfma_fp4(a[q][j], bg[q][j], accg, xa, (sg[q] >> (8 * j)) & 0xFFu);
            accu = mfma_fp4(a[q][j], bu[q][j], accu, xa, (su[q] >> (8 * j)) & 0xFFu);
          }
        }
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
// With the shared expert inside the small-token launches, the workgroups
// after the routed ones form its h from the gate/up partials and quantize
// it (one workgroup per token and 128-block).
__global__ __launch_bounds__(256) void act_quant_kernel(const float* __restrict__ h, int rows, int I,
                                                        uint8_t* __restrict__ q, float* __restrict__ s,
                                                        int routed_blocks, SharedSmall sh, int M, int H) {
  if ((int)blockIdx.x >= routed_blocks) {
    __shared__ float u_lds[130];
    const int snb = sh.Is / 128;
    for (int sb = (int)blockIdx.x - routed_blocks; sb < M * snb; sb += (int)gridDim.x - routed_blocks)
      shared_mid_block(sh, sb / snb, sb % snb, M, H, u_lds);
    return;
  }
  const int nb = I / 128;
  const int total = rows * nb;
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < total; wv += routed_blocks * 4) {
    const int row = wv / nb, b = wv % nb;
    quant_mid_rows(h, row, row + 1, 1, I, b, q, s);
  }
}

hipError_t launch_gate_up(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int I = (int)p->s.I;
  const int64_t n = a.M * p->s.top_k;
  const int64_t t16 = (n + std::min<int64_t>(p->s.E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows;
  const int64_t work_max = t16 * (I / 16);
  const int blocks = (int)std::min<int64_t>(work_max, 2048);
  return launch_k(gate_up_m16_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.xq),
                  wsp<uint8_t>(p, p->L.xs), reinterpret_cast<const uint8_t*>(a.w13),
                  reinterpret_cast<const uint8_t*>(a.s13), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                  wsp<int>(p, p->X.meta), wsp<float>(p, p->X.h), (int)p->s.H, I, (int)p->s.top_k);
}

hipError_t launch_act_quant(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int rows = (int)(a.M * p->s.top_k);
  const int I = (int)p->s.I;
  const SharedSmall sh = shared_small(p, a.M);  // the fused shared expert's h: a workgroup per 128-block
  const int64_t waves = (int64_t)rows * (I / 128);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((waves + 3) / 4, 8192));
  const int sh_blocks = sh.part ? (int)(a.M * (sh.Is / 128)) : 0;
  return launch_k(act_quant_kernel, dim3(blocks + sh_blocks), dim3(256), 0, a.stream, ev, wsp<float>(p, p->X.h),
                  rows, I, wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids), blocks, sh, (int)a.M,
                  (int)p->s.H);
}

}  // namespace qmoe
