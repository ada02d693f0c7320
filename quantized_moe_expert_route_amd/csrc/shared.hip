// Block-FP8 shared expert (E4M3 weights, one fp32 scale per 128x128 block),
// added to the routed output before the bf16 rounding with weight 1.
//
// "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing" (Summary: the
// shared experts keep the base model's block-FP8 configuration) and "feat(
// glm52 mono): serve a BF16-attention checkpoint" (group-128 FP8
// activations): x is quantized per token per 128 channels to E4M3 with an
// fp32 scale (the same rule as the mid blocks), gate/up and down run on the
// FP8 MFMA, every 128-block partial is scaled by the activation scale times
// the weight block scale, and h is quantized like the routed mid.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

// x bf16 [M, H] -> E4M3 [M, H] + fp32 scale per 128, scales stored
// K-block major ([H/128, M]: a block's scales of consecutive rows are
// contiguous, so the GEMM reads them with one contiguous load); one wave per
// block.
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
    if (lane == 0) s[(size_t)b * M + t] = sc;
  }
}

// out[t, o] = sum_kb a_scale[kb, t] * w_scale[o/128, kb] * (a_kb . w_kb), a
// [rows, K] E4M3 with fp32 scales per 128 along K (K-block major), w [N, K] E4M3 with fp32
// scales per 128x128 block. With GATED the output is SiLU(g) * u, g and u
// from weight rows o and o + n_out.
//
// Workgroup tile: 128 token rows x 128 weight rows (GATED: 64 gate + the 64
// matching up rows, 64 outputs; else 128 outputs), one 128-K block per step:
// both operands staged in LDS as E4M3 through two register-held steps in
// flight; each of 8 waves multiplies 64 rows x 32 weight rows: the E4M3 codes are
// widened to bf16 as they are read (exact) and multiplied on the bf16 MFMA
// (exact products, fp32 sums inside the block); the block's sum times
// (activation scale x weight scale) is formed and added in float64, in block
// order, and rounded once to fp32. (The FP8 MFMA drops products far below
// the largest of their 32-group; its error, amplified by the E4M3
// requantization of h, exceeded the output tolerance.) The result is the
// exact one whenever every block sum fits binary32; E4M3 x E4M3 block sums
// can need more than its 24 bits (a tiny product beside large ones), and
// then the output is close to, not equal to, the exact one.
constexpr int kShBM = 128;  // token rows per tile
// Staged 128-byte rows, 16-byte chunk c of row R at R * 128 + 16 * (c ^ ((R >> 1) & 7)):
// a 16-byte access of 16 lanes is served by the 64 banks together, and both
// the staging stores (8 lanes a row, two rows) and the fragment reads (16
// rows, one chunk) then meet 16 different 16-byte bank groups. (Rows padded
// to 144 bytes, read 8 bytes a lane, stalled on 2-way conflicts.)
__device__ __forceinline__ int sw128(int row, int chunk) { return row * 128 + 16 * (chunk ^ ((row >> 1) & 7)); }

struct alignas(16) ShSmem {  // 16-byte aligned: staging and fragment accesses compile to single b128 LDS ops
  uint8_t a[2][kShBM * 128];
  uint8_t b[2][128 * 128];
  float as[2][kShBM];
};

struct ShRegs {
  uint4 a[2], b[2];
  float sa;
};

// 8 E4M3 codes (two dwords, low byte first) -> 8 bf16, exact
__device__ __forceinline__ v8s e4m3x8_to_bf16(uint2 w) {
  const uint32_t d0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false));
  const uint32_t d1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true));
  const uint32_t d2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false));
  const uint32_t d3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true));
  v8s r;
  r[0] = (short)(d0 & 0xFFFF); r[1] = (short)(d0 >> 16);
  r[2] = (short)(d1 & 0xFFFF); r[3] = (short)(d1 >> 16);
  r[4] = (short)(d2 & 0xFFFF); r[5] = (short)(d2 >> 16);
  r[6] = (short)(d3 & 0xFFFF); r[7] = (short)(d3 >> 16);
  return r;
}

constexpr int kShThreads = 512;  // 8 waves: 2 row halves x 4 weight-row quarters

template <bool GATED>
__global__ __launch_bounds__(kShThreads) void sh_gemm_kernel(const uint8_t* __restrict__ a, const float* __restrict__ as,
                                                      const uint8_t* __restrict__ w, const float* __restrict__ ws,
                                                      int rows, int K, int n_out, float* __restrict__ out) {
  __shared__ ShSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;  // wn 0..3
  const int r = lane & 15, g = lane >> 4;
  constexpr int BN = GATED ? 64 : 128;  // outputs per tile
  const int tiles_n = n_out / BN;
  const int row0 = (blockIdx.x / tiles_n) * kShBM, o0 = (blockIdx.x % tiles_n) * BN;
  const int nkb = K / 128;
  // tile weight row rr -> weight matrix row
  auto brow = [&](int rr) { return GATED ? (rr < 64 ? o0 + rr : n_out + o0 + rr - 64) : o0 + rr; };
  // staging: 128-byte rows in 8 chunks of 16; rows past the end read the
  // last row (their results are never written)
  const uint8_t* pa[2];
  const uint8_t* pb[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int idx = tid + kShThreads * q;
    pa[q] = a + (size_t)min(row0 + (idx >> 3), rows - 1) * K + 16 * (idx & 7);
    pb[q] = w + (size_t)brow(idx >> 3) * K + 16 * (idx & 7);
  }
  const float* psa = as + min(row0 + (tid & (kShBM - 1)), rows - 1);  // + kb * rows
  const float* pwg = ws + (size_t)(brow(0) / 128) * nkb;
  const float* pwu = ws + (size_t)(brow(127) / 128) * nkb;
  auto load = [&](int kb, ShRegs& R) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      R.a[q] = ld16(pa[q] + 128 * kb);
      R.b[q] = ld16(pb[q] + 128 * kb);
    }
    R.sa = psa[(size_t)kb * rows];
  };
  auto store = [&](const ShRegs& R, int s) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + kShThreads * q;
      *reinterpret_cast<uint4*>(&sm.a[s][sw128(idx >> 3, idx & 7)]) = R.a[q];
      *reinterpret_cast<uint4*>(&sm.b[s][sw128(idx >> 3, idx & 7)]) = R.b[q];
    }
    if (tid < kShBM) sm.as[s][tid] = R.sa;
  };
  double acc[4][2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
  // wave (wm, wn): rows 64 wm .. + 64; weight rows: GATED gate 16 wn (j = 0)
  // and up 64 + 16 wn (j = 1); else 32 wn + 16 j
  auto wrow = [&](int j) { return GATED ? 64 * j + 16 * wn : 32 * wn + 16 * j; };
  // in bf16 MFMA step q of a 128-block, lane group g supplies K = 32g + 8q .. + 8
  auto compute = [&](int s, int kb) {
    const float swg = pwg[kb], swu = pwu[kb];
    v4f P[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) P[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    // one 16-byte read (chunk 2 g + p) feeds MFMA steps q = 2 p and 2 p + 1
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint4 ra[4], rb[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const uint4*>(&sm.a[s][sw128(64 * wm + 16 * i + r, 2 * g + p)]);
#pragma unroll
      for (int j = 0; j < 2; ++j) rb[j] = *reinterpret_cast<const uint4*>(&sm.b[s][sw128(wrow(j) + r, 2 * g + p)]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8s fa[4], fb[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = e4m3x8_to_bf16(h ? make_uint2(ra[i].z, ra[i].w) : make_uint2(ra[i].x, ra[i].y));
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = e4m3x8_to_bf16(h ? make_uint2(rb[j].z, rb[j].w) : make_uint2(rb[j].x, rb[j].y));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) P[i][j] = mfma_bf16(fa[i], fb[j], P[i][j]);
      }
    }
    // the block sum times (activation scale x weight scale), added in
    // float64 in block order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double sg[4], su[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double sa = (double)sm.as[s][64 * wm + 16 * i + 4 * g + v];
        sg[v] = sa * (double)swg;  // exact
        su[v] = sa * (double)swu;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double t = (GATED && j == 1 ? su[v] : sg[v]) * (double)P[i][j][v];
          acc[i][j][v] = __dadd_rn(acc[i][j][v], t);
        }
    }
  };
  ShRegs S0, S1;
  load(0, S0);
  load(min(1, nkb - 1), S1);
  store(S0, 0);
  barrier_lds();
  // step kb is multiplied while kb + 1 and kb + 2 are in flight; past the last
  // step the loads repeat it and the stores fill a buffer nobody reads
  for (int kb = 0; kb < nkb; kb += 2) {
    load(min(kb + 2, nkb - 1), S0);
    compute(0, kb);
    store(S1, 1);
    barrier_lds();
    load(min(kb + 3, nkb - 1), S1);
    if (kb + 1 < nkb) compute(1, kb + 1);
    store(S0, 0);
    barrier_lds();
  }
  // D row 4g + v of 16-row group i, column r of weight-row group j
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = row0 + 64 * wm + 16 * i + 4 * g + v;
      if (m >= rows) continue;
      if (GATED) {
        out[(size_t)m * n_out + o0 + 16 * wn + r] = silu_mul((float)acc[i][0][v], (float)acc[i][1][v]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) out[(size_t)m * n_out + o0 + 32 * wn + 16 * j + r] = (float)acc[i][j][v];
      }
    }
}

// h fp32 [rows, I] -> E4M3 + fp32 scale per 128 (same rule as the routed mid),
// scales K-block major ([I/128, rows])
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
    if (lane == 0) s[(size_t)b * rows + row] = sc;
  }
}

hipError_t launch_shared(const moe_plan* p, const CallArgs& a, Ev ev) {
  if (p->s.shared_I == 0) return hipSuccess;
  const int M = (int)a.M, H = (int)p->s.H, Is = (int)p->s.shared_I;
  auto blocks_for = [](int64_t waves, int64_t cap) { return (int)std::min<int64_t>((waves + 3) / 4, cap); };
  // above kSmallM the route launch has quantized x for this expert already
  const bool quant_x = small_path(M, p->s.top_k);
  hipError_t e = hipSuccess;
  if (quant_x)
    e = launch_k(sh_quant_x_kernel, dim3(blocks_for((int64_t)M * (H / 128), 8192)), dim3(256), 0, a.stream,
                 Ev{ev.start, nullptr}, reinterpret_cast<const uint16_t*>(a.x), M, H, wsp<uint8_t>(p, p->L.sh_xq),
                 wsp<float>(p, p->L.sh_xs));
  if (e != hipSuccess) return e;
  const int64_t mt = (M + kShBM - 1) / kShBM;
  e = launch_k(sh_gemm_kernel<true>, dim3((unsigned)(mt * (Is / 64))), dim3(kShThreads), 0, a.stream,
               Ev{quant_x ? nullptr : ev.start, nullptr},
               wsp<uint8_t>(p, p->L.sh_xq), wsp<float>(p, p->L.sh_xs), reinterpret_cast<const uint8_t*>(p->ws13),
               p->ss13, M, H, Is, wsp<float>(p, p->X.sh_h));
  if (e != hipSuccess) return e;
  e = launch_k(sh_act_quant_kernel, dim3(blocks_for((int64_t)M * (Is / 128), 8192)), dim3(256), 0, a.stream, Ev{},
               wsp<float>(p, p->X.sh_h), M, Is, wsp<uint8_t>(p, p->L.sh_hq), wsp<float>(p, p->L.sh_hs));
  if (e != hipSuccess) return e;
  return launch_k(sh_gemm_kernel<false>, dim3((unsigned)(mt * (H / 128))), dim3(kShThreads), 0, a.stream,
                  Ev{nullptr, ev.stop}, wsp<uint8_t>(p, p->L.sh_hq), wsp<float>(p, p->L.sh_hs),
                  reinterpret_cast<const uint8_t*>(p->ws2), p->ss2, M, Is, H, wsp<float>(p, p->L.sh_y));
}

}  // namespace qmoe
