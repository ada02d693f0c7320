// Block-FP8 shared expert (E4M3 weights, one fp32 scale per 128x128 block),
// added to the routed output before the bf16 rounding with weight 1.
//
// "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing" (Summary: the
// shared experts keep the base model's block-FP8 configuration) and "feat(
// glm52 mono): serve a BF16-attention checkpoint" (group-128 FP8
// activations): x is quantized per token per 128 channels to E4M3 with an
// fp32 scale (the same rule as the mid blocks), every 128-K block sum of
// E4M3 x E4M3 products is scaled by the activation scale times the weight
// block scale, and h is quantized like the routed mid.
//
// Exactness. A 128-block sum of E4M3 x E4M3 products can need ~43
// significant bits (a product of two subnormal-step values beside products
// of two values near 448), more than binary32 holds, so no fp32-accumulating
// MFMA returns it in every case. Here every E4M3 operand is held as three
// base-128 int8 digits of v * 2^9 (e4m3_digits) and the int8 MFMA sums the
// nine digit-pair products exactly in int32; the five power-of-128 sums of a
// block are folded into two int32 (no overflow: see the bounds below) and one exact
// float64. The block sum times (activation scale x weight scale) is then
// formed and added in float64 in block order and rounded once to fp32.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

// x bf16 [M, H] -> E4M3 digit rows [M, H/128, 3, 128] + fp32 scale per 128,
// scales stored K-block major ([H/128, M]: a block's scales of consecutive
// rows are contiguous); one wave per block.
__global__ __launch_bounds__(256) void sh_quant_x_kernel(const uint16_t* __restrict__ x, int M, int H,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int nb = H / 128;
  const int total = M * nb;
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < total; wv += gridDim.x * 4) {
    const int t = wv / nb, b = wv % nb;
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(x + (size_t)t * H + b * 128 + 2 * lane);
    const float v0 = __uint_as_float(pair << 16), v1 = __uint_as_float(pair & 0xFFFF0000u);
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float sc = __fdiv_rn(amax, 448.0f);
    const uint32_t c01 = sc > 0.f ? e4m3_pack2(__fdiv_rn(v0, sc), __fdiv_rn(v1, sc)) : 0u;
    store_digits2(q + ((size_t)t * nb + b) * kShDigitBlock, 2 * lane, c01);
    if (lane == 0) s[(size_t)b * M + t] = sc;
  }
}

// h fp32 [rows, I] -> E4M3 digit rows + fp32 scale per 128 (same rule as the
// routed mid), scales K-block major ([I/128, rows])
__global__ __launch_bounds__(256) void sh_act_quant_kernel(const float* __restrict__ h, int rows, int I,
                                                           uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int nb = I / 128;
  const int total = rows * nb;
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < total; wv += gridDim.x * 4) {
    const int row = wv / nb, b = wv % nb;
    const float2 v = *reinterpret_cast<const float2*>(h + (size_t)row * I + b * 128 + 2 * lane);
    const float amax = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
    const float sc = __fdiv_rn(amax, 448.0f);
    const uint32_t c01 = sc > 0.f ? e4m3_pack2(__fdiv_rn(v.x, sc), __fdiv_rn(v.y, sc)) : 0u;
    store_digits2(q + ((size_t)row * nb + b) * kShDigitBlock, 2 * lane, c01);
    if (lane == 0) s[(size_t)b * rows + row] = sc;
  }
}

// Row-major E4M3 weights [rows, K] -> digit rows [rows, K/128, 3, 128]; a
// thread per 16 codes.
__global__ __launch_bounds__(256) void sh_pack_kernel(const uint8_t* __restrict__ w, int64_t rows, int K,
                                                      uint8_t* __restrict__ out) {
  const int64_t n16 = rows * (K / 16);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / (K / 16);
    const int c = (int)(i - row * (K / 16)) * 16;  // first column
    const uint4 v = ld16(w + row * K + c);
    uint4 d[3];
    e4m3x4_digits(v.x, d[0].x, d[1].x, d[2].x);
    e4m3x4_digits(v.y, d[0].y, d[1].y, d[2].y);
    e4m3x4_digits(v.z, d[0].z, d[1].z, d[2].z);
    e4m3x4_digits(v.w, d[0].w, d[1].w, d[2].w);
    uint8_t* blk = out + (row * (K / 128) + c / 128) * kShDigitBlock + (c & 127);
#pragma unroll
    for (int p = 0; p < 3; ++p) *reinterpret_cast<uint4*>(blk + 128 * p) = d[p];
  }
}

// out[t, o] = sum_kb a_scale[kb, t] * w_scale[o/128, kb] * (a_kb . w_kb), a
// [rows, K] and w [N, K] E4M3 as digit rows, a's fp32 scales per 128 along K
// (K-block major), w's per 128x128 block. With GATED the output is
// SiLU(g) * u, g and u from weight rows o and o + n_out.
//
// Workgroup tile: 128 token rows x 64 weight rows (GATED: 32 gate + the 32
// matching up rows, 32 outputs; else 64 outputs), one 128-K block per step.
// Both operands' three digit planes go from global memory straight into LDS
// (global_load_lds: each wave instruction fills one contiguous 1 KB, eight
// 128-byte rows, every lane fetching the chunk the swizzle puts at its
// place), two stage buffers, the next block's loads issued before the
// current block is multiplied. Each of 8 waves owns 32 rows x 32 weight
// rows (GATED: 16 gate + 16 up) as 2 x 2 int8-MFMA tiles with five int32
// accumulators each, one per power of 128.
constexpr int kShBM = 128;  // token rows per tile
constexpr int kShBN = 64;   // weight rows per tile
constexpr int kShThreads = 512;

// Staged 128-byte rows, 16-byte chunk c of row R at R * 128 + 16 * (c ^ ((R >> 1) & 7)):
// a 16-byte access of 16 lanes is served by the 64 banks together, and the
// fragment reads (16 rows, one chunk) then meet 16 different 16-byte bank
// groups.
__device__ __forceinline__ int sw128(int row, int chunk) { return row * 128 + 16 * (chunk ^ ((row >> 1) & 7)); }

struct alignas(16) ShStage {  // 16-byte aligned: every fragment read is one b128 op
  uint8_t a[3][kShBM * 128];
  uint8_t b[3][kShBN * 128];
  float as[kShBM];
};

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// 16 bytes a lane from global memory into LDS at dst + 16 * lane (dst the
// same for the whole wave)
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)dst, 16, 0, 0);
}

// s_waitcnt vmcnt(0): the wave's loads into LDS have landed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Block sums from the five power sums P_p = sum over digit pairs
// (i, j) with i + j = p of the int8 dot products. T = sum_p 128^p P_p is the
// block's exact sum times 2^18. Bounds (128 products, |d0|,|d1| <= 127,
// |d2| <= 14): |P0| < 2^21, |P1| < 2^22, so LOW = P0 + 2^7 P1 < 2^30;
// |P2| < 2^21.3, |P3| < 2^18.8, |P4| < 2^14.7, so HIGH = P2 + 2^7 P3 +
// 2^14 P4 < 2^29; T = 2^14 HIGH + LOW < 2^44 is exact in float64.
//
// acc + fl64(s * T) with the product rounded on its own, as the block sums'
// scaling and accumulation are defined (s * T needs up to ~92 bits: a fused
// multiply-add would round once where the definition rounds twice)
__device__ __forceinline__ double add_scaled(double acc, double s, double T) {
#pragma clang fp contract(off)
  const double t = s * T;
  return acc + t;
}

template <bool GATED>
__global__ __launch_bounds__(kShThreads, 1) void sh_gemm_kernel(const uint8_t* __restrict__ a,
                                                                const float* __restrict__ as,
                                                                const uint8_t* __restrict__ w,
                                                                const float* __restrict__ ws, int rows, int K,
                                                                int n_out, float* __restrict__ out) {
  __shared__ ShStage st0, st1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // rows 32 wm .., weight rows of wn
  const int r = lane & 15, g = lane >> 4;
  constexpr int BO = GATED ? kShBN / 2 : kShBN;  // outputs per tile
  const int tiles_n = n_out / BO;
  const int row0 = (blockIdx.x / tiles_n) * kShBM, o0 = (blockIdx.x % tiles_n) * BO;
  const int nkb = K / 128;
  const uint32_t rowbytes = 3u * (uint32_t)K;  // one digit row
  // tile weight row rr (0..63) -> weight matrix row
  auto brow = [&](int rr) { return GATED ? (rr < 32 ? o0 + rr : n_out + o0 + rr - 32) : o0 + rr; };
  // Loads into LDS: the A tile is 48 regions of 1 KB (plane p = region / 16,
  // rows 8 * (region % 16) .. + 8), 6 per wave; the B tile 24 (plane
  // region / 8, rows 8 * (region % 8) ..), 3 per wave. Lane l of a region
  // fills row R = first + l / 8 at chunk place l % 8, which holds logical
  // chunk (l % 8) ^ ((R >> 1) & 7) = (l % 8) ^ (4 * (region % 2) + l / 16):
  // a lane's offset is one of two values (lofs) plus a part common to the
  // wave. A's rows are padded to a multiple of 128 in the workspace, so rows
  // past the end are read (and never written out) without a clamp. Offsets
  // are 32-bit (a tile's A rows span < 2^25 bytes, all of w < 2^30).
  const uint32_t lrow = (uint32_t)(lane >> 3) * rowbytes;
  const uint32_t lofs0 = lrow + 16u * (uint32_t)((lane & 7) ^ (lane >> 4));
  const uint32_t lofs1 = lrow + 16u * (uint32_t)((lane & 7) ^ (4 + (lane >> 4)));
  const uint8_t* abase = a + (size_t)row0 * rowbytes;
  // (the wave-uniform part of an offset goes through readfirstlane, which
  // keeps the compiler from hoisting one register per load out of the loop)
  auto dma = [&](int kb, ShStage& S) {
    const uint32_t o = (uint32_t)kb * kShDigitBlock;
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const int reg = wave * 6 + q, rb = reg & 15;
      const uint32_t u = __builtin_amdgcn_readfirstlane((uint32_t)(8 * rb) * rowbytes + 128u * (reg >> 4) + o);
      dma16(abase + (u + ((rb & 1) ? lofs1 : lofs0)), &S.a[reg >> 4][1024 * rb]);
    }
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int reg = wave * 3 + q, rb = reg & 7;
      const int wr = brow(8 * rb);  // the region's first weight row (its 8 rows are consecutive)
      const uint32_t u = __builtin_amdgcn_readfirstlane((uint32_t)wr * rowbytes + 128u * (reg >> 3) + o);
      dma16(w + (u + ((rb & 1) ? lofs1 : lofs0)), &S.b[reg >> 3][1024 * rb]);
    }
  };
  const float* psa = as + min(row0 + (tid & (kShBM - 1)), rows - 1);  // + kb * rows
  const float* pwg = ws + (size_t)(brow(0) / 128) * nkb;
  const float* pwu = ws + (size_t)(brow(kShBN - 1) / 128) * nkb;
  double acc[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
  // tile weight rows of column group j: GATED gate 16 wn (j = 0) and up
  // 32 + 16 wn (j = 1); else 32 wn + 16 j
  auto wrow = [&](int j) { return GATED ? 32 * j + 16 * wn : 32 * wn + 16 * j; };
  // The two waves on a SIMD (w and w + 4) take turns: waves 0..3 multiply a
  // block and then finish it in float64; waves 4..7 first finish the previous
  // block and then multiply, so one wave's float64 work runs beside the other
  // wave's MFMAs. Right after its MFMAs every wave folds the five power sums
  // into HIGH/LOW (hl); what waits for the float64 step is hl with the
  // block's scales (sa_p, swg_p, swu_p).
  const bool fold_first = wave >= 4;
  v4i P[5][2][2];
  int hl[2][2][4][2];
  float sa_p[2][4];
  float swg_p = 0.f, swu_p = 0.f;
  auto fold = [&]() {
    // the weight scale times 2^-18 (exact)
    const double swg = (double)swg_p * 0x1p-18, swu = (double)swu_p * 0x1p-18;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double sa = (double)sa_p[i][v];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const double sab = sa * (GATED && j == 1 ? swu : swg);
          const double T = fma((double)hl[i][j][v][0], 16384.0, (double)hl[i][j][v][1]);
          acc[i][j][v] = add_scaled(acc[i][j][v], sab, T);
        }
      }
  };
  auto multiply = [&](const ShStage& S, int kb) {
#pragma unroll
    for (int q = 0; q < 5; ++q)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) P[q][i][j] = v4i{0, 0, 0, 0};
    // K half h: lane group g supplies bytes 64 h + 16 g .. + 16 of its row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 B[2][3];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          B[j][p] = *reinterpret_cast<const uint4*>(&S.b[p][sw128(wrow(j) + r, 4 * h + g)]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint4 A[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          A[p] = *reinterpret_cast<const uint4*>(&S.a[p][sw128(32 * wm + 16 * i + r, 4 * h + g)]);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          P[0][i][j] = mfma_i8(A[0], B[j][0], P[0][i][j]);
          P[1][i][j] = mfma_i8(A[0], B[j][1], mfma_i8(A[1], B[j][0], P[1][i][j]));
          P[2][i][j] = mfma_i8(A[0], B[j][2], mfma_i8(A[1], B[j][1], mfma_i8(A[2], B[j][0], P[2][i][j])));
          P[3][i][j] = mfma_i8(A[1], B[j][2], mfma_i8(A[2], B[j][1], P[3][i][j]));
          P[4][i][j] = mfma_i8(A[2], B[j][2], P[4][i][j]);
        }
      }
    }
    // HIGH = P2 + 2^7 P3 + 2^14 P4, LOW = P0 + 2^7 P1, and the block's scales
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hl[i][j][v][0] = P[2][i][j][v] + P[3][i][j][v] * 128 + P[4][i][j][v] * 16384;
          hl[i][j][v][1] = P[0][i][j][v] + P[1][i][j][v] * 128;
        }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) sa_p[i][v] = S.as[32 * wm + 16 * i + 4 * g + v];
    swg_p = pwg[kb];
    swu_p = pwu[kb];
  };
  // (scheduling fences keep the phases apart: interleaved, the compiler's
  // schedule held more values than the register file)
  auto compute = [&](const ShStage& S, int kb) {
    if (fold_first) {
      if (kb > 0) fold();
      __builtin_amdgcn_sched_barrier(0);
      multiply(S, kb);
    } else {
      multiply(S, kb);
      __builtin_amdgcn_sched_barrier(0);
      fold();
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // one step: the next block's loads go out, this block is multiplied, then
  // the wave's loads are waited for and one barrier makes every wave's
  // loads visible (and frees this block's stage for the step after next)
  auto step = [&](int kb, const ShStage& cur, ShStage& nxt) {
    const bool more = kb + 1 < nkb;
    float sa_n = 0.f;
    if (more) {
      dma(kb + 1, nxt);
      if (tid < kShBM) sa_n = psa[(size_t)(kb + 1) * rows];
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, kb);
    if (more && tid < kShBM) nxt.as[tid] = sa_n;
    wait_vm0();
    barrier_lds();
  };
  dma(0, st0);
  if (tid < kShBM) st0.as[tid] = psa[0];
  wait_vm0();
  barrier_lds();
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, st0, st1);
    if (kb + 1 < nkb) step(kb + 1, st1, st0);
  }
  if (fold_first) fold();
  // D row 4g + v of 16-row group i, column r of weight-row group j
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = row0 + 32 * wm + 16 * i + 4 * g + v;
      if (m >= rows) continue;
      if (GATED) {
        out[(size_t)m * n_out + o0 + 16 * wn + r] = silu_mul((float)acc[i][0][v], (float)acc[i][1][v]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) out[(size_t)m * n_out + o0 + 32 * wn + 16 * j + r] = (float)acc[i][j][v];
      }
    }
}

hipError_t launch_pack_shared(const void* ws13, const void* ws2, int64_t Is, int64_t H, void* packed,
                              hipStream_t stream) {
  uint8_t* p13 = reinterpret_cast<uint8_t*>(packed);
  uint8_t* p2 = p13 + 3 * (2 * Is) * H;
  auto blocks = [](int64_t n16) { return (int)std::min<int64_t>((n16 + 255) / 256, 8192); };
  hipError_t e = launch_k(sh_pack_kernel, dim3(blocks(2 * Is * H / 16)), dim3(256), 0, stream, Ev{},
                          reinterpret_cast<const uint8_t*>(ws13), 2 * Is, (int)H, p13);
  if (e != hipSuccess) return e;
  e = launch_k(sh_pack_kernel, dim3(blocks(H * Is / 16)), dim3(256), 0, stream, Ev{},
               reinterpret_cast<const uint8_t*>(ws2), H, (int)Is, p2);
  if (e != hipSuccess) return e;
  // the E4M3 codes as given, for the shared expert inside the small-token launches
  uint8_t* c13 = p13 + 9 * Is * H;
  e = hipMemcpyAsync(c13, ws13, (size_t)(2 * Is * H), hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return e;
  return hipMemcpyAsync(c13 + 2 * Is * H, ws2, (size_t)(H * Is), hipMemcpyDeviceToDevice, stream);
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
  const uint8_t* w13d = reinterpret_cast<const uint8_t*>(p->ws13);
  const uint8_t* w2d = w13d + (size_t)3 * (2 * Is) * H;
  e = launch_k(sh_gemm_kernel<true>, dim3((unsigned)(mt * (Is / (kShBN / 2)))), dim3(kShThreads), 0, a.stream,
               Ev{quant_x ? nullptr : ev.start, nullptr},
               wsp<uint8_t>(p, p->L.sh_xq), wsp<float>(p, p->L.sh_xs), w13d, p->ss13, M, H, Is,
               wsp<float>(p, p->X.sh_h));
  if (e != hipSuccess) return e;
  e = launch_k(sh_act_quant_kernel, dim3(blocks_for((int64_t)M * (Is / 128), 8192)), dim3(256), 0, a.stream, Ev{},
               wsp<float>(p, p->X.sh_h), M, Is, wsp<uint8_t>(p, p->L.sh_hq), wsp<float>(p, p->L.sh_hs));
  if (e != hipSuccess) return e;
  return launch_k(sh_gemm_kernel<false>, dim3((unsigned)(mt * (H / kShBN))), dim3(kShThreads), 0, a.stream,
                  Ev{nullptr, ev.stop}, wsp<uint8_t>(p, p->L.sh_hq), wsp<float>(p, p->L.sh_hs), w2d, p->ss2, M,
                  Is, H, wsp<float>(p, p->L.sh_y));
}

}  // namespace qmoe
