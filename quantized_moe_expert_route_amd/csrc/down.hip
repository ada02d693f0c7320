// down grouped GEMM (FP8 mid x MXFP4 w2) and the routing-weighted combine.
//
// down: y[t, j, :] = sum over mid blocks b of s_b * (q_b . w2_b), K = I,
// reading the FP8 mid bytes and scales produced once per block ("glm53: FP8
// mid hand-off, early split rows, ...", Modifications table, row "mid as FP8
// once"). The E4M3 mid values and the E2M1 * 2^scale weights are widened to
// bf16 (both exactly) and multiplied on the bf16 MFMA, whose products and
// sums are exact while the sum fits binary32; the scaled FP8 MFMA truncates
// products far below the largest of their 32-group, so it would not return
// the block's dot product. Each 128-block's fp32 partial is scaled by s_b in
// float64 and the blocks are summed in order, then rounded once to fp32.
//
// combine: out[t] = bf16(sum_j w[t, j] * y[t, j] (+ shared[t])): products and
// sum in float64 in slot order, one rounding to bf16. Up to kSmallM tokens it
// runs inside the down launch; above, y goes through HBM to its own launch.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

// Up to kSmallM tokens, down and combine are one launch. A workgroup owns 16
// output columns of every token: its four waves take the 16-row tiles in turn
// (tile i to wave i % 4), keep each (sorted row, column) result in LDS, and
// when every tile is done the workgroup forms out[t, c0 .. c0 + 16) from the
// token's k slots, so no slot result leaves the workgroup.
//
// In MFMA step q of a 128-block, lane group g supplies K = 32g + 8q .. + 8:
// a lane reads 32 contiguous mid bytes and 16 contiguous weight bytes (one MX
// block with its one scale byte) per block. Each wave keeps D tiles of loads
// in flight (weights from HBM, mid rows and scales from L2).
constexpr int kDcMaxRows = kSmallM * 16;  // M * k on this path

template <int NB>
struct DcSlot {
  uint4 w[NB];      // this lane's 32 E2M1 weights of each block
  uint4 a[NB][2];   // this lane's 32 E4M3 mid bytes of each block
  uint32_t ws[NB];  // the weights' E8M0 byte
  float sc[NB][4];  // mid scales of the lane's four D rows
};

template <int NB, int D>
__global__ __launch_bounds__(256) void down_combine_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry, const int4* __restrict__ tiles,
    const int* __restrict__ meta, int H, int k, int M, const float* __restrict__ topk_w,
    const float* __restrict__ ys, uint16_t* __restrict__ out) {
  constexpr int I = NB * 128;
  __shared__ float yl[kDcMaxRows * 16];
  __shared__ int inv[kDcMaxRows];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * 16;
  const int n = M * k;
  for (int q = tid; q < n; q += 256) inv[sorted_entry[q]] = q;
  const int nt = meta[0];
  const int my = nt > wave ? (nt - wave + 3) / 4 : 0;  // tiles wave, wave + 4, ...

  auto load = [&](int i, DcSlot<NB>& S) {
    const int4 tl = tiles[wave + 4 * i];
    const uint8_t* pw = w2 + ((size_t)tl.x * H + c0 + r) * (I / 2) + 16 * g;
    const uint8_t* ps = s2 + ((size_t)tl.x * H + c0 + r) * (I / 32) + g;
    // rows past the tile's end read the tile's first row; their results are dropped
    const int row = tl.y + r < tl.z ? tl.y + r : tl.y;
    const uint8_t* pq = midq + (size_t)row * I + 32 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      S.w[b] = ld16(pw + 64 * b);
      S.ws[b] = ps[4 * b];
      S.a[b][0] = ld16(pq + 128 * b);
      S.a[b][1] = ld16(pq + 128 * b + 16);
    }
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int m = tl.y + 4 * g + i2 < tl.z ? tl.y + 4 * g + i2 : tl.y;
#pragma unroll
      for (int b = 0; b < NB; ++b) S.sc[b][i2] = mids[(size_t)m * NB + b];
    }
  };
  auto compute = [&](int i, const DcSlot<NB>& S) {
    const int4 tl = tiles[wave + 4 * i];
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float wsc = e8m0_to_float(S.ws[b]);
      const uint32_t qa[8] = {S.a[b][0].x, S.a[b][0].y, S.a[b][0].z, S.a[b][0].w,
                              S.a[b][1].x, S.a[b][1].y, S.a[b][1].z, S.a[b][1].w};
      const uint32_t qw[4] = {S.w[b].x, S.w[b].y, S.w[b].z, S.w[b].w};
      v4f P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t d0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qa[2 * q], 1.0f, false));
        const uint32_t d1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qa[2 * q], 1.0f, true));
        const uint32_t d2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qa[2 * q + 1], 1.0f, false));
        const uint32_t d3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(qa[2 * q + 1], 1.0f, true));
        v8s fa;
        fa[0] = (short)(d0 & 0xFFFF); fa[1] = (short)(d0 >> 16);
        fa[2] = (short)(d1 & 0xFFFF); fa[3] = (short)(d1 >> 16);
        fa[4] = (short)(d2 & 0xFFFF); fa[5] = (short)(d2 >> 16);
        fa[6] = (short)(d3 & 0xFFFF); fa[7] = (short)(d3 >> 16);
        const uint32_t e0 = cvt_fp4x2_bf16<0>(qw[q], wsc), e1 = cvt_fp4x2_bf16<1>(qw[q], wsc);
        const uint32_t e2 = cvt_fp4x2_bf16<2>(qw[q], wsc), e3 = cvt_fp4x2_bf16<3>(qw[q], wsc);
        v8s fb;
        fb[0] = (short)(e0 & 0xFFFF); fb[1] = (short)(e0 >> 16);
        fb[2] = (short)(e1 & 0xFFFF); fb[3] = (short)(e1 >> 16);
        fb[4] = (short)(e2 & 0xFFFF); fb[5] = (short)(e2 >> 16);
        fb[6] = (short)(e3 & 0xFFFF); fb[7] = (short)(e3 >> 16);
        P = mfma_bf16(fa, fb, P);
      }
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) acc[i2] += (double)S.sc[b][i2] * (double)P[i2];
    }
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int m = tl.y + 4 * g + i2;
      if (m < tl.z) yl[m * 16 + r] = (float)acc[i2];
    }
  };

  if (my > 0) {
    DcSlot<NB> S[D];
#pragma unroll
    for (int d = 0; d < D; ++d) load(d < my ? d : my - 1, S[d]);
    for (int i0 = 0; i0 < my; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int i = i0 + d;
        if (i < my) compute(i, S[d]);
        load(i + D < my ? i + D : my - 1, S[d]);
      }
    }
  }
  __syncthreads();
  // out[t, c0 + 2p .. + 2): float64 products and sum in slot order (+ shared), one bf16 rounding
  for (int idx = tid; idx < M * 8; idx += 256) {
    const int t = idx >> 3, cc = 2 * (idx & 7);
    double a0 = 0.0, a1 = 0.0;
    for (int j = 0; j < k; ++j) {
      const double wj = (double)topk_w[t * k + j];
      const float* py = yl + inv[t * k + j] * 16 + cc;
      a0 += wj * (double)py[0];
      a1 += wj * (double)py[1];
    }
    if (ys) {
      a0 += (double)ys[(size_t)t * H + c0 + cc];
      a1 += (double)ys[(size_t)t * H + c0 + cc + 1];
    }
    *reinterpret_cast<uint32_t*>(out + (size_t)t * H + c0 + cc) =
        bf16_rne_from_double(a0) | (bf16_rne_from_double(a1) << 16);
  }
}

// out[t, c..c+7]: float64 products and sum in slot order (+ shared), then bf16.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const float* __restrict__ ys, int M, int H, int k,
                                                      uint16_t* __restrict__ out) {
  const int per_tok = H / 8;
  const int64_t total = (int64_t)M * per_tok;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / per_tok);
    const int c = (int)(i % per_tok) * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const double wj = (double)w[(size_t)t * k + j];
      const float* py = y + ((size_t)t * k + j) * H + c;
      const float4 a = *reinterpret_cast<const float4*>(py);
      const float4 b = *reinterpret_cast<const float4*>(py + 4);
      acc[0] += wj * (double)a.x; acc[1] += wj * (double)a.y; acc[2] += wj * (double)a.z; acc[3] += wj * (double)a.w;
      acc[4] += wj * (double)b.x; acc[5] += wj * (double)b.y; acc[6] += wj * (double)b.z; acc[7] += wj * (double)b.w;
    }
    if (ys) {
      const float* ps = ys + (size_t)t * H + c;
      const float4 a = *reinterpret_cast<const float4*>(ps);
      const float4 b = *reinterpret_cast<const float4*>(ps + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = bf16_rne_from_double(acc[2 * q]) | (bf16_rne_from_double(acc[2 * q + 1]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_down_combine(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int H = (int)p->s.H;
  if (a.M * p->s.top_k > kDcMaxRows) return hipErrorInvalidValue;
  const float* ys = p->s.shared_I > 0 ? wsp<float>(p, p->L.sh_y) : nullptr;
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(H / 16), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), H, (int)p->s.top_k, (int)a.M, wsp<float>(p, p->L.topk_w), ys,
                    reinterpret_cast<uint16_t*>(a.out));
  };
  switch (p->s.I / 128) {
    case 1: return go(down_combine_kernel<1, 8>);
    case 2: return go(down_combine_kernel<2, 4>);
    case 3: return go(down_combine_kernel<3, 3>);
    case 4: return go(down_combine_kernel<4, 2>);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int H = (int)p->s.H;
  const int64_t total = a.M * (H / 8);
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
  const float* ys = p->s.shared_I > 0 ? wsp<float>(p, p->L.sh_y) : nullptr;
  return launch_k(combine_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<float>(p, p->L.y),
                  wsp<float>(p, p->L.topk_w), ys, (int)a.M, H, (int)p->s.top_k, reinterpret_cast<uint16_t*>(a.out));
}

}  // namespace qmoe
