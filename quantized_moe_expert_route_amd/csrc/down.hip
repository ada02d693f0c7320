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
// sum in float64 in slot order, one rounding to bf16.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

struct E4m3Bf16Table {
  uint16_t v[256];
  constexpr E4m3Bf16Table() : v() {
    for (int c = 0; c < 256; ++c) v[c] = e4m3_to_bf16_bits((uint32_t)c);
  }
};
__constant__ E4m3Bf16Table kE4m3Bf16 = E4m3Bf16Table();

// 8 E4M3 bytes (two dwords) -> 8 bf16 (v8s) through an LDS copy of the table.
__device__ __forceinline__ v8s e4m3x8_to_bf16(uint32_t lo, uint32_t hi, const uint16_t* tab) {
  v8s r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (short)tab[(lo >> (8 * i)) & 0xFFu];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[4 + i] = (short)tab[(hi >> (8 * i)) & 0xFFu];
  return r;
}

// 8 E2M1 codes (one dword, element 2i low nibble) * scale -> 8 bf16.
__device__ __forceinline__ v8s fp4x8_to_bf16(uint32_t src, float scale) {
  uint32_t d0 = cvt_fp4x2_bf16<0>(src, scale);
  uint32_t d1 = cvt_fp4x2_bf16<1>(src, scale);
  uint32_t d2 = cvt_fp4x2_bf16<2>(src, scale);
  uint32_t d3 = cvt_fp4x2_bf16<3>(src, scale);
  v8s r;
  r[0] = (short)(d0 & 0xFFFF); r[1] = (short)(d0 >> 16);
  r[2] = (short)(d1 & 0xFFFF); r[3] = (short)(d1 >> 16);
  r[4] = (short)(d2 & 0xFFFF); r[5] = (short)(d2 >> 16);
  r[6] = (short)(d3 & 0xFFFF); r[7] = (short)(d3 >> 16);
  return r;
}

// Work item = (tile of up to 16 sorted rows, 256 output columns); each of the
// 4 waves owns 4 tiles of 16 columns. For a 128-block the four bf16 MFMAs of
// K=32 take, in step q, K = 32g + 8q.. for lane group g, so a lane reads 32
// contiguous mid bytes and 16 contiguous weight bytes (one MX block, one
// scale byte) per block.
// out[t, c0 .. c0 + n) from y (float64 products and sum in slot order, plus
// the shared expert), one bf16 rounding; thread i does columns c0 + i + kk*step.
__device__ __forceinline__ void combine_cols(const float* __restrict__ y, const float* __restrict__ w,
                                             const float* __restrict__ ys, int t, int k, int H, int c0, int ncols,
                                             uint16_t* __restrict__ out) {
  for (int c = c0 + (int)threadIdx.x; c < c0 + ncols; c += blockDim.x) {
    double acc = 0.0;
    for (int j = 0; j < k; ++j)
      acc += (double)w[(size_t)t * k + j] * (double)y[((size_t)t * k + j) * H + c];
    if (ys) acc += (double)ys[(size_t)t * H + c];
    out[(size_t)t * H + c] = (uint16_t)bf16_rne_from_double(acc);
  }
}

// FUSED: after writing its y rows of a 256-column chunk, the workgroup counts
// one finished slot per (token, chunk); the workgroup that brings a token's
// count to k combines that token's chunk (and resets the counter).
template <int NB, bool FUSED>  // NB = I / 128
__global__ __launch_bounds__(256) void down_m16_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry, const int4* __restrict__ tiles,
    const int* __restrict__ meta, float* __restrict__ y, int H, int k, const float* __restrict__ topk_w,
    const float* __restrict__ ys, uint32_t* __restrict__ cctr, uint16_t* __restrict__ out) {
  constexpr int I = NB * 128;
  __shared__ uint16_t tab[256];
  __shared__ int s_done[16];
  __shared__ int s_ndone;
  tab[threadIdx.x] = kE4m3Bf16.v[threadIdx.x];
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n_chunks = H / 256;
  const int n_work = meta[0] * n_chunks;
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    const int4 tl = tiles[w / n_chunks];
    const int nc = w % n_chunks;
    const int e = tl.x, r0 = tl.y, r1 = tl.z;
    // all weight loads of the wave's 4 column tiles go out first (the weights come from HBM; mid is in L2)
    uint4 wbuf[4][NB];
    uint32_t wsbuf[4][NB];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = nc * 256 + wave * 64 + nt * 16 + r;  // this lane's weight row (B column)
      const uint8_t* pw = w2 + ((size_t)e * H + n) * (I / 2);
      const uint8_t* ps = s2 + ((size_t)e * H + n) * (I / 32);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        wbuf[nt][b] = ld16(pw + b * 64 + g * 16);
        wsbuf[nt][b] = ps[b * 4 + g];
      }
    }
    // A: this lane's mid row (r0 + r), all blocks, widened to bf16
    const bool rv = r0 + r < r1;
    v8s A[NB][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint4 q0 = make_uint4(0, 0, 0, 0), q1 = make_uint4(0, 0, 0, 0);
      if (rv) {
        const uint8_t* pq = midq + (size_t)(r0 + r) * I + b * 128 + g * 32;
        q0 = ld16(pq);
        q1 = ld16(pq + 16);
      }
      A[b][0] = e4m3x8_to_bf16(q0.x, q0.y, tab);
      A[b][1] = e4m3x8_to_bf16(q0.z, q0.w, tab);
      A[b][2] = e4m3x8_to_bf16(q1.x, q1.y, tab);
      A[b][3] = e4m3x8_to_bf16(q1.z, q1.w, tab);
    }
    // mid scales and output rows of this lane's four D rows (4g + i)
    float sc[NB][4];
    int orow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * g + i;
      const bool v = r0 + m < r1;
      orow[i] = v ? sorted_entry[r0 + m] : -1;
#pragma unroll
      for (int b = 0; b < NB; ++b) sc[b][i] = v ? mids[(size_t)(r0 + m) * NB + b] : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint4 wb = wbuf[nt][b];
        const float wsc = e8m0_to_float(wsbuf[nt][b]);
        v4f P = {0.f, 0.f, 0.f, 0.f};
        P = mfma_bf16(A[b][0], fp4x8_to_bf16(wb.x, wsc), P);
        P = mfma_bf16(A[b][1], fp4x8_to_bf16(wb.y, wsc), P);
        P = mfma_bf16(A[b][2], fp4x8_to_bf16(wb.z, wsc), P);
        P = mfma_bf16(A[b][3], fp4x8_to_bf16(wb.w, wsc), P);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += (double)sc[b][i] * (double)P[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (orow[i] >= 0) y[(size_t)orow[i] * H + nc * 256 + wave * 64 + nt * 16 + r] = (float)acc[i];
    }
    if (FUSED) {
      if (threadIdx.x == 0) s_ndone = 0;
      __threadfence();
      __syncthreads();
      if (threadIdx.x < 16 && r0 + (int)threadIdx.x < r1) {
        const int t = sorted_entry[r0 + threadIdx.x] / k;
        if (atomicAdd(&cctr[(size_t)t * n_chunks + nc], 1u) == (uint32_t)(k - 1)) s_done[atomicAdd(&s_ndone, 1)] = t;
      }
      __syncthreads();
      const int nd = s_ndone;
      if (nd > 0) {
        __threadfence();
        for (int q = 0; q < nd; ++q) {
          const int t = s_done[q];
          combine_cols(y, topk_w, ys, t, k, H, nc * 256, 256, out);
          if (threadIdx.x == 0) cctr[(size_t)t * n_chunks + nc] = 0u;
        }
      }
      __syncthreads();
    }
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

hipError_t launch_down(const moe_plan* p, const CallArgs& a, Ev ev, bool fused) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t t16 = (n + std::min<int64_t>(p->s.E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows;
  const int H = (int)p->s.H;
  const int64_t work_max = t16 * (H / 256);
  const int blocks = (int)std::min<int64_t>(work_max, 4096);
  const float* ys = p->s.shared_I > 0 ? wsp<float>(p, p->L.sh_y) : nullptr;
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), wsp<float>(p, p->L.y), H, (int)p->s.top_k, wsp<float>(p, p->L.topk_w),
                    ys, wsp<uint32_t>(p, p->X.cctr), reinterpret_cast<uint16_t*>(a.out));
  };
  switch (p->s.I / 128) {
    case 1: return fused ? go(down_m16_kernel<1, true>) : go(down_m16_kernel<1, false>);
    case 2: return fused ? go(down_m16_kernel<2, true>) : go(down_m16_kernel<2, false>);
    case 3: return fused ? go(down_m16_kernel<3, true>) : go(down_m16_kernel<3, false>);
    case 4: return fused ? go(down_m16_kernel<4, true>) : go(down_m16_kernel<4, false>);
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
