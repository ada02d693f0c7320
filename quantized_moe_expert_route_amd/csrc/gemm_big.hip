// Large-token gate/up and down grouped GEMMs: LDS-staged 128-row tiles.
//
// gate/up (scaled FP4 MFMA, "IQ2R: load GLM-5.3 packed MoE checkpoints
// ...", Summary: SiLU activation; the pages' MXFP4 A4W4 arm) with SiLU(gate) *
// up and the per-128 E4M3 mid quantization ("glm53: FP8 mid hand-off ...",
// Modifications row "mid as FP8 once") done inside the workgroup: a work item
// is (expert, 128 sorted rows, one 128-column mid block), so the 256 weight
// rows it reads (128 gate + 128 up) cover exactly the columns one mid block
// needs and no other workgroup is involved.
//
// Items come ordered (expert, column block, row tile) and the grid walks them
// in contiguous runs per XCD (workgroup b runs on XCD b mod 8), so the row
// tiles that share a weight block run together on one XCD and read it from
// that XCD's L2 after the first fetch from HBM.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

constexpr int kBM = kBigRows;  // 128 sorted rows per tile
constexpr int kLD = 80;        // LDS bytes per row of a 64-byte K-step slice (+16 pad)

struct GuSmem {
  uint8_t a[2][kBM * kLD];      // x rows (MXFP4), K-step slice
  uint8_t b[2][256 * kLD];      // 128 gate + 128 up weight rows
  uint32_t as[2][kBM];          // 4 E8M0 bytes per row per K-step
  uint32_t bs[2][256];
  int tok[kBM];
  float red[2][kBM];            // row amax of the two column halves
};

// Item order inside an XCD-contiguous run: workgroup b handles items
// first(b), first(b) + stride, ... of the run of its XCD.
__device__ __forceinline__ void xcd_run(int n_items, int& first, int& stride, int& end) {
  const int G = gridDim.x;
  const int x = blockIdx.x & 7, l = blockIdx.x >> 3;
  const int per_x = (G + 7 - x) >> 3;           // workgroups on this XCD
  const int run = (n_items + 7) >> 3;           // items per XCD
  first = x * run + l;
  stride = per_x;
  end = min(n_items, (x + 1) * run);
}

__global__ __launch_bounds__(256) void gate_up_big_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ s13, const int* __restrict__ sorted_entry, const int4* __restrict__ items,
    const int* __restrict__ meta, int H, int I, int k, uint8_t* __restrict__ midq, float* __restrict__ mids) {
  __shared__ GuSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const size_t Hb = (size_t)H / 2, Hs = (size_t)H / 32;
  const int nk = H / 128;
  int first, stride, end;
  xcd_run(meta[1], first, stride, end);
  for (int it = first; it < end; it += stride) {
    const int4 item = items[it];
    const int e = item.x, r0 = item.y, r1 = item.z, ib = item.w;
    const int rows = r1 - r0;
    if (tid < kBM) sm.tok[tid] = tid < rows ? sorted_entry[r0 + tid] / k : -1;
    __syncthreads();
    // global -> register staging of one K-step: A 2 chunks, B 4 chunks, 1 scale dword each
    uint4 ra[2], rb[4];
    uint32_t rsa = 0x7F7F7F7Fu, rsb = 0;
    auto load = [&](int kk) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q, row = idx >> 2, c = idx & 3;
        const int t = sm.tok[row];
        ra[q] = t >= 0 ? ld16(xq + (size_t)t * Hb + kk * 64 + 16 * c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q, rr = idx >> 2, c = idx & 3;
        const size_t wrow = (size_t)e * 2 * I + (rr < 128 ? 128 * ib + rr : I + 128 * ib + rr - 128);
        rb[q] = ld16(w13 + wrow * Hb + kk * 64 + 16 * c);
      }
      if (tid < kBM) {
        const int t = sm.tok[tid];
        rsa = t >= 0 ? ld4(xs + (size_t)t * Hs + kk * 4) : 0x7F7F7F7Fu;
      }
      {
        const size_t wrow = (size_t)e * 2 * I + (tid < 128 ? 128 * ib + tid : I + 128 * ib + tid - 128);
        rsb = ld4(s13 + wrow * Hs + kk * 4);
      }
    };
    auto store = [&](int s) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q;
        *reinterpret_cast<uint4*>(&sm.a[s][(idx >> 2) * kLD + 16 * (idx & 3)]) = ra[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q;
        *reinterpret_cast<uint4*>(&sm.b[s][(idx >> 2) * kLD + 16 * (idx & 3)]) = rb[q];
      }
      if (tid < kBM) sm.as[s][tid] = rsa;
      sm.bs[s][tid] = rsb;
    };
    v4f accg[4][4], accu[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        accg[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        accu[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    load(0);
    store(0);
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
      const int s = kk & 1;
      if (kk + 1 < nk) load(kk + 1);
      uint4 fa[4];
      uint32_t sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 64 * wm + 16 * i + r;
        fa[i] = *reinterpret_cast<const uint4*>(&sm.a[s][row * kLD + 16 * g]);
        sa[i] = (sm.as[s][row] >> (8 * g)) & 0xFFu;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 64 * wn + 16 * j + r;
        const uint4 fg = *reinterpret_cast<const uint4*>(&sm.b[s][col * kLD + 16 * g]);
        const uint4 fu = *reinterpret_cast<const uint4*>(&sm.b[s][(col + 128) * kLD + 16 * g]);
        const uint32_t sg = (sm.bs[s][col] >> (8 * g)) & 0xFFu;
        const uint32_t su = (sm.bs[s][col + 128] >> (8 * g)) & 0xFFu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[i][j] = mfma_fp4(fa[i], fg, accg[i][j], sa[i], sg);
          accu[i][j] = mfma_fp4(fa[i], fu, accu[i][j], sa[i], su);
        }
      }
      if (kk + 1 < nk) store(s ^ 1);
      __syncthreads();
    }
    // ---- epilogue: h = SiLU(g) * u (float64, one rounding), row amax over
    // the item's 128 columns, s = amax / 448, q = E4M3(h / s)
    float hv[4][4][4];
    float pm[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hv[i][j][v] = silu_mul(accg[i][j][v], accu[i][j][v]);
          m = fmaxf(m, fabsf(hv[i][j][v]));
        }
        pm[i][v] = m;
      }
    // max over the 16 lanes of a row group (lanes 16g..16g+15 share rows)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint32_t u = __float_as_uint(pm[i][v]);  // non-negative: bit order = value order
        u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));
        u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));
        u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));
        u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));
        if (r == 0) sm.red[wn][64 * wm + 16 * i + 4 * g + v] = __uint_as_float(u);
      }
    __syncthreads();
    uint8_t* qs = reinterpret_cast<uint8_t*>(&sm.a);  // [128][128] codes, in the (now idle) A buffers
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 64 * wm + 16 * i + 4 * g + v;
        const float amax = fmaxf(sm.red[0][row], sm.red[1][row]);
        const float sc = __fdiv_rn(amax, 448.0f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t c = sc > 0.f ? e4m3_code(__fdiv_rn(hv[i][j][v], sc)) : 0u;
          qs[row * 128 + 64 * wn + 16 * j + r] = (uint8_t)c;
        }
        if (wn == 0 && r == 0 && row < rows) mids[(size_t)(r0 + row) * (I / 128) + ib] = sc;
      }
    __syncthreads();
    // coalesced copy of the item's codes: 128 rows x 128 bytes
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + 256 * q, row = idx >> 3, c = idx & 7;
      if (row < rows)
        *reinterpret_cast<uint4*>(midq + (size_t)(r0 + row) * I + 128 * ib + 16 * c) =
            *reinterpret_cast<const uint4*>(&qs[row * 128 + 16 * c]);
    }
    __syncthreads();
  }
}


// ---------------------------------------------------------------- down
// Item = (expert, 128 sorted rows, 128 output columns). Per mid block b
// (128 K): the rows' E4M3 bytes are widened to bf16 while staged in LDS
// (exact), the weights' E2M1 nibbles are widened with their E8M0 scale when a
// wave reads them (exact), and 4 bf16 MFMAs of K = 32 give the block's fp32
// partial, which is exact while the block sum fits binary32; the partial is
// scaled by the row's mid scale in float64 and the blocks are summed in order.
constexpr int kLDA16 = 136;  // bf16 elements per LDS row of a 128-K block (+8 pad)
constexpr int kLDB = 80;     // bytes per LDS row of a weight column's 64-byte block slice

struct DnSmem {
  uint16_t a[2][kBM * kLDA16];   // mid rows as bf16
  uint8_t b[2][kDownCols * kLDB];
  uint32_t bs[2][kDownCols];     // 4 E8M0 bytes per column per block
  float ms[4][kBM];              // mid scales, per block (I <= 512)
  int ent[kBM];
};

template <int NB>
__global__ __launch_bounds__(256) void down_big_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry, const int4* __restrict__ items,
    const int* __restrict__ meta, float* __restrict__ y, int H) {
  constexpr int I = NB * 128;
  __shared__ DnSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  int first, stride, end;
  xcd_run(meta[2], first, stride, end);
  for (int it = first; it < end; it += stride) {
    const int4 item = items[it];
    const int e = item.x, r0 = item.y, r1 = item.z, nc = item.w;
    const int rows = r1 - r0;
    if (tid < kBM) {
      sm.ent[tid] = tid < rows ? sorted_entry[r0 + tid] : -1;
#pragma unroll
      for (int b = 0; b < NB; ++b) sm.ms[b][tid] = tid < rows ? mids[(size_t)(r0 + tid) * NB + b] : 0.f;
    }
    uint4 ra[4], rb[2];
    uint32_t rsb = 0;
    auto load = [&](int b) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q, row = idx >> 3, c = idx & 7;
        ra[q] = row < rows ? ld16(midq + (size_t)(r0 + row) * I + 128 * b + 16 * c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q, col = idx >> 2, c = idx & 3;
        const size_t wrow = (size_t)e * H + (size_t)nc * kDownCols + col;
        rb[q] = ld16(w2 + wrow * (I / 2) + 64 * b + 16 * c);
      }
      if (tid < kDownCols) rsb = ld4(s2 + ((size_t)e * H + (size_t)nc * kDownCols + tid) * (I / 32) + 4 * b);
    };
    auto store = [&](int s) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q, row = idx >> 3, c = idx & 7;
        const uint32_t w[4] = {ra[q].x, ra[q].y, ra[q].z, ra[q].w};
        uint32_t o[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          o[2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], 1.0f, false));
          o[2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[d], 1.0f, true));
        }
        uint4* dst = reinterpret_cast<uint4*>(&sm.a[s][row * kLDA16 + 16 * c]);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q;
        *reinterpret_cast<uint4*>(&sm.b[s][(idx >> 2) * kLDB + 16 * (idx & 3)]) = rb[q];
      }
      if (tid < kDownCols) sm.bs[s][tid] = rsb;
    };
    double acc[4][4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
    __syncthreads();  // ent / ms visible
    load(0);
    store(0);
    __syncthreads();
    for (int b = 0; b < NB; ++b) {
      const int s = b & 1;
      if (b + 1 < NB) load(b + 1);
      v4f P[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) P[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // K = 32 chunks of the block; lane group g: K 32q + 8g ..
        v8s fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 64 * wm + 16 * i + r;
          fa[i] = *reinterpret_cast<const v8s*>(&sm.a[s][row * kLDA16 + 32 * q + 8 * g]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = 64 * wn + 16 * j + r;
          const uint32_t wv = *reinterpret_cast<const uint32_t*>(&sm.b[s][col * kLDB + 16 * q + 4 * g]);
          const float wsc = e8m0_to_float((sm.bs[s][col] >> (8 * q)) & 0xFFu);
          const uint32_t d0 = cvt_fp4x2_bf16<0>(wv, wsc), d1 = cvt_fp4x2_bf16<1>(wv, wsc);
          const uint32_t d2 = cvt_fp4x2_bf16<2>(wv, wsc), d3 = cvt_fp4x2_bf16<3>(wv, wsc);
          v8s fb;
          fb[0] = (short)(d0 & 0xFFFF); fb[1] = (short)(d0 >> 16);
          fb[2] = (short)(d1 & 0xFFFF); fb[3] = (short)(d1 >> 16);
          fb[4] = (short)(d2 & 0xFFFF); fb[5] = (short)(d2 >> 16);
          fb[6] = (short)(d3 & 0xFFFF); fb[7] = (short)(d3 >> 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) P[i][j] = mfma_bf16(fa[i], fb, P[i][j]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double sc = (double)sm.ms[b][64 * wm + 16 * i + 4 * g + v];
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j][v] += sc * (double)P[i][j][v];
        }
      if (b + 1 < NB) store(s ^ 1);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 64 * wm + 16 * i + 4 * g + v;
        const int en = sm.ent[row];
        if (en >= 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            y[(size_t)en * H + (size_t)nc * kDownCols + 64 * wn + 16 * j + r] = (float)acc[i][j][v];
        }
      }
    __syncthreads();
  }
}

hipError_t launch_gate_up_big(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = (n + std::min<int64_t>(p->s.E, n) * (kBM - 1) + kBM - 1) / kBM;
  const int64_t items = tiles * (p->s.I / 128);
  const int blocks = (int)std::min<int64_t>(items, 256);
  return launch_k(gate_up_big_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.xq),
                  wsp<uint8_t>(p, p->L.xs), reinterpret_cast<const uint8_t*>(a.w13),
                  reinterpret_cast<const uint8_t*>(a.s13), wsp<int>(p, p->L.sorted_entry),
                  wsp<int4>(p, p->X.gu_items), wsp<int>(p, p->X.meta), (int)p->s.H, (int)p->s.I,
                  (int)p->s.top_k, wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids));
}


hipError_t launch_down_big(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = (n + std::min<int64_t>(p->s.E, n) * (kBM - 1) + kBM - 1) / kBM;
  const int64_t items = tiles * (p->s.H / kDownCols);
  const int blocks = (int)std::min<int64_t>(items, 256);
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry),
                    wsp<int4>(p, p->X.dn_items), wsp<int>(p, p->X.meta), wsp<float>(p, p->L.y), (int)p->s.H);
  };
  switch (p->s.I / 128) {
    case 1: return go(down_big_kernel<1>);
    case 2: return go(down_big_kernel<2>);
    case 3: return go(down_big_kernel<3>);
    case 4: return go(down_big_kernel<4>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
