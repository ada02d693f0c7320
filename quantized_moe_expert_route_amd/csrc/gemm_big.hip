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

// LDS layout of a K-step slice: 64-byte rows, and 16-byte chunk c of row R
// at R * 64 + 16 * (c ^ ((R >> 1) & 3)). With it both the staging stores
// (four lanes per row) and the fragment reads (sixteen rows, one chunk) hit
// no LDS bank twice (measured with the bank-conflict counter; rows padded to
// 80 bytes cost 4 conflict cycles per read and 8 per store).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
__device__ __forceinline__ int sw64(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 1) & 3)); }
constexpr int kGuStages = 2;  // K-steps of gate/up loads held in registers

// Item = (expert, kGuRows sorted rows, one 128-column mid block): the 256
// weight rows it reads (128 gate + 128 up) cover exactly the columns one mid
// block needs. A 64-row tile keeps a wave's registers within 256 so that two
// workgroups share a CU: one's MFMAs run while the other stages its next
// K-step and waits at its barrier (with one workgroup per CU those phases
// ran one after another).
constexpr int kGuR = kGuRows;

struct GuSmem {
  uint8_t a[2][kGuR * 64];    // x rows (MXFP4), K-step slice (sw64 layout)
  uint8_t b[2][256 * 64];     // 128 gate + 128 up weight rows
  uint32_t as[2][kGuR];       // 4 E8M0 bytes per row per K-step
  uint32_t bs[2][256];
};

// One K-step of global data held in registers: 1 + 4 16-byte chunks and the
// scale dwords of this thread.
struct GuRegs {
  uint4 a, b[4];
  uint32_t sa, sb;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gate_up_big_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ s13, const int* __restrict__ sorted_entry, const int4* __restrict__ items,
    const int* __restrict__ meta, int H, int I, int k, uint8_t* __restrict__ midq, float* __restrict__ mids) {
  __shared__ GuSmem sm;
  __shared__ int tok[kGuR];
  __shared__ float red[4][kGuR];  // row amax of the four column quarters
  // wave w multiplies all kGuR rows with gate columns 32 w .. + 32 and the
  // matching up columns
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave;
  const int r = lane & 15, g = lane >> 4;
  const size_t Hb = (size_t)H / 2, Hs = (size_t)H / 32;
  const int nk = H / 128;
  int first, stride, end;
  xcd_run(meta[1], first, stride, end);
  for (int it = first; it < end; it += stride) {
    const int4 item = items[it];
    const int e = item.x, r0 = item.y, r1 = item.z, ib = item.w;
    const int rows = r1 - r0;
    if (tid < kGuR) tok[tid] = tid < rows ? sorted_entry[r0 + tid] / k : -1;
    __syncthreads();
    auto wrow = [&](int rr) {
      return (size_t)e * 2 * I + (rr < 128 ? 128 * ib + rr : I + 128 * ib + rr - 128);
    };
    // This thread's global addresses do not change between K-steps. Every
    // load is unconditional (rows past the tile read row 0, whose results for
    // those rows are never written), so the number of loads in flight is the
    // same on every path and the waits before each store stay exact.
    const int tok0 = tok[0];
    const int ta = tok[tid >> 2];
    const uint8_t* pa = xq + (size_t)(ta >= 0 ? ta : tok0) * Hb + 16 * (tid & 3);
    // The expert's weights and their scales are read through buffer
    // descriptors (base and size in scalar registers, a 32-bit offset per
    // lane), which keeps the per-thread addresses out of vector registers.
    // Staged weight row (tid >> 2) + 64 q: gate rows for q < 2, up rows for
    // q >= 2; the row offsets per q are the same for every thread.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w13 + (size_t)e * 2 * I * Hb), (short)0, (int)(2 * I * Hb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s13 + (size_t)e * 2 * I * Hs), (short)0, (int)(2 * I * Hs), 0x00020000);
    const int ob = (128 * ib + (tid >> 2)) * (int)Hb + 16 * (tid & 3);
    const int boff[4] = {0, 64 * (int)Hb, (I - 128 + 128) * (int)Hb, (I - 128 + 192) * (int)Hb};
    const int os = (int)(wrow(tid) - (size_t)e * 2 * I) * (int)Hs;
    const int ts = tok[tid & (kGuR - 1)];
    const uint8_t* psa = xs + (size_t)(ts >= 0 ? ts : tok0) * Hs;
    auto load = [&](int kk, GuRegs& R) {
      R.a = ld16(pa + kk * 64);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rw, ob, boff[q] + kk * 64, 0);
        R.b[q] = make_uint4(v.x, v.y, v.z, v.w);
      }
      R.sa = ld4(psa + kk * 4);
      R.sb = __builtin_amdgcn_raw_buffer_load_b32(rs, os, kk * 4, 0);
    };
    auto store = [&](const GuRegs& R, int s) {
      *reinterpret_cast<uint4*>(&sm.a[s][sw64(tid >> 2, tid & 3)]) = R.a;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int idx = tid + 256 * q;
        *reinterpret_cast<uint4*>(&sm.b[s][sw64(idx >> 2, idx & 3)]) = R.b[q];
      }
      if (tid < kGuR) sm.as[s][tid] = R.sa;
      sm.bs[s][tid] = R.sb;
    };
    v4f accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        accg[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        accu[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    auto compute = [&](int s) {
      uint4 fa[4];
      uint32_t sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + r;
        fa[i] = *reinterpret_cast<const uint4*>(&sm.a[s][sw64(row, g)]);
        sa[i] = (sm.as[s][row] >> (8 * g)) & 0xFFu;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = 32 * wn + 16 * j + r;
        const uint4 fg = *reinterpret_cast<const uint4*>(&sm.b[s][sw64(col, g)]);
        const uint4 fu = *reinterpret_cast<const uint4*>(&sm.b[s][sw64(col + 128, g)]);
        const uint32_t sg = (sm.bs[s][col] >> (8 * g)) & 0xFFu;
        const uint32_t su = (sm.bs[s][col + 128] >> (8 * g)) & 0xFFu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[i][j] = mfma_fp4(fa[i], fg, accg[i][j], sa[i], sg);
          accu[i][j] = mfma_fp4(fa[i], fu, accu[i][j], sa[i], su);
        }
      }
    };
    // K-steps kk+1..kk+kGuStages are in flight while kk is multiplied: step
    // kk's registers are refilled with step kk+kGuStages right after they
    // were stored. Past the last step the loads repeat it and the stores fill
    // a buffer nobody reads; only the MFMA work is skipped.
    GuRegs S[kGuStages];
#pragma unroll
    for (int q = 0; q < kGuStages; ++q) load(min(q, nk - 1), S[q]);
    store(S[0], 0);
    barrier_lds();
    for (int kk = 0; kk < nk; kk += kGuStages) {
#pragma unroll
      for (int q = 0; q < kGuStages; ++q) {
        load(min(kk + q + kGuStages, nk - 1), S[q]);
        if (kk + q < nk) compute((kk + q) & 1);
        store(S[(q + 1) % kGuStages], (kk + q + 1) & 1);
        barrier_lds();
      }
    }
    // ---- epilogue: h = SiLU(g) * u (float64, one rounding), row amax over
    // the item's 128 columns, s = amax / 448, q = E4M3(h / s). Its lane
    // indices come from an opaque zero, so the compiler computes its
    // addresses here rather than before the item loop (where they would stay
    // live through the K-loop and crowd it out of registers).
    const int lz = (int)(threadIdx.x & 63) + opaque_zero();
    const int re = lz & 15, ge = lz >> 4;
    // (rows past the tile's end are skipped: a quarter-wave's four rows are
    // uniform per (i, v), so a wave whose rows are all padding branches over)
    float hv[4][2][4];
    float pm[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float m = 0.f;
        const bool live = 16 * i + 4 * ge + v < rows;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          hv[i][j][v] = live ? silu_mul(accg[i][j][v], accu[i][j][v]) : 0.f;
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
        if (re == 0) red[wn][16 * i + 4 * ge + v] = __uint_as_float(u);
      }
    __syncthreads();  // also: every wave is past its last read of the staging buffers
    uint8_t* qs = reinterpret_cast<uint8_t*>(&sm.a);  // [kGuR][128] codes, in the idle A buffers
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * i + 4 * ge + v;
        const float amax = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
        const float sc = __fdiv_rn(amax, 448.0f);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t c = sc > 0.f && row < rows ? e4m3_code(__fdiv_rn(hv[i][j][v], sc)) : 0u;
          qs[row * 128 + 32 * wn + 16 * j + re] = (uint8_t)c;
        }
        if (wn == 0 && re == 0 && row < rows) mids[(size_t)(r0 + row) * (I / 128) + ib] = sc;
      }
    __syncthreads();
    // coalesced copy of the item's codes: kGuR rows x 128 bytes
#pragma unroll
    for (int q = 0; q < kGuR * 8 / 256; ++q) {
      const int idx = tid + 256 * q, row = idx >> 3, c = idx & 7;
      if (row < rows)
        *reinterpret_cast<uint4*>(midq + (size_t)(r0 + row) * I + 128 * ib + 16 * c) =
            *reinterpret_cast<const uint4*>(&qs[row * 128 + 16 * c]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down
// Item = (expert, 128 sorted rows, kDnItemCols output columns). The tile's
// E4M3 mid bytes go to LDS once per item; the weights stream through
// kDnItemCols/128 column sub-tiles x I/128 mid blocks, three steps in flight.
// Per step the E4M3 values and the E2M1 * 2^scale weights are widened to
// bf16 when a wave reads them (both exact) and 4 bf16 MFMAs of K = 32 give
// the 128-block's fp32 partial (exact while the sum fits binary32); it is
// scaled by the row's mid scale in float64 and the blocks are summed in order.
constexpr int kDnItemCols = kDownItemCols;
constexpr int kLDM = 16;   // pad bytes per LDS mid row
constexpr int kLDW = 80;   // LDS bytes per weight column slice (64 + 16 pad)

template <int NB>
struct DnSmem {
  uint8_t a[kBM * (NB * 128 + kLDM)];   // mid rows, E4M3
  uint8_t b[2][kDownCols * kLDW];        // weight column slices of one mid block
  uint32_t bs[2][kDownCols];             // 4 E8M0 bytes per column per block
  float ms[NB][kBM];                     // mid scales
  int ent[kBM];
};

struct DnRegs {
  uint4 b[2];
  uint32_t s;
};

template <int NB>
__global__ __launch_bounds__(256) void down_big_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry, const int4* __restrict__ items,
    const int* __restrict__ meta, float* __restrict__ y, int H) {
  constexpr int I = NB * 128;
  constexpr int LDA = I + kLDM;
  constexpr int NSUB = kDnItemCols / kDownCols;  // column sub-tiles per item
  constexpr int NSTEP = NSUB * NB;               // (sub-tile, block) steps per item
  __shared__ DnSmem<NB> sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  int first, stride, end;
  xcd_run(meta[2], first, stride, end);
  for (int it = first; it < end; it += stride) {
    const int4 item = items[it];
    const int e = item.x, r0 = item.y, r1 = item.z, c0 = item.w * kDnItemCols;
    const int rows = r1 - r0;
    // weight addresses of this thread (2 chunks of a 64-byte block slice, 1 scale dword)
    const uint8_t* pw[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int idx = tid + 256 * q;
      pw[q] = w2 + ((size_t)e * H + c0 + (idx >> 2)) * (I / 2) + 16 * (idx & 3);
    }
    const uint8_t* psw = s2 + ((size_t)e * H + c0 + (tid & (kDownCols - 1))) * (I / 32);
    // step st = (sub-tile st / NB, block st % NB); the step past the last
    // repeats it (loaded, stored to an unread buffer, not multiplied)
    auto load = [&](int st, DnRegs& R) {
      st = min(st, NSTEP - 1);
      const int sub = st / NB, b = st - sub * NB;
      const size_t coff = (size_t)sub * kDownCols * (I / 2) + 64 * b;
#pragma unroll
      for (int q = 0; q < 2; ++q) R.b[q] = ld16(pw[q] + coff);
      R.s = ld4(psw + (size_t)sub * kDownCols * (I / 32) + 4 * b);
    };
    auto store = [&](const DnRegs& R, int sb) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q;
        *reinterpret_cast<uint4*>(&sm.b[sb][(idx >> 2) * kLDW + 16 * (idx & 3)]) = R.b[q];
      }
      if (tid < kDownCols) sm.bs[sb][tid] = R.s;
    };
    DnRegs S0, S1, S2;
    load(0, S0);
    load(1, S1);
    load(2, S2);
    // the tile's mid rows and scales, once per item
    if (tid < kBM) {
      sm.ent[tid] = tid < rows ? sorted_entry[r0 + tid] : -1;
#pragma unroll
      for (int b = 0; b < NB; ++b) sm.ms[b][tid] = tid < rows ? mids[(size_t)(r0 + tid) * NB + b] : 0.f;
    }
    for (int idx = tid; idx < kBM * (I / 16); idx += 256) {
      const int row = idx / (I / 16), c = idx - row * (I / 16);
      const uint4 v = row < rows ? ld16(midq + (size_t)(r0 + row) * I + 16 * c) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&sm.a[row * LDA + 16 * c]) = v;
    }
    store(S0, 0);
    __syncthreads();
    double acc[4][4][4];
    v4f P[4][4];
    auto compute = [&](int st, int sb) {
      const int sub = st / NB, b = st - sub * NB;
      if (b == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) P[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // K = 32 chunks; lane group g holds K 32q + 8g ..
        v8s fa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 64 * wm + 16 * i + r;
          const uint2 raw = *reinterpret_cast<const uint2*>(&sm.a[row * LDA + 128 * b + 32 * q + 8 * g]);
          const uint32_t d0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, false));
          const uint32_t d1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, 1.0f, true));
          const uint32_t d2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, false));
          const uint32_t d3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, 1.0f, true));
          fa[i][0] = (short)(d0 & 0xFFFF); fa[i][1] = (short)(d0 >> 16);
          fa[i][2] = (short)(d1 & 0xFFFF); fa[i][3] = (short)(d1 >> 16);
          fa[i][4] = (short)(d2 & 0xFFFF); fa[i][5] = (short)(d2 >> 16);
          fa[i][6] = (short)(d3 & 0xFFFF); fa[i][7] = (short)(d3 >> 16);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = 64 * wn + 16 * j + r;
          const uint32_t wv = *reinterpret_cast<const uint32_t*>(&sm.b[sb][col * kLDW + 16 * q + 4 * g]);
          const float wsc = e8m0_to_float((sm.bs[sb][col] >> (8 * q)) & 0xFFu);
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
      if (b == NB - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int en = sm.ent[64 * wm + 16 * i + 4 * g + v];
            if (en >= 0) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                y[(size_t)en * H + c0 + sub * kDownCols + 64 * wn + 16 * j + r] = (float)acc[i][j][v];
            }
          }
      }
    };
    auto iter = [&](int st, DnRegs& cur, DnRegs& nxt) {
      load(st + 3, cur);
      if (st < NSTEP) compute(st, st & 1);
      store(nxt, (st + 1) & 1);
      barrier_lds();
    };
    for (int st = 0; st < NSTEP; st += 3) {
      iter(st, S0, S1);
      iter(st + 1, S1, S2);
      iter(st + 2, S2, S0);
    }
    __syncthreads();
  }
}

hipError_t launch_gate_up_big(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = (n + std::min<int64_t>(p->s.E, n) * (kGuR - 1) + kGuR - 1) / kGuR;
  const int64_t items = tiles * (p->s.I / 128);
  const int blocks = (int)std::min<int64_t>(items, 512);  // two per CU
  return launch_k(gate_up_big_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.xq),
                  wsp<uint8_t>(p, p->L.xs), reinterpret_cast<const uint8_t*>(a.w13),
                  reinterpret_cast<const uint8_t*>(a.s13), wsp<int>(p, p->L.sorted_entry),
                  wsp<int4>(p, p->X.gu_items), wsp<int>(p, p->X.meta), (int)p->s.H, (int)p->s.I,
                  (int)p->s.top_k, wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids));
}


hipError_t launch_down_big(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = (n + std::min<int64_t>(p->s.E, n) * (kBM - 1) + kBM - 1) / kBM;
  const int64_t items = tiles * (p->s.H / kDnItemCols);
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
