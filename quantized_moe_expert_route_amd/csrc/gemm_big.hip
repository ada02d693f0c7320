// Large-token gate/up and down grouped GEMMs (tiles of 64 and 32 sorted rows).
//
// gate/up (scaled FP4 MFMA, "IQ2R: load GLM-5.3 packed MoE checkpoints
// ...", Summary: SiLU activation; the pages' MXFP4 A4W4 arm) with SiLU(gate) *
// up and the per-128 E4M3 mid quantization ("glm53: FP8 mid hand-off ...",
// Modifications row "mid as FP8 once") done inside the workgroup: a work item
// is (expert, 64 sorted rows, one 128-column mid block), so the 256 weight
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
#include <type_traits>

namespace qmoe {



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
// at R * 64 + 16 * (c ^ ((R >> 2) & 3)). A 16-byte access of 16 lanes is
// served by the 64 banks (256 bytes) together; here both the staging stores
// of x (four lanes per row) and of the packed weights (sixteen rows, one
// chunk) and the fragment reads (sixteen rows, one chunk) put 16 lanes on 16
// different 16-byte bank groups: rows R and R + 4 k differ in the XOR, rows
// within 4 in the bank group of R * 64. (XOR with (R >> 1) & 3, which
// separates only 8 rows, stalled the kernel about half its time on bank
// conflicts.)
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
__device__ __forceinline__ int sw64(int row, int chunk) { return row * 64 + 16 * (chunk ^ ((row >> 2) & 3)); }

// Item = (expert, kGuRows sorted rows, one 128-column mid block): the 256
// weight rows it reads (128 gate + 128 up) cover exactly the columns one mid
// block needs. A 64-row tile keeps a wave's registers within 256 so that two
// workgroups share a CU: one's MFMAs run while the other waits at its
// barrier.
constexpr int kGuR = kGuRows;

// x scales: a load whose lanes read 4 bytes from each of 64 rows costs the
// memory pipeline about four times one that reads 16 bytes from each of 16
// rows, so the x scales of the tile's rows (192 bytes a row at H = 6144)
// come once per item, row by row, into LDS. (The weight scales come packed:
// one dword a lane per fragment and 512-wide stage.)
constexpr int kGuXsSteps = 48;  // K-steps of x scales staged at a time (all of them up to H = 6144)
constexpr int kGuXsLd = 13;     // 16-byte chunks per staged x-scale row (12 used; 13 keeps reads conflict-free)

struct alignas(16) GuSmem {  // 16-byte aligned: staging and fragment accesses compile to single b128 LDS ops
  uint8_t a[2][kGuR * 64];         // x rows (MXFP4), K-step slice (sw64 layout)
  uint32_t xs[kGuR][4 * kGuXsLd];  // x scales of kGuXsSteps K-steps, 4 E8M0 bytes per K-step
};
constexpr int kGuBD = 2;  // K-steps of a wave's weight fragments held in registers (divides 8)

// MX: the mid leaves as MXFP4 (per 32 columns an E8M0 scale and E2M1 codes,
// the rule x takes), midq [n, I/2], mids bytes [n, I/32]; else E4M3 per 128.
template <bool MX>
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
    // The expert's packed weights (moe_pack_w13) and their scales are read
    // through buffer descriptors (base and size in scalar registers, a
    // 32-bit offset per lane), which keeps the per-thread addresses out of
    // vector registers. A K-step of a 16-row block is 1 KB in MFMA lane
    // order (lane l: row l & 15, MX block l >> 4), so each wave loads its own
    // four fragments straight into registers, one 1 KB load each: gate row
    // blocks 2 wn, 2 wn + 1 of the item and the matching up blocks. An
    // expert's packed bytes start where its rows did; row block b of the
    // expert at 16 b Hb, its scales at b * (H / 512) * 256.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w13 + (size_t)e * 2 * I * Hb), (short)0, (int)(2 * I * Hb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s13 + (size_t)e * 2 * I * Hs), (short)0, (int)(2 * I * Hs), 0x00020000);
    const int ns = nk / 4;  // 512-wide stages
    const int rbg = 8 * ib + 2 * wn, rbu = I / 16 + rbg;
    const int fo[4] = {rbg * 16 * (int)Hb + 16 * lane, (rbg + 1) * 16 * (int)Hb + 16 * lane,
                       rbu * 16 * (int)Hb + 16 * lane, (rbu + 1) * 16 * (int)Hb + 16 * lane};
    const int so[4] = {rbg * ns * 256 + 4 * lane, (rbg + 1) * ns * 256 + 4 * lane, rbu * ns * 256 + 4 * lane,
                       (rbu + 1) * ns * 256 + 4 * lane};
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    auto load_b = [&](int kk, uint4 (&B)[4]) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rw, fo[f], kk * 1024, 0);
        B[f] = make_uint4(v.x, v.y, v.z, v.w);
      }
    };
    // the four K-steps of stage st of each fragment: byte j of lane l's dword
    auto load_sb = [&](int st, uint32_t (&S)[4]) {
#pragma unroll
      for (int f = 0; f < 4; ++f) S[f] = __builtin_amdgcn_raw_buffer_load_b32(rs, so[f], 256 * st, 0);
    };
    v4f accg[4][2], accu[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        accg[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        accu[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    // x rows of K-step kk from LDS buffer kk & 1, the wave's weights from registers
    auto compute = [&](int kk, const uint4 (&B)[4], const uint32_t (&S)[4]) {
      const int s = kk & 1, q4 = kk & 3;
      uint4 fa[4];
      uint32_t sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + r;
        fa[i] = *reinterpret_cast<const uint4*>(&sm.a[s][sw64(row, g)]);
        sa[i] = (sm.xs[row][kk % kGuXsSteps] >> (8 * g)) & 0xFFu;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t sg = (S[j] >> (8 * q4)) & 0xFFu;
        const uint32_t su = (S[2 + j] >> (8 * q4)) & 0xFFu;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          accg[i][j] = mfma_fp4(fa[i], B[j], accg[i][j], sa[i], sg);
          accu[i][j] = mfma_fp4(fa[i], B[2 + j], accu[i][j], sa[i], su);
        }
      }
    };
    // the tile's x scales of K-steps kGuXsSteps m .. (one row of 16-byte
    // chunks per token, read row by row)
    auto stage_xs = [&](int m) {
      const int nxc = min(kGuXsSteps, nk - kGuXsSteps * m) / 4;  // 16-byte chunks per row
      for (int idx = tid; idx < kGuR * nxc; idx += 256) {
        const int row = idx / nxc, c = idx - row * nxc;
        const int t = tok[row];
        *reinterpret_cast<uint4*>(&sm.xs[row][4 * c]) =
            ld16(xs + (size_t)(t >= 0 ? t : tok0) * Hs + kGuXsSteps * 4 * m + 16 * c);
      }
    };
    // Pipeline: x rows go global -> registers (two K-steps ahead) -> LDS
    // (double buffer, one barrier per K-step); the weights go global ->
    // registers kGuBD K-steps ahead and their scales a stage ahead. Loads
    // past the last step repeat it; only the MFMA work is skipped.
    uint4 Bq[kGuBD][4];
    uint32_t Sb[2][4];
    uint4 Sa[2];
    stage_xs(0);
    Sa[0] = ld16(pa);
    Sa[1] = ld16(pa + min(1, nk - 1) * 64);
#pragma unroll
    for (int d = 0; d < kGuBD; ++d) load_b(min(d, nk - 1), Bq[d]);
    load_sb(0, Sb[0]);
    *reinterpret_cast<uint4*>(&sm.a[0][sw64(tid >> 2, tid & 3)]) = Sa[0];
    barrier_lds();
    // unrolled by two stages, so every ring index is a constant
    for (int kk = 0; kk < nk; kk += 8) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = kk + q;
        if (q % 4 == 0) load_sb(min(k / 4 + 1, ns - 1), Sb[(q / 4 + 1) & 1]);  // the next stage's scales
        Sa[q & 1] = ld16(pa + min(k + 2, nk - 1) * 64);
        if (k < nk) {
          if (k > 0 && k % kGuXsSteps == 0) {  // only when H > 6144
            stage_xs(k / kGuXsSteps);  // every wave is past the previous step's barrier
            barrier_lds();
          }
          compute(k, Bq[q % kGuBD], Sb[(q / 4) & 1]);
        }
        load_b(min(k + kGuBD, nk - 1), Bq[q % kGuBD]);
        *reinterpret_cast<uint4*>(&sm.a[(q + 1) & 1][sw64(tid >> 2, tid & 3)]) = Sa[(q + 1) & 1];
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
        if (MX) pm[i][v] = __uint_as_float(u);  // the amax of the row's 32 columns of this wave
        else if (re == 0) red[wn][16 * i + 4 * ge + v] = __uint_as_float(u);
      }
    __syncthreads();  // also: every wave is past its last read of the staging buffers
    uint8_t* qs = reinterpret_cast<uint8_t*>(&sm.a);  // [kGuR][128] codes, in the idle A buffers
    if (MX) {
      // a wave's 32 columns are one MX block of each row: scale byte from
      // the amax's exponent, codes E2M1(h * 2^(127 - s)), one a byte in qs
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * i + 4 * ge + v;
          const uint32_t sc = mx_scale_code_f32(__float_as_uint(pm[i][v]));
          const int sh = 127 - (int)sc;
          const uint32_t cp = row < rows ? e2m1_pack2(ldexpf(hv[i][0][v], sh), ldexpf(hv[i][1][v], sh)) : 0u;
          qs[row * 128 + 32 * wn + re] = (uint8_t)(cp & 15u);
          qs[row * 128 + 32 * wn + 16 + re] = (uint8_t)(cp >> 4);
          if (re == 0 && row < rows)
            reinterpret_cast<uint8_t*>(mids)[(size_t)(r0 + row) * (I / 32) + 4 * ib + wn] = (uint8_t)sc;
        }
      __syncthreads();
      // coalesced copy: kGuR rows x 64 bytes, element 2i in the low nibble
      {
        const int row = tid >> 2, c = tid & 3;  // 16 bytes (32 codes) a thread
        if (row < rows) {
          const uint4 a = *reinterpret_cast<const uint4*>(&qs[row * 128 + 32 * c]);
          const uint4 b = *reinterpret_cast<const uint4*>(&qs[row * 128 + 32 * c + 16]);
          const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w0 = wv[2 * q], w1 = wv[2 * q + 1];
            o[q] = (w0 & 0xFu) | ((w0 >> 4) & 0xF0u) | ((w0 >> 8) & 0xF00u) | ((w0 >> 12) & 0xF000u) |
                   ((w1 & 0xFu) << 16) | ((w1 << 12) & 0xF00000u) | ((w1 << 8) & 0xF000000u) | ((w1 << 4) & 0xF0000000u);
          }
          *reinterpret_cast<uint4*>(midq + (size_t)(r0 + row) * (I / 2) + 64 * ib + 16 * c) =
              make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
      __syncthreads();
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * i + 4 * ge + v;
        const float amax = fmaxf(fmaxf(red[0][row], red[1][row]), fmaxf(red[2][row], red[3][row]));
        const float sc = __fdiv_rn(amax, 448.0f);
        const uint32_t c01 =
            sc > 0.f && row < rows ? e4m3_pack2(__fdiv_rn(hv[i][0][v], sc), __fdiv_rn(hv[i][1][v], sc)) : 0u;
        qs[row * 128 + 32 * wn + re] = (uint8_t)c01;
        qs[row * 128 + 32 * wn + 16 + re] = (uint8_t)(c01 >> 8);
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
// Item = (expert, tile of up to kDnRows sorted rows, kDnItemCols output
// columns); a workgroup takes one item at a time and two workgroups share a
// CU. At the start of an item the tile's E4M3 mid rows, fetched into
// registers during the previous item, are widened to bf16 (exactly) into
// LDS. Wave w then covers all the tile's rows x 64 columns, one 128-block per
// step. The item's 256 w2 rows are contiguous; they are read in halves of up
// to two 128-blocks (128 bytes a row: every load instruction covers whole
// cache lines) into registers while the previous half is multiplied, and
// pass through one LDS buffer to the MFMA layout.
// Within a 128-block, lane group g holds K 32 g .. 32 g + 31 of its column
// (16 bytes and one E8M0 byte), fed to the bf16 MFMA as K 32 g + 8 q .. + 8
// in step q; the mid operand follows the same assignment. Products and block
// sums are exact while the sum fits binary32; the block sum is scaled by the
// row's mid scale in float64 and the blocks are summed in order, then rounded
// once to fp32. Rows past the tile's end repeat its last row: they compute
// the same values and store them to the same place, so every load and store
// is unconditional and each wait counts exactly. The item's E8M0 weight
// scales (its 256 w2 rows' scale rows, one contiguous run) come with the mid
// rows into LDS: a load whose lanes cover whole cache lines costs the memory
// pipeline about a quarter of one that reads 4 bytes from each of 16 rows.
constexpr int kDnRows = kBigRows;
constexpr int kDnItemCols = kDownItemCols;
constexpr int kDnThreads = 256;

// LDS byte offset of 16-byte chunk c (8 bf16) of widened mid row r (rows of
// 2 I bytes): c is XORed with r & 15 inside its aligned group of 16 chunks,
// so that consecutive rows reading one chunk fall in different bank groups.
template <int NB>
__device__ __forceinline__ int sw_mid16(int r, int c) { return r * (NB * 256) + 16 * (c ^ (r & 15)); }

// LDS place of 16-byte chunk c of weight row r in a half of BH blocks (rows
// of 64 BH bytes): c is XORed with a row function inside the row, so that
// sixteen consecutive rows reading one chunk, and a row's chunks written by
// consecutive lanes, fall in different bank groups.
template <int BH>
__device__ __forceinline__ int sw_w(int r, int c) {
  return BH == 2 ? r * 128 + 16 * (c ^ ((r >> 1) & 7)) : r * 64 + 16 * (c ^ ((r >> 2) & 3));
}

template <int NB>
constexpr size_t down_big_lds() {
  return (size_t)kDnRows * NB * 256 + sizeof(float) * NB * kDnRows + sizeof(int) * kDnRows +
         (size_t)kDnItemCols * NB * 4 + (size_t)kDnItemCols * (NB > 1 ? 128 : 64);
}

template <int NB>
__global__ __launch_bounds__(kDnThreads) __attribute__((amdgpu_waves_per_eu(2))) void down_big_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry, const int4* __restrict__ items,
    const int* __restrict__ meta, float* __restrict__ y, int H) {
  constexpr int I = NB * 128;
  constexpr int Wb = I / 2, Sb = I / 32;       // bytes per w2 row / s2 row
  constexpr int CPR = I / 16;                  // E4M3 16-byte chunks per mid row
  constexpr int QA = kDnRows * CPR / kDnThreads;  // of them per thread and tile
  static_assert(kDnRows * CPR % kDnThreads == 0 && kDnRows == 32 && kDnItemCols == 4 * 64, "tile shape");
  extern __shared__ __align__(16) uint8_t dyn_lds[];
  uint8_t* a16 = dyn_lds;                                             // [kDnRows] widened mid rows
  float* ms = reinterpret_cast<float*>(dyn_lds + kDnRows * NB * 256);  // [NB][kDnRows] mid scales
  int* ent = reinterpret_cast<int*>(ms + NB * kDnRows);                // [kDnRows] entries
  uint8_t* wsl = reinterpret_cast<uint8_t*>(ent + kDnRows);           // [kDnItemCols][4 NB] weight scales
  uint8_t* wld = wsl + kDnItemCols * Sb;                               // [kDnItemCols] rows of a weight half
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, g = lane >> 4;
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  constexpr int NH = (NB + 1) / 2;  // weight halves
  int first, stride, end;
  xcd_run(meta[2], first, stride, end);
  if (first >= end) return;

  // a tile's mid rows (past its end: the last row again), entries and scales
  v4u va[QA];
  int ve;
  float vs[NB];
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  v4u vsc4;
  v2u vsc2;
  unsigned vsc1, vsc3[3];
  auto fetch_tile = [&](const int4 item) {
    const int r0 = item.y, rows = item.z - item.y;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(midq + (size_t)r0 * I), (short)0, rows * I, 0x00020000);
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int idx = tid + kDnThreads * q;
      const int row = min(idx / CPR, rows - 1), c = idx % CPR;
      va[q] = __builtin_amdgcn_raw_buffer_load_b128(ra, row * I + 16 * c, 0, 0);
    }
    const int row = min(tid & (kDnRows - 1), rows - 1);
    ve = sorted_entry[r0 + row];
#pragma unroll
    for (int b = 0; b < NB; ++b) vs[b] = mids[(size_t)(r0 + row) * NB + b];
    // the item's scale rows: kDnItemCols x 4 NB contiguous bytes, 4 NB bytes a thread
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(s2 + ((size_t)item.x * H + (size_t)item.w * kDnItemCols) * Sb), (short)0,
        kDnItemCols * Sb, 0x00020000);
    if (NB == 4) vsc4 = __builtin_amdgcn_raw_buffer_load_b128(rsc, 16 * tid, 0, 0);
    else if (NB == 2) vsc2 = __builtin_amdgcn_raw_buffer_load_b64(rsc, 8 * tid, 0, 0);
    else if (NB == 3) {
      vsc3[0] = __builtin_amdgcn_raw_buffer_load_b32(rsc, 12 * tid, 0, 0);
      vsc3[1] = __builtin_amdgcn_raw_buffer_load_b32(rsc, 12 * tid + 4, 0, 0);
      vsc3[2] = __builtin_amdgcn_raw_buffer_load_b32(rsc, 12 * tid + 8, 0, 0);
    } else vsc1 = __builtin_amdgcn_raw_buffer_load_b32(rsc, 4 * tid, 0, 0);
  };
  // weight half h of an item (blocks 2h, 2h+1): thread t holds chunks
  // t + 256 q, 4 BH chunks of 16 bytes to a row
  v4u vw[8];
  auto load_half = [&](const int4 item, auto hc) {
    constexpr int h = decltype(hc)::value, BH = NB - 2 * h >= 2 ? 2 : 1;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(w2 + ((size_t)item.x * H + (size_t)item.w * kDnItemCols) * Wb), (short)0,
        kDnItemCols * Wb, 0x00020000);
#pragma unroll
    for (int q = 0; q < 4 * BH; ++q) {
      const int idx = tid + kDnThreads * q, row = idx / (4 * BH), c = idx % (4 * BH);
      vw[q] = __builtin_amdgcn_raw_buffer_load_b128(rw, row * Wb + 16 * c, 128 * h, 0);
    }
  };
  auto store_half = [&](auto hc) {
    constexpr int h = decltype(hc)::value, BH = NB - 2 * h >= 2 ? 2 : 1;
#pragma unroll
    for (int q = 0; q < 4 * BH; ++q) {
      const int idx = tid + kDnThreads * q, row = idx / (4 * BH), c = idx % (4 * BH);
      *reinterpret_cast<v4u*>(&wld[sw_w<BH>(row, c)]) = vw[q];
    }
  };
  {
    const int4 item = items[first];
    fetch_tile(item);
    load_half(item, std::integral_constant<int, 0>());
  }
  for (int it = first; it < end; it += stride) {
    const int4 item = items[it];
    const int4 next = items[min(it + stride, end - 1)];  // the last item loads itself again, unused
    __syncthreads();  // every wave is done with the previous item's LDS
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int idx = tid + kDnThreads * q;
      const int row = idx / CPR, c = idx % CPR;
      const v4u v = va[q];
      const v4u lo = {fp8x2_bf16<false>(v.x), fp8x2_bf16<true>(v.x), fp8x2_bf16<false>(v.y), fp8x2_bf16<true>(v.y)};
      const v4u hi = {fp8x2_bf16<false>(v.z), fp8x2_bf16<true>(v.z), fp8x2_bf16<false>(v.w), fp8x2_bf16<true>(v.w)};
      *reinterpret_cast<v4u*>(&a16[sw_mid16<NB>(row, 2 * c)]) = lo;
      *reinterpret_cast<v4u*>(&a16[sw_mid16<NB>(row, 2 * c + 1)]) = hi;
    }
    if (tid < kDnRows) {
      ent[tid] = ve;
#pragma unroll
      for (int b = 0; b < NB; ++b) ms[b * kDnRows + tid] = vs[b];
    }
    if (NB == 4) *reinterpret_cast<v4u*>(&wsl[16 * tid]) = vsc4;
    else if (NB == 2) *reinterpret_cast<v2u*>(&wsl[8 * tid]) = vsc2;
    else if (NB == 3) {
#pragma unroll
      for (int q = 0; q < 3; ++q) *reinterpret_cast<unsigned*>(&wsl[12 * tid + 4 * q]) = vsc3[q];
    } else *reinterpret_cast<unsigned*>(&wsl[4 * tid]) = vsc1;
    // RB = 16-row blocks of the tile that hold rows: a tile of at most 16
    // rows computes and stores one (the other is padding), on a path of its
    // own so that neither carries the other's registers
    auto run = [&](auto rbc) {
      constexpr int RB = decltype(rbc)::value;
      double acc[RB][4][4];
      // one 128-block: B fragments from the weight half in LDS
      auto block = [&](auto bc) {
        constexpr int b = decltype(bc)::value, h = b / 2, BH = NB - 2 * h >= 2 ? 2 : 1;
        v4u Sw[4];
  #pragma unroll
        for (int j = 0; j < 4; ++j)
          Sw[j] = *reinterpret_cast<const v4u*>(&wld[sw_w<BH>(64 * wave + 16 * j + m, 4 * (b % 2) + g)]);
        float wsc[4];
  #pragma unroll
        for (int j = 0; j < 4; ++j) wsc[j] = e8m0_to_float(wsl[(64 * wave + 16 * j + m) * Sb + 4 * b + g]);
        v4f P[2][4];
  #pragma unroll
        for (int i = 0; i < RB; ++i)
  #pragma unroll
          for (int j = 0; j < 4; ++j) P[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          v8s fb[4];
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t wq = Sw[j][q];
            fb[j] = as_v8s(cvt_fp4x2_bf16<0>(wq, wsc[j]), cvt_fp4x2_bf16<1>(wq, wsc[j]),
                           cvt_fp4x2_bf16<2>(wq, wsc[j]), cvt_fp4x2_bf16<3>(wq, wsc[j]));
          }
  #pragma unroll
          for (int i = 0; i < RB; ++i) {
            const v8s fa = *reinterpret_cast<const v8s*>(&a16[sw_mid16<NB>(16 * i + m, 16 * b + 4 * g + q)]);
  #pragma unroll
            for (int j = 0; j < 4; ++j) P[i][j] = mfma_bf16(fa, fb[j], P[i][j]);
          }
        }
  #pragma unroll
        for (int i = 0; i < RB; ++i) {
          const float4 sc = *reinterpret_cast<const float4*>(&ms[b * kDnRows + 16 * i + 4 * g]);
          const double scd[4] = {(double)sc.x, (double)sc.y, (double)sc.z, (double)sc.w};
  #pragma unroll
          for (int j = 0; j < 4; ++j)
  #pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[i][j][v] = b == 0 ? scd[v] * (double)P[i][j][v] : fma(scd[v], (double)P[i][j][v], acc[i][j][v]);
        }
      };
      // half 0 (in registers) to LDS; the next half's loads run while a half
      // is multiplied; after the last half's loads go out, the next item's
      // mid rows and first half
      store_half(std::integral_constant<int, 0>());
      __syncthreads();
      if (NH > 1) load_half(item, std::integral_constant<int, 1>());
      else {
        fetch_tile(next);
        load_half(next, std::integral_constant<int, 0>());
      }
      block(std::integral_constant<int, 0>());
      if (NB > 1) block(std::integral_constant<int, 1 % NB>());
      if (NH > 1) {
        __syncthreads();  // every wave is done with half 0
        store_half(std::integral_constant<int, NH - 1>());
        __syncthreads();
        fetch_tile(next);
        load_half(next, std::integral_constant<int, 0>());
        block(std::integral_constant<int, 2 % NB>());
        if (NB > 3) block(std::integral_constant<int, 3 % NB>());
      }
      // y row = entry (rows past the tile's end repeat its last row)
      const int col = item.w * kDnItemCols + 64 * wave + m;
  #pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int4 en = *reinterpret_cast<const int4*>(&ent[16 * i + 4 * g]);
        const int env[4] = {en.x, en.y, en.z, en.w};
  #pragma unroll
        for (int v = 0; v < 4; ++v) {
          float* py = y + (size_t)env[v] * H + col;
  #pragma unroll
          for (int j = 0; j < 4; ++j) py[16 * j] = (float)acc[i][j][v];
        }
      }
    };
    if (item.z - item.y > 16) run(std::integral_constant<int, 2>());
    else run(std::integral_constant<int, 1>());
  }
}

hipError_t launch_gate_up_big(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = (n + std::min<int64_t>(p->s.E, n) * (kGuR - 1) + kGuR - 1) / kGuR;
  const int64_t items = tiles * (p->s.I / 128);
  const int blocks = (int)std::min<int64_t>(items, 512);  // two per CU
  auto kern = p->mid_fmt == MOE_MID_MXFP4 ? gate_up_big_kernel<true> : gate_up_big_kernel<false>;
  return launch_k(kern, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.xq),
                  wsp<uint8_t>(p, p->L.xs), reinterpret_cast<const uint8_t*>(a.w13),
                  reinterpret_cast<const uint8_t*>(a.s13), wsp<int>(p, p->L.sorted_entry),
                  wsp<int4>(p, p->X.gu_items), wsp<int>(p, p->X.meta), (int)p->s.H, (int)p->s.I,
                  (int)p->s.top_k, wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids));
}


hipError_t launch_down_big(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = (n + std::min<int64_t>(p->s.E, n) * (kDnRows - 1) + kDnRows - 1) / kDnRows;
  const int64_t items = tiles * (p->s.H / kDnItemCols);
  const int blocks = (int)std::min<int64_t>(items, 2 * (int64_t)p->num_cus);  // two per CU
  auto go = [&](auto kern, size_t lds) {
    return launch_k(kern, dim3(blocks), dim3(kDnThreads), lds, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry),
                    wsp<int4>(p, p->X.dn_items), wsp<int>(p, p->X.meta), wsp<float>(p, p->L.y), (int)p->s.H);
  };
  switch (p->s.I / 128) {
    case 1: return go(down_big_kernel<1>, down_big_lds<1>());
    case 2: return go(down_big_kernel<2>, down_big_lds<2>());
    case 3: return go(down_big_kernel<3>, down_big_lds<3>());
    case 4: return go(down_big_kernel<4>, down_big_lds<4>());
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
