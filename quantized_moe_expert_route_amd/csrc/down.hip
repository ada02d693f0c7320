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
#include "shared_small.h"

#include <algorithm>
#include <type_traits>

namespace qmoe {

// Up to kSmallM tokens (and kSmallRows entries), down and combine are one
// launch. A workgroup owns cw <= 16 output columns of every token (cw is
// picked per H so that the CUs carry equal shares of w2; lanes of the
// 16-column MFMA past cw repeat column cw - 1 and their results are never
// read): its four waves
// take every fourth 16-row tile (wave w: tiles w, w + 4, ...), keep each (entry, column) result
// in LDS, and when every tile is done the workgroup forms out[t, c0 .. c0+16)
// from the token's k slots, so no slot result leaves the workgroup.
//
// In MFMA step q of a 128-block, lane group g supplies K = 32g + 8q .. + 8:
// a lane reads 16 contiguous weight bytes (one MX block, one scale byte) per
// block. Each wave keeps the weights of D tiles in flight in a ring of
// register slots, issued slot by slot; the ring's steady-state body has no
// branches, so the wait for a slot counts only the loads issued after it,
// and no tile is loaded twice. The tile descriptors arrive through scalar
// loads, so the first weight loads do not queue behind the mid staging.
//
// MID_LDS: the n mid rows are staged in LDS with their scales, widened to
// bf16 once per workgroup while n * I <= kDcMidBytes; above (ST = 12, e.g.
// a ninth slot at M = 16) bf16 rows would leave one workgroup per CU, so
// they stay E4M3 (half the bytes) and each fragment is widened as it is
// read (still once per workgroup, but on the MFMA's path: slower while the
// bf16 rows fit). Otherwise each slot carries its tile's E4M3 mid rows in
// registers and widens them itself.
//
// QF (qd_path: at most kQdBlocks (row, 128-block) pairs of mid, e.g. M = 4
// at top-8 and I = 256): every workgroup quantizes mid itself from h with
// the arithmetic of act_quant_kernel (s = fl32(amax / 448), q = E4M3(fl32(h
// / s))) while its weights are in flight, and workgroup 0 stores the codes
// and scales; the call then has no act_quant launch. Sixteen lanes hold the
// 128 values of a block, eight each.
constexpr int kDcThreads = 256;
constexpr int kDcWaves = kDcThreads / 64;
constexpr int kDcMidBytes = 32 * 1024;  // n * I staged in LDS from E4M3: ST = 8 uint4 per thread
constexpr int kDcMidBytesMax = 48 * 1024;  // ST = 12: n up to 192 at I = 256 (the shared expert as a ninth slot)
constexpr int kDcPad = 16;              // LDS bytes after each staged mid row

// the largest of a value over the 16 lanes of a DPP row (every lane gets it)
__device__ __forceinline__ uint32_t max16_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
}

template <int NB, bool MID_LDS>
struct DcSlot {
  uint4 w[NB];                                            // this lane's 32 E2M1 weights of each block
  typename std::conditional<NB == 1, uint32_t, typename std::conditional<NB == 2, uint2,
      typename std::conditional<NB == 3, uint3, uint4>::type>::type>::type ws;  // the column's E8M0 bytes
  uint4 a[MID_LDS ? 1 : NB][2];                           // this lane's 32 E4M3 mid bytes of each block
  float sc[MID_LDS ? 1 : NB][4];                          // mid scales of the lane's four D rows
  int ent[MID_LDS ? 1 : 4];                               // entries t*k+j of the lane's four D rows
};

__device__ __forceinline__ uint32_t scale_byte(uint32_t v, int b, int g) { return (v >> (8 * g)) & 0xFFu; }
__device__ __forceinline__ uint32_t scale_byte(const uint2& v, int b, int g) {
  return ((b == 0 ? v.x : v.y) >> (8 * g)) & 0xFFu;
}
__device__ __forceinline__ uint32_t scale_byte(const uint3& v, int b, int g) {
  return ((b == 0 ? v.x : b == 1 ? v.y : v.z) >> (8 * g)) & 0xFFu;
}
__device__ __forceinline__ uint32_t scale_byte(const uint4& v, int b, int g) {
  return ((b == 0 ? v.x : b == 1 ? v.y : b == 2 ? v.z : v.w) >> (8 * g)) & 0xFFu;
}

size_t down_combine_lds_bytes(int64_t n, int64_t I, bool mid_lds, bool mid_bf16, int groups = 1) {
  size_t b = (size_t)groups * (n + 1) * 16 * 4;
  if (mid_lds) b += (size_t)n * ((mid_bf16 ? 2 : 1) * I + kDcPad) + (size_t)n * (I / 128) * 4 + (size_t)n * 4;
  return b;
}

// SH: the block-FP8 shared expert runs inside this launch (its own
// instantiations, so that the routed-only ones carry none of its registers)
template <int NB, int D, bool MID_LDS, int ST = 8, bool SH = false, bool LONG = true, bool QF = false, int G = 1>
__global__ __launch_bounds__(kDcThreads * G) void down_combine_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry,
    const int4* __restrict__ tiles, const int* __restrict__ meta, int tmax, int H, int k, int M, int cw,
    const float* __restrict__ topk_w, const float* __restrict__ ys, uint16_t* __restrict__ out,
    double* __restrict__ partial, SharedSmall sh, const float* __restrict__ hin, uint8_t* __restrict__ mq_out,
    float* __restrict__ ms_out) {
  constexpr int I = NB * 128;
  constexpr bool A16 = ST == 8;  // mid staged widened to bf16 (else E4M3, widened at each read)
  static_assert(!QF || (MID_LDS && A16 && !SH), "QF stages the quantized mid as bf16 rows");
  static_assert(G == 1 || (G == 2 && QF), "two column groups share one workgroup only to share the mid quantization");
  // G column groups of four waves each; the groups share the staged mid
  // (with QF: its quantization, half the h traffic and work a group)
  constexpr int kQP = kQdBlocks / (kDcThreads * G / 16);  // blocks of h a thread quantizes (QF)
  constexpr int LDA = (A16 ? 2 : 1) * I + kDcPad;  // bytes per staged mid row; the pad spreads 16 rows over the banks
  extern __shared__ __align__(16) uint8_t dyn[];
  const int n = M * k;
  const int tid = threadIdx.x, wave_all = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = G == 1 ? 0 : wave_all >> 2, wave = G == 1 ? wave_all : wave_all & 3;  // group, wave in it
  const int gtid = G == 1 ? tid : tid & (kDcThreads - 1);                               // thread in the group
  float* yl = reinterpret_cast<float*>(dyn) + grp * (n + 1) * 16;  // [G][n + 1][16]; row n takes dropped rows
  uint8_t* ml = reinterpret_cast<uint8_t*>(reinterpret_cast<float*>(dyn) + G * (n + 1) * 16);  // [n][LDA]  (MID_LDS) bf16 or E4M3 mid
  float* msl = reinterpret_cast<float*>(ml + n * LDA);  // [n][NB]   (MID_LDS)
  int* sel = reinterpret_cast<int*>(msl + n * NB);      // [n]       (MID_LDS) sorted_entry
  const int r = lane & 15, g = lane >> 4;
  const int c0 = (blockIdx.x * G + grp) * cw;
  const int rc = min(r, cw - 1);  // the lane's weight column
  // wave w takes tiles w, w + kDcWaves, ... (my of them); its first D
  // descriptors are read beside meta (indices clamped to the tile array's
  // bound, tmax), so the weight loads wait for one round trip, not two
  const int nt = meta[0];
  int4 T[D];
#pragma unroll
  for (int d = 0; d < D; ++d) T[d] = tiles[min(wave + kDcWaves * d, tmax - 1)];
  const int4 t_first = tiles[0];
  constexpr int kSt = MID_LDS ? ST : 1;
  uint4 st[kSt];
  uint4 hv[QF ? 2 * kQP : 1];  // (QF) the thread's h values
  constexpr int kSs = ST == 8 ? 1 : 2;  // mid scales and entries a thread stages (n * NB <= kSs * kDcThreads)
  float sts[kSs];
  int ste[kSs];
  if (QF) {
    // h of block qb = 16 G p + tid / 16 (row qb / NB, block qb % NB), the
    // lane's 8 values (past the last block the last one again, unused), and
    // the sorted entries: none depends on the descriptors, so they go out
    // before the wait for them
#pragma unroll
    for (int p = 0; p < kQP; ++p) {
      const int qb = min(16 * G * p + (tid >> 4), n * NB - 1);
      const float* ph = hin + (size_t)(qb / NB) * I + 128 * (qb % NB) + 8 * (tid & 15);
      hv[2 * p] = ld16(ph);
      hv[2 * p + 1] = ld16(ph + 4);
    }
#pragma unroll
    for (int q = 0; q < kSs; ++q) {
      const int idx = tid + kDcThreads * G * q;
      ste[q] = idx < n ? sorted_entry[idx] : 0;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // (all of these loads are issued before the first wait)
  asm volatile("" ::"s"(nt), "s"(t_first.x), "s"(T[0].x), "s"(T[min(1, D - 1)].x), "s"(T[min(2, D - 1)].x),
               "s"(T[min(3, D - 1)].x), "s"(T[min(4, D - 1)].x), "s"(T[min(5, D - 1)].x), "s"(T[min(6, D - 1)].x),
               "s"(T[min(7, D - 1)].x));
  const int my = wave < nt ? (nt - 1 - wave) / kDcWaves + 1 : 0;
  auto tile_of = [&](int i) { return wave + kDcWaves * i; };  // the wave's i-th tile

  // ---- descriptors of the wave's first D tiles, then the staging loads
  // (both from L2); the weight loads wait only for the descriptors, the LDS
  // staging waits for its loads after the weight loads have gone out.
  // Slots past the wave's run repeat its last tile (computed again: the
  // same values to the same places); a wave without tiles loads tile 0 and
  // computes nothing. The loads are unconditional so that every later wait
  // counts exactly.
  // the fused shared expert's down operands come first, so they have landed
  // by the end of the ring
  SharedDownPre sdp;
  if (SH) shared_down_fetch(sh, M, c0, cw, sdp);
  // slots past the run repeat its last tile; a wave without tiles holds tile 0
  if (my == 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) T[d] = t_first;
  }
#pragma unroll
  for (int d = 1; d < D; ++d)
    if (d >= my && my > 0) T[d] = T[d - 1];
  __builtin_amdgcn_sched_barrier(0);
  if (!QF && MID_LDS) {
#pragma unroll
    for (int q = 0; q < kSt; ++q) {
      const int idx = tid + kDcThreads * q;
      st[q] = idx < n * (I / 16) ? ld16(midq + 16 * (size_t)idx) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < kSs; ++q) {
      const int idx = tid + kDcThreads * q;
      sts[q] = idx < n * NB ? mids[idx] : 0.f;
      ste[q] = idx < n ? sorted_entry[idx] : 0;
    }
  }

  auto load = [&](const int4 tl, DcSlot<NB, MID_LDS>& S) {
    const size_t col = (size_t)tl.x * H + c0 + rc;
    const uint8_t* pw = w2 + col * (I / 2) + 16 * g;
#pragma unroll
    for (int b = 0; b < NB; ++b) S.w[b] = ld16(pw + 64 * b);
    S.ws = *reinterpret_cast<const decltype(S.ws)*>(s2 + col * (I / 32));
    if (!MID_LDS) {
      // rows past the tile's end read the tile's first row; their results are dropped
      const int row = tl.y + r < tl.z ? tl.y + r : tl.y;
      const uint8_t* pq = midq + (size_t)row * I + 32 * g;
#pragma unroll
      for (int b = 0; b < (MID_LDS ? 1 : NB); ++b) {
        S.a[b][0] = ld16(pq + 128 * b);
        S.a[b][1] = ld16(pq + 128 * b + 16);
      }
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const int m = min(tl.y + 4 * g + i2, tl.z - 1);
#pragma unroll
        for (int b = 0; b < (MID_LDS ? 1 : NB); ++b) S.sc[b][i2] = mids[(size_t)m * NB + b];
        S.ent[MID_LDS ? 0 : i2] = sorted_entry[m];
      }
    }
  };
  auto compute = [&](const int4 tl, const DcSlot<NB, MID_LDS>& S) {
    const int arow = min(tl.y + r, tl.z - 1);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float wsc = e8m0_to_float(scale_byte(S.ws, b, g));
      const uint32_t qw[4] = {S.w[b].x, S.w[b].y, S.w[b].z, S.w[b].w};
      float sc[4];
      v4f P = {0.f, 0.f, 0.f, 0.f};
      if (MID_LDS) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) sc[i2] = msl[min(tl.y + 4 * g + i2, tl.z - 1) * NB + b];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v8s fa;
          if (A16) {
            const uint4 av = *reinterpret_cast<const uint4*>(ml + arow * LDA + 2 * (128 * b + 32 * g + 8 * q));
            fa = as_v8s(av.x, av.y, av.z, av.w);
          } else {  // 8 E4M3 codes widened to bf16 as they are read (exact)
            const uint2 av = *reinterpret_cast<const uint2*>(ml + arow * LDA + 128 * b + 32 * g + 8 * q);
            fa = as_v8s(fp8x2_bf16<false>(av.x), fp8x2_bf16<true>(av.x), fp8x2_bf16<false>(av.y),
                        fp8x2_bf16<true>(av.y));
          }
          const v8s fb = as_v8s(cvt_fp4x2_bf16<0>(qw[q], wsc), cvt_fp4x2_bf16<1>(qw[q], wsc),
                                cvt_fp4x2_bf16<2>(qw[q], wsc), cvt_fp4x2_bf16<3>(qw[q], wsc));
          P = mfma_bf16(fa, fb, P);
        }
      } else {
        const uint4 a0 = S.a[MID_LDS ? 0 : b][0], a1 = S.a[MID_LDS ? 0 : b][1];
        const uint32_t qa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) sc[i2] = S.sc[MID_LDS ? 0 : b][i2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v8s fa = as_v8s(fp8x2_bf16<false>(qa[2 * q]), fp8x2_bf16<true>(qa[2 * q]),
                                fp8x2_bf16<false>(qa[2 * q + 1]), fp8x2_bf16<true>(qa[2 * q + 1]));
          const v8s fb = as_v8s(cvt_fp4x2_bf16<0>(qw[q], wsc), cvt_fp4x2_bf16<1>(qw[q], wsc),
                                cvt_fp4x2_bf16<2>(qw[q], wsc), cvt_fp4x2_bf16<3>(qw[q], wsc));
          P = mfma_bf16(fa, fb, P);
        }
      }
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) acc[i2] += (double)sc[i2] * (double)P[i2];
    }
    // rows past the tile's end go to the dropped row n
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int m = tl.y + 4 * g + i2;
      const int ent = MID_LDS ? sel[min(m, tl.z - 1)] : S.ent[MID_LDS ? 0 : i2];
      yl[(m < tl.z ? ent : n) * 16 + r] = (float)acc[i2];
    }
  };

  __builtin_amdgcn_sched_barrier(0);
  // ---- the first D tiles' weights
  DcSlot<NB, MID_LDS> S[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load(T[d], S[d]);
    __builtin_amdgcn_sched_barrier(0);  // slot by slot, in issue order
  }

  // ---- staged mid to LDS (widened to bf16 when A16)
  if (QF) {
#pragma unroll
    for (int p = 0; p < kQP; ++p) {
      const uint4 v0 = hv[2 * p], v1 = hv[2 * p + 1];
      const uint32_t vb[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t am = 0;  // |h| bit patterns order as the values do
#pragma unroll
      for (int i = 0; i < 8; ++i) am = max(am, vb[i] & 0x7FFFFFFFu);
      am = max16_u32(am);
      const float sc = __fdiv_rn(__uint_as_float(am), 448.0f);
      uint32_t lo = 0, hi = 0;
      if (sc > 0.f) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          lo |= e4m3_pack2(__fdiv_rn(__uint_as_float(vb[i]), sc), __fdiv_rn(__uint_as_float(vb[i + 1]), sc)) << (8 * i);
          hi |= e4m3_pack2(__fdiv_rn(__uint_as_float(vb[4 + i]), sc), __fdiv_rn(__uint_as_float(vb[5 + i]), sc))
                << (8 * i);
        }
      }
      const int qb = 16 * G * p + (tid >> 4);
      if (qb < n * NB) {
        const int row = qb / NB, b = qb % NB, kk = 128 * b + 8 * (tid & 15);
        *reinterpret_cast<uint4*>(ml + row * LDA + 2 * kk) =
            make_uint4(fp8x2_bf16<false>(lo), fp8x2_bf16<true>(lo), fp8x2_bf16<false>(hi), fp8x2_bf16<true>(hi));
        if ((tid & 15) == 0) msl[row * NB + b] = sc;
        if (blockIdx.x == 0) {  // the codes and scales, as the act_quant launch stores them
          *reinterpret_cast<uint2*>(mq_out + (size_t)row * I + kk) = make_uint2(lo, hi);
          if ((tid & 15) == 0) ms_out[(size_t)row * NB + b] = sc;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kSs; ++q) {
      const int idx = tid + kDcThreads * G * q;
      if (idx < n) sel[idx] = ste[q];
    }
    barrier_lds();
  } else if (MID_LDS) {
#pragma unroll
    for (int q = 0; q < kSt; ++q) {
      const int idx = tid + kDcThreads * q;
      if (idx < n * (I / 16)) {
        const int row = idx / (I / 16), c = idx - row * (I / 16);
        if (A16) {
          uint4* dst = reinterpret_cast<uint4*>(ml + row * LDA + 32 * c);  // E4M3 -> bf16, exact
          dst[0] = make_uint4(fp8x2_bf16<false>(st[q].x), fp8x2_bf16<true>(st[q].x), fp8x2_bf16<false>(st[q].y),
                              fp8x2_bf16<true>(st[q].y));
          dst[1] = make_uint4(fp8x2_bf16<false>(st[q].z), fp8x2_bf16<true>(st[q].z), fp8x2_bf16<false>(st[q].w),
                              fp8x2_bf16<true>(st[q].w));
        } else {
          *reinterpret_cast<uint4*>(ml + row * LDA + 16 * c) = st[q];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kSs; ++q) {
      const int idx = tid + kDcThreads * q;
      if (idx < n * NB) msl[idx] = sts[q];
      if (idx < n) sel[idx] = ste[q];
    }
    barrier_lds();
  }

  // ---- the ring. A run that fits the slots is computed straight from the
  // prologue's loads (one path, so each wait counts exactly); a longer one
  // reloads each slot right after computing it, batch by batch.
  if (my > 0 && my <= D) {
#pragma unroll
    for (int d = 0; d < D; d += 2) {
      compute(T[d], S[d]);
      if (d + 1 < D) compute(T[d + 1], S[d + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (LONG && my > D) {  // (without LONG the launch guarantees my <= D)
    // while tiles remain after the batch in the slots, each slot is
    // reloaded as soon as its tile is computed, so the next batch's loads
    // overlap this batch's products; slots past the wave's run reload its
    // last tile (loaded, never computed), so every load is unconditional
    int i0 = 0;
    for (; i0 + D < my; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; d += 2) {  // two independent tiles per step
        const int4 tn0 = tiles[tile_of(min(i0 + D + d, my - 1))];
        const int4 tn1 = tiles[tile_of(min(i0 + D + min(d + 1, D - 1), my - 1))];
        compute(T[d], S[d]);
        if (d + 1 < D) compute(T[d + 1], S[d + 1]);
        __builtin_amdgcn_sched_barrier(0);
        load(tn0, S[d]);
        T[d] = tn0;
        if (d + 1 < D) {
          load(tn1, S[d + 1]);
          T[d + 1] = tn1;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the slots hold tiles i0 .. my - 1 (1 to D of them), then repeats
    const int rest = my - i0;
#pragma unroll
    for (int d = 0; d < D; d += 2) {
      if (d < rest) compute(T[d], S[d]);
      if (d + 1 < D && d + 1 < rest) compute(T[d + 1], S[d + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  // the block-FP8 shared expert's down for this workgroup's columns (run
  // inside the small-token launches), in the LDS after the slot results
  // (the staged mid rows there are no longer read)
  float* ysl = nullptr;
  if (SH) {
    uint8_t* shl = dyn + (((size_t)(n + 1) * 16 * 4 + 15) & ~(size_t)15);
    ysl = reinterpret_cast<float*>(shl + shared_down_lds(sh.Is) - 16 * 16 * 4);
    shared_down_cols(sh, M, c0, cw, sdp, shl, ysl);
  }
  // out[t, c0 + 2p .. + 2): float64 products and sum in slot order (+ shared), one bf16 rounding
  const int pairs = cw >> 1;
  for (int idx = gtid; idx < M * pairs; idx += kDcThreads) {
    const int t = idx / pairs, cc = 2 * (idx - t * pairs);
    double a0 = 0.0, a1 = 0.0;
    for (int j = 0; j < k; ++j) {
      const double wj = (double)topk_w[t * k + j];
      const float* py = yl + (t * k + j) * 16 + cc;
      a0 += wj * (double)py[0];
      a1 += wj * (double)py[1];
    }
    if (ysl) {
      a0 += (double)ysl[t * 16 + cc];
      a1 += (double)ysl[t * 16 + cc + 1];
    } else if (ys) {
      a0 += (double)ys[(size_t)t * H + c0 + cc];
      a1 += (double)ys[(size_t)t * H + c0 + cc + 1];
    }
    if (partial)  // the sum before its rounding, for the tensor-parallel exchange
      *reinterpret_cast<double2*>(partial + (size_t)t * H + c0 + cc) = make_double2(a0, a1);
    else
      *reinterpret_cast<uint32_t*>(out + (size_t)t * H + c0 + cc) =
          bf16_rne_from_double(a0) | (bf16_rne_from_double(a1) << 16);
  }
}

// out[t, c..c+3]: float64 products and sum in slot order (+ shared), then
// bf16. A thread per 4 columns: consecutive lanes read consecutive 16 bytes
// of a y row, so each load instruction covers whole cache lines. The K slots'
// loads all go out before the first product (K is the call's top-k: a loop
// over a runtime count waited for each slot's load before the next).
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const float* __restrict__ ys, int M, int H,
                                                      uint16_t* __restrict__ out, double* __restrict__ partial) {
  const int per_tok = H / 4;
  const int64_t total = (int64_t)M * per_tok;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / per_tok);
    const int c = (int)(i % per_tok) * 4;
    // the shared expert's output (without one: slot 0's y again, which the
    // load below reads anyway; unconditional, so no branch waits for it)
    const float* pb = ys ? ys + (size_t)t * H + c : y + (size_t)t * K * H + c;
    const float4 b = *reinterpret_cast<const float4*>(pb);
    float wv[K];
    v4f a[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      wv[j] = w[(size_t)t * K + j];
      // y is read once: non-temporal loads keep it from displacing cached lines
      a[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(y + ((size_t)t * K + j) * H + c));
    }
    asm volatile("" ::"v"(b.x), "v"(b.y), "v"(b.z), "v"(b.w));  // keeps b's load with the others
    double acc[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const double wj = (double)wv[j];
      acc[0] += wj * (double)a[j][0]; acc[1] += wj * (double)a[j][1];
      acc[2] += wj * (double)a[j][2]; acc[3] += wj * (double)a[j][3];
    }
    if (ys) {  // the shared expert's output, the last term
      acc[0] += b.x; acc[1] += b.y; acc[2] += b.z; acc[3] += b.w;
    }
    if (partial) {  // the sum before its rounding, for the tensor-parallel exchange
      double2* pp = reinterpret_cast<double2*>(partial + (size_t)t * H + c);
      pp[0] = make_double2(acc[0], acc[1]);
      pp[1] = make_double2(acc[2], acc[3]);
    } else {
      const uint32_t o0 = bf16_rne_from_double(acc[0]) | (bf16_rne_from_double(acc[1]) << 16);
      const uint32_t o1 = bf16_rne_from_double(acc[2]) | (bf16_rne_from_double(acc[3]) << 16);
      *reinterpret_cast<uint2*>(out + (size_t)t * H + c) = make_uint2(o0, o1);
    }
  }
}

// Columns per workgroup: the even width in 8..16 that divides H and gives
// the busiest CU the fewest columns (workgroups are spread round-robin over
// the CUs); ties go to the wider one.
int down_combine_cols(int H, int cus) {
  int best = 16, best_load = 1 << 30;
  for (int cw = 16; cw >= 8; cw -= 2) {
    if (H % cw) continue;
    const int wgs = H / cw;
    const int load = (wgs + cus - 1) / cus * cw;
    if (load < best_load) best = cw, best_load = load;
  }
  return best;
}

hipError_t launch_down_combine(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int H = (int)p->s.H;
  const int64_t n = a.M * p->s.top_k, I = p->s.I;
  if (n > kSmallRows) return hipErrorInvalidValue;
  const bool qf = qd_path(p, a.M);  // the mid quantized here from h (no act_quant launch)
  const bool mid_lds = n * I <= kDcMidBytesMax && n * (I / 128) <= 2 * kDcThreads && n <= 2 * kDcThreads;
  const bool wide = n * I > kDcMidBytes;  // 12 staging registers a thread instead of 8
  const SharedSmall sh = shared_small(p, a.M);  // the shared expert inside this launch, or none
  size_t lds = down_combine_lds_bytes(n, I, mid_lds, mid_lds && !wide);
  if (sh.hq) lds = std::max(lds, (((size_t)(n + 1) * 16 * 4 + 15) & ~(size_t)15) + shared_down_lds(sh.Is));
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const float* ys = p->s.shared_I > 0 && !sh.hq ? wsp<float>(p, p->L.sh_y) : nullptr;
  const int cw = down_combine_cols(H, p->num_cus);
  // the tile array's bound for this call (tiles of kTileRows sorted rows)
  const int tmax = (int)((n + std::min<int64_t>(p->s.E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows);
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(H / cw), dim3(kDcThreads), lds, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), tmax, H, (int)p->s.top_k, (int)a.M, cw, wsp<float>(p, p->L.topk_w), ys,
                    reinterpret_cast<uint16_t*>(a.out), tp_own_partial(p), sh, wsp<float>(p, p->X.h),
                    wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids));
  };

  // weights of D tiles in flight per wave; fewer when the slots also carry
  // mid rows. A call of at most kDcWaves * D entries has at most that many
  // tiles, so no wave has more tiles than slots: its kernel carries no
  // reload path (which alone made the c1 down ~0.7 us slower).
  auto pick = [&](auto shc, auto lc) {
    constexpr bool S = decltype(shc)::value, L = decltype(lc)::value;
    switch (I / 128) {
      case 1: return !mid_lds ? go(down_combine_kernel<1, 6, false, 8, S, L>)
                     : wide   ? go(down_combine_kernel<1, 8, true, 12, S, L>) : go(down_combine_kernel<1, 8, true, 8, S, L>);
      case 2: return !mid_lds ? go(down_combine_kernel<2, 3, false, 8, S, L>)
                     : wide   ? go(down_combine_kernel<2, 8, true, 12, S, L>) : go(down_combine_kernel<2, 8, true, 8, S, L>);
      case 3: return !mid_lds ? go(down_combine_kernel<3, 2, false, 8, S, L>)
                     : wide   ? go(down_combine_kernel<3, 5, true, 12, S, L>) : go(down_combine_kernel<3, 5, true, 8, S, L>);
      case 4: return !mid_lds ? go(down_combine_kernel<4, 2, false, 8, S, L>)
                     : wide   ? go(down_combine_kernel<4, 4, true, 12, S, L>) : go(down_combine_kernel<4, 4, true, 8, S, L>);
      default: return hipErrorInvalidValue;
    }
  };
  const int nb = (int)(I / 128);
  const int64_t d_slots = !mid_lds ? (nb == 1 ? 6 : nb == 2 ? 3 : 2) : (nb <= 2 ? 8 : nb == 3 ? 5 : 4);
  const bool lng = n > kDcWaves * d_slots;
  if (qf) {  // at most kQdBlocks mid blocks, no wave with more tiles than slots
    if (!mid_lds || wide || sh.hq || lng) return hipErrorInvalidValue;
    if (H % (2 * cw) == 0) {
      // two column groups a workgroup share the mid quantization: half the
      // h reads and quantizing work of one workgroup per group
      const size_t lds2 = down_combine_lds_bytes(n, I, true, true, 2);
      auto go2 = [&](auto kern) {
        return launch_k(kern, dim3(H / (2 * cw)), dim3(2 * kDcThreads), lds2, a.stream, ev,
                        wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                        reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry),
                        wsp<int4>(p, p->X.tiles), wsp<int>(p, p->X.meta), tmax, H, (int)p->s.top_k, (int)a.M, cw,
                        wsp<float>(p, p->L.topk_w), ys, reinterpret_cast<uint16_t*>(a.out), tp_own_partial(p), sh,
                        wsp<float>(p, p->X.h), wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids));
      };
      switch (nb) {
        case 1: return go2(down_combine_kernel<1, 8, true, 8, false, false, true, 2>);
        case 2: return go2(down_combine_kernel<2, 8, true, 8, false, false, true, 2>);
        case 3: return go2(down_combine_kernel<3, 5, true, 8, false, false, true, 2>);
        case 4: return go2(down_combine_kernel<4, 4, true, 8, false, false, true, 2>);
        default: return hipErrorInvalidValue;
      }
    }
    switch (nb) {
      case 1: return go(down_combine_kernel<1, 8, true, 8, false, false, true>);
      case 2: return go(down_combine_kernel<2, 8, true, 8, false, false, true>);
      case 3: return go(down_combine_kernel<3, 5, true, 8, false, false, true>);
      case 4: return go(down_combine_kernel<4, 4, true, 8, false, false, true>);
      default: return hipErrorInvalidValue;
    }
  }
  if (sh.hq) return lng ? pick(std::true_type(), std::true_type()) : pick(std::true_type(), std::false_type());
  return lng ? pick(std::false_type(), std::true_type()) : pick(std::false_type(), std::false_type());
}

hipError_t launch_combine(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int H = (int)p->s.H;
  const int64_t total = a.M * (H / 4);
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
  const float* ys = p->s.shared_I > 0 ? wsp<float>(p, p->L.sh_y) : nullptr;
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<float>(p, p->L.y), wsp<float>(p, p->L.topk_w),
                    ys, (int)a.M, H, reinterpret_cast<uint16_t*>(a.out), tp_own_partial(p));
  };
  switch (p->s.top_k) {
    case 1: return go(combine_kernel<1>);
    case 2: return go(combine_kernel<2>);
    case 3: return go(combine_kernel<3>);
    case 4: return go(combine_kernel<4>);
    case 5: return go(combine_kernel<5>);
    case 6: return go(combine_kernel<6>);
    case 7: return go(combine_kernel<7>);
    case 8: return go(combine_kernel<8>);
    case 9: return go(combine_kernel<9>);
    case 10: return go(combine_kernel<10>);
    case 11: return go(combine_kernel<11>);
    case 12: return go(combine_kernel<12>);
    case 13: return go(combine_kernel<13>);
    case 14: return go(combine_kernel<14>);
    case 15: return go(combine_kernel<15>);
    case 16: return go(combine_kernel<16>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
