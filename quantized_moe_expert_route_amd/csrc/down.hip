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
#include <type_traits>

namespace qmoe {

// Up to kSmallM tokens (and kSmallRows entries), down and combine are one
// launch. A workgroup owns cw <= 16 output columns of every token (cw is
// picked per H so that the CUs carry equal shares of w2; lanes of the
// 16-column MFMA past cw repeat column cw - 1 and their results are never
// read): its four waves
// take contiguous runs of the 16-row tiles, keep each (entry, column) result
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
// registers and widens them itself. (Quantizing mid inside this launch
// instead, redundantly per workgroup, measured slower than its own launch.)
constexpr int kDcThreads = 256;
constexpr int kDcWaves = kDcThreads / 64;
constexpr int kDcMidBytes = 32 * 1024;  // n * I staged in LDS from E4M3: ST = 8 uint4 per thread
constexpr int kDcMidBytesMax = 48 * 1024;  // ST = 12: n up to 192 at I = 256 (the shared expert as a ninth slot)
constexpr int kDcPad = 16;              // LDS bytes after each staged mid row

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

size_t down_combine_lds_bytes(int64_t n, int64_t I, bool mid_lds, bool mid_bf16) {
  size_t b = (size_t)(n + 1) * 16 * 4;
  if (mid_lds) b += (size_t)n * ((mid_bf16 ? 2 : 1) * I + kDcPad) + (size_t)n * (I / 128) * 4 + (size_t)n * 4;
  return b;
}

template <int NB, int D, bool MID_LDS, int ST = 8>
__global__ __launch_bounds__(kDcThreads) void down_combine_kernel(
    const uint8_t* __restrict__ midq, const float* __restrict__ mids, const uint8_t* __restrict__ w2, const uint8_t* __restrict__ s2, const int* __restrict__ sorted_entry,
    const int4* __restrict__ tiles, const int* __restrict__ meta, int H, int k, int M, int cw,
    const float* __restrict__ topk_w, const float* __restrict__ ys, uint16_t* __restrict__ out) {
  constexpr int I = NB * 128;
  constexpr bool A16 = ST == 8;  // mid staged widened to bf16 (else E4M3, widened at each read)
  constexpr int LDA = (A16 ? 2 : 1) * I + kDcPad;  // bytes per staged mid row; the pad spreads 16 rows over the banks
  extern __shared__ __align__(16) uint8_t dyn[];
  const int n = M * k;
  float* yl = reinterpret_cast<float*>(dyn);            // [n + 1][16]; row n takes dropped rows
  uint8_t* ml = reinterpret_cast<uint8_t*>(yl + (n + 1) * 16);  // [n][LDA]  (MID_LDS) bf16 or E4M3 mid
  float* msl = reinterpret_cast<float*>(ml + n * LDA);  // [n][NB]   (MID_LDS)
  int* sel = reinterpret_cast<int*>(msl + n * NB);      // [n]       (MID_LDS) sorted_entry
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * cw;
  const int rc = min(r, cw - 1);  // the lane's weight column
  const int nt = meta[0];
  const int per = (nt + kDcWaves - 1) / kDcWaves;
  const int base = wave * per;                                    // this wave's tiles [base, base + my)
  const int my = max(0, min(per, nt - base));

  // ---- descriptors of the wave's first D tiles, then the staging loads
  // (both from L2); the weight loads wait only for the descriptors, the LDS
  // staging waits for its loads after the weight loads have gone out.
  // Slots past the wave's run repeat its last tile (computed again: the
  // same values to the same places); a wave without tiles loads tile 0 and
  // computes nothing. The loads are unconditional so that every later wait
  // counts exactly.
  int4 T[D];
#pragma unroll
  for (int d = 0; d < D; ++d) T[d] = tiles[my > 0 ? base + min(d, my - 1) : 0];
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kSt = MID_LDS ? ST : 1;
  uint4 st[kSt];
  constexpr int kSs = ST == 8 ? 1 : 2;  // mid scales and entries a thread stages (n * NB <= kSs * kDcThreads)
  float sts[kSs];
  int ste[kSs];
  if (MID_LDS) {
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
  if (MID_LDS) {
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
  // goes through full batches (every reload is a new tile), then the tail.
  if (my > 0 && my <= D) {
#pragma unroll
    for (int d = 0; d < D; d += 2) {
      compute(T[d], S[d]);
      if (d + 1 < D) compute(T[d + 1], S[d + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if (my > D) {
    int i0 = 0;
    for (; i0 + 2 * D <= my; i0 += D) {
#pragma unroll
      for (int d = 0; d < D; d += 2) {  // two independent tiles per step
        const int4 tn0 = tiles[base + i0 + D + d];
        const int4 tn1 = tiles[base + i0 + D + min(d + 1, D - 1)];
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
    // the slots hold tiles i0 .. i0 + D - 1 (past my: repeats of the last);
    // fewer than D tiles remain after them
#pragma unroll
    for (int d = 0; d < D; d += 2) {
      compute(T[d], S[d]);
      if (d + 1 < D) compute(T[d + 1], S[d + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int rest = my - i0 - D;  // tiles after the slots' ones: fewer than D
    if (rest > 0) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (d < rest) {
          T[d] = tiles[base + i0 + D + d];
          load(T[d], S[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int d = 0; d < D; ++d)
        if (d < rest) compute(T[d], S[d]);
    }
  }
  __syncthreads();
  // out[t, c0 + 2p .. + 2): float64 products and sum in slot order (+ shared), one bf16 rounding
  const int pairs = cw >> 1;
  for (int idx = tid; idx < M * pairs; idx += kDcThreads) {
    const int t = idx / pairs, cc = 2 * (idx - t * pairs);
    double a0 = 0.0, a1 = 0.0;
    for (int j = 0; j < k; ++j) {
      const double wj = (double)topk_w[t * k + j];
      const float* py = yl + (t * k + j) * 16 + cc;
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

// out[t, c..c+3]: float64 products and sum in slot order (+ shared), then
// bf16. A thread per 4 columns: consecutive lanes read consecutive 16 bytes
// of a y row, so each load instruction covers whole cache lines.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const float* __restrict__ w,
                                                      const float* __restrict__ ys, int M, int H, int k,
                                                      uint16_t* __restrict__ out) {
  const int per_tok = H / 4;
  const int64_t total = (int64_t)M * per_tok;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / per_tok);
    const int c = (int)(i % per_tok) * 4;
    double acc[4] = {0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const double wj = (double)w[(size_t)t * k + j];
      // y is read once: non-temporal loads keep it from displacing cached lines
      const v4f a = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(y + ((size_t)t * k + j) * H + c));
      acc[0] += wj * (double)a[0]; acc[1] += wj * (double)a[1]; acc[2] += wj * (double)a[2]; acc[3] += wj * (double)a[3];
    }
    if (ys) {
      const float4 a = *reinterpret_cast<const float4*>(ys + (size_t)t * H + c);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    }
    const uint32_t o0 = bf16_rne_from_double(acc[0]) | (bf16_rne_from_double(acc[1]) << 16);
    const uint32_t o1 = bf16_rne_from_double(acc[2]) | (bf16_rne_from_double(acc[3]) << 16);
    *reinterpret_cast<uint2*>(out + (size_t)t * H + c) = make_uint2(o0, o1);
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
  const bool mid_lds = n * I <= kDcMidBytesMax && n * (I / 128) <= 2 * kDcThreads && n <= 2 * kDcThreads;
  const bool wide = n * I > kDcMidBytes;  // 12 staging registers a thread instead of 8
  const size_t lds = down_combine_lds_bytes(n, I, mid_lds, mid_lds && !wide);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const float* ys = p->s.shared_I > 0 ? wsp<float>(p, p->L.sh_y) : nullptr;
  const int cw = down_combine_cols(H, p->num_cus);
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(H / cw), dim3(kDcThreads), lds, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint8_t*>(a.s2), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), H, (int)p->s.top_k, (int)a.M, cw, wsp<float>(p, p->L.topk_w), ys,
                    reinterpret_cast<uint16_t*>(a.out));
  };
  // weights of D tiles in flight per wave; fewer when the slots also carry mid rows
  switch (I / 128) {
    case 1: return !mid_lds ? go(down_combine_kernel<1, 6, false>)
                   : wide   ? go(down_combine_kernel<1, 8, true, 12>) : go(down_combine_kernel<1, 8, true>);
    case 2: return !mid_lds ? go(down_combine_kernel<2, 3, false>)
                   : wide   ? go(down_combine_kernel<2, 8, true, 12>) : go(down_combine_kernel<2, 8, true>);
    case 3: return !mid_lds ? go(down_combine_kernel<3, 2, false>)
                   : wide   ? go(down_combine_kernel<3, 5, true, 12>) : go(down_combine_kernel<3, 5, true>);
    case 4: return !mid_lds ? go(down_combine_kernel<4, 2, false>)
                   : wide   ? go(down_combine_kernel<4, 4, true, 12>) : go(down_combine_kernel<4, 4, true>);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int H = (int)p->s.H;
  const int64_t total = a.M * (H / 4);
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 8192);
  const float* ys = p->s.shared_I > 0 ? wsp<float>(p, p->L.sh_y) : nullptr;
  return launch_k(combine_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<float>(p, p->L.y),
                  wsp<float>(p, p->L.topk_w), ys, (int)a.M, H, (int)p->s.top_k, reinterpret_cast<uint16_t*>(a.out));
}

}  // namespace qmoe
