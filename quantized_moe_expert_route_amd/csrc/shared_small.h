// The block-FP8 shared expert inside the small-token launches (up to
// kSmallM tokens, E4M3 mid): no launch of its own. The routed launches take
// its parts as extra work:
//   route launch    x -> E4M3 per 128 with an fp32 scale (extra workgroups)
//   gate/up launch  block partials of gate and up (extra workgroups)
//   mid launch      the partials summed in block order, SiLU(g) * u, h -> E4M3
//                   per 128 (extra waves)
//   down launch     each workgroup's output columns of the shared down, added
//                   as the last term of the combine
// "[HIP] IQ2R: GLM-5.3 packed MoE path for TP4/TP8 on gfx950" (Summary: the
// shared expert rides the routed launches as one more slot) and "IQ2R: load
// GLM-5.3 packed MoE checkpoints with TP slicing" (Summary: the shared expert
// keeps its block-FP8 format).
//
// Arithmetic: the same as the separate shared-expert pass. A 128-K block sum
// of E4M3 x E4M3 products is formed in float64 on the vector ALUs: every
// product of two E4M3 values is a multiple of 2^-18 below 448^2, so every
// partial sum of a block (< 2^25) is exact in float64 in any order. The block
// sum times (activation scale x weight scale) is rounded once (t), and the
// t of a row are added in block order, rounded once to fp32 at the end.
#pragma once

#include "common.h"
#include "internal.h"

namespace qmoe {

// Gate/up work item: 16 outputs (their 16 gate and 16 up weight rows) over
// two 128-K blocks; the x slice of those blocks is staged in LDS as float64.
constexpr int kSsOut = 16;
constexpr int kSsKb = 2;

struct SharedSmall {
  const uint8_t* x8;   // x as E4M3 codes [M, H] (route launch)
  const float* xs;     // x's scales, K-block major [H/128, M]
  const uint8_t* w13;  // gate/up E4M3 codes [2 Is, H], rows [0, Is) gate
  const float* ss13;   // [2 Is/128, H/128]
  const uint8_t* w2;   // down E4M3 codes [H, Is]
  const float* ss2;    // [H/128, Is/128]
  double* part;        // block partials t [M, H/128, 2 Is]
  float* h;            // SiLU(g) * u [M, Is] (kept for inspection)
  uint8_t* hq;         // h as E4M3 codes [M, Is]
  float* hs;           // h's scales, K-block major [Is/128, M]
  int Is;
};

// The plan's buffers of the fused shared expert (all null when the call
// does not fuse it).
inline SharedSmall shared_small(const moe_plan* p, int64_t M) {
  SharedSmall sh{};
  if (!shared_fused(p, M)) return sh;
  const size_t Is = (size_t)p->s.shared_I, H = (size_t)p->s.H;
  const uint8_t* codes = reinterpret_cast<const uint8_t*>(p->ws13) + 9 * Is * H;
  sh.x8 = wsp<uint8_t>(p, p->L.sh_xq);
  sh.xs = wsp<float>(p, p->L.sh_xs);
  sh.w13 = codes;
  sh.ss13 = p->ss13;
  sh.w2 = codes + 2 * Is * H;
  sh.ss2 = p->ss2;
  sh.part = wsp<double>(p, p->X.sh_part);
  sh.h = wsp<float>(p, p->X.sh_h);
  sh.hq = wsp<uint8_t>(p, p->L.sh_hq);
  sh.hs = wsp<float>(p, p->L.sh_hs);
  sh.Is = (int)Is;
  return sh;
}

typedef float v2f __attribute__((ext_vector_type(2)));

// 4 E4M3 codes (one dword) -> float64 (exact)
__device__ __forceinline__ void e4m3x4_f64(uint32_t w, double* d) {
  const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  d[0] = (double)lo[0];
  d[1] = (double)lo[1];
  d[2] = (double)hi[0];
  d[3] = (double)hi[1];
}

// fl64(s * S) with the product rounded on its own (no contraction with a
// following add)
__device__ __forceinline__ double scaled_block(double s, double S) {
#pragma clang fp contract(off)
  return s * S;
}

__device__ __forceinline__ double add_rounded(double acc, double t) {
#pragma clang fp contract(off)
  return acc + t;
}

// Dynamic LDS of a gate/up workgroup that takes shared items: the x slice of
// an item as float64 [M][256] and its 32 weight rows' codes [32][256].
__host__ __device__ constexpr size_t shared_gate_up_lds(int M) {
  return (size_t)M * kSsKb * 128 * sizeof(double) + (size_t)2 * kSsOut * kSsKb * 128;
}

// One gate/up item on a workgroup of 256 threads. The x slice and the
// weight rows are staged in LDS (16-byte loads, x widened to float64 once);
// then thread t takes weight row t % 32 of the item (gate rows first), block
// t / 32 % 2 of its pair and the tokens m = t / 64 + 4 j. Writes
// part[m][b][row] = fl64((xs * ws) * S).
__device__ __forceinline__ void shared_gate_up_item(const SharedSmall& sh, int item, int M, int H, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int nkb = H / 128, npair = nkb / kSsKb;
  const int og = item / npair, kp = item - og * npair;
  const int k0 = kp * kSsKb * 128;  // first K of the slice
  const int Is = sh.Is;
  double* sx = reinterpret_cast<double*>(lds);                    // [M][256]
  uint8_t* swl = lds + (size_t)M * kSsKb * 128 * sizeof(double);  // [32][256] codes
  // weight rows: 32 x 16 chunks of 16 bytes, two a thread
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + 256 * q, rr = i >> 4, c = 16 * (i & 15);
    const int wrow = rr < kSsOut ? og * kSsOut + rr : Is + og * kSsOut + (rr - kSsOut);
    *reinterpret_cast<uint4*>(swl + rr * 256 + c) = ld16(sh.w13 + (size_t)wrow * H + k0 + c);
  }
  {
    const int m = tid >> 4, c = 16 * (tid & 15);  // up to 16 tokens x 256 columns
    if (m < M) {
      const uint4 v = ld16(sh.x8 + (size_t)m * H + k0 + c);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double d[4];
        e4m3x4_f64(w[q], d);
        *reinterpret_cast<double2*>(&sx[m * 256 + c + 4 * q]) = make_double2(d[0], d[1]);
        *reinterpret_cast<double2*>(&sx[m * 256 + c + 4 * q + 2]) = make_double2(d[2], d[3]);
      }
    }
  }
  __syncthreads();
  const int r = tid & 31, bb = (tid >> 5) & 1, mq = tid >> 6;
  const int wrow = r < kSsOut ? og * kSsOut + r : Is + og * kSsOut + (r - kSsOut);
  double S[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
  for (int i = 0; i < 32; ++i) {  // 4 codes at a time
    double wd[4];
    e4m3x4_f64(*reinterpret_cast<const uint32_t*>(swl + r * 256 + 128 * bb + 4 * i), wd);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = mq + 4 * j;
      if (m < M) {
        const double* px = sx + m * 256 + 128 * bb + 4 * i;
        const double2 x01 = *reinterpret_cast<const double2*>(px);
        const double2 x23 = *reinterpret_cast<const double2*>(px + 2);
        S[j] = fma(x01.x, wd[0], S[j]);
        S[j] = fma(x01.y, wd[1], S[j]);
        S[j] = fma(x23.x, wd[2], S[j]);
        S[j] = fma(x23.y, wd[3], S[j]);
      }
    }
  }
  const int b = kp * kSsKb + bb;
  const double sw = (double)sh.ss13[(size_t)(wrow / 128) * nkb + b];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = mq + 4 * j;
    if (m < M)
      sh.part[((size_t)m * nkb + b) * (2 * Is) + wrow] = scaled_block((double)sh.xs[(size_t)b * M + m] * sw, S[j]);
  }
  __syncthreads();  // the LDS is reused by the workgroup's next item
}

// One wave: token m, columns 128 c + 2 lane (+1) of h: the gate and up
// partials added in block order, rounded to fp32, SiLU(g) * u, then the
// block's E4M3 codes and scale (the routed mid's rule).
__device__ __forceinline__ void shared_mid_wave(const SharedSmall& sh, int m, int c, int M, int H) {
  const int lane = threadIdx.x & 63;
  const int nkb = H / 128, Is = sh.Is;
  const int col = 128 * c + 2 * lane;
  double g0 = 0.0, g1 = 0.0, u0 = 0.0, u1 = 0.0;
  const double* p = sh.part + (size_t)m * nkb * (2 * Is) + col;
  for (int b0 = 0; b0 < nkb; b0 += 4) {  // (H/128 is a multiple of 4)
    double2 gv[4], uv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = min(b0 + i, nkb - 1);
      gv[i] = *reinterpret_cast<const double2*>(p + (size_t)b * (2 * Is));
      uv[i] = *reinterpret_cast<const double2*>(p + (size_t)b * (2 * Is) + Is);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (b0 + i < nkb) {
        g0 = add_rounded(g0, gv[i].x);
        g1 = add_rounded(g1, gv[i].y);
        u0 = add_rounded(u0, uv[i].x);
        u1 = add_rounded(u1, uv[i].y);
      }
    }
  }
  const float h0 = silu_mul((float)g0, (float)u0), h1 = silu_mul((float)g1, (float)u1);
  *reinterpret_cast<float2*>(sh.h + (size_t)m * Is + col) = make_float2(h0, h1);
  const float amax = wave_max(fmaxf(fabsf(h0), fabsf(h1)));
  const float sc = __fdiv_rn(amax, 448.0f);
  uint32_t c0 = 0, c1 = 0;
  if (sc > 0.f) {
    c0 = e4m3_code(__fdiv_rn(h0, sc));
    c1 = e4m3_code(__fdiv_rn(h1, sc));
  }
  *reinterpret_cast<uint16_t*>(sh.hq + (size_t)m * Is + col) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) sh.hs[(size_t)c * M + m] = sc;
}

// LDS bytes the shared down of one down workgroup needs (M <= 16 tokens,
// up to 16 columns): staged h codes and weight rows, the block terms and
// the outputs.
__host__ __device__ constexpr size_t shared_down_lds(int Is) {
  return (size_t)16 * Is + (size_t)16 * Is + (size_t)16 * 16 * 4 * 8 + (size_t)16 * 16 * 4;
}

// The shared down for output columns [c0, c0 + cw) of a 256-thread
// workgroup: ys[m * 16 + cc] = fl32(sum over blocks, in order, of
// fl64((hs * ws) * S)). `lds` holds shared_down_lds(Is) bytes.
__device__ __forceinline__ void shared_down_cols(const SharedSmall& sh, int M, int c0, int cw, uint8_t* lds,
                                                 float* __restrict__ ys) {
  const int tid = threadIdx.x;
  const int Is = sh.Is, nb = Is / 128;
  uint8_t* hql = lds;                                              // [16][Is] h codes
  uint8_t* wl = hql + (size_t)16 * Is;                             // [16][Is] weight rows (columns c0 ..)
  double* tl = reinterpret_cast<double*>(wl + (size_t)16 * Is);   // [16 m][16 cc][4 b]
  // stage: 16-byte chunks, h rows first, then the weight rows
  const int cpr = Is / 16, nh = M * cpr, nw = cw * cpr;
  for (int i = tid; i < nh + nw; i += 256) {
    if (i < nh) {
      const int m = i / cpr, c = i - m * cpr;
      *reinterpret_cast<uint4*>(hql + (size_t)m * Is + 16 * c) = ld16(sh.hq + (size_t)m * Is + 16 * c);
    } else {
      const int j = i - nh, cc = j / cpr, c = j - cc * cpr;
      *reinterpret_cast<uint4*>(wl + (size_t)cc * Is + 16 * c) = ld16(sh.w2 + (size_t)(c0 + cc) * Is + 16 * c);
    }
  }
  __syncthreads();
  {
    const int cc = tid & 15, b = (tid >> 4) & 3, mq = tid >> 6;
    if (cc < cw && b < nb) {
      double S[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
      for (int i = 0; i < 32; ++i) {  // 4 codes at a time
        double wd[4];
        e4m3x4_f64(*reinterpret_cast<const uint32_t*>(wl + (size_t)cc * Is + 128 * b + 4 * i), wd);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = mq + 4 * j;
          if (m < M) {
            double hd[4];
            e4m3x4_f64(*reinterpret_cast<const uint32_t*>(hql + (size_t)m * Is + 128 * b + 4 * i), hd);
#pragma unroll
            for (int e = 0; e < 4; ++e) S[j] = fma(hd[e], wd[e], S[j]);
          }
        }
      }
      const double sw = (double)sh.ss2[(size_t)((c0 + cc) / 128) * nb + b];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = mq + 4 * j;
        if (m < M) tl[(m * 16 + cc) * 4 + b] = scaled_block((double)sh.hs[(size_t)b * M + m] * sw, S[j]);
      }
    }
  }
  __syncthreads();
  {
    const int m = tid >> 4, cc = tid & 15;
    if (m < M && cc < cw) {
      double acc = 0.0;
      for (int b = 0; b < nb; ++b) acc = add_rounded(acc, tl[(m * 16 + cc) * 4 + b]);
      ys[m * 16 + cc] = (float)acc;
    }
  }
  __syncthreads();
}

}  // namespace qmoe
