// The block-FP8 shared expert inside the small-token launches (up to
// kSmallM tokens, E4M3 mid): no launch of its own. The routed launches take
// its parts as extra work:
//   route launch    block partials of gate and up (extra workgroups, beside
//                   the routing workgroup; each quantizes its x slice to
//                   E4M3 per 128 with an fp32 scale)
//   mid launch      the partials summed in block order, SiLU(g) * u, h -> E4M3
//                   per 128 (extra workgroups)
//   down launch     each workgroup's output columns of the shared down, added
//                   as the last term of the combine (its operands fetched
//                   before the routed weights)
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
// KB 128-K blocks (2 or 4: the fewer, the more items; the launch takes 4
// when 2 would need more workgroups than the chip holds at once).
constexpr int kSsOut = 16;

struct SharedSmall {
  uint8_t* x8;         // x as E4M3 codes [M, H] (route launch)
  float* xs;           // x's scales, K-block major [H/128, M]
  const uint8_t* w13;  // gate/up E4M3 codes [2 Is, H], rows [0, Is) gate
  const float* ss13;   // [2 Is/128, H/128]
  const uint8_t* w2;   // down E4M3 codes [H, Is]
  const float* ss2;    // [H/128, Is/128]
  double* part;        // block partials t [M, H/128, 2 Is]
  float* h;            // SiLU(g) * u [M, Is] (kept for inspection)
  uint8_t* hq;         // h as E4M3 codes [M, Is]
  float* hs;           // h's scales, K-block major [Is/128, M]
  int Is;
  int kb;              // K-blocks per gate/up item (2 or 4)
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
  sh.kb = 2;
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

// Dynamic LDS of a route workgroup that takes shared gate/up items of KB
// blocks: the x slice as float64 [16][128 KB], the 32 weight rows' codes
// [32][128 KB] and the x scales [16][KB].
__host__ __device__ constexpr size_t shared_gate_up_lds(int KB) {
  return (size_t)16 * 128 * KB * sizeof(double) + (size_t)2 * kSsOut * (128 * KB + 16) + 16 * KB * sizeof(float);
}

// Gate/up items of a 1024-thread workgroup: item = (16 outputs, KB blocks).
// x's slice is quantized here, per token and 128-block (s = fl32(amax /
// 448), codes E4M3(fl32(x / s)); the items of the first 16 outputs also
// store the codes and scales), and widened to float64 in LDS beside the 32
// weight rows' codes. Then thread t takes weight row t % 32 of the item
// (gate rows first), block t / 32 % KB and the tokens t / (32 KB) + j *
// 32 / KB. Writes part[m][b][row] = fl64((xs * ws) * S).
template <int KB>
__device__ __forceinline__ void shared_gate_up_item(const SharedSmall& sh, const uint16_t* __restrict__ x, int item,
                                                    int M, int H, uint8_t* lds) {
  constexpr int KW = 128 * KB;       // K of the slice
  constexpr int SW = KW + 16;        // LDS bytes per weight row (the pad spreads 16-byte reads over the banks)
  constexpr int G = 1024 / (32 * KB);  // token groups
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nkb = H / 128, nslice = nkb / KB;
  const int og = item / nslice, kp = item - og * nslice;
  const int k0 = kp * KW;  // first K of the slice
  const int Is = sh.Is;
  double* sx = reinterpret_cast<double*>(lds);                      // [16][KW]
  uint8_t* swl = lds + (size_t)16 * KW * sizeof(double);            // [32][SW] codes
  float* ssc = reinterpret_cast<float*>(swl + 2 * kSsOut * SW);     // [16][KB] x scales
  // weight rows: 32 x KW / 16 chunks of 16 bytes
  if (tid < 2 * kSsOut * KW / 16) {
    const int rr = tid / (KW / 16), c = 16 * (tid % (KW / 16));
    const int wrow = rr < kSsOut ? og * kSsOut + rr : Is + og * kSsOut + (rr - kSsOut);
    *reinterpret_cast<uint4*>(swl + rr * SW + c) = ld16(sh.w13 + (size_t)wrow * H + k0 + c);
  }
  // x: one wave per (token, block) of the slice, two values a lane; the
  // wave's loads (up to four pairs) go out together
  uint32_t xv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pq = wave + 16 * u, m = pq / KB, bb = pq % KB;
    xv[u] = pq < M * KB ? *reinterpret_cast<const uint32_t*>(x + (size_t)m * H + k0 + 128 * bb + 2 * lane) : 0u;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int pq = wave + 16 * u, m = pq / KB, bb = pq % KB;
    if (pq < M * KB) {
      const float v0 = __uint_as_float(xv[u] << 16), v1 = __uint_as_float(xv[u] & 0xFFFF0000u);
      const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
      const float sc = __fdiv_rn(amax, 448.0f);
      const uint32_t c01 = sc > 0.f ? e4m3_pack2(__fdiv_rn(v0, sc), __fdiv_rn(v1, sc)) : 0u;
      const v2f d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c01, 1.0f, false);
      *reinterpret_cast<double2*>(&sx[m * KW + 128 * bb + 2 * lane]) = make_double2((double)d[0], (double)d[1]);
      if (lane == 0) ssc[m * KB + bb] = sc;
      if (og == 0) {
        *reinterpret_cast<uint16_t*>(sh.x8 + (size_t)m * H + k0 + 128 * bb + 2 * lane) = (uint16_t)c01;
        if (lane == 0) sh.xs[(size_t)(k0 / 128 + bb) * M + m] = sc;
      }
    }
  }
  __syncthreads();
  const int r = tid & 31, bb = (tid >> 5) % KB, mg = tid / (32 * KB);
  if (mg < M) {
    const int wrow = r < kSsOut ? og * kSsOut + r : Is + og * kSsOut + (r - kSsOut);
    double S[16 / G];
#pragma unroll
    for (int j = 0; j < 16 / G; ++j) S[j] = 0.0;
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {  // 16 codes at a time
      const uint4 w4 = *reinterpret_cast<const uint4*>(swl + r * SW + 128 * bb + 16 * i);
      const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int j = 0; j < 16 / G; ++j) {
        const int m = mg + G * j;
        if (m < M) {
          const double* px = sx + m * KW + 128 * bb + 16 * i;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            double wd[4];
            e4m3x4_f64(ww[q], wd);
            const double2 x01 = *reinterpret_cast<const double2*>(px + 4 * q);
            const double2 x23 = *reinterpret_cast<const double2*>(px + 4 * q + 2);
            S[j] = fma(x01.x, wd[0], S[j]);
            S[j] = fma(x01.y, wd[1], S[j]);
            S[j] = fma(x23.x, wd[2], S[j]);
            S[j] = fma(x23.y, wd[3], S[j]);
          }
        }
      }
    }
    const int b = kp * KB + bb;
    const double sw = (double)sh.ss13[(size_t)(wrow / 128) * nkb + b];
#pragma unroll
    for (int j = 0; j < 16 / G; ++j) {
      const int m = mg + G * j;
      if (m < M)
        sh.part[((size_t)m * nkb + b) * (2 * Is) + wrow] = scaled_block((double)ssc[m * KB + bb] * sw, S[j]);
    }
  }
  __syncthreads();  // the LDS is reused by the workgroup's next item
}

// Token m, columns [128 c, 128 c + 128) of h on a group of 256 threads (tid
// 0..255; the workgroup's barriers are reached by all its threads, valid or
// not): thread t adds the partials of column 128 c + t % 128 of gate
// (t < 128) or of up in block order, rounded to fp32; then SiLU(g) * u and
// the block's E4M3 codes and scale (the routed mid's rule). `u_lds` holds
// 130 floats. A group without an item (valid false) only takes the barriers.
__device__ __forceinline__ void shared_mid_block(const SharedSmall& sh, int m, int c, int M, int H, float* u_lds,
                                                 int tid, bool valid) {
  if (!valid) {
    __syncthreads();
    __syncthreads();
    __syncthreads();
    return;
  }
  const int nkb = H / 128, Is = sh.Is;
  const int col = 128 * c + (tid & 127);
  const double* p = sh.part + (size_t)m * nkb * (2 * Is) + (tid >= 128 ? Is : 0) + col;
  double acc = 0.0;
  constexpr int kB = 16;  // partials a thread has in flight
  for (int b0 = 0; b0 < nkb; b0 += kB) {
    double v[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) v[i] = p[(size_t)min(b0 + i, nkb - 1) * (2 * Is)];
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (b0 + i < nkb) acc = add_rounded(acc, v[i]);
  }
  if (tid >= 128) u_lds[tid - 128] = (float)acc;
  __syncthreads();
  float h = 0.f;
  if (tid < 128) {
    h = silu_mul((float)acc, u_lds[tid]);
    sh.h[(size_t)m * Is + col] = h;
    const float wm = wave_max(fabsf(h));
    if ((tid & 63) == 0) u_lds[128 + (tid >> 6)] = wm;
  }
  __syncthreads();
  if (tid < 128) {
    const float amax = fmaxf(u_lds[128], u_lds[129]);
    const float sc = __fdiv_rn(amax, 448.0f);
    const uint32_t code = sc > 0.f ? e4m3_pack2(__fdiv_rn(h, sc), 0.f) & 0xFFu : 0u;
    sh.hq[(size_t)m * Is + col] = (uint8_t)code;
    if (tid == 0) sh.hs[(size_t)c * M + m] = sc;
  }
  __syncthreads();  // u_lds is reused by the workgroup's next block
}

// LDS bytes the shared down of one down workgroup needs (M <= 16 tokens,
// up to 16 columns): staged h codes and weight rows, the block terms and
// the outputs.
__host__ __device__ constexpr size_t shared_down_lds(int Is) {
  return (size_t)16 * Is + (size_t)16 * (Is + 16) + (size_t)16 * 16 * 4 * 8 + (size_t)16 * 16 * 4;
}

// What the shared down of one down workgroup fetches before the routed
// weights: its cw weight rows as 16-byte chunks (chunk tid + 256 q in v[q]:
// at most 16 * 512 / 16 = 2 * 256), the first 256 chunks of its h rows
// (the rest, if any, are read at the end) and the scales of the thread's
// block terms (thread t: column t % 16, block t / 16 % 4, tokens t / 64 +
// 4 j).
constexpr int kSdPre = 2;
struct SharedDownPre {
  uint4 v[kSdPre];
  uint4 h;
  float sw;
  float hs[4];
};
__device__ __forceinline__ void shared_down_fetch(const SharedSmall& sh, int M, int c0, int cw, SharedDownPre& pre) {
  const int tid = threadIdx.x, Is = sh.Is, nb = Is / 128;
  const int cpr = Is / 16, nw = cw * cpr;
#pragma unroll
  for (int q = 0; q < kSdPre; ++q) {
    const int i = tid + 256 * q;
    if (i < nw) {
      const int cc = i / cpr, c = i - cc * cpr;
      pre.v[q] = ld16(sh.w2 + (size_t)(c0 + cc) * Is + 16 * c);
    }
  }
  if (tid < M * cpr) pre.h = ld16(sh.hq + (size_t)(tid / cpr) * Is + 16 * (tid % cpr));
  const int cc = tid & 15, b = (tid >> 4) & 3, mq = tid >> 6;
  pre.sw = cc < cw && b < nb ? sh.ss2[(size_t)((c0 + cc) / 128) * nb + b] : 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) pre.hs[j] = b < nb && mq + 4 * j < M ? sh.hs[(size_t)b * M + mq + 4 * j] : 0.f;
}

// The shared down for output columns [c0, c0 + cw) of a 256-thread
// workgroup, from the operands shared_down_fetch brought in:
// ys[m * 16 + cc] = fl32(sum over blocks, in order, of fl64((hs * ws) * S)).
// `lds` holds shared_down_lds(Is) bytes.
__device__ __forceinline__ void shared_down_cols(const SharedSmall& sh, int M, int c0, int cw,
                                                 const SharedDownPre& pre, uint8_t* lds, float* __restrict__ ys) {
  const int tid = threadIdx.x;
  const int Is = sh.Is, nb = Is / 128;
  const int WS = Is + 16;                                          // weight row stride (the pad spreads the banks)
  uint8_t* hql = lds;                                              // [16][Is] h codes
  uint8_t* wl = hql + (size_t)16 * Is;                             // [16][WS] weight rows (columns c0 ..)
  double* tl = reinterpret_cast<double*>(wl + (size_t)16 * WS);   // [16 m][16 cc][4 b]
  const int cpr = Is / 16, nh = M * cpr, nw = cw * cpr;
  uint4 hv[2];  // the h rows: at most 16 * 512 / 16 = 2 * 256 chunks, the first 256 fetched already
  hv[0] = pre.h;
  if (tid + 256 < nh) hv[1] = ld16(sh.hq + (size_t)((tid + 256) / cpr) * Is + 16 * ((tid + 256) % cpr));
#pragma unroll
  for (int q = 0; q < kSdPre; ++q) {
    const int i = tid + 256 * q;
    if (i < nw) *reinterpret_cast<uint4*>(wl + (size_t)(i / cpr) * WS + 16 * (i % cpr)) = pre.v[q];
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = tid + 256 * q;
    if (i < nh) *reinterpret_cast<uint4*>(hql + (size_t)(i / cpr) * Is + 16 * (i % cpr)) = hv[q];
  }
  __syncthreads();
  {
    const int cc = tid & 15, b = (tid >> 4) & 3, mq = tid >> 6;
    if (cc < cw && b < nb) {
      double S[4] = {0.0, 0.0, 0.0, 0.0};
      // the thread's 128 weight codes (8 reads of 16 bytes), then each
      // token's 128 h codes (the wave's lanes read the same ones)
      uint4 wv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) wv[i] = *reinterpret_cast<const uint4*>(wl + (size_t)cc * WS + 128 * b + 16 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = mq + 4 * j;
        if (m < M) {
          uint4 hv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[i] = *reinterpret_cast<const uint4*>(hql + (size_t)m * Is + 128 * b + 16 * i);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t ww[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
            const uint32_t hh[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              double wd[4], hd[4];
              e4m3x4_f64(ww[q], wd);
              e4m3x4_f64(hh[q], hd);
#pragma unroll
              for (int e = 0; e < 4; ++e) S[j] = fma(hd[e], wd[e], S[j]);
            }
          }
        }
      }
      const double sw = (double)pre.sw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = mq + 4 * j;
        if (m < M) tl[(m * 16 + cc) * 4 + b] = scaled_block((double)pre.hs[j] * sw, S[j]);
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
