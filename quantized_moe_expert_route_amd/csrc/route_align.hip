// Routing (top-k + weights), x -> MXFP4, and the stable expert-major sort.
//
// Routing: "glm53: FP8 mid hand-off, early split rows, per-row up/gate jobs,
// ..." (Modifications table, row "per-row up/gate jobs", and its commit):
// top-8 by rounds, each round a wave maximum of the lane heads, a tie going
// to the lower expert ID. Here a wave routes one token; every round is one
// 64-bit wave maximum over keys (order-preserving logit bits, ~expert) so a
// tie resolves to the lower ID inside the same compare.
//
// x -> MXFP4 happens once per token in the same launch (the pages' frontend
// converts activations next to the route sort: "IQ2R: load GLM-5.3 packed MoE
// checkpoints ...", status comment "paired FP8 conversion in the frontend").
//
// Sort: the entries (t, j) of each expert in ascending t, so each expert's
// weights are read once for all its rows ("glm53_flash: Score a verify
// request's index tiles once for its rows", commit "Run verify steps of up
// to 16 rows": expert-major MoE). Route waves set bit t of expert e's row in
// a bitmap; the align pass turns per-row prefix popcounts into each entry's
// rank, which is deterministic and needs no ordering between waves.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

template <int EC>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int E, int k, int H,
    float scaling, int* __restrict__ topk_ids, float* __restrict__ topk_w,
    uint32_t* __restrict__ bitmap, int words, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + wave; t < M; t += gridDim.x * 4) {
    // ---- top-k
    uint64_t key[EC];
#pragma unroll
    for (int c = 0; c < EC; ++c) {
      int e = lane + 64 * c;
      key[c] = e < E ? ((uint64_t)order_key(logits[(size_t)t * E + e]) << 32) | (0xFFFFFFFFu - (uint32_t)e) : 0;
    }
    uint32_t sel_e = 0;
    float sel_l = 0.f;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int c = 0; c < EC; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int c = 0; c < EC; ++c)
        if (key[c] == best) key[c] = 0;
      if (lane == j) {
        sel_e = 0xFFFFFFFFu - (uint32_t)best;
        sel_l = key_to_float((uint32_t)(best >> 32));
      }
    }
    // ---- weights: sigmoid scores, renormalised over the k slots, scaled
    float sig = 0.f;
    if (lane < k) sig = (float)(1.0 / (1.0 + exp(-(double)sel_l)));
    float S = 0.f;
    for (int j = 0; j < k; ++j) S += __shfl(sig, j, 64);
    if (lane < k) {
      float w = __fdiv_rn(sig, S + 1e-20f) * scaling;
      topk_ids[(size_t)t * k + lane] = (int)sel_e;
      topk_w[(size_t)t * k + lane] = w;
      atomicOr(&bitmap[(size_t)sel_e * words + (t >> 5)], 1u << (t & 31));
    }
    // ---- x -> MXFP4: per 32-block, E8M0 = floor(log2 amax) - 2, E2M1 RNE
    const uint16_t* xr = x + (size_t)t * H;
    const int nblk = H >> 5;
    for (int b = lane; b < nblk; b += 64) {
      uint32_t w32[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 v = ld16(xr + b * 32 + q * 8);
        w32[4 * q + 0] = v.x; w32[4 * q + 1] = v.y; w32[4 * q + 2] = v.z; w32[4 * q + 3] = v.w;
      }
      uint32_t amax = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        amax = max(amax, w32[i] & 0x7FFFu);
        amax = max(amax, (w32[i] >> 16) & 0x7FFFu);
      }
      const uint32_t sc = mx_scale_code(amax);
      const int sh = 127 - (int)sc;
      uint32_t packed[4] = {0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float f0 = ldexpf(__uint_as_float(w32[i] << 16), sh);
        float f1 = ldexpf(__uint_as_float(w32[i] & 0xFFFF0000u), sh);
        uint32_t byte = e2m1_code(f0) | (e2m1_code(f1) << 4);
        packed[i >> 2] |= byte << (8 * (i & 3));
      }
      *reinterpret_cast<uint4*>(xq + (size_t)t * (H >> 1) + b * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      xs[(size_t)t * nblk + b] = (uint8_t)sc;
    }
  }
}

// Exclusive prefix over the block (blockDim.x == 1024): returns the prefix
// of v and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? s_tmp[lane] : 0;
    int wi = w;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      int n = __shfl_up(wi, o, 64);
      if (lane >= o) wi += n;
    }
    if (lane < 16) s_tmp[16 + lane] = wi - w;
    if (lane == 15) s_tmp[32] = wi;
  }
  __syncthreads();
  int r = s_tmp[16 + wave] + incl - v;
  *total = s_tmp[32];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void align_kernel(
    const int* __restrict__ topk_ids, int M, int E, int k, uint32_t* __restrict__ bitmap,
    int* __restrict__ pre, int words, int* __restrict__ count, int* __restrict__ offset,
    int* __restrict__ sorted_entry, int4* __restrict__ tiles, int* __restrict__ meta) {
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // 1. per expert row: prefix popcount of each bitmap word, and the row total
  for (int e = wave; e < E; e += 16) {
    int carry = 0;
    for (int w0 = 0; w0 < words; w0 += 64) {
      const int w = w0 + lane;
      const uint32_t bits = w < words ? bitmap[(size_t)e * words + w] : 0u;
      const int c = __popc(bits);
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(incl, o, 64);
        if (lane >= o) incl += n;
      }
      if (w < words) pre[(size_t)e * words + w] = carry + incl - c;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_cnt[e] = carry;
  }
  __syncthreads();
  // 2. offsets and tiles of kTileRows sorted rows per expert
  const int c = tid < E ? s_cnt[tid] : 0;
  const int nt = (c + kTileRows - 1) / kTileRows;
  int total_rows, total_tiles;
  const int off = block_exclusive_scan(c, s_tmp, &total_rows);
  const int toff = block_exclusive_scan(nt, s_tmp, &total_tiles);
  if (tid < E) {
    count[tid] = c;
    offset[tid] = off;
    s_off[tid] = off;
    for (int i = 0; i < nt; ++i) {
      const int r0 = off + i * kTileRows;
      tiles[toff + i] = make_int4(tid, r0, min(r0 + kTileRows, off + c), 0);
    }
  }
  if (tid == 0) {
    offset[E] = total_rows;
    meta[0] = total_tiles;
  }
  __syncthreads();
  // 3. each entry's slot in its expert's run: rows of earlier tokens first
  const int n = M * k;
  for (int i = tid; i < n; i += 1024) {
    const int e = topk_ids[i];
    const int t = i / k;
    const size_t wi = (size_t)e * words + (t >> 5);
    const int rank = pre[wi] + __popc(bitmap[wi] & ((1u << (t & 31)) - 1u));
    sorted_entry[s_off[e] + rank] = i;
  }
  __syncthreads();
  // 4. leave the bitmap zero for the next call
  for (int i = tid; i < E * words; i += 1024) bitmap[i] = 0u;
}

__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<uint4*>(ptr), n16);
  return hipGetLastError();
}

hipError_t launch_route(const moe_plan* p, const CallArgs& a) {
  const int M = (int)a.M, E = (int)p->s.E, k = (int)p->s.top_k, H = (int)p->s.H;
  const int blocks = (int)std::min<int64_t>((a.M + 3) / 4, 2048);
  const int words = (int)((a.M + 31) / 32);
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, a.stream, a.logits,
                       reinterpret_cast<const uint16_t*>(a.x), M, E, k, H, p->s.routed_scaling,
                       wsp<int>(p, p->L.topk_ids), wsp<float>(p, p->L.topk_w),
                       wsp<uint32_t>(p, p->X.bitmap), words, wsp<uint8_t>(p, p->L.xq),
                       wsp<uint8_t>(p, p->L.xs));
  };
  const int ec = (E + 63) / 64;
  if (ec <= 1) args(route_kernel<1>);
  else if (ec <= 2) args(route_kernel<2>);
  else if (ec <= 4) args(route_kernel<4>);
  else if (ec <= 8) args(route_kernel<8>);
  else args(route_kernel<16>);
  return hipGetLastError();
}

hipError_t launch_align(const moe_plan* p, const CallArgs& a) {
  const int words = (int)((a.M + 31) / 32);
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(1024), 0, a.stream, wsp<int>(p, p->L.topk_ids),
                     (int)a.M, (int)p->s.E, (int)p->s.top_k, wsp<uint32_t>(p, p->X.bitmap),
                     wsp<int>(p, p->X.pre), words, wsp<int>(p, p->L.count), wsp<int>(p, p->L.offset),
                     wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles), wsp<int>(p, p->X.meta));
  return hipGetLastError();
}

}  // namespace qmoe
