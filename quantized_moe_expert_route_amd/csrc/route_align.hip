// Routing (top-k + weights), x -> MXFP4, and the stable expert-major sort.
//
// Routing: "glm53: FP8 mid hand-off, early split rows, per-row up/gate jobs,
// ..." (Modifications table, row "per-row up/gate jobs", and its commit):
// top-8 by rounds, each round a wave maximum of the lane heads, a tie going
// to the lower expert ID. Here a wave routes one token: each round takes the
// wave maximum of the lanes' best order-preserving logit keys (DPP within
// rows, scalar reads across rows), then the lowest expert ID among the lanes
// holding that key (ballots over the key slots), so a tie resolves to the
// lower ID.
//
// x -> MXFP4 happens once per token in the same launch (the pages' frontend
// converts activations next to the route sort: "IQ2R: load GLM-5.3 packed MoE
// checkpoints ...", status comment "paired FP8 conversion in the frontend").
//
// Sort: the entries (t, j) of each expert in ascending t, so each expert's
// weights are read once for all its rows ("glm53_flash: Score a verify
// request's index tiles once for its rows", commit "Run verify steps of up
// to 16 rows": expert-major MoE). Every token sets bit t of its experts'
// rows of a token bitmap; an entry's rank is the popcount of its row below t,
// so the order is deterministic and needs no ordering between waves. Up to
// kSmallM tokens the bitmap lives in LDS and one workgroup routes, quantizes and
// sorts in a single launch; above that the route launch sets the bits in
// global memory and a one-workgroup align launch ranks the entries.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

// Top-k of one logits row by one wave. Lane j < k receives slot j's expert
// and logit.
// Keys of one logits row: lane l holds experts l + 64c; every real key is > 0.
template <int EC>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int E, int lane, uint32_t (&key)[EC]) {
#pragma unroll
  for (int c = 0; c < EC; ++c) key[c] = lane + 64 * c < E ? order_key(row[lane + 64 * c]) : 0u;
}

// k rounds: the wave's largest key, and of the experts holding it the lowest
// id 64 c + lane (the first slot c with a hit, then its lowest lane, found
// with ballots), which leaves the race.
template <int EC>
__device__ __forceinline__ void topk_wave(uint32_t (&key)[EC], int k, int lane, uint32_t& sel_e, float& sel_l) {
  for (int j = 0; j < k; ++j) {
    uint32_t bk = 0;
#pragma unroll
    for (int c = 0; c < EC; ++c) bk = max(bk, key[c]);
    const uint32_t kmax = wave_max_u32(bk);
    int wc = EC - 1;
    unsigned long long hits = 0;
#pragma unroll
    for (int c = 0; c < EC; ++c) {
      hits = __ballot(key[c] == kmax);
      if (hits) {
        wc = c;
        break;
      }
    }
    const int wl = __builtin_ctzll(hits);
#pragma unroll
    for (int c = 0; c < EC; ++c) key[c] = (lane == wl && c == wc) ? 0u : key[c];
    if (lane == j) {
      sel_e = (uint32_t)(64 * wc + wl);
      sel_l = key_to_float(kmax);
    }
  }
}

// Sigmoid scores of the k selected logits (float64, one rounding), their
// binary32 sum in slot order, w = fl32(fl32(s / (S + 1e-20)) * scaling).
__device__ __forceinline__ float route_weight(float sel_l, int k, int lane, float scaling) {
  float sig = 0.f;
  if (lane < k) sig = (float)(1.0 / (1.0 + exp(-(double)sel_l)));
  float S = 0.f;
  for (int j = 0; j < k; ++j) S += __shfl(sig, j, 64);
  return __fdiv_rn(sig, S + 1e-20f) * scaling;
}

// One token's slots, lane j < k holding slot j's expert and weight. With
// shared_slot the shared expert is the last expert and the last slot
// ("[HIP] IQ2R: GLM-5.3 packed MoE path for TP4/TP8 on gfx950", Summary:
// the shared expert fused as expert 256 of a top-9 call): slots 0..k-2 are
// routed over the first E-1 logits, slot k-1 is expert E-1 with weight 1.
template <int EC>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, float scaling,
                                            int shared_slot, int lane, uint32_t& sel_e, float& w) {
  const int kr = k - shared_slot, er = E - shared_slot;
  uint32_t key[EC];
  float sel_l = 0.f;
  load_keys<EC>(row, er, lane, key);
  topk_wave<EC>(key, kr, lane, sel_e, sel_l);
  w = route_weight(sel_l, kr, lane, scaling);
  if (shared_slot && lane == k - 1) {
    sel_e = (uint32_t)(E - 1);
    w = 1.0f;
  }
}

// One 32-element block of a bf16 row -> 16 bytes of E2M1 + an E8M0 byte.
__device__ __forceinline__ void quant_block_mx(const uint16_t* __restrict__ src, uint8_t* __restrict__ dq,
                                               uint8_t* __restrict__ ds) {
  uint32_t w32[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = ld16(src + q * 8);
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
    const float f0 = ldexpf(__uint_as_float(w32[i] << 16), sh);
    const float f1 = ldexpf(__uint_as_float(w32[i] & 0xFFFF0000u), sh);
    packed[i >> 2] |= (e2m1_code(f0) | (e2m1_code(f1) << 4)) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(dq) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  *ds = (uint8_t)sc;
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

static_assert(kSmallRows < (1 << 16) && kMidM * 16 < (1 << 16), "rows and tiles share one packed scan");

// Offsets (and with_tiles: tiles of kTileRows sorted rows, meta[0]) from
// per-expert counts (thread e holds count c of expert e). Leaves offsets in
// s_off. Tiles are written only where the 16-row-tile gate/up runs (up to
// kMidM tokens), where the row total is below 2^16: rows and tiles then
// share one scan, packed as rows | tiles << 16.
__device__ void write_offsets_tiles(int c, int E, int* s_off, int* s_tmp, int* __restrict__ count,
                                    int* __restrict__ offset, int4* __restrict__ tiles, int* __restrict__ meta,
                                    bool with_tiles = true) {
  const int tid = threadIdx.x;
  const int nt = with_tiles ? (c + kTileRows - 1) / kTileRows : 0;
  int total;
  const int pre = block_exclusive_scan(with_tiles ? c | (nt << 16) : c, s_tmp, &total);
  const int off = with_tiles ? pre & 0xFFFF : pre, toff = pre >> 16;
  const int total_rows = with_tiles ? total & 0xFFFF : total, total_tiles = total >> 16;
  if (tid < E) {
    count[tid] = c;
    offset[tid] = off;
    s_off[tid] = off;
    for (int i = 0; with_tiles && i < nt; ++i) {
      const int r0 = off + i * kTileRows;
      tiles[toff + i] = make_int4(tid, r0, min(r0 + kTileRows, off + c), 0);
    }
  }
  if (tid == 0) {
    offset[E] = total_rows;
    if (with_tiles) meta[0] = total_tiles;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- M <= kSmallM
// Workgroup 0 routes, sorts and writes the tiles; workgroups 1.. quantize x.
template <int EC>
__global__ __launch_bounds__(1024) void route_align_small_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int E, int k, int H, float scaling,
    int* __restrict__ topk_ids, float* __restrict__ topk_w, int* __restrict__ count, int* __restrict__ offset,
    int* __restrict__ sorted_entry, int4* __restrict__ tiles, int* __restrict__ meta, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs, int shared_slot) {
  __shared__ uint32_t s_mask[1024][2];  // expert -> tokens 0..63
  __shared__ int s_ids[64 * 16];
  __shared__ int s_off[1024];
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.x > 0) {
    // x -> MXFP4 is independent of the routing: workgroups 1.. take 64
    // blocks of 32 each, on their own CUs (the conversion is ALU work)
    const int nblk = H >> 5;
    const int bi = (blockIdx.x - 1) * 64 + tid;
    if (tid < 64 && bi < M * nblk) {
      const int t = bi / nblk, b = bi - t * nblk;
      quant_block_mx(x + (size_t)t * H + b * 32, xq + (size_t)t * (H >> 1) + b * 16, xs + (size_t)t * nblk + b);
    }
    return;
  }
  for (int e = tid; e < E; e += 1024) s_mask[e][0] = s_mask[e][1] = 0u;
  __syncthreads();
  // top-k, one wave per token
  for (int t = wave; t < M; t += 16) {
    uint32_t sel_e = 0;
    float w = 0.f;
    route_token<EC>(logits + (size_t)t * E, E, k, scaling, shared_slot, lane, sel_e, w);
    if (lane < k) {
      topk_ids[t * k + lane] = (int)sel_e;
      topk_w[t * k + lane] = w;
      s_ids[t * k + lane] = (int)sel_e;
      atomicOr(&s_mask[sel_e][t >> 5], 1u << (t & 31));
    }
  }
  __syncthreads();
  const int c = tid < E ? __popc(s_mask[tid][0]) + __popc(s_mask[tid][1]) : 0;
  write_offsets_tiles(c, E, s_off, s_tmp, count, offset, tiles, meta);
  for (int i = tid; i < M * k; i += 1024) {
    const int e = s_ids[i], t = i / k;
    const uint32_t lo = s_mask[e][0], hi = s_mask[e][1];
    const int rank = t < 32 ? __popc(lo & ((1u << t) - 1u)) : __popc(lo) + __popc(hi & ((1u << (t - 32)) - 1u));
    sorted_entry[s_off[e] + rank] = i;
  }
}

// ---------------------------------------------------------------- M > kSmallM
// x of one token, 8 elements a lane, 512 a load instruction (whole cache
// lines): the 4 lanes of a 32-block form its E8M0 scale and E2M1 codes (the
// same arithmetic as quant_block_mx), and with SH the 16 lanes of a
// 128-block also form the shared expert's E4M3 codes and fp32 scale, so x is
// read once for both. A unit is kXU loads of one row.
constexpr int kXU = 4;

template <bool SH>
__device__ __forceinline__ void quant_x_unit(const uint16_t* __restrict__ x, int H, int M, int t, int c0, int lane,
                                             uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                             uint8_t* __restrict__ sq, float* __restrict__ ss) {
  uint4 v[kXU];
#pragma unroll
  for (int i = 0; i < kXU; ++i)
    v[i] = c0 + 512 * i < H ? ld16(x + (size_t)t * H + c0 + 512 * i + 8 * lane) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < kXU; ++i) {
    if (c0 + 512 * i >= H) break;  // H is a multiple of 512: a load is all in or all out
    const int e0 = c0 + 512 * i + 8 * lane;
    const uint32_t w32[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t am = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) am = max(am, max(w32[q] & 0x7FFFu, (w32[q] >> 16) & 0x7FFFu));
    // max over the quad (one 32-block)
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, false));
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, false));
    {
      const uint32_t sc = mx_scale_code(am);
      const int sh = 127 - (int)sc;
      uint32_t packed = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float f0 = ldexpf(__uint_as_float(w32[q] << 16), sh);
        const float f1 = ldexpf(__uint_as_float(w32[q] & 0xFFFF0000u), sh);
        packed |= (e2m1_code(f0) | (e2m1_code(f1) << 4)) << (8 * q);
      }
      *reinterpret_cast<uint32_t*>(xq + (size_t)t * (H >> 1) + (e0 >> 1)) = packed;
      if ((lane & 3) == 0) xs[(size_t)t * (H >> 5) + (e0 >> 5)] = (uint8_t)sc;
    }
    if (SH) {
      // on to the 16 lanes of the 128-block (max is order-free: mirrors suffice)
      am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x141, 0xF, 0xF, false));
      am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x140, 0xF, 0xF, false));
      const float sc = __fdiv_rn(__uint_as_float(am << 16), 448.0f);
      uint32_t lo = 0, hi = 0;
      if (sc > 0.f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t c = e4m3_code(__fdiv_rn(__uint_as_float(w32[q] << 16), sc)) |
                             (e4m3_code(__fdiv_rn(__uint_as_float(w32[q] & 0xFFFF0000u), sc)) << 8);
          if (q < 2) lo |= c << (16 * q); else hi |= c << (16 * (q - 2));
        }
      }
      *reinterpret_cast<uint2*>(sq + (size_t)t * H + e0) = make_uint2(lo, hi);
      if ((lane & 15) == 0) ss[(size_t)(e0 >> 7) * M + t] = sc;
    }
  }
}

// Workgroups [0, route_blocks) route, one wave per token (top-k, weights,
// the token's bits in the expert x token bitmap); the rest quantize x, one
// wave per unit of kXU loads of a row. The two roles share no registers.
template <int EC, bool SH>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int E, int k, int H,
    float scaling, int* __restrict__ topk_ids, float* __restrict__ topk_w,
    uint32_t* __restrict__ bitmap, int words, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
    uint8_t* __restrict__ sh_xq, float* __restrict__ sh_xs, int route_blocks, int shared_slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < route_blocks) {
    for (int t = blockIdx.x * 4 + wave; t < M; t += route_blocks * 4) {
      uint32_t sel_e = 0;
      float w = 0.f;
      route_token<EC>(logits + (size_t)t * E, E, k, scaling, shared_slot, lane, sel_e, w);
      if (lane < k) {
        topk_ids[(size_t)t * k + lane] = (int)sel_e;
        topk_w[(size_t)t * k + lane] = w;
        atomicOr(&bitmap[(size_t)sel_e * words + (t >> 5)], 1u << (t & 31));
      }
    }
    return;
  }
  const int upr = (H + 512 * kXU - 1) / (512 * kXU);  // units per row
  const int64_t units = (int64_t)M * upr;
  const int qb = gridDim.x - route_blocks;
  for (int64_t u = (int64_t)(blockIdx.x - route_blocks) * 4 + wave; u < units; u += (int64_t)qb * 4) {
    const int t = (int)(u / upr), c0 = (int)(u - (int64_t)t * upr) * 512 * kXU;
    quant_x_unit<SH>(x, H, M, t, c0, lane, xq, xs, sh_xq, sh_xs);
  }
}

// Work items of the large-token GEMMs, per expert in the order (column
// block, row tile) so that the row tiles sharing a weight block are adjacent:
// gate/up items on tiles of kGuRows rows, down items on tiles of kBigRows.
// One workgroup forms the tile prefixes (write_tile_prefixes); the items
// themselves are written by every workgroup of the placement launch, a
// thread per item, the expert found by binary search of the prefix in LDS
// (one workgroup writing all of them was bound by one CU's store rate).
__device__ void write_tile_prefixes(int c, int E, int n_iblk, int n_nc, int* s_tmp, int* __restrict__ toff,
                                    int* __restrict__ meta) {
  const int tid = threadIdx.x;
  for (int pass = 0; pass < 2; ++pass) {
    const int tr = pass == 0 ? kGuRows : kBigRows;
    const int nt = (c + tr - 1) / tr;
    int total_tiles;
    const int t0 = block_exclusive_scan(nt, s_tmp, &total_tiles);
    if (tid < E) toff[pass * (E + 1) + tid] = t0;
    if (tid == 0) {
      toff[pass * (E + 1) + E] = total_tiles;
      meta[1 + pass] = total_tiles * (pass == 0 ? n_iblk : n_nc);
    }
    __syncthreads();  // s_tmp is reused
  }
}

// Item i of a pass from the tile prefix s_toff and the row offsets s_off.
__device__ __forceinline__ int4 big_item(int i, int E, int nb, int tr, const int* s_toff, const int* s_off) {
  const int tile = i / nb;  // items of expert e occupy [toff[e] * nb, toff[e + 1] * nb)
  int lo = 0, hi = E;       // largest e with toff[e] <= tile and a tile of its own
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_toff[mid] <= tile) lo = mid; else hi = mid;
  }
  int e = lo;
  while (s_toff[e + 1] == s_toff[e]) ++e;  // skip experts without tiles
  const int nte = s_toff[e + 1] - s_toff[e];
  const int local = i - s_toff[e] * nb;
  const int b = local / nte, mt = local - b * nte;
  const int r0 = s_off[e] + mt * tr;
  return make_int4(e, r0, min(r0 + tr, s_off[e + 1]), b);
}

// Sort for M > kSmallM in three launches, none with a serial chain:
// 1. one workgroup per expert row of the token bitmap (bit t of row e: token
//    t picked e): the exclusive prefix of the words' popcounts, stored with
//    the word, and the row total (the expert's count); it is the bitmap's
//    only reader and leaves it zero for the next call;
// 2. one workgroup: offsets and the tile prefixes from the counts;
// 3. one thread per entry t*k+j: its place in expert e's run is offset[e]
//    plus the number of e's tokens before t (prefix + popcount below bit t),
//    so entries of earlier tokens come first; and one thread per work item.
__global__ __launch_bounds__(256) void align_rows_kernel(uint32_t* __restrict__ bitmap, int words,
                                                         int2* __restrict__ pw, int* __restrict__ count) {
  __shared__ int s_wsum[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* row = bitmap + (size_t)e * words;
  int2* prow = pw + (size_t)e * words;
  int carry = 0;
  for (int w0 = 0; w0 < words; w0 += 256) {
    const int w = w0 + tid;
    const uint32_t bits = w < words ? row[w] : 0u;
    const int c = __popc(bits);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      before += q < wave ? s_wsum[q] : 0;
      total += s_wsum[q];
    }
    if (w < words) {
      prow[w] = make_int2(carry + before + incl - c, (int)bits);
      if (bits) row[w] = 0u;
    }
    carry += total;
    __syncthreads();  // s_wsum is reused
  }
  if (tid == 0) count[e] = carry;
}

__global__ __launch_bounds__(1024) void align_offsets_kernel(
    const int* __restrict__ count_in, int E, int* __restrict__ count, int* __restrict__ offset,
    int4* __restrict__ tiles, int* __restrict__ meta, int n_iblk, int n_nc, int* __restrict__ toff,
    int with_tiles) {
  __shared__ int s_off[1024];
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x;
  const int c = tid < E ? count_in[tid] : 0;
  __syncthreads();  // count_in may be count itself
  write_offsets_tiles(c, E, s_off, s_tmp, count, offset, tiles, meta, with_tiles != 0);
  write_tile_prefixes(c, E, n_iblk, n_nc, s_tmp, toff, meta);
}

__global__ __launch_bounds__(256) void align_place_kernel(const int* __restrict__ topk_ids, int n, int k, int words,
                                                          const int2* __restrict__ pw, const int* __restrict__ offset,
                                                          int* __restrict__ sorted_entry, int E, int n_iblk, int n_nc,
                                                          const int* __restrict__ toff, const int* __restrict__ meta,
                                                          int4* __restrict__ gu_items, int4* __restrict__ dn_items) {
  __shared__ int s_off[1025];
  __shared__ int s_toff[2][1025];
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int e = topk_ids[i], t = i / k;
    const int2 v = pw[(size_t)e * words + (t >> 5)];
    const int rank = v.x + __popc((uint32_t)v.y & ((1u << (t & 31)) - 1u));
    sorted_entry[offset[e] + rank] = i;
  }
  for (int i = threadIdx.x; i <= E; i += 256) {
    s_off[i] = offset[i];
    s_toff[0][i] = toff[i];
    s_toff[1][i] = toff[E + 1 + i];
  }
  __syncthreads();
  const int n_gu = meta[1], n_dn = meta[2];
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_gu; i += gridDim.x * 256)
    gu_items[i] = big_item(i, E, n_iblk, kGuRows, s_toff[0], s_off);
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n_dn; i += gridDim.x * 256)
    dn_items[i] = big_item(i, E, n_nc, kBigRows, s_toff[1], s_off);
}

// The sort for kSmallM < M <= kMidM in one workgroup (the token bitmap has
// at most kMidM / 32 words a row, so the whole of it fits in LDS): the
// bitmap is read once and left zero, an expert's count is the popcount of
// its row, the offsets and the 16-row tiles come from one scan, and an
// entry's place is its expert's offset plus the popcount of the row below
// its token; the down work items (tiles of kBigRows rows) follow from a
// second scan. Same results as the three-launch sort.
constexpr int kMidWords = kMidM / 32;
__global__ __launch_bounds__(1024) void align_mid_kernel(uint32_t* __restrict__ bitmap, int words,
                                                         const int* __restrict__ topk_ids, int n, int k, int E,
                                                         int* __restrict__ count, int* __restrict__ offset,
                                                         int* __restrict__ sorted_entry, int4* __restrict__ tiles,
                                                         int* __restrict__ meta, int n_nc, int4* __restrict__ dn_items) {
  __shared__ uint32_t s_bm[1024 * kMidWords];
  __shared__ int s_off[1025];
  __shared__ int s_toff[1025];
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * words; i += 1024) {
    const uint32_t v = bitmap[i];
    s_bm[i] = v;
    if (v) bitmap[i] = 0u;
  }
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int w = 0; w < words; ++w) c += __popc(s_bm[tid * words + w]);
  write_offsets_tiles(c, E, s_off, s_tmp, count, offset, tiles, meta, true);  // ends with a barrier
  int n_tb;
  const int tb = (c + kBigRows - 1) / kBigRows;
  const int t0 = block_exclusive_scan(tb, s_tmp, &n_tb);
  if (tid < E) s_toff[tid] = t0;
  if (tid == 0) {
    s_off[E] = n;
    s_toff[E] = n_tb;
    meta[1] = 0;
    meta[2] = n_tb * n_nc;
  }
  __syncthreads();
  for (int i = tid; i < n; i += 1024) {
    const int e = topk_ids[i], t = i / k;
    const uint32_t* row = s_bm + e * words;
    int rank = __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(row[w]);
    sorted_entry[s_off[e] + rank] = i;
  }
  const int n_dn = n_tb * n_nc;
  for (int i = tid; i < n_dn; i += 1024) dn_items[i] = big_item(i, E, n_nc, kBigRows, s_toff, s_off);
}

__global__ void zero_kernel(uint4* p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((n16 + 255) / 256, 4096);
  return launch_k(zero_kernel, dim3(blocks), dim3(256), 0, s, Ev{}, reinterpret_cast<uint4*>(ptr), n16);
}

template <typename F>
static hipError_t by_ec(int E, F&& f) {
  const int ec = (E + 63) / 64;
  if (ec <= 1) return f(std::integral_constant<int, 1>{});
  if (ec <= 2) return f(std::integral_constant<int, 2>{});
  if (ec <= 4) return f(std::integral_constant<int, 4>{});
  if (ec <= 8) return f(std::integral_constant<int, 8>{});
  return f(std::integral_constant<int, 16>{});
}

hipError_t launch_route_small(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int M = (int)a.M, E = (int)p->s.E, k = (int)p->s.top_k, H = (int)p->s.H;
  const int xq_groups = (int)((a.M * (H / 32) + 63) / 64);
  return by_ec(E, [&](auto ec) {
    return launch_k(route_align_small_kernel<decltype(ec)::value>, dim3(1 + xq_groups), dim3(1024), 0, a.stream, ev,
                    a.logits,
                    reinterpret_cast<const uint16_t*>(a.x), M, E, k, H, p->s.routed_scaling,
                    wsp<int>(p, p->L.topk_ids), wsp<float>(p, p->L.topk_w), wsp<int>(p, p->L.count),
                    wsp<int>(p, p->L.offset), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), wsp<uint8_t>(p, p->L.xq), wsp<uint8_t>(p, p->L.xs), p->shared_slot);
  });
}

hipError_t launch_route(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int M = (int)a.M, E = (int)p->s.E, k = (int)p->s.top_k, H = (int)p->s.H;
  const int route_blocks = (int)std::min<int64_t>((a.M + 3) / 4, 2048);
  const int64_t units = a.M * ((H + 512 * kXU - 1) / (512 * kXU));
  const int blocks = route_blocks + (int)std::min<int64_t>((units + 3) / 4, 2048);
  const int words = (int)((a.M + 31) / 32);
  // with a shared expert, its E4M3 x comes from the same read of x
  const bool sh = p->s.shared_I > 0;
  uint8_t* sh_xq = sh ? wsp<uint8_t>(p, p->L.sh_xq) : nullptr;
  float* sh_xs = sh ? wsp<float>(p, p->L.sh_xs) : nullptr;
  return by_ec(E, [&](auto ec) {
    constexpr int EC = decltype(ec)::value;
    return launch_k(sh ? route_kernel<EC, true> : route_kernel<EC, false>, dim3(blocks), dim3(256), 0, a.stream,
                    ev, a.logits, reinterpret_cast<const uint16_t*>(a.x), M, E, k, H, p->s.routed_scaling,
                    wsp<int>(p, p->L.topk_ids), wsp<float>(p, p->L.topk_w), wsp<uint32_t>(p, p->X.bitmap), words,
                    wsp<uint8_t>(p, p->L.xq), wsp<uint8_t>(p, p->L.xs), sh_xq, sh_xs, route_blocks, p->shared_slot);
  });
}

hipError_t launch_align(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int words = (int)((a.M + 31) / 32);
  const int64_t n = a.M * p->s.top_k;
  if (mid_path(a.M, p->s.top_k))
    return launch_k(align_mid_kernel, dim3(1), dim3(1024), 0, a.stream, ev, wsp<uint32_t>(p, p->X.bitmap), words,
                    wsp<int>(p, p->L.topk_ids), (int)n, (int)p->s.top_k, (int)p->s.E, wsp<int>(p, p->L.count),
                    wsp<int>(p, p->L.offset), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), (int)(p->s.H / kDownItemCols), wsp<int4>(p, p->X.dn_items));
  hipError_t e = launch_k(align_rows_kernel, dim3((unsigned)p->s.E), dim3(256), 0, a.stream, Ev{ev.start, nullptr},
                          wsp<uint32_t>(p, p->X.bitmap), words, wsp<int2>(p, p->X.pw), wsp<int>(p, p->L.count));
  if (e != hipSuccess) return e;
  e = launch_k(align_offsets_kernel, dim3(1), dim3(1024), 0, a.stream, Ev{}, wsp<int>(p, p->L.count),
               (int)p->s.E, wsp<int>(p, p->L.count), wsp<int>(p, p->L.offset), wsp<int4>(p, p->X.tiles),
               wsp<int>(p, p->X.meta), (int)(p->s.I / 128), (int)(p->s.H / kDownItemCols), wsp<int>(p, p->X.toff),
               (int)mid_path(a.M, p->s.top_k));  // the 16-row tiles of the mid-range gate/up
  if (e != hipSuccess) return e;
  // a thread per entry and per work item: with few rows per expert the items
  // (tiles x column blocks) far outnumber the entries
  const int64_t items = p->tb_max * std::max<int64_t>(p->s.H / kDownItemCols, p->s.I / 128);
  const int64_t threads = std::max(n, items);
  return launch_k(align_place_kernel, dim3((unsigned)std::min<int64_t>((threads + 255) / 256, 4096)), dim3(256), 0,
                  a.stream, Ev{nullptr, ev.stop}, wsp<int>(p, p->L.topk_ids), (int)n, (int)p->s.top_k, words,
                  wsp<int2>(p, p->X.pw), wsp<int>(p, p->L.offset), wsp<int>(p, p->L.sorted_entry), (int)p->s.E,
                  (int)(p->s.I / 128), (int)(p->s.H / kDownItemCols), wsp<int>(p, p->X.toff), wsp<int>(p, p->X.meta),
                  wsp<int4>(p, p->X.gu_items), wsp<int4>(p, p->X.dn_items));
}

}  // namespace qmoe
