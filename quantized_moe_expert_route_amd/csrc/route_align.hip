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
#include "route_common.h"
#include "shared_small.h"

#include <algorithm>

namespace qmoe {

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

// Offsets, 16-row tiles of sorted rows and meta[0] from per-expert counts
// (thread e holds count c of expert e), for the small-token kernels and the
// mid-range gate/up up to kMidM tokens; leaves the offsets in s_off. The row
// total is below 2^16, so rows and tiles share one scan, packed as rows |
// tiles << 16.
__device__ void write_offsets_tiles(int c, int E, int* s_off, int* s_tmp, int* __restrict__ count,
                                    int* __restrict__ offset, int4* __restrict__ tiles, int* __restrict__ meta) {
  const int tid = threadIdx.x;
  const int nt = (c + kTileRows - 1) / kTileRows;
  int total;
  const int pre = block_exclusive_scan(c | (nt << 16), s_tmp, &total);
  const int off = pre & 0xFFFF, toff = pre >> 16;
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
    offset[E] = total & 0xFFFF;
    s_off[E] = total & 0xFFFF;
    meta[0] = total >> 16;
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
    uint8_t* __restrict__ xs, int shared_slot, SharedSmall sh) {
  __shared__ uint32_t s_mask[1024][2];  // expert -> tokens 0..63
  __shared__ int s_ids[64 * 16];
  __shared__ int s_off[1025];
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int xq_groups = (M * (H >> 5) + 63) >> 6;
  if ((int)blockIdx.x > xq_groups) {
    // the block-FP8 shared expert's gate/up partials (run inside the
    // small-token launches, beside the routing workgroup)
    extern __shared__ __align__(16) uint8_t sh_lds[];
    const int items = (sh.Is / kSsOut) * (H / 128 / sh.kb);
    const int first = (int)blockIdx.x - 1 - xq_groups, stride = (int)gridDim.x - 1 - xq_groups;
    for (int it = first; it < items; it += stride) shared_gate_up_item<2>(sh, x, it, M, H, sh_lds);
    return;
  }
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
// 128-block also form the shared expert's E4M3 codes (stored as int8 digits)
// and fp32 scale, so x is read once for both. A unit is kXU loads of one row.
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
        packed |= e2m1_pack2(f0, f1) << (8 * q);
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
          const uint32_t c = e4m3_pack2(__fdiv_rn(__uint_as_float(w32[q] << 16), sc),
                                        __fdiv_rn(__uint_as_float(w32[q] & 0xFFFF0000u), sc));
          if (q < 2) lo |= c << (16 * q); else hi |= c << (16 * (q - 2));
        }
      }
      // as digit rows ([H/128][3][128] per token) for the exact int8 GEMM
      store_digits8(sq + ((size_t)t * (H >> 7) + (e0 >> 7)) * kShDigitBlock, e0 & 127, lo, hi);
      if ((lane & 15) == 0) ss[(size_t)(e0 >> 7) * M + t] = sc;
    }
  }
}

// Workgroups [0, route_blocks) route, one wave per token: workgroup b takes
// tokens [4 b, 4 b + 4), an eighth of word b / 8 of each expert row of the
// expert x token bitmap; the bits of its tokens gather in LDS and each
// nonzero eighth goes to the bitmap with one atomic OR, so at most 8 atomics
// meet on a word even when every token picks the same experts (one per token
// and slot met 32 there, and serialized: t4 hot routing 26 -> 17 us). The
// rest quantize x, one wave per unit of kXU loads of a row. The two roles
// share no registers.
template <int EC, bool SH>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int E, int k, int H,
    float scaling, int* __restrict__ topk_ids, float* __restrict__ topk_w,
    uint32_t* __restrict__ bitmap, int words, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
    uint8_t* __restrict__ sh_xq, float* __restrict__ sh_xs, int route_blocks, int shared_slot) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if ((int)blockIdx.x < route_blocks) {
    __shared__ uint32_t s_bits[kRouteMaxE];
    for (int e = threadIdx.x; e < E; e += 256) s_bits[e] = 0u;
    const int t = blockIdx.x * 4 + wave;
    uint32_t key[EC];
    load_keys<EC>(logits + (size_t)min(t, M - 1) * E, E - shared_slot, lane, key);
    __syncthreads();
    if (t < M) {
      uint32_t sel_e = 0;
      float w = 0.f;
      route_keys<EC>(key, E, k, scaling, shared_slot, lane, sel_e, w);
      if (lane < k) {
        topk_ids[(size_t)t * k + lane] = (int)sel_e;
        topk_w[(size_t)t * k + lane] = w;
        atomicOr(&s_bits[sel_e], 1u << (t & 31));
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
      const uint32_t bits = s_bits[e];
      if (bits) atomicOr(&bitmap[(size_t)e * words + (blockIdx.x >> 3)], bits);
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
// Every workgroup of the placement launch forms the offsets and tile
// prefixes from the counts itself and writes its share of the items, a
// thread per item, the expert found by binary search of the prefix in LDS
// (one workgroup writing all of them was bound by one CU's store rate).
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

// Sort for M > kSmallM in two launches, none with a serial chain:
// 1. one workgroup per expert row of the token bitmap (bit t of row e: token
//    t picked e): the exclusive prefix of the words' popcounts, stored with
//    the word, and the row total (the expert's count); it is the bitmap's
//    only reader and leaves it zero for the next call;
// 2. every workgroup forms the offsets and the tile prefixes from the counts
//    (workgroup 0 also stores them); then one thread per entry t*k+j: its
//    place in expert e's run is offset[e] plus the number of e's tokens
//    before t (prefix + popcount below bit t), so entries of earlier tokens
//    come first; and one thread per work item (and per 64-row tile of the
//    MXFP4-mid down).
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

// The offsets and the tile prefixes (gate/up kGuRows, down kBigRows, with
// fp4_tiles the MXFP4-mid down's kFp4BigRows) from the experts' counts
// (thread e < E holds count e) into s_off / s_toff; workgroup 0 also stores
// offset[] and meta. Ends with a barrier.
__device__ void align_scans(int c, int E, int fp4_tiles, int n_iblk, int n_nc, int* s_off, int (*s_toff)[1025],
                            int* s_tmp, int* __restrict__ offset, int* __restrict__ meta, int& ng, int& nd,
                            int& nf) {
  const int tid = threadIdx.x;
  int tot;
  nf = 0;
  const int off = block_exclusive_scan(c, s_tmp, &tot);
  const int pg = block_exclusive_scan((c + kGuRows - 1) / kGuRows, s_tmp, &ng);
  const int pd = block_exclusive_scan((c + kBigRows - 1) / kBigRows, s_tmp, &nd);
  const int pf = fp4_tiles ? block_exclusive_scan((c + kFp4BigRows - 1) / kFp4BigRows, s_tmp, &nf) : 0;
  if (tid < E) {
    s_off[tid] = off;
    s_toff[0][tid] = pg;
    s_toff[1][tid] = pd;
    s_toff[2][tid] = pf;
  }
  if (tid == 0) {
    s_off[E] = tot;
    s_toff[0][E] = ng;
    s_toff[1][E] = nd;
    s_toff[2][E] = nf;
  }
  if (blockIdx.x == 0) {
    if (tid <= E) offset[tid] = tid < E ? off : tot;
    if (tid == 0) {
      meta[0] = nf;
      meta[1] = ng * n_iblk;
      meta[2] = nd * n_nc;
    }
  }
  __syncthreads();
}

// The gate/up and down work items and the MXFP4-mid down's 64-row tiles, a
// thread each over the grid.
__device__ void align_items(int E, int n_iblk, int n_nc, int ng, int nd, int nf, const int* s_off,
                            const int (*s_toff)[1025], int4* __restrict__ tiles, int4* __restrict__ gu_items,
                            int4* __restrict__ dn_items) {
  const int gsz = (int)gridDim.x * 1024, g0 = (int)blockIdx.x * 1024 + threadIdx.x;
  for (int i = g0; i < ng * n_iblk; i += gsz) gu_items[i] = big_item(i, E, n_iblk, kGuRows, s_toff[0], s_off);
  for (int i = g0; i < nd * n_nc; i += gsz) dn_items[i] = big_item(i, E, n_nc, kBigRows, s_toff[1], s_off);
  // the MXFP4-mid down's tiles: the expert by binary search of their prefix
  for (int i = g0; i < nf; i += gsz) {
    int lo = 0, hi = E;  // largest e with s_toff[2][e] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_toff[2][mid] <= i) lo = mid; else hi = mid;
    }
    int e = lo;
    while (s_toff[2][e + 1] == s_toff[2][e]) ++e;  // skip experts without tiles
    const int r0 = s_off[e] + (i - s_toff[2][e]) * kFp4BigRows;
    tiles[i] = make_int4(e, r0, min(r0 + kFp4BigRows, s_off[e + 1]), 0);
  }
}

__global__ __launch_bounds__(1024) void align_place_kernel(const int* __restrict__ topk_ids, int n, int k, int words,
                                                           const int2* __restrict__ pw, const int* __restrict__ count,
                                                           int* __restrict__ offset, int* __restrict__ sorted_entry,
                                                           int E, int n_iblk, int n_nc, int* __restrict__ meta,
                                                           int4* __restrict__ tiles, int fp4_tiles,
                                                           int4* __restrict__ gu_items, int4* __restrict__ dn_items) {
  __shared__ int s_off[1025];
  __shared__ int s_toff[3][1025];  // tile prefixes: gate/up (kGuRows), down (kBigRows), MXFP4-mid down (kFp4BigRows)
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x;
  int ng, nd, nf;
  align_scans(tid < E ? count[tid] : 0, E, fp4_tiles, n_iblk, n_nc, s_off, s_toff, s_tmp, offset, meta, ng, nd, nf);
  const int gsz = (int)gridDim.x * 1024, g0 = (int)blockIdx.x * 1024 + tid;
  for (int i = g0; i < n; i += gsz) {
    const int e = topk_ids[i], t = i / k;
    const int2 v = pw[(size_t)e * words + (t >> 5)];
    const int rank = v.x + __popc((uint32_t)v.y & ((1u << (t & 31)) - 1u));
    sorted_entry[s_off[e] + rank] = i;
  }
  align_items(E, n_iblk, n_nc, ng, nd, nf, s_off, s_toff, tiles, gu_items, dn_items);
}

// The large-token sort in one launch while the whole token bitmap fits in
// LDS (align_one_launch): every workgroup copies it into
// LDS, forms the popcount prefix of each row at every 8th word and the
// experts' counts, then as align_place_kernel the offsets, the entries'
// places (prefix + popcounts of the words between + popcount below bit t)
// and the work items. The workgroup whose copy completes last (a counter in
// the workspace, reset by it) clears the bitmap for the next call: every
// other workgroup's copy is complete by then.
__global__ __launch_bounds__(1024) void align_big_kernel(uint32_t* __restrict__ bitmap, int words,
                                                         int* __restrict__ done, const int* __restrict__ topk_ids,
                                                         int n, int k, int* __restrict__ count,
                                                         int* __restrict__ offset, int* __restrict__ sorted_entry,
                                                         int E, int n_iblk, int n_nc, int* __restrict__ meta,
                                                         int4* __restrict__ tiles, int fp4_tiles,
                                                         int4* __restrict__ gu_items, int4* __restrict__ dn_items) {
  __shared__ __align__(16) uint32_t s_bm[kAlignLdsWords];
  __shared__ __align__(16) uint16_t s_pre[kAlignLdsWords / 8 + kRouteMaxE];
  __shared__ int s_off[1025];
  __shared__ int s_toff[3][1025];
  __shared__ int s_tmp[64];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int nw = E * words, ng8 = (words + 7) >> 3;
  const int gsz = (int)gridDim.x * 1024, g0 = (int)blockIdx.x * 1024 + tid;
  int e_first = topk_ids[min(g0, n - 1)];  // this thread's first entry's expert, read beside the copy
  {
    // the copy in 16-byte pieces, all of a thread's loads in flight together
    // (unconditional, from a clamped index; kAlignLdsWords / 4 / 1024 of them)
    const int nw4 = nw >> 2;
    const uint4* src = reinterpret_cast<const uint4*>(bitmap);
    uint4* dst = reinterpret_cast<uint4*>(s_bm);
    uint4 v[kAlignLdsWords / 4096];
    if (nw4 > 0) {
#pragma unroll
      for (int q = 0; q < kAlignLdsWords / 4096; ++q) v[q] = src[min(tid + 1024 * q, nw4 - 1)];
      // (the loads are used here, so none sinks into its store's branch)
#pragma unroll
      for (int q = 0; q < kAlignLdsWords / 4096; ++q)
        asm volatile("" : "+v"(v[q].x), "+v"(v[q].y), "+v"(v[q].z), "+v"(v[q].w));
      asm volatile("" : "+v"(e_first));
#pragma unroll
      for (int q = 0; q < kAlignLdsWords / 4096; ++q)
        if (tid + 1024 * q < nw4) dst[tid + 1024 * q] = v[q];
    }
    for (int i = 4 * nw4 + tid; i < nw; i += 1024) s_bm[i] = bitmap[i];
  }
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(done, 1) == (int)gridDim.x - 1;
  // popcounts of the rows' 8-word groups, then each row's exclusive prefix
  // over its groups (a thread a row) and its total, the expert's count
  for (int q = tid; q < E * ng8; q += 1024) {
    const int e = q / ng8, w0 = 8 * (q - e * ng8);
    const uint32_t* row = s_bm + e * words;
    int c = 0;
    for (int w = w0; w < min(w0 + 8, words); ++w) c += __popc(row[w]);
    s_pre[q] = (uint16_t)c;
  }
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int g = 0; g < ng8; ++g) {
      const int c = s_pre[tid * ng8 + g];
      s_pre[tid * ng8 + g] = (uint16_t)run;
      run += c;
    }
    s_off[tid] = run;
  }
  __syncthreads();
  const int c = tid < E ? s_off[tid] : 0;
  if (blockIdx.x == 0 && tid < E) count[tid] = c;
  __syncthreads();  // s_off is rewritten by the scans
  int ng, nd, nf;
  align_scans(c, E, fp4_tiles, n_iblk, n_nc, s_off, s_toff, s_tmp, offset, meta, ng, nd, nf);
  for (int i = g0; i < n; i += gsz) {
    const int e = i == g0 ? e_first : topk_ids[i], t = i / k, w = t >> 5;
    const uint32_t* row = s_bm + e * words;
    int rank = s_pre[e * ng8 + (w >> 3)] + __popc(row[w] & ((1u << (t & 31)) - 1u));
    for (int v = w & ~7; v < w; ++v) rank += __popc(row[v]);
    sorted_entry[s_off[e] + rank] = i;
  }
  align_items(E, n_iblk, n_nc, ng, nd, nf, s_off, s_toff, tiles, gu_items, dn_items);
  if (s_last) {  // (s_last was written before two barriers)
    const int nw4 = nw >> 2;
    for (int i = tid; i < nw4; i += 1024) reinterpret_cast<uint4*>(bitmap)[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = 4 * nw4 + tid; i < nw; i += 1024) bitmap[i] = 0u;
    if (tid == 0) *done = 0;
  }
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
                                                         int* __restrict__ meta, int n_nc, int4* __restrict__ dn_items,
                                                         int fp4_tiles) {
  __shared__ uint32_t s_bm[1024 * kMidWords];
  __shared__ int s_off[1025];
  __shared__ int s_toff[1025];
  __shared__ int s_tmp[64];
  const int tid = threadIdx.x;
  // the entries' experts are read beside the bitmap (n <= kMidM * 16)
  constexpr int kPre = kMidM * 16 / 1024;
  int pre_e[kPre];
#pragma unroll
  for (int q = 0; q < kPre; ++q) pre_e[q] = topk_ids[min(tid + 1024 * q, n - 1)];
  for (int i = tid; i < E * words; i += 1024) {
    const uint32_t v = bitmap[i];
    s_bm[i] = v;
    if (v) bitmap[i] = 0u;
  }
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int w = 0; w < words; ++w) c += __popc(s_bm[tid * words + w]);
  write_offsets_tiles(c, E, s_off, s_tmp, count, offset, tiles, meta);  // ends with a barrier
  int n_tb;
  // the E4M3 down's items are on tiles of kBigRows rows; with the MXFP4 mid
  // the down runs on tiles of kFp4BigRows rows instead, written to the same
  // place ({expert, row_begin, row_end, 0}; their count in meta[3])
  const int tr = fp4_tiles ? kFp4BigRows : kBigRows;
  const int tb = (c + tr - 1) / tr;
  const int t0 = block_exclusive_scan(tb, s_tmp, &n_tb);
  if (tid < E) s_toff[tid] = t0;
  if (tid == 0) {
    s_off[E] = n;
    s_toff[E] = n_tb;
    meta[1] = 0;
    meta[2] = fp4_tiles ? 0 : n_tb * n_nc;
    meta[3] = fp4_tiles ? n_tb : 0;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const int i = tid + 1024 * q;
    if (i >= n) break;
    const int e = pre_e[q], t = i / k;
    const uint32_t* row = s_bm + e * words;
    int rank = __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(row[w]);
    sorted_entry[s_off[e] + rank] = i;
  }
  if (fp4_tiles) {
    if (tid < E)
      for (int i = 0; i < tb; ++i) {
        const int r0 = s_off[tid] + i * kFp4BigRows;
        dn_items[t0 + i] = make_int4(tid, r0, min(r0 + kFp4BigRows, s_off[tid] + c), 0);
      }
    return;
  }
  // the down items, a thread per (expert, column block): the expert's items
  // fill [toff[e] n_nc, toff[e+1] n_nc) in the order (column block, row tile)
  // of big_item, without a search per item
  for (int pr = tid; pr < E * n_nc; pr += 1024) {
    const int e = pr / n_nc, b = pr - e * n_nc;
    const int nte = s_toff[e + 1] - s_toff[e];
    int4* dst = dn_items + (size_t)s_toff[e] * n_nc + (size_t)b * nte;
    for (int mt = 0; mt < nte; ++mt) {
      const int r0 = s_off[e] + mt * kBigRows;
      dst[mt] = make_int4(e, r0, min(r0 + kBigRows, s_off[e + 1]), b);
    }
  }
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
  // with the shared expert inside the small-token launches: its gate/up
  // items on the workgroups the routing leaves free (two per CU)
  // (one 1024-thread workgroup of this kernel per CU)
  const SharedSmall sh = shared_small(p, a.M);
  const int free_cus = std::max(1, p->num_cus - 1 - xq_groups);
  const int sh_items = sh.part ? (sh.Is / kSsOut) * (H / 128 / sh.kb) : 0;
  const int sh_groups = std::min(sh_items, free_cus);
  const size_t lds = sh.part ? shared_gate_up_lds(sh.kb) : 0;
  return by_ec(E, [&](auto ec) {
    return launch_k(route_align_small_kernel<decltype(ec)::value>, dim3(1 + xq_groups + sh_groups), dim3(1024), lds,
                    a.stream, ev,
                    a.logits,
                    reinterpret_cast<const uint16_t*>(a.x), M, E, k, H, p->s.routed_scaling,
                    wsp<int>(p, p->L.topk_ids), wsp<float>(p, p->L.topk_w), wsp<int>(p, p->L.count),
                    wsp<int>(p, p->L.offset), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), wsp<uint8_t>(p, p->L.xq), wsp<uint8_t>(p, p->L.xs), p->shared_slot, sh);
  });
}

hipError_t launch_route(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int M = (int)a.M, E = (int)p->s.E, k = (int)p->s.top_k, H = (int)p->s.H;
  // a routing workgroup per 4 tokens
  const int words = (int)((a.M + 31) / 32), route_blocks = (int)((a.M + 3) / 4);
  const int64_t units = a.M * ((H + 512 * kXU - 1) / (512 * kXU));
  const int blocks = route_blocks + (int)std::min<int64_t>((units + 3) / 4, 2048);
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
                    wsp<int>(p, p->X.meta), (int)(p->s.H / kDownItemCols), wsp<int4>(p, p->X.dn_items),
                    p->mid_fmt == MOE_MID_MXFP4 ? 1 : 0);
  const int64_t items = p->tb_max * std::max<int64_t>(p->s.H / kDownItemCols, p->s.I / 128);
  const int64_t threads = std::max(n, items);
  const unsigned grid = (unsigned)std::min<int64_t>((threads + 1023) / 1024, 1024);
  if (align_one_launch(p->s.E, a.M))
    return launch_k(align_big_kernel, dim3(grid), dim3(1024), 0, a.stream, ev, wsp<uint32_t>(p, p->X.bitmap), words,
                    wsp<int>(p, p->X.done), wsp<int>(p, p->L.topk_ids), (int)n, (int)p->s.top_k,
                    wsp<int>(p, p->L.count), wsp<int>(p, p->L.offset), wsp<int>(p, p->L.sorted_entry), (int)p->s.E,
                    (int)(p->s.I / 128), (int)(p->s.H / kDownItemCols), wsp<int>(p, p->X.meta),
                    wsp<int4>(p, p->X.tiles), p->mid_fmt == MOE_MID_MXFP4 ? 1 : 0, wsp<int4>(p, p->X.gu_items),
                    wsp<int4>(p, p->X.dn_items));
  hipError_t e = launch_k(align_rows_kernel, dim3((unsigned)p->s.E), dim3(256), 0, a.stream, Ev{ev.start, nullptr},
                          wsp<uint32_t>(p, p->X.bitmap), words, wsp<int2>(p, p->X.pw), wsp<int>(p, p->L.count));
  if (e != hipSuccess) return e;
  return launch_k(align_place_kernel, dim3(grid), dim3(1024), 0,
                  a.stream, Ev{nullptr, ev.stop}, wsp<int>(p, p->L.topk_ids), (int)n, (int)p->s.top_k, words,
                  wsp<int2>(p, p->X.pw), wsp<int>(p, p->L.count), wsp<int>(p, p->L.offset),
                  wsp<int>(p, p->L.sorted_entry), (int)p->s.E, (int)(p->s.I / 128), (int)(p->s.H / kDownItemCols),
                  wsp<int>(p, p->X.meta), wsp<int4>(p, p->X.tiles), p->mid_fmt == MOE_MID_MXFP4 ? 1 : 0,
                  wsp<int4>(p, p->X.gu_items), wsp<int4>(p, p->X.dn_items));
}

}  // namespace qmoe
