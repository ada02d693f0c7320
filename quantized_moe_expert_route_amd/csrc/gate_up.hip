// gate/up grouped GEMM on MXFP4 (scaled FP4 MFMA), SiLU(gate) * up, and the
// one-time per-128 FP8 E4M3 quantization of mid.
//
// gate/up: "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing"
// (Summary: SiLU activation after the usual expert selection) and the pages'
// MXFP4 (A4W4) arm. Mid: "glm53: FP8 mid hand-off, early split rows, ..."
// (Modifications table, row "mid as FP8 once": each 128-element mid block is
// quantized to FP8 once with its scale, and the down GEMM reads those bytes).
//
// gate_up_m16_kernel (its mid quantized by act_quant_kernel, a launch of
// its own): work item = (tile of up to 16 sorted rows of one expert, 16
// columns of I).
// A workgroup of 4 waves computes the gate and the up columns of the item,
// each wave a quarter of the K super-steps (4 K-steps of 128); the four
// partial sums are added in wave order through LDS. In K-step ks lane
// 16 g + r supplies row r's MX block 4 ks + g (16 bytes and one scale byte),
// for x and for the weights alike, so every MFMA pairs matching K. The
// weights come packed (moe_pack_w13): a K-step of the item's 16 gate (or up)
// rows is 1 KB contiguous in lane order, and a row block's scales of a
// super-step are one dword per lane. gate_up_quant_kernel (below) does
// gate/up and the mid quantization in one launch on larger work items.
#include "common.h"
#include "internal.h"
#include "route_common.h"
#include "shared_small.h"

#include <algorithm>

namespace qmoe {

constexpr int kSS = 3;  // super-steps (512 K each) whose loads a wave keeps in flight

// One wave quantizes rows [r0, r1) of mid block b: s = fl32(amax / 448),
// q = E4M3(fl32(h / s)); 128 values = 2 per lane.
__device__ __forceinline__ void quant_mid_rows(const float* __restrict__ h, int r0, int r1, int row_step, int I, int b,
                                               uint8_t* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int nb = I / 128;
  for (int row = r0; row < r1; row += row_step) {
    const size_t base = (size_t)row * I + b * 128 + 2 * lane;
    const float2 v = *reinterpret_cast<const float2*>(h + base);
    const float amax = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
    const float sc = __fdiv_rn(amax, 448.0f);
    const uint32_t c01 = sc > 0.f ? e4m3_pack2(__fdiv_rn(v.x, sc), __fdiv_rn(v.y, sc)) : 0u;
    *reinterpret_cast<uint16_t*>(q + base) = (uint16_t)c01;
    if (lane == 0) s[(size_t)row * nb + b] = sc;
  }
}

__global__ __launch_bounds__(256) void gate_up_m16_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const uint8_t* __restrict__ w13p,
    const uint8_t* __restrict__ s13p, const int* __restrict__ sorted_entry,
    const int4* __restrict__ tiles, const int* __restrict__ meta, float* __restrict__ hout, int H,
    int I, int k) {
  __shared__ v4f red[2][4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n_it = I / 16;
  // The first item's tile is read beside meta (the grid never exceeds the
  // tile array's bound, so the read is in bounds; it is used only when the
  // item exists): one memory round trip fewer before the weights move.
  int4 tl = tiles[blockIdx.x / n_it];
  int n_tiles = meta[0];
  asm volatile("" : "+s"(n_tiles), "+s"(tl.x), "+s"(tl.y), "+s"(tl.z));  // both loads in flight together
  const int n_work = n_tiles * n_it;
  const size_t Hb = (size_t)H / 2, Hs = (size_t)H / 32;
  const int nss = H / 512, nks = H / 128;
  const size_t nrb = (size_t)I / 8;  // 16-row blocks of an expert's 2I rows
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    if (w != (int)blockIdx.x) tl = tiles[w / n_it];
    const int it = w % n_it;
    const int e = tl.x, r0 = tl.y, r1 = tl.z;
    const bool rv = r0 + r < r1;
    // the row's entry is waited for only after the first weight loads are
    // out (the empty asm keeps its use inside the loop, behind them)
    int se = sorted_entry[min(r0 + r, r1 - 1)];
    const uint8_t* pa = xq;   // the row's token's x: + 64 ks (set once the entry is in)
    const uint8_t* psa = xs;  // its scales: + 16 ss: byte 4 j + g is K-step 4 ss + j
    const size_t rbg = (size_t)e * nrb + it, rbu = rbg + I / 16;
    const uint8_t* pg = w13p + rbg * nks * 1024 + 16 * lane;  // + 1024 ks
    const uint8_t* pu = w13p + rbu * nks * 1024 + 16 * lane;
    const uint8_t* psg = s13p + rbg * nss * 256 + 4 * lane;  // + 256 ss: byte j is K-step 4 ss + j
    const uint8_t* psu = s13p + rbu * nss * 256 + 4 * lane;
    v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    // wave w owns the contiguous super-steps [w*per, (w+1)*per); all loads of
    // up to kSS of them are in flight before the first MFMA
    const int per = (nss + 3) / 4;
    const int ss_end = min(nss, (wave + 1) * per);
    for (int ss0 = wave * per; ss0 < ss_end; ss0 += kSS) {
      uint4 a[kSS][4], bg[kSS][4], bu[kSS][4], sa[kSS];
      uint32_t sg[kSS], su[kSS];
#pragma unroll
      for (int q = 0; q < kSS; ++q) {
        const int ss = min(ss0 + q, ss_end - 1);  // clamped: a duplicate step is loaded but not used
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bg[q][j] = ld16(pg + (size_t)(4 * ss + j) * 1024);
          bu[q][j] = ld16(pu + (size_t)(4 * ss + j) * 1024);
        }
        sg[q] = ld4(psg + 256 * ss);
        su[q] = ld4(psu + 256 * ss);
        if (q == 0) {
          asm volatile("" : "+v"(se));
          const size_t tok = rv ? (size_t)(se / k) : 0;
          pa = xq + tok * Hb + 16 * g;
          psa = xs + tok * Hs;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) a[q][j] = rv ? ld16(pa + (4 * ss + j) * 64) : make_uint4(0, 0, 0, 0);
        sa[q] = rv ? ld16(psa + 16 * ss) : make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
      }
#pragma unroll
      for (int q = 0; q < kSS; ++q) {
        if (ss0 + q < ss_end) {
          const uint32_t xw[4] = {sa[q].x, sa[q].y, sa[q].z, sa[q].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t xa = (xw[j] >> (8 * g)) & 0xFFu;
            accg = mfma_fp4(a[q][j], bg[q][j], accg, xa, (sg[q] >> (8 * j)) & 0xFFu);
            accu = mfma_fp4(a[q][j], bu[q][j], accu, xa, (su[q] >> (8 * j)) & 0xFFu);
          }
        }
      }
    }
    red[0][wave][lane] = accg;
    red[1][wave][lane] = accu;
    __syncthreads();
    {
      // thread -> (row m, column n) of the 16x16 item
      const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
      const int l = n + 16 * (m >> 2), i = m & 3;
      const float G = ((red[0][0][l][i] + red[0][1][l][i]) + red[0][2][l][i]) + red[0][3][l][i];
      const float U = ((red[1][0][l][i] + red[1][1][l][i]) + red[1][2][l][i]) + red[1][3][l][i];
      if (r0 + m < r1) hout[(size_t)(r0 + m) * I + it * 16 + n] = silu_mul(G, U);
    }
    __syncthreads();
  }
}

// Gate/up that routes for itself (rq_path: up to kRqM tokens, E <= kRqMaxE,
// H <= kRqMaxH, the E4M3 mid, no shared expert): the call has no routing
// launch. Every workgroup ranks the M tokens' logits (a wave per token, the
// rounds of the routing launch, so the same ids and weights), orders the
// M k entries expert-major in LDS (each expert holds at most M <= kRqM
// rows: one 16-row tile per active expert), finds its item's expert and rows,
// issues the item's x and weight loads, and quantizes its rows of x to MXFP4
// into LDS while the weights are in flight; then the item runs as in
// gate_up_m16_kernel, x read from LDS. Workgroup 0 stores the routing, the
// sort and the tiles for the launches after this one; the workgroup of each
// tile's first column group stores its rows' x codes. The weights thus start
// moving one logits round trip after the launch, where a routing launch of
// its own put its whole span (launch, logits, ranking, sort, stores) first
// ("glm53: FP8 mid hand-off, ...", Modifications table, row "per-row up/gate
// jobs": the routing rounds overlapped with the first weight loads).
constexpr int kRqXB = kRqM * (kRqMaxH / 32) / 256;  // x blocks a thread quantizes (at most)
static_assert(kRqM * (kRqMaxH / 32) % 256 == 0 && kRqMaxH / 512 <= 4 * kSS && kRqM <= 16, "rq tile shape");
static_assert(kRqMaxE == 256 && kRqM <= 4, "a thread per expert, a wave per token");

template <int EC>
__global__ __launch_bounds__(256) void gate_up_route_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int M, int E, int k, int H, float scaling,
    const uint8_t* __restrict__ w13p, const uint8_t* __restrict__ s13p, int I, int* __restrict__ topk_ids,
    float* __restrict__ topk_w, int* __restrict__ count, int* __restrict__ offset, int* __restrict__ sorted_entry,
    int4* __restrict__ tiles, int* __restrict__ meta, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
    float* __restrict__ hout) {
  __shared__ v4f red[2][4][64];
  __shared__ uint32_t s_bits[kRqMaxE];  // expert -> its tokens (bit t)
  __shared__ int s_ids[kRqM * 16];      // entry t k + j -> expert
  __shared__ int s_off[kRqMaxE + 1];    // expert -> its first sorted row
  __shared__ int s_te[kRqMaxE];         // tile -> expert
  __shared__ int s_tmp[4];
  __shared__ __align__(16) uint8_t s_xq[kRqM][kRqMaxH / 2];   // the tile's rows of x: E2M1 codes
  __shared__ __align__(16) uint8_t s_xs[kRqM][kRqMaxH / 32];  // and E8M0 scales
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;

  // ---- routing: wave t ranks token t (its logits requested first)
  uint32_t key[EC];
  load_keys<EC>(logits + (size_t)min(wave, M - 1) * E, E, lane, key);
  s_bits[tid] = 0u;  // kRqMaxE == blockDim
  __syncthreads();
  // the ids only: the weights matter to the combine alone, so workgroup 0
  // forms them (route_weight) once its weight loads are out
  float sel_l = 0.f;
  if (wave < M) {
    uint32_t sel_e = 0;
    topk_wave<EC>(key, k, lane, sel_e, sel_l);
    if (lane < k) {
      s_ids[wave * k + lane] = (int)sel_e;
      atomicOr(&s_bits[sel_e], 1u << wave);
      if (blockIdx.x == 0) topk_ids[wave * k + lane] = (int)sel_e;
    }
  }
  __syncthreads();
  // counts, offsets and the tile list: thread e, one packed scan of
  // rows | tiles << 16 (a tile per active expert)
  const int c = tid < E ? __popc(s_bits[tid]) : 0;
  const int v = c | ((c > 0 ? 1 : 0) << 16);
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int nb = __shfl_up(incl, o, 64);
    if (lane >= o) incl += nb;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int pre = incl - v;
  for (int ww = 0; ww < wave; ++ww) pre += s_tmp[ww];
  const int total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  const int nt = total >> 16;
  if (tid < E) {
    s_off[tid] = pre & 0xFFFF;
    if (c) s_te[pre >> 16] = tid;
  }
  __syncthreads();
  if (blockIdx.x == 0) {  // the routing, the sort and the tiles for the later launches
    if (tid < E) {
      count[tid] = c;
      offset[tid] = pre & 0xFFFF;
      if (c) tiles[pre >> 16] = make_int4(tid, pre & 0xFFFF, (pre & 0xFFFF) + c, 0);
    }
    if (tid == 0) {
      offset[E] = total & 0xFFFF;
      meta[0] = nt;
    }
    if (tid < M * k) {
      const int e = s_ids[tid], t = tid / k;
      sorted_entry[s_off[e] + __popc(s_bits[e] & ((1u << t) - 1u))] = tid;
    }
  }

  const int n_it = I / 16;
  const int n_work = nt * n_it;
  const size_t Hs = (size_t)H / 32;
  const int nss = H / 512, nks = H / 128, nblk = H / 32;
  const size_t nrb = (size_t)I / 8;  // 16-row blocks of an expert's 2I rows
  const int per = (nss + 3) / 4;     // super-steps a wave owns (at most kSS)
  const int ss_beg = min(nss, wave * per), ss_end = min(nss, (wave + 1) * per);
  for (int wi = blockIdx.x; wi < n_work; wi += gridDim.x) {
    const int it = wi % n_it;
    const int e = s_te[wi / n_it];
    const uint32_t bits = s_bits[e];
    const int r0 = s_off[e], nrow = __popc(bits);
    // x of the tile's rows: thread b takes blocks b, b + 256, ... of the
    // nrow x H/32 (row, 32-block) pairs, loaded before the weights so that
    // waiting for them does not wait for the weights (past the last pair:
    // its last block again, not used)
    const int nxb = nrow * nblk;
    uint4 xv[kRqXB][4];
    int xrow[kRqXB], xblk[kRqXB];
#pragma unroll
    for (int q = 0; q < kRqXB; ++q) {
      const int b = min(tid + 256 * q, nxb - 1);
      xrow[q] = b / nblk;
      xblk[q] = b - xrow[q] * nblk;
      uint32_t rb = bits;  // token of row xrow[q]: its xrow[q]-th set bit
      for (int z = 0; z < xrow[q]; ++z) rb &= rb - 1u;
      const uint16_t* src = x + (size_t)(__ffs(rb) - 1) * H + 32 * xblk[q];
#pragma unroll
      for (int u = 0; u < 4; ++u) xv[q][u] = ld16(src + 8 * u);
    }
    // the wave's weight fragments, all its super-steps at once
    const size_t rbg = (size_t)e * nrb + it, rbu = rbg + I / 16;
    const uint8_t* pg = w13p + rbg * nks * 1024 + 16 * lane;  // + 1024 ks
    const uint8_t* pu = w13p + rbu * nks * 1024 + 16 * lane;
    const uint8_t* psg = s13p + rbg * nss * 256 + 4 * lane;  // + 256 ss: byte j is K-step 4 ss + j
    const uint8_t* psu = s13p + rbu * nss * 256 + 4 * lane;
    uint4 bg[kSS][4], bu[kSS][4];
    uint32_t sg[kSS], su[kSS];
#pragma unroll
    for (int q = 0; q < kSS; ++q) {
      const int ss = min(ss_beg + q, ss_end - 1);  // clamped (also for a wave without steps): loaded, not used
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bg[q][j] = ld16(pg + (size_t)(4 * ss + j) * 1024);
        bu[q][j] = ld16(pu + (size_t)(4 * ss + j) * 1024);
      }
      sg[q] = ld4(psg + 256 * ss);
      su[q] = ld4(psu + 256 * ss);
    }
    if (blockIdx.x == 0 && wi == 0 && wave < M) {  // the routing weights (route_keys' second half)
      const float w = route_weight(sel_l, k, lane, scaling);
      if (lane < k) topk_w[wave * k + lane] = w;
    }
    // x -> MXFP4 into LDS (the routing launch's quantizer, the same codes)
#pragma unroll
    for (int q = 0; q < kRqXB; ++q) {
      if (tid + 256 * q < nxb) {
        uint32_t w32[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          w32[4 * u] = xv[q][u].x; w32[4 * u + 1] = xv[q][u].y; w32[4 * u + 2] = xv[q][u].z; w32[4 * u + 3] = xv[q][u].w;
        }
        quant_block_mx_words(w32, &s_xq[xrow[q]][16 * xblk[q]], &s_xs[xrow[q]][xblk[q]]);
      }
    }
    __syncthreads();
    if (it == 0) {  // the tile's rows of x for the caller (a token in several tiles: the same bytes again)
      const int rowb = (int)(H / 2 + Hs);
      for (int b = tid; b < nrow * (rowb / 16); b += 256) {
        const int rr = b / (rowb / 16), o = 16 * (b - rr * (rowb / 16));
        uint32_t rb = bits;
        for (int z = 0; z < rr; ++z) rb &= rb - 1u;
        const size_t t = (size_t)(__ffs(rb) - 1);
        if (o < H / 2) *reinterpret_cast<uint4*>(xq + t * (H / 2) + o) = *reinterpret_cast<const uint4*>(&s_xq[rr][o]);
        else *reinterpret_cast<uint4*>(xs + t * Hs + (o - H / 2)) = *reinterpret_cast<const uint4*>(&s_xs[rr][o - H / 2]);
      }
    }
    // the products: lane 16 g + r supplies row r's MX block 4 ks + g
    const bool rv = r < nrow;
    const int rl = rv ? r : 0;
    v4f accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kSS; ++q) {
      const int ss = ss_beg + q;
      if (ss < ss_end) {
        const uint4 sa = rv ? *reinterpret_cast<const uint4*>(&s_xs[rl][16 * ss])
                            : make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
        const uint32_t xw[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 a = rv ? *reinterpret_cast<const uint4*>(&s_xq[rl][64 * (4 * ss + j) + 16 * g])
                             : make_uint4(0, 0, 0, 0);
          const uint32_t xa = (xw[j] >> (8 * g)) & 0xFFu;
          accg = mfma_fp4(a, bg[q][j], accg, xa, (sg[q] >> (8 * j)) & 0xFFu);
          accu = mfma_fp4(a, bu[q][j], accu, xa, (su[q] >> (8 * j)) & 0xFFu);
        }
      }
    }
    red[0][wave][lane] = accg;
    red[1][wave][lane] = accu;
    __syncthreads();
    {
      // thread -> (row m, column n) of the 16x16 item
      const int m = tid >> 4, n = tid & 15;
      const int l = n + 16 * (m >> 2), i = m & 3;
      const float G = ((red[0][0][l][i] + red[0][1][l][i]) + red[0][2][l][i]) + red[0][3][l][i];
      const float U = ((red[1][0][l][i] + red[1][1][l][i]) + red[1][2][l][i]) + red[1][3][l][i];
      if (m < nrow) hout[(size_t)(r0 + m) * I + it * 16 + n] = silu_mul(G, U);
    }
    __syncthreads();
  }
}

// One wave per (row, 128-block): s = fl32(amax / 448), q = E4M3(fl32(h / s)).
// With the shared expert inside the small-token launches, the workgroups
// after the routed ones form its h from the gate/up partials and quantize
// it (one workgroup per token and 128-block).
__global__ __launch_bounds__(256) void act_quant_kernel(const float* __restrict__ h, int rows, int I,
                                                        uint8_t* __restrict__ q, float* __restrict__ s,
                                                        int routed_blocks, SharedSmall sh, int M, int H) {
  if ((int)blockIdx.x >= routed_blocks) {
    __shared__ float u_lds[130];
    const int snb = sh.Is / 128;
    for (int sb = (int)blockIdx.x - routed_blocks; sb < M * snb; sb += (int)gridDim.x - routed_blocks)
      shared_mid_block(sh, sb / snb, sb % snb, M, H, u_lds, threadIdx.x, true);
    return;
  }
  const int nb = I / 128;
  const int total = rows * nb;
  for (int wv = blockIdx.x * 4 + (threadIdx.x >> 6); wv < total; wv += routed_blocks * 4) {
    const int row = wv / nb, b = wv % nb;
    quant_mid_rows(h, row, row + 1, 1, I, b, q, s);
  }
}

// Gate/up with the mid quantization in the same launch (gq_path): a
// workgroup of 16 waves owns one 128-column mid block b of one 16-row tile;
// wave w < 8 takes gate row block w of the block, wave 8 + w up row block w,
// each over all of K with its weights streamed straight into registers (a
// ring of R super-steps of 4 K-steps: 1 KB packed pieces, one scale dword a
// lane per super-step). The tile's x rows (MXFP4 codes and scales, zeros past
// the tile's end) sit in LDS, rows padded by 16 bytes. The gate and up
// results meet in LDS; wave m then forms row m's SiLU(g) * u, its 128-block
// amax and E4M3 codes by the same arithmetic as the mid quantization's own
// launch. Workgroups past the routed ones form the fused shared expert's mid
// blocks, four (token, block) items each. With the MXFP4 mid the epilogue
// forms the mid per 32 columns instead (E8M0 scale + E2M1 codes).
constexpr int kGqThreads = 1024;

size_t gate_up_quant_lds(int64_t H) { return (size_t)16 * (H / 2 + 16) + (size_t)16 * (H / 32 + 16) + 2 * 16 * 128 * 4; }

template <int KST, bool MX>
__global__ __launch_bounds__(kGqThreads) void gate_up_quant_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const uint8_t* __restrict__ w13p,
    const uint8_t* __restrict__ s13p, const int* __restrict__ sorted_entry, const int4* __restrict__ tiles,
    const int* __restrict__ meta, int I, int k, int tmax, uint8_t* __restrict__ midq, float* __restrict__ mids,
    int routed_wgs, SharedSmall sh, int M) {
  constexpr int H = 2048 * KST;                 // KST: 16-byte x chunks a staging thread
  constexpr int NKS = H / 128, NSS = H / 512;   // K-steps, super-steps (4 K-steps)
  constexpr int CPR = H / 32, SPR = H / 512;    // 16-byte chunks per x row / scale row
  constexpr int LX = H / 2 + 16, LS = H / 32 + 16;  // LDS bytes per staged x row / scale row
  constexpr int R = NSS < 4 ? NSS : 4;          // super-steps of weights in flight
  extern __shared__ __align__(16) uint8_t gq_lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  if ((int)blockIdx.x >= routed_wgs) {
    float* u_lds = reinterpret_cast<float*>(gq_lds) + 132 * (tid >> 8);
    const int snb = sh.Is / 128, items = M * snb;
    const int stride = 4 * ((int)gridDim.x - routed_wgs);
    for (int i0 = 4 * ((int)blockIdx.x - routed_wgs); i0 < items; i0 += stride) {
      const int it = i0 + (tid >> 8);
      shared_mid_block(sh, it / snb, it % snb, M, H, u_lds, tid & 255, it < items);
    }
    return;
  }
  const int nblk = I / 128;
  const int tile = (int)blockIdx.x / nblk, b = (int)blockIdx.x - tile * nblk;
  // the tile is read beside meta (index clamped to the tile array's bound)
  const int4 tl = tiles[min(tile, tmax - 1)];
  const int nt = meta[0];
  asm volatile("" ::"s"(nt), "s"(tl.x));
  if (tile >= nt) return;
  const int e = tl.x, r0 = tl.y, rows = tl.z - tl.y;
  uint8_t* xl = gq_lds;                                 // [16][LX] E2M1 codes
  uint8_t* sl = xl + 16 * LX;                           // [16][LS] E8M0 scales
  float* gul = reinterpret_cast<float*>(sl + 16 * LS);  // [2][16][128] gate, up
  // The staging threads' entries first, so that waiting for them does not
  // wait for the weights (loads complete in issue order); every load is
  // unconditional (rows past the tile's end read its last row and are
  // stored as zeros), so no branch makes the compiler wait early.
  int se[KST];
#pragma unroll
  for (int q = 0; q < KST; ++q) se[q] = sorted_entry[r0 + min((tid + kGqThreads * q) / CPR, rows - 1)];
  const int sse = sorted_entry[r0 + min(tid / SPR, rows - 1)];
  // wave w: gate row block w (w < 8) or up row block w - 8 of mid block b
  const size_t rb = (size_t)e * (I / 8) + (wave < 8 ? 0 : I / 16) + 8 * b + (wave & 7);
  const uint8_t* pw = w13p + rb * NKS * 1024 + 16 * lane;  // + 1024 ks
  const uint8_t* ps = s13p + rb * NSS * 256 + 4 * lane;    // + 256 ss: byte j is K-step 4 ss + j
  uint4 wb[R][4];
  uint32_t ws[R];
  auto load = [&](int ss, int q) {
#pragma unroll
    for (int j = 0; j < 4; ++j) wb[q][j] = ld16(pw + (size_t)(4 * ss + j) * 1024);
    ws[q] = ld4(ps + 256 * ss);
  };
#pragma unroll
  for (int q = 0; q < R; ++q) load(q, q);
  // the tile's x rows into LDS
  uint4 xv[KST];
#pragma unroll
  for (int q = 0; q < KST; ++q) xv[q] = ld16(xq + (size_t)(se[q] / k) * (H / 2) + 16 * ((tid + kGqThreads * q) % CPR));
  const uint4 sv = ld16(xs + (size_t)(sse / k) * (H / 32) + 16 * (tid % SPR));
#pragma unroll
  for (int q = 0; q < KST; ++q) {
    const int idx = tid + kGqThreads * q, row = idx / CPR;  // 16 CPR = KST x 1024: every idx is a chunk
    *reinterpret_cast<uint4*>(xl + row * LX + 16 * (idx % CPR)) = row < rows ? xv[q] : make_uint4(0, 0, 0, 0);
  }
  if (tid < 16 * SPR)
    *reinterpret_cast<uint4*>(sl + (tid / SPR) * LS + 16 * (tid % SPR)) =
        tid / SPR < rows ? sv : make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
  __syncthreads();
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* xr = xl + r * LX + 16 * g;  // + 64 ks
  const uint8_t* sr = sl + r * LS;            // + 16 ss: byte 4 j + g is K-step 4 ss + j
#pragma unroll
  for (int ss = 0; ss < NSS; ++ss) {
    const int q = ss % R;
    const uint4 sa4 = *reinterpret_cast<const uint4*>(sr + 16 * ss);
    const uint32_t xw[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 a = *reinterpret_cast<const uint4*>(xr + 64 * (4 * ss + j));
      acc = mfma_fp4(a, wb[q][j], acc, (xw[j] >> (8 * g)) & 0xFFu, (ws[q] >> (8 * j)) & 0xFFu);
    }
    if (ss + R < NSS) load(ss + R, q);  // the slot's next super-step
  }
  // D[4 g + i][r]: tile row 4 g + i, column r of the wave's 16 (gate or up) columns
  float* gw = gul + (wave < 8 ? 0 : 16 * 128) + 16 * (wave & 7) + r;
#pragma unroll
  for (int i = 0; i < 4; ++i) gw[(4 * g + i) * 128] = acc[i];
  __syncthreads();
  // wave m: tile row m, columns 2 lane, 2 lane + 1 of the block
  const float2 G = *reinterpret_cast<const float2*>(gul + wave * 128 + 2 * lane);
  const float2 U = *reinterpret_cast<const float2*>(gul + 16 * 128 + wave * 128 + 2 * lane);
  const float h0 = silu_mul(G.x, U.x), h1 = silu_mul(G.y, U.y);
  if (MX) {
    // MXFP4 mid: the 16 lanes of a 32-column block form its E8M0 scale from
    // the largest |h| bits and the E2M1 codes of h 2^(127 - s) (the rule of
    // the separate MXFP4 mid quantization); rows of I/2 code bytes and I/32
    // scale bytes
    uint32_t am = max(__float_as_uint(h0) & 0x7FFFFFFFu, __float_as_uint(h1) & 0x7FFFFFFFu);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, o, 64));
    const uint32_t sc = mx_scale_code_f32(am);
    const int sh = 127 - (int)sc;
    const uint32_t code = e2m1_pack2(ldexpf(h0, sh), ldexpf(h1, sh));
    if (wave < rows) {
      midq[(size_t)(r0 + wave) * (I / 2) + 64 * b + lane] = (uint8_t)code;
      if ((lane & 15) == 0)
        reinterpret_cast<uint8_t*>(mids)[(size_t)(r0 + wave) * (I / 32) + 4 * b + (lane >> 4)] = (uint8_t)sc;
    }
  } else {
    const float amax = wave_max(fmaxf(fabsf(h0), fabsf(h1)));
    const float sc = __fdiv_rn(amax, 448.0f);
    const uint32_t c01 = sc > 0.f ? e4m3_pack2(__fdiv_rn(h0, sc), __fdiv_rn(h1, sc)) : 0u;
    if (wave < rows) {
      *reinterpret_cast<uint16_t*>(midq + (size_t)(r0 + wave) * I + 128 * b + 2 * lane) = (uint16_t)c01;
      if (lane == 0) mids[(size_t)(r0 + wave) * nblk + b] = sc;
    }
  }
}

hipError_t launch_gate_up_quant(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int64_t H = p->s.H, I = p->s.I, n = a.M * p->s.top_k;
  const int tmax = (int)((n + std::min<int64_t>(p->s.E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows);
  const int routed = tmax * (int)(I / 128);
  const SharedSmall sh = shared_small(p, a.M);  // the fused shared expert's h: four 128-blocks a workgroup
  const int sh_wgs = sh.part ? (int)((a.M * (sh.Is / 128) + 3) / 4) : 0;
  const size_t lds = std::max(gate_up_quant_lds(H), (size_t)4 * 132 * 4);
  if (H % 2048 || H > kGqMaxH || lds > 160 * 1024) return hipErrorInvalidValue;
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(routed + sh_wgs), dim3(kGqThreads), lds, a.stream, ev, wsp<uint8_t>(p, p->L.xq),
                    wsp<uint8_t>(p, p->L.xs), reinterpret_cast<const uint8_t*>(a.w13),
                    reinterpret_cast<const uint8_t*>(a.s13), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                    wsp<int>(p, p->X.meta), (int)I, (int)p->s.top_k, tmax, wsp<uint8_t>(p, p->L.midq),
                    wsp<float>(p, p->L.mids), routed, sh, (int)a.M);
  };
  auto pick = [&](auto mxc) {
    constexpr bool MXV = decltype(mxc)::value;
    switch (H / 2048) {
      case 1: return go(gate_up_quant_kernel<1, MXV>);
      case 2: return go(gate_up_quant_kernel<2, MXV>);
      case 3: return go(gate_up_quant_kernel<3, MXV>);
      case 4: return go(gate_up_quant_kernel<4, MXV>);
      default: return hipErrorInvalidValue;
    }
  };
  return p->mid_fmt == MOE_MID_MXFP4 ? pick(std::true_type()) : pick(std::false_type());
}

hipError_t launch_gate_up(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int I = (int)p->s.I;
  const int64_t n = a.M * p->s.top_k;
  const int64_t t16 = (n + std::min<int64_t>(p->s.E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows;
  const int64_t work_max = t16 * (I / 16);
  const int blocks = (int)std::min<int64_t>(work_max, 2048);
  return launch_k(gate_up_m16_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.xq),
                  wsp<uint8_t>(p, p->L.xs), reinterpret_cast<const uint8_t*>(a.w13),
                  reinterpret_cast<const uint8_t*>(a.s13), wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles),
                  wsp<int>(p, p->X.meta), wsp<float>(p, p->X.h), (int)p->s.H, I, (int)p->s.top_k);
}

hipError_t launch_gate_up_route(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int I = (int)p->s.I, E = (int)p->s.E, H = (int)p->s.H;
  if (a.M > kRqM || E > kRqMaxE || H > kRqMaxH || p->s.top_k > 16) return hipErrorInvalidValue;
  const int64_t n = a.M * p->s.top_k;
  const int64_t tiles = std::min<int64_t>(E, n);  // one tile per active expert
  const int blocks = (int)std::min<int64_t>(tiles * (I / 16), 2048);
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(blocks), dim3(256), 0, a.stream, ev, a.logits, reinterpret_cast<const uint16_t*>(a.x),
                    (int)a.M, E, (int)p->s.top_k, H, p->s.routed_scaling, reinterpret_cast<const uint8_t*>(a.w13),
                    reinterpret_cast<const uint8_t*>(a.s13), I, wsp<int>(p, p->L.topk_ids),
                    wsp<float>(p, p->L.topk_w), wsp<int>(p, p->L.count), wsp<int>(p, p->L.offset),
                    wsp<int>(p, p->L.sorted_entry), wsp<int4>(p, p->X.tiles), wsp<int>(p, p->X.meta),
                    wsp<uint8_t>(p, p->L.xq), wsp<uint8_t>(p, p->L.xs), wsp<float>(p, p->X.h));
  };
  return E <= 64 ? go(gate_up_route_kernel<1>) : E <= 128 ? go(gate_up_route_kernel<2>) : go(gate_up_route_kernel<4>);
}

hipError_t launch_act_quant(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int rows = (int)(a.M * p->s.top_k);
  const int I = (int)p->s.I;
  const SharedSmall sh = shared_small(p, a.M);  // the fused shared expert's h: a workgroup per 128-block
  const int64_t waves = (int64_t)rows * (I / 128);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((waves + 3) / 4, 8192));
  const int sh_blocks = sh.part ? (int)(a.M * (sh.Is / 128)) : 0;
  return launch_k(act_quant_kernel, dim3(blocks + sh_blocks), dim3(256), 0, a.stream, ev, wsp<float>(p, p->X.h),
                  rows, I, wsp<uint8_t>(p, p->L.midq), wsp<float>(p, p->L.mids), blocks, sh, (int)a.M,
                  (int)p->s.H);
}

}  // namespace qmoe
