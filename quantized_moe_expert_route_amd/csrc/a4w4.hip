// The MXFP4 mid hand-off: the comparison arm the pages time IQ2R against,
// stock experts quantized online to MXFP4 ("IQ2R: load GLM-5.3 packed MoE
// checkpoints with TP slicing", Results (MXFP4 vs IQ2R)), read as FP4
// activations in both GEMMs. mid is quantized per 32 with the rule x takes
// (E8M0 scale 2^(floor(log2 amax) - 2), E2M1 round-to-nearest-even,
// saturating), and down multiplies two MXFP4 operands on the scaled FP4 MFMA,
// so no operand is widened. Used on the 16-row tiles (up to kMidM tokens);
// y goes through HBM to the combine launch.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

constexpr int kDfCbs = 4;  // column blocks whose weights a wave has in flight

// A thread quantizes 8 consecutive elements of a row; the 4 lanes of a quad
// form one 32-block (I/8 is a multiple of 16, so quads never straddle rows
// and a grid-stride step keeps them whole).
__global__ __launch_bounds__(256) void act_quant_mx_kernel(const float* __restrict__ h, int rows, int I,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int per_row = I / 8;
  const int64_t total = (int64_t)rows * per_row;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < total; u += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(u / per_row), c = (int)(u - (int64_t)row * per_row) * 8;
    const float4 v0 = *reinterpret_cast<const float4*>(h + (size_t)row * I + c);
    const float4 v1 = *reinterpret_cast<const float4*>(h + (size_t)row * I + c + 4);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = max(am, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    const uint32_t sc = mx_scale_code_f32(am);
    const int sh = 127 - (int)sc;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed |= e2m1_pack2(ldexpf(v[2 * i], sh), ldexpf(v[2 * i + 1], sh)) << (8 * i);
    *reinterpret_cast<uint32_t*>(q + (size_t)row * (I / 2) + c / 2) = packed;
    if ((u & 3) == 0) s[(size_t)row * (I / 32) + c / 32] = (uint8_t)sc;
  }
}

// down on MXFP4 x MXFP4, w2 packed by moe_pack_w2. Work item = (tile of RB
// x 16 sorted rows, group of cbg 64-column blocks): 16-row tiles up to
// kSmallM tokens, 64-row tiles above (RB = 4: each weight fragment then feeds
// four MFMA row blocks instead of one). The workgroup stages the row blocks
// of the tile that hold rows (up to RB x 16 x I/2 bytes, contiguous in
// sorted order) and their scale bytes in
// LDS with one coalesced read; each wave then holds its A fragments in
// registers and streams the B fragments of its 16 columns of every column
// block in the group: in K-step ks lane 16 g + r supplies MX block 4 ks + g
// of tile row r (A) and of weight column r (B), and a packed K-step of a
// 16-column block is 1 KB contiguous in lane order. Items are ordered column
// group first, so the tiles of one expert sharing a w2 slice are adjacent,
// and each XCD (blockIdx % 8) walks its own contiguous eighth of them.
template <int NKS, int RB>
__global__ __launch_bounds__(256) void down_fp4_kernel(const uint8_t* __restrict__ midq, const uint8_t* __restrict__ mids,
                                                       const uint8_t* __restrict__ w2p, const uint32_t* __restrict__ s2p,
                                                       const int* __restrict__ sorted_entry,
                                                       const int4* __restrict__ tiles, const int* __restrict__ meta,
                                                       int H, int cbg, float* __restrict__ y) {
  constexpr int I = NKS * 128;
  constexpr int Ib = I / 2, Isc = I / 32;
  constexpr int LDA = Ib + 16;  // padded row: the 16 rows of a fragment read meet 16 different bank groups
  constexpr int TR = 16 * RB;   // rows per tile
  __shared__ __align__(16) uint8_t sm_a[TR * LDA];
  __shared__ uint8_t sm_s[TR * 16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int nt = meta[0];
  const int ncb = H / 64;
  const int ncg = (ncb + cbg - 1) / cbg;
  const int64_t n_work = (int64_t)nt * ncg;
  const int per_x = (int)gridDim.x / 8;  // the grid is a multiple of 8
  const int xcd = (int)blockIdx.x & 7, slot = (int)blockIdx.x >> 3;
  const int64_t chunk = (n_work + 7) / 8;
  const int64_t w_end = min(n_work, (int64_t)(xcd + 1) * chunk);
  for (int64_t w = (int64_t)xcd * chunk + slot; w < w_end; w += per_x) {
    const int cg = (int)(w / nt), ti = (int)(w - (int64_t)cg * nt);
    const int4 tl = tiles[ti];  // {expert, row_begin, row_end, 0}
    __syncthreads();  // the previous item's LDS reads are done
    // rows past the tile's end repeat its last row (their results are
    // dropped); only the row blocks that hold rows are staged
    const int nrb = min(RB, (tl.z - tl.y + 15) / 16);
    constexpr int cpr = Ib / 16;  // 16-byte chunks per row
#pragma unroll
    for (int q = 0; q < (TR * cpr + 255) / 256; ++q) {
      const int idx = tid + 256 * q;
      if (idx < 16 * nrb * cpr) {
        const int rr = idx / cpr, c = idx - rr * cpr;
        const int row = min(tl.y + rr, tl.z - 1);
        *reinterpret_cast<uint4*>(sm_a + rr * LDA + 16 * c) = ld16(midq + (size_t)row * Ib + 16 * c);
      }
    }
    for (int idx = tid; idx < 16 * nrb * Isc; idx += 256) {
      const int rr = idx / Isc, c = idx - rr * Isc;
      sm_s[rr * 16 + c] = mids[(size_t)min(tl.y + rr, tl.z - 1) * Isc + c];
    }
    __syncthreads();
    // (a 64-row tile of a small expert computes only its first row blocks)
    uint4 a[RB][NKS];
    uint32_t sa[RB][NKS];
    int ent[RB][4];
#pragma unroll
    for (int i2 = 0; i2 < RB; ++i2) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        a[i2][ks] = *reinterpret_cast<const uint4*>(sm_a + (16 * i2 + r) * LDA + 64 * ks + 16 * g);
        sa[i2][ks] = sm_s[(16 * i2 + r) * 16 + 4 * ks + g];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = tl.y + 16 * i2 + 4 * g + i;
        ent[i2][i] = m < tl.z ? sorted_entry[m] : -1;
      }
    }
    const int cb0 = cg * cbg, cb1 = min(ncb, cb0 + cbg);
    for (int cb = cb0; cb < cb1; cb += kDfCbs) {
      uint4 b[kDfCbs][NKS];
      uint32_t sb[kDfCbs];
#pragma unroll
      for (int q = 0; q < kDfCbs; ++q) {
        if (cb + q < cb1) {
          const size_t rb = (size_t)tl.x * (H / 16) + (size_t)(cb + q) * 4 + wave;  // packed 16-row block
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) b[q][ks] = ld16(w2p + (rb * NKS + ks) * 1024 + 16 * lane);
          sb[q] = s2p[rb * 64 + lane];
        }
      }
#pragma unroll
      for (int q = 0; q < kDfCbs; ++q) {
        if (cb + q < cb1) {
          const int col = (cb + q) * 64 + wave * 16 + r;
#pragma unroll
          for (int i2 = 0; i2 < RB; ++i2) {
            if (i2 < nrb) {
              v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < NKS; ++ks)
                acc = mfma_fp4(a[i2][ks], b[q][ks], acc, sa[i2][ks], (sb[q] >> (8 * ks)) & 0xFFu);
              // D row 16 i2 + 4 g + i of the tile, column r
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (ent[i2][i] >= 0) y[(size_t)ent[i2][i] * H + col] = acc[i];
            }
          }
        }
      }
    }
  }
}

hipError_t launch_act_quant_mx(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int rows = (int)(a.M * p->s.top_k);
  const int I = (int)p->s.I;
  const int64_t threads = (int64_t)rows * (I / 8);
  const int blocks = (int)std::min<int64_t>((threads + 255) / 256, 8192);
  return launch_k(act_quant_mx_kernel, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<float>(p, p->X.h), rows, I,
                  wsp<uint8_t>(p, p->L.midq), wsp<uint8_t>(p, p->L.mids));
}

hipError_t launch_down_fp4(const moe_plan* p, const CallArgs& a, Ev ev) {
  const int H = (int)p->s.H, I = (int)p->s.I;
  const int64_t n = a.M * p->s.top_k;
  // 64-row tiles above kSmallM tokens: above kMidM in the tile array, from
  // the one-workgroup sort of mid-range calls where the E4M3 down keeps its
  // items (their count in meta[3]); 16-row tiles for the small path
  const bool big = !small_path(a.M, p->s.top_k);
  const bool mid = big && mid_path(a.M, p->s.top_k);
  const int4* tiles = mid ? wsp<int4>(p, p->X.dn_items) : wsp<int4>(p, p->X.tiles);
  const int* meta = wsp<int>(p, p->X.meta) + (mid ? 3 : 0);
  const int tr = big ? kFp4BigRows : kTileRows;
  const int64_t t16 = (n + std::min<int64_t>(p->s.E, n) * (tr - 1) + tr - 1) / tr;
  const int ncb = H / 64;
  // column blocks per item: as many as still leave ~2048 items to spread
  int cbg = 1;
  while (cbg < 16 && t16 * ((ncb + 2 * cbg - 1) / (2 * cbg)) >= 2048) cbg *= 2;
  const int64_t items = t16 * ((ncb + cbg - 1) / cbg);
  const int blocks = (int)std::min<int64_t>((items + 7) / 8 * 8, 2048);
  auto go = [&](auto kern) {
    return launch_k(kern, dim3(blocks), dim3(256), 0, a.stream, ev, wsp<uint8_t>(p, p->L.midq),
                    wsp<uint8_t>(p, p->L.mids), reinterpret_cast<const uint8_t*>(a.w2),
                    reinterpret_cast<const uint32_t*>(a.s2), wsp<int>(p, p->L.sorted_entry),
                    tiles, meta, H, cbg, wsp<float>(p, p->L.y));
  };
  switch (I / 128) {
    case 1: return big ? go(down_fp4_kernel<1, 4>) : go(down_fp4_kernel<1, 1>);
    case 2: return big ? go(down_fp4_kernel<2, 4>) : go(down_fp4_kernel<2, 1>);
    case 3: return big ? go(down_fp4_kernel<3, 4>) : go(down_fp4_kernel<3, 1>);
    case 4: return big ? go(down_fp4_kernel<4, 4>) : go(down_fp4_kernel<4, 1>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qmoe
