// Host-side plan and the launch interface between the C ABI (api.hip) and
// the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qmoe.h"

namespace qmoe {

constexpr int kTileRows = 16;  // sorted rows per tile of the small-token kernels
constexpr int kFp4BigRows = 64;  // sorted rows per tile of the MXFP4-mid down above kMidM tokens
constexpr int kBigRows = 32;   // sorted rows per tile of the large-token down kernel
constexpr int kGuRows = 64;    // sorted rows per tile of the large-token gate/up kernel
constexpr int kDownItemCols = 256; // output columns per down work item of the large-token kernel

// Workspace regions beyond the public layout.
struct Internal {
  size_t tiles;    // int4 [T16]: {expert, row_begin, row_end, 0}
  size_t meta;     // int32 [64]: meta[0] tiles, meta[1] gate/up items, meta[2] down items, meta[3] 64-row tiles of the MXFP4-mid down (mid-range calls)
  size_t gu_items; // int4 [TG * I/128]: {expert, row_begin, row_end, column block}, tiles of kGuRows, large M
  size_t dn_items; // int4 [TB * H/kDownItemCols]: {expert, row_begin, row_end, column chunk} (M > kSmallM); mid-range calls with the MXFP4 mid: its 64-row tiles
  size_t bitmap;   // uint32 [E, ceil(M/32)]: bit t of row e = token t picked e; zero between calls
  size_t done;     // int: workgroups of the one-launch sort past their bitmap copy; zero between calls
  size_t pw;       // int2 [E, ceil(M/32)]: {set bits of row e before word w, word w}
  size_t h;        // fp32 [n, I]: SiLU(gate)*up, rows in sorted order
  size_t sh_h;     // fp32 [M, Is]
  size_t sh_part;  // float64 [min(M, kSmallM), H/128, 2 Is]: block partials of the fused shared gate/up
  size_t sync_begin, sync_bytes;  // region zeroed once when the workspace is bound
};

}  // namespace qmoe

struct moe_plan {
  moe_shape s;
  int device;
  int num_cus;     // compute units of the device
  int64_t n_max;   // M * top_k
  int64_t t16_max; // upper bound on tiles of 16 sorted rows
  int64_t words;   // ceil(M / 32)
  int64_t tb_max;  // upper bound on tiles of kBigRows sorted rows
  moe_ws_layout L;
  qmoe::Internal X;
  uint8_t* ws;
  size_t ws_bytes;
  const void* ws13;   // the shared expert's gate/up and down weights as digit rows (moe_plan_set_shared)
  const float* ss13;
  const float* ss2;
  hipEvent_t events[16];
  int n_events;
  hipEvent_t call_start, call_stop;
  moe_tp_exchange tpx;  // tensor-parallel exchange epilogue (tpx.tp > 0: on)
  int mid_fmt;     // moe_mid_format
  unsigned layout; // moe_weight_layout flags declared by the caller
  int shared_slot; // 1: expert E-1 is the shared expert, slot top_k-1 of every token
};

namespace qmoe {

// Stage timing: a launch with non-null events records them around itself.
struct Ev {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename... KArgs, typename... Args>
inline hipError_t launch_k(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, Ev ev,
                           Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kern, grid, block, lds, s, ev.start, ev.stop, 0, static_cast<KArgs>(args)...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, s, static_cast<KArgs>(args)...);
  return hipGetLastError();
}

// Largest M (and M * top_k) served by the single-workgroup routing/sort
// path and the small-token kernels (down and combine in one launch, whose
// per-entry results must fit in LDS).
constexpr int kSmallM = 16;
constexpr int kSmallRows = 512;
inline bool small_path(int64_t M, int64_t k) { return M <= kSmallM && M * k <= kSmallRows; }
// Up to kMidM tokens (and at most 16 slots) gate/up runs on 16-row tiles
// with the mid quantization in its own launch (the large path's routing and
// sort otherwise): with few rows per expert, 64-row tiles leave most of the
// chip idle.
constexpr int kMidM = 256;
// Largest E of a plan (a routing workgroup gathers its tokens' bitmap bits
// per expert in LDS).
constexpr int kRouteMaxE = 1024;
// Above kMidM tokens the sort runs in one launch while the token bitmap (E x
// ceil(M/32) words) is small enough for every workgroup to copy it into LDS
// (c3's 8192 words: align 12.7 -> 10.1 us; at 32768 words, c4's, the copies
// made the one launch slower than two: 14.5 against 12.9 us) and its rows'
// prefixes fit 16 bits (M <= 65536); in two launches otherwise.
constexpr int kAlignLdsWords = 8192;
inline bool align_one_launch(int64_t E, int64_t M) {
  const int64_t words = (M + 31) / 32;
  return E * words <= kAlignLdsWords && words <= 2048;
}
inline bool mid_path(int64_t M, int64_t k) { return M <= kMidM && k <= 16; }
// Up to kSmallM tokens with the E4M3 mid, a block-FP8 shared expert of at
// most kSmallSharedI columns runs inside the routed launches
// (shared_small.h) instead of a pass of its own.
constexpr int kSmallSharedI = 512;

struct CallArgs {
  int64_t M;
  const void* x;
  const float* logits;
  const void* w13;
  const void* s13;
  const void* w2;
  const void* s2;
  void* out;
  hipStream_t stream;
};

template <typename T>
inline T* wsp(const moe_plan* p, size_t off) { return reinterpret_cast<T*>(p->ws + off); }

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t s);
// row-major MXFP4 gate/up weights and scales -> the packed layout (pack.hip)
hipError_t launch_pack_w13(const void* w13, const void* s13, int64_t E, int64_t I, int64_t H, void* w13p, void* s13p,
                           hipStream_t stream);
// row-major MXFP4 down weights and scales -> the packed layout of the
// MXFP4-mid down (pack.hip)
hipError_t launch_pack_w2(const void* w2, const void* s2, int64_t E, int64_t I, int64_t H, void* w2p, void* s2p,
                          hipStream_t stream);
// Small M (<= kSmallM): route + sort + x quantization in one workgroup.
hipError_t launch_route_small(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_route(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_align(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_gate_up(const moe_plan* p, const CallArgs& a, Ev ev);
// Mid-range calls with at least 8 entries per expert on average (M k >= 8 E)
// and H a multiple of 2048 up to kGqMaxH (the tile's x rows
// staged whole in LDS): gate/up and the mid quantization in one launch
// (gate_up.hip), no h and no act_quant launch. Its work unit streams a whole
// 128-column mid block's weights (786 KB at H 6144) at up to ~45 GB/s per
// CU: with fewer entries the units are too few, or too unequal, to keep the
// chip busy, and the 16-column items of the two-launch path win (c1 41 us
// against 34; TP8 M 32..128 hot and mixed +1..+12 us; M 256: hot 73.5 ->
// 64.7, mixed 171 -> 169, spread 163 -> 158 us).
constexpr int kGqMaxH = 8192;
inline bool gq_path(const moe_plan* p, int64_t M) {
  return mid_path(M, p->s.top_k) && M * p->s.top_k >= 8 * p->s.E && p->s.H % 2048 == 0 && p->s.H <= kGqMaxH;
}
hipError_t launch_gate_up_quant(const moe_plan* p, const CallArgs& a, Ev ev);
// Up to kRqM tokens (E <= kRqMaxE, H <= kRqMaxH, the E4M3 mid, no shared
// expert, no shared slot): gate/up routes, sorts and quantizes x itself
// (gate_up.hip), so the call has no routing launch.
constexpr int kRqM = 4;
constexpr int kRqMaxE = 256;
constexpr int kRqMaxH = 6144;
inline bool rq_path(const moe_plan* p, int64_t M) {
  return M >= 1 && M <= kRqM && p->s.E <= kRqMaxE && p->s.H <= kRqMaxH && p->s.top_k <= 16 &&
         p->mid_fmt == MOE_MID_E4M3 && p->s.shared_I == 0 && !p->shared_slot;
}
hipError_t launch_gate_up_route(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_act_quant(const moe_plan* p, const CallArgs& a, Ev ev);
// small M: down and the combine in one launch; y stays on chip
int down_combine_cols(int H, int cus);
hipError_t launch_down_combine(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_shared(const moe_plan* p, const CallArgs& a, Ev ev);
inline bool shared_fused(const moe_plan* p, int64_t M) {
  return p->s.shared_I > 0 && p->s.shared_I <= kSmallSharedI && p->mid_fmt == MOE_MID_E4M3 &&
         small_path(M, p->s.top_k);
}
// Up to kQdBlocks (row, 128-block) pairs of the E4M3 mid (M = 4 at top-8 and
// I = 256) on the routing gate/up path (rq_path): every down workgroup
// quantizes the mid from h itself while its weights are in flight
// (workgroup 0 stores the codes), so the call has no act_quant launch.
constexpr int kQdBlocks = 64;
inline bool qd_path(const moe_plan* p, int64_t M) {
  const int64_t n = M * p->s.top_k, nb = p->s.I / 128;
  const int64_t slots = nb <= 2 ? 8 : nb == 3 ? 5 : 4;  // the small down's ring slots at this I
  return rq_path(p, M) && n * nb <= kQdBlocks && n <= 4 * slots;  // no wave with more tiles than slots
}
// row-major E4M3 shared-expert weights -> digit rows: gate/up [2 Is, H/128,
// 3, 128], then down [H, Is/128, 3, 128], then the E4M3 codes themselves
// (gate/up [2 Is, H], down [H, Is]), at `packed` (shared.hip)
hipError_t launch_pack_shared(const void* ws13, const void* ws2, int64_t Is, int64_t H, void* packed,
                              hipStream_t stream);
// large M: LDS-staged tiles (kGuRows rows for gate/up, which includes the mid
// quantization; kBigRows rows for down)
hipError_t launch_gate_up_big(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_down_big(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_combine(const moe_plan* p, const CallArgs& a, Ev ev);
// With the tensor-parallel exchange on, the combines write the rank's float64
// partial into its own inbox slot instead of bf16 `out` (else nullptr).
inline double* tp_own_partial(const moe_plan* p) {
  return p->tpx.tp > 0 ? p->tpx.inbox + (size_t)p->tpx.rank * (size_t)p->s.M * (size_t)p->s.H : nullptr;
}
// the exchange: push the partial to the peers, wait for theirs, sum in rank
// order, one bf16 rounding into `out` (tp_exchange.hip)
hipError_t launch_tp_exchange(const moe_plan* p, const CallArgs& a, Ev ev);
// MXFP4 mid hand-off (a4w4.hip): mid per 32 as E2M1 + E8M0; down on the
// scaled FP4 MFMA over 16-row tiles, y to HBM
hipError_t launch_act_quant_mx(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_down_fp4(const moe_plan* p, const CallArgs& a, Ev ev);

}  // namespace qmoe
