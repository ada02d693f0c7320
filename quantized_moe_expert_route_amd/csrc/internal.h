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
constexpr int kBigRows = 32;   // sorted rows per tile of the large-token down kernel
constexpr int kGuRows = 64;    // sorted rows per tile of the large-token gate/up kernel
constexpr int kDownItemCols = 256; // output columns per down work item of the large-token kernel

// Workspace regions beyond the public layout.
struct Internal {
  size_t tiles;    // int4 [T16]: {expert, row_begin, row_end, 0}
  size_t meta;     // int32 [64]: meta[0] tiles, meta[1] gate/up items, meta[2] down items
  size_t gu_items; // int4 [TG * I/128]: {expert, row_begin, row_end, column block}, tiles of kGuRows, large M
  size_t dn_items; // int4 [TB * H/kDownItemCols]: {expert, row_begin, row_end, column chunk}, large M
  size_t toff;     // int32 [2][E + 1]: tile prefix per expert of the gate/up and the down tiles, large M
  size_t bitmap;   // uint32 [E, ceil(M/32)]: bit t of row e = token t picked e; zero between calls
  size_t pw;       // int2 [E, ceil(M/32)]: {set bits of row e before word w, word w}
  size_t h;        // fp32 [n, I]: SiLU(gate)*up, rows in sorted order
  size_t sh_h;     // fp32 [M, Is]
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
  const void* ws13;
  const float* ss13;
  const void* ws2;
  const float* ss2;
  hipEvent_t events[16];
  int n_events;
  hipEvent_t call_start, call_stop;
  int mid_fmt;     // moe_mid_format
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
inline bool mid_path(int64_t M, int64_t k) { return M <= kMidM && k <= 16; }

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
hipError_t launch_act_quant(const moe_plan* p, const CallArgs& a, Ev ev);
// small M: down and the combine in one launch; y stays on chip
int down_combine_cols(int H, int cus);
hipError_t launch_down_combine(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_shared(const moe_plan* p, const CallArgs& a, Ev ev);
// large M: LDS-staged tiles (kGuRows rows for gate/up, which includes the mid
// quantization; kBigRows rows for down)
hipError_t launch_gate_up_big(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_down_big(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_combine(const moe_plan* p, const CallArgs& a, Ev ev);
// MXFP4 mid hand-off (a4w4.hip): mid per 32 as E2M1 + E8M0; down on the
// scaled FP4 MFMA over 16-row tiles, y to HBM
hipError_t launch_act_quant_mx(const moe_plan* p, const CallArgs& a, Ev ev);
hipError_t launch_down_fp4(const moe_plan* p, const CallArgs& a, Ev ev);

}  // namespace qmoe
