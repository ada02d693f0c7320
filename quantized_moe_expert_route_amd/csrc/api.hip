// C ABI of the routed-MoE call: validation, workspace layout and the launch
// sequence. Nothing here allocates device memory or synchronizes a stream.
#include <string.h>

#include <algorithm>
#include <new>

#include "internal.h"

#include <climits>
#include <mutex>

using namespace qmoe;

namespace {

const char* kStageNames[] = {"route", "align", "gate_up", "act_quant", "shared", "down", "combine"};
constexpr int kStages = 7;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->M < 0 || s->H <= 0 || s->E <= 0 || s->I <= 0 || s->top_k <= 0 || s->shared_I < 0)
    return MOE_ERR_INVALID_ARG;
  if (!(s->routed_scaling > 0.f) || s->routed_scaling > 3.0e38f) return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->E) return MOE_ERR_INVALID_ARG;
  if (s->H % 512 != 0 || s->I % 128 != 0 || s->I > 512 || s->E > 1024 || s->top_k > 16 ||
      s->shared_I % 128 != 0 || s->shared_I > 2048)
    return MOE_ERR_UNSUPPORTED;
  if (s->M > (int64_t)1 << 20 || s->H > 65536) return MOE_ERR_UNSUPPORTED;
  if (s->M * (s->H / 2) > INT32_MAX) return MOE_ERR_UNSUPPORTED;  // x codes addressed with 32-bit offsets
  return MOE_OK;
}

struct Layout {
  moe_ws_layout L;
  Internal X;
  int64_t t16, tb, tg, words;
};

Layout make_layout(const moe_shape& s) {
  Layout r;
  memset(&r, 0, sizeof(r));
  const size_t M = (size_t)s.M, H = (size_t)s.H, E = (size_t)s.E, I = (size_t)s.I, k = (size_t)s.top_k;
  const size_t Is = (size_t)s.shared_I;
  const size_t n = M * k;
  r.t16 = (int64_t)((n + std::min(E, n) * (kTileRows - 1) + kTileRows - 1) / kTileRows);
  r.tb = (int64_t)((n + std::min(E, n) * (kBigRows - 1) + kBigRows - 1) / kBigRows);
  r.tg = (int64_t)((n + std::min(E, n) * (kGuRows - 1) + kGuRows - 1) / kGuRows);
  r.words = (int64_t)((M + 31) / 32);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    off = align256(off);
    size_t at = off;
    off += bytes;
    return at;
  };
  r.L.topk_ids = take(4 * n);
  r.L.topk_w = take(4 * n);
  r.L.count = take(4 * E);
  r.L.offset = take(4 * (E + 1));
  r.L.sorted_entry = take(4 * n);
  r.X.tiles = take(16 * (size_t)r.t16);
  r.X.meta = take(256);
  r.X.gu_items = take(16 * (size_t)r.tg * (I / 128));
  r.X.dn_items = take(16 * (size_t)r.tb * (H / kDownItemCols));
  // the token bitmap and the one-launch sort's counter: zeroed when the
  // workspace is bound, and left zero by every call
  r.X.bitmap = take(4 * E * (size_t)r.words);
  r.X.done = take(4);
  r.X.sync_begin = r.X.bitmap;
  r.X.sync_bytes = align256(off) - r.X.bitmap;
  r.X.pw = take(8 * E * (size_t)r.words);
  r.L.xq = take(M * H / 2);
  r.L.xs = take(M * H / 32);
  r.X.h = take(4 * n * I);
  r.L.midq = take(n * I);
  r.L.mids = take(4 * n * (I / 128));
  r.L.y = take(4 * n * H);
  if (Is > 0) {
    // int8 digit rows, padded to whole 128-row tiles of the shared-expert GEMMs
    const size_t M128 = (M + 127) / 128 * 128;
    r.L.sh_xq = take(3 * M128 * H);
    r.L.sh_xs = take(4 * M * (H / 128));
    r.X.sh_h = take(4 * M * Is);
    r.L.sh_hq = take(3 * M128 * Is);
    r.L.sh_hs = take(4 * M * (Is / 128));
    r.L.sh_y = take(4 * M * H);
    r.X.sh_part = take(8 * std::min<size_t>(M, kSmallM) * (H / 128) * 2 * Is);
  }
  r.L.total_bytes = align256(off);
  return r;
}

// Device that owns a device pointer, or -1.
int ptr_device(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) return -1;
  return a.device;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) { ok = false; return; }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Checks of a call shared by moe_forward and moe_forward_noalloc (the
// workspace, `ws` of `ws_bytes` or none, is the caller's concern).
moe_status check_call(const moe_plan* plan, int64_t M, const void* const ptrs[7], const void* ws, size_t ws_bytes) {
  if (plan->s.shared_I > 0 && !plan->ws13) return MOE_ERR_INVALID_ARG;
  const bool mx = plan->mid_fmt == MOE_MID_MXFP4;
  // the weights must be in the layout the kernels read, as declared: gate/up
  // packed (row-major is not served), down packed exactly for the MXFP4 mid
  if (!(plan->layout & MOE_LAYOUT_W13_PACKED) || mx != ((plan->layout & MOE_LAYOUT_W2_PACKED) != 0))
    return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  for (int i = 0; i < 7; ++i)
    if (!ptrs[i] || !aligned16(ptrs[i])) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < 7; ++i)
    if (ptr_device(ptrs[i]) != plan->device) return MOE_ERR_DEVICE;
  const void* x = ptrs[0];
  const void* logits = ptrs[1];
  const void* out = ptrs[6];
  const size_t H = (size_t)plan->s.H, E = (size_t)plan->s.E;
  const size_t out_bytes = (size_t)M * H * 2;
  if (overlaps(out, out_bytes, x, (size_t)M * H * 2) || overlaps(out, out_bytes, logits, (size_t)M * E * 4) ||
      (ws && overlaps(out, out_bytes, ws, ws_bytes)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The launch sequence of one call on the workspace of `plan` (the plan's
// device current, the call's arguments checked).
hipError_t enqueue_call(const moe_plan* plan, const CallArgs& a) {
  const int64_t M = a.M;
  const bool mx = plan->mid_fmt == MOE_MID_MXFP4;
  const bool small = small_path(M, plan->s.top_k);
  const bool fused_combine = small && !mx;  // down and combine in one launch
  Ev ev[kStages];
  if (plan->n_events)
    for (int i = 0; i < kStages; ++i) ev[i] = Ev{plan->events[2 * i], plan->events[2 * i + 1]};
  const bool rq = rq_path(plan, M);  // gate/up routes for itself: no routing launch
  if (plan->call_start) {
    ev[rq ? 2 : 0].start = plan->call_start;    // the route launch (or the routing gate/up) comes first
    // down (+ combine), the combine, or the exchange comes last
    ev[fused_combine && plan->tpx.tp == 0 ? 5 : 6].stop = plan->call_stop;
  }
  // a stage with no launch of its own still records its (empty) interval
  auto none = [&](int i) -> hipError_t {
    if (!plan->n_events) return hipSuccess;
    hipError_t e = hipEventRecord(ev[i].start, a.stream);
    return e != hipSuccess ? e : hipEventRecord(ev[i].stop, a.stream);
  };
  // Up to kSmallM tokens: routing + sort + x quantization in one launch
  // (workgroup 0 routes and sorts, the others quantize x); gate/up on 16-row
  // tiles; the mid quantization; down with the combine (a workgroup owns 16
  // output columns of every slot, so the slot results never leave it). Up
  // to kRqM tokens (rq_path) gate/up routes, sorts and quantizes x itself,
  // and for at most kQdBlocks mid blocks (qd_path) down quantizes the mid.
  // (With the block-FP8 shared expert the routing launch also runs its
  // gate/up partials, so that case keeps it.)
  // Above kSmallM: routing spread over the GPU, a second launch sorts;
  // gate/up on 16-row tiles and the mid quantization up to kMidM tokens (in
  // one launch where M k >= 8 E: gq_path), above on 64-row tiles with the
  // mid quantization inside (every item owns whole mid blocks); down to y in
  // HBM; the combine.
  // With the MXFP4 mid: its own quantization (inside the 64-row-tile gate/up
  // above kMidM) and down kernel on the 16-row tiles, then the combine, for
  // every M.
  // A stage is never folded into its producer through a last-arriver
  // counter: the device-scope release/acquire that needs writes back and
  // invalidates a whole L2 of an XCD per workgroup and costs more than a
  // launch.
  hipError_t e = rq ? none(0) : small ? launch_route_small(plan, a, ev[0]) : launch_route(plan, a, ev[0]);
  if (e == hipSuccess) e = small ? none(1) : launch_align(plan, a, ev[1]);
  const bool tiles16 = mid_path(M, plan->s.top_k);  // 16-row-tile gate/up, mid quantization on its own
  const bool gq = gq_path(plan, M);  // 16-row tiles, the mid quantized inside gate/up
  if (e == hipSuccess)
    e = rq ? launch_gate_up_route(plan, a, ev[2]) : gq ? launch_gate_up_quant(plan, a, ev[2])
        : tiles16 ? launch_gate_up(plan, a, ev[2])
                  : launch_gate_up_big(plan, a, ev[2]);
  if (e == hipSuccess)
    e = !tiles16 || gq || qd_path(plan, M) ? none(3)
        : mx                              ? launch_act_quant_mx(plan, a, ev[3])
                                          : launch_act_quant(plan, a, ev[3]);
  // (a fused shared expert runs inside the routed launches: no pass of its own)
  if (e == hipSuccess) e = plan->s.shared_I > 0 && !shared_fused(plan, M) ? launch_shared(plan, a, ev[4]) : none(4);
  if (e == hipSuccess)
    e = mx ? launch_down_fp4(plan, a, ev[5]) : small ? launch_down_combine(plan, a, ev[5]) : launch_down_big(plan, a, ev[5]);
  if (plan->tpx.tp > 0) {
    // the combine (its own launch, or inside down) left the rank's partial
    // in its inbox slot; the exchange epilogue forms `out`
    if (e == hipSuccess && !fused_combine) e = launch_combine(plan, a, Ev{ev[6].start, nullptr});
    if (e == hipSuccess) e = launch_tp_exchange(plan, a, fused_combine ? ev[6] : Ev{nullptr, ev[6].stop});
    return e;
  }
  if (e == hipSuccess) e = fused_combine ? none(6) : launch_combine(plan, a, ev[6]);
  return e;
}

// Scratch of moe_forward_noalloc: the workspace of its calls, one copy per
// device, held until the process ends. In host code `scratch` names a host
// stand-in; the device address of a device's copy comes from
// hipGetSymbolAddress with that device current, looked up once per device
// (at plan creation, else at the first call) and kept in g_scratch.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// With `dev` current: the device address of its copy of `scratch`.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return e != hipSuccess ? e : hipErrorInvalidSymbol;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case MOE_ERR_DEVICE: return "no usable gfx950 device, or pointer on another device";
    case MOE_ERR_HIP: return "HIP runtime error while enqueueing";
  }
  return "unknown status";
}

int moe_stage_count(void) { return kStages; }

int moe_plan_stage_launches(const moe_plan* plan, int64_t M, int stage) {
  if (!plan || M < 0 || M > plan->s.M || stage < 0 || stage >= kStages) return -1;
  if (M == 0) return 0;
  const bool small = small_path(M, plan->s.top_k);
  const bool mx = plan->mid_fmt == MOE_MID_MXFP4;
  switch (stage) {
    case 0: return rq_path(plan, M) ? 0 : 1;      // route + x quantization (+ sort when small; + the shared expert's x when large, its gate/up partials when fused); inside gate/up on the rq path
    case 1: return small ? 0 : mid_path(M, plan->s.top_k) ? 1 : 2;  // align
    case 2: return 1;                             // gate_up (+ mid quantization when large)
    case 3: return mid_path(M, plan->s.top_k) && !gq_path(plan, M) && !qd_path(plan, M) ? 1 : 0;  // act_quant (inside gate/up above kMidM and on the gq path, inside down on the qd path)
    case 4: return plan->s.shared_I > 0 && !shared_fused(plan, M) ? (small ? 4 : 3) : 0;  // shared expert (0: inside the routed launches)
    case 5: return 1;                             // down (+ combine when small, E4M3 mid)
    default: return (small && !mx ? 0 : 1) + (plan->tpx.tp > 0 ? 1 : 0);  // combine (+ the exchange)
  }
}

const char* moe_stage_name(int i) { return (i >= 0 && i < kStages) ? kStageNames[i] : nullptr; }

moe_status moe_shape_workspace_bytes(const moe_shape* shape, size_t* bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = make_layout(*shape).L.total_bytes;
  return MOE_OK;
}

moe_status moe_plan_create(const moe_shape* shape, moe_plan** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_DEVICE;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_ERR_DEVICE;
  // set-up of moe_forward_noalloc's scratch on this device (a failure here
  // is reported by that entry point, which looks again)
  void* sp = nullptr;
  (void)scratch_address(dev, &sp);
  moe_plan* p = new (std::nothrow) moe_plan;
  if (!p) return MOE_ERR_INVALID_ARG;
  memset(p, 0, sizeof(*p));
  p->s = *shape;
  p->device = dev;
  p->num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  p->n_max = shape->M * shape->top_k;
  Layout lay = make_layout(*shape);
  p->L = lay.L;
  p->X = lay.X;
  p->t16_max = lay.t16;
  p->words = lay.words;
  p->tb_max = lay.tb;
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan* plan) { delete plan; }

size_t moe_plan_workspace_bytes(const moe_plan* plan) { return plan ? plan->L.total_bytes : 0; }

moe_status moe_plan_layout(const moe_plan* plan, moe_ws_layout* out) {
  if (!plan || !out) return MOE_ERR_INVALID_ARG;
  *out = plan->L;
  return MOE_OK;
}

moe_status moe_plan_set_workspace(moe_plan* plan, void* workspace, size_t bytes, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (!workspace || ((uintptr_t)workspace & 255u) != 0 || bytes < plan->L.total_bytes) return MOE_ERR_WORKSPACE;
  if (ptr_device(workspace) != plan->device) return MOE_ERR_DEVICE;
  DeviceGuard guard(plan->device);
  if (!guard.ok) return MOE_ERR_DEVICE;
  plan->ws = reinterpret_cast<uint8_t*>(workspace);
  plan->ws_bytes = bytes;
  if (launch_zero(plan->ws + plan->X.sync_begin, plan->X.sync_bytes, (hipStream_t)stream) != hipSuccess) {
    plan->ws = nullptr;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

size_t moe_plan_shared_pack_bytes(const moe_plan* plan) {
  if (!plan || plan->s.shared_I == 0) return 0;
  // three digit planes of the 3 Is x H values, then the values' E4M3 codes
  return (size_t)12 * (size_t)plan->s.shared_I * (size_t)plan->s.H;
}

moe_status moe_plan_set_shared(moe_plan* plan, const void* ws13, const float* ss13, const void* ws2,
                               const float* ss2, void* packed, size_t packed_bytes, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (plan->s.shared_I == 0) return MOE_ERR_INVALID_ARG;
  const void* ptrs[5] = {ws13, ss13, ws2, ss2, packed};
  for (const void* q : ptrs) {
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
    if (ptr_device(q) != plan->device) return MOE_ERR_DEVICE;
  }
  const size_t Is = (size_t)plan->s.shared_I, H = (size_t)plan->s.H;
  const size_t need = moe_plan_shared_pack_bytes(plan);
  if (packed_bytes < need) return MOE_ERR_INVALID_ARG;
  if (overlaps(packed, need, ws13, 2 * Is * H) || overlaps(packed, need, ws2, H * Is) ||
      overlaps(packed, need, ss13, 4 * (2 * Is / 128) * (H / 128)) ||
      overlaps(packed, need, ss2, 4 * (H / 128) * (Is / 128)))
    return MOE_ERR_INVALID_ARG;
  DeviceGuard guard(plan->device);
  if (!guard.ok) return MOE_ERR_DEVICE;
  if (launch_pack_shared(ws13, ws2, (int64_t)Is, (int64_t)H, packed, (hipStream_t)stream) != hipSuccess) {
    plan->ws13 = nullptr;
    return MOE_ERR_HIP;
  }
  plan->ws13 = packed;
  plan->ss13 = ss13;
  plan->ss2 = ss2;
  return MOE_OK;
}

moe_status moe_plan_set_shared_slot(moe_plan* plan, int on) {
  if (!plan || (on != 0 && on != 1)) return MOE_ERR_INVALID_ARG;
  if (on && (plan->s.top_k < 2 || plan->s.shared_I > 0)) return MOE_ERR_INVALID_ARG;
  plan->shared_slot = on;
  return MOE_OK;
}

moe_status moe_plan_set_tp_exchange(moe_plan* plan, const moe_tp_exchange* x) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (!x) {
    memset(&plan->tpx, 0, sizeof(plan->tpx));
    return MOE_OK;
  }
  if (x->tp < 1 || x->tp > MOE_TP_MAX || x->rank < 0 || x->rank >= x->tp || x->epoch == 0 || x->spin_limit <= 0)
    return MOE_ERR_INVALID_ARG;
  if (plan->s.H % 512 != 0 || plan->mid_fmt == MOE_MID_MXFP4) return MOE_ERR_UNSUPPORTED;
  auto ok = [&](const void* q, unsigned align) -> moe_status {
    if (!q || ((uintptr_t)q & (align - 1))) return MOE_ERR_INVALID_ARG;
    return ptr_device(q) == plan->device ? MOE_OK : MOE_ERR_DEVICE;
  };
  moe_status st = ok(x->inbox, 16);
  if (st == MOE_OK) st = ok(x->inbox_tags, 4);
  if (st == MOE_OK) st = ok(x->status, 4);
  for (int p = 0; st == MOE_OK && p < x->tp; ++p) {
    if (p == x->rank) continue;
    st = ok(x->push[p], 16);
    if (st == MOE_OK) st = ok(x->push_tags[p], 4);
  }
  if (st != MOE_OK) return st;
  plan->tpx = *x;
  return MOE_OK;
}

moe_status moe_plan_set_weight_layout(moe_plan* plan, unsigned layout) {
  if (!plan || (layout & ~(unsigned)(MOE_LAYOUT_W13_PACKED | MOE_LAYOUT_W2_PACKED))) return MOE_ERR_INVALID_ARG;
  plan->layout = layout;
  return MOE_OK;
}

moe_status moe_plan_set_mid_format(moe_plan* plan, int format) {
  if (!plan || (format != MOE_MID_E4M3 && format != MOE_MID_MXFP4)) return MOE_ERR_INVALID_ARG;
  if (format == MOE_MID_MXFP4 && plan->tpx.tp > 0) return MOE_ERR_UNSUPPORTED;  // exchange is for the E4M3 mid
  plan->mid_fmt = format;
  return MOE_OK;
}

moe_status moe_plan_set_stage_events(moe_plan* plan, void* const* events, int n) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (!events) {
    plan->n_events = 0;
    return MOE_OK;
  }
  if (n != 2 * kStages) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    if (!events[i]) return MOE_ERR_INVALID_ARG;
    plan->events[i] = (hipEvent_t)events[i];
  }
  plan->n_events = n;
  plan->call_start = plan->call_stop = nullptr;
  return MOE_OK;
}

moe_status moe_plan_set_call_events(moe_plan* plan, void* start, void* stop) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (!start != !stop) return MOE_ERR_INVALID_ARG;
  plan->call_start = (hipEvent_t)start;
  plan->call_stop = (hipEvent_t)stop;
  if (start) plan->n_events = 0;
  return MOE_OK;
}

moe_status moe_pack_w13(const void* w13, const void* s13, int64_t E, int64_t I, int64_t H, void* w13_packed,
                        void* s13_packed, void* stream) {
  if (!w13 || !s13 || !w13_packed || !s13_packed) return MOE_ERR_INVALID_ARG;
  if (E <= 0 || I <= 0 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 512 != 0 || I % 128 != 0 || I > 512 || E > 1024 || H > 65536) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[4] = {w13, s13, w13_packed, s13_packed};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_INVALID_ARG;
  const size_t wb = (size_t)E * 2 * I * (H / 2), sb = (size_t)E * 2 * I * (H / 32);
  if (overlaps(w13_packed, wb, w13, wb) || overlaps(w13_packed, wb, s13, sb) || overlaps(s13_packed, sb, w13, wb) ||
      overlaps(s13_packed, sb, s13, sb) || overlaps(w13_packed, wb, s13_packed, sb))
    return MOE_ERR_INVALID_ARG;
  const int dev = ptr_device(w13);
  if (dev < 0) return MOE_ERR_DEVICE;
  for (const void* q : ptrs)
    if (ptr_device(q) != dev) return MOE_ERR_DEVICE;
  DeviceGuard guard(dev);
  if (!guard.ok) return MOE_ERR_DEVICE;
  return launch_pack_w13(w13, s13, E, I, H, w13_packed, s13_packed, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

moe_status moe_pack_w2(const void* w2, const void* s2, int64_t E, int64_t I, int64_t H, void* w2_packed,
                       void* s2_packed, void* stream) {
  if (!w2 || !s2 || !w2_packed || !s2_packed) return MOE_ERR_INVALID_ARG;
  if (E <= 0 || I <= 0 || H <= 0) return MOE_ERR_INVALID_ARG;
  if (H % 512 != 0 || I % 128 != 0 || I > 512 || E > 1024 || H > 65536) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[4] = {w2, s2, w2_packed, s2_packed};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_INVALID_ARG;
  const size_t wb = (size_t)E * H * (I / 2), sb = (size_t)E * H * (I / 32), spb = (size_t)E * H * 16;
  if (overlaps(w2_packed, wb, w2, wb) || overlaps(w2_packed, wb, s2, sb) || overlaps(s2_packed, spb, w2, wb) ||
      overlaps(s2_packed, spb, s2, sb) || overlaps(w2_packed, wb, s2_packed, spb))
    return MOE_ERR_INVALID_ARG;
  const int dev = ptr_device(w2);
  if (dev < 0) return MOE_ERR_DEVICE;
  for (const void* q : ptrs)
    if (ptr_device(q) != dev) return MOE_ERR_DEVICE;
  DeviceGuard guard(dev);
  if (!guard.ok) return MOE_ERR_DEVICE;
  return launch_pack_w2(w2, s2, E, I, H, w2_packed, s2_packed, (hipStream_t)stream) == hipSuccess ? MOE_OK
                                                                                               : MOE_ERR_HIP;
}

moe_status moe_forward(moe_plan* plan, int64_t M, const void* x, const float* logits, const void* w13,
                       const void* s13, const void* w2, const void* s2, void* out, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (M < 0 || M > plan->s.M) return MOE_ERR_INVALID_ARG;
  if (!plan->ws) return MOE_ERR_WORKSPACE;
  const void* ptrs[7] = {x, logits, w13, s13, w2, s2, out};
  moe_status st = check_call(plan, M, ptrs, plan->ws, plan->L.total_bytes);
  if (st != MOE_OK || M == 0) return st;
  DeviceGuard guard(plan->device);
  if (!guard.ok) return MOE_ERR_DEVICE;
  CallArgs a{M, x, logits, w13, s13, w2, s2, out, (hipStream_t)stream};
  if (enqueue_call(plan, a) != hipSuccess) {
    // a launch after the routing may have left bits in the token bitmap that
    // only the sort clears: unbind the workspace so that no later call runs
    // on it before moe_plan_set_workspace zeroes it again
    plan->ws = nullptr;
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status moe_forward_noalloc(moe_plan* plan, int64_t M, const void* x, const float* logits, const void* w13,
                               const void* s13, const void* w2, const void* s2, void* out, void* stream) {
  if (!plan) return MOE_ERR_INVALID_ARG;
  if (M < 0 || M > plan->s.M) return MOE_ERR_INVALID_ARG;
  if (plan->L.total_bytes > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[7] = {x, logits, w13, s13, w2, s2, out};
  moe_status st = check_call(plan, M, ptrs, nullptr, 0);
  if (st != MOE_OK || M == 0) return st;
  DeviceGuard guard(plan->device);
  if (!guard.ok) return MOE_ERR_DEVICE;
  void* sp = nullptr;
  if (scratch_address(plan->device, &sp) != hipSuccess) return MOE_ERR_HIP;
  // the call runs on a copy of the plan whose workspace is this device's
  // scratch; the plan itself (and its bound workspace) is not touched
  moe_plan q = *plan;
  q.ws = reinterpret_cast<uint8_t*>(sp);
  q.ws_bytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
  CallArgs a{M, x, logits, w13, s13, w2, s2, out, (hipStream_t)stream};
  // every call on the device shares the scratch, and a call of another plan
  // leaves other data where this plan keeps its token bitmap: clear it (a
  // fill kernel, not a memset node, so the call can be captured) before the
  // routing sets its bits; the single-workgroup sort up to kSmallM tokens
  // keeps its bitmap in LDS and needs none
  hipError_t e = hipSuccess;
  if (!small_path(M, q.s.top_k)) e = launch_zero(q.ws + q.X.sync_begin, q.X.sync_bytes, a.stream);
  if (e == hipSuccess) e = enqueue_call(&q, a);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
