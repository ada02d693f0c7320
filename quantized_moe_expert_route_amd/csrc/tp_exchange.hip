// Tensor-parallel partial-sum exchange, the epilogue of a call whose plan has
// an exchange set ("glm53: FP8 mid hand-off, early split rows, per-row
// up/gate jobs, ...", Accuracy Tests: the peers' partial sums arrive tagged
// with the launch's epoch; pushes from a rank run alone go to scratch sinks).
//
// The combine has left the rank's float64 partial in its inbox slot. A
// workgroup per (token, 512-column chunk): it sends the chunk to every peer
// (then makes it visible system-wide before the chunk's tag, the epoch),
// waits for every peer's chunk tag to show the epoch (a bounded poll: a wait
// that gives up sets the status word and the chunk is summed as it stands,
// so the launch always ends), adds the tp partials in float64 in rank order
// and rounds once to bf16. Every rank adds the same values in the same order
// and forms the same bits.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace qmoe {

constexpr int kTpChunk = 512;  // columns a tag covers; 256 threads x 2

struct TpArgs {
  int tp, rank, spin_limit;
  uint32_t epoch;
  const double* inbox;
  const uint32_t* inbox_tags;
  double* push[MOE_TP_MAX];
  uint32_t* push_tags[MOE_TP_MAX];
  uint32_t* status;
  size_t slot;  // doubles per inbox slot: M_max * H
  size_t tag_slot;  // tags per slot: M_max * H / 512
};

// A float64 read that goes to the coherence point (the value a peer wrote
// arrives by another path than this CU's caches).
__device__ __forceinline__ double load_sys(const double* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return __longlong_as_double((long long)v);
}

__global__ __launch_bounds__(256) void tp_exchange_kernel(TpArgs a, int H, uint16_t* __restrict__ out) {
  const int chunks = H / kTpChunk;
  const int t = blockIdx.x / chunks, ch = blockIdx.x - t * chunks;
  const size_t off = (size_t)t * H + (size_t)ch * kTpChunk + 2 * threadIdx.x;
  const size_t toff = (size_t)t * chunks + ch;
  const double2 own = *reinterpret_cast<const double2*>(a.inbox + (size_t)a.rank * a.slot + off);
  // push: the chunk to every peer, visible system-wide before its tag
  for (int p = 0; p < a.tp; ++p)
    if (p != a.rank) *reinterpret_cast<double2*>(a.push[p] + off) = own;
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0)
    for (int p = 0; p < a.tp; ++p)
      if (p != a.rank) __hip_atomic_store(a.push_tags[p] + toff, a.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  // wait: every peer's tag of this chunk shows the epoch
  if (threadIdx.x == 0) {
    bool ok = true;
    for (int p = 0; p < a.tp; ++p) {
      if (p == a.rank) continue;
      const uint32_t* tag = a.inbox_tags + (size_t)p * a.tag_slot + toff;
      for (int n = 0; __hip_atomic_load(tag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) != a.epoch; ++n) {
        if (n + 1 >= a.spin_limit) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    if (!ok) atomicOr(a.status, 1u);
  }
  __syncthreads();
  // the sum in rank order, from zero, one bf16 rounding
  double s0 = 0.0, s1 = 0.0;
  for (int r = 0; r < a.tp; ++r) {
    double v0 = own.x, v1 = own.y;
    if (r != a.rank) {
      v0 = load_sys(a.inbox + (size_t)r * a.slot + off);
      v1 = load_sys(a.inbox + (size_t)r * a.slot + off + 1);
    }
    s0 += v0;
    s1 += v1;
  }
  *reinterpret_cast<uint32_t*>(out + off) = bf16_rne_from_double(s0) | (bf16_rne_from_double(s1) << 16);
}

hipError_t launch_tp_exchange(const moe_plan* p, const CallArgs& a, Ev ev) {
  const moe_tp_exchange& x = p->tpx;
  TpArgs t;
  t.tp = x.tp;
  t.rank = x.rank;
  t.spin_limit = x.spin_limit;
  t.epoch = x.epoch;
  t.inbox = x.inbox;
  t.inbox_tags = x.inbox_tags;
  for (int i = 0; i < MOE_TP_MAX; ++i) {
    t.push[i] = x.push[i];
    t.push_tags[i] = x.push_tags[i];
  }
  t.status = x.status;
  t.slot = (size_t)p->s.M * (size_t)p->s.H;
  t.tag_slot = (size_t)p->s.M * (size_t)(p->s.H / kTpChunk);
  const int64_t blocks = a.M * (p->s.H / kTpChunk);
  return launch_k(tp_exchange_kernel, dim3((unsigned)blocks), dim3(256), 0, a.stream, ev, t, (int)p->s.H,
                  reinterpret_cast<uint16_t*>(a.out));
}

}  // namespace qmoe
