// Per-token routing and the MXFP4 quantization of one 32-element block of x,
// shared by the routing launches (route_align.hip) and the gate/up launch
// that routes for itself (gate_up.hip).
//
// Routing: "glm53: FP8 mid hand-off, early split rows, per-row up/gate jobs,
// ..." (Modifications table, row "per-row up/gate jobs"): top-k by rounds,
// each round a wave maximum, a tie going to the lower expert ID; weights are
// the sigmoid scores renormalised over the k slots times the routed scaling.
// x -> MXFP4 (OCP MX: E8M0 scale floor(log2 amax) - 2 per 32 elements, E2M1
// nearest-even codes) once per token, the activations' frontend conversion
// of "IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing" (status
// comments).
#pragma once

#include "common.h"

namespace qmoe {

// Top-k of one logits row by one wave. Lane j < k receives slot j's expert
// and logit.
// Keys of one logits row: lane l holds experts l + 64c; every real key is > 0.
// The loads are unconditional (lanes past E read the row's last logit) so
// that all of them are in flight together: each one under its own branch
// waited for the one before it, one memory round trip per 64 experts.
template <int EC>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int E, int lane, uint32_t (&key)[EC]) {
  float v[EC];
#pragma unroll
  for (int c = 0; c < EC; ++c) v[c] = row[max(min(lane + 64 * c, E - 1), 0)];
#pragma unroll
  for (int c = 0; c < EC; ++c) key[c] = lane + 64 * c < E ? order_key(v[c]) : 0u;
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
__device__ __forceinline__ void route_keys(uint32_t (&key)[EC], int E, int k, float scaling, int shared_slot,
                                           int lane, uint32_t& sel_e, float& w) {
  const int kr = k - shared_slot;
  float sel_l = 0.f;
  topk_wave<EC>(key, kr, lane, sel_e, sel_l);
  w = route_weight(sel_l, kr, lane, scaling);
  if (shared_slot && lane == k - 1) {
    sel_e = (uint32_t)(E - 1);
    w = 1.0f;
  }
}

template <int EC>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, float scaling,
                                            int shared_slot, int lane, uint32_t& sel_e, float& w) {
  uint32_t key[EC];
  load_keys<EC>(row, E - shared_slot, lane, key);
  route_keys<EC>(key, E, k, scaling, shared_slot, lane, sel_e, w);
}

// One 32-element block of a bf16 row (as 16 words of two elements, the
// lower first) -> 16 bytes of E2M1 + an E8M0 byte.
__device__ __forceinline__ void quant_block_mx_words(const uint32_t (&w32)[16], uint8_t* __restrict__ dq,
                                                     uint8_t* __restrict__ ds) {
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
    packed[i >> 2] |= e2m1_pack2(f0, f1) << (8 * (i & 3));
  }
  *reinterpret_cast<uint4*>(dq) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  *ds = (uint8_t)sc;
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
  quant_block_mx_words(w32, dq, ds);
}

}  // namespace qmoe
