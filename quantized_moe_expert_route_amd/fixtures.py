"""Seeded synthetic inputs for one tensor-parallel rank's routed-MoE call.

This module holds random draws and byte packing only: it computes no step of
the MoE call (no routing, no quantization rule, no GEMM). Both the CPU oracle
and the HIP path consume the byte tensors it returns.

Workloads (shapes from "[HIP] IQ2R: GLM-5.3 packed MoE path for TP4/TP8 on
gfx950", Summary: 256 routed experts, top-k routing, hidden 6144, intermediate
512 per rank at TP4 and 256 at TP8):

  c0  tiny: H 512, E 16, top-2, I 128, M 4, logits N(0,1)
  c1  TP8 decode: H 6144, E 256, top-8, I 256, M 4, logits U[0,1)
  c2  TP8 verify: as c1 with M 16, 4 groups of 4 tokens sharing 6 of 8 experts
  c3  TP4 prefill: H 6144, E 256, top-8, I 512, M 1024, Zipf(1.1) popularity
  c4  TP4 large prefill: as c3 with M 4096, plus a block-FP8 shared expert

Weights are drawn directly as MXFP4 codes (E2M1 nibbles, low nibble = even
element, and one E8M0 byte per 32 along K). The code distribution is the one
that N(0, 0.02) weights take under per-32 MX quantization, tabulated once
offline; the table below is the only trace of that, as plain probabilities.

Every tensor has its own PCG64 stream, seeded with [seed, tensor id, expert],
so any subset of experts can be generated alone and equals the same experts of
the full tensor.
"""

from __future__ import annotations

import dataclasses
import os
from typing import Dict, Optional

import numpy as np

# Tensor ids of the independent random streams.
_T_X, _T_LOGITS, _T_W13, _T_W2, _T_SH13, _T_SH2, _T_PERM = 1, 2, 3, 4, 5, 6, 7

# E8M0 scale bytes of N(0, 0.02) blocks of 32, with their frequencies.
_SCALE_BYTES = np.array([119, 120, 121], dtype=np.uint8)
_SCALE_P = np.array([0.018, 0.927, 0.055])
# E2M1 magnitude-code frequencies (codes 0..7 = 0, .5, 1, 1.5, 2, 3, 4, 6)
# for each of the three scale bytes above.
_MAG_P = np.array([
    [0.0441, 0.0877, 0.0868, 0.0848, 0.1218, 0.1486, 0.1873, 0.2389],
    [0.0777, 0.1526, 0.1441, 0.1310, 0.1654, 0.1571, 0.1221, 0.0500],
    [0.1505, 0.2787, 0.2220, 0.1523, 0.1168, 0.0433, 0.0348, 0.0016],
])


@dataclasses.dataclass(frozen=True)
class Shape:
    """One rank's MoE shape. M tokens, hidden H, E experts, top_k, intermediate I."""

    M: int
    H: int
    E: int
    I: int
    top_k: int
    routed_scaling: float = 2.5
    shared_I: int = 0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    logits: str  # "normal" | "uniform" | "correlated" | "zipf" | "hot" | "mixed" | "spread"
    seed: int
    shared_slot: bool = False  # expert E-1 is the shared expert, the last slot of every token


WORKLOADS: Dict[str, Workload] = {
    "c0": Workload("c0", Shape(M=4, H=512, E=16, I=128, top_k=2), "normal", 0),
    "c1": Workload("c1", Shape(M=4, H=6144, E=256, I=256, top_k=8), "uniform", 1),
    "c2": Workload("c2", Shape(M=16, H=6144, E=256, I=256, top_k=8), "correlated", 2),
    "c3": Workload("c3", Shape(M=1024, H=6144, E=256, I=512, top_k=8), "zipf", 3),
    "c4": Workload("c4", Shape(M=4096, H=6144, E=256, I=512, top_k=8, shared_I=512), "zipf", 4),
}

# Mid-range batches (MTP verify at M = 4 x concurrency) on the TP8 shapes,
# with the expert-reuse patterns above; they share c1's weights (seed 1).
for _m in (32, 64, 128, 256):
    for _kind in ("hot", "mixed", "spread"):
        WORKLOADS[f"m{_m}_{_kind}"] = Workload(f"m{_m}_{_kind}", Shape(M=_m, H=6144, E=256, I=256, top_k=8), _kind, 1)

# The TP4 shape at M = 16 with hot routing (a row the pages time for their
# MXFP4 arm); it shares c3's weights (seed 3).
WORKLOADS["t4_m16_hot"] = Workload("t4_m16_hot", Shape(M=16, H=6144, E=256, I=512, top_k=8), "hot", 3)

# The TP4 shape at M = 4096 with spread and hot routing (rows the pages time
# for both weight formats; c3's weights, no shared expert).
WORKLOADS["t4_m4096_spread"] = Workload("t4_m4096_spread", Shape(M=4096, H=6144, E=256, I=512, top_k=8), "spread", 3)
WORKLOADS["t4_m4096_hot"] = Workload("t4_m4096_hot", Shape(M=4096, H=6144, E=256, I=512, top_k=8), "hot", 3)

# The pages' fused form of the shared expert: 256 routed experts plus the
# shared expert as expert 256, top-9 (TP8 shapes of c1 and c2; experts
# 0..255 are c1's / c2's, the logits are drawn for 257 columns and the last
# column is not read).
WORKLOADS["c1s"] = Workload("c1s", Shape(M=4, H=6144, E=257, I=256, top_k=9), "uniform", 1, True)
WORKLOADS["c2s"] = Workload("c2s", Shape(M=16, H=6144, E=257, I=256, top_k=9), "correlated", 2, True)

# c1 and c2 with the block-FP8 shared expert at its TP8 share (I 256 of the
# 512 it has at TP4 in c4): up to 16 tokens it runs inside the routed
# launches, as the pages' fused decode does.
WORKLOADS["c1b"] = Workload("c1b", Shape(M=4, H=6144, E=256, I=256, top_k=8, shared_I=256), "uniform", 1)
WORKLOADS["c2b"] = Workload("c2b", Shape(M=16, H=6144, E=256, I=256, top_k=8, shared_I=256), "correlated", 2)

WORKLOAD_TITLES = {
    "c0": "tiny H512 E16 top2 I128 M4",
    "c1": "TP8-rank decode H6144 E256 top8 I256 M4, MXFP4 experts, uniform logits",
    "c2": "TP8-rank verify H6144 E256 top8 I256 M16, MXFP4 experts, correlated rows",
    "c3": "TP4-rank prefill H6144 E256 top8 I512 M1024, MXFP4 experts, Zipf(1.1) routing",
    "c4": "TP4-rank large prefill H6144 E256 top8 I512 M4096 + block-FP8 shared expert I512, Zipf(1.1)",
    "t4_m16_hot": "TP4-rank batch H6144 E256 top8 I512 M16, hot routing (every token on the same 8 experts)",
    "t4_m4096_spread": "TP4-rank prefill H6144 E256 top8 I512 M4096, spread routing (token t on experts 8t..8t+7 mod 256)",
    "t4_m4096_hot": "TP4-rank prefill H6144 E256 top8 I512 M4096, hot routing (every token on the same 8 experts)",
    "c1s": "TP8-rank decode H6144 E256+1 top9 I256 M4, shared expert fused as expert 256 (slot 9), uniform logits",
    "c2s": "TP8-rank verify H6144 E256+1 top9 I256 M16, shared expert fused as expert 256 (slot 9), correlated rows",
    "c1b": "TP8-rank decode H6144 E256 top8 I256 M4 + block-FP8 shared expert I256 inside the routed launches",
    "c2b": "TP8-rank verify H6144 E256 top8 I256 M16 + block-FP8 shared expert I256 inside the routed launches",
}
for _name, _wl in WORKLOADS.items():
    if _name not in WORKLOAD_TITLES:
        WORKLOAD_TITLES[_name] = f"TP8-rank batch H6144 E256 top8 I256 M{_wl.shape.M}, {_wl.logits} routing"


def _rng(seed: int, tid: int, e: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tid, e])


def _luts() -> np.ndarray:
    """[3 * 65536] uint8: a 16-bit uniform draw -> signed E2M1 code, per scale class.

    Bit 0 of the draw is the sign, bits 1..15 pick the magnitude by inverse CDF.
    """
    out = np.empty((3, 65536), dtype=np.uint8)
    r = np.arange(65536)
    u = (r >> 1) / 32768.0
    sign = (r & 1).astype(np.uint8) << 3
    for c in range(3):
        cdf = np.cumsum(_MAG_P[c])
        cdf[-1] = 1.0 + 1e-9
        mag = np.searchsorted(cdf, u, side="right").astype(np.uint8)
        out[c] = mag | sign
    return out.reshape(-1)


_LUT = _luts()


def mxfp4_rows(seed: int, tid: int, e: int, rows: int, K: int):
    """MXFP4 weight rows for expert e: (values [rows, K/2] u8, scales [rows, K/32] u8)."""
    assert K % 32 == 0
    rng = _rng(seed, tid, e)
    nb = K // 32
    cls = np.searchsorted(np.cumsum(_SCALE_P), rng.random((rows, nb)), side="right")
    cls = np.minimum(cls, 2).astype(np.int64)
    scales = _SCALE_BYTES[cls]
    draw = rng.integers(0, 65536, size=(rows, K), dtype=np.uint16)
    idx = (np.repeat(cls, 32, axis=1) << 16) | draw
    codes = _LUT[idx]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) through torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def make_x(shape: Shape, seed: int) -> np.ndarray:
    """x [M, H] as bf16 bits: N(0, 1) samples cast to bf16."""
    a = _rng(seed, _T_X).standard_normal((shape.M, shape.H), dtype=np.float32)
    return bf16_bits_from_f32(a)


def make_logits(shape: Shape, kind: str, seed: int) -> np.ndarray:
    """Router logits [M, E] fp32 of the given kind."""
    M, E, k = shape.M, shape.E, shape.top_k
    rng = _rng(seed, _T_LOGITS)
    if kind == "normal":
        return rng.standard_normal((M, E), dtype=np.float32)
    if kind == "uniform":
        return rng.random((M, E), dtype=np.float32)
    if kind == "correlated":
        # Groups of 4 consecutive tokens share 6 experts; each token adds 2 of
        # its own. The 8 chosen get +2.0 so they are exactly the top 8.
        assert k == 8
        out = rng.random((M, E), dtype=np.float32)
        for g0 in range(0, M, 4):
            shared = rng.choice(E, 6, replace=False)
            rest = np.setdiff1d(np.arange(E), shared)
            for t in range(g0, min(g0 + 4, M)):
                own = rng.choice(rest, 2, replace=False)
                out[t, shared] += np.float32(2.0)
                out[t, own] += np.float32(2.0)
        return out
    if kind == "zipf":
        # Zipf(1.1) popularity over experts, a seeded rank -> expert
        # permutation, and Gumbel noise: top-k of log p + Gumbel samples k
        # distinct experts with probability proportional to p.
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
        p /= p.sum()
        perm = _rng(seed, _T_PERM).permutation(E)
        pe = np.empty(E)
        pe[perm] = p
        g = rng.gumbel(size=(M, E))
        return (np.log(pe)[None, :] + g).astype(np.float32)
    if kind in ("hot", "spread", "mixed"):
        # Expert-reuse patterns of the mid-range batches (the pages name hot /
        # spread / mixed routing without defining them; these are our
        # readings): hot = every token picks the same k experts (fewest
        # active, most rows each); spread = token t picks experts
        # perm[(k t + j) mod E], so the batch covers as many experts as it
        # can; mixed = the first half hot, the second half spread. The chosen
        # k get +2.0 on U[0,1) logits, so they are exactly the top k.
        out = rng.random((M, E), dtype=np.float32)
        perm = _rng(seed, _T_PERM).permutation(E)
        hot = perm[:k]
        for t in range(M):
            if kind == "hot" or (kind == "mixed" and t < M // 2):
                chosen = hot
            else:
                chosen = perm[(k * t + np.arange(k)) % E]
            out[t, chosen] += np.float32(2.0)
        return out
    if kind == "ties":
        # Few distinct values, both zeros: stresses the lower-index tie rule.
        vals = np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 1.0], dtype=np.float32)
        return vals[rng.integers(0, len(vals), size=(M, E))]
    raise ValueError(kind)


def make_expert_weights(shape: Shape, seed: int, e: int):
    """Expert e's (w13 [2I, H/2], s13 [2I, H/32], w2 [H, I/2], s2 [H, I/32]), all u8.

    w13 rows [0, I) are the gate projection and rows [I, 2I) the up projection.
    """
    w13, s13 = mxfp4_rows(seed, _T_W13, e, 2 * shape.I, shape.H)
    w2, s2 = mxfp4_rows(seed, _T_W2, e, shape.H, shape.I)
    return w13, s13, w2, s2


def make_weights(shape: Shape, seed: int, experts: Optional[np.ndarray] = None):
    """Full expert stacks; experts outside `experts` (if given) stay zero."""
    E, H, I = shape.E, shape.H, shape.I
    w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
    s13 = np.zeros((E, 2 * I, H // 32), np.uint8)
    w2 = np.zeros((E, H, I // 2), np.uint8)
    s2 = np.zeros((E, H, I // 32), np.uint8)
    def one(e):
        w13[e], s13[e], w2[e], s2[e] = make_expert_weights(shape, seed, int(e))

    todo = list(range(E) if experts is None else experts)
    if len(todo) > 8:
        import concurrent.futures as cf

        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(one, todo))
    else:
        for e in todo:
            one(e)
    return w13, s13, w2, s2


def make_shared(shape: Shape, seed: int):
    """Block-FP8 shared expert: E4M3 bytes with one fp32 scale per 128x128 block.

    ws13 [2*Is, H] (rows [0, Is) gate, [Is, 2*Is) up), ss13 [2*Is/128, H/128];
    ws2 [H, Is], ss2 [H/128, Is/128]. Values: N(0, 112) samples cast to E4M3 by
    torch (saturated to +-448 first), scales 0.08/448 * (1 + U[0, .25)).
    """
    import torch

    Is, H = shape.shared_I, shape.H
    assert Is > 0 and Is % 128 == 0 and H % 128 == 0

    def codes(tid, rows, cols):
        a = _rng(seed, tid).standard_normal((rows, cols), dtype=np.float32) * np.float32(112.0)
        a = np.clip(a, -448.0, 448.0)
        t = torch.from_numpy(a).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy().copy()

    def scales(tid, rows, cols):
        u = _rng(seed, tid, 1).random((rows, cols), dtype=np.float32)
        return (np.float32(0.08 / 448.0) * (np.float32(1.0) + np.float32(0.25) * u)).astype(np.float32)

    ws13 = codes(_T_SH13, 2 * Is, H)
    ss13 = scales(_T_SH13, 2 * Is // 128, H // 128)
    ws2 = codes(_T_SH2, H, Is)
    ss2 = scales(_T_SH2, H // 128, Is // 128)
    return ws13, ss13, ws2, ss2


def make_extreme_inputs(shape: Shape, seed: int):
    """Inputs whose scale bytes reach both ends of the E8M0 range, for the
    edge cases of the formats (scale byte 0, whose power 2^-127 lies below
    binary32's normal range; bf16 subnormal x; widened weights below bf16's
    normal range; magnitudes near 2^+-100).

    Token t belongs to group g = t % 4 and is routed to experts 2g and 2g + 1
    only (those two logits get +2.0 on U[0, 1) draws), so each expert sees
    tokens of one magnitude. Starting from make_inputs' draws (weight scale
    bytes 119..121), per group:
      g0  x ~ N(0, 1)                     w13 bytes as drawn   w2 bytes as drawn
      g1  x * 2^-100                      w13 bytes + 100      w2 bytes - 119 (0..2)
      g2  x * 2^100                       w13 bytes - 100      w2 bytes + 110 (229..231)
      g3  x * 0.3 * 2^-126 in even blocks
          of 32 (some bf16 subnormals),
          x * 2^-124 in odd blocks        w13 bytes + 128      w2 bytes - 60
    Needs E >= 8, top_k == 2 and H a multiple of 64.
    """
    assert shape.E >= 8 and shape.top_k == 2 and shape.H % 64 == 0 and shape.shared_I == 0
    M, H, E = shape.M, shape.H, shape.E
    d = make_inputs(shape, "uniform", seed)
    grp = np.arange(M) % 4
    lg = d["logits"]
    lg[np.arange(M), 2 * grp] += np.float32(2.0)
    lg[np.arange(M), 2 * grp + 1] += np.float32(2.0)
    a = _rng(seed, _T_X).standard_normal((M, H), dtype=np.float32).astype(np.float64)
    even = (np.arange(H) // 32) % 2 == 0
    factor = np.ones((M, H))
    factor[grp == 1] = 2.0 ** -100
    factor[grp == 2] = 2.0 ** 100
    factor[np.ix_(grp == 3, even)] = 0.3 * 2.0 ** -126
    factor[np.ix_(grp == 3, ~even)] = 2.0 ** -124
    d["x"] = bf16_bits_from_f32((a * factor).astype(np.float32))
    for g, d13, d2 in ((1, 100, -119), (2, -100, 110), (3, 128, -60)):
        for e in (2 * g, 2 * g + 1):
            d["s13"][e] = (d["s13"][e].astype(np.int64) + d13).astype(np.uint8)
            d["s2"][e] = (d["s2"][e].astype(np.int64) + d2).astype(np.uint8)
    return d


def make_inputs(name_or_shape, logits: Optional[str] = None, seed: Optional[int] = None,
                experts: Optional[np.ndarray] = None, with_weights: bool = True, shared_slot: bool = False):
    """All inputs of one call as numpy arrays.

    `name_or_shape` is a workload name ("c0".."c4") or a Shape (then `logits`
    and `seed` are required). Returns a dict with shape, x (bf16 bits), logits,
    w13, s13, w2, s2 and, when shape.shared_I > 0, the shared expert tensors.
    """
    slot = shared_slot
    if isinstance(name_or_shape, str):
        wl = WORKLOADS[name_or_shape]
        shape, kind, sd = wl.shape, wl.logits, wl.seed
        slot = slot or wl.shared_slot
        if logits is not None:
            kind = logits
        if seed is not None:
            sd = seed
    else:
        shape, kind, sd = name_or_shape, logits, seed
        assert kind is not None and sd is not None
    if slot:
        # the routed experts' logits as for E-1 experts and k-1 slots, then the
        # shared expert's column (never read)
        routed = dataclasses.replace(shape, E=shape.E - 1, top_k=shape.top_k - 1)
        lg = np.concatenate([make_logits(routed, kind, sd), np.zeros((shape.M, 1), np.float32)], axis=1)
    else:
        lg = make_logits(shape, kind, sd)
    d = {"shape": shape, "seed": sd, "x": make_x(shape, sd), "logits": lg}
    if with_weights:
        d["w13"], d["s13"], d["w2"], d["s2"] = make_weights(shape, sd, experts)
    if shape.shared_I > 0:
        d["ws13"], d["ss13"], d["ws2"], d["ss2"] = make_shared(shape, sd)
    return d
