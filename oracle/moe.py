"""CPU oracle of one tensor-parallel rank's routed-MoE call (plain numpy, float64).

TEST INFRASTRUCTURE ONLY (see the package header).

What the call computes, in the pages' order:

1. route: top-k experts per token from fp32 router logits ("glm53: FP8 mid
   hand-off ...", Modifications table row "per-row up/gate jobs" and its
   commit: top-8 by rounds, a tie broken by expert ID). The scoring function
   is not stated on the pages; the reading taken is sigmoid scores of the
   selected logits, renormalized over the k slots and multiplied by the routed
   scaling factor (the GLM/DeepSeek-V3 convention).
2. align: entries (token t, slot j) grouped by expert, tokens ascending inside
   an expert, so each expert's weights are read once for all its rows
   ("glm53_flash: Score a verify request's index tiles once ...", commit "Run
   verify steps of up to 16 rows": expert-major MoE above 8 rows).
3. x -> MXFP4 once per token (the pages' A4W4 arm, "IQ2R: load GLM-5.3 packed
   MoE checkpoints ...", status comments; "paired conversion in the frontend").
4. gate/up: g = x.w_gate, u = x.w_up, exact sums rounded once to fp32;
   h = fl32(SiLU(g) * u) ("IQ2R: load GLM-5.3 ...", Summary: SiLU activation).
5. mid: each 128-element block of a (token, slot) row quantized once to E4M3
   with an fp32 scale ("glm53: FP8 mid hand-off ...", row "mid as FP8 once").
6. down: y[t, j] = sum over mid blocks b of s_b * (q_b . w2_b); each block
   sum exact, the scales applied in float64, one rounding to fp32.
5'/6'. the MXFP4 comparison arm (mid_format "mxfp4"): mid quantized per 32
   with the rule of step 3, down as one exact sum of MXFP4 x MXFP4 products.
7. combine: out[t] = bf16(sum_j w[t, j] * y[t, j] (+ shared[t])), one
   rounding to bf16.
8. shared expert (block-FP8, 128x128 weight scales; "IQ2R: load GLM-5.3 ...",
   Summary: shared experts keep block-FP8): x -> E4M3 per token per 128 along
   H, gate/up and down on FP8 with the block scales, added before step 7's
   rounding with weight 1.

Exactness: every product in the two GEMMs is a product of two short-mantissa
values (E2M1 x E2M1, E4M3 x E2M1, E4M3 x E4M3) with power-of-two scales, so
float64 block sums are exact when their span fits 53 bits; `_exact_matmul`
asserts that bound on every call.

Parity pins (tests/test_oracle_moe.py): brute-force routing and sorting on
small inputs, closed-form routing weights, GEMMs on the FP4/FP8 grids with
unit scales against plain matmul, a dense evaluation of every expert masked
by the routing, and the invariants (weights sum to the scaling factor; zero
output with no active expert; token-permutation and expert-relabelling
equivariance; scaling linearity).
"""

from __future__ import annotations

import numpy as np

from . import formats as F

SCORE_EPS = np.float32(1e-20)


# ------------------------------------------------------------------ helpers
def _quantum(v: np.ndarray) -> float:
    """Largest power of two dividing every nonzero |v| (1.0 if all zero)."""
    nz = np.abs(v[v != 0])
    if nz.size == 0:
        return 1.0
    m, e = np.frexp(nz)
    mi = np.ldexp(m, 53).astype(np.int64)
    low = mi & -mi
    tz = np.round(np.log2(low.astype(np.float64))).astype(np.int64)
    return float(np.ldexp(1.0, int((e - 53 + tz).min())))


def _exact_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a [m, K] @ b [n, K]^T in float64, asserting that every partial sum is
    exact (all terms are multiples of qa*qb and the magnitude stays < 2^53
    of them), so the result does not depend on the summation order."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0 or b.size == 0:
        return np.zeros((a.shape[0], b.shape[0]))
    bound = (np.abs(a) @ np.abs(b).T).max(initial=0.0)
    q = _quantum(a) * _quantum(b)
    assert bound == 0.0 or bound / q < 2.0 ** 52, "float64 sum would not be exact"
    return a @ b.T


def _silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(-g))


# ------------------------------------------------------------------ 1. route
def route(logits: np.ndarray, k: int, scaling: float):
    """Top-k by (logit descending, expert ascending); weights from sigmoid scores.

    Returns ids [M, k] int32 and w [M, k] float32:
      sigma_j = fl32(1 / (1 + exp(-l_j)))  (float64, rounded once)
      S = fl32 sum of sigma_j in slot order
      w_j = fl32(fl32(sigma_j / (S + 1e-20)) * scaling)
    """
    logits = np.asarray(logits, np.float32)
    M, E = logits.shape
    assert 1 <= k <= E
    assert np.all(np.isfinite(logits) | np.isneginf(logits)), "logits must be finite or -inf"
    ids = np.zeros((M, k), np.int32)
    w = np.zeros((M, k), np.float32)
    experts = np.arange(E)
    for t in range(M):
        l = logits[t].astype(np.float64)
        # numeric keys: -0.0 and +0.0 compare equal, so they tie
        order = np.lexsort((experts, -l))
        sel = order[:k]
        ids[t] = sel
        sig = (1.0 / (1.0 + np.exp(-l[sel]))).astype(np.float32)
        S = np.float32(0.0)
        for j in range(k):
            S = np.float32(S + sig[j])
        den = np.float32(S + SCORE_EPS)
        for j in range(k):
            w[t, j] = np.float32(np.float32(sig[j] / den) * np.float32(scaling))
    return ids, w


def route_shared_slot(logits: np.ndarray, k: int, scaling: float):
    """Routing with the shared expert fused as the last expert and the last
    slot ("[HIP] IQ2R: GLM-5.3 packed MoE path for TP4/TP8 on gfx950",
    Summary: 256 routed experts plus the shared expert as expert 256, top-9).
    Reading: slots 0..k-2 are the top-(k-1) of the first E-1 logits with the
    weights of `route` over those k-1 slots; slot k-1 is expert E-1 with
    weight 1 (the shared expert's output is added unscaled). The last logits
    column is not read."""
    logits = np.asarray(logits, np.float32)
    M, E = logits.shape
    assert k >= 2 and E >= 2
    ids_r, w_r = route(logits[:, :E - 1], k - 1, scaling)
    ids = np.concatenate([ids_r, np.full((M, 1), E - 1, np.int32)], axis=1)
    w = np.concatenate([w_r, np.ones((M, 1), np.float32)], axis=1)
    return ids, w


# ------------------------------------------------------------------ 2. align
def align(ids: np.ndarray, E: int):
    """Stable grouping of the M*k entries (entry = t*k + j) by expert.

    Returns count [E], offset [E+1] (exclusive prefix, offset[E] = M*k) and
    sorted_entry [M*k] (entries of expert e at offset[e]..offset[e+1], t
    ascending).
    """
    flat = np.asarray(ids).reshape(-1)
    count = np.bincount(flat, minlength=E).astype(np.int32)
    offset = np.zeros(E + 1, np.int32)
    offset[1:] = np.cumsum(count)
    sorted_entry = np.argsort(flat, kind="stable").astype(np.int32)
    return count, offset, sorted_entry


# ------------------------------------------------------------------ 3. x -> MXFP4
def quantize_x(x_bits: np.ndarray):
    """bf16 x [M, H] -> (E2M1 codes [M, H], E8M0 scale codes [M, H/32])."""
    return F.mx_fp4_quantize(F.bf16_decode(x_bits), 32)


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return F.mx_fp4_decode(F.unpack_fp4(packed), scales, 32)


# ------------------------------------------------------------------ 4. gate/up
def gate_up(xd: np.ndarray, w13d: np.ndarray, I: int) -> np.ndarray:
    """xd [r, H] and w13d [2I, H] dequantized; returns h [r, I] float32."""
    gu = _exact_matmul(xd, w13d).astype(np.float32)
    g, u = gu[:, :I], gu[:, I:]
    return (_silu(g.astype(np.float64)) * u.astype(np.float64)).astype(np.float32)


# ------------------------------------------------------------------ 5. mid quant
def quantize_mid(h: np.ndarray):
    """h [r, I] float32 -> (E4M3 codes [r, I], fp32 scales [r, I/128])."""
    return F.fp8_block_quantize(h, 128)


# ------------------------------------------------------------------ 6. down
def down(q: np.ndarray, s: np.ndarray, w2d: np.ndarray) -> np.ndarray:
    """q [r, I] E4M3 codes, s [r, I/128] fp32 scales, w2d [H, I] dequantized.

    y = fl32(sum_b s_b * S_b), S_b = exact sum of the block's products.
    """
    qd = F.e4m3_decode(q)
    r, I = qd.shape
    acc = np.zeros((r, w2d.shape[0]))
    for b in range(I // 128):
        Sb = _exact_matmul(qd[:, 128 * b:128 * (b + 1)], w2d[:, 128 * b:128 * (b + 1)])
        acc += np.asarray(s[:, b], np.float64)[:, None] * Sb
    return acc.astype(np.float32)


# ------------------------------------------------------------------ 5'/6'. MXFP4 mid
# The comparison arm the pages time against IQ2R is stock MXFP4: experts
# quantized online to MXFP4 ("IQ2R: load GLM-5.3 packed MoE checkpoints ...",
# Results (MXFP4 vs IQ2R)). Reading: its activations are MXFP4 in both GEMMs,
# so mid takes the rule of step 3 (per 32, E8M0 scale, E2M1 codes) in place of
# step 5, and down multiplies two MXFP4 operands.
def quantize_mid_mx(h: np.ndarray):
    """h [r, I] float32 -> (E2M1 codes [r, I], E8M0 scale codes [r, I/32])."""
    return F.mx_fp4_quantize(h, 32)


def down_mx(q: np.ndarray, s: np.ndarray, w2d: np.ndarray) -> np.ndarray:
    """q [r, I] E2M1 codes, s [r, I/32] E8M0 codes, w2d [H, I] dequantized.

    y = fl32(exact sum over I of mid * w2): every term is a product of two
    E2M1 values times a power of two.
    """
    return _exact_matmul(F.mx_fp4_decode(q, s, 32), w2d).astype(np.float32)


# ------------------------------------------------------------------ 8. shared expert
def _block_fp8_linear(aq, as_, wq, ws) -> np.ndarray:
    """a [r, K] E4M3 codes with fp32 scales per 128 along K; w [n, K] E4M3 codes
    with fp32 scales per 128x128 block. Returns fl32(sum over K blocks of
    a_scale * w_scale * exact block sum)."""
    ad = F.e4m3_decode(aq)
    wd = F.e4m3_decode(wq)
    r, K = ad.shape
    n = wd.shape[0]
    acc = np.zeros((r, n))
    for kb in range(K // 128):
        S = _exact_matmul(ad[:, 128 * kb:128 * (kb + 1)], wd[:, 128 * kb:128 * (kb + 1)])
        wsc = np.repeat(np.asarray(ws[:, kb], np.float64), 128)[:n]  # per output row
        acc += (np.asarray(as_[:, kb], np.float64)[:, None] * wsc[None, :]) * S
    return acc.astype(np.float32)


def shared_expert(x_bits, ws13, ss13, ws2, ss2):
    """Block-FP8 shared expert; returns (y_s [M, H] fp32, intermediates)."""
    Is = ws13.shape[0] // 2
    xf = F.bf16_decode(x_bits).astype(np.float32)
    xq8, xs8 = F.fp8_block_quantize(xf, 128)
    gu = _block_fp8_linear(xq8, xs8, ws13, ss13)
    g, u = gu[:, :Is], gu[:, Is:]
    h = (_silu(g.astype(np.float64)) * u.astype(np.float64)).astype(np.float32)
    hq, hs = F.fp8_block_quantize(h, 128)
    y = _block_fp8_linear(hq, hs, ws2, ss2)
    return y, {"xq8": xq8, "xs8": xs8, "h": h, "hq": hq, "hs": hs}


# ------------------------------------------------------------------ 7. combine
def combine_partial(w: np.ndarray, y: np.ndarray, ys=None) -> np.ndarray:
    """The combine's float64 sum before its rounding: w [M, k] fp32, y [M, k, H]
    fp32 (+ ys [M, H]) -> [M, H] float64, products of two fp32 values (exact)
    added in slot order, then ys."""
    acc = np.zeros((y.shape[0], y.shape[2]))
    for j in range(y.shape[1]):
        acc += np.asarray(w[:, j], np.float64)[:, None] * y[:, j, :].astype(np.float64)
    if ys is not None:
        acc += np.asarray(ys, np.float64)
    return acc


def combine(w: np.ndarray, y: np.ndarray, ys=None) -> np.ndarray:
    """w [M, k] fp32, y [M, k, H] fp32 (+ ys [M, H]) -> out bf16 bits [M, H].

    Float64 sum in slot order (products of two fp32 values are exact), then
    one rounding to bf16.
    """
    return F.bf16_encode(combine_partial(w, y, ys))


def tp_exchange_sum(partials) -> np.ndarray:
    """Tensor-parallel partial-sum exchange ("glm53: FP8 mid hand-off, early
    split rows, ...", Accuracy Tests: a rank's peers' partial sums arrive
    tagged with the launch's epoch). Reading: every rank's float64 partial
    (combine_partial of its slice) is exchanged whole, the partials are added
    in float64 in rank order 0, 1, ... starting from zero, and the sum is
    rounded once to bf16, so every rank forms the same output bits.
    partials: sequence of [M, H] float64 -> out bf16 bits [M, H]."""
    acc = np.zeros(np.asarray(partials[0]).shape)
    for p in partials:
        acc = acc + np.asarray(p, np.float64)
    return F.bf16_encode(acc)


# ------------------------------------------------------------------ whole call
def _mid_steps(mid_format: str):
    """(quantize, down) of the mid hand-off: "e4m3" (steps 5, 6) or "mxfp4"."""
    if mid_format == "e4m3":
        return quantize_mid, down
    if mid_format == "mxfp4":
        return quantize_mid_mx, down_mx
    raise ValueError(mid_format)


def moe_forward(x_bits, logits, w13, s13, w2, s2, top_k, scaling, shared=None, mid_format="e4m3",
                shared_slot=False):
    """The routed-MoE call on all M tokens.

    x_bits [M, H] bf16 bits; logits [M, E] fp32; w13 [E, 2I, H/2] u8 and s13
    [E, 2I, H/32] u8 (MXFP4, rows [0, I) gate, [I, 2I) up); w2 [E, H, I/2]
    and s2 [E, H, I/32] (MXFP4 along I); shared = (ws13, ss13, ws2, ss2) or
    None. Returns a dict of every intermediate; rows of h / midq / mids are in
    sorted (expert-major) order, y is indexed by entry t*k + j. midq holds
    one code per element (E4M3, or E2M1 with mid_format "mxfp4"), mids the
    fp32 scales per 128 (or the E8M0 scale codes per 32). With shared_slot,
    expert E-1 is the shared expert, routed by `route_shared_slot`.
    """
    qmid, dmid = _mid_steps(mid_format)
    x_bits = np.asarray(x_bits, np.uint16)
    M, H = x_bits.shape
    E = logits.shape[1]
    I = w13.shape[1] // 2
    k = top_k
    ids, w = (route_shared_slot if shared_slot else route)(logits, k, scaling)
    count, offset, sorted_entry = align(ids, E)
    xq, xs = quantize_x(x_bits)
    xd = F.mx_fp4_decode(xq, xs, 32)
    n = M * k
    h = np.zeros((n, I), np.float32)
    midq = np.zeros((n, I), np.uint8)
    mids = (np.zeros((n, I // 128), np.float32) if mid_format == "e4m3"
            else np.zeros((n, I // 32), np.uint8))
    y = np.zeros((n, H), np.float32)
    for e in range(E):
        lo, hi = offset[e], offset[e + 1]
        if hi == lo:
            continue
        entries = sorted_entry[lo:hi]
        toks = entries // k
        he = gate_up(xd[toks], dequant_mxfp4(w13[e], s13[e]), I)
        qe, se = qmid(he)
        h[lo:hi], midq[lo:hi], mids[lo:hi] = he, qe, se
        y[entries] = dmid(qe, se, dequant_mxfp4(w2[e], s2[e]))
    ys, sh = (None, None)
    if shared is not None:
        ys, sh = shared_expert(x_bits, *shared)
    out = combine(w, y.reshape(M, k, H), ys)
    return {"ids": ids, "w": w, "count": count, "offset": offset,
            "sorted_entry": sorted_entry, "xq": xq, "xs": xs, "h": h,
            "midq": midq, "mids": mids, "y": y, "ys": ys, "shared": sh,
            "out": out}


def expert_dense(xd: np.ndarray, w13e, s13e, w2e, s2e, I: int, mid_format="e4m3") -> np.ndarray:
    """One expert applied to every row of xd (steps 4-6): [r, H] -> [r, H] fp32."""
    qmid, dmid = _mid_steps(mid_format)
    h = gate_up(xd, dequant_mxfp4(w13e, s13e), I)
    q, s = qmid(h)
    return dmid(q, s, dequant_mxfp4(w2e, s2e))


def moe_dense(x_bits, logits, w13, s13, w2, s2, top_k, scaling, shared=None, mid_format="e4m3",
              shared_slot=False):
    """Brute force: every expert on every token, then masked by the routing.

    Shares the per-expert arithmetic with moe_forward but none of its
    grouping: a check on the routing, the sort and the gather/scatter.
    """
    M, H = x_bits.shape
    E = logits.shape[1]
    I = w13.shape[1] // 2
    ids, w = (route_shared_slot if shared_slot else route)(logits, top_k, scaling)
    xq, xs = quantize_x(x_bits)
    xd = F.mx_fp4_decode(xq, xs, 32)
    all_y = np.stack([expert_dense(xd, w13[e], s13[e], w2[e], s2[e], I, mid_format) for e in range(E)])
    y = np.zeros((M, top_k, H), np.float32)
    for t in range(M):
        for j in range(top_k):
            y[t, j] = all_y[ids[t, j], t]
    ys = shared_expert(x_bits, *shared)[0] if shared is not None else None
    return combine(w, y, ys)
