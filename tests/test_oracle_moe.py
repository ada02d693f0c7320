"""Pins of the MoE oracle: brute force, closed forms, library special cases,
a dense masked evaluation, invariants and the page-printed block arithmetic."""

import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as O
from quantized_moe_expert_route_amd import fixtures as X

HERE = os.path.dirname(os.path.abspath(__file__))


def _brute_topk(l, k):
    """Repeatedly take the largest remaining logit, lowest index on ties."""
    l = [float(v) for v in l]
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(l):
            if e in taken:
                continue
            if best is None or v > l[best]:
                best = e
        taken.append(best)
    return taken


@pytest.mark.parametrize("kind", ["normal", "uniform", "ties", "correlated", "zipf"])
def test_route_ids_brute_force(kind):
    shape = X.Shape(M=24, H=512, E=64 if kind != "correlated" else 64, I=128, top_k=8)
    logits = X.make_logits(shape, kind, 11)
    ids, w = O.route(logits, 8, 2.5)
    for t in range(shape.M):
        assert list(ids[t]) == _brute_topk(logits[t], 8)


def test_route_ties_signed_zero():
    l = np.array([[-0.0, 0.0, -0.0, 0.0, -1.0, -0.0]], np.float32)
    ids, _ = O.route(l, 4, 1.0)
    assert list(ids[0]) == [0, 1, 2, 3]


def test_route_weights_closed_forms():
    # equal logits 0: sigma = 1/2, S = k/2, w = scaling / k exactly
    ids, w = O.route(np.zeros((3, 16), np.float32), 8, 2.5)
    assert list(ids[0]) == list(range(8))
    assert np.all(w == np.float32(2.5 / 8))
    # sum of weights = scaling factor
    l = X.make_logits(X.Shape(M=64, H=512, E=256, I=128, top_k=8), "zipf", 5)
    _, w = O.route(l, 8, 2.5)
    assert np.allclose(w.astype(np.float64).sum(1), 2.5, rtol=1e-6, atol=0)
    # two selected logits a, b: w_a = 2.5 * s(a) / (s(a) + s(b))
    l = np.array([[3.0, -1.0, -5.0]], np.float32)
    _, w = O.route(l, 2, 2.5)
    sa, sb = 1 / (1 + np.exp(-3.0)), 1 / (1 + np.exp(1.0))
    assert abs(w[0, 0] - 2.5 * sa / (sa + sb)) < 1e-6
    # all selected logits -inf: zero weights
    _, w = O.route(np.full((1, 8), -np.inf, np.float32), 4, 2.5)
    assert np.all(w == 0)


def test_align_brute_force():
    rng = np.random.default_rng(0)
    for M, E, k in [(1, 4, 1), (5, 16, 2), (37, 32, 8), (64, 256, 8)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(M)])
        count, offset, se = O.align(ids, E)
        expect = []
        for e in range(E):
            for t in range(M):
                for j in range(k):
                    if ids[t, j] == e:
                        expect.append(t * k + j)
        assert list(se) == expect
        assert offset[E] == M * k and offset[0] == 0
        assert all(count[e] == sum(1 for v in ids.ravel() if v == e) for e in range(E))


def _grid_x(rng, M, H):
    """bf16 x whose 32-blocks sit on the E2M1 grid with block max 4: MX
    quantization is then the identity (scale code 127)."""
    x = F.e2m1_decode(rng.integers(0, 16, size=(M, H)))
    x[:, ::32] = 4.0
    return F.bf16_encode(x), x


def test_dequant_nibbles_and_scales():
    # byte 0x21 with scale code 128 -> [0.5, 1.0] * 2
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x21
    d = O.dequant_mxfp4(packed, np.array([[128]], np.uint8))
    assert d[0, 0] == 1.0 and d[0, 1] == 2.0 and np.all(d[0, 2:] == 0)


def test_gate_up_on_grid_is_matmul():
    rng = np.random.default_rng(1)
    M, H, I = 5, 256, 128
    xb, x = _grid_x(rng, M, H)
    xq, xs = O.quantize_x(xb)
    assert np.all(xs == 127)
    xd = F.mx_fp4_decode(xq, xs)
    assert np.array_equal(xd, x)
    wc = rng.integers(0, 16, size=(2 * I, H)).astype(np.uint8)
    w13 = F.pack_fp4(wc)
    s13 = np.full((2 * I, H // 32), 127, np.uint8)
    wd = O.dequant_mxfp4(w13, s13)
    assert np.array_equal(wd, F.e2m1_decode(wc))
    h = O.gate_up(xd, wd, I)
    g = np.matmul(x, F.e2m1_decode(wc[:I]).T).astype(np.float32)
    u = np.matmul(x, F.e2m1_decode(wc[I:]).T).astype(np.float32)
    silu = g.astype(np.float64) / (1 + np.exp(-g.astype(np.float64)))
    assert np.array_equal(h, (silu * u).astype(np.float32))
    # the halves are not interchangeable: gate rows are [0, I)
    swapped = np.concatenate([wd[I:], wd[:I]])
    assert not np.array_equal(O.gate_up(xd, swapped, I), h)


def test_down_on_grid_is_matmul():
    rng = np.random.default_rng(2)
    r, H, I = 6, 256, 256
    q = (rng.integers(0, 126, size=(r, I)) | (rng.integers(0, 2, size=(r, I)) << 7)).astype(np.uint8)
    s = np.ones((r, I // 128), np.float32)
    wc = rng.integers(0, 16, size=(H, I)).astype(np.uint8)
    w2d = O.dequant_mxfp4(F.pack_fp4(wc), np.full((H, I // 32), 127, np.uint8))
    y = O.down(q, s, w2d)
    assert np.array_equal(y, np.matmul(F.e4m3_decode(q), F.e2m1_decode(wc).T).astype(np.float32))
    # a power-of-two block scale scales that block's contribution exactly
    s2 = s.copy()
    s2[:, 1] = 4.0
    q0 = q.copy()
    q0[:, :128] = 0
    assert np.array_equal(O.down(q0, s2, w2d), (4 * O.down(q0, s, w2d)).astype(np.float32))


def test_shared_linear_on_grid_is_matmul():
    rng = np.random.default_rng(3)
    a = (rng.integers(0, 120, size=(4, 256))).astype(np.uint8)
    w = (rng.integers(0, 120, size=(256, 256))).astype(np.uint8)
    y = O._block_fp8_linear(a, np.ones((4, 2), np.float32), w, np.ones((2, 2), np.float32))
    assert np.array_equal(y, np.matmul(F.e4m3_decode(a), F.e4m3_decode(w).T).astype(np.float32))
    ws = np.array([[1.0, 2.0], [0.5, 8.0]], np.float32)  # per 128x128 block
    y2 = O._block_fp8_linear(a, np.ones((4, 2), np.float32), w, ws)
    ad, wd = F.e4m3_decode(a), F.e4m3_decode(w)
    ref = np.zeros((4, 256))
    for nb in range(2):
        for kb in range(2):
            ref[:, 128 * nb:128 * (nb + 1)] += ws[nb, kb] * (
                ad[:, 128 * kb:128 * (kb + 1)] @ wd[128 * nb:128 * (nb + 1), 128 * kb:128 * (kb + 1)].T)
    assert np.array_equal(y2, ref.astype(np.float32))


def _run(d, fn=O.moe_forward, **kw):
    s = d["shape"]
    shared = (d["ws13"], d["ss13"], d["ws2"], d["ss2"]) if s.shared_I else None
    args = dict(x_bits=d["x"], logits=d["logits"], w13=d["w13"], s13=d["s13"], w2=d["w2"],
                s2=d["s2"], top_k=s.top_k, scaling=s.routed_scaling, shared=shared)
    args.update(kw)
    return fn(**args)


@pytest.mark.parametrize("M,E,k,kind", [(4, 16, 2, "normal"), (1, 4, 1, "normal"), (8, 16, 4, "ties"),
                                        (3, 4, 4, "uniform"), (6, 8, 2, "normal")])
def test_dense_equals_sparse(M, E, k, kind):
    shape = X.Shape(M=M, H=512, E=E, I=128, top_k=k)
    d = X.make_inputs(shape, kind, 7)
    sparse = _run(d)["out"]
    dense = _run(d, fn=O.moe_dense)
    assert np.array_equal(sparse, dense)


def test_dense_equals_sparse_c0_and_shared():
    d = X.make_inputs("c0")
    assert np.array_equal(_run(d)["out"], _run(d, fn=O.moe_dense))
    shape = X.Shape(M=3, H=256, E=4, I=128, top_k=2, shared_I=128)
    d = X.make_inputs(shape, "normal", 9)
    assert np.array_equal(_run(d)["out"], _run(d, fn=O.moe_dense))


def test_zero_input_and_no_active_expert():
    d = X.make_inputs("c0")
    out = _run(d, x_bits=np.zeros_like(d["x"]))["out"]
    assert np.all(F.bf16_decode(out) == 0)
    out = _run(d, logits=np.full_like(d["logits"], -np.inf))["out"]
    assert np.all(F.bf16_decode(out) == 0)


def test_token_permutation_equivariance():
    d = X.make_inputs("c0")
    p = np.array([2, 0, 3, 1])
    a = _run(d)["out"]
    b = _run(d, x_bits=d["x"][p], logits=d["logits"][p])["out"]
    assert np.array_equal(a[p], b)


def test_expert_relabelling_invariance():
    d = X.make_inputs("c0")
    assert len(np.unique(d["logits"])) == d["logits"].size  # tie-free
    p = np.random.default_rng(4).permutation(16)  # new expert e holds old p[e]
    a = _run(d)["out"]
    b = _run(d, logits=d["logits"][:, p], w13=d["w13"][p], s13=d["s13"][p], w2=d["w2"][p],
             s2=d["s2"][p])["out"]
    assert np.array_equal(a, b)


def test_scaling_linearity():
    d = X.make_inputs("c0")
    a = F.bf16_decode(_run(d, scaling=2.5)["out"])
    b = F.bf16_decode(_run(d, scaling=5.0)["out"])
    assert np.array_equal(2 * a, b)


def test_intermediate_layout():
    d = X.make_inputs("c0")
    r = _run(d)
    s = d["shape"]
    n = s.M * s.top_k
    assert r["midq"].shape == (n, s.I) and r["mids"].shape == (n, s.I // 128)
    assert r["y"].shape == (n, s.H) and r["xq"].shape == (s.M, s.H) and r["xs"].shape == (s.M, s.H // 32)
    # midq rows are in sorted order: row r belongs to entry sorted_entry[r]
    ids = r["ids"].ravel()
    for e in range(s.E):
        assert np.all(ids[r["sorted_entry"][r["offset"][e]:r["offset"][e + 1]]] == e)


def test_page_mid_block_arithmetic():
    """288 blocks at TP4 with 8 rows x 9 slots; ~19 / ~38 KB of FP8 + scales;
    fp32 mid four times the FP8 bytes (tests/golden/mid_blocks.txt)."""
    rows = [l.split() for l in open(os.path.join(HERE, "golden", "mid_blocks.txt"))
            if l.strip() and not l.startswith("#")]
    for rws, slots, I, blocks, kb_fp8, kb_f32 in [[int(v) for v in r] for r in rows]:
        h = np.random.default_rng(0).normal(size=(rws * slots, I)).astype(np.float32)
        q, s = O.quantize_mid(h)
        assert s.size == blocks
        nbytes = q.size * q.itemsize + s.size * s.itemsize
        assert round(nbytes / 1000) == kb_fp8
        assert round(h.size * 4 / 1000) == kb_f32


# ------------------------------------------------------------ MXFP4 mid (the comparison arm)
def _grid_mid(rng, r, I):
    """Mid rows on the MXFP4 grid: random E2M1 codes and E8M0 scales per 32,
    each block holding a +-6 so that the MX rule recovers its scale."""
    codes = rng.integers(0, 16, size=(r, I)).astype(np.uint8)
    codes[:, ::32] = np.where(rng.integers(0, 2, size=(r, I // 32)) == 1, 15, 7)
    sc = rng.integers(118, 136, size=(r, I // 32)).astype(np.uint8)
    return codes, sc, F.mx_fp4_decode(codes, sc).astype(np.float32)


def test_mx_mid_on_grid_round_trips():
    rng = np.random.default_rng(11)
    codes, sc, h = _grid_mid(rng, 5, 256)
    q, s = O.quantize_mid_mx(h)
    assert np.array_equal(s, sc)
    assert np.array_equal(q, codes)  # signs of zeros included
    # amax 4 * 2^e picks the same scale as 6 * 2^e (floor(log2) - 2)
    h4 = np.zeros((1, 32), np.float32)
    h4[0, 3] = -4.0 * 2.0 ** -5
    q4, s4 = O.quantize_mid_mx(h4)
    assert s4[0, 0] == 127 - 5 and q4[0, 3] == 8 | 6


def test_mx_down_brute_force_fractions():
    """y[r, n] = fl32(sum_i mid[r, i] * w2[n, i]), summed exactly with Fractions
    on a tiny case with a different scale in every 32-block of both operands."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    r, H, I = 3, 4, 128
    codes, sc, _ = _grid_mid(rng, r, I)
    wc = rng.integers(0, 16, size=(H, I)).astype(np.uint8)
    ws = rng.integers(117, 124, size=(H, I // 32)).astype(np.uint8)
    w2d = O.dequant_mxfp4(F.pack_fp4(wc), ws)
    y = O.down_mx(codes, sc, w2d)
    mag = [0, 1, 2, 3, 4, 6, 8, 12]  # E2M1 magnitudes times 2

    def val(c, e):
        v = Fraction(mag[c & 7], 2) * Fraction(2) ** (int(e) - 127)
        return -v if c & 8 else v

    for a in range(r):
        for n in range(H):
            tot = sum(val(codes[a, i], sc[a, i // 32]) * val(wc[n, i], ws[n, i // 32]) for i in range(I))
            assert float(tot) == float(Fraction(float(tot)))  # exact in float64 here
            assert y[a, n] == np.float32(float(tot)), (a, n)


@pytest.mark.parametrize("M,E,k,kind", [(4, 16, 2, "normal"), (8, 16, 4, "ties"), (3, 4, 4, "uniform")])
def test_mx_mid_dense_equals_sparse(M, E, k, kind):
    shape = X.Shape(M=M, H=512, E=E, I=128, top_k=k)
    d = X.make_inputs(shape, kind, 17)
    sparse = _run(d, mid_format="mxfp4")
    assert sparse["midq"].shape == (M * k, 128) and sparse["mids"].shape == (M * k, 4)
    assert sparse["mids"].dtype == np.uint8
    assert np.array_equal(sparse["out"], _run(d, fn=O.moe_dense, mid_format="mxfp4"))


def test_mx_mid_invariants():
    d = X.make_inputs("c0")
    out = _run(d, x_bits=np.zeros_like(d["x"]), mid_format="mxfp4")["out"]
    assert np.all(F.bf16_decode(out) == 0)
    p = np.array([2, 0, 3, 1])
    a = _run(d, mid_format="mxfp4")["out"]
    b = _run(d, x_bits=d["x"][p], logits=d["logits"][p], mid_format="mxfp4")["out"]
    assert np.array_equal(a[p], b)
    # the E4M3 and MXFP4 arms share routing, sort, x and h, and differ after
    r8, r4 = _run(d), _run(d, mid_format="mxfp4")
    for key in ("ids", "sorted_entry", "xq", "h"):
        assert np.array_equal(r8[key], r4[key])
    assert not np.array_equal(r8["out"], r4["out"])


# ------------------------------------------------------------ shared expert as the last slot
def test_shared_slot_routing_brute_force():
    """Slots 0..k-2: the brute-force top-(k-1) of the first E-1 logits, with
    weights summing to the scaling factor over those slots; slot k-1: expert
    E-1 with weight exactly 1; the last logits column is never read."""
    rng = np.random.default_rng(21)
    M, E, k = 6, 17, 4
    lg = rng.normal(size=(M, E)).astype(np.float32)
    ids, w = O.route_shared_slot(lg, k, 2.5)
    for t in range(M):
        assert list(ids[t, :k - 1]) == _brute_topk(lg[t, :E - 1], k - 1)
        assert ids[t, k - 1] == E - 1 and w[t, k - 1] == np.float32(1.0)
        assert abs(float(np.sum(w[t, :k - 1], dtype=np.float64)) - 2.5) < 1e-5
    lg2 = lg.copy()
    lg2[:, E - 1] = 1e30  # would win every routed slot if it were read
    assert np.array_equal(O.route_shared_slot(lg2, k, 2.5)[0], ids)


def test_shared_slot_equals_routed_plus_shared_expert():
    """The fused call equals the routed call over the first E-1 experts with
    k-1 slots plus the shared expert applied to every token, added with weight
    1 before the one bf16 rounding (dense evaluation of the shared expert)."""
    shape = X.Shape(M=5, H=512, E=9, I=128, top_k=3)
    d = X.make_inputs(shape, "normal", 23)
    fused = _run(d, shared_slot=True)
    k, E = shape.top_k, shape.E
    routed = _run(d, logits=d["logits"][:, :E - 1], w13=d["w13"][:E - 1], s13=d["s13"][:E - 1],
                  w2=d["w2"][:E - 1], s2=d["s2"][:E - 1], top_k=k - 1)
    xd = F.mx_fp4_decode(*O.quantize_x(d["x"]))
    ysh = O.expert_dense(xd, d["w13"][E - 1], d["s13"][E - 1], d["w2"][E - 1], d["s2"][E - 1], shape.I)
    ref = O.combine(routed["w"], routed["y"].reshape(shape.M, k - 1, shape.H), ysh)
    assert np.array_equal(fused["out"], ref)
    assert np.array_equal(fused["out"], _run(d, fn=O.moe_dense, shared_slot=True))


def test_shared_slot_workloads_extend_c1_and_c2():
    """c1s / c2s are c1 / c2 with one more expert: the same x, the same
    routed experts' weights and logits; the shared expert's logits column is
    present but never read, and the oracle's routed slots equal c1's / c2's."""
    for fused, base in (("c1s", "c1"), ("c2s", "c2")):
        d, b = X.make_inputs(fused), X.make_inputs(base)
        E = b["shape"].E
        assert d["shape"].E == E + 1 and d["shape"].top_k == b["shape"].top_k + 1
        assert np.array_equal(d["x"], b["x"]) and np.array_equal(d["logits"][:, :E], b["logits"])
        for key in ("w13", "s13", "w2", "s2"):
            assert np.array_equal(d[key][:E], b[key])
        ids, w = O.route_shared_slot(d["logits"], d["shape"].top_k, 2.5)
        ids_b, w_b = O.route(b["logits"], b["shape"].top_k, 2.5)
        assert np.array_equal(ids[:, :-1], ids_b) and np.array_equal(w[:, :-1], w_b)


# ------------------------------------------------------------ shared expert, whole chain
def _e4m3_grid(rng, shape):
    return (rng.integers(0, 126, size=shape) | (rng.integers(0, 2, size=shape) << 7)).astype(np.uint8)


def _torch_fp8_quant(h):
    """Per-128 E4M3 quantization written with torch ops (an independent
    library): s = amax / 448 in binary32, codes = torch's E4M3 cast of h / s."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(h, np.float32)).reshape(h.shape[0], -1, 128)
    s = t.abs().amax(-1) / 448.0
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = (t / safe[..., None]).to(torch.float8_e4m3fn).to(torch.float64)
    q = torch.where(s[..., None] > 0, q, torch.zeros_like(q))
    return q.reshape(h.shape).numpy(), s.numpy()


def test_shared_expert_chain_on_grid():
    """The block-FP8 shared expert as an explicit chain. x on the E4M3 grid
    with every 128-block's amax 448 (so its quantization is the identity) and
    unit weight scales make the first GEMM a plain float64 matmul; then
    h = fl32(SiLU(gate rows [0, Is)) * up rows [Is, 2 Is)), h requantized per
    128 with torch's E4M3 cast, and the down GEMM with per-128x128 scales
    (powers of two per block, to see each block scale land on its block)."""
    rng = np.random.default_rng(11)
    M, H, Is = 3, 256, 256
    xc = _e4m3_grid(rng, (M, H))
    xc[:, ::128] = 0x7E  # +448 in every block
    xv = F.e4m3_decode(xc)
    x_bits = F.bf16_encode(xv)  # E4M3 values are exact in bf16
    ws13 = _e4m3_grid(rng, (2 * Is, H))
    # one power-of-two weight scale puts g and u in SiLU's curved range
    ss13 = np.full((2 * Is // 128, H // 128), 2.0 ** -17, np.float32)
    ws2 = _e4m3_grid(rng, (H, Is))
    ss2 = np.array([[1.0, 0.25], [4.0, 0.5]], np.float32)  # [H/128, Is/128]
    y, inter = O.shared_expert(x_bits, ws13, ss13, ws2, ss2)
    assert np.array_equal(inter["xq8"], xc) and np.all(inter["xs8"] == 1.0)

    w13v = F.e4m3_decode(ws13)
    g = (np.matmul(xv, w13v[:Is].T) * 2.0 ** -17).astype(np.float32).astype(np.float64)
    u = (np.matmul(xv, w13v[Is:].T) * 2.0 ** -17).astype(np.float32).astype(np.float64)
    assert 0.5 < np.median(np.abs(g)) < 8.0
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    assert np.array_equal(inter["h"], h)
    qv, hs = _torch_fp8_quant(h)
    assert np.array_equal(inter["hs"], hs)
    assert np.array_equal(F.e4m3_decode(inter["hq"]), qv)
    w2v = F.e4m3_decode(ws2)
    acc = np.zeros((M, H))
    for b in range(Is // 128):
        blk = slice(128 * b, 128 * (b + 1))
        S = np.matmul(qv[:, blk], w2v[:, blk].T)
        acc += hs[:, b].astype(np.float64)[:, None] * np.repeat(ss2[:, b].astype(np.float64), 128)[None, :] * S
    assert np.array_equal(y, acc.astype(np.float32))

    # plausible mistakes change the result
    swapped = np.concatenate([ws13[Is:], ws13[:Is]])
    assert not np.array_equal(O.shared_expert(x_bits, swapped, ss13, ws2, ss2)[0], y)
    h_wrong = (u / (1.0 + np.exp(-u)) * g).astype(np.float32)  # SiLU on the up half
    assert not np.array_equal(h_wrong, h)
    y_unquant = np.matmul(h.astype(np.float64), w2v.T)  # h not requantized
    assert not np.array_equal(y_unquant.astype(np.float32), y)
    ss2_t = np.ascontiguousarray(ss2[::-1])  # block scales on the wrong output rows
    assert not np.array_equal(O.shared_expert(x_bits, ws13, ss13, ws2, ss2_t)[0], y)



# ------------------------------------------------------------ tensor-parallel partial exchange
def test_tp_exchange_sum_pins():
    """A single rank's exchange equals the plain combine; zero peer partials
    (the one-GPU loopback) change nothing, whatever the rank; with values
    exact in float64 the result is the exact sum rounded once (checked with
    integer arithmetic); the rank order is the summation order."""
    d = X.make_inputs("c0")
    ref = _run(d)
    s = d["shape"]
    y = ref["y"].reshape(s.M, s.top_k, s.H)
    P = O.combine_partial(ref["w"], y)
    assert np.array_equal(F.bf16_encode(P), ref["out"])
    assert np.array_equal(O.tp_exchange_sum([P]), ref["out"])
    z = np.zeros_like(P)
    for r in range(8):
        parts = [z] * 8
        parts[r] = P
        assert np.array_equal(O.tp_exchange_sum(parts), ref["out"])
    rng = np.random.default_rng(5)
    ints = [rng.integers(-2 ** 40, 2 ** 40, size=(3, 64)) for _ in range(4)]
    exact = sum(int_ for int_ in ints)  # int64, exact
    got = O.tp_exchange_sum([np.ldexp(i.astype(np.float64), -30) for i in ints])
    assert np.array_equal(got, F.bf16_encode(np.ldexp(exact.astype(np.float64), -30)))
    # order matters where float64 rounds: (big + 1) - big != (big - big) + 1
    big = np.full((1, 1), 2.0 ** 60)
    one = np.full((1, 1), 1.0)
    assert F.bf16_decode(O.tp_exchange_sum([big, one, -big]))[0, 0] == 0.0
    assert F.bf16_decode(O.tp_exchange_sum([big, -big, one]))[0, 0] == 1.0


@pytest.mark.parametrize("M", [8, 300])
def test_extreme_scale_inputs_reach_the_edges(M):
    """The extreme-scale fixture reaches scale byte 0 on x and on w2, bf16
    subnormal x and binary32-subnormal outputs, routes each token group to its
    own experts only, and the oracle's exactness assertions hold on it."""
    shape = X.Shape(M=M, H=512, E=16, I=128, top_k=2)
    d = X.make_extreme_inputs(shape, 7)
    r = O.moe_forward(d["x"], d["logits"], d["w13"], d["s13"], d["w2"], d["s2"], 2, 2.5)
    grp = np.arange(M) % 4
    assert np.array_equal(np.sort(r["ids"], axis=1), np.stack([2 * grp, 2 * grp + 1], axis=1))
    assert (r["xs"][grp == 3] == 0).any() and (d["s2"][2:4] == 0).any()
    assert int(d["s13"].max()) >= 247 and int(d["s2"].max()) >= 229
    xv = F.bf16_decode(d["x"])
    assert ((np.abs(xv) < 2.0 ** -126) & (xv != 0)).any()
    y = np.abs(r["y"].reshape(M, 2, -1)[grp == 1])
    assert ((y < 2.0 ** -126) & (y > 0)).any()
    assert np.all(np.isfinite(F.bf16_decode(r["out"])))
