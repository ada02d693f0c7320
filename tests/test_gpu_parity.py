"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (from the method's acceptance criteria): top-k ids, token-to-expert
order, counts and offsets bit-exact; x's MXFP4 codes equal as decoded values
with equal scale bytes; FP8 mid codes within one E4M3 step on >= 99.9% of
elements and mid scales within 1e-6 relative; final bf16 output within a
max-abs error of 1e-2 x RMS(output). The kernels reproduce the oracle's
rounding points, so these tests also record how many elements differ at all
(expected: none on these inputs) and assert the routing weights bit-exact.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as O
from quantized_moe_expert_route_amd import fixtures as X

from moe_gpu import e4m3_ulp_distance, oracle, out_error, rows_by_entry, run, upload, make_plan

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2  # max-abs error / RMS(out)


def _check_routing(gi, ids, w, count, offset, se):
    assert np.array_equal(gi["ids"], ids), "top-k ids differ"
    assert np.array_equal(gi["w"].view(np.uint32), w.view(np.uint32)), \
        f"routing weights differ: max rel {np.max(np.abs(gi['w'] - w) / np.maximum(np.abs(w), 1e-30))}"
    assert np.array_equal(gi["count"], count)
    assert np.array_equal(gi["offset"], offset)
    assert np.array_equal(gi["sorted_entry"], se), "token-to-expert order differs"


def _check_xq(gi, ref, tokens=None):
    xq = F.unpack_fp4(gi["xq"])
    xs = gi["xs"]
    if tokens is not None:
        xq, xs = xq[tokens], xs[tokens]
    assert np.array_equal(xs, ref["xs"]), "x scale bytes differ"
    assert np.array_equal(F.e2m1_decode(xq), F.e2m1_decode(ref["xq"])), "x E2M1 values differ"


def _check_mid(gi_midq, gi_mids, ref_midq, ref_mids):
    d = e4m3_ulp_distance(gi_midq, ref_midq)
    assert d.max(initial=0) <= 1, f"mid codes more than one step apart: {d.max()}"
    frac_exact = float(np.mean(d == 0)) if d.size else 1.0
    assert frac_exact >= 0.999, f"only {frac_exact:.5f} of mid codes equal"
    rel = np.abs(gi_mids.astype(np.float64) - ref_mids) / np.maximum(np.abs(ref_mids), 1e-30)
    assert rel.max(initial=0) <= 1e-6, f"mid scales differ by {rel.max()}"
    return frac_exact


def _check_y(gy, ry):
    """Down output: equal to the oracle's fp32 value except where a 128-block
    dot product needs more than binary32's 24 bits (the MFMA then rounds
    inside the block): at most one fp32 step, on at most 1e-4 of elements."""
    a = gy.astype(np.float32).view(np.int32).astype(np.int64)
    b = ry.astype(np.float32).view(np.int32).astype(np.int64)
    same_sign = np.sign(gy) == np.sign(ry)
    steps = np.where(same_sign, np.abs(a - b), np.where(gy == ry, 0, 1 << 40))
    ndiff = int(np.count_nonzero(steps))
    assert steps.max(initial=0) <= 1, f"down output off by {steps.max()} fp32 steps"
    assert ndiff <= max(1, 1e-4 * gy.size), f"down output differs in {ndiff} elements"
    return ndiff


def _check_out(gout, rout):
    err, ndiff = out_error(gout, rout)
    print(f"out: max-abs/RMS {err:.3e}, {ndiff} of {rout.size} bf16 elements differ")
    assert err <= OUT_TOL, f"max-abs error {err:.3e} x RMS exceeds {OUT_TOL}"
    return ndiff


def _check_shared_x(gi, ref, tokens=None):
    """The shared expert's E4M3 x codes and per-128 scales: bit-exact (the
    scale and the division deciding each code are binary32 on both sides)."""
    q, s = gi["sh_xq"], gi["sh_xs"]
    if tokens is not None:
        q, s = q[tokens], s[tokens]
    np.testing.assert_array_equal(F.e4m3_decode(q), F.e4m3_decode(ref["shared"]["xq8"]))
    np.testing.assert_array_equal(s.view(np.uint32), ref["shared"]["xs8"].view(np.uint32))


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "t4_m16_hot"])
def test_stagewise_full(name):
    d = X.make_inputs(name)
    s = d["shape"]
    gout, gi = run(d)
    ref = oracle(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    n = s.M * s.top_k
    frac = _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    print(f"{name}: mid exact fraction {frac}")
    if gi["y"] is not None:  # (the combine inside the down launch: no y)
        ydiff = _check_y(gi["y"], ref["y"])
        print(f"{name}: y differs in {ydiff} of {ref['y'].size}")
    ndiff = _check_out(gout, ref["out"])
    assert ndiff == 0, "expected the oracle's bf16 output exactly on these inputs"


@pytest.mark.parametrize("name,n_tok", [("c3", 12), ("c4", 15), ("m32_spread", 6), ("m64_mixed", 6),
                                        ("m128_spread", 8), ("m256_hot", 8), ("m256_mixed", 8)])
def test_sampled_full_size(name, n_tok):
    """Full-size call as the benchmark runs it; routing/sort checked on every
    token, everything else on a sample of tokens the oracle evaluates alone.
    The mid-range batches (M = 32..256, hot / mixed / spread expert reuse)
    cover both paths at the sizes between decode and prefill."""
    d = X.make_inputs(name)
    s = d["shape"]
    gout, gi = run(d)
    ids, w = O.route(d["logits"], s.top_k, s.routed_scaling)
    count, offset, se = O.align(ids, s.E)
    _check_routing(gi, ids, w, count, offset, se)
    rng = np.random.default_rng(123)
    tokens = rng.choice(s.M, n_tok, replace=False)
    if name == "c4":
        # token rows whose outputs an fp32-accumulated shared expert once
        # moved by up to 3.7e-2 x RMS (an E4M3 x E4M3 block sum rounded
        # inside the MFMA flipped a shared mid code)
        tokens = np.concatenate([tokens[:8], [686, 693, 831, 1970, 2551, 2680, 3739]])
    tokens = np.sort(tokens)
    ref = oracle(d, tokens)
    _check_xq(gi, ref, tokens)
    k = s.top_k
    ent = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    g_midq = rows_by_entry(gi["midq"], gi["sorted_entry"], s.M * k)[ent]
    g_mids = rows_by_entry(gi["mids"], gi["sorted_entry"], s.M * k)[ent]
    r_midq = rows_by_entry(ref["midq"], ref["sorted_entry"], n_tok * k)
    r_mids = rows_by_entry(ref["mids"], ref["sorted_entry"], n_tok * k)
    _check_mid(g_midq, g_mids, r_midq, r_mids)
    if gi["y"] is not None:  # (the combine inside the down launch: no y)
        ydiff = _check_y(gi["y"][ent], ref["y"])
        print(f"{name}: y differs in {ydiff} of {ref['y'].size} sampled elements")
    if s.shared_I:
        _check_shared_x(gi, ref, tokens)
        sdiff = int(np.count_nonzero(gi["sh_y"][tokens].view(np.uint32) != ref["ys"].view(np.uint32)))
        print(f"{name}: shared-expert output differs in {sdiff} of {ref['ys'].size}")
    _check_out(gout[tokens], ref["out"])


SMALL = [
    # (M, H, E, I, k, logits, shared_I)
    # up to 16 tokens: one workgroup routes and sorts, down and combine in one launch
    (1, 512, 16, 128, 2, "normal", 0),
    (16, 512, 64, 128, 8, "ties", 0),          # the last size of the small path
    (4, 65536, 4, 128, 2, "normal", 0),        # largest H
    (5, 1024, 4, 256, 1, "normal", 0),         # top-1
    (9, 512, 8, 384, 8, "ties", 0),            # k = E, many ties, I = 384
    (33, 512, 64, 128, 8, "ties", 0),          # ties and signed zeros
    (40, 1024, 32, 256, 4, "zipf", 0),         # skew: one expert takes most tokens
    (3, 512, 4, 128, 2, "normal", 128),        # shared expert (inside the small-token launches)
    (1, 512, 4, 128, 2, "normal", 512),        # one token, the widest fused shared expert
    (16, 1536, 16, 256, 8, "ties", 384),       # 16 tokens with a fused shared expert
    (12, 65536, 4, 128, 2, "normal", 128),     # fused shared expert at the largest H
    (5, 512, 8, 128, 2, "normal", 640),        # a shared expert too wide to fuse: its own pass
    # above 16 tokens: the large path's routing and sort; up to 256 tokens gate/up on
    # 16-row tiles with its own mid quantization, above on 64-row tiles with it inside
    (17, 512, 16, 128, 2, "normal", 0),        # one token past the small path; ragged tiles
    (20, 512, 1024, 128, 16, "uniform", 0),    # largest E and k
    (20, 65536, 4, 128, 2, "normal", 0),       # largest H (mid-range path)
    (65, 512, 16, 128, 2, "normal", 0),
    (257, 512, 64, 128, 8, "uniform", 0),      # one token past the 16-row-tile gate/up
    (130, 1024, 32, 256, 8, "zipf", 0),        # skewed: a tile of 128 plus ragged tails
    (300, 512, 8, 512, 2, "normal", 0),        # several full tiles per expert, I = 512
    (257, 65536, 2, 128, 1, "normal", 0),      # largest H (large path: x scales staged in 11 parts)
    (96, 512, 64, 384, 8, "ties", 0),
    (70, 512, 4, 128, 2, "normal", 128),       # with the shared expert
    (72, 8192, 8, 128, 2, "normal", 0),        # H past 6144: x scales staged in two parts
    (80, 1536, 8, 128, 2, "normal", 128),      # shared expert, H = 3 x 512
    (66, 9216, 4, 128, 2, "normal", 128),      # x rows past 8192: the route reads them in two chunks
    # at least 8 entries per expert (M k >= 8 E) and H a multiple of 2048 up to
    # 8192: gate/up and the mid quantization in one launch
    (16, 2048, 16, 256, 8, "ties", 256),       # with the fused shared expert's mid blocks (32 of them)
    (13, 4096, 8, 384, 8, "normal", 128),      # three mid blocks; 13 shared mid blocks, 4 to a workgroup
    (200, 6144, 16, 256, 8, "zipf", 0),        # ragged tiles of a skewed mid-range call
    (8, 2048, 1, 128, 1, "normal", 0),         # one expert, one tile
    (64, 2048, 8, 512, 2, "normal", 0),        # I = 512: four mid blocks a tile
]


@pytest.mark.parametrize("M,H,E,I,k,kind,Is", SMALL)
def test_small_shapes(M, H, E, I, k, kind, Is):
    shape = X.Shape(M=M, H=H, E=E, I=I, top_k=k, shared_I=Is)
    d = X.make_inputs(shape, kind, 1000 + M)
    gout, gi = run(d)
    ref = oracle(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    if Is:
        _check_shared_x(gi, ref)
        _check_shared_mid(gi, ref)
    _check_out(gout, ref["out"])


def _check_shared_mid(gi, ref, tokens=None):
    """The shared expert's E4M3 mid codes and per-128 scales: bit-exact."""
    q, s = gi["sh_hq"], gi["sh_hs"]
    if tokens is not None:
        q, s = q[tokens], s[tokens]
    np.testing.assert_array_equal(F.e4m3_decode(q), F.e4m3_decode(ref["shared"]["hq"]))
    np.testing.assert_array_equal(s.view(np.uint32), ref["shared"]["hs"].view(np.uint32))


@pytest.mark.parametrize("name", ["c1b", "c2b"])
def test_fused_shared_expert(name):
    """Up to 16 tokens the block-FP8 shared expert runs inside the routed
    launches (its stage launches nothing of its own): its x codes and scales,
    its mid codes and scales and the output equal the oracle bit for bit."""
    d = X.make_inputs(name)
    s = d["shape"]
    g = upload(d)
    plan = make_plan(s)
    plan.set_shared(g["ws13"], g["ss13"], g["ws2"], g["ss2"])
    launches = plan.stage_launches(s.M)
    assert launches[4] == 0 and launches == [1, 0, 1, 1, 0, 1, 0]
    gout, gi = run(d, plan=plan, g=g)
    ref = oracle(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    _check_shared_x(gi, ref)
    _check_shared_mid(gi, ref)
    ndiff = _check_out(gout, ref["out"])
    assert ndiff == 0, "expected the oracle's bf16 output exactly"


def test_shared_x_codes_on_exact_midpoints():
    """x blocks whose amax is 672 (scale fl32(672 / 448) = 1.5, whose
    reciprocal is not exact) and whose other entries are 1.5 x an E4M3
    rounding midpoint, so fl32(x / s) lands exactly on a tie (normal
    midpoints over every binade, and the subnormal grid's): the E4M3 codes
    must follow round-half-to-even, bit for bit with the oracle."""
    import itertools

    shape = X.Shape(M=80, H=512, E=8, I=128, top_k=2, shared_I=128)
    d = X.make_inputs(shape, "normal", 4242)
    mids = [(1 + (2 * j + 1) / 16) * 2.0 ** e for e in range(-6, 9) for j in range(8)]
    mids = [m for m in mids if m < 448] + [(k + 0.5) / 512 for k in range(8)]
    vals = np.array([1.5 * m for m in mids], np.float64)
    x = np.empty((shape.M, shape.H), np.float64)
    cyc = itertools.cycle(range(len(vals)))
    for t in range(shape.M):
        for b in range(shape.H // 128):
            blk = np.array([vals[next(cyc)] for _ in range(128)])
            blk *= np.where(np.arange(128) % 3 == 0, -1.0, 1.0)
            blk[(t + b) % 128] = 672.0
            x[t, 128 * b:128 * b + 128] = blk
    bits = F.bf16_encode(x)
    assert np.array_equal(F.bf16_decode(bits), x), "test values must be exact in bf16"
    d["x"] = bits
    gout, gi = run(d)
    ref = oracle(d)
    _check_shared_x(gi, ref)
    _check_xq(gi, ref)
    _check_out(gout, ref["out"])


@pytest.mark.parametrize("M", [3, 6, 40, 300])  # routing inside gate/up, small, mid-range and large paths
def test_degenerate_inputs(M):
    """x = 0; all logits -inf (every token on experts 0..k-1 with weight 0:
    the most skewed sort); all logits equal."""
    shape = X.Shape(M=M, H=512, E=16, I=128, top_k=4)
    d = X.make_inputs(shape, "normal", 5)
    # x = 0: every output zero
    d0 = dict(d, x=np.zeros_like(d["x"]))
    gout, _ = run(d0)
    assert np.all(F.bf16_decode(gout) == 0)
    # all logits -inf: no active weight, output zero
    d1 = dict(d, logits=np.full_like(d["logits"], -np.inf))
    gout, gi = run(d1)
    assert np.all(F.bf16_decode(gout) == 0)
    assert np.all(gi["w"] == 0)
    # all logits equal: experts 0..k-1, weights scaling / k
    d2 = dict(d, logits=np.zeros_like(d["logits"]))
    gout, gi = run(d2)
    assert np.all(gi["ids"] == np.arange(4)[None, :])
    assert np.all(gi["w"] == np.float32(2.5 / 4))
    ref = oracle(d2)
    _check_out(gout, ref["out"])


def test_m_zero_is_a_noop():
    import torch

    shape = X.Shape(M=8, H=512, E=16, I=128, top_k=2)
    d = X.make_inputs(shape, "normal", 2)
    g = upload(d)
    plan = make_plan(shape)
    out = torch.full((8, 512), 7, dtype=torch.int16, device="cuda")
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], g["w2"], g["s2"], out, M=0)
    torch.cuda.synchronize()
    assert bool((out == 7).all())


def test_variable_m_and_changing_inputs_one_plan():
    """200 calls with fresh inputs and varying M through one plan and one
    workspace: catches state left behind by a previous call."""
    import torch

    base = X.Shape(M=24, H=512, E=16, I=128, top_k=4)
    plan = make_plan(base)
    rng = np.random.default_rng(9)
    w = X.make_inputs(base, "normal", 77)
    g = upload(w)
    for it in range(200):
        M = int(rng.integers(1, 25))
        shape = X.Shape(M=M, H=512, E=16, I=128, top_k=4)
        d = X.make_inputs(shape, ["normal", "ties", "uniform"][it % 3], 5000 + it, with_weights=False)
        for key in ("w13", "s13", "w2", "s2"):
            d[key] = w[key]
        gd = dict(g)
        gd["x"] = torch.from_numpy(d["x"].view(np.int16)).cuda()
        gd["logits"] = torch.from_numpy(d["logits"]).cuda()
        gout, gi = run(d, plan=plan, g=gd, M=M)
        if it % 20 == 0 or it < 3:
            ref = oracle(d)
            _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
            assert np.array_equal(gout, ref["out"]), f"iteration {it}: output differs"


def test_run_to_run_bitwise():
    d = X.make_inputs("c2")
    g = upload(d)
    plan = make_plan(d["shape"])
    a, _ = run(d, plan=plan, g=g)
    b, _ = run(d, plan=plan, g=g)
    assert np.array_equal(a, b)


# block-FP8 shared expert in a pass of its own: above kSmallM, and at
# M <= kSmallM with shared_I above the limit of the fused form
_GRAPH_SHAPES = {
    "shared_large": (X.Shape(M=200, H=1024, E=32, I=256, top_k=4, shared_I=256), "zipf", 41),
    "shared_small_wide": (X.Shape(M=12, H=1024, E=32, I=256, top_k=4, shared_I=640), "normal", 42),
}


@pytest.mark.parametrize("name,mxfp4", [("c1", False), ("c1b", False), ("m64_mixed", False), ("c3", False),
                                        ("m256_hot", True), ("shared_large", False), ("shared_small_wide", False)])
def test_graph_replay_matches_eager(name, mxfp4):
    """Replays of a captured call (small, mid-range and large paths; the
    MXFP4 mid; the block-FP8 shared expert's own pass) equal the eager call
    bitwise, with eager calls between them: every call leaves the token
    bitmap zero for the next."""
    import torch

    from quantized_moe_expert_route_amd.binding import MID_MXFP4, layout_for, pack_w2

    d = X.make_inputs(*_GRAPH_SHAPES[name]) if name in _GRAPH_SHAPES else X.make_inputs(name)
    s = d["shape"]
    g = upload(d)
    plan = make_plan(s)
    if s.shared_I:
        plan.set_shared(g["ws13"], g["ss13"], g["ws2"], g["ss2"])
    w2, s2 = g["w2"], g["s2"]
    if mxfp4:
        plan.set_mid_format(MID_MXFP4)
        plan.set_weight_layout(layout_for(MID_MXFP4))
        w2, s2 = pack_w2(w2, s2)
    call = lambda o: plan.forward(g["x"], g["logits"], g["w13"], g["s13"], w2, s2, o)
    eager = torch.empty((s.M, s.H), dtype=torch.int16, device="cuda")
    call(eager)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call(out)  # warm-up off-graph
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    for i in range(5):
        out.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager call"
        call(eager)  # eager work between
        torch.cuda.synchronize()


def test_variable_m_across_paths_one_plan():
    """One plan, calls alternating between the small-token and large-token paths."""
    base = X.Shape(M=300, H=512, E=16, I=256, top_k=4)
    plan = make_plan(base)
    w = X.make_inputs(base, "normal", 31)
    import torch

    for it, M in enumerate([70, 4, 300, 65, 16, 17, 257, 256, 64, 128, 1]):
        shape = X.Shape(M=M, H=512, E=16, I=256, top_k=4)
        d = X.make_inputs(shape, "zipf" if it % 2 else "normal", 900 + it, with_weights=False)
        for key in ("w13", "s13", "w2", "s2"):
            d[key] = w[key]
        g = upload(d)
        gout, gi = run(d, plan=plan, g=g, M=M)
        ref = oracle(d)
        _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
        _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
        assert np.array_equal(gout, ref["out"]), f"M={M}: output differs"


@pytest.mark.parametrize("name,n_tok", [("c3", 6), ("c4", 6)])
def test_stage_isolated_full_size(name, n_tok):
    """Each late stage fed the GPU's own inputs, at the benchmark's sizes: the
    oracle's down on the GPU's mid rows against the GPU's y, the oracle's
    combine on the GPU's y (and shared-expert y) against the GPU's output, and
    at c4 the oracle's shared down on the GPU's shared mid. This separates a
    stage's own error from differences it inherits (a mid code one E4M3 step
    off moves every output of its token)."""
    d = X.make_inputs(name)
    s = d["shape"]
    k, H = s.top_k, s.H
    gout, gi = run(d)
    tokens = np.sort(np.random.default_rng(77).choice(s.M, n_tok, replace=False))
    ent = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    pos = np.empty(s.M * k, np.int64)
    pos[gi["sorted_entry"]] = np.arange(s.M * k)  # sorted row of each entry
    ids = gi["ids"].ravel()
    y_ref = np.empty((len(ent), H), np.float32)
    for i, e_i in enumerate(ent):
        r, e = pos[e_i], ids[e_i]
        y_ref[i] = O.down(gi["midq"][r:r + 1], gi["mids"][r:r + 1], O.dequant_mxfp4(d["w2"][e], d["s2"][e]))[0]
    ydiff = _check_y(gi["y"][ent], y_ref)
    ys = None
    if s.shared_I:
        ys = gi["sh_y"][tokens]
        ys_ref = O._block_fp8_linear(gi["sh_hq"][tokens], gi["sh_hs"][tokens], d["ws2"], d["ss2"])
        # the int8-digit GEMM forms every E4M3 x E4M3 block sum exactly
        sdiff = int(np.count_nonzero(ys.view(np.uint32) != ys_ref.view(np.uint32)))
        assert sdiff == 0, f"shared down (isolated) differs in {sdiff} of {ys_ref.size}"
    out_ref = O.combine(gi["w"][tokens], gi["y"][ent].reshape(n_tok, k, H), ys)
    assert np.array_equal(gout[tokens], out_ref), "combine on the GPU's own y differs from the oracle's"
    print(f"{name}: down (isolated) differs in {ydiff} of {y_ref.size}; combine (isolated) exact")


def test_largest_m_sampled():
    """16384 tokens (131072 entries) at a small H: routing, weights and the
    sort checked on every token, x, mid and output on sampled tokens."""
    shape = X.Shape(M=16384, H=512, E=64, I=128, top_k=8)
    d = X.make_inputs(shape, "zipf", 4242)
    gout, gi = run(d)
    ids, w = O.route(d["logits"], shape.top_k, shape.routed_scaling)
    count, offset, se = O.align(ids, shape.E)
    _check_routing(gi, ids, w, count, offset, se)
    tokens = np.sort(np.random.default_rng(8).choice(shape.M, 12, replace=False))
    ref = oracle(d, tokens)
    _check_xq(gi, ref, tokens)
    k = shape.top_k
    ent = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    g_midq = rows_by_entry(gi["midq"], gi["sorted_entry"], shape.M * k)[ent]
    g_mids = rows_by_entry(gi["mids"], gi["sorted_entry"], shape.M * k)[ent]
    _check_mid(g_midq, g_mids, rows_by_entry(ref["midq"], ref["sorted_entry"], len(tokens) * k),
               rows_by_entry(ref["mids"], ref["sorted_entry"], len(tokens) * k))
    _check_y(gi["y"][ent], ref["y"])
    _check_out(gout[tokens], ref["out"])


def test_c4_shared_expert_every_token():
    """c4 (4096 tokens, block-FP8 shared expert): the shared expert's x codes
    and scales, mid codes and scales and output against the oracle's shared
    expert on every token, all bitwise (its block sums are exact); then the
    final output of every token against the oracle's combine of the GPU's own
    routed y with the oracle's shared output, bitwise (the routed part is
    checked against the oracle on sampled tokens in test_sampled_full_size)."""
    d = X.make_inputs("c4")
    s = d["shape"]
    gout, gi = run(d)
    ys_ref, sh = O.shared_expert(d["x"], d["ws13"], d["ss13"], d["ws2"], d["ss2"])
    assert np.array_equal(F.e4m3_decode(gi["sh_xq"]), F.e4m3_decode(sh["xq8"])), "shared x codes differ"
    assert np.array_equal(gi["sh_xs"].view(np.uint32), sh["xs8"].view(np.uint32)), "shared x scales differ"
    qdiff = int(np.count_nonzero(F.e4m3_decode(gi["sh_hq"]) != F.e4m3_decode(sh["hq"])))
    hdiff = int(np.count_nonzero(gi["sh_hs"].view(np.uint32) != sh["hs"].view(np.uint32)))
    ydiff = int(np.count_nonzero(gi["sh_y"].view(np.uint32) != ys_ref.view(np.uint32)))
    print(f"c4 shared: mid codes differ in {qdiff} of {sh['hq'].size}, mid scales in {hdiff}, "
          f"output in {ydiff} of {ys_ref.size}")
    assert qdiff == 0 and hdiff == 0 and ydiff == 0
    ids, w = O.route(d["logits"], s.top_k, s.routed_scaling)
    count, offset, se = O.align(ids, s.E)
    _check_routing(gi, ids, w, count, offset, se)
    out_ref = O.combine(gi["w"], gi["y"].reshape(s.M, s.top_k, s.H), ys_ref)
    _check_out(gout, out_ref)
    assert np.array_equal(gout, out_ref), "out differs from the combine of the GPU's y and the oracle's shared output"


def test_declared_weight_layout_is_required():
    """A call is refused (MOE_ERR_UNSUPPORTED, nothing enqueued, out left as
    it was) unless the plan declares the weight layout its kernels read:
    packed gate/up weights, and packed down weights exactly with the MXFP4
    mid."""
    import torch

    from quantized_moe_expert_route_amd.binding import (LAYOUT_W13_PACKED, LAYOUT_W2_PACKED, MID_E4M3, MID_MXFP4,
                                                        MOE_ERR_UNSUPPORTED, lib)

    shape = X.Shape(M=4, H=512, E=16, I=128, top_k=2)
    d = X.make_inputs(shape, "normal", 3)
    g = upload(d)
    plan = make_plan(shape)
    out = torch.full((4, 512), 7, dtype=torch.int16, device=g["x"].device)
    for fmt, layout in ((MID_E4M3, 0), (MID_E4M3, LAYOUT_W2_PACKED), (MID_E4M3, LAYOUT_W13_PACKED | LAYOUT_W2_PACKED),
                        (MID_MXFP4, LAYOUT_W13_PACKED)):
        plan.set_mid_format(fmt)
        plan.set_weight_layout(layout)
        # straight through the C ABI: the binding's own size checks would
        # refuse the row-major down scales under a packed declaration first
        args = [g[k].data_ptr() for k in ("x", "logits", "w13", "s13", "w2", "s2")] + [out.data_ptr(), None]
        assert lib().moe_forward(plan._h, 4, *args) == MOE_ERR_UNSUPPORTED
        assert lib().moe_forward_noalloc(plan._h, 4, *args) == MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7).all()), "a refused call wrote its output"
    plan.set_mid_format(MID_E4M3)
    plan.set_weight_layout(LAYOUT_W13_PACKED)
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], g["w2"], g["s2"], out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle(d)["out"])


@pytest.mark.parametrize("active", [33, 40, 63, 64, 65, 100, 128])
def test_small_down_ring_batches(active):
    """Sixteen tokens whose top-8 cover exactly `active` experts, one 16-row
    tile each: the small-path down's waves take up to 32 tiles against 8
    ring slots, so runs of 9, 16, 17, 25 and 32 tiles exercise the reloads
    of full batches, of a last partial batch (slots past the run reload its
    last tile and skip its products) and none. Output, mid and routing equal
    the oracle's bit for bit."""
    shape = X.Shape(M=16, H=1024, E=128, I=256, top_k=8)
    d = X.make_inputs(shape, "normal", 500 + active)
    lg = np.random.default_rng(active).standard_normal((16, 128)).astype(np.float32)
    for t in range(16):
        for j in range(8):
            lg[t, (8 * t + j) % active] = np.float32(10.0 - 0.5 * j)  # slot j: expert (8t + j) mod active
    d["logits"] = lg
    gout, gi = run(d)
    ref = oracle(d)
    assert int(np.count_nonzero(ref["count"])) == active
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    assert _check_out(gout, ref["out"]) == 0, "expected the oracle's bf16 output exactly"


@pytest.mark.parametrize("M,H,E,I,k,kind,inside,qd", [
    (1, 6144, 256, 256, 8, "uniform", True, True),
    (2, 2048, 200, 256, 8, "ties", True, True),     # tied logits: the lower expert id wins, as in the routing launch
    (3, 2048, 128, 128, 4, "normal", True, True),
    (4, 1024, 64, 512, 2, "normal", True, True),    # four mid blocks a row: 32 of 64 blocks
    (4, 512, 16, 128, 16, "normal", True, False),   # k = E: every expert active; 64 rows, more than the ring holds
    (4, 6144, 256, 256, 8, "uniform", True, True),  # c1's shape: 64 mid blocks, at the limit
    (4, 2048, 64, 256, 12, "normal", True, False),  # 96 mid blocks: the mid quantization in its own launch
    (4, 8192, 64, 128, 4, "normal", False, False),  # H past 6144: the routing launch
    (4, 2048, 320, 128, 8, "uniform", False, False),  # E past 256: the routing launch
    (4, 2048, 64, 512, 16, "normal", True, False),  # 256 mid blocks, 32 KB of mid (four blocks a row)
])
def test_routing_inside_gate_up(M, H, E, I, k, kind, inside, qd):
    """Up to 4 tokens (E <= 256, H <= 6144, no shared expert) the gate/up
    launch routes, sorts and quantizes x itself: the call has no routing
    launch; with at most 64 mid blocks (and no more 16-row tiles than the
    small down's ring holds) each down workgroup also quantizes the mid from
    h itself, so the call has no act_quant launch either. Ids, weights,
    counts, offsets, the sorted entries, x's codes, the mid codes and scales
    and the output equal the oracle's bit for bit on every path."""
    shape = X.Shape(M=M, H=H, E=E, I=I, top_k=k)
    d = X.make_inputs(shape, kind, 900 + M + E)
    plan = make_plan(shape)
    assert plan.stage_launches(M) == [0 if inside else 1, 0, 1, 0 if qd else 1, 0, 1, 0]
    gout, gi = run(d, plan=plan)
    ref = oracle(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    np.testing.assert_array_equal(gi["midq"], ref["midq"])
    np.testing.assert_array_equal(gi["mids"].view(np.uint32), ref["mids"].astype(np.float32).view(np.uint32))
    assert _check_out(gout, ref["out"]) == 0, "expected the oracle's bf16 output exactly"

