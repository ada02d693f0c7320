"""GPU parity of the MXFP4 mid hand-off (the stock MXFP4 comparison arm,
moe_plan_set_mid_format(MOE_MID_MXFP4)) against the oracle's mid_format
"mxfp4".

Bars: routing, sort and x as in the E4M3 path (bit-exact); the MXFP4 mid
codes and E8M0 scale bytes bit-exact (h is the same fp32 value on both sides
and the quantization is exact arithmetic on it); y equal to the oracle's
fp32 value up to one fp32 step on at most 1e-4 of elements (the scaled FP4
MFMA sums a K-step's four 32-blocks in binary32); output within 1e-2 x RMS.
"""

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as O
from quantized_moe_expert_route_amd import fixtures as X

from moe_gpu import make_plan, rows_by_entry, upload
from test_gpu_parity import _check_out, _check_routing, _check_xq, _check_y

pytestmark = pytest.mark.gpu


def _upload_mx(d):
    """upload() plus the down weights packed for the MXFP4-mid down."""
    from quantized_moe_expert_route_amd.binding import pack_w2

    g = upload(d)
    g["w2p"], g["s2p"] = pack_w2(g["w2"], g["s2"])
    return g


def _run_mx(d, plan=None, g=None, M=None, fmt=None):
    import torch

    from quantized_moe_expert_route_amd.binding import MID_MXFP4, layout_for

    s = d["shape"]
    M = s.M if M is None else M
    g = _upload_mx(d) if g is None else g
    fmt = MID_MXFP4 if fmt is None else fmt
    if plan is None:
        plan = make_plan(s)
        if s.shared_I:
            plan.set_shared(g["ws13"], g["ss13"], g["ws2"], g["ss2"])
    plan.set_mid_format(fmt)
    plan.set_weight_layout(layout_for(fmt))
    out = torch.full((max(M, 1), s.H), -1, dtype=torch.int16, device=g["x"].device)
    w2, s2 = (g["w2p"], g["s2p"]) if fmt == MID_MXFP4 else (g["w2"], g["s2"])
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], w2, s2, out, M=M)
    torch.cuda.synchronize()
    k, n, I, H = s.top_k, M * s.top_k, s.I, s.H
    v = plan.view
    gi = {
        "ids": v("topk_ids", torch.int32, (M, k)),
        "w": v("topk_w", torch.float32, (M, k)),
        "count": v("count", torch.int32, (s.E,)),
        "offset": v("offset", torch.int32, (s.E + 1,)),
        "sorted_entry": v("sorted_entry", torch.int32, (n,)),
        "xq": v("xq", torch.uint8, (M, H // 2)),
        "xs": v("xs", torch.uint8, (M, H // 32)),
        "midq": v("midq", torch.uint8, (n, I // 2)),
        "mids": v("mids", torch.uint8, (n, I // 32)),
        "y": v("y", torch.float32, (n, H)),
    }
    gi = {key: t.cpu().numpy() for key, t in gi.items()}
    return out[:M].cpu().numpy().view(np.uint16), gi, plan, g


def _oracle_mx(d, tokens=None):
    s = d["shape"]
    x, lg = d["x"], d["logits"]
    if tokens is not None:
        x, lg = x[tokens], lg[tokens]
    shared = (d["ws13"], d["ss13"], d["ws2"], d["ss2"]) if s.shared_I else None
    return O.moe_forward(x, lg, d["w13"], d["s13"], d["w2"], d["s2"], s.top_k, s.routed_scaling, shared,
                         mid_format="mxfp4")


def _check_mid_mx(g_midq, g_mids, r_codes, r_scales):
    assert np.array_equal(g_mids, r_scales), "mid E8M0 scale bytes differ"
    assert np.array_equal(F.unpack_fp4(g_midq), r_codes), "mid E2M1 codes differ"


SHAPES = [
    # (M, H, E, I, k, logits, shared_I)
    (4, 512, 16, 128, 2, "normal", 0),         # small path routing, fused-free down
    (16, 512, 64, 256, 8, "ties", 0),          # the last size of the small path
    (17, 512, 16, 128, 2, "normal", 0),        # grid-wide routing; ragged tiles
    (40, 1024, 32, 256, 4, "zipf", 0),         # skew: one expert takes most rows
    (20, 512, 1024, 128, 16, "uniform", 0),    # largest E and k
    (3, 512, 4, 128, 2, "normal", 128),        # with the shared expert
    (256, 512, 16, 384, 4, "normal", 0),       # the largest M served; I = 384 (3 K-steps)
    (70, 512, 8, 512, 2, "normal", 0),         # I = 512 (4 K-steps)
    (257, 512, 16, 128, 4, "normal", 0),       # above 256 tokens: the mid quantized inside the 64-row gate/up
    (300, 1024, 32, 256, 8, "zipf", 0),        # large path, skewed
    (600, 512, 8, 512, 2, "normal", 128),      # large path, I = 512, with the shared expert
    # M k >= 8 E, H a multiple of 2048 up to 8192: gate/up and the MXFP4 mid in one launch
    (16, 2048, 16, 256, 8, "ties", 0),
    (100, 4096, 8, 384, 4, "zipf", 0),         # three mid blocks, skewed tiles
    (64, 2048, 8, 512, 2, "normal", 0),        # I = 512: four mid blocks a tile
]


@pytest.mark.parametrize("M,H,E,I,k,kind,Is", SHAPES)
def test_mx_small_shapes(M, H, E, I, k, kind, Is):
    shape = X.Shape(M=M, H=H, E=E, I=I, top_k=k, shared_I=Is)
    d = X.make_inputs(shape, kind, 2000 + M)
    gout, gi, _, _ = _run_mx(d)
    ref = _oracle_mx(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    _check_mid_mx(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    ydiff = _check_y(gi["y"], ref["y"])
    ndiff = _check_out(gout, ref["out"])
    print(f"M={M}: y differs in {ydiff}, out in {ndiff} elements")


@pytest.mark.parametrize("name,n_tok", [("c1", 0), ("c2", 0), ("t4_m16_hot", 0), ("m256_hot", 8),
                                        ("m256_mixed", 8), ("m64_spread", 6), ("c3", 8),
                                        ("t4_m4096_spread", 6), ("t4_m4096_hot", 6)])
def test_mx_full_size(name, n_tok):
    """The benchmark's shapes: every token (n_tok = 0) or a sample the oracle
    evaluates alone; routing and sort on every token."""
    d = X.make_inputs(name)
    s = d["shape"]
    gout, gi, _, _ = _run_mx(d)
    ids, w = O.route(d["logits"], s.top_k, s.routed_scaling)
    count, offset, se = O.align(ids, s.E)
    _check_routing(gi, ids, w, count, offset, se)
    k = s.top_k
    tokens = (np.arange(s.M) if n_tok == 0
              else np.sort(np.random.default_rng(321).choice(s.M, n_tok, replace=False)))
    ref = _oracle_mx(d, tokens)
    _check_xq(gi, ref, tokens)
    ent = (tokens[:, None] * k + np.arange(k)[None, :]).ravel()
    g_midq = rows_by_entry(gi["midq"], gi["sorted_entry"], s.M * k)[ent]
    g_mids = rows_by_entry(gi["mids"], gi["sorted_entry"], s.M * k)[ent]
    r_midq = rows_by_entry(ref["midq"], ref["sorted_entry"], len(tokens) * k)
    r_mids = rows_by_entry(ref["mids"], ref["sorted_entry"], len(tokens) * k)
    _check_mid_mx(g_midq, g_mids, r_midq, r_mids)
    ydiff = _check_y(gi["y"][ent], ref["y"])
    ndiff = _check_out(gout[tokens], ref["out"])
    print(f"{name}: y differs in {ydiff}, out in {ndiff} of {ref['out'].size} elements")


def test_mx_and_e4m3_alternate_on_one_plan():
    """One plan switching formats between calls: each call matches its own
    oracle; the format is read at every call."""
    from quantized_moe_expert_route_amd.binding import MID_E4M3, MID_MXFP4

    shape = X.Shape(M=48, H=512, E=16, I=256, top_k=4)
    d = X.make_inputs(shape, "normal", 77)
    plan, g = None, None
    for fmt in (MID_MXFP4, MID_E4M3, MID_MXFP4, MID_E4M3):
        gout, gi, plan, g = _run_mx(d, plan=plan, g=g, fmt=fmt)
        s = d["shape"]
        ref = O.moe_forward(d["x"], d["logits"], d["w13"], d["s13"], d["w2"], d["s2"], s.top_k,
                            s.routed_scaling, None, mid_format="mxfp4" if fmt == MID_MXFP4 else "e4m3")
        assert np.array_equal(gout, ref["out"]), f"format {fmt}: output differs"


def test_mx_served_above_256_tokens_on_one_plan():
    """One plan at 300 tokens switching formats: the MXFP4 mid (quantized
    inside the 64-row-tile gate/up) and the E4M3 mid each match their own
    oracle; the stages launch what the plan reports."""
    import torch

    from quantized_moe_expert_route_amd.binding import MID_E4M3, MID_MXFP4

    shape = X.Shape(M=300, H=512, E=16, I=128, top_k=2)
    d = X.make_inputs(shape, "normal", 5)
    plan, g = None, None
    for fmt in (MID_MXFP4, MID_E4M3):
        gout, gi, plan, g = _run_mx(d, plan=plan, g=g, fmt=fmt)
        ref = O.moe_forward(d["x"], d["logits"], d["w13"], d["s13"], d["w2"], d["s2"], 2, 2.5, None,
                            mid_format="mxfp4" if fmt == MID_MXFP4 else "e4m3")
        if fmt == MID_MXFP4:
            _check_mid_mx(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
            assert plan.stage_launches(300)[3] == 0  # the mid quantization is inside gate/up
        _check_out(gout, ref["out"])
        assert np.array_equal(gout, ref["out"]), f"format {fmt}: output differs"
