"""GPU parity of the shared expert fused as the last expert and the last slot
(moe_plan_set_shared_slot), against the oracle's shared_slot routing: the
same bars as the routed call (ids, weights and sort bit-exact, mid within one
E4M3 step, output within 1e-2 x RMS), on the small, mid-range and large
paths and at the pages' model shape (256 routed experts + the shared one as
expert 256, top-9)."""

import numpy as np
import pytest

from quantized_moe_expert_route_amd import fixtures as X

from moe_gpu import make_plan, oracle, run, upload
from test_gpu_parity import _check_mid, _check_out, _check_routing, _check_xq

pytestmark = pytest.mark.gpu


def _run_slot(d):
    plan = make_plan(d["shape"])
    plan.set_shared_slot(True)
    return run(d, plan=plan)


@pytest.mark.parametrize("M,H,E,I,k,kind", [
    (4, 512, 17, 128, 3, "normal"),      # small path
    (16, 512, 65, 256, 9, "ties"),       # small path, ties among the routed logits
    (40, 1024, 33, 256, 5, "zipf"),      # mid-range path
    (300, 512, 17, 128, 3, "normal"),    # large path
])
def test_shared_slot_shapes(M, H, E, I, k, kind):
    shape = X.Shape(M=M, H=H, E=E, I=I, top_k=k)
    d = X.make_inputs(shape, kind, 3000 + M)
    gout, gi = _run_slot(d)
    ref = oracle(d, shared_slot=True)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    assert np.all(gi["ids"][:, -1] == E - 1) and np.all(gi["w"][:, -1] == 1.0)
    assert gi["count"][E - 1] == M
    _check_xq(gi, ref)
    _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    _check_out(gout, ref["out"])


@pytest.mark.parametrize("name", ["c1s", "c2s"])
def test_shared_slot_full_size(name):
    d = X.make_inputs(name)
    assert X.WORKLOADS[name].shared_slot
    gout, gi = _run_slot(d)
    ref = oracle(d, shared_slot=True)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    ndiff = _check_out(gout, ref["out"])
    print(f"{name}: {ndiff} of {ref['out'].size} bf16 outputs differ")


def test_shared_slot_last_logits_column_not_read():
    """Changing the shared expert's logits column changes nothing."""
    import torch

    shape = X.Shape(M=8, H=512, E=17, I=128, top_k=3)
    d = X.make_inputs(shape, "normal", 55)
    a, _ = _run_slot(d)
    d2 = dict(d)
    lg = d["logits"].copy()
    lg[:, -1] = 1e30
    d2["logits"] = lg
    b, _ = _run_slot(d2)
    assert np.array_equal(a, b)
    torch.cuda.synchronize()


def test_shared_slot_argument_checks():
    """The setter refuses what it cannot serve, before any call."""
    from quantized_moe_expert_route_amd.binding import MOE_ERR_INVALID_ARG, MoeError

    plan = make_plan(X.Shape(M=4, H=512, E=8, I=128, top_k=1))
    with pytest.raises(MoeError) as ei:
        plan.set_shared_slot(True)  # top_k 1: no routed slot left
    assert ei.value.status == MOE_ERR_INVALID_ARG
    plan = make_plan(X.Shape(M=4, H=512, E=8, I=128, top_k=2, shared_I=128))
    with pytest.raises(MoeError) as ei:
        plan.set_shared_slot(True)  # a block-FP8 shared expert is bound to this shape
    assert ei.value.status == MOE_ERR_INVALID_ARG
    plan.set_shared_slot(False)


@pytest.mark.parametrize("M", [4, 40])
def test_shared_slot_with_mxfp4_mid(M):
    """The two plan options together: the shared expert as the last slot and
    the MXFP4 mid hand-off (w2 packed by pack_w2)."""
    import torch

    from oracle import formats as F
    from quantized_moe_expert_route_amd.binding import MID_MXFP4, layout_for, pack_w2

    shape = X.Shape(M=M, H=512, E=17, I=256, top_k=5)
    d = X.make_inputs(shape, "normal", 4100 + M)
    g = upload(d)
    plan = make_plan(shape)
    plan.set_shared_slot(True)
    plan.set_mid_format(MID_MXFP4)
    plan.set_weight_layout(layout_for(MID_MXFP4))
    w2p, s2p = pack_w2(g["w2"], g["s2"])
    out = torch.full((M, shape.H), -1, dtype=torch.int16, device="cuda")
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], w2p, s2p, out)
    torch.cuda.synchronize()
    ref = oracle(d, shared_slot=True, mid_format="mxfp4")
    midq = plan.view("midq", torch.uint8, (M * shape.top_k, shape.I // 2)).cpu().numpy()
    assert np.array_equal(F.unpack_fp4(midq), ref["midq"])
    _check_out(out.cpu().numpy().view(np.uint16), ref["out"])
