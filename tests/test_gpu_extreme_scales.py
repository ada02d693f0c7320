"""GPU parity at the ends of the formats' ranges (fixtures.make_extreme_inputs):
E8M0 scale byte 0 (2^-127, below binary32's normal range) on x and on the
down weights, bf16-subnormal x, down weights that widen to bf16 subnormals,
and magnitudes near 2^+-100, on the small, mid-range and large paths and
with the MXFP4 mid. Token groups never share an expert, so each group is
checked against its own magnitude."""

import numpy as np
import pytest

from oracle import formats as F
from quantized_moe_expert_route_amd import fixtures as X

from moe_gpu import oracle, run
from test_gpu_parity import _check_mid, _check_routing, _check_xq, _check_y

pytestmark = pytest.mark.gpu


def _check_out_by_group(gout, rout, M):
    """Per token group (its own RMS): max-abs error and differing elements."""
    grp = np.arange(M) % 4
    total = 0
    for g in range(4):
        a, b = gout[grp == g], rout[grp == g]
        ga, rb = F.bf16_decode(a), F.bf16_decode(b)
        rms = float(np.sqrt(np.mean(rb * rb)))
        err = float(np.max(np.abs(ga - rb))) / rms
        nd = int(np.count_nonzero(a != b))
        total += nd
        print(f"group {g}: RMS {rms:.3e}, max-abs/RMS {err:.3e}, {nd} of {a.size} bf16 elements differ")
        assert np.all(np.isfinite(ga)), f"group {g}: non-finite outputs"
        assert err <= 1e-2, f"group {g}: max-abs error {err:.3e} x RMS"
    return total


@pytest.mark.parametrize("M", [4, 8, 40, 300])  # routing gate/up with the mid quantized in down, small, mid-range and large paths
def test_extreme_scales(M):
    shape = X.Shape(M=M, H=512, E=16, I=128, top_k=2)
    d = X.make_extreme_inputs(shape, 7)
    gout, gi = run(d)
    ref = oracle(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    assert (ref["xs"] == 0).any() and (d["s2"] == 0).any(), "the inputs reach scale byte 0"
    _check_mid(gi["midq"], gi["mids"], ref["midq"], ref["mids"])
    if gi["y"] is not None:  # (the combine inside the down launch: no y)
        _check_y(gi["y"], ref["y"])
    nd = _check_out_by_group(gout, ref["out"], M)
    print(f"M={M}: {nd} differing bf16 elements in all")


@pytest.mark.parametrize("M", [8, 40])
def test_extreme_scales_mxfp4_mid(M):
    from test_gpu_a4w4 import _oracle_mx, _run_mx

    shape = X.Shape(M=M, H=512, E=16, I=128, top_k=2)
    d = X.make_extreme_inputs(shape, 8)
    gout, gi, _, _ = _run_mx(d)
    ref = _oracle_mx(d)
    _check_routing(gi, ref["ids"], ref["w"], ref["count"], ref["offset"], ref["sorted_entry"])
    _check_xq(gi, ref)
    assert np.array_equal(F.unpack_fp4(gi["midq"]), ref["midq"]), "MXFP4 mid codes differ"
    assert np.array_equal(gi["mids"], ref["mids"]), "MXFP4 mid scale bytes differ"
    _check_y(gi["y"], ref["y"])
    _check_out_by_group(gout, ref["out"], M)
