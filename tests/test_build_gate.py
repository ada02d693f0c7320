"""Build gate: every kernel of this build compiles for gfx950 with no scratch
memory and no vector-register spills (read from the compiler's resource
remarks of our own sources). Scalar registers the compiler parks in lanes of
a vector register (v_writelane / v_readlane) touch no memory and are
allowed; any spill that needs scratch memory is not."""

from quantized_moe_expert_route_amd import build


def test_no_scratch_no_spills():
    usage = build.resource_usage()
    assert usage, "no kernels found"
    bad = {k: v for k, v in usage.items() if v.get("ScratchSize", 0) or v.get("VGPRsSpill", 0)}
    assert not bad, f"kernels with scratch or spills: {bad}"
    for name, v in usage.items():
        assert v.get("VGPRs", 0) + v.get("AGPRs", 0) <= 512, name
