"""Host-side checks of the C ABI: the library loads, exports every function
that include/*.h declares, and validates shapes and arguments before touching
a device. No compute call is made here."""

import ctypes
import glob
import os
import re

import pytest

from quantized_moe_expert_route_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"moe_forward", "moe_plan_create", "moe_plan_set_workspace"} <= names
    L = B.lib()
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, f"not exported: {missing}"


def test_status_strings_and_stages():
    assert B.status_str(B.MOE_OK) == "ok"
    for st in range(1, 6):
        assert B.status_str(st) and B.status_str(st) != "ok"
    assert B.stage_names() == ["route", "align", "gate_up", "act_quant", "shared", "down", "combine"]
    assert B.lib().moe_stage_name(99) is None


@pytest.mark.parametrize("kw,status", [
    (dict(M=4, H=6144, E=256, I=256, top_k=8), B.MOE_OK),
    (dict(M=0, H=6144, E=256, I=256, top_k=8), B.MOE_OK),
    (dict(M=4, H=6144, E=256, I=256, top_k=300), B.MOE_ERR_INVALID_ARG),      # k > E
    (dict(M=-1, H=6144, E=256, I=256, top_k=8), B.MOE_ERR_INVALID_ARG),
    (dict(M=4, H=6144, E=256, I=256, top_k=8, routed_scaling=0.0), B.MOE_ERR_INVALID_ARG),
    (dict(M=4, H=6144 + 128, E=256, I=256, top_k=8), B.MOE_ERR_UNSUPPORTED),  # H % 512
    (dict(M=4, H=6144, E=256, I=200, top_k=8), B.MOE_ERR_UNSUPPORTED),        # I % 128
    (dict(M=4, H=6144, E=256, I=1024, top_k=8), B.MOE_ERR_UNSUPPORTED),       # I > 512
    (dict(M=4, H=6144, E=2048, I=256, top_k=8), B.MOE_ERR_UNSUPPORTED),       # E > 1024
    (dict(M=4, H=6144, E=256, I=256, top_k=17), B.MOE_ERR_UNSUPPORTED),       # k > 16
    (dict(M=4, H=6144, E=256, I=256, top_k=8, shared_I=100), B.MOE_ERR_UNSUPPORTED),
    (dict(M=1 << 20, H=4096, E=256, I=256, top_k=8), B.MOE_ERR_UNSUPPORTED),  # M * H / 2 >= 2^31
    (dict(M=1 << 19, H=8192, E=256, I=256, top_k=1), B.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    if status == B.MOE_OK:
        assert B.shape_workspace_bytes(**kw) % 256 == 0
    else:
        with pytest.raises(B.MoeError) as e:
            B.shape_workspace_bytes(**kw)
        assert e.value.status == status


def test_workspace_holds_the_documented_intermediates():
    M, H, E, I, k, Is = 4096, 6144, 256, 512, 8, 512
    nbytes = B.shape_workspace_bytes(M, H, E, I, k, 2.5, Is)
    n = M * k
    documented = (4 * n * 3 + 4 * E + 4 * (E + 1) + M * H // 2 + M * H // 32 + n * I + 4 * n * I // 128
                  + 4 * n * H + 3 * M * H + 4 * M * H // 128 + 3 * M * Is + 4 * M * Is // 128 + 4 * M * H)
    assert nbytes >= documented
    assert nbytes < documented * 1.5


def test_null_and_unbound_arguments_fail_before_any_device_work():
    L = B.lib()
    out = ctypes.c_void_p()
    assert L.moe_plan_create(None, ctypes.byref(out)) == B.MOE_ERR_INVALID_ARG
    s = B.moe_shape(4, 512, 16, 128, 2, 2.5, 0)
    assert L.moe_plan_create(ctypes.byref(s), None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_forward(None, 4, None, None, None, None, None, None, None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_layout(None, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_set_stage_events(None, None, 0) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_workspace_bytes(None) == 0
    assert L.moe_plan_set_mid_format(None, B.MID_MXFP4) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_set_shared_slot(None, 1) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_set_shared(None, None, None, None, None, None, 0, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_shared_pack_bytes(None) == 0
    assert L.moe_plan_set_weight_layout(None, B.LAYOUT_W13_PACKED) == B.MOE_ERR_INVALID_ARG
    assert L.moe_plan_set_tp_exchange(None, None) == B.MOE_ERR_INVALID_ARG
    L.moe_plan_destroy(None)


def test_pack_w13_validates_before_any_device_work():
    L = B.lib()
    a, b, c, d = 0x10000, 0x20000, 0x30000, 0x40000  # never dereferenced: every case fails first
    assert L.moe_pack_w13(None, b, 4, 128, 512, c, d, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_w13(a, b, 4, 128, 512, None, d, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_w13(a, b, 0, 128, 512, c, d, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_w13(a, b, 4, 128, 640, c, d, None) == B.MOE_ERR_UNSUPPORTED   # H % 512
    assert L.moe_pack_w13(a, b, 4, 192, 512, c, d, None) == B.MOE_ERR_UNSUPPORTED   # I % 128
    assert L.moe_pack_w13(a, b, 2048, 128, 512, c, d, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_w13(a + 8, b, 4, 128, 512, c, d, None) == B.MOE_ERR_INVALID_ARG  # misaligned
    # the packed weights would overlap the input
    assert L.moe_pack_w13(a, b, 4, 128, 512, a + 256, d, None) == B.MOE_ERR_INVALID_ARG
    # the down-weight packing validates the same way
    assert L.moe_pack_w2(None, b, 4, 128, 512, c, d, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_w2(a, b, 4, 128, 640, c, d, None) == B.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_w2(a, b, 4, 640, 512, c, d, None) == B.MOE_ERR_UNSUPPORTED    # I > 512
    assert L.moe_pack_w2(a, b + 4, 4, 128, 512, c, d, None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_pack_w2(a, b, 4, 128, 512, c, a + 16, None) == B.MOE_ERR_INVALID_ARG  # overlap


def test_plan_needs_a_gfx950_device():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    s = B.moe_shape(4, 512, 16, 128, 2, 2.5, 0)
    out = ctypes.c_void_p()
    assert B.lib().moe_plan_create(ctypes.byref(s), ctypes.byref(out)) == B.MOE_ERR_DEVICE
    assert not out.value
    # host addresses are not device memory
    assert B.lib().moe_pack_w13(0x10000, 0x80000, 4, 128, 512, 0x100000, 0x180000, None) == B.MOE_ERR_DEVICE


def test_header_compiles_as_plain_c(tmp_path):
    """include/qmoe.h is a C ABI: it compiles as C99 (pedantic) and as C++."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "use.c"
    src.write_text('#include "qmoe.h"\nint main(void) { moe_plan* p = 0; '
                   'return (int)moe_plan_set_mid_format(p, MOE_MID_MXFP4) + (int)moe_plan_set_shared_slot(p, 1); }\n')
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only"],
                ["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c++"]):
        r = subprocess.run(cmd + ["-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "qmoe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
    assert B.lib().moe_forward_noalloc(None, 4, None, None, None, None, None, None, None, None) == B.MOE_ERR_INVALID_ARG


def test_plan_call_checks_reject_bad_tensors():
    """The binding checks every tensor a call passes before the library sees
    its bare pointer (host logic only: a plan object without a device plan)."""
    import torch

    M, H, E, I = 4, 512, 16, 128
    p = B.Plan.__new__(B.Plan)
    p._h = ctypes.c_void_p()
    p.shape = B.moe_shape(M, H, E, I, 2, 2.5, 0)
    p.device = torch.device("cpu")
    p._layout = B.LAYOUT_W13_PACKED
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    good = dict(x=torch.zeros((M, H), dtype=torch.int16), logits=torch.zeros((M, E)),
                w13=u8(E * 2 * I * H // 2), s13=u8(E * 2 * I * H // 32), w2=u8(E * H * I // 2), s2=u8(E * H * I // 32),
                out=torch.zeros((M, H), dtype=torch.bfloat16))
    p._check_call(M, **good)
    p._check_call(2, **dict(good, x=torch.zeros((2, H), dtype=torch.int16)))  # rows >= the call's M suffice
    bad = [
        (M, dict(x=torch.zeros((M - 1, H), dtype=torch.int16))),           # fewer rows than M
        (M, dict(x=torch.zeros((H, M), dtype=torch.int16).t())),           # strided view
        (M, dict(logits=torch.zeros((M, E), dtype=torch.float64))),       # wrong dtype
        (M, dict(logits=torch.zeros((M, E + 1)))),                        # wrong width
        (M, dict(out=torch.zeros((M, H), dtype=torch.int32))),
        (M, dict(w13=u8(E * 2 * I * H // 2 - 1))),
        (M, dict(w2=u8(E * H * I // 2 + 16))),
        (M, dict(s2=u8(E * H * 16))),                                     # packed scales, row-major declared
        (M + 1, dict(x=torch.zeros((M + 1, H), dtype=torch.int16))),      # beyond the plan's M
    ]
    for m, change in bad:
        with pytest.raises(ValueError):
            p._check_call(m, **dict(good, **change))
    with pytest.raises(TypeError):
        p._check_call(M, **dict(good, x=None))
    p._layout = B.LAYOUT_W13_PACKED | B.LAYOUT_W2_PACKED
    p._check_call(M, **dict(good, s2=u8(E * H * 16)))
