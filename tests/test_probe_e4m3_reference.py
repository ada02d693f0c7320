"""The probe library's reference encoders (host builds) equal the oracle's:
qmoe_probe_e4m3_ref equals e4m3_encode on every rounding boundary of the
E4M3 grid and its fp32 neighbours, on every grid value, and on random fp32
values of both signs below 464; qmoe_probe_e2m1_ref equals e2m1_encode the
same way below 8 (saturation from 6 on). The GPU tests in
test_gpu_mfma_probe.py then compare the hardware conversions with these
references on every fp32 of those ranges. No GPU is needed here: the
functions are host code."""

import ctypes
import os

import numpy as np
import pytest

from oracle import formats as F

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libmfma_probe.so")


def _ref(name):
    if not os.path.exists(LIB):
        pytest.skip(f"{LIB} is not built (__graft_entry__.build() builds it)")
    L = ctypes.CDLL(LIB)
    f = getattr(L, name)
    f.argtypes = [ctypes.c_float]
    f.restype = ctypes.c_uint32
    return np.vectorize(lambda v: f(float(v)), otypes=[np.uint32])


@pytest.fixture(scope="module")
def ref():
    return _ref("qmoe_probe_e4m3_ref")


def _fp32_neighbours(v):
    v = np.asarray(v, np.float32)
    up = np.nextafter(v, np.float32(np.inf))
    dn = np.nextafter(v, np.float32(-np.inf))
    return np.concatenate([dn, v, up])


def test_reference_matches_oracle_on_boundaries_and_samples(ref):
    grid = F.E4M3_POS  # the 127 non-negative values, ascending
    mids = (grid[:-1] + grid[1:]) / 2  # rounding boundaries (exact in fp32)
    pts = [_fp32_neighbours(grid.astype(np.float32)), _fp32_neighbours(mids.astype(np.float32)),
           _fp32_neighbours(np.float32([448.0, 456.0, 463.99997, 2.0 ** -10, 2.0 ** -11, 2.0 ** -126]))]
    rng = np.random.default_rng(7)
    pts.append(rng.uniform(0, 464, 20000).astype(np.float32))
    pts.append((2.0 ** rng.uniform(-20, 8.8, 20000)).astype(np.float32))
    v = np.concatenate(pts)
    v = v[(v >= 0) & (v < 464)]
    v = np.concatenate([v, -v])
    got = ref(v)
    want = F.e4m3_encode(v.astype(np.float64)).astype(np.uint32)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(v[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]


def test_e2m1_reference_matches_oracle_on_boundaries_and_samples():
    ref = _ref("qmoe_probe_e2m1_ref")
    grid = F.E2M1_MAG
    mids = (grid[:-1] + grid[1:]) / 2  # 0.25, 0.75, ..., 5: the rounding boundaries
    pts = [_fp32_neighbours(grid.astype(np.float32)), _fp32_neighbours(mids.astype(np.float32)),
           _fp32_neighbours(np.float32([7.0, 7.9999995, 2.0 ** -126, 2.0 ** -149]))]
    rng = np.random.default_rng(11)
    pts.append(rng.uniform(0, 8, 20000).astype(np.float32))
    pts.append((2.0 ** rng.uniform(-30, 2.99, 5000)).astype(np.float32))
    v = np.concatenate(pts)
    v = v[(v >= 0) & (v < 8)]
    v = np.concatenate([v, -v])
    got = ref(v)
    want = F.e2m1_encode(v.astype(np.float64)).astype(np.uint32)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(v[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]
    # the sign is kept on values that round to zero
    assert int(ref(np.float32(-0.0))) == 8 and int(ref(np.float32(-0.1))) == 8
