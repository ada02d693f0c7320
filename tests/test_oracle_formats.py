"""Pins of the oracle's number formats against definitions and an independent library.

E4M3 is checked against torch.float8_e4m3fn, bf16 against torch's binary32 ->
bfloat16 cast; E2M1 and the MX scale rule against values derived by hand from
the OCP Microscaling v1.0 definitions.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F


def test_e2m1_decode_table():
    # OCP MX v1.0, FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.
    expect = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = F.e2m1_decode(np.arange(16))
    assert list(got[:8]) == expect
    assert list(got[8:]) == [-v for v in expect]
    assert np.signbit(got[8])


def test_e2m1_encode_roundtrip_and_ties():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(codes)), codes)
    # midpoints go to the even code
    mids = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in mids.items():
        assert F.e2m1_decode(F.e2m1_encode(np.array([v])))[0] == want, v
        assert F.e2m1_decode(F.e2m1_encode(np.array([-v])))[0] == -want, v
        above = np.nextafter(v, np.inf)
        below = np.nextafter(v, -np.inf)
        grid = F.E2M1_MAG
        hi = grid[grid > v].min()
        lo = grid[grid < v].max()
        assert F.e2m1_decode(F.e2m1_encode(np.array([above])))[0] == hi
        assert F.e2m1_decode(F.e2m1_encode(np.array([below])))[0] == lo


def test_e2m1_saturates():
    v = np.array([5.0001, 6.0, 6.5, 1e6, -7.0])
    assert list(F.e2m1_decode(F.e2m1_encode(v))) == [6.0, 6.0, 6.0, 6.0, -6.0]


def test_fp4_nibble_order():
    # element 2i in the low nibble: byte 0x21 -> [code 1, code 2] = [0.5, 1.0]
    assert list(F.unpack_fp4(np.array([0x21], np.uint8))) == [1, 2]
    c = np.random.default_rng(0).integers(0, 16, size=64).astype(np.uint8)
    assert np.array_equal(F.unpack_fp4(F.pack_fp4(c)), c)


def test_e8m0():
    assert F.e8m0_decode(np.array([127]))[0] == 1.0
    assert F.e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert F.e8m0_decode(np.array([254]))[0] == 2.0 ** 127
    with pytest.raises(ValueError):
        F.e8m0_decode(np.array([255]))


def _torch_e4m3_decode(codes):
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def test_e4m3_decode_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = _torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert F.E4M3_POS[-1] == 448.0 and len(F.E4M3_POS) == 127


def _torch_e4m3_encode(v32):
    t = torch.from_numpy(np.asarray(v32, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_vs_torch():
    rng = np.random.default_rng(1)
    pos = F.E4M3_POS
    mids = (pos[:-1] + pos[1:]) / 2  # every midpoint (exact in binary32)
    vals = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000), rng.normal(0, 0.01, 5000),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        pos, -pos, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -9 * 0.5],
    ]).astype(np.float32)
    ours = F.e4m3_encode(vals.astype(np.float64))
    ref = _torch_e4m3_encode(vals)
    assert np.array_equal(F.e4m3_decode(ours), F.e4m3_decode(ref))
    # saturation (torch would give NaN above its rounding range)
    assert F.e4m3_decode(F.e4m3_encode(np.array([464.0, 500.0, 1e30, -1e30]))).tolist() == \
        [448.0, 448.0, 448.0, -448.0]


def test_bf16_vs_torch_single_rounding():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.normal(0, 1, 50000), rng.normal(0, 1e-3, 5000) * 1e-30,
                        rng.normal(0, 1e30, 5000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_encode(v.astype(np.float64)), ref)
    assert np.array_equal(F.bf16_decode(ref), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_bf16_no_double_rounding():
    # 1 + 2^-8 + 2^-30: above the midpoint between 1 and 1 + 2^-7, so it rounds
    # up; a binary32 step first would land on the midpoint and tie to 1.0.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_encode(np.array([v]))[0] == 0x3F81
    assert F.bf16_encode(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80  # exact tie -> even
    assert F.bf16_encode(np.array([1e40]))[0] == 0x7F80  # overflow -> inf


def test_mx_scale_rule_closed_forms():
    def q(block):
        x = np.zeros(32)
        x[:len(block)] = block
        return F.mx_fp4_quantize(x[None, :])

    # amax 1.0: floor(log2 1) - 2 = -2 -> code 125; 1.0 * 4 = 4 -> code 6
    c, s = q([1.0])
    assert s[0, 0] == 125 and c[0, 0] == 6
    # amax 6: exponent 2 - 2 = 0 -> code 127, element 6 -> code 7
    c, s = q([6.0, -3.0])
    assert s[0, 0] == 127 and c[0, 0] == 7 and c[0, 1] == 8 | 5
    # amax 7: same scale, 7 saturates to 6
    c, s = q([7.0])
    assert s[0, 0] == 127 and c[0, 0] == 7
    # amax 0.75: floor(log2 .75) = -1 -> exponent -3 -> code 124; .75 * 8 = 6
    c, s = q([0.75, 0.1])
    assert s[0, 0] == 124 and c[0, 0] == 7
    # 0.1 * 8 = 0.8 -> nearest 1.0 (code 2)
    assert c[0, 1] == 2
    # all-zero block: scale code 0, zero elements
    c, s = q([])
    assert s[0, 0] == 0 and np.all(F.e2m1_decode(c) == 0)


def test_mx_identity_on_grid():
    # values on the E2M1 grid whose block max is 4 or 6 have scale 1 and
    # quantize to themselves
    rng = np.random.default_rng(3)
    x = F.e2m1_decode(rng.integers(0, 16, size=(8, 128)))
    x[:, ::32] = 4.0
    c, s = F.mx_fp4_quantize(x)
    assert np.all(s == 127)
    assert np.array_equal(F.mx_fp4_decode(c, s), x)


def test_fp8_block_quantize_identity_and_scale():
    rng = np.random.default_rng(4)
    h = F.e4m3_decode(rng.integers(0, 126, size=(4, 256)) | (rng.integers(0, 2, size=(4, 256)) << 7))
    h[:, 0] = 448.0
    h[:, 128] = -448.0
    c, s = F.fp8_block_quantize(h.astype(np.float32))
    assert np.all(s == 1.0)
    assert np.array_equal(F.e4m3_decode(c), h)
    # amax 2.0 -> scale fl32(2/448); values scale by 224 (up to rounding)
    z = np.zeros((1, 128), np.float32)
    z[0, 3] = 2.0
    c, s = F.fp8_block_quantize(z)
    assert s[0, 0] == np.float32(2.0) / np.float32(448.0)
    assert F.e4m3_decode(c)[0, 3] == 448.0
    # zero block
    c, s = F.fp8_block_quantize(np.zeros((1, 128), np.float32))
    assert s[0, 0] == 0 and np.all(c & 0x7F == 0)


def _fl32_exact(q):
    """Nearest binary32 to the rational q (ties to the even significand), by
    exact comparison with the neighbours of a first guess."""
    from fractions import Fraction

    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - q), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


@pytest.mark.parametrize("amax_bits,h_bits", [(1080849678, 1052916628), (1076355820, 1066788362),
                                             (1081177291, 990226892), (1057125413, 1029067032)])
def test_fp8_block_quantize_divides(amax_bits, h_bits):
    """Codes come from the IEEE quotient fl32(h / s), not from h * fl32(1/s):
    on these (amax, h) pairs the two land on opposite sides of an E4M3
    rounding midpoint (pairs found by a seeded search over midpoints). The
    expected code is derived independently: the exact rational quotient
    rounded to binary32 by comparison, then torch's E4M3 cast."""
    import torch
    from fractions import Fraction

    amax = np.array([amax_bits], np.uint32).view(np.float32)[0]
    h = np.array([h_bits], np.uint32).view(np.float32)[0]
    block = np.zeros((1, 128), np.float32)
    block[0, 0] = amax
    block[0, 5] = h
    c, s = F.fp8_block_quantize(block)
    s_ref = _fl32_exact(Fraction(float(amax)) / 448)
    assert s[0, 0] == s_ref
    q = _fl32_exact(Fraction(float(h)) / Fraction(float(s_ref)))
    want = torch.tensor([float(q)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
    assert int(c[0, 5]) == want
    recip = np.float32(h * np.float32(np.float32(1.0) / s_ref))
    assert int(F.e4m3_encode(np.float64(recip))) != want, "the case must tell division from reciprocal"
