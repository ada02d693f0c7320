"""The one-time packing of the gate/up weights (moe_pack_w13) on the GPU:
the packed bytes are the documented permutation of the row-major inputs,
written out here with numpy reshapes, and nothing else."""

import numpy as np
import pytest


def expected_packed(w13, s13):
    """w13 [E, 2I, H/2] -> [E*2I/16][H/128][4 g][16 r][16 B];
    s13 [E, 2I, H/32] -> [E*2I/16][H/512][4 g][16 r][4 j], byte j of (g, r)
    being MX block 16 kq + 4 j + g of the row."""
    E, R, Hb = w13.shape
    nrb, nks, nkq = E * R // 16, Hb // 64, Hb // 256
    wp = w13.reshape(nrb, 16, nks, 4, 16).transpose(0, 2, 3, 1, 4)
    sp = s13.reshape(nrb, 16, nkq, 4, 4).transpose(0, 2, 4, 1, 3)
    return np.ascontiguousarray(wp).ravel(), np.ascontiguousarray(sp).ravel()


@pytest.mark.gpu
@pytest.mark.parametrize("E,I,H", [(3, 128, 512), (2, 384, 1536), (5, 256, 1024)])
def test_pack_w13_is_the_documented_permutation(E, I, H):
    import torch

    from quantized_moe_expert_route_amd.binding import pack_w13

    rng = np.random.default_rng(E * 1000 + I + H)
    w13 = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    s13 = rng.integers(0, 256, (E, 2 * I, H // 32), dtype=np.uint8)
    dev = torch.device("cuda", 0)
    wt, st = torch.from_numpy(w13).to(dev), torch.from_numpy(s13).to(dev)
    wp, sp = pack_w13(wt, st)
    torch.cuda.synchronize()
    ew, es = expected_packed(w13, s13)
    np.testing.assert_array_equal(wp.cpu().numpy().ravel(), ew)
    np.testing.assert_array_equal(sp.cpu().numpy().ravel(), es)
    # the inputs are left as they were
    np.testing.assert_array_equal(wt.cpu().numpy(), w13)
    np.testing.assert_array_equal(st.cpu().numpy(), s13)


def test_expected_layout_places_a_known_byte():
    """The numpy statement of the layout, checked on single marked bytes."""
    E, I, H = 2, 128, 1024
    w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
    s13 = np.zeros((E, 2 * I, H // 32), np.uint8)
    e, row, ks, g, b = 1, 37, 5, 2, 9      # byte 64 ks + 16 g + b of the row
    w13[e, row, 64 * ks + 16 * g + b] = 7
    kq, j, gs = 1, 3, 1                    # MX block 16 kq + 4 j + gs
    s13[e, row, 16 * kq + 4 * j + gs] = 9
    ew, es = expected_packed(w13, s13)
    rb, r = (e * 2 * I + row) // 16, row % 16
    assert ew[(((rb * (H // 128) + ks) * 4 + g) * 16 + r) * 16 + b] == 7 and ew.sum() == 7
    assert es[(((rb * (H // 512) + kq) * 4 + gs) * 16 + r) * 4 + j] == 9 and es.sum() == 9


def expected_packed_w2(w2, s2):
    """w2 [E, H, I/2] -> [E*H/16][I/128][4 g][16 r][16 B];
    s2 [E, H, I/32] -> [E*H/16][4 g][16 r][4 ks], byte ks of (g, r) being MX
    block 4 ks + g of the row for ks < I/128, zero above."""
    E, H, Ib = w2.shape
    nrb, nks = E * H // 16, Ib // 64
    wp = w2.reshape(nrb, 16, nks, 4, 16).transpose(0, 2, 3, 1, 4)
    sp = np.zeros((nrb, 4, 16, 4), np.uint8)
    sp[..., :nks] = s2.reshape(nrb, 16, nks, 4).transpose(0, 3, 1, 2)
    return np.ascontiguousarray(wp).ravel(), sp.ravel()


@pytest.mark.gpu
@pytest.mark.parametrize("E,I,H", [(3, 128, 512), (2, 384, 1536), (5, 256, 1024), (2, 512, 512)])
def test_pack_w2_is_the_documented_permutation(E, I, H):
    import torch

    from quantized_moe_expert_route_amd.binding import pack_w2

    rng = np.random.default_rng(E * 999 + I + H)
    w2 = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    s2 = rng.integers(0, 256, (E, H, I // 32), dtype=np.uint8)
    dev = torch.device("cuda", 0)
    wt, st = torch.from_numpy(w2).to(dev), torch.from_numpy(s2).to(dev)
    wp, sp = pack_w2(wt, st)
    torch.cuda.synchronize()
    ew, es = expected_packed_w2(w2, s2)
    np.testing.assert_array_equal(wp.cpu().numpy().ravel(), ew)
    np.testing.assert_array_equal(sp.cpu().numpy().ravel(), es)
    np.testing.assert_array_equal(wt.cpu().numpy(), w2)
    np.testing.assert_array_equal(st.cpu().numpy(), s2)


def test_expected_w2_layout_places_a_known_byte():
    E, I, H = 2, 256, 512
    w2 = np.zeros((E, H, I // 2), np.uint8)
    s2 = np.zeros((E, H, I // 32), np.uint8)
    e, row, ks, g, b = 1, 300, 1, 3, 11    # byte 64 ks + 16 g + b of output column `row`
    w2[e, row, 64 * ks + 16 * g + b] = 5
    s2[e, row, 4 * ks + g] = 6             # MX block 4 ks + g
    ew, es = expected_packed_w2(w2, s2)
    rb, r = (e * H + row) // 16, row % 16
    assert ew[(((rb * (I // 128) + ks) * 4 + g) * 16 + r) * 16 + b] == 5 and ew.sum() == 5
    assert es[((rb * 4 + g) * 16 + r) * 4 + ks] == 6 and es.sum() == 6
