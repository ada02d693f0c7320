"""The tensor-parallel partial-sum exchange epilogue on one GPU: a loopback
rank whose peers' partials are zeros tagged with the call's epoch and whose
pushes go to scratch sinks (as the pages check their kernels on one GPU),
peers holding real partials, and a wait that gives up."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import moe as O
from quantized_moe_expert_route_amd import fixtures as X

from moe_gpu import make_plan, oracle, rows_by_entry, run, upload

pytestmark = pytest.mark.gpu


def _group(plan, tp, rank, epoch, peer_partials=None, peer_epoch=None, spin_limit=1 << 20):
    """Inbox with the peers' slots filled (zeros unless given) and tagged, and
    scratch sinks for this rank's pushes."""
    import torch

    s = plan.shape
    dev = torch.device("cuda", 0)
    inbox = torch.zeros((tp, s.M, s.H), dtype=torch.float64, device=dev)
    tags = torch.zeros((tp, s.M, s.H // 512), dtype=torch.int32, device=dev)
    for p in range(tp):
        if p == rank:
            continue
        if peer_partials is not None:
            inbox[p] = torch.from_numpy(peer_partials[p]).to(dev)
        tags[p] = epoch if peer_epoch is None else peer_epoch
    sinks = [None if p == rank else torch.full((s.M, s.H), np.nan, dtype=torch.float64, device=dev) for p in range(tp)]
    sink_tags = [None if p == rank else torch.zeros((s.M, s.H // 512), dtype=torch.int32, device=dev) for p in range(tp)]
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    plan.set_tp_exchange(tp, rank, epoch, inbox, tags, sinks, sink_tags, status, spin_limit)
    return inbox, tags, sinks, sink_tags, status


@pytest.mark.parametrize("name,tp", [("c1", 8), ("c2", 8), ("c3", 4)])
def test_loopback_zero_peers_equals_plain_call(name, tp):
    """Rank 0 alone: out equals the plain call's bits (so the oracle's); the
    rank's own slot holds the oracle's float64 partial (sampled tokens at c3);
    every sink received that partial with the epoch on every chunk."""
    import torch

    d = X.make_inputs(name)
    s = d["shape"]
    g = upload(d)
    plan = make_plan(s)
    plain, gi = run(d, plan=plan, g=g)
    epoch = 0x5EED0001
    inbox, tags, sinks, sink_tags, status = _group(plan, tp, 0, epoch)
    out = torch.full((s.M, s.H), -1, dtype=torch.int16, device="cuda")
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], g["w2"], g["s2"], out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert int(status.item()) == 0
    assert np.array_equal(got, plain), "exchange with zero peers differs from the plain call"
    own = inbox[0].cpu().numpy()
    tokens = np.arange(s.M) if s.M <= 16 else np.sort(np.random.default_rng(3).choice(s.M, 6, replace=False))
    ref = oracle(d, tokens)
    yr = ref["y"].reshape(len(tokens), s.top_k, s.H)
    P = O.combine_partial(ref["w"], yr)
    # the routed down's y may sit one fp32 step off where a 128-block sum
    # needs more than 24 bits inside the bf16 MFMA (at most 1e-4 of y): the
    # partial then moves by at most w * that step
    step = np.einsum("tj,tjh->th", np.abs(ref["w"]).astype(np.float64), np.abs(yr).astype(np.float64)) * 2.0 ** -23
    dev_ = np.abs(own[tokens] - P)
    ndiff = int(np.count_nonzero(own[tokens] != P))
    assert np.all(dev_ <= step) and ndiff <= max(1, 1e-4 * P.size), f"own partial off in {ndiff} elements"
    assert np.array_equal(O.tp_exchange_sum([own[tokens]] + [np.zeros_like(P)] * (tp - 1)), got[tokens])
    for p in range(1, tp):
        assert np.array_equal(sinks[p].cpu().numpy().view(np.uint64), own.view(np.uint64)), f"sink {p}"
        assert bool((sink_tags[p] == epoch).all()), f"sink tags {p}"
    plan.set_tp_exchange(None)


def test_peers_with_partials_rank_order():
    """Rank 2 of 4 with peers holding float64 partials (large and small
    magnitudes, so the order of the additions matters): out equals the
    oracle's exchange sum in rank order."""
    import torch

    shape = X.Shape(M=6, H=1024, E=16, I=128, top_k=4)
    d = X.make_inputs(shape, "normal", 21)
    g = upload(d)
    plan = make_plan(shape)
    rng = np.random.default_rng(9)
    peers = [rng.standard_normal((shape.M, shape.H)) * 10.0 ** rng.integers(-3, 3, size=(shape.M, shape.H))
             for _ in range(4)]
    inbox, *_, status = _group(plan, 4, 2, 77, peer_partials=peers)
    out = torch.full((shape.M, shape.H), -1, dtype=torch.int16, device="cuda")
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], g["w2"], g["s2"], out)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    own = inbox[2].cpu().numpy()
    ref = oracle(d)
    P = O.combine_partial(ref["w"], ref["y"].reshape(shape.M, shape.top_k, shape.H))
    assert np.array_equal(own.view(np.uint64), P.view(np.uint64))
    want = O.tp_exchange_sum([peers[0], peers[1], own, peers[3]])
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)


def test_stale_peer_tag_gives_up():
    """A peer slot tagged with an older epoch: the bounded wait (a small spin
    limit set from the host) gives up, the status word is set, the call ends."""
    import torch

    shape = X.Shape(M=2, H=512, E=8, I=128, top_k=2)
    d = X.make_inputs(shape, "normal", 22)
    g = upload(d)
    plan = make_plan(shape)
    *_, status = _group(plan, 2, 0, 9, peer_epoch=8, spin_limit=16)
    out = torch.zeros((shape.M, shape.H), dtype=torch.int16, device="cuda")
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], g["w2"], g["s2"], out)
    torch.cuda.synchronize()
    assert int(status.item()) == 1
