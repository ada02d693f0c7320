"""Helpers of the GPU tests: run the HIP path through the C ABI binding and
read back every intermediate it leaves in the workspace; compare with the
oracle stage by stage."""

from __future__ import annotations

import numpy as np

from oracle import formats as F
from oracle import moe as O


def upload(d):
    import torch

    dev = torch.device("cuda", 0)
    g = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
         for k in ("logits", "w13", "s13", "w2", "s2") if k in d}
    g["x"] = torch.from_numpy(np.ascontiguousarray(d["x"]).view(np.int16)).to(dev)
    if "w13" in g:
        from quantized_moe_expert_route_amd.binding import pack_w13

        # the call reads gate/up weights in the library's packed layout
        g["w13"], g["s13"] = pack_w13(g["w13"], g["s13"])
    if d["shape"].shared_I:
        for k in ("ws13", "ss13", "ws2", "ss2"):
            g[k] = torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
    return g


def make_plan(shape, M_max=None):
    from quantized_moe_expert_route_amd.binding import Plan

    s = shape
    return Plan(s.M if M_max is None else M_max, s.H, s.E, s.I, s.top_k, s.routed_scaling, s.shared_I)


def run(d, plan=None, g=None, M=None):
    """One call on GPU; returns (out bits [M, H] uint16, intermediates dict of numpy)."""
    import torch

    s = d["shape"]
    M = s.M if M is None else M
    if g is None:
        g = upload(d)
    if plan is None:
        plan = make_plan(s)
        if s.shared_I:
            plan.set_shared(g["ws13"], g["ss13"], g["ws2"], g["ss2"])
    out = torch.full((max(M, 1), s.H), -1, dtype=torch.int16, device=g["x"].device)
    plan.forward(g["x"], g["logits"], g["w13"], g["s13"], g["w2"], g["s2"], out, M=M)
    torch.cuda.synchronize()
    return out[:M].cpu().numpy().view(np.uint16), read_intermediates(plan, s, M)


def y_written(plan, M):
    """Whether the call wrote y: its combine stage has a launch of its own
    (besides the tensor-parallel exchange, when that is on)."""
    tp = 1 if getattr(plan, "_tpx", None) is not None else 0
    return plan.stage_launches(M)[6] > tp


def read_intermediates(plan, s, M):
    import torch

    k, n, I, H, E = s.top_k, M * s.top_k, s.I, s.H, s.E
    v = plan.view
    r = {
        "ids": v("topk_ids", torch.int32, (M, k)),
        "w": v("topk_w", torch.float32, (M, k)),
        "count": v("count", torch.int32, (E,)),
        "offset": v("offset", torch.int32, (E + 1,)),
        "sorted_entry": v("sorted_entry", torch.int32, (n,)),
        "xq": v("xq", torch.uint8, (M, H // 2)),
        "xs": v("xs", torch.uint8, (M, H // 32)),
        "midq": v("midq", torch.uint8, (n, I)),
        "mids": v("mids", torch.float32, (n, I // 128)),
        # y (the down output per entry) is in the workspace only when the
        # combine has a launch of its own (else it runs inside the down launch)
        "y": v("y", torch.float32, (n, H)) if y_written(plan, M) else None,
    }
    fused = shared_fused(s, M)
    if s.shared_I:
        Is = s.shared_I
        if fused:  # inside the small-token launches: E4M3 codes, no sh_y
            r["sh_xq"] = v("sh_xq", torch.uint8, (M, H))
            r["sh_hq"] = v("sh_hq", torch.uint8, (M, Is))
        else:
            r["sh_xq"] = v("sh_xq", torch.int8, (M, H // 128, 3, 128))
            r["sh_hq"] = v("sh_hq", torch.int8, (M, Is // 128, 3, 128))
            r["sh_y"] = v("sh_y", torch.float32, (M, H))
        r["sh_xs"] = v("sh_xs", torch.float32, (H // 128, M)).t()  # stored K-block major
        r["sh_hs"] = v("sh_hs", torch.float32, (Is // 128, M)).t()
    out = {key: None if t is None else t.cpu().numpy() for key, t in r.items()}
    if not fused:
        for key in ("sh_xq", "sh_hq"):
            if key in out:
                out[key] = digit_rows_to_codes(out[key])
    return out


def shared_fused(s, M, mid_format="e4m3"):
    """Whether a call of M tokens runs the block-FP8 shared expert inside the
    small-token launches (the library's rule: up to 16 tokens and 512 slots,
    the E4M3 mid, shared_I up to 512)."""
    return bool(s.shared_I) and s.shared_I <= 512 and M <= 16 and M * s.top_k <= 512 and mid_format == "e4m3"


def digit_rows_to_codes(d):
    """Shared-expert operands as stored, [rows, K/128, 3, 128] int8 digits d0,
    d1, d2 of v * 2^9 = d0 + 2^7 d1 + 2^14 d2, -> E4M3 codes [rows, K] (a zero
    value gives code 0; compare decoded values where -0 may occur)."""
    d = d.astype(np.int64)
    alpha = d[:, :, 0] + 128 * d[:, :, 1] + 16384 * d[:, :, 2]
    v = np.ldexp(alpha.astype(np.float64), -9).reshape(d.shape[0], -1)
    codes = F.e4m3_encode(v)
    assert np.array_equal(F.e4m3_decode(codes), v), "digits do not form E4M3 values"
    # the three digits of a value carry its sign
    s = np.sign(d)
    assert np.all((s[:, :, 0] * s[:, :, 1] >= 0) & (s[:, :, 0] * s[:, :, 2] >= 0) & (s[:, :, 1] * s[:, :, 2] >= 0))
    return codes


def oracle(d, tokens=None, **kw):
    """Oracle on all tokens, or only on `tokens` (per-token results are
    independent of the other tokens); keyword options go to moe_forward."""
    s = d["shape"]
    x, lg = d["x"], d["logits"]
    if tokens is not None:
        x, lg = x[tokens], lg[tokens]
    shared = (d["ws13"], d["ss13"], d["ws2"], d["ss2"]) if s.shared_I else None
    return O.moe_forward(x, lg, d["w13"], d["s13"], d["w2"], d["s2"], s.top_k, s.routed_scaling, shared, **kw)


def rows_by_entry(sorted_rows, sorted_entry, n):
    """Reorder rows given in sorted order into entry order (t*k + j)."""
    out = np.empty((n,) + sorted_rows.shape[1:], sorted_rows.dtype)
    out[sorted_entry] = sorted_rows
    return out


def e4m3_ulp_distance(a, b):
    """|difference| in E4M3 steps between codes of equal sign (or both zero)."""
    va, vb = F.e4m3_decode(a), F.e4m3_decode(b)
    ia = np.searchsorted(F.E4M3_POS, np.abs(va)) * np.sign(va)
    ib = np.searchsorted(F.E4M3_POS, np.abs(vb)) * np.sign(vb)
    return np.abs(ia - ib)


def out_error(gpu_bits, ref_bits):
    """(max |gpu - ref| / RMS(ref), number of differing elements)."""
    g = F.bf16_decode(gpu_bits)
    r = F.bf16_decode(ref_bits)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = float(np.max(np.abs(g - r))) if r.size else 0.0
    return (err / rms if rms > 0 else err), int(np.count_nonzero(gpu_bits != ref_bits))
