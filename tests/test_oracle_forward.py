"""Pins of the oracle forward: exact rational GEMM rows, an independent
per-token reference built from library routines, the interleave layout, and
exact invariants of the quantised pipeline."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from moe_expert_ffn_plan_amd import inputs
from oracle import formats as F
from oracle.forward import (deinterleave_gate_up, dequant_fp4_rows, dequant_fp8_rows, forward_ref,
                            forward_tokens, matmul_f32)


@pytest.fixture(scope="module")
def tiny():
    w = inputs.WORKLOADS["tiny"]
    return w, inputs.to_numpy(inputs.make_inputs(w))


def run(w, d, **over):
    args = dict(d)
    args.update(over)
    return forward_ref(args["x"], args["x_sf"], args["topk_idx"], args["topk_w"], args["w1"], args["w1_sf"],
                       args["w2"], args["w2_sf"], num_experts=w.num_experts, expert_begin=0, block_m=w.block_m)


def round_fraction_to_f32(q: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (nearest, ties to even)."""
    c = np.float32(float(q))
    lo, hi = np.nextafter(c, np.float32(-np.inf)), np.nextafter(c, np.float32(np.inf))
    best = min((abs(Fraction(float(v)) - q), int(np.float32(v).view(np.uint32)) & 1, v) for v in (lo, c, hi))
    return np.float32(best[2])


def test_gemm_rows_exact_rational(tiny):
    w, d = tiny
    a = dequant_fp8_rows(d["x"][:3], d["x_sf"][:3])
    b = dequant_fp4_rows(d["w1"][0][:24], d["w1_sf"][0][:24])
    z = matmul_f32(a, b)
    for i in range(3):
        for n in range(24):
            exact = sum(Fraction(float(p)) * Fraction(float(r)) for p, r in zip(a[i], b[n]))
            assert z[i, n] == round_fraction_to_f32(exact)


def test_deinterleave_layout():
    # W1 rows: [gate 0..7, up 0..7, gate 8..15, up 8..15, ...]
    I = 32
    z = np.arange(2 * I, dtype=np.float32)[None, :]
    g, u = deinterleave_gate_up(z)
    want_g = [16 * (c // 8) + c % 8 for c in range(I)]
    assert list(g[0]) == want_g and list(u[0]) == [v + 8 for v in want_g]


# ---- independent reference: per token, per valid hit, with torch library routines ----
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # OCP MX E2M1 magnitudes


def t_fp8(codes, sf):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.ldexp(torch.ones(sf.shape, dtype=torch.float64), torch.from_numpy(sf.astype(np.int64) - 127))
    return v * s.repeat_interleave(32, dim=-1)


def t_fp4(packed, sf):
    p = torch.from_numpy(packed).to(torch.int64)
    nib = torch.stack([p & 15, p >> 4], dim=-1).reshape(p.shape[0], -1)
    mag = torch.tensor(E2M1, dtype=torch.float64)[nib & 7]
    v = torch.where(nib >= 8, -mag, mag)
    s = torch.ldexp(torch.ones(sf.shape, dtype=torch.float64), torch.from_numpy(sf.astype(np.int64) - 127))
    return v * s.repeat_interleave(32, dim=-1)


def brute_code(amax):
    for c in range(255):
        if amax * 2.0 ** (127 - c) <= 448.0:
            return c
    return 254


def reference_token(t, d, E):
    H = d["x"].shape[1]
    acc = torch.zeros(H, dtype=torch.float32)
    x = t_fp8(d["x"][t:t + 1], d["x_sf"][t:t + 1])
    for j in range(d["topk_idx"].shape[1]):
        e = int(d["topk_idx"][t, j])
        if not 0 <= e < E:
            continue
        w1 = t_fp4(d["w1"][e], d["w1_sf"][e])
        rows = torch.arange(w1.shape[0])
        gate_rows = rows[(rows % 16) < 8]
        up_rows = rows[(rows % 16) >= 8]
        zg = (x @ w1[gate_rows].T).to(torch.float32)
        zu = (x @ w1[up_rows].T).to(torch.float32)
        g = zg.to(torch.bfloat16).to(torch.float64)
        u = zu.to(torch.bfloat16).to(torch.float32)
        s = torch.nn.functional.silu(g).to(torch.float32)
        h = (s * u) * torch.tensor(d["topk_w"][t, j], dtype=torch.float32)
        hb = h.reshape(-1, 32).to(torch.float64)
        codes = [brute_code(float(a)) for a in hb.abs().amax(dim=1)]
        inv = torch.tensor([2.0 ** (127 - c) for c in codes], dtype=torch.float64)
        q = (hb * inv[:, None]).to(torch.float32).to(torch.float8_e4m3fn)
        hdq = q.to(torch.float64) / inv[:, None]
        w2 = t_fp4(d["w2"][e], d["w2_sf"][e])
        y2 = (hdq.reshape(1, -1) @ w2.T).to(torch.float32).to(torch.bfloat16).to(torch.float32)
        acc = acc + y2[0]
    return acc.to(torch.bfloat16).to(torch.float32).numpy()


def test_forward_vs_independent_reference(tiny):
    w, d = tiny
    r = run(w, d)
    for t in range(0, w.num_tokens, 3):
        ref = reference_token(t, d, w.num_experts)
        assert np.array_equal(r["y"][t].view(np.uint32), ref.view(np.uint32)), t


def test_forward_tokens_matches_full(tiny):
    w, d = tiny
    r = run(w, d)
    toks = np.array([0, 5, 17, 63])
    y, hits = forward_tokens(toks, d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"],
                             d["w2"], d["w2_sf"], num_experts=w.num_experts, expert_begin=0)
    assert np.array_equal(y, r["y"][toks])
    p = r["plan"]
    for (t, j), (q, s, yv) in hits.items():
        row = p.slot[t, j]
        assert np.array_equal(q, r["h_q"][row]) and np.array_equal(s, r["h_sf"][row])


def test_topk_weight_power_of_two_scaling(tiny):
    # w * 2^m: H_q codes identical, H_sf + m, y * 2^m exactly (no saturation at these sizes)
    w, d = tiny
    r0 = run(w, d)
    r1 = run(w, d, topk_w=(d["topk_w"] * 4.0).astype(np.float32))
    p = r0["plan"]
    valid = p.row_token >= 0
    assert np.array_equal(r0["h_q"][valid], r1["h_q"][valid])
    assert np.array_equal(r0["h_sf"][valid].astype(int) + 2, r1["h_sf"][valid].astype(int))
    assert np.array_equal(r0["y"] * 4.0, r1["y"])


def test_w2_scale_shift(tiny):
    w, d = tiny
    r0 = run(w, d)
    r1 = run(w, d, w2_sf=(d["w2_sf"].astype(np.int64) + 3).astype(np.uint8))
    assert np.array_equal(r0["y"] * 8.0, r1["y"])


def test_zero_weight_and_no_hit_tokens(tiny):
    w, d = tiny
    tw = d["topk_w"].copy()
    tw[:5] = 0.0
    ids = d["topk_idx"].copy()
    ids[5:9] = np.array([-1, 99])           # no local hit
    r = run(w, d, topk_w=tw, topk_idx=ids)
    assert np.all(r["y"][:9] == 0.0)
    assert np.any(r["y"][9:] != 0.0)


def test_token_permutation(tiny):
    w, d = tiny
    r0 = run(w, d)
    perm = np.random.default_rng(7).permutation(w.num_tokens)
    r1 = run(w, d, x=d["x"][perm], x_sf=d["x_sf"][perm], topk_idx=d["topk_idx"][perm], topk_w=d["topk_w"][perm])
    assert np.array_equal(r1["y"], r0["y"][perm])


def test_expert_permutation(tiny):
    w, d = tiny
    r0 = run(w, d)
    perm = np.random.default_rng(8).permutation(w.num_experts)   # new expert e' holds old expert perm[e']
    inv = np.argsort(perm)
    r1 = run(w, d, topk_idx=inv[d["topk_idx"]], w1=d["w1"][perm], w1_sf=d["w1_sf"][perm],
             w2=d["w2"][perm], w2_sf=d["w2_sf"][perm])
    assert np.array_equal(r1["y"], r0["y"])


def test_single_expert_dense_ffn():
    # k=1, E=1, w=1: a dense quantised SwiGLU FFN
    w = inputs.Workload("dense", 16, 128, 64, 1, 1, 1, 16, "uniform", seed=5, weight_seed=6)
    d = inputs.to_numpy(inputs.make_inputs(w))
    d["topk_idx"][:] = 0
    d["topk_w"][:] = 1.0
    r = forward_ref(d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"], d["w2_sf"],
                    num_experts=1, expert_begin=0, block_m=16)
    for t in range(w.num_tokens):
        assert np.array_equal(r["y"][t], reference_token(t, d, 1))


def test_swiglu_clamp_closed_form():
    # activation clamp (reading notes, "activation clamp"): gate bounded above, up on both sides;
    # expected values from math.exp on Python floats, rounded to float32 step by step
    import math
    from oracle.forward import swiglu_weight
    cases = [  # (gate, up, w, limit)
        (20.0, -30.0, 0.5, 10.0),    # both clamped
        (-30.0, 4.0, 1.0, 10.0),     # gate below -limit is not clamped
        (3.0, 12.5, 2.0, 10.0),      # up clamped from above only
        (10.0, -10.0, 1.0, 10.0),    # exactly at the limit
        (7.0, 2.0, 0.25, 0.0),       # limit 0: no clamp
    ]
    for g, u, wt, lim in cases:
        h = swiglu_weight(np.array([[g]], np.float32), np.array([[u]], np.float32), np.array([wt], np.float32), lim)
        gc = min(g, lim) if lim > 0 else g
        uc = max(-lim, min(u, lim)) if lim > 0 else u
        s = np.float32(gc / (1.0 + math.exp(-gc)))
        expect = np.float32(np.float32(s * np.float32(uc)) * np.float32(wt))
        assert h[0, 0] == expect, (g, u, wt, lim, h[0, 0], expect)


def test_swiglu_clamp_bounds_and_identity(tiny):
    from oracle.forward import swiglu_weight
    rng = np.random.default_rng(5)
    zg = (rng.standard_normal((64, 96)) * 40).astype(np.float32)
    zu = (rng.standard_normal((64, 96)) * 40).astype(np.float32)
    wt = rng.random(64).astype(np.float32)
    plain = swiglu_weight(zg, zu, wt)
    # a limit above every value changes nothing (bit for bit)
    assert np.array_equal(swiglu_weight(zg, zu, wt, 1e30), plain)
    # with limit L: |h| <= max(L, max |silu| on the negative axis) * L * w
    L = 3.0
    h = swiglu_weight(zg, zu, wt, L)
    assert np.all(np.abs(h) <= max(L, 0.2785) * L * wt[:, None] * (1 + 1e-6))
    assert not np.array_equal(h, plain)
    # the whole forward: a clamp at 1e30 is the unclamped forward
    w, d = tiny
    r0 = run(w, d)
    r1 = forward_ref(d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"], d["w2_sf"],
                     num_experts=w.num_experts, expert_begin=0, block_m=w.block_m, swiglu_limit=1e30)
    assert np.array_equal(r0["y"], r1["y"]) and np.array_equal(r0["h_q"], r1["h_q"])
