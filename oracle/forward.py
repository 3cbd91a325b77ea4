"""Fused MoE expert FFN forward, one GPU's share (oracle side, test infrastructure).

Steps, in the order the pages give them:

1. Grouped Linear1 (reading notes, "stage three: FP8 x FP4 two-layer GEMM",
   Z_e = X_e W1_e^T with W1_e of shape [2*d_ff, d_model]).  Operands are the
   exactly dequantized FP8/FP4 values with their per-32 UE8M0 scales; the dot
   products are accumulated in float64 and rounded once to float32.  The
   pages' kernel accumulates in FP32; float64 makes the oracle independent of
   summation order.
2. Gate/up de-interleave: W1 rows come as [gate 0..7, up 0..7, gate 8..15,
   up 8..15, ...] ("MegaMoE" walk-through section 7.3; SymmBuffer page
   section 7.2).
3. SwiGLU x top-k weight (walk-through section 4.6, L1 epilogue; reading
   notes "SwiGLU computation"): gate and up accumulators rounded to BF16 and
   read back as float, silu(g) = g / (1 + exp(-g)), then h = (silu(g) * u) * w
   with two float32 multiplies in that order.  The optional activation clamp
   (reading notes, "activation clamp": the gate path bounded from above, the
   up path on both sides, default threshold 10) is applied to the BF16 values
   before silu when a limit > 0 is given; by default it is off.
4. Requant (reading notes, "amax, scale factor and FP8 intermediate"): per
   row and 32-channel group, amax = max |h|; a power-of-two UE8M0 scale (rule
   in ``formats.requant_scale_code``); q = E4M3 round-to-nearest-even of
   h / scale.
5. Grouped Linear2 (Y_e = H_e W2_e^T, W2_e of shape [d_model, d_ff]) on the
   dequantized FP8 codes, float64 accumulation, rounded to float32 and then
   to BF16 (reading notes, "stage five": L2 accumulators cast to BF16).
6. Top-k combine (walk-through section 4.6 "combine reduction"; reading notes
   "stage six"): per token, the BF16 rows of its valid slots read as float
   and added in float32 in ascending top-k order, result rounded to BF16.
   The routing weight is already inside h (step 3), so this sum is
   unweighted.  A token with no valid slot gets +0.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .routing import Plan, plan_ref


def dequant_fp8_rows(codes: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """E4M3 codes [R, K] with UE8M0 scales [R, K/32] -> float64 values."""
    return F.dequant_blocks(F.decode_e4m3(codes), sf)


def dequant_fp4_rows(packed: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """Packed E2M1 [R, K/2] with UE8M0 scales [R, K/32] -> float64 values."""
    return F.dequant_blocks(F.decode_e2m1_packed(packed), sf)


def matmul_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """float32(a @ b.T) with float64 accumulation (a [M, K], b [N, K])."""
    return (np.asarray(a, np.float64) @ np.asarray(b, np.float64).T).astype(np.float32)


def deinterleave_gate_up(z: np.ndarray):
    """Split [.., 2I] Linear1 outputs interleaved by 8 into gate [.., I] and up [.., I]."""
    n2 = z.shape[-1]
    zz = z.reshape(z.shape[:-1] + (n2 // 16, 2, 8))
    gate = zz[..., 0, :].reshape(z.shape[:-1] + (n2 // 2,))
    up = zz[..., 1, :].reshape(z.shape[:-1] + (n2 // 2,))
    return gate, up


def silu_f32(g: np.ndarray) -> np.ndarray:
    """float32(g / (1 + exp(-g))) evaluated in float64 and rounded once."""
    g64 = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return (g64 / (1.0 + np.exp(-g64))).astype(np.float32)


def swiglu_weight(z_gate: np.ndarray, z_up: np.ndarray, w: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """h = fl32(fl32(silu(bf16(g)) * bf16(u)) * w); w broadcasts per row.  With limit > 0,
    g = min(bf16(g), limit) and u = clip(bf16(u), -limit, limit) first.

    The pages print no numeric example of the epilogue; the step is pinned
    by an independent per-token reference that evaluates it with torch's
    silu and casts (the forward matches it bit for bit).
    """
    g = F.bf16_rne(z_gate)
    u = F.bf16_rne(z_up)
    if limit > 0:
        lim = np.float32(limit)
        g = np.minimum(g, lim)
        u = np.clip(u, -lim, lim)
    s = silu_f32(g)
    su = (s * u).astype(np.float32)
    w32 = np.asarray(w, np.float32)
    return (su * w32[..., None]).astype(np.float32)


def requant_fp8(h: np.ndarray):
    """h [R, I] float32 -> (codes uint8 [R, I], scale codes uint8 [R, I/32])."""
    R, I = h.shape
    hb = np.asarray(h, np.float64).reshape(R, I // 32, 32)
    amax = np.abs(hb).max(axis=-1)
    sc = F.requant_scale_code(amax)
    inv = np.ldexp(1.0, 127 - sc.astype(np.int64))          # exact power of two
    q = F.encode_e4m3_rne(hb * inv[..., None])
    return q.reshape(R, I), sc


def combine(yslot_vals: np.ndarray, slot: np.ndarray) -> np.ndarray:
    """y[t] = bf16(sum_j float32 Yslot[slot[t, j]]) over valid j ascending."""
    T, k = slot.shape
    H = yslot_vals.shape[1]
    acc = np.zeros((T, H), dtype=np.float32)
    for j in range(k):
        s = slot[:, j]
        v = s >= 0
        acc[v] = (acc[v] + yslot_vals[s[v]]).astype(np.float32)
    return F.bf16_rne(acc)


def expert_rows_forward(xq_rows, xsf_rows, w_rows, w1, w1_sf, w2, w2_sf, swiglu_limit: float = 0.0):
    """Rows of one expert: FP8 activations [n, H] -> (H_q, H_sf, Yslot BF16 values)."""
    a = dequant_fp8_rows(xq_rows, xsf_rows)
    z = matmul_f32(a, dequant_fp4_rows(w1, w1_sf))
    gate, up = deinterleave_gate_up(z)
    h = swiglu_weight(gate, up, w_rows, swiglu_limit)
    hq, hsf = requant_fp8(h)
    y2 = matmul_f32(dequant_fp8_rows(hq, hsf), dequant_fp4_rows(w2, w2_sf))
    return hq, hsf, F.bf16_rne(y2)


def forward_ref(x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, *, num_experts: int,
                expert_begin: int, block_m: int, plan: Plan | None = None, swiglu_limit: float = 0.0):
    """Whole forward.  Returns a dict with the plan, H_q/H_sf/Yslot over [R_pad] rows and y.

    Shapes: x uint8 [T, H] (E4M3), x_sf uint8 [T, H/32], topk_idx int64 [T, k],
    topk_w float32 [T, k], w1 uint8 [E, 2I, H/2] (E2M1 pairs, gate/up interleaved
    by 8), w1_sf uint8 [E, 2I, H/32], w2 uint8 [E, H, I/2], w2_sf uint8 [E, H, I/32].
    Padding rows of H_q/H_sf/Yslot are left zero.
    """
    T, H = x.shape
    I = w2.shape[2] * 2
    if plan is None:
        plan = plan_ref(topk_idx, num_experts, expert_begin, block_m)
    hq = np.zeros((plan.r_pad, I), np.uint8)
    hsf = np.zeros((plan.r_pad, I // 32), np.uint8)
    ys = np.zeros((plan.r_pad, H), np.float32)
    tw = np.asarray(topk_w, np.float32)
    for e in range(num_experts):
        r0, n = int(plan.offsets[e]), int(plan.counts[e])
        if n == 0:
            continue
        rows = np.arange(r0, r0 + n)
        tok, j = plan.row_token[rows], plan.row_topk[rows]
        q, s, yv = expert_rows_forward(x[tok], x_sf[tok], tw[tok, j], w1[e], w1_sf[e], w2[e], w2_sf[e],
                                       swiglu_limit)
        hq[rows], hsf[rows], ys[rows] = q, s, yv
    y = combine(ys, plan.slot)
    return {"plan": plan, "h_q": hq, "h_sf": hsf, "yslot": ys, "y": y}


def forward_tokens(tokens, x, x_sf, topk_idx, topk_w, w1, w1_sf, w2, w2_sf, *,
                   num_experts: int, expert_begin: int, swiglu_limit: float = 0.0):
    """y rows (BF16 values as float32) for a subset of tokens only.

    Each token's rows are independent of every other token's, so the result
    equals the corresponding rows of ``forward_ref``; used at sizes where the
    full forward is too slow for the oracle.  Returns (y [len(tokens), H],
    per-hit dict {(t, j): (H_q row, H_sf row, Yslot row)}).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    H = x.shape[1]
    ids = np.asarray(topk_idx, np.int64)
    tw = np.asarray(topk_w, np.float32)
    k = ids.shape[1]
    by_expert: dict[int, list] = {}
    for t in tokens:
        for j in range(k):
            e = int(ids[t, j]) - expert_begin
            if 0 <= e < num_experts:
                by_expert.setdefault(e, []).append((int(t), j))
    per_hit = {}
    for e, hits in by_expert.items():
        tt = np.array([h[0] for h in hits])
        jj = np.array([h[1] for h in hits])
        q, s, yv = expert_rows_forward(x[tt], x_sf[tt], tw[tt, jj], w1[e], w1_sf[e], w2[e], w2_sf[e],
                                       swiglu_limit)
        for i, h in enumerate(hits):
            per_hit[h] = (q[i], s[i], yv[i])
    y = np.zeros((tokens.size, H), np.float32)
    for i, t in enumerate(tokens):
        acc = np.zeros(H, np.float32)
        for j in range(k):
            if (int(t), j) in per_hit:
                acc = (acc + per_hit[(int(t), j)][2]).astype(np.float32)
        y[i] = F.bf16_rne(acc)
    return y, per_hit
