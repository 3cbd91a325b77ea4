"""Seeded synthetic workloads for the fused MoE expert FFN.

This module only draws random inputs and stores them in the formats the
forward consumes.  It holds none of the forward's own arithmetic: the FP8
input cast is torch's ``float8_e4m3fn`` conversion and the FP4 weight cast
is a plain nearest-value table lookup.  Both the library's tests and the
benchmark use it, and so does the CPU oracle's test side.

Workloads (one GPU's share each; expert ids are global, experts
[0, num_experts) are local):

* ``tiny``     64 tokens, hidden 256, intermediate 128, 8 experts, top-2 of a
  softmax over N(0,1) logits, weights renormalised; block_m 128.
* ``tp_slice`` 2048 tokens, hidden 4096, intermediate 768, 64 experts all
  local, top-8 distinct uniform experts, Dirichlet(1) weights; block_m 128.
  This is one tensor-parallel rank's slice of the practice page's layer.
* ``decode``   128 tokens, hidden 7168, intermediate 2048, 32 local of 256
  experts, top-8 distinct uniform over 256, only local hits kept; block_m 16.
* ``prefill``  as decode with 4096 tokens; block_m 32.
* ``skewed``   as decode with 16384 tokens, experts drawn Zipf(s=1.2) over
  256 ranks without replacement (Gumbel-top-k), expert id = rank - 1; 10% of
  tokens have x scaled by 50 before quantisation; block_m 128.
* ``dsv4``     one rank's share of the DeepSeek-V4 expert shape the reading
  notes' tests use: 8 ranks x 8192 tokens = 65536 tokens routed, hidden
  7168, intermediate 3072, 48 local of 384 experts, top-6 distinct uniform,
  Dirichlet(1) weights; block_m 192, the pages' block for this test (and
  what the block heuristic picks for the shape).

Values: x ~ N(0, 1); weights ~ N(0, std = 1/sqrt(K)) with K the reduction
size of that GEMM.  Both are quantised per 32 consecutive K elements with a
power-of-two (UE8M0) scale chosen so that the block's largest magnitude fits
the element format (448 for E4M3, 6 for E2M1).  W1 rows are generated
directly in the interleaved gate/up order (groups of 8 gate rows, then 8 up
rows); since rows are i.i.d. this is the same distribution as interleaving
separately drawn gate and up matrices.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    num_tokens: int
    hidden: int
    intermediate: int
    num_experts: int          # local experts
    global_experts: int       # expert ids are drawn from [0, global_experts)
    topk: int
    block_m: int
    routing: str              # softmax_top | uniform | zipf
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    seed: int = 0
    weight_seed: int = 0


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 128, 8, 8, 2, 128, "softmax_top", seed=1000, weight_seed=2000),
    "tp_slice": Workload("tp_slice", 2048, 4096, 768, 64, 64, 8, 128, "uniform", seed=1001, weight_seed=2001),
    "decode": Workload("decode", 128, 7168, 2048, 32, 256, 8, 16, "uniform", seed=1002, weight_seed=2002),
    "prefill": Workload("prefill", 4096, 7168, 2048, 32, 256, 8, 32, "uniform", seed=1003, weight_seed=2002),
    "skewed": Workload("skewed", 16384, 7168, 2048, 32, 256, 8, 128, "zipf", 0.1, 50.0, seed=1004,
                       weight_seed=2002),
    "dsv4": Workload("dsv4", 65536, 7168, 3072, 48, 384, 6, 192, "uniform", seed=1005, weight_seed=2005),
}
ORDER = ["tiny", "tp_slice", "decode", "prefill", "skewed", "dsv4"]


def _pow2_scale_exponent(amax: torch.Tensor, fmt_max_mant: float, fmt_max_exp: int) -> torch.Tensor:
    """Smallest s with amax / 2**s <= fmt_max, fmt_max = fmt_max_mant * 2**fmt_max_exp, mant in [0.5, 1)."""
    m, e = torch.frexp(amax)
    s = torch.where(m <= fmt_max_mant, e - fmt_max_exp, e - fmt_max_exp + 1)
    return torch.where(amax > 0, s, torch.zeros_like(s))


def quantize_e4m3_blocks(v: torch.Tensor):
    """float32 [R, K] -> (E4M3 codes uint8 [R, K], UE8M0 codes uint8 [R, K/32])."""
    R, K = v.shape
    b = v.reshape(R, K // 32, 32)
    amax = b.abs().amax(dim=-1)
    s = _pow2_scale_exponent(amax, 0.875, 9)                  # 448 = 0.875 * 2**9
    q = (b * torch.ldexp(torch.ones_like(amax), -s)[..., None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).reshape(R, K), (s + 127).clamp(0, 254).to(torch.uint8)


_FP4_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)   # midpoints between E2M1 magnitudes


def quantize_e2m1_blocks(v: torch.Tensor):
    """float32 [R, K] -> (packed E2M1 uint8 [R, K/2], UE8M0 codes uint8 [R, K/32]).

    Nearest E2M1 magnitude, ties to the even code; even K in the low nibble.
    """
    R, K = v.shape
    b = v.reshape(R, K // 32, 32)
    amax = b.abs().amax(dim=-1)
    s = _pow2_scale_exponent(amax, 0.75, 3)                   # 6 = 0.75 * 2**3
    a = (b * torch.ldexp(torch.ones_like(amax), -s)[..., None]).abs()
    code = torch.zeros_like(a, dtype=torch.uint8)
    for c, mid in enumerate(_FP4_MID):
        # between code c and c+1 a tie goes to the even code
        code += (a > mid if c % 2 == 0 else a >= mid).to(torch.uint8)
    code |= (b < 0).to(torch.uint8) << 3
    code = code.reshape(R, K)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (s + 127).clamp(0, 254).to(torch.uint8)


def _routing(w: Workload, g: torch.Generator, device, T: int):
    k, G = w.topk, w.global_experts
    if w.routing == "softmax_top":
        logits = torch.randn(T, G, generator=g, device=device)
        probs = torch.softmax(logits, dim=-1)
        top_p, top_i = torch.topk(probs, k, dim=-1)
        weights = top_p / top_p.sum(dim=-1, keepdim=True)
        return top_i.to(torch.int64), weights.to(torch.float32)
    if w.routing == "uniform":
        ids = torch.rand(T, G, generator=g, device=device).argsort(dim=-1)[:, :k]
    elif w.routing == "zipf":
        ranks = torch.arange(1, G + 1, device=device, dtype=torch.float64)
        logp = -1.2 * torch.log(ranks)
        u = torch.rand(T, G, generator=g, device=device, dtype=torch.float64).clamp_min(1e-300)
        gumbel = -torch.log(-torch.log(u))
        ids = torch.topk(logp[None, :] + gumbel, k, dim=-1).indices
    else:
        raise ValueError(w.routing)
    e = -torch.log(torch.rand(T, k, generator=g, device=device, dtype=torch.float64).clamp_min(1e-300))
    weights = (e / e.sum(dim=-1, keepdim=True)).to(torch.float32)   # Dirichlet(1, ..., 1)
    return ids.to(torch.int64), weights


def make_inputs(w: Workload | str, device="cpu", num_tokens: int | None = None, seed: int | None = None,
                weight_seed: int | None = None, with_weights: bool = True, with_outlier_mask: bool = False):
    """Draw one workload.  Returns a dict of tensors on ``device``:

    x uint8 [T, H] (E4M3), x_sf uint8 [T, H/32], topk_idx int64 [T, k],
    topk_w float32 [T, k], w1 uint8 [E, 2I, H/2], w1_sf uint8 [E, 2I, H/32],
    w2 uint8 [E, H, I/2], w2_sf uint8 [E, H, I/32]; with ``with_outlier_mask``
    also outlier bool [T], the tokens whose x was scaled before quantisation.
    Draw order: routing, top-k weights, x, outlier rows; then W1, W2 from
    their own generator.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    T = w.num_tokens if num_tokens is None else num_tokens
    H, I, E = w.hidden, w.intermediate, w.num_experts
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    ids, tw = _routing(w, g, device, T)
    x = torch.randn(T, H, generator=g, device=device)
    outlier = torch.zeros(T, dtype=torch.bool, device=device)
    if w.outlier_frac > 0 and T > 0:
        perm = torch.randperm(T, generator=g, device=device)
        x[perm[: int(T * w.outlier_frac)]] *= w.outlier_scale
        outlier[perm[: int(T * w.outlier_frac)]] = True
    xq, xsf = quantize_e4m3_blocks(x) if T > 0 else (torch.zeros(0, H, dtype=torch.uint8, device=device),
                                                   torch.zeros(0, H // 32, dtype=torch.uint8, device=device))
    out = {"x": xq.contiguous(), "x_sf": xsf.contiguous(), "topk_idx": ids.contiguous(),
           "topk_w": tw.contiguous()}
    if with_outlier_mask:
        out["outlier"] = outlier
    if with_weights:
        out.update(make_weights(w, device, weight_seed))
    return out


def make_weights(w: Workload | str, device="cpu", weight_seed: int | None = None):
    if isinstance(w, str):
        w = WORKLOADS[w]
    H, I, E = w.hidden, w.intermediate, w.num_experts
    gw = torch.Generator(device=device)
    gw.manual_seed(w.weight_seed if weight_seed is None else weight_seed)
    w1 = torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, device=device)
    w1sf = torch.empty(E, 2 * I, H // 32, dtype=torch.uint8, device=device)
    w2 = torch.empty(E, H, I // 2, dtype=torch.uint8, device=device)
    w2sf = torch.empty(E, H, I // 32, dtype=torch.uint8, device=device)
    for e in range(E):
        v = torch.randn(2 * I, H, generator=gw, device=device) * (1.0 / H ** 0.5)
        w1[e], w1sf[e] = quantize_e2m1_blocks(v)
    for e in range(E):
        v = torch.randn(H, I, generator=gw, device=device) * (1.0 / I ** 0.5)
        w2[e], w2sf[e] = quantize_e2m1_blocks(v)
    return {"w1": w1, "w1_sf": w1sf, "w2": w2, "w2_sf": w2sf}


def to_numpy(inputs: dict) -> dict:
    return {k: v.detach().cpu().numpy() for k, v in inputs.items()}
