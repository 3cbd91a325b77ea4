"""Seeded random shapes through the whole forward (moe_plan + moe_forward), each compared in full
with the CPU oracle: routing tables bit-exact, FP8 intermediates and y within the parity gates.

The draws cover every routing block (16, 32, 64, 96, 128, 192), hidden and intermediate sizes that select
either GEMM schedule (one persistent launch or two; 512- or 256-column tiles), one to sixteen local
experts out of up to four times as many, top-1 to top-8 with uniform or Zipf routing, a shifted
range of local expert ids, a few tokens up to a few hundred, the activation clamp and the accurate
SiLU, and inputs with outlier rows.  Two degenerate cases are fixed: a single hit, and a batch with
no local hit at all (y must be exactly +0).

Every case must have exact tables, every FP8 mismatch within 1 ulp (outside Linear1 cancellation) and
y within its gates; the 0.1% bound on the share of mismatching FP8 elements applies to the elements of
all random cases together, since a case of a few thousand elements moves by 0.05% per mismatch.  A
case that fails the y gate's max clause as stated may pass it widened by the carry of its admitted FP8
differences into y (tests/parity.py); the test prints how many cases needed that, and at most a few
percent of the cases may.
"""
import numpy as np
import pytest

from moe_expert_ffn_plan_amd import binding as B
from moe_expert_ffn_plan_amd import inputs
from test_gpu_forward import check_full, run_gpu

pytestmark = pytest.mark.gpu

N_CASES = 120


def fuzz_case(i):
    r = np.random.default_rng(9000 + i)
    H = int(r.choice([256, 512, 768, 1024, 1536]))
    I = int(r.choice([128, 256, 384, 512, 768]))
    E = int(r.integers(1, 17))
    G = int(r.integers(E, 4 * E + 1))
    k = int(r.integers(1, min(8, G) + 1))
    T = int(r.choice([1, 2, 7, 63, 64, 65, 130, 257, 411]))
    bm = int(r.choice([16, 32, 64, 96, 128, 192]))
    routing = str(r.choice(["uniform", "zipf"]))
    outliers = float(r.choice([0.0, 0.1]))
    begin = int(r.choice([0, G - E]))
    limit = float(r.choice([0.0, 0.0, 10.0]))
    exact = bool(r.integers(0, 4) == 0)
    w = inputs.Workload(f"fuzz{i}", T, H, I, E, G, k, bm, routing, outliers, 50.0, seed=9100 + i,
                        weight_seed=9200 + i)
    return w, begin, limit, exact


def _run_case(w, begin, limit, exact, gpu, fp8_rate=True, fuzz_allowance=False):
    s = B.shape_of(w, expert_begin=begin)
    print(f"fuzz {w.name}: T={w.num_tokens} H={w.hidden} I={w.intermediate} E={w.num_experts} of "
          f"{w.global_experts} k={w.topk} bm={w.block_m} {w.routing} begin={begin} limit={limit} exact={exact} "
          f"launches={B.gemm_launches(s)}", flush=True)
    d = inputs.make_inputs(w, device="cpu")
    out = run_gpu(w, d, gpu, expert_begin=begin, swiglu_limit=limit, exact_silu=exact)
    ref = check_full(w, d, out, expert_begin=begin, swiglu_limit=limit, fp8_rate=fp8_rate,
                     fuzz_allowance=fuzz_allowance)
    if ref["y_widened"]:
        print(f"fuzz {w.name}: y gate met only with the FP8 carry allowance", flush=True)
    return d, out, ref


def test_forward_fuzz(gpu):
    bad = total = widened = 0
    for i in range(N_CASES):
        w, begin, limit, exact = fuzz_case(i)
        _, _, ref = _run_case(w, begin, limit, exact, gpu, fp8_rate=False, fuzz_allowance=True)
        b, n = ref["fp8_counts"]
        bad, total, widened = bad + b, total + n, widened + int(ref["y_widened"])
    print(f"fuzz: FP8 mismatches {bad} of {total} elements ({bad / max(total, 1):.4%}); {widened} of {N_CASES} "
          f"cases met the y gate only with the FP8 carry allowance", flush=True)
    assert bad <= 1e-3 * total
    assert widened <= N_CASES // 20


def test_forward_single_hit(gpu):
    w = inputs.Workload("fuzz_single", 1, 512, 256, 1, 1, 1, 16, "uniform", seed=9301, weight_seed=9302)
    _run_case(w, 0, 0.0, False, gpu)


def test_forward_no_local_hit(gpu):
    # local experts [8, 12) of ids drawn from [0, 8): nothing is computed on this GPU
    w = inputs.Workload("fuzz_none", 70, 512, 256, 4, 8, 3, 32, "uniform", seed=9303, weight_seed=9304)
    d, out, _ = _run_case(w, 8, 0.0, False, gpu)
    assert np.all(out["y"] == 0) and not np.any(np.signbit(out["y"]))
