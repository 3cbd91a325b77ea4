"""GPU parity of the routing tables (moe_plan): bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from moe_expert_ffn_plan_amd import binding as B
from moe_expert_ffn_plan_amd import inputs
from oracle.routing import plan_ref
from parity import assert_plan_equal, gpu_plan_to_numpy

pytestmark = pytest.mark.gpu


def gpu_plan(ids: np.ndarray, E: int, bm: int, begin: int, dev, H=256, I=128, repeat=1):
    T, k = ids.shape
    s = B.make_shape(T, H, I, E, k, bm, begin)
    t_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int64)).to(dev)
    ws = torch.full((B.plan_workspace_bytes(s),), 0xAB, dtype=torch.uint8, device=dev)   # garbage-filled
    outs = []
    for _ in range(repeat):
        B.plan(s, t_ids, ws)
        torch.cuda.synchronize()
        outs.append(gpu_plan_to_numpy(B.plan_view(s, ws), T, k))
    return outs


@pytest.mark.parametrize("name", inputs.ORDER)
def test_plan_workloads(gpu, name):
    w = inputs.WORKLOADS[name]
    print(f"plan parity: workload {name}", flush=True)
    d = inputs.make_inputs(w, device="cpu", with_weights=False)
    ids = d["topk_idx"].numpy()
    (g,) = gpu_plan(ids, w.num_experts, w.block_m, 0, gpu)
    assert_plan_equal(g, plan_ref(ids, w.num_experts, 0, w.block_m))


def test_plan_deterministic(gpu):
    w = inputs.WORKLOADS["skewed"]
    ids = inputs.make_inputs(w, device="cpu", with_weights=False)["topk_idx"].numpy()
    a, b = gpu_plan(ids, w.num_experts, w.block_m, 0, gpu, repeat=2)
    for f in a:
        assert np.array_equal(a[f], b[f]), f


@pytest.mark.parametrize("case", ["invalid_ids", "offset_begin", "duplicates", "one_token", "one_expert",
                                  "all_invalid", "max_experts", "max_topk", "hot_expert"])
def test_plan_edge_cases(gpu, case):
    rng = np.random.default_rng(abs(hash(case)) % 2**32)
    E, bm, begin = 16, 32, 0
    if case == "invalid_ids":
        ids = rng.integers(-5, 40, size=(300, 6))
    elif case == "offset_begin":
        begin = 96
        ids = rng.integers(0, 256, size=(500, 8))
    elif case == "duplicates":
        ids = rng.integers(0, 4, size=(200, 8))
        E = 4
    elif case == "one_token":
        ids = np.array([[3, 7, 3, 15]])
    elif case == "one_expert":
        E, bm = 1, 16
        ids = rng.integers(0, 2, size=(77, 3))
    elif case == "all_invalid":
        ids = rng.integers(100, 200, size=(64, 4))
    elif case == "max_experts":
        E, bm = 512, 16
        ids = rng.integers(0, 600, size=(3000, 8))
    elif case == "max_topk":
        ids = np.stack([rng.permutation(80)[:64] for _ in range(100)])
        E, bm = 48, 64
    else:  # hot_expert: most hits on one expert, long runs in one wave's range
        ids = np.where(rng.random((5000, 4)) < 0.8, 5, rng.integers(0, 16, size=(5000, 4)))
        bm = 128
    print(f"plan edge case {case}: T={ids.shape[0]} k={ids.shape[1]} E={E} bm={bm}", flush=True)
    (g,) = gpu_plan(ids, E, bm, begin, gpu)
    assert_plan_equal(g, plan_ref(ids, E, begin, bm))


@pytest.mark.parametrize("T,k,E", [(4096, 8, 64), (4097, 8, 64), (32768, 1, 7), (32769, 1, 7), (5000, 8, 512),
                                   (16384, 8, 32), (16385, 6, 48), (32769, 2, 48), (70000, 1, 300), (33000, 64, 16)])
def test_plan_path_boundary(gpu, T, k, E):
    """Inputs just below and above the one-workgroup limit (32768 hits) take different kernels;
    both must give the oracle's tables.  Past 16384 tokens the groups grow from 64 to 128 tokens,
    past 32768 to 256 (16385 and 32769 tokens: a last group of one token; 70000 tokens of 300
    experts: 256-token groups with the separate scan; top-64: the largest group LDS table)."""
    rng = np.random.default_rng(T * 31 + k)
    ids = rng.integers(-2, E + 3, size=(T, k))
    print(f"plan path boundary: T={T} k={k} E={E} hits={T * k}", flush=True)
    (g,) = gpu_plan(ids, E, 32, 0, gpu)
    assert_plan_equal(g, plan_ref(ids, E, 0, 32))


@pytest.mark.parametrize("bm", [96, 192])
@pytest.mark.parametrize("T,k,E", [(300, 8, 40), (4096, 8, 64), (20000, 6, 48), (9000, 8, 512)])
def test_plan_blocks_96_192(gpu, bm, T, k, E):
    """The two routing blocks of the ladder that are not powers of two, through every routing path
    (one workgroup; counts + fused scan; counts, scan, scatter for the largest group x expert table)."""
    rng = np.random.default_rng(T + 7 * bm + E)
    ids = rng.integers(-2, E + 5, size=(T, k))
    print(f"plan block {bm}: T={T} k={k} E={E}", flush=True)
    (g,) = gpu_plan(ids, E, bm, 0, gpu)
    assert_plan_equal(g, plan_ref(ids, E, 0, bm))


@pytest.mark.parametrize("seed", range(12))
def test_plan_fuzz(gpu, seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 9000))
    k = int(rng.integers(1, 10))
    E = int(rng.integers(1, 100))
    bm = int(rng.choice([16, 32, 64, 96, 128, 192]))
    begin = int(rng.integers(0, 50))
    ids = rng.integers(begin - 3, begin + 2 * E, size=(T, k))
    print(f"plan fuzz seed {seed}: T={T} k={k} E={E} bm={bm} begin={begin}", flush=True)
    (g,) = gpu_plan(ids, E, bm, begin, gpu)
    assert_plan_equal(g, plan_ref(ids, E, begin, bm))
