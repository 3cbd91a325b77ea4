"""GPU tests of moe_expert_ffn: Linear1 and Linear2 in one persistent launch.

moe_expert_ffn runs the same tile arithmetic as moe_linear1 followed by
moe_linear2, so its intermediates and outputs must match theirs bit for bit
(the staged path is checked against the oracle elsewhere, and moe_forward,
which runs the fused launch, is checked against the oracle in
test_gpu_forward.py).  The cases cover every kernel variant of the fused
launch (M-tile 16, 128 over whole blocks, 128 over 32-row blocks), a shape
that falls back to two launches, repeated launches on one workspace (flags
left by the previous launch), a second routing on the same workspace and the
full-size workloads (the DeepSeek-V4 shape included, which moe_forward runs as
two launches but moe_expert_ffn runs as one).
"""
import pytest
import torch

from moe_expert_ffn_plan_amd import binding as B
from moe_expert_ffn_plan_amd import inputs

pytestmark = pytest.mark.gpu

CASES = {
    # block_m 16: 16-row M-tiles, K-loops of 8 and 6 steps (the minimum for that tile is 6)
    "fused_bm16": inputs.Workload("fused_bm16", 300, 1024, 768, 6, 10, 4, 16, "uniform", seed=31, weight_seed=41),
    # block_m 32: 128-row M-tiles over four blocks, ragged expert ends; I = 512 gives 4 K-steps (minimum)
    "fused_bm32": inputs.Workload("fused_bm32", 700, 1024, 512, 7, 9, 5, 32, "uniform", seed=32, weight_seed=42),
    # block_m 128 with skewed routing and outliers
    "fused_bm128": inputs.Workload("fused_bm128", 1200, 1536, 512, 8, 40, 6, 128, "zipf", 0.1, 50.0, seed=33,
                                   weight_seed=43),
    # I = 256: 2 K-steps in Linear2, too short for the persistent kernel -> two launches
    "fallback": inputs.Workload("fallback", 400, 1024, 256, 5, 5, 3, 64, "uniform", seed=34, weight_seed=44),
}


def runs_fused(w) -> bool:
    return B.expert_ffn_is_fused(B.shape_of(w))


def _setup(w, dev, seed=None):
    s = B.shape_of(w)
    d = {k: v.to(dev) for k, v in inputs.make_inputs(w, device="cpu", seed=seed).items()}
    d.update(B.prepare_all(s, d))
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=dev)
    B.plan(s, d["topk_idx"], plan_ws)
    return s, d, plan_ws


def _outputs(s, ws, plan_ws):
    fv = B.forward_view(s, ws)
    pv = B.plan_view(s, plan_ws)
    r_pad = int(pv["scalars"][0])
    valid = pv["row_token"][:r_pad] >= 0
    return {"h_q": fv["h_q"][:r_pad][valid].clone(), "h_sf": fv["h_sf"][:r_pad][valid].clone(),
            "yslot": fv["yslot"][:r_pad][valid].clone()}


def _staged(s, d, plan_ws, dev):
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=dev)
    B.linear1(s, d["x"], d["x_sf"], d["topk_w"], d["w1"], d["w1_sf"], plan_ws, ws)
    B.linear2(s, d["w2"], d["w2_sf"], plan_ws, ws)
    torch.cuda.synchronize()
    return _outputs(s, ws, plan_ws)


def _fused(s, d, plan_ws, ws):
    B.expert_ffn(s, d["x"], d["x_sf"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"], d["w2_sf"], plan_ws, ws)
    torch.cuda.synchronize()
    return _outputs(s, ws, plan_ws)


def _assert_same(a, b, what):
    for k in ("h_q", "h_sf", "yslot"):
        assert torch.equal(a[k], b[k]), f"{what}: {k} differs from the staged launches"


@pytest.mark.parametrize("name", list(CASES))
def test_expert_ffn_matches_staged(gpu, name):
    w = CASES[name]
    print(f"expert_ffn vs staged: {name} T={w.num_tokens} H={w.hidden} I={w.intermediate} E={w.num_experts} "
          f"k={w.topk} bm={w.block_m} fused={runs_fused(w)}", flush=True)
    s, d, plan_ws = _setup(w, gpu)
    ref = _staged(s, d, plan_ws, gpu)
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=gpu)
    status = B.forward_view(s, ws)["sync_status"]
    status.zero_()
    for rep in range(3):  # later launches find the previous launch's flags in the workspace
        _assert_same(_fused(s, d, plan_ws, ws), ref, f"{name} launch {rep}")
    assert int(status.item()) == 0, "a Linear2 tile gave up waiting"


def test_expert_ffn_new_routing_same_workspace(gpu):
    w = CASES["fused_bm32"]
    print("expert_ffn: two routings on one workspace", flush=True)
    ws = None
    for seed in (51, 52):
        s, d, plan_ws = _setup(w, gpu, seed=seed)
        ref = _staged(s, d, plan_ws, gpu)
        if ws is None:
            ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=gpu)
            B.forward_view(s, ws)["sync_status"].zero_()
        _assert_same(_fused(s, d, plan_ws, ws), ref, f"seed {seed}")
    assert int(B.forward_view(s, ws)["sync_status"].item()) == 0


@pytest.mark.parametrize("name", ["tp_slice", "decode", "prefill", "dsv4"])
def test_expert_ffn_full_size_matches_staged(gpu, name):
    w = inputs.WORKLOADS[name]
    assert runs_fused(w)
    print(f"expert_ffn vs staged: {name} full size", flush=True)
    s = B.shape_of(w)
    d = {k: v.to(gpu) for k, v in inputs.make_inputs(w, device=gpu).items()}
    d.update(B.prepare_all(s, d))
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=gpu)
    B.plan(s, d["topk_idx"], plan_ws)
    ref = _staged(s, d, plan_ws, gpu)
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=gpu)
    status = B.forward_view(s, ws)["sync_status"]
    status.zero_()
    for rep in range(2):
        _assert_same(_fused(s, d, plan_ws, ws), ref, f"{name} launch {rep}")
    assert int(status.item()) == 0


@pytest.mark.parametrize("name", ["fused_bm32", "fallback"])
def test_status_word_poisons_combine(gpu, name):
    """A non-zero status word (what a single launch leaves when a Linear2 tile gave up waiting) makes
    moe_combine write NaN over all of y; the next GEMM launch clears the word (the single launch's
    prepare kernel, or moe_linear1 in the two-launch schedule) and y is whole again.  The word is set
    from the host: no kernel is made to give up."""
    w = CASES[name]
    print(f"status word: {name} fused={runs_fused(w)}", flush=True)
    s, d, plan_ws = _setup(w, gpu)
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=gpu)
    y = torch.empty(w.num_tokens, w.hidden, dtype=torch.bfloat16, device=gpu)
    args = (d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"], d["w2_sf"], y, ws)
    B.forward(s, *args, plan_ws=plan_ws)
    torch.cuda.synchronize()
    good = y.clone()
    status = B.forward_view(s, ws)["sync_status"]
    assert int(status.item()) == 0
    assert torch.isfinite(good.float()).all()
    status.fill_(1)
    B.combine(s, plan_ws, ws, y)
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()
    B.forward(s, *args, plan_ws=plan_ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(y.view(torch.int16), good.view(torch.int16))
