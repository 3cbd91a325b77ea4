"""moe_forward_noalloc (the forward whose workspace is the library's own device array) against
moe_forward with a caller workspace: bit-identical outputs on two calls in a row, the second on a
smaller input, so the second call finds the first call's contents in the array."""
import pytest
import torch

from moe_expert_ffn_plan_amd import binding as B
from moe_expert_ffn_plan_amd import inputs

pytestmark = pytest.mark.gpu

# the largest batch the array holds (the decode workload), then a smaller one of another shape
CASES = [inputs.WORKLOADS["decode"],
         inputs.Workload("noalloc_small", 300, 1024, 512, 6, 10, 4, 32, "uniform", 0.1, 50.0, seed=81,
                         weight_seed=91)]


def _with_ws(s, d, dev):
    y = torch.empty(s.num_tokens, s.hidden, dtype=torch.bfloat16, device=dev)
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=dev)
    B.forward(s, d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"], d["w2_sf"], y, ws)
    torch.cuda.synchronize()
    return y


def test_noalloc_matches_forward(gpu):
    outs = []
    for w in CASES:
        s = B.shape_of(w)
        assert B.forward_workspace_bytes(s) <= B.NOALLOC_WORKSPACE_BYTES
        print(f"no-alloc forward: {w.name} T={w.num_tokens} H={w.hidden} I={w.intermediate} "
              f"ws={B.forward_workspace_bytes(s)} B", flush=True)
        d = {k: v.to(gpu) for k, v in inputs.make_inputs(w, device="cpu").items()}
        d.update(B.prepare_all(s, d))
        y = torch.full((w.num_tokens, w.hidden), float("nan"), dtype=torch.bfloat16, device=gpu)
        B.forward_noalloc(s, d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"],
                          d["w2_sf"], y)
        torch.cuda.synchronize()
        want = _with_ws(s, d, gpu)
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"{w.name}: differs from moe_forward"
        outs.append(y)
    assert all(torch.isfinite(o.float()).all() for o in outs)
