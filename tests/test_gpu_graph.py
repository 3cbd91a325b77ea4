"""GPU tests of stream capture: moe_plan + moe_forward recorded into a HIP graph and replayed.

The practice page rebuilds its schedule tables with a captured graph and keeps every buffer
allocated once so that the layer can be replayed (sections 2 and 5).  Here the whole forward is
recorded once; each replay runs on new inputs copied into the captured buffers, and its output
must equal an eager moe_forward on the same inputs bit for bit.  Eager work and synchronisation
run between the replays.  The single-launch GEMM stamps its completion flags with an epoch
that a recorded one-thread kernel advances on every replay; a replay that reused the previous
replay's epoch would find its flags already set and could read rows Linear1 has not yet written.
"""
import pytest
import torch

from moe_expert_ffn_plan_amd import binding as B
from moe_expert_ffn_plan_amd import inputs

pytestmark = pytest.mark.gpu

CASES = {
    # one persistent launch for both GEMMs (128-row tiles over 32-row blocks)
    "one_launch": inputs.Workload("graph_one_launch", 700, 1024, 512, 7, 9, 5, 32, "uniform", seed=61,
                                  weight_seed=71),
    # 16-row tiles, one launch
    "one_launch_bm16": inputs.Workload("graph_bm16", 300, 1024, 768, 6, 10, 4, 16, "uniform", seed=62,
                                       weight_seed=72),
    # I = 256: the GEMMs run as two launches
    "two_launches": inputs.Workload("graph_two", 400, 1024, 256, 5, 5, 3, 64, "uniform", seed=63, weight_seed=73),
}


def _eager(s, d, dev):
    y = torch.empty(d["x"].shape[0], s.hidden, dtype=torch.bfloat16, device=dev)
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=dev)
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=dev)
    B.plan(s, d["topk_idx"], plan_ws)
    B.forward(s, d["x"], d["x_sf"], d["topk_idx"], d["topk_w"], d["w1"], d["w1_sf"], d["w2"], d["w2_sf"], y, ws,
              plan_ws=plan_ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("internal_plan", [False, True])
@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replays(gpu, name, internal_plan):
    """internal_plan: moe_forward builds the plan inside its workspace, and its routing kernels also
    advance the launch counter that the single launch's flags take their value from."""
    w = CASES[name]
    s = B.shape_of(w)
    print(f"graph replay: {name} T={w.num_tokens} bm={w.block_m} launches={B.gemm_launches(s)} "
          f"internal plan={internal_plan}", flush=True)
    weights = {k: v.to(gpu) for k, v in inputs.make_weights(w, device="cpu").items()}
    weights.update(B.prepare_all(s, weights))

    def draw(seed):
        d = {k: v.to(gpu) for k, v in inputs.make_inputs(w, device="cpu", seed=seed, with_weights=False).items()}
        d.update(weights)
        return d

    static = draw(100)
    y = torch.empty(w.num_tokens, w.hidden, dtype=torch.bfloat16, device=gpu)
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=gpu)
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=gpu)
    status = B.forward_view(s, ws)["sync_status"]
    status.zero_()

    def run():
        if not internal_plan:
            B.plan(s, static["topk_idx"], plan_ws)
        B.forward(s, static["x"], static["x_sf"], static["topk_idx"], static["topk_w"], static["w1"],
                  static["w1_sf"], static["w2"], static["w2_sf"], y, ws, plan_ws=None if internal_plan else plan_ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # eager call before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep, seed in enumerate((101, 102, 103, 101)):
        new = draw(seed)
        for key in ("x", "x_sf", "topk_idx", "topk_w"):
            static[key].copy_(new[key])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = _eager(s, new, gpu)  # eager work between replays
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"{name}: replay {rep} differs from eager"
        if internal_plan:  # an eager forward on the captured workspace between replays
            run()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"{name}: eager call {rep} differs"
    assert int(status.item()) == 0, "a Linear2 tile gave up waiting"


@pytest.mark.parametrize("fill", [0x00, 0x5A, 0xFF])
def test_graphs_share_workspace(gpu, fill):
    """Two forwards (two layers: different weights) recorded into one graph on ONE workspace, a second
    graph with the layers in the other order on the same workspace, and eager calls on it in between.
    Every launch on the workspace must stamp completion flags no earlier launch stamped, whatever the
    workspace held at first; each output is compared bit for bit with an eager run on a fresh
    workspace."""
    w = CASES["one_launch"]
    s = B.shape_of(w)
    assert B.forward_uses_expert_ffn(s)
    print(f"graph replay: two layers on one workspace, fill 0x{fill:02X}", flush=True)
    layers = []
    for ws_seed in (71, 171):
        lw = {k: v.to(gpu) for k, v in inputs.make_weights(w, device="cpu", weight_seed=ws_seed).items()}
        lw.update(B.prepare_all(s, lw))
        layers.append(lw)
    static = {k: v.to(gpu) for k, v in inputs.make_inputs(w, device="cpu", seed=200, with_weights=False).items()}
    ws = torch.full((B.forward_workspace_bytes(s),), fill, dtype=torch.uint8, device=gpu)
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=gpu)
    ys = [torch.empty(w.num_tokens, w.hidden, dtype=torch.bfloat16, device=gpu) for _ in range(2)]

    def run(order):
        B.plan(s, static["topk_idx"], plan_ws)
        for li, yi in zip(order, (0, 1)):
            lw = layers[li]
            B.forward(s, static["x"], static["x_sf"], static["topk_idx"], static["topk_w"], lw["w1"], lw["w1_sf"],
                      lw["w2"], lw["w2_sf"], ys[yi], ws, plan_ws=plan_ws)

    def expect(order):
        d = dict(static)
        return [_eager(s, {**d, **layers[li]}, gpu) for li in order]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run((0, 1))  # eager call before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for order in ((0, 1), (1, 0)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(order)
        graphs[order] = g
    torch.cuda.synchronize()
    status = B.forward_view(s, ws)["sync_status"]
    seq = [("g", (0, 1)), ("g", (1, 0)), ("e", (0, 1)), ("g", (0, 1)), ("g", (0, 1)), ("e", (1, 0)),
           ("g", (1, 0)), ("g", (0, 1))]
    for rep, (kind, order) in enumerate(seq):
        new = {k: v.to(gpu) for k, v in inputs.make_inputs(w, device="cpu", seed=300 + rep,
                                                           with_weights=False).items()}
        for key in ("x", "x_sf", "topk_idx", "topk_w"):
            static[key].copy_(new[key])
        torch.cuda.synchronize()
        if kind == "g":
            graphs[order].replay()
        else:
            run(order)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"step {rep}: a Linear2 tile gave up waiting"
        got = [y.view(torch.int16).clone() for y in ys]
        want = expect(order)
        for li in range(2):
            assert torch.equal(got[li], want[li].view(torch.int16)), f"step {rep} ({kind}{order}) layer {li} differs"


@pytest.mark.parametrize("name", ["skewed", "tp_slice"])
def test_bench_graph_segments_full_size(gpu, name):
    """The launch configuration bench.py times, at full size: each step recorded as three graphs (the
    calls before the dominant GEMM launch, that launch, the calls after it) on a side stream, the
    graphs of two steps with different weights replayed in turn on one workspace, each output equal
    bit for bit to an eager moe_forward (the path compared with the oracle at full size) on the same
    inputs and weights."""
    w = inputs.WORKLOADS[name]
    s = B.shape_of(w)
    fused = B.forward_uses_expert_ffn(s) and B.expert_ffn_is_fused(s)
    print(f"bench graph segments: {name} full size, one launch={fused}", flush=True)
    d = {k: v.to(gpu) for k, v in inputs.make_inputs(w, device=gpu).items()}
    layers = [B.prepare_all(s, d)]
    lw = {k: v.to(gpu) for k, v in inputs.make_weights(w, device=gpu, weight_seed=w.weight_seed + 1000).items()}
    layers.append(B.prepare_all(s, lw))
    del lw
    ws = torch.full((B.forward_workspace_bytes(s),), 0x5A, dtype=torch.uint8, device=gpu)
    plan_ws = torch.empty(B.plan_workspace_bytes(s), dtype=torch.uint8, device=gpu)
    y = torch.empty(w.num_tokens, w.hidden, dtype=torch.bfloat16, device=gpu)

    def segments(wt):
        pre = [lambda st: B.plan(s, d["topk_idx"], plan_ws, st)]
        if fused:
            dom = lambda st: B.expert_ffn(s, d["x"], d["x_sf"], d["topk_w"], wt["w1"], wt["w1_sf"], wt["w2"],  # noqa
                                          wt["w2_sf"], plan_ws, ws, st)
            post = [lambda st: B.combine(s, plan_ws, ws, y, st)]
        else:
            dom = lambda st: B.linear1(s, d["x"], d["x_sf"], d["topk_w"], wt["w1"], wt["w1_sf"], plan_ws, ws, st)  # noqa
            post = [lambda st: B.linear2(s, wt["w2"], wt["w2_sf"], plan_ws, ws, st),
                    lambda st: B.combine(s, plan_ws, ws, y, st)]
        return [pre, [dom], post]

    side = torch.cuda.Stream()
    steps = []
    for wt in layers:
        graphs = []
        for part in segments(wt):
            side.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for call in part:
                    call(torch.cuda.current_stream())
            graphs.append(g)
        steps.append(graphs)
    torch.cuda.synchronize()
    want = []
    for wt in layers:
        want.append(_eager(s, {**d, **wt}, gpu).view(torch.int16).clone())
    status = B.forward_view(s, ws)["sync_status"]
    for rep, li in enumerate((0, 1, 1, 0)):
        for g in steps[li]:
            g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"{name}: replay {rep}: a GEMM launch gave up waiting"
        assert torch.equal(y.view(torch.int16), want[li]), f"{name}: replay {rep} (weights {li}) differs from eager"
