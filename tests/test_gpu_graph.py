"""HIP-graph capture of whole module steps: replays must match eager execution.

The C-ABI path makes no host synchronisation, allocation or memset, so a step
(scale updates, LayerNormLinear forward and backward) can be captured once and
replayed.  Every replay is compared with an eager run of the same step from the
same state, with eager work (new inputs copied in) between the replays."""
import pytest
import torch

from fp8_delayed_scaling_row_amd import inputs, ops

pytestmark = pytest.mark.gpu


def _state(M, K, N, recipe):
    mf, mb = ops.linear_metas(recipe)
    return dict(mf=mf, mb=mb, ctx=ops.LinearCtx(M, K, N, training=True),
                out=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                dx=torch.empty((M, K), dtype=torch.bfloat16, device="cuda"),
                dgamma=torch.empty(K, device="cuda"), dbeta=torch.empty(K, device="cuda"),
                dw=torch.empty((N, K), device="cuda"), dbias=torch.empty(N, device="cuda"))


def _step(recipe, st, x, dy, g, b, w, bias, ws):
    ops.scaling_update(recipe, st["mf"])
    ops.ln_linear_fwd(recipe, x, g, b, w, bias, st["out"], st["mf"], st["ctx"])
    ops.scaling_update(recipe, st["mb"])
    ops.ln_linear_bwd(recipe, dy, x, g, st["ctx"], st["mf"], st["mb"], st["dx"], st["dgamma"],
                      st["dbeta"], st["dw"], st["dbias"], workspace=ws)


def _snapshot(st):
    keys = ["out", "dx", "dgamma", "dbeta", "dw", "dbias"]
    snap = {k: st[k].clone() for k in keys}
    for m in ("mf", "mb"):
        snap[m] = (st[m].history.clone(), st[m].scale.clone(), st[m].scale_inv.clone())
    return snap


def test_linear_step_replays_match_eager():
    M, K, N = 256, 768, 2304
    recipe = ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16)
    wl = "graph-replay"
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    bias = (torch.randn(N, device="cuda") * 0.1).to(torch.bfloat16)
    xs = [inputs.normal_bf16((M, K), inputs.seed_for(wl, "x", s), device="cuda") for s in range(5)]
    dys = [inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy", s), std=1e-3, device="cuda")
           for s in range(5)]
    ws = torch.empty(ops.workspace_size(ops.OP_LN_LINEAR_BWD, M, K, N), dtype=torch.uint8,
                     device="cuda")
    eager, graphed = _state(M, K, N, recipe), _state(M, K, N, recipe)
    x_in = torch.empty_like(xs[0])
    dy_in = torch.empty_like(dys[0])

    # step 0 eagerly on both states (also warms the launchers' one-time queries)
    for st in (eager, graphed):
        _step(recipe, st, xs[0], dys[0], g, b, w, bias, ws)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    x_in.copy_(xs[1])
    dy_in.copy_(dys[1])
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _step(recipe, graphed, x_in, dy_in, g, b, w, bias, ws)
    # capture records the step without running it: graphed is still at step 0
    for s in range(1, 5):
        _step(recipe, eager, xs[s], dys[s], g, b, w, bias, ws)
        torch.cuda.synchronize()
        want = _snapshot(eager)
        x_in.copy_(xs[s])
        dy_in.copy_(dys[s])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(graphed)
        for k in ["out", "dx", "dgamma", "dbeta", "dw", "dbias"]:
            assert torch.equal(got[k], want[k]), f"replay {s}: {k}"
        for m in ("mf", "mb"):
            for a, e in zip(got[m], want[m]):
                assert torch.equal(a, e), f"replay {s}: {m} state"
