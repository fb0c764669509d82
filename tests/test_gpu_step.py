"""The forward step with the scaling update folded in, against the two calls it
stands for (fp8ln_scaling_update, then the forward): the same history, scales,
codes, statistics and outputs, bit for bit, step after step, eagerly and from a
replayed HIP graph.  The two-call path is itself checked against the oracle by
the module tests, so this identity carries that parity over."""
import pytest
import torch

from fp8_delayed_scaling_row_amd import inputs, ops

pytestmark = pytest.mark.gpu


def _linear_state(M, K, N, recipe, training):
    mf, _ = ops.linear_metas(recipe)
    return dict(mf=mf, ctx=ops.LinearCtx(M, K, N, training=training),
                out=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))


def _linear_snapshot(st):
    c = st["ctx"]
    snap = dict(out=st["out"].clone(), hist=st["mf"].history.clone(),
                scale=st["mf"].scale.clone(), scale_inv=st["mf"].scale_inv.clone(),
                ln_q=c.ln_q.clone(), w_q=c.w_q.clone(), mean=c.mean.clone(),
                rstd=c.rstd.clone(), w_scale_inv=c.w_scale_inv.clone())
    if c.ln_qt is not None:
        snap.update(ln_qt=c.ln_qt.clone(), w_qt=c.w_qt.clone())
    return snap


def _same(a, b, what):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)   # bit patterns (NaN too)
        elif x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), f"{what}: {k} differs"


def _x(M, K, wl, s, poison):
    x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x", s), device="cuda")
    if poison and M > 3:
        x[1, 5] = float("nan")     # a NaN row amax enters the history
        x[3, 0] = float("inf")
    return x * (1.0 + 0.5 * s)


# (tokens, in, out, format, history length, margin, FP8 weight storage, training)
CASES = [
    (256, 768, 2304, ops.FORMAT_HYBRID, 16, 0, False, False),   # the pages' QKV layer
    (256, 768, 2304, ops.FORMAT_HYBRID, 16, 0, True, False),    # FP8 weight storage
    (130, 272, 144, ops.FORMAT_E4M3, 1024, 1, False, False),    # ragged, long window
    (64, 2048, 512, ops.FORMAT_E5M2, 16, 0, False, True),       # widest rows, transposes
    (8192, 2048, 2048, ops.FORMAT_HYBRID, 16, 0, False, False), # update as its own launch
    (0, 64, 32, ops.FORMAT_HYBRID, 16, 0, False, False),        # no tokens: the update only
]


@pytest.mark.parametrize("M,K,N,fmt,L,margin,reuse,training", CASES)
def test_ln_linear_fwd_step_equals_update_then_forward(M, K, N, fmt, L, margin, reuse, training):
    recipe = ops.Recipe(format=fmt, amax_history_len=L, margin=margin)
    wl = f"step-{M}x{K}x{N}"
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    bias = (torch.randn(N, device="cuda") * 0.1).to(torch.bfloat16)
    two, one = _linear_state(M, K, N, recipe, training), _linear_state(M, K, N, recipe, training)
    ws = ops.step_workspace()
    for s in range(6):
        x = _x(M, K, wl, s, poison=(s == 2 and M == 256 and not reuse))
        if reuse and s == 1:
            two["ctx"].reuse_weight_codes = one["ctx"].reuse_weight_codes = True
        ops.scaling_update(recipe, two["mf"])
        ops.ln_linear_fwd(recipe, x, g, b, w, bias, two["out"], two["mf"], two["ctx"])
        ops.ln_linear_fwd_step(recipe, x, g, b, w, bias, one["out"], one["mf"], one["ctx"], ws)
        torch.cuda.synchronize()
        _same(_linear_snapshot(two), _linear_snapshot(one), f"step {s}")
        assert int(ws.abs().sum().item()) == 0, f"step {s}: workspace not cleared"


def test_ln_linear_fwd_step_graph_replays_match_eager():
    M, K, N = 256, 768, 2304
    recipe = ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16)
    wl = "step-graph"
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    bias = (torch.randn(N, device="cuda") * 0.1).to(torch.bfloat16)
    xs = [_x(M, K, wl, s, poison=False) for s in range(5)]
    eager, graphed = _linear_state(M, K, N, recipe, False), _linear_state(M, K, N, recipe, False)
    ws = ops.step_workspace()
    x_in = torch.empty_like(xs[0])
    ops.scaling_update(recipe, eager["mf"])
    ops.ln_linear_fwd(recipe, xs[0], g, b, w, bias, eager["out"], eager["mf"], eager["ctx"])
    ops.ln_linear_fwd_step(recipe, xs[0], g, b, w, bias, graphed["out"], graphed["mf"],
                           graphed["ctx"], ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.ln_linear_fwd_step(recipe, x_in, g, b, w, bias, graphed["out"], graphed["mf"],
                               graphed["ctx"], ws)
    for s in range(1, 5):
        ops.scaling_update(recipe, eager["mf"])
        ops.ln_linear_fwd(recipe, xs[s], g, b, w, bias, eager["out"], eager["mf"], eager["ctx"])
        torch.cuda.synchronize()
        x_in.copy_(xs[s])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_linear_snapshot(eager), _linear_snapshot(graphed), f"replay {s}")
        assert int(ws.abs().sum().item()) == 0


def _mlp_state(M, H, F, recipe, training):
    mf, _ = ops.mlp_metas(recipe)
    return dict(mf=mf, ctx=ops.MlpCtx(M, H, F, training=training),
                out=torch.empty((M, H), dtype=torch.bfloat16, device="cuda"))


def _mlp_snapshot(st):
    c = st["ctx"]
    snap = dict(out=st["out"].clone(), hist=st["mf"].history.clone(),
                scale=st["mf"].scale.clone(), scale_inv=st["mf"].scale_inv.clone(),
                ln_q=c.ln_q.clone(), w1_q=c.w1_q.clone(), w2_q=c.w2_q.clone(), g_q=c.g_q.clone(),
                mean=c.mean.clone(), rstd=c.rstd.clone(), w_scale_inv=c.w_scale_inv.clone())
    for k in ("ln_qt", "w1_qt", "w2_qt", "g_qt", "h"):
        if getattr(c, k) is not None:
            snap[k] = getattr(c, k).clone()
    return snap


# (tokens, hidden, ffn, format, history length, activation, FP8 weight storage, training)
MLP_CASES = [
    (2048, 768, 3072, ops.FORMAT_E4M3, 16, ops.GELU_TANH, False, False),   # the pages' MLP
    (2048, 768, 3072, ops.FORMAT_E4M3, 16, ops.GELU_TANH, True, False),    # FP8 weights
    (144, 256, 400, ops.FORMAT_HYBRID, 1024, ops.GELU_ERF, False, True),   # ragged, long window
    (16384, 2048, 8192, ops.FORMAT_HYBRID, 16, ops.GELU_TANH, False, False),  # update apart
]


@pytest.mark.parametrize("M,H,F,fmt,L,act,reuse,training", MLP_CASES)
def test_ln_mlp_fwd_step_equals_update_then_forward(M, H, F, fmt, L, act, reuse, training):
    recipe = ops.Recipe(format=fmt, amax_history_len=L, activation=act)
    wl = f"mlp-step-{M}x{H}x{F}"
    g, b = inputs.layernorm_params(H, wl, device="cuda")
    w1 = inputs.linear_weight(F, H, wl, "w1", device="cuda")
    w2 = inputs.linear_weight(H, F, wl, "w2", device="cuda")
    b1 = (torch.randn(F, device="cuda") * 0.1).to(torch.bfloat16)
    b2 = (torch.randn(H, device="cuda") * 0.1).to(torch.bfloat16)
    two, one = _mlp_state(M, H, F, recipe, training), _mlp_state(M, H, F, recipe, training)
    ws = ops.step_workspace()
    for s in range(4 if M > 4096 else 6):
        x = _x(M, H, wl, s, poison=(s == 2 and M == 2048 and not reuse))
        if reuse and s == 1:
            two["ctx"].reuse_weight_codes = one["ctx"].reuse_weight_codes = True
        ops.scaling_update(recipe, two["mf"])
        ops.ln_mlp_fwd(recipe, x, g, b, w1, b1, w2, b2, two["out"], two["mf"], two["ctx"])
        ops.ln_mlp_fwd_step(recipe, x, g, b, w1, b1, w2, b2, one["out"], one["mf"], one["ctx"],
                            ws)
        torch.cuda.synchronize()
        _same(_mlp_snapshot(two), _mlp_snapshot(one), f"step {s}")
        assert int(ws.abs().sum().item()) == 0, f"step {s}: workspace not cleared"


# ---- backward steps -----------------------------------------------------------

def _dy(M, N, wl, s, poison):
    dy = inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy", s), std=1e-3, device="cuda")
    if poison and M > 3:
        dy[2, 7] = float("nan")    # a NaN gradient amax enters the backward history
        dy[3, 1] = float("-inf")
    return dy * (1.0 + 0.5 * s)


def _meta_snapshot(m):
    return dict(hist=m.history.clone(), scale=m.scale.clone(), scale_inv=m.scale_inv.clone())


# (tokens, in, out, format, history length, margin, backward slots)
LIN_BWD_CASES = [
    (2048, 768, 2304, ops.FORMAT_HYBRID, 16, 0, 1),    # the pages' QKV layer, 2048 tokens
    (272, 208, 144, ops.FORMAT_E4M3, 1024, 1, 1),      # ragged tiles, long window
    (64, 2048, 512, ops.FORMAT_E5M2, 16, 0, 2),        # E5M2 everywhere, an idle slot
    (96, 256, 128, ops.FORMAT_HYBRID, 16, 0, 3),       # 3 slots: the update as its own launch
]


@pytest.mark.parametrize("M,K,N,fmt,L,margin,slots", LIN_BWD_CASES)
def test_ln_linear_bwd_step_equals_update_then_backward(M, K, N, fmt, L, margin, slots):
    recipe = ops.Recipe(format=fmt, amax_history_len=L, margin=margin)
    wl = f"bwd-step-{M}x{K}x{N}"
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    mf, _ = ops.linear_metas(recipe)
    ctx = ops.LinearCtx(M, K, N, training=True)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mbs = [ops.Meta(recipe, slots, ops.META_BACKWARD) for _ in range(2)]
    h0 = torch.rand((L, slots), device="cuda") * 1e-2   # every slot's history has values
    for m in mbs:
        m.history.copy_(h0)
    grads = [dict(dx=torch.empty((M, K), dtype=torch.bfloat16, device="cuda"),
                  dgamma=torch.empty(K, device="cuda"), dbeta=torch.empty(K, device="cuda"),
                  dw=torch.empty((N, K), device="cuda"), db=torch.empty(N, device="cuda"))
             for _ in range(2)]
    ws = ops.step_workspace()
    for s in range(5):
        x = _x(M, K, wl, s, poison=False)
        ops.scaling_update(recipe, mf)
        ops.ln_linear_fwd(recipe, x, g, b, w, None, out, mf, ctx)
        dy = _dy(M, N, wl, s, poison=(s == 2 and M == 272))
        a, c = grads
        ops.scaling_update(recipe, mbs[0])
        ops.ln_linear_bwd(recipe, dy, x, g, ctx, mf, mbs[0], a["dx"], a["dgamma"], a["dbeta"],
                          a["dw"], a["db"])
        ops.ln_linear_bwd_step(recipe, dy, x, g, ctx, mf, mbs[1], c["dx"], c["dgamma"],
                               c["dbeta"], c["dw"], ws, c["db"])
        torch.cuda.synchronize()
        _same(dict(a, **_meta_snapshot(mbs[0])), dict(c, **_meta_snapshot(mbs[1])), f"step {s}")
        assert int(ws.abs().sum().item()) == 0, f"step {s}: workspace not cleared"


def test_ln_linear_bwd_step_graph_replays_match_eager():
    M, K, N = 2048, 768, 2304
    recipe = ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16)
    wl = "bwd-step-graph"
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    mf, _ = ops.linear_metas(recipe)
    ctx = ops.LinearCtx(M, K, N, training=True)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    x = _x(M, K, wl, 0, poison=False)
    ops.scaling_update(recipe, mf)
    ops.ln_linear_fwd(recipe, x, g, b, w, None, out, mf, ctx)
    dys = [_dy(M, N, wl, s, poison=False) for s in range(5)]
    mbs = [ops.Meta(recipe, 1, ops.META_BACKWARD) for _ in range(2)]
    grads = [dict(dx=torch.empty((M, K), dtype=torch.bfloat16, device="cuda"),
                  dgamma=torch.empty(K, device="cuda"), dbeta=torch.empty(K, device="cuda"),
                  dw=torch.empty((N, K), device="cuda"), db=torch.empty(N, device="cuda"))
             for _ in range(2)]
    a, c = grads
    ws = ops.step_workspace()
    wsp = torch.empty(ops.workspace_size(ops.OP_LN_LINEAR_BWD, M, K, N), dtype=torch.uint8,
                      device="cuda")
    dy_in = torch.empty_like(dys[0])

    def eager(dy):
        ops.scaling_update(recipe, mbs[0])
        ops.ln_linear_bwd(recipe, dy, x, g, ctx, mf, mbs[0], a["dx"], a["dgamma"], a["dbeta"],
                          a["dw"], a["db"])

    def stepped():
        ops.ln_linear_bwd_step(recipe, dy_in, x, g, ctx, mf, mbs[1], c["dx"], c["dgamma"],
                               c["dbeta"], c["dw"], ws, c["db"], workspace=wsp)

    eager(dys[0])
    dy_in.copy_(dys[0])
    stepped()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stepped()
    for s in range(1, 5):
        eager(dys[s])
        torch.cuda.synchronize()
        dy_in.copy_(dys[s])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(dict(a, **_meta_snapshot(mbs[0])), dict(c, **_meta_snapshot(mbs[1])), f"replay {s}")
        assert int(ws.abs().sum().item()) == 0


# (tokens, hidden, ffn, format, history length, activation, backward slots)
MLP_BWD_CASES = [
    (2048, 768, 3072, ops.FORMAT_HYBRID, 16, ops.GELU_TANH, 2),    # the pages' MLP
    (144, 256, 400, ops.FORMAT_E4M3, 1024, ops.GELU_ERF, 2),       # ragged, long window
    (96, 256, 512, ops.FORMAT_HYBRID, 16, ops.GELU_TANH, 3),       # 3 slots: apart
    (4096, 2048, 8192, ops.FORMAT_HYBRID, 16, ops.GELU_TANH, 2),   # large tiles
]


@pytest.mark.parametrize("M,H,F,fmt,L,act,slots", MLP_BWD_CASES)
def test_ln_mlp_bwd_step_equals_update_then_backward(M, H, F, fmt, L, act, slots):
    recipe = ops.Recipe(format=fmt, amax_history_len=L, activation=act)
    wl = f"mlp-bwd-step-{M}x{H}x{F}"
    g, b = inputs.layernorm_params(H, wl, device="cuda")
    w1 = inputs.linear_weight(F, H, wl, "w1", device="cuda")
    w2 = inputs.linear_weight(H, F, wl, "w2", device="cuda")
    b1 = (torch.randn(F, device="cuda") * 0.1).to(torch.bfloat16)
    mf, _ = ops.mlp_metas(recipe)
    ctx = ops.MlpCtx(M, H, F, training=True)
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    mbs = [ops.Meta(recipe, slots, ops.META_BACKWARD) for _ in range(2)]
    h0 = torch.rand((L, slots), device="cuda") * 1e-2
    for m in mbs:
        m.history.copy_(h0)
    grads = [dict(dx=torch.empty((M, H), dtype=torch.bfloat16, device="cuda"),
                  dgamma=torch.empty(H, device="cuda"), dbeta=torch.empty(H, device="cuda"),
                  dw1=torch.empty((F, H), device="cuda"), db1=torch.empty(F, device="cuda"),
                  dw2=torch.empty((H, F), device="cuda"), db2=torch.empty(H, device="cuda"))
             for _ in range(2)]
    ws = ops.step_workspace()
    for s in range(3 if M > 2048 else 5):
        x = _x(M, H, wl, s, poison=False)
        ops.scaling_update(recipe, mf)
        ops.ln_mlp_fwd(recipe, x, g, b, w1, b1, w2, None, out, mf, ctx)
        dy = _dy(M, H, wl, s, poison=(s == 2 and M == 144))
        a, c = grads
        ops.scaling_update(recipe, mbs[0])
        ops.ln_mlp_bwd(recipe, dy, x, g, ctx, mf, mbs[0], a["dx"], a["dgamma"], a["dbeta"],
                       a["dw1"], a["db1"], a["dw2"], a["db2"])
        ops.ln_mlp_bwd_step(recipe, dy, x, g, ctx, mf, mbs[1], c["dx"], c["dgamma"], c["dbeta"],
                            c["dw1"], c["db1"], c["dw2"], c["db2"], ws)
        torch.cuda.synchronize()
        _same(dict(a, **_meta_snapshot(mbs[0])), dict(c, **_meta_snapshot(mbs[1])), f"step {s}")
        assert int(ws.abs().sum().item()) == 0, f"step {s}: workspace not cleared"
