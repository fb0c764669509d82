"""Benchmark of the FP8 delayed-scaling LayerNorm path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu-baseline]

The headline line times the standalone LayerNorm + FP8 E4M3 cast + per-tensor
amax step on 65536 rows x 2048 (0.1 % of entries x100, input scale drifting
1 -> 4 over 32 steps, amax history 1024): one step is the scale update plus the
fused kernel over one of 32 resident input buffers.  `value` is GB/s of
algorithmic traffic (2 B read + 1 B written per element, 8 B of row statistics
per row).  Further workloads (the pages' GPT-style shapes: LayerNormLinear
768 -> 2304 forward on 8 x 32 tokens and backward on 8 x 256 tokens,
LayerNormMLP 768 -> 3072 -> 768 forward on 8 x 256 tokens, and the
2048 / 8192 / 12-layer scale-up on 64 x 256 tokens, fwd + bwd) are reported in
"workloads" with TFLOP/s against the FP8 MFMA peak, and the same modules without
FP8 (bf16 GEMMs, "_bf16" workloads, against the BF16 MFMA peak) with the FP8
speedup over them, the comparison the pages make.

Step times are replays of consecutive steps captured once in a HIP graph (the
same kernels on the same buffers, without host launch gaps); the host-launched
step time is reported beside them as eager_ms_per_step.  The roofline's kernel
duration comes from HIP events around graph-replayed back-to-back launches of that
kernel (an event pair around each host-launched kernel is reported beside it).

Every input is synthetic and generated on the device before timing.  The CPU
baseline runs the C++ oracle (float64, OpenMP on the host's cores) on a bounded
sample of the headline workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LayerNormLinear FP8 fwd TFLOP/s (% MFMA peak); LN+cast+amax GB/s (% HBM)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, TFLOP/s
PROFILE_DIR = os.path.join(ROOT, "profiles")
# sources of the headline LayerNorm kernel (a counter summary holds for these only)
LN_SOURCES = ["layernorm.hip", "ln_fwd_body.hpp", "device_common.hpp"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=32)
    p.add_argument("--warmup", type=int, default=32)
    p.add_argument("--quick", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default=None, help="run one named workload")
    p.add_argument("--profile-ln", type=int, default=0, metavar="N",
                   help="counter run: N headline launches plus 3 plain 1 GiB copies")
    p.add_argument("--profile-gemm", type=int, nargs=4, metavar=("M", "N", "K", "REPS"),
                   help="counter run: REPS launches of one E4M3 GEMM (fp32 output)")
    p.add_argument("--profile-kernel", nargs=2, metavar=("KIND", "REPS"),
                   help="counter run: REPS launches of one kernel of the 16384-token "
                        "scale-up layer: fc1, fc2_dgrad, fc2_fwd, wgrad, ln_bwd, cast_dy, "
                        "cast_w (plus 3 plain 1 GiB copies for the HBM calibration)")
    p.add_argument("--bf16", action="store_true",
                   help="with --profile-gemm: the bf16 GEMM instead of the FP8 one")
    p.add_argument("--oracle-workloads", action="store_true",
                   help="time the oracle on each GEMM-bound workload's shapes (host only)")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write the counter summary of a --profile-ln run to profiles/")
    return p.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "fp8_delayed_scaling_row_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(kernel_tag, src_names):
    """HBM bytes per launch from a committed counter summary, if it was taken on
    the current kernel source (else None)."""
    path = os.path.join(PROFILE_DIR, f"{kernel_tag}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != source_hash(*src_names):
        return None
    return d.get("hbm_bytes_per_launch")


class Timer:
    """HIP events on the stream the kernels run on (torch's current stream)."""

    def __init__(self, torch):
        self.t = torch
        self.pairs = []

    def start(self):
        e = self.t.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, s):
        e = self.t.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.append((s, e))

    def mean_ms(self):
        self.t.cuda.synchronize()
        if not self.pairs:
            return float("nan")
        return sum(a.elapsed_time(b) for a, b in self.pairs) / len(self.pairs)


# ---- headline: LN + cast + amax ----------------------------------------------

def bench_ln_cast(torch, ops, inputs, steps, warmup):
    rows, hidden, n_buf = 65536, 2048, 32
    recipe = ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=1024)
    wl = "ln_cast_amax_65536x2048"
    xs = [inputs.spiky_normal_bf16((rows, hidden), inputs.seed_for(wl, "x", s),
                                   drift=inputs.drift_factor(s, n_buf), device="cuda")
          for s in range(n_buf)]
    g, b = inputs.layernorm_params(hidden, wl, device="cuda")
    meta = ops.Meta(recipe, 1, ops.META_FORWARD)
    out = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    scale = meta.scale[0:1]
    amax = meta.amax_ptr(0)

    def step(s, timer=None):
        ops.scaling_update(recipe, meta)
        ev = timer.start() if timer else None
        ops.ln_cast_amax(recipe, xs[s % n_buf], g, b, ops.E4M3, scale, amax, out, None, mean, rstd)
        if timer:
            timer.stop(ev)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    # whole steps replayed from a HIP graph of n_buf consecutive steps (one per
    # input buffer), so no host launch gap sits between the update and the kernel;
    # the capture's warm run also sweeps every input buffer once more
    ms = _graph_ms(torch, step, n_buf, max(1, steps // n_buf)) / n_buf
    # host-launched steps, the kernel timed alone with HIP events on its stream
    kt = Timer(torch)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        step(s, kt)
    t1.record()
    torch.cuda.synchronize()
    eager_ms = t0.elapsed_time(t1) / steps
    event_kernel_ms = kt.mean_ms()   # one event pair around each host-launched kernel

    # The kernel alone: n_buf back-to-back launches (one per input buffer) in a HIP
    # graph, HIP events around the replays on the launch stream.  The event pairs
    # above also hold each launch's dispatch; this is the kernel's own duration,
    # which the kernel trace of the same command reports.
    def ln_only(s):
        ops.ln_cast_amax(recipe, xs[s % n_buf], g, b, ops.E4M3, scale, amax, out, None, mean,
                         rstd)

    kernel_ms = _graph_ms(torch, ln_only, n_buf, max(2, steps // n_buf)) / n_buf
    bytes_step = rows * hidden * 3 + rows * 8
    return dict(rows=rows, hidden=hidden, ms=ms, eager_ms=eager_ms, kernel_ms=kernel_ms,
                event_kernel_ms=event_kernel_ms, bytes=bytes_step,
                scale=float(meta.scale[0].item()))


COPY_BYTES = 1 << 30     # each calibration copy reads and writes this many bytes
PROBE_ELEMS = 1 << 29    # stream probe: 1 GiB of bf16 read, 512 MiB of bytes written


def stream_probe_gbs(torch, ops, reps=10):
    """GB/s of the library's streaming probe (fp8ln_stream_probe): the LayerNorm +
    cast step's traffic, 2 B read and 1 B written per element with non-temporal
    accesses and no arithmetic, over 1.5 GiB per launch (past the 256 MB
    last-level cache), HIP events on the launch stream."""
    x = torch.empty(PROBE_ELEMS, dtype=torch.bfloat16, device="cuda").fill_(1.5)
    out = torch.empty(PROBE_ELEMS, dtype=torch.uint8, device="cuda")
    ops.stream_probe(x, out)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        ops.stream_probe(x, out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del x, out
    torch.cuda.empty_cache()
    return 3 * PROBE_ELEMS / (ms * 1e-3) / 1e9


def copy_ceiling_gbs(torch, reps=10):
    """Read + write GB/s of a plain device-to-device copy of 1 GiB (torch's copy
    kernel) on this machine: a practical ceiling for a streaming kernel, next to the
    8 TB/s of the spec sheet."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def profile_ln(torch, ops, inputs, n):
    """Launches for a rocprofv3 --pmc run: n headline LayerNorm+cast launches and
    three elementwise copies (neg) of a 1 GiB bf16 tensor, a plain kernel of known
    traffic to calibrate FETCH_SIZE / WRITE_SIZE."""
    rows, hidden = 65536, 2048
    recipe = ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=1024)
    wl = "ln_cast_amax_65536x2048"
    xs = [inputs.spiky_normal_bf16((rows, hidden), inputs.seed_for(wl, "x", s),
                                   drift=inputs.drift_factor(s, 32), device="cuda")
          for s in range(min(n, 4))]
    g, b = inputs.layernorm_params(hidden, wl, device="cuda")
    meta = ops.Meta(recipe, 1, ops.META_FORWARD)
    out = torch.empty((rows, hidden), dtype=torch.uint8, device="cuda")
    mean = torch.empty(rows, dtype=torch.float32, device="cuda")
    rstd = torch.empty(rows, dtype=torch.float32, device="cuda")
    for s in range(n):
        ops.scaling_update(recipe, meta)
        ops.ln_cast_amax(recipe, xs[s % len(xs)], g, b, ops.E4M3, meta.scale[0:1],
                         meta.amax_ptr(0), out, None, mean, rstd)
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps(dict(profile_ln=n, copies=3, copy_bytes=COPY_BYTES)), flush=True)


def profile_kernel(torch, ops, inputs, kind, reps):
    """Launches for a rocprofv3 run on one kernel of the scale-up layer (16384
    tokens, 2048 -> 8192 -> 2048, HYBRID): the GEMMs with their step's epilogues
    and operand formats, the LayerNorm backward and the casts; then three
    elementwise copies of a 1 GiB bf16 tensor (FETCH_SIZE / WRITE_SIZE
    calibration)."""
    M, H, F = 16384, 2048, 8192
    E4, E5 = ops.E4M3, ops.E5M2
    one = torch.ones(1, device="cuda")
    amax = torch.zeros(1, device="cuda")
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    wl = "profile"
    if kind == "fc1":
        a, b, q, qt, h = _codes(torch, M, H), _codes(torch, F, H), u8(M, F), u8(F, M), bf(M, F)
        fn = lambda: ops.gemm_gelu_fp8(a, E4, b, E4, one, one, E4, one, amax.data_ptr(), q, qt, h)
    elif kind == "fc2_dgrad":
        a, b, q, qt = _codes(torch, M, H), _codes(torch, F, H), u8(M, F), u8(F, M)
        h = (torch.randn((M, F), device="cuda") * 2).to(torch.bfloat16)
        db = torch.empty(F, device="cuda")
        ws = torch.empty(ops.workspace_size(ops.OP_GEMM_DGELU_FP8, M, F), dtype=torch.uint8,
                         device="cuda")
        fn = lambda: ops.gemm_dgelu_fp8(a, E5, b, E4, one, one, h, E5, one, amax.data_ptr(), q,
                                        qt, db, workspace=ws)
    elif kind == "fc2_fwd":
        a, b, o = _codes(torch, M, F), _codes(torch, H, F), bf(M, H)
        fn = lambda: ops.gemm(a, E4, b, E4, one, one, o)
    elif kind == "wgrad":
        a, b = _codes(torch, F, M), _codes(torch, H, M)
        o = torch.empty((F, H), device="cuda")
        fn = lambda: ops.gemm(a, E5, b, E4, one, one, o)
    elif kind == "ln_bwd":
        x = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"), device="cuda")
        g, _ = inputs.layernorm_params(H, wl, device="cuda")
        dln = torch.randn((M, H), device="cuda") * 1e-3
        mean = x.float().mean(dim=1)
        rstd = torch.rsqrt(x.float().var(dim=1, unbiased=False) + 1e-5)
        dx, dg, db = bf(M, H), torch.empty(H, device="cuda"), torch.empty(H, device="cuda")
        fn = lambda: ops.layernorm_bwd(dln, x, mean, rstd, g, dx, dg, db)
    elif kind == "cast_dy":
        dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy"), std=1e-3, device="cuda")
        q, qt, cs = u8(M, H), u8(H, M), torch.empty(H, device="cuda")
        fn = lambda: ops.cast_amax(dy, E5, one, amax.data_ptr(), q, qt, cs)
    elif kind == "cast_w":
        w = inputs.linear_weight(F, H, wl, "w1", device="cuda")
        q, qt = u8(F, H), u8(H, F)
        fn = lambda: ops.cast_amax(w, E4, one, amax.data_ptr(), q, qt)
    else:
        raise SystemExit(f"unknown kernel kind {kind!r}")
    for _ in range(reps):
        fn()
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps(dict(profile_kernel=kind, reps=reps, copies=3, copy_bytes=COPY_BYTES)),
          flush=True)


def _read_counter_csv(path, counter):
    """{kernel name: [values per dispatch]} for one counter of a rocprofv3 csv."""
    import csv
    per = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return per


def summarize_counters(fetch_csv, write_csv):
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")

    def pick(d, key):
        names = [k for k in d if key in k]
        if not names:
            raise SystemExit(f"no kernel matching {key!r} in the counter file")
        vals = d[names[0]]
        return names[0], sum(vals) / len(vals)

    ln_name, ln_fetch = pick(fetch, "ln_cast_amax_kernel")
    _, ln_write = pick(write, "ln_cast_amax_kernel")
    cp_name, cp_fetch = pick(fetch, "neg")
    _, cp_write = pick(write, "neg")
    # counters are in KiB per dispatch; the copy moves COPY_BYTES each way
    f_read = COPY_BYTES / (cp_fetch * 1024.0)
    f_write = COPY_BYTES / (cp_write * 1024.0)
    rows, hidden = 65536, 2048
    read_b = ln_fetch * 1024.0 * f_read
    write_b = ln_write * 1024.0 * f_write
    d = dict(kernel=ln_name, workload="ln_cast_amax_65536x2048",
             source_hash=source_hash(*LN_SOURCES),
             fetch_kib_per_launch=ln_fetch, write_kib_per_launch=ln_write,
             copy_kernel=cp_name, copy_fetch_kib=cp_fetch, copy_write_kib=cp_write,
             copy_scale_read=f_read, copy_scale_write=f_write,
             hbm_read_bytes_per_launch=read_b, hbm_write_bytes_per_launch=write_b,
             hbm_bytes_per_launch=read_b + write_b,
             algorithmic_bytes_per_launch=rows * hidden * 3 + rows * 8,
             commands=["rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch --output-format csv -- "
                       "python bench.py --profile-ln 8",
                       "rocprofv3 --pmc WRITE_SIZE -d <dir> -o write --output-format csv -- "
                       "python bench.py --profile-ln 8",
                       "python bench.py --summarize-counters <fetch csv> <write csv>"])
    os.makedirs(PROFILE_DIR, exist_ok=True)
    path = os.path.join(PROFILE_DIR, "ln_cast_amax_65536x2048_counters.json")
    with open(path, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d))


# ---- GEMM-bound workloads ------------------------------------------------------

def gemm_kernel_ms(torch, ops, M, N, K, out_dtype, reps=20, bf16=False):
    """Average duration of one fp8ln_gemm (or fp8ln_gemm_bf16) launch at this
    shape: `reps` launches captured in a HIP graph and replayed, timed with HIP
    events on the replay stream (no host launch overhead between them)."""
    out = torch.empty((M, N), dtype=out_dtype, device="cuda")
    if bf16:
        a = torch.randn((M, K), device="cuda").to(torch.bfloat16)
        b = torch.randn((N, K), device="cuda").to(torch.bfloat16)
    else:
        a = torch.randint(0, 0x77, (M, K), dtype=torch.uint8, device="cuda")
        b = torch.randint(0, 0x77, (N, K), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")

    def launches(_):
        for _ in range(reps):
            if bf16:
                ops.gemm_bf16(a, b, out)
            else:
                ops.gemm(a, ops.E4M3, b, ops.E4M3, one, one, out)

    return _graph_ms(torch, launches, 1, 3) / reps


def _codes(torch, *shape):
    """Random finite FP8 codes of both signs (0x77 keeps E4M3 and E5M2 finite)."""
    c = torch.randint(0, 0x77, shape, dtype=torch.uint8, device="cuda")
    return c | (torch.randint(0, 2, shape, dtype=torch.uint8, device="cuda") << 7)


def mlp_gemm_kinds(torch, ops, M, H, F, backward, bwd_fp8=None, reps=10):
    """Each GEMM of one LayerNormMLP layer step launched alone through the C-ABI
    entry point that runs the same kernel (tile, epilogue, operand formats) as
    the module step: average ms per launch over `reps` graph-replayed launches,
    TFLOP/s and fraction of the FP8 peak."""
    E4 = ops.E4M3
    bf = ops.E5M2 if bwd_fp8 is None else bwd_fp8
    one = torch.ones(1, device="cuda")
    amax = torch.zeros(1, device="cuda")
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device="cuda")
    out = []

    def run(name, m, n, k, make):
        fn = make()
        ms = _graph_ms(torch, lambda _: [fn() for _ in range(reps)], 1, 3) / reps
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        out.append(dict(kind=name, mnk=[m, n, k], kernel_ms=round(ms, 5),
                        achieved=round(tf, 1), frac=round(tf / FP8_PEAK_TFLOPS, 4)))
        torch.cuda.empty_cache()

    def fc1():
        a, b, q, qt = _codes(torch, M, H), _codes(torch, F, H), u8(M, F), u8(F, M)
        h = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
        return lambda: ops.gemm_gelu_fp8(a, E4, b, E4, one, one, E4, one, amax.data_ptr(), q,
                                         q_out_t=qt if backward else None,
                                         h_out=h if backward else None)

    def fc2():
        a, b = _codes(torch, M, F), _codes(torch, H, F)
        o = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        return lambda: ops.gemm(a, E4, b, E4, one, one, o)

    run("fc1 fwd: GELU epilogue" + (", bf16 h, FP8 codes + transpose" if backward else
                                     ", FP8 codes"), M, F, H, fc1)
    run("fc2 fwd: bf16 out", M, H, F, fc2)
    if backward:
        def dgrad2():
            a, b = _codes(torch, M, H), _codes(torch, F, H)
            h = (torch.randn((M, F), device="cuda") * 2).to(torch.bfloat16)
            q, qt = u8(M, F), u8(F, M)
            db = torch.empty(F, device="cuda")
            ws = torch.empty(ops.workspace_size(ops.OP_GEMM_DGELU_FP8, M, F), dtype=torch.uint8,
                             device="cuda")
            return lambda: ops.gemm_dgelu_fp8(a, bf, b, E4, one, one, h, bf, one,
                                              amax.data_ptr(), q, qt, db, workspace=ws)

        def fp32(m, n, k):
            def make():
                a, b = _codes(torch, m, k), _codes(torch, n, k)
                o = torch.empty((m, n), device="cuda")
                return lambda: ops.gemm(a, bf, b, E4, one, one, o)
            return make

        run("fc2 dgrad: GELU' + dH FP8 cast, transpose, dbias partials", M, F, H, dgrad2)
        run("fc2 wgrad: fp32 out", H, F, M, fp32(H, F, M))
        run("fc1 dgrad: fp32 out", M, H, F, fp32(M, H, F))
        run("fc1 wgrad: fp32 out", F, H, M, fp32(F, H, M))
    return out


def _graph_ms(torch, step, unroll, replays):
    """Capture steps 0 .. unroll-1 in one HIP graph (after a warm run on the
    capture stream) and return the average replay time in ms."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in range(unroll):
            step(s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(unroll):
            step(s)
    graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / replays
    del graph
    return ms


def bench_linear_fwd(torch, ops, inputs, steps, warmup, M=256, K=768, N=2304, reuse=False):
    recipe = ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16)
    wl = f"ln_linear_fwd_{M}x{K}x{N}"
    xs = [inputs.normal_bf16((M, K), inputs.seed_for(wl, "x", s), device="cuda") for s in range(16)]
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    bias = torch.zeros(N, dtype=torch.bfloat16, device="cuda")
    mf, _ = ops.linear_metas(recipe)
    ctx = ops.LinearCtx(M, K, N, training=False)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = ops.step_workspace()
    if reuse:   # FP8 weight storage: cast once, then reuse the codes
        ops.ln_linear_fwd_step(recipe, xs[0], g, b, w, bias, out, mf, ctx, ws)
        ctx.reuse_weight_codes = True

    def step(s):
        # the step's scaling update and forward (the update folded into the
        # forward's first launch)
        ops.ln_linear_fwd_step(recipe, xs[s % 16], g, b, w, bias, out, mf, ctx, ws)

    t = _time_steps(torch, step, steps, warmup, unroll=16)
    flops = 2.0 * M * N * K
    return dict(t, flops=flops, gemm=(M, N, K, torch.bfloat16))


def bench_linear_bwd(torch, ops, inputs, steps, warmup, M=2048, K=768, N=2304):
    recipe = ops.Recipe(format=ops.FORMAT_HYBRID, amax_history_len=16)
    wl = f"ln_linear_bwd_{M}x{K}x{N}"
    x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x"), device="cuda")
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    dys = [inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy", s), std=1e-3, device="cuda")
           for s in range(4)]
    mf, mb = ops.linear_metas(recipe)
    ctx = ops.LinearCtx(M, K, N, training=True)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dgamma = torch.empty(K, device="cuda")
    dbeta = torch.empty(K, device="cuda")
    dw = torch.empty((N, K), device="cuda")
    dbias = torch.empty(N, device="cuda")
    ws = torch.empty(ops.workspace_size(ops.OP_LN_LINEAR_BWD, M, K, N), dtype=torch.uint8, device="cuda")
    ops.scaling_update(recipe, mf)
    ops.ln_linear_fwd(recipe, x, g, b, w, None, out, mf, ctx)
    step_ws = ops.step_workspace()

    def step(s):
        # the backward state's scaling update folded into the gradient cast
        ops.ln_linear_bwd_step(recipe, dys[s % 4], x, g, ctx, mf, mb, dx, dgamma, dbeta, dw,
                               step_ws, dbias, workspace=ws)

    t = _time_steps(torch, step, steps, warmup, unroll=4)
    flops = 2 * 2.0 * M * N * K
    return dict(t, flops=flops, gemm=(N, K, M, torch.float32))


def bench_mlp_fwd(torch, ops, inputs, steps, warmup, M=2048, H=768, F=3072, reuse=False):
    recipe = ops.Recipe(format=ops.FORMAT_E4M3, amax_history_len=16)
    wl = f"ln_mlp_fwd_{M}x{H}x{F}"
    xs = [inputs.normal_bf16((M, H), inputs.seed_for(wl, "x", s), device="cuda") for s in range(4)]
    g, b = inputs.layernorm_params(H, wl, device="cuda")
    w1 = inputs.linear_weight(F, H, wl, "w1", device="cuda")
    w2 = inputs.linear_weight(H, F, wl, "w2", device="cuda")
    mf, _ = ops.mlp_metas(recipe)
    ctx = ops.MlpCtx(M, H, F, training=False)
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = ops.step_workspace()
    if reuse:   # FP8 weight storage: cast once, then reuse the codes
        ops.ln_mlp_fwd_step(recipe, xs[0], g, b, w1, None, w2, None, out, mf, ctx, ws)
        ctx.reuse_weight_codes = True

    def step(s):
        # the step's scaling update and forward (the update folded in)
        ops.ln_mlp_fwd_step(recipe, xs[s % 4], g, b, w1, None, w2, None, out, mf, ctx, ws)

    t = _time_steps(torch, step, steps, warmup, unroll=4)
    flops = 2 * 2.0 * M * H * F
    return dict(t, flops=flops, gemm=(M, F, H, torch.bfloat16), kinds=(M, H, F, False))


def bench_linear_fwd_bf16(torch, ops, inputs, steps, warmup, M=256, K=768, N=2304):
    wl = f"ln_linear_fwd_{M}x{K}x{N}"
    xs = [inputs.normal_bf16((M, K), inputs.seed_for(wl, "x", s), device="cuda") for s in range(16)]
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    bias = torch.zeros(N, dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ln_out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")

    def step(s):
        ops.ln_linear_fwd_bf16(xs[s % 16], g, b, w, bias, out, ln_out)

    t = _time_steps(torch, step, steps, warmup, unroll=16)
    return dict(t, flops=2.0 * M * N * K, gemm=(M, N, K, torch.bfloat16), bf16=True)


def bench_linear_bwd_bf16(torch, ops, inputs, steps, warmup, M=2048, K=768, N=2304):
    wl = f"ln_linear_bwd_{M}x{K}x{N}"
    x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x"), device="cuda")
    g, b = inputs.layernorm_params(K, wl, device="cuda")
    w = inputs.linear_weight(N, K, wl, "w", device="cuda")
    dys = [inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy", s), std=1e-3, device="cuda")
           for s in range(4)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ln_out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    mean = torch.empty(M, device="cuda")
    rstd = torch.empty(M, device="cuda")
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dgamma = torch.empty(K, device="cuda")
    dbeta = torch.empty(K, device="cuda")
    dw = torch.empty((N, K), device="cuda")
    dbias = torch.empty(N, device="cuda")
    ws = torch.empty(ops.workspace_size(ops._abi.OP_LN_LINEAR_BWD_BF16, M, K, N),
                     dtype=torch.uint8, device="cuda")
    ops.ln_linear_fwd_bf16(x, g, b, w, None, out, ln_out, mean, rstd)

    def step(s):
        ops.ln_linear_bwd_bf16(dys[s % 4], x, g, w, ln_out, mean, rstd, dx, dgamma, dbeta, dw,
                               dbias, workspace=ws)

    t = _time_steps(torch, step, steps, warmup, unroll=4)
    return dict(t, flops=2 * 2.0 * M * N * K, gemm=(N, K, M, torch.float32), bf16=True)


def bench_mlp_fwd_bf16(torch, ops, inputs, steps, warmup, M=2048, H=768, F=3072):
    wl = f"ln_mlp_fwd_{M}x{H}x{F}"
    xs = [inputs.normal_bf16((M, H), inputs.seed_for(wl, "x", s), device="cuda") for s in range(4)]
    g, b = inputs.layernorm_params(H, wl, device="cuda")
    w1 = inputs.linear_weight(F, H, wl, "w1", device="cuda")
    w2 = inputs.linear_weight(H, F, wl, "w2", device="cuda")
    out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ln_out = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    gg = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")

    def step(s):
        ops.ln_mlp_fwd_bf16(xs[s % 4], g, b, w1, None, w2, None, out, ln_out, gg)

    t = _time_steps(torch, step, steps, warmup, unroll=4)
    return dict(t, flops=2 * 2.0 * M * H * F, gemm=(M, F, H, torch.bfloat16), bf16=True)


def bench_mlp_stack(torch, ops, inputs, steps, warmup, fmt, M=16384, H=2048, F=8192, layers=12):
    recipe = ops.Recipe(format=fmt, amax_history_len=1024)
    wl = f"ln_mlp_x{layers}_{M}x{H}x{F}"
    x0 = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"), device="cuda")
    dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy"), std=1e-3, device="cuda")
    L = []
    for l in range(layers):
        g, b = inputs.layernorm_params(H, f"{wl}/{l}", device="cuda")
        w1 = inputs.linear_weight(F, H, f"{wl}/{l}", "w1", device="cuda")
        w2 = inputs.linear_weight(H, F, f"{wl}/{l}", "w2", device="cuda")
        mf, mb = ops.mlp_metas(recipe)
        L.append(dict(g=g, b=b, w1=w1, w2=w2, mf=mf, mb=mb, ctx=ops.MlpCtx(M, H, F),
                      out=torch.empty((M, H), dtype=torch.bfloat16, device="cuda"),
                      dw1=torch.empty((F, H), device="cuda"), db1=torch.empty(F, device="cuda"),
                      dw2=torch.empty((H, F), device="cuda"), db2=torch.empty(H, device="cuda"),
                      dg=torch.empty(H, device="cuda"), dbt=torch.empty(H, device="cuda")))
    dxs = [torch.empty((M, H), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = torch.empty(ops.workspace_size(ops.OP_LN_MLP_BWD, M, H, F), dtype=torch.uint8, device="cuda")

    metas = [d["mf"] for d in L] + [d["mb"] for d in L]

    def step(s):
        # every state block of the model advances at the step's start in one
        # launch (each block's update reads only its own history, which none of
        # the step's other kernels has touched yet)
        ops.scaling_update_batch(recipe, metas)
        x = x0
        for d in L:
            ops.ln_mlp_fwd(recipe, x, d["g"], d["b"], d["w1"], None, d["w2"], None, d["out"],
                           d["mf"], d["ctx"])
            x = d["out"]
        grad = dy
        for i, d in enumerate(reversed(L)):
            xin = x0 if i == layers - 1 else L[layers - 2 - i]["out"]
            dx = dxs[i % 2]
            ops.ln_mlp_bwd(recipe, grad, xin, d["g"], d["ctx"], d["mf"], d["mb"], dx, d["dg"],
                           d["dbt"], d["dw1"], d["db1"], d["dw2"], d["db2"], workspace=ws)
            grad = dx

    t = _time_steps(torch, step, steps, warmup, unroll=1)
    flops = layers * 6 * 2.0 * M * H * F
    bwd = ops.E4M3 if fmt == ops.FORMAT_E4M3 else ops.E5M2
    return dict(t, flops=flops, gemm=(M, F, H, torch.float32), kinds=(M, H, F, True, bwd))


def bench_mlp_stack_bf16(torch, ops, inputs, steps, warmup, M=16384, H=2048, F=8192, layers=12):
    """The 12-layer stack of bench_mlp_stack without FP8 (same inputs)."""
    wl = f"ln_mlp_x{layers}_{M}x{H}x{F}"
    x0 = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"), device="cuda")
    dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy"), std=1e-3, device="cuda")
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device="cuda")
    f32 = lambda *s: torch.empty(s, device="cuda")
    L = []
    for l in range(layers):
        g, b = inputs.layernorm_params(H, f"{wl}/{l}", device="cuda")
        w1 = inputs.linear_weight(F, H, f"{wl}/{l}", "w1", device="cuda")
        w2 = inputs.linear_weight(H, F, f"{wl}/{l}", "w2", device="cuda")
        L.append(dict(g=g, b=b, w1=w1, w2=w2, out=bf(M, H), ln=bf(M, H), h=bf(M, F),
                      gg=bf(M, F), mean=f32(M), rstd=f32(M), dw1=f32(F, H), db1=f32(F),
                      dw2=f32(H, F), db2=f32(H), dg=f32(H), dbt=f32(H)))
    dxs = [bf(M, H) for _ in range(2)]
    ws = torch.empty(ops.workspace_size(ops._abi.OP_LN_MLP_BWD_BF16, M, H, F), dtype=torch.uint8,
                     device="cuda")

    def step(s):
        x = x0
        for d in L:
            ops.ln_mlp_fwd_bf16(x, d["g"], d["b"], d["w1"], None, d["w2"], None, d["out"],
                                d["ln"], d["gg"], h=d["h"], mean=d["mean"], rstd=d["rstd"])
            x = d["out"]
        grad = dy
        for i, d in enumerate(reversed(L)):
            xin = x0 if i == layers - 1 else L[layers - 2 - i]["out"]
            dx = dxs[i % 2]
            ops.ln_mlp_bwd_bf16(grad, xin, d["g"], d["w1"], d["w2"], d["ln"], d["h"], d["gg"],
                                d["mean"], d["rstd"], dx, d["dg"], d["dbt"], d["dw1"], d["db1"],
                                d["dw2"], d["db2"], workspace=ws)
            grad = dx

    t = _time_steps(torch, step, steps, warmup, unroll=1)
    flops = layers * 6 * 2.0 * M * H * F
    return dict(t, flops=flops, gemm=(M, F, H, torch.float32), bf16=True)


def _time_steps(torch, step, steps, warmup, unroll=4):
    """Step time two ways on the same kernels and buffers: `eager_ms` with every
    step launched from the host, and `ms` with `unroll` consecutive steps
    replayed from one captured HIP graph (the launch-bound small workloads are
    host-bound when launched eagerly from Python)."""
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s in range(steps):
        step(s)
    t1.record()
    torch.cuda.synchronize()
    eager = t0.elapsed_time(t1) / steps
    replays = max(1, steps // unroll)
    return dict(ms=_graph_ms(torch, step, unroll, replays) / unroll, eager_ms=eager)


# ---- CPU baseline ----------------------------------------------------------------

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inputs, budget_s=12.0, single_s=4.0):
    """The C++ oracle's LayerNorm + cast + amax (float64, OpenMP over rows, -O2)
    on a sampled 8192-row block of the headline workload, repeated until
    budget_s has passed, on all the threads OpenMP is given; then the same on
    one thread for single_s."""
    import numpy as np
    import oracle.cxx as X
    from fp8_delayed_scaling_row_amd.inputs import spiky_normal_bf16, seed_for
    rows, hidden = 8192, 2048
    x = spiky_normal_bf16((rows, hidden), seed_for("cpu-baseline", "x"), drift=2.0)
    g, b = inputs.layernorm_params(hidden, "cpu-baseline")
    bits = lambda t: t.view(__import__("torch").int16).numpy().view(np.uint16)
    xb, gb, bb = bits(x), bits(g), bits(b)
    eps = float(np.float32(1e-5))
    byts = rows * hidden * 3 + rows * 8

    def run(budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            X.ln_cast_amax(xb, gb, bb, eps, np.float32(7.0), "e4m3")
            n += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
        return n, dt, n * byts / dt / 1e9

    threads = X.threads()
    n, dt, gbs = run(budget_s)
    X.set_threads(1)
    n1, dt1, gbs1 = run(single_s)
    X.set_threads(threads)
    return dict(value=round(gbs, 4), unit="GB/s", cores=threads, kind="oracle",
                cpu=_cpu_model(), nproc=os.cpu_count(), one_thread_gbs=round(gbs1, 4),
                sample=f"{n} x LayerNorm+cast+amax of an 8192 x 2048 bf16 block of the headline "
                       f"workload ({dt:.1f} s, C++ oracle, float64, OpenMP on {threads} "
                       f"threads; one thread: {n1} blocks in {dt1:.1f} s)")


def oracle_workloads(inputs, log):
    """The C++ oracle (float64, exact integer-accumulated GEMMs, OpenMP over rows)
    timed on one step of each GEMM-bound workload's shapes on this host:
    LayerNormLinear forward at 8 x 32 tokens, its backward at 2048 tokens,
    LayerNormMLP forward at 2048 tokens, and one layer (forward + backward) of the
    16384-token 2048/8192 scale-up, whose 12-layer step is that time x 12."""
    import numpy as np
    import torch
    import oracle
    import oracle.cxx as X
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    orc = oracle.Recipe(format=oracle.FORMAT_HYBRID, amax_history_len=16)

    def linear_parts(M, K, N, wl):
        g, b = inputs.layernorm_params(K, wl)
        w = inputs.linear_weight(N, K, wl, "w")
        x = inputs.normal_bf16((M, K), inputs.seed_for(wl, "x"))
        dy = inputs.normal_bf16((M, N), inputs.seed_for(wl, "dy"), std=1e-3)
        return bits(x), bits(g), bits(b), bits(w), bits(dy)

    def mlp_parts(M, H, F, wl):
        g, b = inputs.layernorm_params(H, wl)
        w1 = inputs.linear_weight(F, H, wl, "w1")
        w2 = inputs.linear_weight(H, F, wl, "w2")
        x = inputs.normal_bf16((M, H), inputs.seed_for(wl, "x"))
        dy = inputs.normal_bf16((M, H), inputs.seed_for(wl, "dy"), std=1e-3)
        return bits(x), bits(g), bits(b), bits(w1), bits(w2), bits(dy)

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return time.perf_counter() - t0, r

    out = []
    # LayerNormLinear fwd, 256 tokens, 768 -> 2304
    x, g, b, w, dy = linear_parts(256, 768, 2304, "oracle/ln_linear_fwd")
    mf = oracle.linear_fwd_meta(orc)
    dt, _ = timed(lambda: X.ln_linear_fwd(orc, mf, x, g, b, w))
    out.append(dict(workload="ln_linear_fwd", oracle_ms=dt * 1e3, flops=2.0 * 256 * 2304 * 768))
    # LayerNormLinear bwd, 2048 tokens
    x, g, b, w, dy = linear_parts(2048, 768, 2304, "oracle/ln_linear_bwd")
    mf, mb = oracle.linear_fwd_meta(orc), oracle.linear_bwd_meta(orc)
    _, (o, ctx) = timed(lambda: X.ln_linear_fwd(orc, mf, x, g, b, w))
    dt, _ = timed(lambda: X.ln_linear_bwd(orc, mf, mb, dy, ctx, x, g))
    out.append(dict(workload="ln_linear_bwd", oracle_ms=dt * 1e3,
                    flops=2 * 2.0 * 2048 * 2304 * 768))
    # LayerNormMLP fwd, 2048 tokens, 768 -> 3072 -> 768
    orc4 = oracle.Recipe(format=oracle.FORMAT_E4M3, amax_history_len=16)
    x, g, b, w1, w2, dy = mlp_parts(2048, 768, 3072, "oracle/ln_mlp_fwd")
    mf = oracle.mlp_fwd_meta(orc4)
    dt, _ = timed(lambda: X.ln_mlp_fwd(orc4, mf, x, g, b, w1, None, w2, None))
    out.append(dict(workload="ln_mlp_fwd", oracle_ms=dt * 1e3, flops=2 * 2.0 * 2048 * 3072 * 768))
    # one layer of the scale-up, forward + backward
    log("oracle: one 16384 x 2048 x 8192 layer ...")
    orc_h = oracle.Recipe(format=oracle.FORMAT_HYBRID, amax_history_len=1024)
    x, g, b, w1, w2, dy = mlp_parts(16384, 2048, 8192, "oracle/ln_mlp_x12")
    mf, mb = oracle.mlp_fwd_meta(orc_h), oracle.mlp_bwd_meta(orc_h)
    dtf, (o, ctx) = timed(lambda: X.ln_mlp_fwd(orc_h, mf, x, g, b, w1, None, w2, None))
    log(f"oracle: layer forward {dtf:.1f} s; backward ...")
    dtb, _ = timed(lambda: X.ln_mlp_bwd(orc_h, mf, mb, dy, ctx, x, g))
    log(f"oracle: layer backward {dtb:.1f} s")
    out.append(dict(workload="ln_mlp_x12_hybrid", oracle_ms_one_layer=(dtf + dtb) * 1e3,
                    oracle_ms=(dtf + dtb) * 12e3, extrapolated_from="one layer x 12",
                    flops=12 * 6 * 2.0 * 16384 * 8192 * 2048))
    for r in out:
        r["oracle_tflops"] = r["flops"] / (r["oracle_ms"] * 1e-3) / 1e12
    return dict(kind="oracle", implementation="C++ (oracle/cpp), OpenMP", threads=X.threads(),
                cpu=_cpu_model(), nproc=os.cpu_count(), workloads=out)


def main():
    args = parse()
    if args.oracle_workloads:
        from fp8_delayed_scaling_row_amd import inputs
        print(json.dumps(dict(oracle_workloads=oracle_workloads(
            inputs, lambda m: print(m, file=sys.stderr, flush=True)))), flush=True)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "design is described, not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    from fp8_delayed_scaling_row_amd import inputs, ops
    ok, why = ops.check_support(0)
    if not ok:
        print(f"device 0 unsupported: {why}", file=sys.stderr)
        sys.exit(1)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.profile_ln:
        profile_ln(torch, ops, inputs, args.profile_ln)
        return
    if args.profile_kernel:
        profile_kernel(torch, ops, inputs, args.profile_kernel[0], int(args.profile_kernel[1]))
        return
    if args.profile_gemm:
        M, N, K, reps = args.profile_gemm
        ms = gemm_kernel_ms(torch, ops, M, N, K, torch.float32, reps=reps, bf16=args.bf16)
        print(json.dumps(dict(profile_gemm=[M, N, K], bf16=args.bf16, reps=reps, kernel_ms=ms,
                              tflops=2.0 * M * N * K / (ms * 1e-3) / 1e12)), flush=True)
        return

    workloads = []
    head = None
    if args.only in (None, "ln_cast"):
        log("ln_cast_amax 65536x2048 ...")
        head = bench_ln_cast(torch, ops, inputs, args.steps, args.warmup)
        torch.cuda.empty_cache()
        head["copy_gbs"] = copy_ceiling_gbs(torch)
        head["probe_gbs"] = stream_probe_gbs(torch, ops)
    if not args.quick:
        runs = [
            ("ln_linear_fwd", "LayerNormLinear fwd 8x32 tokens, 768->2304, HYBRID, history 16",
             lambda: bench_linear_fwd(torch, ops, inputs, 200, 20)),
            ("ln_linear_bwd", "LayerNormLinear bwd 2048 tokens, 768->2304, HYBRID (E5M2 grads)",
             lambda: bench_linear_bwd(torch, ops, inputs, 100, 10)),
            ("ln_mlp_fwd", "LayerNormMLP fwd 2048 tokens, 768->3072->768, E4M3, history 16",
             lambda: bench_mlp_fwd(torch, ops, inputs, 100, 10)),
            ("ln_linear_fwd_fp8w", "LayerNormLinear fwd 8x32 tokens, 768->2304, HYBRID, FP8 weight storage",
             lambda: bench_linear_fwd(torch, ops, inputs, 200, 20, reuse=True)),
            ("ln_mlp_fwd_fp8w", "LayerNormMLP fwd 2048 tokens, 768->3072->768, E4M3, FP8 weight storage",
             lambda: bench_mlp_fwd(torch, ops, inputs, 100, 10, reuse=True)),
            ("ln_linear_fwd_bf16", "LayerNormLinear fwd 8x32 tokens, 768->2304, bf16 (no FP8)",
             lambda: bench_linear_fwd_bf16(torch, ops, inputs, 200, 20)),
            ("ln_linear_bwd_bf16", "LayerNormLinear bwd 2048 tokens, 768->2304, bf16 (no FP8)",
             lambda: bench_linear_bwd_bf16(torch, ops, inputs, 100, 10)),
            ("ln_mlp_fwd_bf16", "LayerNormMLP fwd 2048 tokens, 768->3072->768, bf16 (no FP8)",
             lambda: bench_mlp_fwd_bf16(torch, ops, inputs, 100, 10)),
            ("ln_mlp_fwd_16384", "LayerNormMLP fwd 16384 tokens, 2048->8192->2048, E4M3",
             lambda: bench_mlp_fwd(torch, ops, inputs, 20, 3, M=16384, H=2048, F=8192)),
            ("ln_mlp_fwd_16384_bf16", "LayerNormMLP fwd 16384 tokens, 2048->8192->2048, bf16 (no FP8)",
             lambda: bench_mlp_fwd_bf16(torch, ops, inputs, 20, 3, M=16384, H=2048, F=8192)),
            ("ln_mlp_x12_hybrid", "LayerNormMLP x12 fwd+bwd, 16384 tokens, 2048->8192->2048, HYBRID, history 1024",
             lambda: bench_mlp_stack(torch, ops, inputs, 20, 5, ops.FORMAT_HYBRID)),
            ("ln_mlp_x12_e4m3", "LayerNormMLP x12 fwd+bwd, 16384 tokens, 2048->8192->2048, E4M3, history 1024",
             lambda: bench_mlp_stack(torch, ops, inputs, 20, 5, ops.FORMAT_E4M3)),
            ("ln_mlp_x12_bf16", "LayerNormMLP x12 fwd+bwd, 16384 tokens, 2048->8192->2048, bf16 (no FP8)",
             lambda: bench_mlp_stack_bf16(torch, ops, inputs, 20, 5)),
        ]
        for name, desc, fn in runs:
            if args.only is not None and name not in args.only.split(","):
                continue
            log(f"{name} ...")
            r = fn()
            M, N, K, odt = r["gemm"]
            bf16 = r.get("bf16", False)
            tflops = r["flops"] / (r["ms"] * 1e-3) / 1e12
            peak = BF16_PEAK_TFLOPS if bf16 else FP8_PEAK_TFLOPS
            w = dict(
                workload=name, description=desc, precision="bf16" if bf16 else "fp8",
                ms_per_step=round(r["ms"], 5), eager_ms_per_step=round(r["eager_ms"], 5),
                value=round(tflops, 2), unit="TFLOP/s",
                frac_of_peak=round(tflops / peak, 4))
            if r.get("kinds"):
                # the step's own GEMM kernels, each timed alone; the roofline
                # names the one furthest below the peak
                kinds = mlp_gemm_kinds(torch, ops, *r["kinds"])
                worst = min(kinds, key=lambda k: k["frac"])
                w["gemm_kinds"] = kinds
                w["roofline"] = dict(bound="mfma", kernel=worst["kind"],
                                     achieved=worst["achieved"], peak=peak, unit="TFLOP/s",
                                     frac=worst["frac"], kernel_ms=worst["kernel_ms"])
            else:
                gk_ms = gemm_kernel_ms(torch, ops, M, N, K, odt, bf16=bf16)
                gflops = 2.0 * M * N * K
                w["roofline"] = dict(
                    bound="mfma", kernel=f"{'bf16' if bf16 else 'fp8'} gemm {M}x{N}x{K}",
                    achieved=round(gflops / (gk_ms * 1e-3) / 1e12, 2), peak=peak,
                    unit="TFLOP/s", frac=round(gflops / (gk_ms * 1e-3) / 1e12 / peak, 4),
                    kernel_ms=round(gk_ms, 5))
            twin = name.replace("_bf16", "")
            twin = "ln_mlp_x12_hybrid" if twin == "ln_mlp_x12" else twin
            fp8_twin = [x for x in workloads if x["workload"] == twin]
            if bf16 and fp8_twin:
                w["fp8_speedup"] = round(r["ms"] / fp8_twin[0]["ms_per_step"], 3)
            workloads.append(w)
            torch.cuda.empty_cache()

    line = dict(metric=METRIC, n_gpus=1, steps=args.steps, warmup=args.warmup,
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32",
                data="synthetic")
    if head:
        gbs = head["bytes"] / (head["ms"] * 1e-3) / 1e9
        kgbs = head["bytes"] / (head["kernel_ms"] * 1e-3) / 1e9
        traffic = counter_traffic("ln_cast_amax_65536x2048", LN_SOURCES)
        line.update(value=round(gbs, 2), unit="GB/s", ms_per_step=round(head["ms"], 5),
                    eager_ms_per_step=round(head["eager_ms"], 5),
                    config=dict(workload="ln_cast_amax_65536x2048", rows=head["rows"],
                                hidden=head["hidden"], out_dtype="fp8_e4m3",
                                amax_history_len=1024, input="N(0,1) x drift 1->4, 0.1% x100",
                                buffers=32),
                    roofline=dict(bound="hbm", kernel="ln_cast_amax",
                                  achieved=round(kgbs, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                                  frac=round(kgbs / HBM_PEAK_GBS, 4), traffic=traffic,
                                  kernel_ms=round(head["kernel_ms"], 5),
                                  kernel_timing="graph of 32 back-to-back launches, HIP events",
                                  eager_event_kernel_ms=round(head["event_kernel_ms"], 5),
                                  bytes_per_launch=head["bytes"],
                                  copy_ceiling=round(head["probe_gbs"], 1),
                                  copy_ceiling_kernel="fp8ln_stream_probe (2 B read + 1 B "
                                                      "written per element, non-temporal)",
                                  frac_of_copy_ceiling=round(kgbs / head["probe_gbs"], 4),
                                  torch_copy_gbs=round(head["copy_gbs"], 1)))
    line["workloads"] = workloads
    parts = {}
    lf = [x for x in workloads if x["workload"] == "ln_linear_fwd"]
    if lf:
        parts.update(ln_linear_fwd_tflops=lf[0]["value"],
                     ln_linear_fwd_frac_of_fp8_peak=lf[0]["frac_of_peak"],
                     ln_linear_fwd_config="8x32 tokens, 768->2304, HYBRID, history 16")
    if head:
        parts.update(ln_cast_amax_gbs=line["value"],
                     ln_cast_amax_frac_of_hbm=round(line["value"] / HBM_PEAK_GBS, 4),
                     ln_cast_amax_kernel_frac_of_hbm=line["roofline"]["frac"])
    if parts:
        line["metric_parts"] = parts
    if not args.no_cpu_baseline and head:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
