"""Benchmark of the direct-access split operators on one MI355X.

A step is the split-operator work of one Llama-8B-shaped decoder layer at
batch 16: the QKV (6144x4096), O (4096x4096), gate+up (28672x4096) and down
(4096x14336) split GEMMs with N = 16 activations, and split-KV grouped-query
decode attention over 16 requests x 32768 tokens (32 query heads on 8 KV heads,
head_dim 128).  A fraction x of every weight matrix's 64-row tile-rows and of
the requests' KV caches lives in pinned host memory and is read in place by the
kernels; the rest is in HBM.  The headline is x = 0.25.

Metric: effective bandwidth = bytes of weights and KV touched (both tiers, each
byte once) / step time, and its fraction of the two-tier roofline
max((1 - x) C / B_hbm, x C / B_host) summed over the ops, with B_hbm and B_host
measured by the library's streaming-read probes in the same run.

Inputs are seeded synthetic tensors drawn with the recipe of synth.py (std
0.02 weights, std 1 activations and KV), generated on the GPU.  Weights and KV
are held in both tiers, so every ratio of the sweep is a different descriptor
over the same buffers.

Prints ONE JSON line.  --gpus above 1 is refused: the library runs on one GPU (no collectives or sharding).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

M_TILE = 64
BATCH = 16
HQ, HKV, HD, CTX = 32, 8, 128, 32768
PCIE_GEN5_X16_GBPS = 64.0      # published per-direction host link peak
HBM_PEAK_GBPS = 8000.0         # published MI355X HBM3E peak


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def host_units(k, den, n):
    return -(-k * n // den)


class Workload:
    """Weights and KV in both tiers, plus outputs and workspace."""

    def __init__(self, torch, dak, seed=0, n_act=BATCH):
        self.torch, self.dak = torch, dak
        dev = torch.device("cuda")
        self.lin = []
        for i, (name, M, K) in enumerate(synth.LLAMA8B_LINEARS):
            A, X = synth.gemm_inputs(M, K, n_act, seed=seed + i, device="cuda")
            A_host = torch.empty((M, K), dtype=torch.bfloat16, pin_memory=True)
            A_host.copy_(A)
            y = torch.empty((n_act, M), dtype=torch.float32, device=dev)
            self.lin.append(dict(name=name, M=M, K=K, A_dev=A, A_host=A_host, x=X.contiguous(), y=y))
        q, K, V = synth.attn_inputs(BATCH, HQ, HKV, HD, CTX, seed=seed + 10, device="cuda")
        self.q, self.K_dev, self.V_dev = q, K, V
        self.K_host = torch.empty(K.shape, dtype=torch.bfloat16, pin_memory=True)
        self.V_host = torch.empty(V.shape, dtype=torch.bfloat16, pin_memory=True)
        self.K_host.copy_(K)
        self.V_host.copy_(V)
        self.out = torch.empty((BATCH, HQ, HD), dtype=torch.float32, device=dev)
        kv0 = self.kv_desc(0)
        self.ws = torch.empty((dak.decode_attn_workspace_bytes(kv0, HQ),), dtype=torch.uint8, device=dev)
        self.scale = 1.0 / math.sqrt(HD)
        torch.cuda.synchronize()

    def mat_desc(self, L, h):
        rows = h * M_TILE
        return self.dak.SplitMatrix(L["A_host"] if rows else None, L["A_dev"][rows:] if rows < L["M"] else None,
                                    L["M"], L["K"], M_TILE, h)

    def kv_desc(self, h):
        d = self.dak
        return d.SplitKV(self.K_host if h else None, self.V_host if h else None,
                         self.K_dev[h:] if h < BATCH else None, self.V_dev[h:] if h < BATCH else None,
                         BATCH, h, HKV, HD, CTX)

    def plan(self, k, den=20):
        """Descriptors for x = k/den (host units rounded up per op)."""
        mats = [(L, self.mat_desc(L, host_units(k, den, L["M"] // M_TILE))) for L in self.lin]
        kv = self.kv_desc(host_units(k, den, BATCH))
        return mats, kv

    def op_bytes(self):
        """(name, total bytes C, units n) per op in step order."""
        ops = []
        for L in self.lin:
            ops.append((L["name"], L["M"] * L["K"] * 2, L["M"] // M_TILE))
        kvb = 2 * BATCH * HKV * CTX * HD * 2
        # attention runs after QKV
        return [ops[0], ("attn", kvb, BATCH)] + ops[1:]


OP_ORDER = ("qkv", "attn", "o", "gate_up", "down")


def run_step(wl, plan, cfg=None, events=None, only=None):
    """One pass of the hot path: QKV, attention, O, gate+up, down (or one of them)."""
    dak = wl.dak
    mats, kv = plan
    seq = [("gemm", mats[0]), ("attn", kv), ("gemm", mats[1]), ("gemm", mats[2]), ("gemm", mats[3])]
    for i, (kind, obj) in enumerate(seq):
        if only is not None and OP_ORDER[i] != only:
            continue
        if events is not None:
            events[i][0].record()
        if kind == "gemm":
            L, S = obj
            dak.splitk_gemm(S, L["x"], y=L["y"], cfg=cfg)
        else:
            dak.splitk_decode_attn(wl.q, obj, wl.scale, out=wl.out, ws=wl.ws, cfg=cfg)
        if events is not None:
            events[i][1].record()


def kernel_traffic(kernel_src: str, key: str):
    """Per-launch DRAM/link traffic of a kernel from the committed rocprofv3
    counter summary (profiles/traffic.json), or None when the kernel's source
    has changed since the counters were taken."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f).get(key)
        with open(os.path.join(ROOT, "tiered_memory_offloading_amd", "csrc", kernel_src), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != sha:
        return None
    return rec


def calibrate_copy(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, so that a counter run can
    scale FETCH_SIZE and WRITE_SIZE to bytes."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def measure_bandwidths(torch, dak):
    """B_hbm (4 GiB device buffer) and B_host (1 GiB pinned) from the probes, GB/s."""
    g = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    best_g = 0.0
    for wg, w in ((256, 8), (512, 4), (1024, 1), (2048, 1), (1024, 2)):
        ms = dak.probe_read(g, wg, w, reps=5)
        best_g = max(best_g, g.numel() / ms / 1e6)
    del g
    h = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    best_h = 0.0
    for wg, w in ((16, 4), (32, 4), (8, 8), (64, 2)):
        ms = dak.probe_read(h, wg, w, reps=3)
        best_h = max(best_h, h.numel() / ms / 1e6)
    del h
    torch.cuda.empty_cache()
    return best_g, best_h


def two_tier_roofline_ms(wl, k, den, b_hbm, b_host):
    t = 0.0
    for name, C, n in wl.op_bytes():
        h = host_units(k, den, n)
        x = h / n
        t += max((1 - x) * C / (b_hbm * 1e9), x * C / (b_host * 1e9))
    return t * 1e3


def host_bytes(wl, k, den):
    tot = 0
    for name, C, n in wl.op_bytes():
        tot += host_units(k, den, n) * (C // n)
    return tot


def capture_step(torch, wl, plan):
    """The step's launches recorded in one HIP graph (a decode step is replayed
    this way in serving), or None if capture fails.  The library's entry points
    allocate nothing and only launch kernels on the given stream, so they
    record as plain kernel nodes."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_step(wl, plan)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, capture_error_mode="relaxed"):
            run_step(wl, plan)
        torch.cuda.synchronize()
        return g
    except Exception as e:  # noqa: BLE001 - a failed capture only drops the graph timing
        log(f"graph capture failed ({e}); reporting no graph timing")
        torch.cuda.synchronize()
        return None


def time_steps(torch, wl, plan, steps, warmup, per_op=True, only=None, graph=True):
    """(ms per step, per-op ms, ms per graph-replayed step or None).  The
    steps are timed as plain stream launches with nothing between them (the
    fastest mode measured on MI355X); the same step captured in a HIP graph is
    timed as well when capture works.  Per-op durations come from a separate
    pass with events around each op, so the events stay out of the timed
    steps."""
    g = capture_step(torch, wl, plan) if graph and only is None else None

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    ms = timed(lambda: run_step(wl, plan, only=only))
    graph_ms = timed(g.replay) if g is not None else None
    # per-step spread, from a separate pass with an event pair around each step
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in sev:
        e0.record()
        run_step(wl, plan, only=only)
        e1.record()
    torch.cuda.synchronize()
    st = sorted(e0.elapsed_time(e1) for e0, e1 in sev)
    pct = lambda p: st[min(len(st) - 1, int(round(p * (len(st) - 1))))]
    time_steps.spread = {"p10": round(pct(0.1), 4), "p50": round(pct(0.5), 4), "p90": round(pct(0.9), 4),
                         "steps": len(st)}
    op_ms = None
    if per_op:
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
               for _ in range(steps)]
        for st in range(steps):
            run_step(wl, plan, events=evs[st], only=only)
        torch.cuda.synchronize()
        idx = range(5) if only is None else [OP_ORDER.index(only)]
        op_ms = [0.0] * 5
        for i in idx:
            op_ms[i] = statistics.mean(evs[st][i][0].elapsed_time(evs[st][i][1]) for st in range(steps))
    del g
    return ms, op_ms, graph_ms


def cpu_baseline(wl, reps=5):
    """The oracle, as it stands, on the whole step at x = 0 (the result does
    not depend on x): the four split-GEMM oracles at N = 16 and the attention
    oracle over all 16 requests x 32 query heads, on the host CPU, from the
    same tensors the GPU step reads (copied to the host first, untimed)."""
    import numpy as np  # noqa: F401
    from oracle import attention as oa
    from oracle import gemm as og

    t0 = time.perf_counter()
    lin = [(L["A_dev"].cpu(), L["x"].cpu()) for L in wl.lin]
    q, K, V = wl.q.cpu(), wl.K_dev.cpu(), wl.V_dev.cpu()
    t_copy = time.perf_counter() - t0

    def step_runs(n):
        runs = []
        for _ in range(n):
            t1 = time.perf_counter()
            for A, X in lin:
                og.gemm(og.to_f64(A), og.to_f64(X))
            t_lin = time.perf_counter() - t1
            t2 = time.perf_counter()
            for b in range(BATCH):
                oa.decode_attention(og.to_f64(q[b:b + 1]), og.to_f64(K[b:b + 1]), og.to_f64(V[b:b + 1]), wl.scale)
            t_att = time.perf_counter() - t2
            runs.append((t_lin + t_att, t_lin, t_att))
        runs.sort()
        return runs[len(runs) // 2]

    t_step, t_lin, t_att = step_runs(reps)
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = step_runs(1)
    except ImportError:
        pass
    step_bytes = sum(C for _, C, _ in wl.op_bytes())
    res = {
        "value": round(step_bytes / t_step / 1e9, 4),
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model_name(),
        "kind": "oracle",
        "sample": (f"the whole step, median of {reps} runs: fp64 numpy oracle of the four split GEMMs at N=16 "
                   f"({t_lin:.2f} s) and of the split-KV attention over 16 requests x 32 query heads x 32768 tokens "
                   f"({t_att:.2f} s), on the same inputs as the GPU step (copied to the host first, {t_copy:.1f} s, "
                   f"untimed); BLAS on every core the process may use"),
        "seconds_per_step": round(t_step, 3),
    }
    if one is not None:
        res["single_thread"] = {"value": round(step_bytes / one[0] / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "seconds_per_step": round(one[0], 3), "gemm_s": round(one[1], 3),
                                "attention_s": round(one[2], 3), "what": "the same step once, BLAS held to 1 thread"}
    return res


def _cold_timer(torch, dak, reps):
    """Mean ms per launch over `reps` rotations through every descriptor
    (each a different HBM copy), after one untimed rotation."""
    def timed(descs, x, y):
        for S in descs:
            dak.splitk_gemm(S, x, y=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for S in descs:
                dak.splitk_gemm(S, x, y=y)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(descs))
    return timed


def headline_extras(torch, dak, b_hbm, b_host, warm_seconds=1.5, reps=3):
    """Compact numbers from the other configurations, for the headline line:
    the 1024x1024 GEMV (N = 1) cold at x = 0 and 1/4 against its two-tier
    roofline; the x = 0 fraction of B_hbm of each Llama-8B decode linear at
    N in {1, 16, 64}, cold (at least 1 GiB of HBM copies in rotation); and the
    28672x8192x2048 prefill GEMM's MFMA rate at x = 0 and at the planner's
    turning point, against the 2.5 PFLOP/s spec and the library's MFMA
    probe."""
    timed = _cold_timer(torch, dak, reps)
    out = {}
    rows = {}
    ops = [("gemv_1024x1024", 1024, 1024)] + list(synth.LLAMA8B_LINEARS)
    for oi, (name, M, K) in enumerate(ops):
        n = M // M_TILE
        C = M * K * 2
        copies = max(2, -(-(1 << 30) // C))
        A = synth.gemm_inputs(M, K, 1, seed=oi, device="cuda")[0]
        As = [A] + [A.clone() for _ in range(copies - 1)]
        if name == "gemv_1024x1024":
            h = host_units(1, 4, n)
            A_host = torch.empty((h * M_TILE, K), dtype=torch.bfloat16, pin_memory=True)
            A_host.copy_(A[:h * M_TILE])
            X = synth.gemm_inputs(M, K, 1, seed=oi, device="cuda")[1].contiguous()
            y = torch.empty((1, M), dtype=torch.float32, device="cuda")
            t0 = timed([dak.SplitMatrix(None, a, M, K, M_TILE, 0) for a in As], X, y)
            t1 = timed([dak.SplitMatrix(A_host, a[h * M_TILE:], M, K, M_TILE, h) for a in As], X, y)
            roof = max((n - h) * (C // n) / (b_hbm * 1e9), h * (C // n) / (b_host * 1e9)) * 1e3
            out["gemv_1024x1024_cold"] = {"x0_us": round(t0 * 1e3, 2), "x025_us": round(t1 * 1e3, 2),
                                          "x025_frac_two_tier": round(roof / t1, 4),
                                          "x0_frac_b_hbm": round(C / (b_hbm * 1e9) * 1e3 / t0, 4)}
            del A_host
        else:
            for N in (1, 16, 64):
                X = synth.gemm_inputs(M, K, N, seed=oi, device="cuda")[1].contiguous()
                y = torch.empty((N, M), dtype=torch.float32, device="cuda")
                t = timed([dak.SplitMatrix(None, a, M, K, M_TILE, 0) for a in As], X, y)
                rows[f"{name}_N{N}"] = round(C / (b_hbm * 1e9) * 1e3 / t, 4)
                del X, y
        del A, As
        torch.cuda.empty_cache()
    out["linears_x0_frac_b_hbm_cold"] = rows

    M, K, N = 28672, 8192, 2048
    n = M // M_TILE
    flops = 2 * M * K * N
    A, X = synth.gemm_inputs(M, K, N, seed=0, device="cuda")
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    S0 = dak.SplitMatrix(None, A, M, K, M_TILE, 0)
    t_end = time.perf_counter() + warm_seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            dak.splitk_gemm(S0, X, y=y)
        torch.cuda.synchronize()

    def med(S, k=7):
        ts = []
        for _ in range(k):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dak.splitk_gemm(S, X, y=y)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)

    t0 = med(S0)
    _, b, _ = dak.op_turning_points(dak.Op(n, (M * K * 2) // n, t0 * 1e-3), b_hbm * 1e9, b_host * 1e9)
    b = min(b, host_units(3, 4, n))
    A_host = torch.empty((b * M_TILE, K), dtype=torch.bfloat16, pin_memory=True)
    A_host.copy_(A[:b * M_TILE])
    t0p = med(S0)
    tb = med(dak.SplitMatrix(A_host if b else None, A[b * M_TILE:], M, K, M_TILE, b))
    _, tf_probe = dak.probe_mfma(workgroups=1024, iters=8192, reps=5)
    tf0, tfb = flops / t0 / 1e9, flops / tb / 1e9
    out["prefill_28672x8192x2048"] = {
        "x0_TFLOPs": round(tf0, 1), "x0_frac_spec": round(tf0 / MFMA_BF16_DENSE_TFLOPS, 4),
        "x0_frac_probe": round(tf0 / tf_probe, 4), "probe_TFLOPs": round(tf_probe, 1),
        "planner_x": round(b / n, 4), "planner_TFLOPs": round(tfb, 1),
        "planner_frac_spec": round(tfb / MFMA_BF16_DENSE_TFLOPS, 4),
        "planner_slowdown_vs_paired_x0": round(tb / t0p, 4)}
    del A, X, y, A_host
    torch.cuda.empty_cache()
    return out


def cpu_model_name():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_llama70b(torch, model, seed=0):
    """The oracle on a bounded sample of the 70B-shaped step: 256 seeded rows
    of each GEMM kind (all batch columns; layers drawn at random) and two
    seeded (request, KV head) pairs of every layer's attention (all their
    query heads).  Each sampled op runs alone on the GPU and its output is
    compared with the fp64 oracle on inputs read back from the placed tiers
    (both untimed); the oracle's own time gives the rate.  Returns the
    cpu_baseline object with the worst normwise error of each kind."""
    import numpy as np  # noqa: F401
    from oracle import attention as oa
    from oracle import fp8 as of
    from oracle import gemm as og

    g = torch.Generator().manual_seed(seed)
    s = model.shape
    G = s.n_q_heads // s.n_kv_heads
    by_op = {}
    layers = s.layers
    for kind in ("qkv", "o", "gate_up", "down"):
        idx = [i for i, o in enumerate(model.slots) if o.kind == kind]
        M = model.slots[idx[0]].units * model.m
        for _ in range(256):
            li = int(torch.randint(0, layers, (1,), generator=g))
            by_op.setdefault(idx[li], []).append(int(torch.randint(0, M, (1,), generator=g)))
    for i, o in enumerate(model.slots):
        if o.kind == "attn":
            by_op[i] = [(int(torch.randint(0, model.batch, (1,), generator=g)),
                         int(torch.randint(0, s.n_kv_heads, (1,), generator=g))) for _ in range(2)]
    worst, t_oracle, nbytes = {}, 0.0, 0
    q = None
    for i in sorted(by_op):
        o = model.slots[i]
        model.run_op(i)
        torch.cuda.synchronize()
        if o.kind == "attn":
            out = model.out.cpu()
            if q is None:
                q = og.to_f64(model.q)
            for b, kvh in by_op[i]:
                Kb, Vb = model.kv_block(i, b, kvh)
                t0 = time.perf_counter()
                Kf, Vf = og.to_f64(Kb), og.to_f64(Vb)
                refs = [oa.attend_one(q[b, j], Kf, Vf, model.scale) for j in range(kvh * G, (kvh + 1) * G)]
                t_oracle += time.perf_counter() - t0
                nbytes += 2 * Kb.numel() * 2
                for j, ref in zip(range(kvh * G, (kvh + 1) * G), refs):
                    worst["attn"] = max(worst.get("attn", 0.0), og.normwise_error(out[b, j].numpy(), ref))
        else:
            rows = sorted(set(by_op[i]))
            y = model.y[o.kind].cpu()[:, rows].numpy()
            W, sc = model.weight_rows(i, rows)
            x = model.x[o.kind].cpu()
            t0 = time.perf_counter()
            ref = of.gemm_fp8(W, sc, x) if model.weights == "fp8" else og.gemm_rows(og.to_f64(W), og.to_f64(x))
            t_oracle += time.perf_counter() - t0
            nbytes += W.numel() * W.element_size()
            worst[o.kind] = max(worst.get(o.kind, 0.0), og.normwise_error(y, ref))
    n_rows = sum(len(set(v)) for i, v in by_op.items() if model.slots[i].kind != "attn")
    n_pairs = sum(len(v) for i, v in by_op.items() if model.slots[i].kind == "attn")
    return {
        "value": round(nbytes / t_oracle / 1e9, 4), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{n_rows} seeded weight rows (256 draws per GEMM kind over the {layers} layers, all "
                   f"{model.batch} columns) and {n_pairs} seeded (request, KV head) pairs (2 per layer, "
                   f"{G} query heads each, {model.ctx} tokens) of the planned step; fp64 numpy oracle on "
                   f"inputs read back from the placed tiers; {nbytes / 1e9:.3f} GB of weights and KV in "
                   f"{t_oracle:.2f} s"),
        "seconds": round(t_oracle, 3),
        "worst_normwise_error": {k: float(f"{v:.3e}") for k, v in worst.items()},
        "parity_ok": max(worst.values()) <= 1e-2,
    }


def run_llama70b(torch, dak, args, b_hbm, b_host):
    """70B-shaped decode step (80 layers, hidden 8192, GQA 64/8, hd 128, FFN
    28672, `--b70-batch` requests (16) x 32768 tokens): the planner spreads the
    footprint (~309 GB at batch 16 with bf16 weights) over HBM and pinned host
    memory; the step is timed against its model.  `--b70-weights fp8` stores
    the weights as e4m3 codes with per-row scales; `--b70-kv-unit head` lets
    the planner place single (request, KV head) KV blocks."""
    from tiered_memory_offloading_amd.model import LLAMA70B, DecodeModel

    free, total = torch.cuda.mem_get_info()
    reserve = int(args.hbm_reserve_gib * (1 << 30))
    H = free - reserve
    log(f"HBM free {free / 2**30:.2f} GiB of {total / 2**30:.2f} GiB; planning with H = {H / 2**30:.2f} GiB")
    B = args.b70_batch
    kv_unit = dak.KV_UNIT_HEAD if args.b70_kv_unit == "head" else dak.KV_UNIT_REQUEST
    model = DecodeModel(LLAMA70B, B, 32768, b_hbm * 1e9, b_host * 1e9, H, log=log, weights=args.b70_weights,
                        kv_unit=kv_unit)
    for _ in range(args.warmup):
        model.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        model.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    n = len(model.slots)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    model.step(events=evs)
    torch.cuda.synchronize()
    per_kind = {}
    for i, o in enumerate(model.slots):
        d = per_kind.setdefault(o.kind, {"measured_ms": 0.0, "modeled_ms": 0.0, "host_units": 0, "units": 0,
                                         "host_bytes": 0, "bytes": 0})
        d["measured_ms"] += evs[i][0].elapsed_time(evs[i][1])
        d["modeled_ms"] += model.op_model_s(i) * 1e3
        d["host_units"] += o.host_units
        d["units"] += o.units
        d["host_bytes"] += o.host_units * o.unit_bytes
        d["bytes"] += o.bytes
    for d in per_kind.values():
        d["measured_ms"] = round(d["measured_ms"], 3)
        d["modeled_ms"] = round(d["modeled_ms"], 3)
    ops_with_host = sum(1 for o in model.slots if o.host_units)
    res = {
        "metric": "effective GB/s (HBM+host) of a 70B-shaped decode step at the planned ratios",
        "value": round(model.footprint / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "dtype": ("e4m3 weights, " if args.b70_weights == "fp8" else "") + "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "Llama-70B-shaped decode step: 80 layers x {QKV 10240x8192, split-KV attention "
                               f"64q/8kv hd128, O 8192x8192, gate+up 57344x8192, down 8192x28672}}, batch {B}, "
                               "32768 ctx/request", "weights": args.b70_weights, "kv_unit": args.b70_kv_unit,
                   "footprint_bytes": model.footprint, "hbm_budget_bytes": H, "hbm_reserve_bytes": reserve},
        "x_global": round(model.x_global, 6), "host_bytes": model.host_bytes, "ops": n,
        "ops_with_host_units": ops_with_host, "modeled_ms": round(model.modeled_s * 1e3, 3),
        "frac_of_model": round(model.modeled_s * 1e3 / ms, 4),
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "per_kind": per_kind,
    }
    if not args.no_cpu_baseline:
        log("checking sampled rows and KV pairs of the planned step against the CPU oracle")
        res["cpu_baseline"] = cpu_baseline_llama70b(torch, model)
        log(f"worst normwise error per kind: {res['cpu_baseline']['worst_normwise_error']}")
    print(json.dumps(res), flush=True)
    return 0


MFMA_BF16_DENSE_TFLOPS = 2500.0   # published MI355X dense bf16 matrix peak


def run_prefill(torch, dak, args, b_hbm, b_host):
    """Compute-bound split GEMM: A 28672x8192 ~N(0, 0.02), B 8192x2048 ~N(0, 1)
    (x holds B^T, N = 2048), 64-row tile-rows.  The op's compute time at x = 0
    gives the planner's turning point b (DAK paper §4.2.1: host reads hide
    behind compute while x C / B_host <= T_comp); the kernel is timed at x = 0,
    at b / n and on a sweep of x up to 0.75, and its MFMA utilisation reported.
    `--prefill-weights fp8`: the same shape with FP8 weights (e4m3 codes, one
    fp32 scale per row, widened to bf16 for the same MFMAs): half the bytes per
    tile-row, so about twice the host share before the turning point."""
    M, K, N = 28672, 8192, 2048
    n = M // M_TILE
    fp8 = args.prefill_weights == "fp8"
    C = M * K * (1 if fp8 else 2)
    flops = 2 * M * K * N
    if fp8:
        A, scale, X = synth.fp8_gemm_inputs(M, K, N, seed=0, device="cuda")
    else:
        A, X = synth.gemm_inputs(M, K, N, seed=0, device="cuda")
    hmax = host_units(3, 4, n)
    A_host = torch.empty((hmax * M_TILE, K), dtype=A.dtype, pin_memory=True)
    A_host.copy_(A[:hmax * M_TILE])
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    gemm = dak.splitk_gemm_fp8 if fp8 else dak.splitk_gemm

    def desc(h):
        hp, gp = A_host[:h * M_TILE] if h else None, A[h * M_TILE:] if h < n else None
        if fp8:
            return dak.SplitMatrixFP8(hp, gp, scale, M, K, M_TILE, h)
        return dak.SplitMatrix(hp, gp, M, K, M_TILE, h)

    def time_h(h, reps):
        S = desc(h)
        for _ in range(args.warmup):
            gemm(S, X, y=y)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            e0.record()
            gemm(S, X, y=y)
            e1.record()
        torch.cuda.synchronize()
        return statistics.mean(e0.elapsed_time(e1) for e0, e1 in ev)

    reps = max(args.steps, 5)
    # The chip's clock climbs over the first second or so of sustained MFMA
    # load; warm it up, then time every host share right after an x = 0
    # measurement of its own, so that each slowdown compares like with like.
    S0 = desc(0)
    t_end = time.perf_counter() + args.warm_seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            gemm(S0, X, y=y)
        torch.cuda.synchronize()
    t0s = [time_h(0, reps)]
    a, b, mb = dak.op_turning_points(dak.Op(n, C // n, t0s[0] * 1e-3), b_hbm * 1e9, b_host * 1e9)
    log(f"x=0: {t0s[0]:.3f} ms, {flops / t0s[0] / 1e9:.1f} TFLOP/s; turning points a={a} b={b} of n={n}")
    xs = sorted({(b, n)} | (set() if args.no_sweep else {(kk, 20) for kk in (1, 2, 3, 4, 6, 10, 15)}))
    sweep = []
    for num, den in xs:
        h = host_units(num, den, n) if den != n else num
        t0p = time_h(0, reps)
        t0s.append(t0p)
        t = time_h(h, reps)
        model = max(t0p, h * (C // n) / (b_host * 1e9) * 1e3)
        sweep.append({"x": round(h / n, 5), "h": h, "ms": round(t, 4), "TFLOPs": round(flops / t / 1e9, 1),
                      "x0_ms_paired": round(t0p, 4), "slowdown_vs_x0": round(t / t0p, 4),
                      "model_ms": round(model, 4), "frac_of_model": round(model / t, 4)})
        log(f"x={h / n:.4f} (h={h}): {t:.3f} ms (x=0 paired {t0p:.3f}), slowdown {t / t0p:.3f}, "
            f"model {model:.3f} ms")
    t0 = statistics.median(t0s)
    sweep.insert(0, {"x": 0.0, "h": 0, "ms": round(t0, 4), "TFLOPs": round(flops / t0 / 1e9, 1),
                     "x0_ms_paired": round(t0, 4), "slowdown_vs_x0": 1.0, "model_ms": round(t0, 4),
                     "frac_of_model": 1.0})
    # a library GEMM of the same shape (bf16 weights), all in HBM, as context
    # for the MFMA rate
    if fp8:
        del A_host
        A = synth.gemm_inputs(M, K, 1, seed=0, device="cuda")[0]   # timing only
    Bt = X.t()
    for _ in range(args.warmup):
        torch.matmul(A, Bt)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        torch.matmul(A, Bt)
        e1.record()
    torch.cuda.synchronize()
    t_lib = statistics.mean(e0.elapsed_time(e1) for e0, e1 in ev)
    at_b = next(r for r in sweep if r["h"] == b)
    tf0 = flops / t0 / 1e9
    _, tf_probe = dak.probe_mfma(workgroups=1024, iters=8192, reps=5)
    res = {
        "metric": "TFLOP/s of the compute-bound split GEMM and its slowdown at the planner's host share",
        "value": round(flops / at_b["ms"] / 1e9, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": reps,
        "warmup": args.warmup, "ms_per_step": at_b["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3 weights widened to bf16, " if fp8 else "") + "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "prefill split GEMM A 28672x8192 . B 8192x2048, 64-row tile-rows"
                               + (", FP8 weights" if fp8 else ""),
                   "x": at_b["x"], "h": b, "n": n},
        "turning_points": {"a": a, "b": b, "memory_bound": mb, "t_comp_ms": round(t0s[0], 4)},
        "slowdown_at_b": at_b["slowdown_vs_x0"], "x0_ms_all": [round(t, 4) for t in t0s],
        "roofline": {"bound": "mfma", "kernel": "gemm_tiled_split", "achieved": round(tf0, 1),
                     "peak": MFMA_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf0 / MFMA_BF16_DENSE_TFLOPS, 4), "traffic": None,
                     "ms_per_launch": round(t0, 4), "flops_per_launch": flops,
                     "measured_peak_TFLOPs": round(tf_probe, 1), "frac_of_measured_peak": round(tf0 / tf_probe, 4),
                     "note": "measured peak: the library's MFMA-only probe (8 independent bf16 MFMA chains per "
                             "wave, 1024 work-groups) at the clock the chip holds under that load"},
        "library_gemm_all_hbm": {"ms": round(t_lib, 4), "TFLOPs": round(flops / t_lib / 1e9, 1),
                                 "what": "torch.matmul (hipBLASLt) of the same bf16 shape, all operands in HBM"},
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "sweep": sweep,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_linears(torch, dak, args, b_hbm, b_host):
    """The Llama-8B decode linears one by one (QKV 6144x4096, O 4096x4096, gate+up
    28672x4096, down 4096x14336; A ~N(0, 0.02), x [N, K] ~N(0, 1)) at N in
    {1, 16, 64} and x = k/20 for k = 0..10, and the 1024x1024 GEMV (N = 1, x = 0
    and 1/4) hot and cold.  Cold: every launch reads a different copy of the
    HBM part (at least 1 GiB of copies in rotation, beyond the memory-side
    cache); host bytes always cross the link.  Each point is the mean over
    `--sweep-steps` rotations of all copies after one untimed rotation; outputs
    at every x are checked bit-identical to x = 0."""
    reps = max(1, args.sweep_steps)

    def timed(descs, x, y):
        for S in descs:
            dak.splitk_gemm(S, x, y=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for S in descs:
                dak.splitk_gemm(S, x, y=y)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(descs))

    points = []
    ops = [("gemv_1024x1024", 1024, 1024)] + list(synth.LLAMA8B_LINEARS)
    for oi, (name, M, K) in enumerate(ops):
        n = M // M_TILE
        C = M * K * 2
        copies = max(2, -(-(1 << 30) // C))
        A = synth.gemm_inputs(M, K, 1, seed=oi, device="cuda")[0]
        As = [A] + [A.clone() for _ in range(copies - 1)]
        hmax = host_units(1, 2, n)
        A_host = torch.empty((hmax * M_TILE, K), dtype=torch.bfloat16, pin_memory=True)
        A_host.copy_(A[:hmax * M_TILE])
        ns = (1,) if name == "gemv_1024x1024" else (1, 16, 64)
        ks = (0, 5) if name == "gemv_1024x1024" else tuple(range(11))
        for N in ns:
            X = synth.gemm_inputs(M, K, N, seed=oi, device="cuda")[1].contiguous()
            y = torch.empty((N, M), dtype=torch.float32, device="cuda")
            ref = None
            for k in ks:
                h = host_units(k, 20, n)
                descs = [dak.SplitMatrix(A_host[:h * M_TILE] if h else None, a[h * M_TILE:] if h < n else None,
                                         M, K, M_TILE, h) for a in As]
                t = timed(descs, X, y)
                if ref is None:
                    ref = y.clone()
                same = bool(torch.equal(y, ref))
                t_roof = max((n - h) * (C // n) / (b_hbm * 1e9), h * (C // n) / (b_host * 1e9)) * 1e3
                pt = {"op": name, "M": M, "K": K, "N": N, "x": round(h / n, 4), "h": h, "ms": round(t, 5),
                      "GBps": round(C / (t * 1e-3) / 1e9, 2), "frac_two_tier": round(t_roof / t, 4),
                      "frac_b_hbm_at_x0": round(t_roof / t, 4) if h == 0 else None, "bit_identical_to_x0": same,
                      "cold_copies": copies}
                if name == "gemv_1024x1024":
                    pt["hot_ms"] = round(timed(descs[:1], X, y), 5)
                points.append(pt)
                log(f"{name} N={N} x={h / n:.3f}: {t * 1e3:.1f} us, {pt['GBps']:.0f} GB/s, "
                    f"{pt['frac_two_tier']:.3f} of roofline{'' if same else ' BITS DIFFER'}")
            del X, y
        del A, As, A_host
        torch.cuda.empty_cache()
    llama_points = [p for p in points if p["op"] != "gemv_1024x1024"]
    worst_x_pos = min(p["frac_two_tier"] for p in llama_points if p["x"] > 0)
    x0 = [p for p in llama_points if p["h"] == 0]
    res = {
        "metric": "effective GB/s (HBM+host) and % of two-tier roofline vs offload ratio x, per decode linear",
        "value": round(statistics.mean(p["frac_two_tier"] for p in llama_points if p["x"] > 0), 4),
        "unit": "mean fraction of the two-tier roofline over N in {1,16,64}, 4 ops, x = 0.05..0.5",
        "n_gpus": 1, "steps": reps, "warmup": 1, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate", "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "Llama-8B decode linears QKV 6144x4096, O 4096x4096, gate+up 28672x4096, "
                               "down 4096x14336 at N in {1,16,64}, x = k/20 (k = 0..10), 64-row tile-rows, cold; "
                               "plus the 1024x1024 GEMV (N = 1, x = 0 and 1/4) hot and cold"},
        "worst_frac_two_tier_x_pos": worst_x_pos,
        "frac_b_hbm_at_x0": {f"{p['op']}_N{p['N']}": p["frac_two_tier"] for p in x0},
        "all_bit_identical_across_x": all(p["bit_identical_to_x0"] for p in points),
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "points": points,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_linears_x0(torch, dak, args, b_hbm, b_host):
    """The Llama-8B decode linears at x = 0 and N in {16, 64}: each (op, N)
    launched once on each of three copies of its weights (cold in L2), in a
    fixed order that the JSON line lists, for counter runs that attribute
    each dispatch (L2 requests per weight line)."""
    order, rows = [], {}
    for oi, (name, M, K) in enumerate(synth.LLAMA8B_LINEARS):
        A = synth.gemm_inputs(M, K, 1, seed=oi, device="cuda")[0]
        copies = [A.clone() for _ in range(3)]
        for N in (16, 64):
            X = synth.gemm_inputs(M, K, N, seed=oi, device="cuda")[1].contiguous()
            y = torch.empty((N, M), dtype=torch.float32, device="cuda")
            ts = []
            for c in copies:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                dak.splitk_gemm(dak.SplitMatrix(None, c, M, K, M_TILE, 0), X, y=y)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
                order.append(f"{name}_N{N}")
            rows[f"{name}_N{N}"] = {"us": [round(t * 1e3, 1) for t in ts],
                                    "GBps_median": round(M * K * 2 / (statistics.median(ts) * 1e6), 1)}
            del X, y
        del A, copies
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "x = 0 GB/s of the decode linears, one launch per cold weight copy", "unit": "GB/s",
                      "n_gpus": 1, "higher_is_better": True, "data": "synthetic (seeded)",
                      "config": {"workload": "Llama-8B decode linears at x = 0, N in {16, 64}, three cold copies"},
                      "b_hbm_GBps": round(b_hbm, 1), "dispatch_order": order, "ops": rows}), flush=True)
    return 0


def run_fp8_linears(torch, dak, args, b_hbm, b_host):
    """The Llama-8B decode linears (QKV 6144x4096, O 4096x4096, gate+up
    28672x4096, down 4096x14336) with FP8 weights (e4m3 codes, one fp32 scale
    per row, from N(0, 0.02) weights) at N in {1, 16, 64} and x = k/20 for
    k in {0, 1, 2, 5, 10}, cold (at least 1 GiB of copies of the HBM part in
    rotation), beside the bf16 kernel at x = 0 and 1/4 on the same shapes.
    Each point is the mean over `--sweep-steps` rotations after one untimed
    rotation; FP8 outputs at every x are checked bit-identical to x = 0."""
    reps = max(1, args.sweep_steps)

    def timed(fn, descs, x, y):
        for S in descs:
            fn(S, x, y=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for S in descs:
                fn(S, x, y=y)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(descs))

    points = []
    for oi, (name, M, K) in enumerate(synth.LLAMA8B_LINEARS):
        n = M // M_TILE
        C8 = M * K
        copies = max(2, -(-(1 << 30) // C8))
        codes, scale, _ = synth.fp8_gemm_inputs(M, K, 1, seed=oi, device="cuda")
        Cs = [codes] + [codes.clone() for _ in range(copies - 1)]
        scale = scale.contiguous()
        hmax = host_units(1, 2, n)
        C_host = torch.empty((hmax * M_TILE, K), dtype=torch.uint8, pin_memory=True)
        C_host.copy_(codes[:hmax * M_TILE])
        A16 = synth.gemm_inputs(M, K, 1, seed=oi, device="cuda")[0]
        copies16 = max(2, -(-(1 << 30) // (2 * C8)))
        A16s = [A16] + [A16.clone() for _ in range(copies16 - 1)]
        A16_host = torch.empty((host_units(1, 4, n) * M_TILE, K), dtype=torch.bfloat16, pin_memory=True)
        A16_host.copy_(A16[:A16_host.shape[0]])
        for N in (1, 16, 64):
            X = synth.gemm_inputs(M, K, N, seed=oi, device="cuda")[1].contiguous()
            y = torch.empty((N, M), dtype=torch.float32, device="cuda")
            bf16_ms = {}
            for k in (0, 5):
                h = host_units(k, 20, n)
                d16 = [dak.SplitMatrix(A16_host[:h * M_TILE] if h else None, a[h * M_TILE:], M, K, M_TILE, h)
                       for a in A16s]
                bf16_ms[k] = timed(dak.splitk_gemm, d16, X, y)
            ref = None
            for k in (0, 1, 2, 5, 10):
                h = host_units(k, 20, n)
                descs = [dak.SplitMatrixFP8(C_host[:h * M_TILE] if h else None, c[h * M_TILE:] if h < n else None,
                                            scale, M, K, M_TILE, h) for c in Cs]
                t = timed(dak.splitk_gemm_fp8, descs, X, y)
                if ref is None:
                    ref = y.clone()
                same = bool(torch.equal(y, ref))
                t_roof = max((n - h) * (C8 // n) / (b_hbm * 1e9), h * (C8 // n) / (b_host * 1e9)) * 1e3
                pt = {"op": name, "M": M, "K": K, "N": N, "x": round(h / n, 4), "h": h, "ms": round(t, 5),
                      "GBps": round(C8 / (t * 1e-3) / 1e9, 1), "frac_two_tier": round(t_roof / t, 4),
                      "bit_identical_to_x0": same}
                if k in bf16_ms:
                    pt["bf16_ms"] = round(bf16_ms[k], 5)
                    pt["speedup_over_bf16"] = round(bf16_ms[k] / t, 3)
                points.append(pt)
                log(f"fp8 {name} N={N} x={h / n:.3f}: {t * 1e3:.1f} us, {pt['GBps']:.0f} GB/s, "
                    f"{pt['frac_two_tier']:.3f} of roofline"
                    + (f", {pt['speedup_over_bf16']:.2f}x over bf16" if k in bf16_ms else "")
                    + ("" if same else " BITS DIFFER"))
            del X, y
        del codes, Cs, C_host, A16, A16s, A16_host
        torch.cuda.empty_cache()
    pos = [p for p in points if p["x"] > 0]
    res = {
        "metric": "FP8-weight split GEMM: % of the two-tier roofline vs offload ratio x, and speedup over bf16",
        "value": round(statistics.mean(p["frac_two_tier"] for p in pos), 4),
        "unit": "mean fraction of the two-tier roofline over N in {1,16,64}, 4 ops, x = 0.05..0.5",
        "n_gpus": 1, "steps": reps, "warmup": 1, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3 weights, bf16 activations, fp32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "Llama-8B decode linears QKV 6144x4096, O 4096x4096, gate+up 28672x4096, "
                               "down 4096x14336 with FP8 weights at N in {1,16,64}, x in {0, .05, .1, .25, .5}, "
                               "64-row tile-rows, cold"},
        "frac_b_hbm_at_x0": {f"{p['op']}_N{p['N']}": p["frac_two_tier"] for p in points if p["h"] == 0},
        "speedup_over_bf16": {f"{p['op']}_N{p['N']}_x{p['x']}": p["speedup_over_bf16"]
                              for p in points if "speedup_over_bf16" in p},
        "all_bit_identical_across_x": all(p["bit_identical_to_x0"] for p in points),
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "points": points,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_paged(torch, dak, args, b_hbm, b_host):
    """Paged against dense split decode attention at the Llama-8B decode size
    (batch 16, 32 query / 8 KV heads, head_dim 128, 32768 cached tokens; K, V
    ~N(0, 1)).  Paged: 16-token pages at seeded random pool indices (a pool
    after churn) and a seeded random set of host (request, KV head) units, as
    BOOST's single-head-host placement leaves them; dense: the same number of
    head units, the first ones.  Two length mixes: every request full, and
    lengths uniform in [1, 32768] (seeded).  Each point is the mean over
    `--sweep-steps` launches after one untimed launch; paged outputs are
    checked bit-identical to dense."""
    reps = max(1, args.sweep_steps)
    B, Hq, Hkv, D, ctx, page = 16, 32, 8, 128, 32768, 16
    units = B * Hkv
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=7, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    gen = torch.Generator().manual_seed(11)
    mixes = {"full": [ctx] * B, "ragged": torch.randint(1, ctx + 1, (B,), generator=gen).tolist()}
    points = []
    for mix, lens in mixes.items():
        lens_t = torch.tensor(lens, dtype=torch.int32)
        unit_bytes = [lens[u // Hkv] * D * 2 * 2 for u in range(units)]
        total = sum(unit_bytes)
        for h in (0, 4, 8, 16):
            host_set = torch.randperm(units, generator=torch.Generator().manual_seed(100 + h))[:h].tolist()
            kvd = dak.place_kv(K, V, h, unit=dak.KV_UNIT_HEAD, ctx_lens=lens_t)
            kvp = dak.place_paged_kv(K, V, lens_t, page, host_set, seed=h)
            od = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
            op_ = torch.empty_like(od)
            wsd = torch.empty(dak.decode_attn_workspace_bytes(kvd, Hq), dtype=torch.uint8, device="cuda")
            wsp = torch.empty(dak.paged_decode_attn_workspace_bytes(kvp, Hq), dtype=torch.uint8, device="cuda")
            td = timed(lambda: dak.splitk_decode_attn(q, kvd, scale, out=od, ws=wsd))
            tp = timed(lambda: dak.paged_decode_attn(q, kvp, scale, out=op_, ws=wsp))
            same = bool(torch.equal(od, op_))
            for kind, t, hb in (("dense", td, sum(unit_bytes[:h])), ("paged", tp, sum(unit_bytes[u] for u in host_set))):
                t_roof = max((total - hb) / (b_hbm * 1e9), hb / (b_host * 1e9)) * 1e3
                points.append({"mix": mix, "kind": kind, "host_units": h, "x": round(hb / total, 4),
                               "ms": round(t, 4), "GBps": round(total / (t * 1e-3) / 1e9, 1),
                               "frac_two_tier": round(t_roof / t, 4)})
            log(f"{mix} h={h}: dense {td:.3f} ms, paged {tp:.3f} ms ({tp / td:.3f}x)"
                f"{'' if same else ' BITS DIFFER'}")
            points[-1]["bit_identical_to_dense"] = points[-2]["bit_identical_to_dense"] = same
            del kvd, kvp, wsd, wsp
            torch.cuda.empty_cache()
    del q, K, V
    torch.cuda.empty_cache()
    # Granularity at a small batch: 4 requests, a host-share target of 1/10.
    # Whole requests step in quarters (h = ceil(0.1 * 4) = 1 request, 25 % of
    # the cache on the host); (request, KV head) units step in 1/32 (h = 4,
    # 12.5 %).  Time against the all-HBM time and the two-tier roofline.
    Bs = 4
    q4, K4, V4 = synth.attn_inputs(Bs, Hq, Hkv, D, ctx, seed=8, device="cuda")
    total4 = Bs * Hkv * ctx * D * 2 * 2
    gran = []
    for label, unit, h in (("all HBM", dak.KV_UNIT_REQUEST, 0), ("request units", dak.KV_UNIT_REQUEST, 1),
                           ("head units", dak.KV_UNIT_HEAD, 4)):
        kv4 = dak.place_kv(K4, V4, h, unit=unit)
        o4 = torch.empty((Bs, Hq, D), dtype=torch.float32, device="cuda")
        ws4 = torch.empty(dak.decode_attn_workspace_bytes(kv4, Hq), dtype=torch.uint8, device="cuda")
        t = timed(lambda: dak.splitk_decode_attn(q4, kv4, scale, out=o4, ws=ws4))
        hb = kv4.host_bytes
        t_roof = max((total4 - hb) / (b_hbm * 1e9), hb / (b_host * 1e9)) * 1e3
        gran.append({"placement": label, "host_units": h, "host_share": round(hb / total4, 4), "ms": round(t, 4),
                     "frac_two_tier": round(t_roof / t, 4)})
        log(f"batch 4, target x = 0.1: {label}: host share {hb / total4:.3f}, {t:.3f} ms")
        del kv4, ws4
    paged_pts = [p for p in points if p["kind"] == "paged"]
    ratios = [p["ms"] / d["ms"] for p, d in zip(points[1::2], points[0::2])]
    res = {
        "metric": "paged split decode attention: time relative to the dense split kernel, and % of two-tier roofline",
        "value": round(statistics.mean(p["frac_two_tier"] for p in paged_pts), 4),
        "unit": "mean fraction of the two-tier roofline over the paged points",
        "n_gpus": 1, "steps": reps, "warmup": 1, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate", "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "Llama-8B decode attention, batch 16, 32q/8kv heads, head_dim 128, 32768 tokens, "
                               "16-token pages at random pool indices, 0/4/8/16 host (request, KV head) units; "
                               "full and ragged (uniform [1, 32768]) lengths"},
        "paged_over_dense_time": {"mean": round(statistics.mean(ratios), 4), "max": round(max(ratios), 4)},
        "all_bit_identical_to_dense": all(p["bit_identical_to_dense"] for p in points),
        "ragged_lengths": mixes["ragged"],
        "granularity_batch4_target_x0.1": gran,
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "points": points,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_plan_compare(torch, dak, args, b_hbm, b_host):
    """Greedy per-op ratios against one uniform ratio (DAK §4.2.2 and its
    evaluation of per-op ratios at large batch): one Llama-8B decoder layer at
    batch `--plan-batch` (its linears then run at N = batch) over
    `--plan-ctx` tokens per request, with the same global host share x for
    both plans.  T_comp of each GEMM is its measured all-HBM time when that
    exceeds its HBM streaming time by 20 % (compute-bound), else 0; attention
    is memory-bound (T_comp = 0).  Each plan's step is timed and set beside
    the model's time for it."""
    from tiered_memory_offloading_amd.model import LLAMA8B_ONE_LAYER, DecodeModel
    batch, ctx = args.plan_batch, args.plan_ctx
    free, _ = torch.cuda.mem_get_info()

    def time_model(mdl):
        for _ in range(args.warmup):
            mdl.step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            mdl.step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in mdl.slots]
        mdl.step(events=evs)
        torch.cuda.synchronize()
        return ms, [a.elapsed_time(b) for a, b in evs]

    log(f"all-HBM layer at batch {batch}, ctx {ctx}: per-op times for T_comp")
    wts = args.plan_weights
    base = DecodeModel(LLAMA8B_ONE_LAYER, batch, ctx, b_hbm * 1e9, b_host * 1e9, free, x_global=0.0, log=log,
                       weights=wts)
    _, op0 = time_model(base)
    t_comp = {}
    for o, t in zip(base.slots, op0):
        stream_ms = o.bytes / (b_hbm * 1e9) * 1e3
        t_comp[o.kind] = t * 1e-3 if (o.kind != "attn" and t > 1.2 * stream_ms) else 0.0
        log(f"  {o.kind}: {t:.3f} ms all-HBM, streaming {stream_ms:.3f} ms, T_comp {t_comp[o.kind] * 1e3:.3f} ms")
    footprint = base.footprint
    del base
    torch.cuda.empty_cache()
    rows = []
    for xg in args.plan_x:
        row = {"x_global": xg}
        for policy in ("uniform", "greedy"):
            mdl = DecodeModel(LLAMA8B_ONE_LAYER, batch, ctx, b_hbm * 1e9, b_host * 1e9, free, x_global=xg,
                              policy=policy, t_comp=lambda o: t_comp[o.kind], log=lambda *_: None, weights=wts)
            ms, op_ms = time_model(mdl)
            row[policy] = {"ms": round(ms, 4), "modeled_ms": round(mdl.modeled_s * 1e3, 4),
                           "host_bytes": mdl.host_bytes,
                           "host_units": {o.kind: o.host_units for o in mdl.slots},
                           "op_ms": {o.kind: round(t, 4) for o, t in zip(mdl.slots, op_ms)}}
            log(f"x_global {xg}: {policy:7s} {ms:.3f} ms (model {mdl.modeled_s * 1e3:.3f}), host units "
                + ", ".join(f"{o.kind}={o.host_units}/{o.units}" for o in mdl.slots))
            del mdl
            torch.cuda.empty_cache()
        row["speedup_greedy_over_uniform"] = round(row["uniform"]["ms"] / row["greedy"]["ms"], 4)
        row["modeled_speedup"] = round(row["uniform"]["modeled_ms"] / row["greedy"]["modeled_ms"], 4)
        rows.append(row)
    res = {
        "metric": "decode-layer step time with greedy per-op ratios vs one uniform ratio at the same global x",
        "value": round(statistics.mean(r["speedup_greedy_over_uniform"] for r in rows), 4),
        "unit": "mean speedup (uniform ms / greedy ms)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("e4m3 weights, " if wts == "fp8" else "") + "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": f"one Llama-8B decoder layer (QKV, split-KV attention 32q/8kv hd128, O, gate+up, "
                               f"down) at batch {batch}, {ctx} ctx/request"
                               + (", FP8 weights" if wts == "fp8" else ""), "footprint_bytes": footprint},
        "t_comp_ms": {k: round(v * 1e3, 4) for k, v in t_comp.items()},
        "all_hbm_op_ms": {"qkv": round(op0[0], 4), "attn": round(op0[1], 4), "o": round(op0[2], 4),
                          "gate_up": round(op0[3], 4), "down": round(op0[4], 4)},
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "rows": rows,
    }
    print(json.dumps(res), flush=True)
    return 0


def run_prefetch(torch, dak, args, b_hbm, b_host):
    """Direct access against copy-based prefetch on the same step (DAK paper
    §1 Fig. 1 and §2.3 Fig. 2; BOOST §2.5).  For each x the Llama-8B decode
    layer's split operators run twice on the same placement: directly (host
    units read in place over the link) and prefetched (the host units of each
    op copied into a two-slot HBM staging buffer one op ahead by the DMA
    engine, then the op run from HBM).  Beside them: the direct two-tier
    roofline, sum_i max(x_i C_i / B_host, (1 - x_i) C_i / B_hbm), and the
    theoretical prefetch bound with perfect overlap, sum_i max(x_i C_i /
    B_host, (1 + x_i) C_i / B_hbm) (each prefetched byte is written into HBM
    and read back).  Then the copy-interference probe: a 4 GiB HBM streaming
    read alone and beside a 1 GiB host-to-HBM copy."""
    from tiered_memory_offloading_amd.prefetch import PrefetchStep, concurrent_copy_stream

    log("building the workload on the GPU")
    wl = Workload(torch, dak, n_act=args.n_act)
    ops = wl.op_bytes()
    step_bytes = sum(C for _, C, _ in ops)

    def op_list(plan):
        mats, kv = plan
        seq = []
        for L, S in mats:
            seq.append((S, lambda S_, cfg, L=L: dak.splitk_gemm(S_, L["x"], y=L["y"], cfg=cfg)))
        seq.insert(1, (kv, lambda kv_, cfg: dak.splitk_decode_attn(wl.q, kv_, wl.scale, out=wl.out, ws=wl.ws,
                                                                   cfg=cfg)))
        return seq

    def timed(fn, steps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            for _ in range(steps):
                fn()
            torch.cuda.synchronize()
            runs.append((time.perf_counter() - t0) / steps * 1e3)
        return statistics.median(runs)

    den = 20
    rows = []
    # one copy stream for every prefetcher and the probe, checked to run beside
    # the compute stream (streams that share its hardware queue serialize)
    side = concurrent_copy_stream()
    for k in range(0, 11):
        plan = wl.plan(k, den)
        seq = op_list(plan)
        direct_ms = timed(lambda: [fn(op, None) for op, fn in seq], args.sweep_steps)
        pf = PrefetchStep(seq, copy_stream=side)
        prefetch_ms = timed(pf.step, args.sweep_steps)
        t_pf = t_da = 0.0
        for name, C, n in ops:
            h = host_units(k, den, n)
            hb = h * (C // n)
            t_pf += max(hb / (b_host * 1e9), (C + hb) / (b_hbm * 1e9))
            t_da += max(hb / (b_host * 1e9), (C - hb) / (b_hbm * 1e9))
        row = {"x": k / den, "direct_ms": round(direct_ms, 4), "prefetch_ms": round(prefetch_ms, 4),
               "theory_direct_ms": round(t_da * 1e3, 4), "theory_prefetch_ms": round(t_pf * 1e3, 4),
               "direct_GBps": round(step_bytes / (direct_ms * 1e-3) / 1e9, 2),
               "prefetch_GBps": round(step_bytes / (prefetch_ms * 1e-3) / 1e9, 2),
               "speedup_direct": round(prefetch_ms / direct_ms, 4),
               "staging_bytes": pf.staging_bytes, "host_bytes": host_bytes(wl, k, den)}
        rows.append(row)
        log(f"x={k / den:.2f}: direct {direct_ms:.3f} ms (theory {t_da * 1e3:.3f}), prefetch {prefetch_ms:.3f} ms "
            f"(theory {t_pf * 1e3:.3f}), staging {pf.staging_bytes / 2**20:.0f} MiB")
        del pf
        torch.cuda.synchronize()
    torch.cuda.empty_cache()

    log("copy interference: a 4 GiB HBM read alone and beside a 1 GiB host-to-HBM copy")
    g = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    interference = []
    for wg, w in ((1024, 2), (512, 4)):
        alone, beside, copy_ms, n = dak.probe_copy_interference(g, wg, w, src, dst, reps=32, copy_stream=side)
        interference.append({"workgroups": wg, "window": w, "read_alone_ms": round(alone, 4),
                             "read_beside_copy_ms": round(beside, 4), "reads_overlapped": n,
                             "read_GBps_alone": round(g.numel() / alone / 1e6, 1),
                             "read_GBps_beside_copy": round(g.numel() / beside / 1e6, 1) if beside else None,
                             "hbm_bandwidth_loss": round(1 - alone / beside, 4) if beside else None,
                             "copy_ms": round(copy_ms, 3), "copy_GBps": round(src.numel() / copy_ms / 1e6, 2)})
        log(f"  {wg} WGs x {w}: {interference[-1]}")
    del g, src, dst
    torch.cuda.empty_cache()

    sp = [r["speedup_direct"] for r in rows if r["x"] > 0]
    res = {
        "metric": "step time of direct access vs copy-based prefetch over offload ratio x",
        "value": round(math.exp(sum(math.log(v) for v in sp) / len(sp)), 4),
        "unit": "geometric-mean speedup of direct access (prefetch ms / direct ms) over x = 0.05..0.5",
        "n_gpus": 1, "steps": args.sweep_steps, "warmup": 2, "higher_is_better": True, "vs_baseline": None,
        "dtype": "bf16 in, fp32 accumulate", "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": "Llama-8B decode layer split operators, batch 16 (as the headline step); prefetch: "
                               "two-slot HBM staging buffer, copies one op ahead on a second stream",
                   "step_bytes": step_bytes},
        "b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3), "sweep": rows,
        "copy_interference": interference,
        "pages_context": {"gh200_speedup_over_prefetch": "up to 3x", "pcie_speedup_over_prefetch": "up to 1.8x",
                          "gh200_local_bandwidth_loss_from_background_copy": "up to ~10 %",
                          "pcie_gpu_local_bandwidth_loss": "4-7 %"},
    }
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--x-num", type=int, default=5, help="headline ratio numerator over 20 (5 -> 0.25)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="leave out the other configurations' compact numbers from the headline line")
    ap.add_argument("--sweep-steps", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=1.5,
                    help="prefill: seconds of sustained x = 0 launches before timing (the clock climbs under load)")
    ap.add_argument("--workload", choices=("llama8b-layer", "llama70b", "prefill", "linears", "linears-x0",
                                           "plan-compare", "paged", "fp8-linears", "prefetch"),
                    default="llama8b-layer",
                    help="llama70b: the 80-layer 70B-shaped decode step with planner-chosen ratios; prefill: "
                         "the compute-bound 28672x8192x2048 split GEMM; linears: the decode linears one by one "
                         "at N in {1,16,64} over x = 0..0.5, cold; linears-x0: each decode linear at x = 0, "
                         "N in {16, 64}, once per cold weight copy (for counter runs); plan-compare: greedy per-op ratios against a "
                         "uniform ratio for one decoder layer at large batch; paged: paged against dense "
                         "split attention; fp8-linears: the decode linears with FP8 weights; prefetch: direct "
                         "access against copy-based prefetch of the host units, and the copy-interference probe "
                         "(each prints its own JSON line)")
    ap.add_argument("--plan-batch", type=int, default=512, help="plan-compare: batch (activation rows N)")
    ap.add_argument("--plan-ctx", type=int, default=2048, help="plan-compare: tokens per request")
    ap.add_argument("--plan-x", type=float, nargs="+", default=[0.01, 0.02, 0.05],
                    help="plan-compare: global host shares to compare at")
    ap.add_argument("--b70-batch", type=int, default=16, help="llama70b: requests (activation rows N)")
    ap.add_argument("--b70-weights", choices=("bf16", "fp8"), default="bf16", help="llama70b: weight format")
    ap.add_argument("--prefill-weights", choices=("bf16", "fp8"), default="bf16", help="prefill: weight format")
    ap.add_argument("--plan-weights", choices=("bf16", "fp8"), default="bf16", help="plan-compare: weight format")
    ap.add_argument("--b70-kv-unit", choices=("request", "head"), default="request",
                    help="llama70b: KV host unit (whole requests or single (request, KV head) pairs)")
    ap.add_argument("--hbm-reserve-gib", type=float, default=3.0,
                    help="HBM kept free for activations, outputs and workspace in the llama70b plan")
    ap.add_argument("--n-act", type=int, default=BATCH,
                    help="activation rows N of the split GEMMs (config sweeps use 1, 16, 64)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (scale reference for counter runs)")
    ap.add_argument("--only", choices=OP_ORDER, default=None,
                    help="time one operator of the step (for profiling); the JSON then covers that op only")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU (no collectives or sharding); use --gpus 1",
              file=sys.stderr)
        return 2

    import torch
    import tiered_memory_offloading_amd as dak
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dak.library()

    if args.calibrate_copy:
        calibrate_copy(torch)
    log("measuring B_hbm / B_host with the streaming-read probes")
    b_hbm, b_host = measure_bandwidths(torch, dak)
    log(f"B_hbm {b_hbm:.0f} GB/s, B_host {b_host:.2f} GB/s")
    if args.workload == "llama70b":
        return run_llama70b(torch, dak, args, b_hbm, b_host)
    if args.workload == "prefill":
        return run_prefill(torch, dak, args, b_hbm, b_host)
    if args.workload == "linears":
        return run_linears(torch, dak, args, b_hbm, b_host)
    if args.workload == "linears-x0":
        return run_linears_x0(torch, dak, args, b_hbm, b_host)
    if args.workload == "plan-compare":
        return run_plan_compare(torch, dak, args, b_hbm, b_host)
    if args.workload == "paged":
        return run_paged(torch, dak, args, b_hbm, b_host)
    if args.workload == "fp8-linears":
        return run_fp8_linears(torch, dak, args, b_hbm, b_host)
    if args.workload == "prefetch":
        return run_prefetch(torch, dak, args, b_hbm, b_host)
    log("building the workload on the GPU")
    wl = Workload(torch, dak, n_act=args.n_act)
    ops = wl.op_bytes()
    step_bytes = sum(C for _, C, _ in ops)
    den = 20
    k = args.x_num
    plan = wl.plan(k, den)
    log(f"timing {args.steps} steps at x = {k}/{den}")
    if args.only is not None:
        ms, op_ms, _ = time_steps(torch, wl, plan, args.steps, args.warmup, only=args.only)
        i = OP_ORDER.index(args.only)
        name, C, n = ops[i]
        h = host_units(k, den, n)
        print(json.dumps({"only": name, "x": k / den, "ms_per_launch": op_ms[i], "bytes": C,
                          "host_bytes": h * (C // n), "GBps": C / (op_ms[i] * 1e-3) / 1e9,
                          "b_hbm_GBps": b_hbm, "b_host_GBps": b_host}), flush=True)
        return 0
    ms, op_ms, graph_ms = time_steps(torch, wl, plan, args.steps, args.warmup)
    value = step_bytes / (ms * 1e-3) / 1e9
    t_roof = two_tier_roofline_ms(wl, k, den, b_hbm, b_host)
    names = [n for n, _, _ in ops]

    # dominant kernel: the op with the largest measured time
    i_dom = max(range(5), key=lambda i: op_ms[i])
    dom_name, dom_C, dom_n = ops[i_dom]
    dom_h = host_units(k, den, dom_n)
    dom_host_bytes = dom_h * (dom_C // dom_n)
    dom_ms = op_ms[i_dom]
    tr = kernel_traffic("split_attn.hip", f"attn_partial_x{k}_{den}") if dom_name == "attn" else None
    traffic = tr["bytes_per_launch"] if tr else None
    if dom_h > 0:
        ach = dom_host_bytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "host-link", "kernel": dom_name, "achieved": round(ach, 3), "peak": PCIE_GEN5_X16_GBPS,
                "unit": "GB/s", "frac": round(ach / PCIE_GEN5_X16_GBPS, 4), "traffic": traffic,
                "bytes_per_launch": dom_host_bytes, "ms_per_launch": round(dom_ms, 4),
                "note": "host-tier bytes of the op (read once) / its average duration; peak = PCIe Gen5 x16 "
                        "per-direction published rate"}
    else:
        ach = dom_C / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom_name, "achieved": round(ach, 3), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": traffic, "bytes_per_launch": dom_C,
                "ms_per_launch": round(dom_ms, 4)}

    if tr:
        roof["traffic_note"] = tr.get("note", "")
    result = {
        "metric": "effective GB/s (HBM+host) and % of two-tier roofline vs offload ratio x",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms_spread": time_steps.spread,
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms is not None else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp32 accumulate",
        "data": "synthetic (seeded, generated on the GPU; Llama-8B shapes, random weights)",
        "config": {"workload": "Llama-8B decode layer split operators, batch 16: QKV/O/gate+up/down split GEMMs "
                               "(N=16, 64-row tile-rows) + split-KV GQA decode attention (32q/8kv heads, hd 128, "
                               "32768 ctx/request)",
                   "x": k / den, "global_batch": BATCH, "seq_len": CTX, "parallelism": "none (1 GPU)",
                   "step_bytes": step_bytes, "host_bytes": host_bytes(wl, k, den)},
        "two_tier": {"b_hbm_GBps": round(b_hbm, 1), "b_host_GBps": round(b_host, 3),
                     "spec_hbm_GBps": HBM_PEAK_GBPS, "spec_host_GBps": PCIE_GEN5_X16_GBPS,
                     "t_roof_ms": round(t_roof, 4), "frac": round(t_roof / ms, 4),
                     "op_ms": {n: round(t, 4) for n, t in zip(names, op_ms)}},
        "roofline": roof,
    }

    if not args.no_sweep:
        sweep = []
        for kk in range(0, 11):
            p = wl.plan(kk, den)
            sms, sop, sgraph = time_steps(torch, wl, p, args.sweep_steps, 1)
            tr = two_tier_roofline_ms(wl, kk, den, b_hbm, b_host)
            sweep.append({"x": kk / den, "GBps": round(step_bytes / (sms * 1e-3) / 1e9, 2),
                          "frac_two_tier": round(tr / sms, 4), "ms": round(sms, 4),
                          "graph_ms": round(sgraph, 4) if sgraph is not None else None,
                          "op_ms": [round(t, 4) for t in sop]})
            log(f"sweep x={kk / den:.2f}: {sweep[-1]['GBps']} GB/s, {sweep[-1]['frac_two_tier']:.3f} of roofline")
        result["sweep"] = sweep
        x0 = sweep[0]
        i0 = max(range(5), key=lambda i: x0["op_ms"][i])
        ach0 = ops[i0][1] / (x0["op_ms"][i0] * 1e-3) / 1e9
        result["roofline_x0"] = {"bound": "hbm", "kernel": ops[i0][0], "achieved": round(ach0, 1),
                                 "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach0 / HBM_PEAK_GBPS, 4),
                                 "frac_of_measured_b_hbm": round(ach0 / b_hbm, 4)}

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl)
    if not args.no_extras:
        log("other configurations: the 1024x1024 GEMV, the decode linears at x = 0, the prefill GEMM")
        del wl
        torch.cuda.empty_cache()
        result["extras"] = headline_extras(torch, dak, b_hbm, b_host, warm_seconds=args.warm_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
