"""Offline parameter sweep for the host role (DAK paper §4.3.1, "Congestion
Control Strategy": the host SM count and the per-SM congestion window are fixed
by a lightweight sweep before launch).

Three measurements, all through the C ABI:
  * congestion (Fig. 7 analogue): HBM-role and host-role durations of one
    concurrent streaming launch while the number of host work-groups and their
    window vary, against the HBM role alone;
  * per-operator host throughput: split GEMM (N in {1, 16, 64}; bf16 and FP8
    weights) and split decode attention with all units on the host, over host
    work-groups x window;
  * the chosen (host_cus, window) per operator class, written as JSON.

Run:  python -m tiered_memory_offloading_amd.tune --out tuning.json
      python -m tiered_memory_offloading_amd.tune --header-from tuning.json

tuning_mi355x.json beside this file is the table measured on MI355X with the
current kernels.  The library's host work-group defaults come from it: the
second command writes csrc/tuning_defaults.hpp, which the build includes.
Per operator class the default cap is the sweep's choice, the fewest host
work-groups within 1 % of the best host rate: the split GEMM at N = 1 (the
path for N <= 4), at N = 128 (64 < N <= 256) and split attention.  The staged
bf16 and FP8 GEMMs (4 < N <= 64) size their host role by the link's
bandwidth-delay product instead; their sweeps' choices (N = 16 and 64) bound
that rule from below and above.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import torch

from . import LaunchConfig, place_kv, probe_read, probe_read_concurrent, splitk_decode_attn, splitk_gemm
from . import SplitMatrix, SplitMatrixFP8, SplitKV, library, splitk_gemm_fp8

HOST_CUS = (4, 8, 12, 16, 24, 32, 48, 64)
WINDOWS = (1, 2, 4, 8)


def _time(fn, reps):
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts.sort()
    return ts[len(ts) // 2]


def congestion(hbm_gib=4, host_mib=512, log=print):
    """Fig. 7 analogue: how host readers slow the HBM readers (one launch)."""
    g = torch.empty(hbm_gib << 30, dtype=torch.uint8, device="cuda")
    h = torch.empty(host_mib << 20, dtype=torch.uint8, pin_memory=True)
    alone = probe_read(g, 1024, 2, reps=3)
    out = {"hbm_alone_ms": alone, "hbm_alone_GBps": g.numel() / alone / 1e6, "points": []}
    # Keep the host role busy for the whole HBM pass: size its volume to ~1.5x
    # the HBM time at the link rate.
    host_bytes = min(h.numel(), int(1.5 * alone * 1e-3 * 57e9) // 16 * 16)
    for hw in (1, 2, 4, 8, 16, 32, 64):
        for win in (1, 4, 16):
            t, mg, mh = probe_read_concurrent(g, 1024, 2, h, hw, win, host_bytes=host_bytes)
            pt = {"host_wgs": hw, "host_window": win, "hbm_ms": mg, "host_ms": mh,
                  "hbm_GBps": g.numel() / mg / 1e6, "host_GBps": host_bytes / mh / 1e6,
                  "hbm_slowdown": mg / alone}
            out["points"].append(pt)
            log(f"congestion host_wgs={hw:3d} window={win:2d}: HBM {pt['hbm_GBps']:.0f} GB/s "
                f"({pt['hbm_slowdown']:.3f}x), host {pt['host_GBps']:.1f} GB/s")
    del g, h
    torch.cuda.empty_cache()
    return out


def gemm_host_sweep(N, M=8192, K=4096, reps=3, log=print):
    """All tile-rows on the host: host GB/s per (host_cus, window)."""
    A = torch.randn((M, K), device="cuda").mul_(0.02).to(torch.bfloat16)
    A_host = torch.empty((M, K), dtype=torch.bfloat16, pin_memory=True)
    A_host.copy_(A)
    S = SplitMatrix(A_host, None, M, K, 64, M // 64)
    x = torch.randn((N, K), device="cuda").to(torch.bfloat16)
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    res = []
    for hc in HOST_CUS:
        for w in WINDOWS:
            cfg = LaunchConfig(host_cus=hc, window=w)
            ms = _time(lambda: splitk_gemm(S, x, y=y, cfg=cfg), reps)
            res.append({"host_cus": hc, "window": w, "ms": ms, "host_GBps": M * K * 2 / ms / 1e6})
        log(f"gemm N={N} host_cus={hc}: " + ", ".join(f"w{r['window']}={r['host_GBps']:.1f}" for r in res[-4:]))
    del A, A_host
    return res


def gemm_fp8_host_sweep(N, M=8192, K=8192, reps=3, log=print):
    """FP8 weights, all tile-rows on the host: host GB/s per host_cus (the
    FP8 kernel's ring has a fixed depth, so the window does not apply)."""
    codes = torch.randint(0, 0x7E, (M, K), dtype=torch.uint8, device="cuda")
    C_host = torch.empty((M, K), dtype=torch.uint8, pin_memory=True)
    C_host.copy_(codes)
    scale = torch.full((M,), 1e-3, dtype=torch.float32, device="cuda")
    S = SplitMatrixFP8(C_host, None, scale, M, K, 64, M // 64)
    x = torch.randn((N, K), device="cuda").to(torch.bfloat16)
    y = torch.empty((N, M), dtype=torch.float32, device="cuda")
    res = []
    for hc in HOST_CUS:
        cfg = LaunchConfig(host_cus=hc)
        ms = _time(lambda: splitk_gemm_fp8(S, x, y=y, cfg=cfg), reps)
        res.append({"host_cus": hc, "window": 0, "ms": ms, "host_GBps": M * K / ms / 1e6})
    log(f"gemm fp8 N={N}: " + ", ".join(f"{r['host_cus']}={r['host_GBps']:.1f}" for r in res))
    del codes, C_host
    return res


def attn_host_sweep(B=2, ctx=32768, reps=3, log=print):
    """All requests on the host: host GB/s per (host_cus, window)."""
    Hq, Hkv, D = 32, 8, 128
    K = torch.randn((B, Hkv, ctx, D), device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, ctx, D), device="cuda").to(torch.bfloat16)
    q = torch.randn((B, Hq, D), device="cuda").to(torch.bfloat16)
    kv = place_kv(K, V, B)
    del K, V
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    res = []
    nbytes = 2 * B * Hkv * ctx * D * 2
    for hc in HOST_CUS:
        for w in WINDOWS:
            cfg = LaunchConfig(host_cus=hc, window=w)
            ms = _time(lambda: splitk_decode_attn(q, kv, 1 / math.sqrt(D), out=out, cfg=cfg), reps)
            res.append({"host_cus": hc, "window": w, "ms": ms, "host_GBps": nbytes / ms / 1e6})
        log(f"attn host_cus={hc}: " + ", ".join(f"w{r['window']}={r['host_GBps']:.1f}" for r in res[-4:]))
    return res


def _best(res):
    top = max(r["host_GBps"] for r in res)
    # fewest host work-groups, then smallest window, within 1 % of the best
    ok = [r for r in res if r["host_GBps"] >= 0.99 * top]
    ok.sort(key=lambda r: (r["host_cus"], r["window"]))
    return {"host_cus": ok[0]["host_cus"], "window": ok[0]["window"], "host_GBps": ok[0]["host_GBps"],
            "best_GBps": top}


HEADER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "tuning_defaults.hpp")


def defaults_from_table(table):
    """The library's default host work-group caps from a sweep table."""
    g = table["gemm"]
    ring = [g["16"]["best"]["host_cus"], g["64"]["best"]["host_cus"]]
    ring += [table["gemm_fp8"][n]["best"]["host_cus"] for n in ("1", "16", "64")]
    return {"gemm_fma": g["1"]["best"]["host_cus"], "gemm_mfma": g["128"]["best"]["host_cus"],
            "attn": table["attn"]["best"]["host_cus"], "ring_min": min(ring), "ring_max": max(ring)}


def write_header(table, path=HEADER, source="tuning_mi355x.json"):
    d = defaults_from_table(table)
    text = f"""// Host work-group defaults of the split operators, written by
// `python -m tiered_memory_offloading_amd.tune --header-from {source}`
// from the host-role sweep measured on {table.get("device", "the device")}.  Do not edit: re-run
// the sweep and regenerate.  DAK paper section 4.3.1: the number of compute units
// reading the host comes from an offline sweep; each value is the fewest host
// work-groups whose host rate is within 1 % of the best in its sweep.
#pragma once

namespace dak {{

// Split GEMM, N <= 4 (swept at N = 1, all tile-rows on the host).
constexpr int kTunedGemmFmaHostCus = {d["gemm_fma"]};
// Split GEMM, 64 < N <= 256 (swept at N = 128).
constexpr int kTunedGemmMfmaHostCus = {d["gemm_mfma"]};
// Split decode attention (swept with all requests on the host).
constexpr int kTunedAttnHostCus = {d["attn"]};
// Bounds of the bandwidth-delay rule of the LDS-ring GEMMs (bf16 at
// 4 < N <= 64, FP8 at N <= 64): the smallest and largest choice of their
// sweeps (bf16 at N = 16 and 64, FP8 at N = 1, 16 and 64).
constexpr int kTunedRingHostCusMin = {d["ring_min"]};
constexpr int kTunedRingHostCusMax = {d["ring_max"]};

}}  // namespace dak
"""
    with open(path, "w") as f:
        f.write(text)
    return d


def main(argv=None):
    ap = argparse.ArgumentParser(description="host-role parameter sweep")
    ap.add_argument("--out", default=None)
    ap.add_argument("--skip-congestion", action="store_true")
    ap.add_argument("--header-from", default=None,
                    help="write csrc/tuning_defaults.hpp from this sweep table and exit (no GPU needed)")
    args = ap.parse_args(argv)
    if args.header_from:
        with open(args.header_from) as f:
            d = write_header(json.load(f), source=os.path.basename(args.header_from))
        print(json.dumps(d))
        return 0
    library()
    log = lambda s: print(s, file=sys.stderr, flush=True)
    t0 = time.time()
    table = {"device": torch.cuda.get_device_name(0)}
    if not args.skip_congestion:
        table["congestion"] = congestion(log=log)
    table["gemm"] = {}
    for N in (1, 16, 64, 128):
        res = gemm_host_sweep(N, log=log)
        table["gemm"][str(N)] = {"best": _best(res), "sweep": res}
    table["gemm_fp8"] = {}
    for N in (1, 16, 64):
        res = gemm_fp8_host_sweep(N, log=log)
        table["gemm_fp8"][str(N)] = {"best": _best(res), "sweep": res}
    res = attn_host_sweep(log=log)
    table["attn"] = {"best": _best(res), "sweep": res}
    table["wall_s"] = time.time() - t0
    s = json.dumps(table, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(s)
    print(json.dumps({k: (v["best"] if isinstance(v, dict) and "best" in v else None)
                      for k, v in [("attn", table["attn"])] + [(f"gemm{n}", table["gemm"][n]) for n in table["gemm"]]
                      + [(f"gemm_fp8_{n}", table["gemm_fp8"][n]) for n in table["gemm_fp8"]]}))
    return 0


if __name__ == "__main__":
    sys.exit(main())
