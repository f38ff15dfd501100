"""The C-ABI library loads, exports every symbol include/dak.h declares, and its
host-side logic (capacity bound, planner, host work-group rule, argument
validation) matches the oracle -- no GPU needed, nothing is launched."""
import ctypes as C
import os
import random
import re

import pytest

import tiered_memory_offloading_amd as dak
from tiered_memory_offloading_amd import _lib as L
from oracle import planner as op
from oracle import schedule as sc
from conftest import ROOT


def _declared_symbols():
    txt = open(os.path.join(ROOT, "include", "dak.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dak_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = dak.library()
    declared = _declared_symbols()
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(n for n, _, _ in L.SIGNATURES) == declared
    assert lib.dak_abi_version() == L.ABI_VERSION


def test_min_offload_ratio_matches_oracle():
    for M, H in [(0, 5), (100, 200), (150 * 10**9, 96 * 10**9), (308_700_000_000, 300_000_000_000), (7, 3)]:
        assert dak.min_offload_ratio(M, H) == op.min_offload_ratio(M, H)


def test_host_workgroups_matches_oracle():
    for items in range(0, 300, 7):
        for cap in (1, 2, 5, 8, 16, 33):
            assert dak.host_workgroups(items, cap) == sc.host_workgroups(items, cap)
    assert dak.host_workgroups(5, 0) == -1


def _rand_instance(rng):
    ops = []
    for _ in range(rng.randint(1, 30)):
        n = rng.randint(1, 200)
        u = rng.choice([1, 3, 512, 1 << 20, 7 << 19, 3 << 26])
        kind = rng.random()
        tc = 0.0 if kind < 0.3 else rng.uniform(0, 3) * n * u / 6.4e12
        ops.append(op.Op(n, u, tc))
    return ops


def test_plans_are_bit_exact_with_oracle_on_random_instances():
    rng = random.Random(21)
    for _ in range(150):
        ops = _rand_instance(rng)
        bg, bh = rng.uniform(1e12, 8e12), rng.uniform(2e10, 5e11)
        x = rng.choice([0.0, 1.0, rng.random(), rng.random() * 0.05])
        ref_h, ref_t = op.plan(ops, bg, bh, x)
        got_h, got_t = dak.plan_offload([dak.Op(o.units, o.unit_bytes, o.t_comp) for o in ops], bg, bh, x)
        assert got_h == ref_h
        assert got_t == ref_t


def test_turning_points_match_oracle():
    rng = random.Random(22)
    for _ in range(200):
        o = op.Op(rng.randint(1, 300), rng.randint(1, 1 << 22), rng.choice([0.0, rng.random() * 1e-3]))
        bg, bh = rng.uniform(1e12, 8e12), rng.uniform(2e10, 5e11)
        a, b, mb = dak.op_turning_points(dak.Op(o.units, o.unit_bytes, o.t_comp), bg, bh)
        assert (a, b) == op.argmin_range(o, bg, bh)
        assert mb == op.memory_bound(o, bg, bh)



def test_turning_points_match_oracle_on_plateaus():
    # Dyadic sizes and bandwidths make T_i(h) hit exact ties, and T_comp set to
    # one side's time at some h makes flat stretches: the first and last
    # minimisers must still be the oracle's (a scan of every h).
    rng = random.Random(23)
    for _ in range(400):
        n = rng.choice([1, 2, 3, 7, 64, 333])
        u = 1 << rng.randint(0, 24)
        bg, bh = 2.0 ** rng.randint(30, 43), 2.0 ** rng.randint(20, 36)
        k = rng.randint(0, n)
        tc = rng.choice([0.0, (n - k) * u / bg, k * u / bh, 2.0 * n * u / bg, 2.0 ** -rng.randint(5, 40)])
        o = op.Op(n, u, tc)
        a, b, mb = dak.op_turning_points(dak.Op(n, u, tc), bg, bh)
        assert (a, b) == op.argmin_range(o, bg, bh), (n, u, tc, bg, bh)
        assert mb == op.memory_bound(o, bg, bh)


def test_turning_points_of_a_huge_op_are_minimisers():
    # 2^40 units: too many to scan.  The library's answer must be minimal at
    # both ends, strictly worse one unit outside, no better at sampled h, and
    # (with T_comp = 0) sit where (n - h) / B_g = h / B_h, i.e. h* = n B_h / (B_g + B_h).
    n, u = 1 << 40, 4096
    bg, bh = 6.4e12, 5.76e10
    t = lambda h, tc: op.unit_time(n, u, h, tc, bg, bh)
    for tc in (0.0, 1e-3, 500.0, 1e6):
        a, b, _ = dak.op_turning_points(dak.Op(n, u, tc), bg, bh)
        assert 0 <= a <= b <= n
        best = t(a, tc)
        assert t(b, tc) == best
        if a > 0:
            assert t(a - 1, tc) > best
        if b < n:
            assert t(b + 1, tc) > best
        rng = random.Random(int(tc * 1000) + 1)
        for h in [rng.randint(0, n) for _ in range(2000)] + [0, n, (a + b) // 2]:
            assert t(h, tc) >= best
        if tc == 0.0:
            assert abs(a - n * bh / (bg + bh)) <= 2 and b - a <= 2
        if tc == 1e6:   # above both sides' time at every split (n u / B_h = 7.8e4 s): every h ties
            assert (a, b) == (0, n)


def test_error_messages_stay_with_their_thread():
    # The last error is thread-local: threads that fail in different ways at
    # the same time, between successful calls, each read back their own message.
    import threading
    good = [dak.Op(8, 1 << 20, 0.0), dak.Op(3, 4096, 1e-6)]
    cases = [
        ("must lie in [0, 1]", lambda: dak.plan_offload(good, 6.4e12, 5.76e10, 1.5)),
        ("bandwidths must be positive", lambda: dak.plan_offload(good, -1.0, 5.76e10, 0.1)),
        ("units and unit_bytes", lambda: dak.plan_offload([dak.Op(0, 8, 0.0)], 6.4e12, 5.76e10, 0.1)),
        ("t_comp_s must be finite", lambda: dak.plan_offload([dak.Op(4, 8, float("nan"))], 6.4e12, 5.76e10, 0.1)),
    ]
    bad = []

    def worker(k):
        want, call = cases[k % len(cases)]
        for i in range(400):
            if i % 2:
                h, _ = dak.plan_offload(good, 6.4e12, 5.76e10, 0.25)
                if sum(hi * o.unit_bytes for hi, o in zip(h, good)) < 0.25 * sum(o.units * o.unit_bytes for o in good):
                    bad.append((k, "budget"))
                continue
            try:
                call()
                bad.append((k, "no error"))
            except dak.DakError as e:
                if want not in str(e):
                    bad.append((k, str(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:5]

def test_decode_step_plan_of_a_70b_shape_matches_oracle():
    # 80 layers x {QKV, attention, O, gate+up, down} with 64-row tile-rows and
    # one request per attention unit; KV for 16 requests of 32768 tokens.
    MiB = 1 << 20
    layer = [op.Op(160, 1 * MiB, 0.0), op.Op(16, 128 * MiB, 0.0), op.Op(128, 1 * MiB, 0.0),
             op.Op(896, 1 * MiB, 0.0), op.Op(128, 7 * MiB // 2, 0.0)]
    ops = layer * 80
    total = sum(o.bytes for o in ops)
    hbm = 280 * (1 << 30)
    x = op.min_offload_ratio(total, hbm)
    ref = op.plan(ops, 6.4e12, 5.75e10, x)
    got = dak.plan_offload([dak.Op(o.units, o.unit_bytes, o.t_comp) for o in ops], 6.4e12, 5.75e10, x)
    assert got == ref
    assert sum(h * o.unit_bytes for h, o in zip(got[0], ops)) >= op.required_host_bytes(x, total)


def test_planner_argument_errors():
    ops = [dak.Op(4, 10, 0.0)]
    for bad in [dict(b_hbm=0.0), dict(b_host=-1.0), dict(x_global=1.5), dict(x_global=float("nan"))]:
        kw = dict(b_hbm=4.0, b_host=1.0, x_global=0.5)
        kw.update(bad)
        with pytest.raises(dak.DakError) as e:
            dak.plan_offload(ops, kw["b_hbm"], kw["b_host"], kw["x_global"])
        assert e.value.status == L.DAK_EINVAL
    with pytest.raises(dak.DakError) as e:
        dak.plan_offload([dak.Op(0, 10, 0.0)], 4.0, 1.0, 0.1)
    assert e.value.status == L.DAK_EINVAL
    with pytest.raises(dak.DakError) as e:
        dak.plan_offload([dak.Op(4, 10, -1.0)], 4.0, 1.0, 0.1)
    assert e.value.status == L.DAK_EINVAL


def _gemm_status(**kw):
    lib = dak.library()
    d = dict(host=None, hbm=None, M=1024, K=1024, m=64, h=0)
    n = kw.pop("N", 1)
    d.update(kw)
    desc = L.SplitMatrixDesc(d["host"], d["hbm"], d["M"], d["K"], d["m"], 0, d["h"])
    return lib.dak_splitk_gemm(C.byref(desc), None, n, None, None, None)


def test_gemm_shape_errors_are_reported_before_any_launch():
    assert _gemm_status(K=1020) == L.DAK_EINVAL          # K % 8 != 0
    assert _gemm_status(m=24) == L.DAK_EINVAL            # m not a multiple of 16
    assert _gemm_status(M=1000) == L.DAK_EINVAL          # M % m != 0
    assert _gemm_status(h=17) == L.DAK_EINVAL            # h > M / m
    assert _gemm_status(h=-1) == L.DAK_EINVAL
    assert _gemm_status(N=0) == L.DAK_EINVAL
    assert _gemm_status(N=2049) == L.DAK_EUNSUPPORTED     # wider than the library takes
    lib = dak.library()
    assert lib.dak_splitk_gemm(None, None, 1, None, None, None) == L.DAK_EINVAL
    assert b"A is NULL" in lib.dak_last_error()
    # a launch configuration outside the documented values
    bad = L.LaunchCfg(0, 3, 0, 0, None)
    desc = L.SplitMatrixDesc(None, None, 1024, 1024, 64, 0, 0)
    assert lib.dak_splitk_gemm(C.byref(desc), None, 1, None, C.byref(bad), None) == L.DAK_EINVAL


def test_attention_shape_errors_are_reported_before_any_launch():
    lib = dak.library()
    kv = L.SplitKVDesc(None, None, None, None, 16, 4, 8, 64, 1024)
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 32, C.c_float(0.1), None, None, 0, None, None) == L.DAK_EUNSUPPORTED
    kv = L.SplitKVDesc(None, None, None, None, 16, 17, 8, 128, 1024)
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 32, C.c_float(0.1), None, None, 0, None, None) == L.DAK_EINVAL
    kv = L.SplitKVDesc(None, None, None, None, 16, 4, 8, 128, 1024)
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 12, C.c_float(0.1), None, None, 0, None, None) == L.DAK_EINVAL
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 128, C.c_float(0.1), None, None, 0, None, None) == L.DAK_EUNSUPPORTED
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 32, C.c_float(float("inf")), None, None, 0, None, None) == L.DAK_EINVAL
    # workspace too small is caught before pointers are looked at
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 32, C.c_float(0.1), None, None, 16, None, None) == L.DAK_EINVAL
    # workspace size: B * Hq * chunks * (D + 2) fp32, chunks of 2048 tokens,
    # or of 4096 where no length array is given and (B * Hkv) * ceil(ctx /
    # 4096) >= 1024 items
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv), 32) == 16 * 32 * 1 * 130 * 4
    kv2 = L.SplitKVDesc(None, None, None, None, 16, 4, 8, 128, 32768)   # 128 units x 8 chunks of 4096
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv2), 32) == 16 * 32 * 8 * 130 * 4
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv2), 30) == 0
    kv3 = L.SplitKVDesc(None, None, None, None, 16, 4, 8, 128, 28673)   # 128 units x 8 chunks of 4096
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv3), 32) == 16 * 32 * 8 * 130 * 4
    kv4 = L.SplitKVDesc(None, None, None, None, 16, 4, 8, 128, 28672)   # 7 chunks of 4096: 2048-token chunks
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv4), 32) == 16 * 32 * 14 * 130 * 4
    kv5 = L.SplitKVDesc(None, None, None, None, 4, 1, 8, 128, 32768)    # 32 units: 2048-token chunks
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv5), 32) == 4 * 32 * 16 * 130 * 4
    # with per-request lengths (any non-null array; not read here): 2048-token chunks
    kv6 = L.SplitKVDesc(None, None, None, None, 16, 4, 8, 128, 32768, 0, 0, 0x1000)
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv6), 32) == 16 * 32 * 16 * 130 * 4


def test_mfma_probe_argument_errors_before_any_launch():
    lib = dak.library()
    ms, tf = C.c_float(), C.c_double()
    assert lib.dak_probe_mfma(0, 16, 1, None, C.byref(ms), C.byref(tf)) == L.DAK_EINVAL
    assert lib.dak_probe_mfma(4, 0, 1, None, C.byref(ms), C.byref(tf)) == L.DAK_EINVAL
    assert lib.dak_probe_mfma(4, 16, 0, None, C.byref(ms), C.byref(tf)) == L.DAK_EINVAL
    assert lib.dak_probe_mfma(4, 16, 1, None, None, None) == L.DAK_EINVAL


def test_binding_structs_match_the_header_layout(tmp_path):
    # Compile the header with the C compiler and compare every struct's size and
    # field offsets with the ctypes mirrors the binding passes across the ABI.
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = [("dak_op_desc", L.OpDesc), ("dak_launch_cfg", L.LaunchCfg),
               ("dak_split_matrix", L.SplitMatrixDesc),
               ("dak_split_matrix_fp8", L.SplitMatrixFP8Desc), ("dak_split_kv", L.SplitKVDesc),
               ("dak_paged_kv", L.PagedKVDesc)]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dak.h"', "int main(void) {"]
    for cname, py in structs:
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, py in structs:
        assert got[(cname, "sizeof")] == C.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_op_time_is_bit_exact_with_oracle():
    # The library's T_i(h) (DAK §4.2.1) against the oracle's, every h of
    # random ops, including compute-bound ones and huge byte counts.
    from oracle import cost_model as cm
    rng = random.Random(31)
    for _ in range(300):
        n = rng.randint(1, 400)
        u = rng.choice([1, 7, 512, 1 << 20, 7 << 19, 3 << 26, (1 << 44) // 401])
        tc = rng.choice([0.0, rng.random() * 1e-3, rng.uniform(0, 3) * n * u / 6.4e12])
        bg, bh = rng.uniform(1e12, 8e12), rng.uniform(2e10, 5e11)
        o = dak.Op(n, u, tc)
        for h in sorted({0, n, rng.randint(0, n), rng.randint(0, n)}):
            assert dak.op_time(o, h, bg, bh) == cm.unit_time(n, u, h, tc, bg, bh)
    with pytest.raises(dak.DakError) as e:
        dak.op_time(dak.Op(4, 10, 0.0), 5, 4.0, 1.0)
    assert e.value.status == L.DAK_EINVAL


def test_uniform_plan_is_bit_exact_with_oracle():
    # The uniform baseline of DAK §4.2.1: h_i = ceil(x n_i), and the
    # modelled time summed in op order, against the oracle.
    rng = random.Random(32)
    for _ in range(150):
        ops = _rand_instance(rng)
        bg, bh = rng.uniform(1e12, 8e12), rng.uniform(2e10, 5e11)
        x = rng.choice([0.0, 1.0, rng.random(), rng.random() * 0.05, 0.05, 0.1, 0.3, 1 / 3, 5e-324])
        ref_h = op.uniform_plan(ops, x)
        ref_t = op.modeled_time(ops, ref_h, bg, bh)
        got_h, got_t = dak.plan_uniform([dak.Op(o.units, o.unit_bytes, o.t_comp) for o in ops], bg, bh, x)
        assert got_h == ref_h
        assert got_t == ref_t
    with pytest.raises(dak.DakError) as e:
        dak.plan_uniform([dak.Op(4, 10, 0.0)], 4.0, 1.0, 1.5)
    assert e.value.status == L.DAK_EINVAL


def test_noalloc_attention_rejects_shapes_beyond_its_scratch_before_any_launch():
    lib = dak.library()
    cap = lib.dak_decode_attn_scratch_max_bytes()
    assert cap == 16 << 20
    # 16 requests x 64 query heads x 32768 tokens: 16 * 64 * 8 records of 520 bytes fit
    kv = L.SplitKVDesc(None, None, None, None, 16, 0, 8, 128, 32768)
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv), 64) <= cap
    # four times the batch (64 * 64 * 8 records) does not
    kv = L.SplitKVDesc(None, None, None, None, 64, 0, 8, 128, 32768)
    assert lib.dak_decode_attn_workspace_bytes(C.byref(kv), 64) > cap
    st = lib.dak_splitk_decode_attn_noalloc(None, C.byref(kv), 64, C.c_float(0.1), None, None, None)
    assert st == L.DAK_EINVAL
    assert b"scratch" in lib.dak_last_error()
    # the workspace entry point still refuses a NULL workspace
    assert lib.dak_splitk_decode_attn(None, C.byref(kv), 64, C.c_float(0.1), None, None, 1 << 30, None,
                                      None) == L.DAK_EINVAL


def test_tuning_defaults_header_matches_the_sweep_table():
    # The library's host work-group defaults are the generated header's, and
    # the header is what the committed sweep table gives.
    import json
    from tiered_memory_offloading_amd import tune
    with open(os.path.join(ROOT, "tiered_memory_offloading_amd", "tuning_mi355x.json")) as f:
        d = tune.defaults_from_table(json.load(f))
    txt = open(tune.HEADER).read()
    consts = dict(re.findall(r"constexpr int (kTuned\w+) = (\d+);", txt))
    assert consts == {"kTunedGemmFmaHostCus": str(d["gemm_fma"]), "kTunedGemmMfmaHostCus": str(d["gemm_mfma"]),
                      "kTunedAttnHostCus": str(d["attn"]), "kTunedRingHostCusMin": str(d["ring_min"]),
                      "kTunedRingHostCusMax": str(d["ring_max"])}
