"""Benchmark of the SLA2 forward pass on one MI355X.

A step is one pass of the whole hot path over one batch: the router
(pool + projection + score + top-k) and the forward (block summaries, sparse
branch, linear branch, combine), issued as one sla2_attention call (which
overlaps the block summaries with the router), on the
Wan2.1-14B-720P attention shape (B=1, H=40, N=75600, d=128, bf16, b_q=128,
b_kv=64, top-k 3 % = 36 of 1182 KV blocks), with inputs resident in HBM.

Metric: dense-equivalent attention TOPS = 4 B H N^2 d / step time (the pages'
kernel metric, "SLA2 深度解读" 01/13: TOPS of the attention kernel against
FlashAttention2's dense work).  Prints ONE JSON line.

Options: --steps K --warmup W; --gpus N (only 1: the path runs on one GPU);
--no-cpu-baseline skips the oracle timing; --workload wan13b for the smaller
shape; --no-fp8 skips the extra timings of sla2_attention_fp8 (route + the
low-bit sparse branch on the same inputs: e4m3 or int8 Q/K, V bf16 or e4m3);
--no-sla1 skips the extra timing of the SLA (v1) mode (sla1_route +
sla1_forward, k_h 5 %, k_l 10 %, softmax phi) on the same inputs;
--no-train skips the timing of the training-side calls on the same inputs
(sla2_backward; sla2_soft_topk + sla2_soft_topk_grad + sla2_route_grad); --copy-calibration runs only a plain 1 GiB
device copy (used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE);
--counters-summary FETCH WRITE COPY_FETCH COPY_WRITE turns four rocprofv3
--pmc output folders (the bench, then the copy) into the per-launch HBM
traffic of the fused kernel, written to profiles/ and read back by later
runs while the kernel source is unchanged; --traffic-table FETCH WRITE
COPY_FETCH COPY_WRITE prints the same scaled traffic, the mean dispatch
time and the achieved GB/s for every kernel in those folders;
--counter-table DIR prints every counter's mean per dispatch and the mean
dispatch time for every kernel in one rocprofv3 --pmc folder; --peaks
measures the attainable HBM and matrix-core rates of this GPU with plain
library kernels (the measured peaks the roofline fractions are set against,
beside the datasheet's).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "fused128_bf16_wan14b_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the fused kernel's sources (counters are void once it changes)."""
    h = hashlib.sha256()
    for f in ("fused128.hip", "cdna4.h", "hz_layout.h"):
        h.update(open(os.path.join(ROOT, "sparse_linear_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# work accounting (algorithmic: what the method must compute)
# --------------------------------------------------------------------------
def dense_equivalent_flop(B, H, N, d) -> float:
    return 4.0 * B * H * N * N * d


def sparse_flop(idx_host: np.ndarray, N: int, d: int, bq: int, bkv: int) -> float:
    """4 d sum_i n_q(i) sum_{j in S_i} n_kv(j): Q K^T and P V over the
    selected tokens only (valid-token counts for ragged blocks)."""
    BH, Tq, k = idx_host.shape
    Tkv = -(-N // bkv)
    nkv = np.full(Tkv, bkv, np.int64)
    nkv[-1] = N - (Tkv - 1) * bkv
    nq = np.full(Tq, bq, np.int64)
    nq[-1] = N - (Tq - 1) * bq
    if k == 0:
        return 0.0
    sel_tokens = nkv[idx_host].sum(axis=-1)  # [BH, Tq]
    return float(4 * d * (sel_tokens * nq[None, :]).sum())


def linear_apply_flop(BH, N, d) -> float:
    """phi(Q) H_i: 2 N d^2 per head (the linear branch's per-query work)."""
    return 2.0 * BH * N * d * d


def linear_summary_flop(BH, N, d) -> float:
    """sum_j phi(K_j)^T V_j: 2 N d^2 per head."""
    return 2.0 * BH * N * d * d


# Sizes of the linear-branch product (csrc/linear.hip): per head U (T_q rows,
# padded to tiles of 320) times the block summaries (T_kv rows padded to 64,
# 16640 columns: d*d entries of h_j plus d of z_j, padded to tiles of 128).
HZ_COLS, HZ_PITCH, GEMM_M = 128 * 128 + 128, 65 * 256, 320


def product_work(BH, Tq, Tkv):
    """(executed MFMA FLOP, HBM bytes: summaries read once + H written in
    bf16 and Z in fp32) of one linear-branch product launch."""
    tq_pad = -(-Tq // GEMM_M) * GEMM_M
    tkv_pad = -(-Tkv // 64) * 64
    flop = 2.0 * BH * tq_pad * HZ_PITCH * tkv_pad
    byts = BH * (Tkv * HZ_PITCH * 2 + Tq * (128 * 128 * 2 + 128 * 4))
    return flop, byts


def summaries_bytes(BH, N, d, Tkv):
    """Block-summaries pass: read K and V, write V^T (fp16) and the bf16
    per-block summaries rows."""
    return BH * (2 * N * d * 2 + Tkv * 64 * d * 2 + Tkv * HZ_COLS * 2)


# --------------------------------------------------------------------------
COPY_BYTES = 1 << 30
FUSED_KERNEL_RX = r"fused128_kernel<true, 0, false, false, false>"


def copy_calibration():
    import torch
    n = COPY_BYTES
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))


def measured_peaks():
    """Attainable rates of this GPU: HBM by a 4 GiB device-to-device copy
    (read + write counted) and by a read-only sum over 4 GiB; the dense bf16
    matrix cores by an 8192^3 product (torch.mm on contiguous operands, i.e.
    the vendor GEMM library); the matrix-core instruction rate itself (bf16
    32x32x16 and 16x16x32, fp16 32x32x16, e4m3 32x32x64, no memory traffic)
    by the library's
    sla2_mfma_rate_probe.  Mean of 10 (copy, sum), 20 (product) or 5 (probe)
    launches after one warm-up."""
    import torch

    def timeit(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    res = {}
    n = 4 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    x.fill_(1)
    ms = timeit(lambda: y.copy_(x), 10)
    res["hbm_copy"] = {"bytes": 2 * n, "ms": ms, "gbs": 2 * n / ms / 1e6,
                       "frac_of_8tbs": 2 * n / ms / 1e6 / PEAK_HBM_GBS}
    xf = x.view(torch.float32)
    ms = timeit(lambda: xf.sum(), 10)
    res["hbm_read"] = {"bytes": n, "ms": ms, "gbs": n / ms / 1e6,
                       "frac_of_8tbs": n / ms / 1e6 / PEAK_HBM_GBS}
    del x, y, xf
    m = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((m, m), generator=g, device="cuda", dtype=torch.bfloat16)
    b = torch.randn((m, m), generator=g, device="cuda", dtype=torch.bfloat16)
    ms = timeit(lambda: torch.mm(a, b), 20)
    flop = 2.0 * m ** 3
    res["bf16_mm"] = {"m": m, "flop": flop, "ms": ms, "tflops": flop / ms / 1e9,
                      "frac_of_2500": flop / ms / 1e9 / PEAK_BF16_TFLOPS}
    del a, b
    from sparse_linear_attention_amd import sla2 as S
    groups, iters = 2048, 4000
    out = torch.empty(groups * 4, dtype=torch.float32, device="cuda")
    for kind, name, per in ((0, "mfma_bf16_probe", 2.0 * 32 * 32 * 16),
                            (1, "mfma_fp8_probe", 2.0 * 32 * 32 * 64),
                            (2, "mfma_bf16_16x16x32_probe", 2.0 * 16 * 16 * 32),
                            (3, "mfma_fp16_probe", 2.0 * 32 * 32 * 16)):
        ms = timeit(lambda: S.sla2_mfma_rate_probe(kind, iters, groups, out), 5)
        flop = groups * 4.0 * iters * 4.0 * per
        peak = PEAK_FP8_TFLOPS if kind == 1 else PEAK_BF16_TFLOPS
        res[name] = {"flop": flop, "ms": ms, "tflops": flop / ms / 1e9,
                     "frac_of_datasheet": flop / ms / 1e9 / peak}
    res["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(res))


def _counter_means(folder, counter, name_rx):
    """Mean per dispatch (KiB) of one counter over the dispatches whose kernel
    name matches name_rx, from a rocprofv3 --pmc csv folder."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = {}
    names = set()
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or not re.search(name_rx, r["Kernel_Name"]):
                continue
            names.add(r["Kernel_Name"])
            per[(f, r["Dispatch_Id"])] = per.get((f, r["Dispatch_Id"]), 0.0) + float(
                r["Counter_Value"])
    if not per:
        raise SystemExit(f"{counter}: no dispatch of /{name_rx}/ in {folder}")
    v = list(per.values())
    return sum(v) / len(v), len(v), sorted(names)


def _per_kernel(folder):
    """{short kernel name: {"n": dispatches, "ns": mean duration, counter: mean
    per dispatch}} from a rocprofv3 --pmc csv folder (durations from the
    dispatch timestamps of the counter run)."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    disp = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            name = re.sub(r"^(void )?sla2::\(anonymous namespace\)::", "", r["Kernel_Name"])
            name = re.sub(r"\(.*$", "", name)
            d = disp.setdefault((name, f, r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = {}
    for (name, _, _), d in disp.items():
        e = out.setdefault(name, {"n": 0})
        e["n"] += 1
        for k, v in d.items():
            e[k] = e.get(k, 0.0) + v
    for e in out.values():
        for k in list(e):
            if k != "n":
                e[k] /= e["n"]
    return out


def traffic_table(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    cf, _, _ = _counter_means(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _, _ = _counter_means(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    f_fac = COPY_BYTES / (cf * 1024.0)
    w_fac = COPY_BYTES / (cw * 1024.0)
    fk, wk = _per_kernel(fetch_dir), _per_kernel(write_dir)
    print(f"scale: FETCH_SIZE x {f_fac:.3f}, WRITE_SIZE x {w_fac:.3f} "
          f"(1 GiB device copy: {cf:.0f} KiB fetched, {cw:.0f} KiB written per dispatch)")
    print(f"{'kernel':58s} {'disp':>4s} {'read GB':>9s} {'write GB':>9s} {'ms':>8s} "
          f"{'GB/s':>8s} {'of 8 TB/s':>9s}")
    for name in sorted(fk, key=lambda n: -fk[n]["ns"]):
        if "copyBuffer" in name or name not in wk or "FETCH_SIZE" not in fk[name]:
            continue
        rd = fk[name]["FETCH_SIZE"] * 1024.0 * f_fac
        wr = wk[name].get("WRITE_SIZE", 0.0) * 1024.0 * w_fac
        ns = fk[name]["ns"]
        gbs = (rd + wr) / ns
        print(f"{name[:58]:58s} {fk[name]['n']:4d} {rd / 1e9:9.3f} {wr / 1e9:9.3f} "
              f"{ns / 1e6:8.3f} {gbs:8.0f} {gbs / 8000:9.1%}")


def counter_table(folder):
    pk = _per_kernel(folder)
    for name in sorted(pk, key=lambda n: -pk[n]["ns"]):
        e = pk[name]
        print(f"{name}: {e['n']} dispatches, {e['ns'] / 1e6:.3f} ms per dispatch")
        for k in sorted(e):
            if k not in ("n", "ns"):
                print(f"    {k:32s} {e[k]:.6g}")


def counters_summary(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload):
    fk, fn, names = _counter_means(fetch_dir, "FETCH_SIZE", FUSED_KERNEL_RX)
    wk, wn, _ = _counter_means(write_dir, "WRITE_SIZE", FUSED_KERNEL_RX)
    cf, _, _ = _counter_means(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _, _ = _counter_means(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    f_fac = COPY_BYTES / (cf * 1024.0)
    w_fac = COPY_BYTES / (cw * 1024.0)
    read_b = fk * 1024.0 * f_fac
    write_b = wk * 1024.0 * w_fac
    res = {
        "kernel": names[0] if names else FUSED_KERNEL_RX,
        "workload": workload,
        "kernel_source_sha": kernel_source_sha(),
        "fetch_kib_per_dispatch": fk, "fetch_dispatches": fn,
        "write_kib_per_dispatch": wk, "write_dispatches": wn,
        "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": f_fac, "write_scale": w_fac,
        "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": read_b + write_b,
    }
    with open(COUNTERS, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def host_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(x, dense_flop, budget_s=12.0):
    """Times the oracle on a bounded sample of the same workload: whole heads
    (router + forward of every query block of the head), one after another,
    until about `budget_s` seconds of oracle time; the whole-job CPU time is
    the mean time per head times the number of heads."""
    from oracle import oracle as orc
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    threads = max(1, threads)
    w = x.wl
    p = orc.problem_of(x)
    BH = w.B * w.H
    times = []
    while len(times) < BH and sum(times) < budget_s:
        bh = len(times)
        t0 = time.perf_counter()
        idx, _, _, _ = orc.route(p, x.q, x.k, x.wq, x.wk, heads=[bh], nthreads=threads)
        orc.forward(p, x.q, x.k, x.v, idx, x.alpha, [(bh, i) for i in range(w.Tq)],
                    nthreads=threads)
        times.append(time.perf_counter() - t0)
    t_head = sum(times) / len(times)
    t_job = BH * t_head
    return {
        "value": dense_flop / t_job / 1e12,
        "unit": "TOPS",
        "cores": threads,
        "threads": threads,
        **host_info(),
        "kind": "oracle",
        "sample": (f"{len(times)} of {BH} heads, each routed and then run through the forward "
                   f"for all {w.Tq} query blocks ({sum(times):.1f} s, {t_head:.2f} s per head); "
                   f"whole-job CPU time extrapolated as {BH} x per-head time = {t_job:.0f} s"),
        "sample_seconds": sum(times),
    }


def time_calls(torch, S, fn, stream, steps, warmup):
    """(ms per call, {kernel: ms per launch}) of `steps` calls after `warmup`."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    S.timing_start(64 * steps + 64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    st = {n_: ms_ / c_ for n_, (ms_, c_) in S.timing_stop().items()}
    return e0.elapsed_time(e1) / steps, st


def sweep(args, torch, I, S, dev):
    """Sparsity sweep at the Wan-1.3B shape (10 / 5 / 3 / 1 % of the KV
    blocks): per fraction the one-call step, and the same call with the
    linear branch left out (sparse branch alone) and with the sparse branch
    left out (linear branch alone); then the dense baseline, k = T_kv,
    alpha = 1 and no linear branch, i.e. plain softmax attention on the same
    kernels ("SLA2 深度解读" 13 compares with a dense FlashAttention2
    kernel)."""
    base = I.WAN13B
    x = I.make_inputs(base)
    stream = torch.cuda.current_stream()

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v, wq, wk, al = t(x.q), t(x.k), t(x.v), t(x.wq), t(x.wk), t(x.alpha)
    dense = dense_equivalent_flop(base.B, base.H, base.N, base.d)
    O = torch.empty((base.B, base.H, base.N, base.d), dtype=torch.float32, device=dev)
    route_k = ("pool_project", "score", "topk_select", "score_topk")
    rows = []
    for frac in I.SWEEP_FRACS:
        res = {"topk_frac": frac}
        for name, flags in (("full", 0), ("sparse_only", S.FLAG_SKIP_LINEAR),
                            ("linear_only", S.FLAG_SKIP_SPARSE)):
            p = S.problem(base.B, base.H, base.N, base.d, base.bq, base.bkv, frac, 1,
                          base.dtype, flags=flags)
            kk = S.topk(p)
            idx = torch.empty((base.B, base.H, S.num_q_blocks(p), kk), dtype=torch.int32,
                              device=dev)
            ws = S.workspace(p, S.OP_ATTENTION)
            ms, st = time_calls(torch, S, lambda: S.sla2_attention(
                p, q, k, v, wq, wk, al, idx, O, ws, stream), stream, args.steps, args.warmup)
            res["k"] = kk
            res[name] = {"ms_per_step": ms, "stages_ms": st,
                         "route_ms": sum(st.get(n_, 0.0) for n_ in route_k)}
            del ws
        res["tops"] = dense / (res["full"]["ms_per_step"] * 1e-3) / 1e12
        res["sparse_branch_ms"] = res["sparse_only"]["stages_ms"].get("fused_mfma")
        res["linear_branch_ms"] = (res["full"]["stages_ms"].get("lin_gemm", 0.0) +
                                   res["linear_only"]["stages_ms"].get("fused_mfma", 0.0))
        log(f"sweep {frac}: {res['full']['ms_per_step']:.3f} ms/step, sparse "
            f"{res['sparse_branch_ms']:.3f}, linear {res['linear_branch_ms']:.3f}")
        rows.append(res)
    # dense baseline: every block selected, alpha = 1, no linear branch
    p = S.problem(base.B, base.H, base.N, base.d, base.bq, base.bkv, 1.0, 1, base.dtype,
                  flags=S.FLAG_SKIP_LINEAR)
    idx = torch.empty((base.B, base.H, S.num_q_blocks(p), S.topk(p)), dtype=torch.int32,
                      device=dev)
    ones = torch.ones_like(al)
    ws = S.workspace(p, S.OP_ATTENTION)
    ms, st = time_calls(torch, S, lambda: S.sla2_attention(p, q, k, v, wq, wk, ones, idx, O, ws,
                                                           stream), stream, args.steps,
                        args.warmup)
    fused = st.get("fused_mfma")
    dense_res = {"k": S.topk(p), "ms_per_step": ms, "stages_ms": st, "fused_ms": fused,
                 "fused_tflops": dense / (fused * 1e-3) / 1e12 if fused else None}
    for r in rows:
        r["speedup_vs_dense_kernel"] = fused / r["full"]["ms_per_step"] if fused else None
    print(json.dumps({"sweep": rows, "dense_baseline": dense_res,
                      "workload": f"wan13b: B={base.B} H={base.H} N={base.N} d={base.d} "
                                  f"b_q={base.bq} b_kv={base.bkv}",
                      "steps": args.steps, "warmup": args.warmup}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b", choices=["wan14b", "wan13b"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-sla1", action="store_true")
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--counters-summary", nargs=4, metavar="DIR")
    ap.add_argument("--traffic-table", nargs=4, metavar="DIR")
    ap.add_argument("--counter-table", metavar="DIR")
    ap.add_argument("--peaks", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="sparsity sweep at the 1.3B shape with per-branch times and the "
                         "dense baseline (one JSON line)")
    args = ap.parse_args()

    if args.counters_summary:
        counters_summary(*args.counters_summary, workload=args.workload)
        return
    if args.traffic_table:
        traffic_table(*args.traffic_table)
        return
    if args.counter_table:
        counter_table(args.counter_table)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (no sharding, no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration()
        return
    if args.peaks:
        measured_peaks()
        return

    from sparse_linear_attention_amd import inputs as I
    from sparse_linear_attention_amd import sla2 as S

    S.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.sweep:
        sweep(args, torch, I, S, dev)
        return
    w = I.WORKLOADS[args.workload]
    log(f"bench: generating {w.name} inputs")
    x = I.make_inputs(w)

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v, wq, wk, al = t(x.q), t(x.k), t(x.v), t(x.wq), t(x.wk), t(x.alpha)
    p = S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype)
    Tq, Tkv, kk = S.num_q_blocks(p), S.num_kv_blocks(p), S.topk(p)
    idx = torch.empty((w.B, w.H, Tq, kk), dtype=torch.int32, device=dev)
    O = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
    ws_r = S.workspace(p, S.OP_ROUTE)
    ws_f = S.workspace(p, S.OP_FORWARD)
    ws_a = S.workspace(p, S.OP_ATTENTION)
    stream = torch.cuda.current_stream()

    # one step = sla2_attention: the router and the forward in one call (the
    # block summaries overlap the router on a helper stream)
    def step():
        S.sla2_attention(p, q, k, v, wq, wk, al, idx, O, ws_a, stream)

    def step_sequential():
        S.sla2_route(p, q, k, wq, wk, idx, None, ws_r, stream)
        S.sla2_forward(p, q, k, v, idx, al, O, ws_f, stream)

    log("bench: warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    idx_host = idx.cpu().numpy().reshape(w.B * w.H, Tq, kk)

    # timed region: K steps between two synchronisations, HIP events on the
    # launch stream around the whole region and around every kernel launch
    S.timing_start(64 * args.steps + 64)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    kernels = S.timing_stop()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"bench: {ms_step:.3f} ms/step (wall {1e3 * t_wall / args.steps:.3f})")
    # the same work as separate sla2_route + sla2_forward calls, for reference
    # (every kernel alone on one stream: the per-kernel times without overlap)
    for _ in range(args.warmup):
        step_sequential()
    torch.cuda.synchronize()
    S.timing_start(64 * args.steps + 64)
    ev0.record(stream)
    for _ in range(args.steps):
        step_sequential()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_seq = ev0.elapsed_time(ev1) / args.steps
    seq_stages = {name: ms / n for name, (ms, n) in S.timing_stop().items()}

    BH = w.B * w.H
    dense = dense_equivalent_flop(w.B, w.H, w.N, w.d)
    fl_sparse = sparse_flop(idx_host, w.N, w.d, w.bq, w.bkv)
    fl_apply = linear_apply_flop(BH, w.N, w.d)
    stages = {name: ms / n for name, (ms, n) in kernels.items()}
    fused_ms = stages.get("fused_mfma")
    fwd_ms = sum(v for kname, v in stages.items()
                 if kname in ("summaries_mfma", "summaries_reduce", "fused_mfma", "lin_gemm"))
    route_ms = sum(v for kname, v in stages.items()
                   if kname in ("pool_project", "score", "topk_select", "score_topk"))

    achieved = (fl_sparse + fl_apply) / (fused_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(COUNTERS):
        cj = json.load(open(COUNTERS))
        if cj.get("kernel_source_sha") == kernel_source_sha() and cj.get("workload") == w.name:
            traffic = cj.get("hbm_bytes_per_launch")
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": "fused_mfma", "algorithmic_flop_per_launch": fl_sparse + fl_apply,
                "avg_launch_ms": fused_ms}

    qk_bytes = 2.0 * BH * w.N * w.d * 2  # one read of Q and K (router)
    s_bytes = summaries_bytes(BH, w.N, w.d, Tkv)
    g_flop, g_bytes = product_work(BH, Tq, Tkv)

    def hbm(byts, ms):  # achieved rate of algorithmic bytes, alone (sequential calls)
        if not ms:
            return None
        gbs = byts / (ms * 1e-3) / 1e9
        return {"bytes": byts, "ms_alone": ms, "gbs": gbs, "frac_of_8tbs": gbs / PEAK_HBM_GBS}
    out = {
        "metric": "dense-equivalent attention TOPS at 97% sparsity (Wan-14B-720P shape), 1 GPU"
        if w.name == "wan14b" else "dense-equivalent attention TOPS (Wan-1.3B-480P shape), 1 GPU",
        "value": dense / (ms_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded smooth-field Q/K, N(0,1) V; Wan2.1 latent-grid shape)",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} b_q={w.bq} "
                               f"b_kv={w.bkv} top-k {kk} of {Tkv} KV blocks per query block",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "bq": w.bq, "bkv": w.bkv,
                   "topk": kk, "Tq": Tq, "Tkv": Tkv},
        "roofline": roofline,
        "stages_ms": stages,
        "route_ms": route_ms,
        "sequential_ms_per_step": ms_seq,
        "sequential_stages_ms": seq_stages,
        "forward_ms": fwd_ms,
        "forward_only_tops": dense / (fwd_ms * 1e-3) / 1e12 if fwd_ms else None,
        "sparse_flop_per_step": fl_sparse,
        "sparse_fraction_of_dense": fl_sparse / dense,
        # pooling reads Q and K; the summaries read K, V and write V^T and the
        # per-block rows of h_j, z_j; the product reads those rows once and
        # writes H_i, Z_i (fp32): algorithmic bytes over each kernel's time
        # alone (the sequential calls), as a fraction of 8 TB/s
        "router_pool_hbm": hbm(qk_bytes, seq_stages.get("pool_project")),
        "summaries_hbm": hbm(s_bytes, seq_stages.get("summaries_mfma")),
        "linear_product": dict(
            hbm(g_bytes, seq_stages.get("lin_gemm")) or {},
            mfma_flop=g_flop,
            tflops=(g_flop / (seq_stages["lin_gemm"] * 1e-3) / 1e12
                    if seq_stages.get("lin_gemm") else None)),
        "kernel_source_sha": kernel_source_sha(),
    }

    if not args.no_fp8:
        # the low-bit sparse branch on the same inputs: Q, K and P in e4m3
        # ("fp8"), with V quantised per channel as well ("fp8_v"), and the
        # same two with int8 Q/K codes ("i8", "i8_v")
        for key, lb in (("fp8", S.LOWBIT_QK), ("fp8_v", S.LOWBIT_QKV),
                        ("i8", S.LOWBIT_I8QK), ("i8_v", S.LOWBIT_I8QKV)):
            p8 = S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, w.topk_frac, 1, w.dtype, lowbit=lb)
            ws8 = S.workspace(p8, S.OP_ATTENTION_FP8)

            def step8():  # route + low-bit forward in one call, as the bf16 step
                S.sla2_attention_fp8(p8, q, k, v, wq, wk, al, idx, O, ws8, stream)

            for _ in range(args.warmup):
                step8()
            torch.cuda.synchronize()
            S.timing_start(64 * args.steps + 64)
            ev0.record(stream)
            for _ in range(args.steps):
                step8()
            ev1.record(stream)
            torch.cuda.synchronize()
            k8 = S.timing_stop()
            ms8 = ev0.elapsed_time(ev1) / args.steps
            st8 = {n_: ms_ / c_ for n_, (ms_, c_) in k8.items()}
            f8_ms = st8.get("fused_i8" if lb & S.LOWBIT_I8QK else "fused_fp8")
            out[key] = {"ms_per_step": ms8, "tops": dense / (ms8 * 1e-3) / 1e12,
                        "stages_ms": st8,
                        "fused_lowbit_tflops": (fl_sparse + fl_apply) / (f8_ms * 1e-3) / 1e12
                        if f8_ms else None}
            del ws8

    if not args.no_sla1:
        # the SLA (v1) mode on the same inputs: k_h = 5 %, k_l = 10 %, softmax
        # phi, O = O_s + O_l W_p (SLA notes, training section)
        low = 0.10
        p1 = S.problem(w.B, w.H, w.N, w.d, w.bq, w.bkv, 0.05, 1, w.dtype, phi=S.PHI_SOFTMAX)
        kh1, kl1 = S.topk(p1), S.num_negligible(p1, low)
        crit1 = torch.empty((w.B, w.H, Tq, kh1), dtype=torch.int32, device=dev)
        negl1 = torch.empty((w.B, w.H, Tq, kl1), dtype=torch.int32, device=dev)
        wp1 = torch.from_numpy(np.random.default_rng(0).normal(
            0, w.d ** -0.5, (1, w.d, w.d)).astype(np.float32)).to(dev)
        ws1 = S.workspace(p1, S.OP_SLA1_FORWARD)

        def step1():
            S.sla1_route(p1, q, k, low, crit1, negl1, None, ws_r, stream)
            S.sla1_forward(p1, q, k, v, crit1, negl1, low, wp1, O, ws1, stream)

        for _ in range(args.warmup):
            step1()
        torch.cuda.synchronize()
        S.timing_start(64 * args.steps + 64)
        ev0.record(stream)
        for _ in range(args.steps):
            step1()
        ev1.record(stream)
        torch.cuda.synchronize()
        st1 = {n_: ms_ / c_ for n_, (ms_, c_) in S.timing_stop().items()}
        ms1 = ev0.elapsed_time(ev1) / args.steps
        out["sla1"] = {"k_h": kh1, "k_l": kl1, "phi": "softmax", "ms_per_step": ms1,
                       "tops": dense / (ms1 * 1e-3) / 1e12, "stages_ms": st1}
        del ws1

    if not args.no_train:
        # training side on the same inputs: the backward with the selection
        # of the timed steps, and the Stage-1 router calls
        reps = max(1, min(args.steps, 3))
        dO = torch.randn((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        f32 = lambda: torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
        dQ, dK, dV = f32(), f32(), f32()
        dal = torch.empty_like(al)
        wsb = S.workspace(p, S.OP_BACKWARD)
        M = torch.empty((w.B, w.H, Tq, Tkv), dtype=torch.float32, device=dev)
        dM = torch.randn_like(M)
        dSg = torch.empty_like(M)
        dWq, dWk = torch.empty_like(wq), torch.empty_like(wk)
        wsg = S.workspace(p, S.OP_ROUTE_GRAD)
        legs = {
            "backward": lambda: S.sla2_backward(p, q, k, v, idx, al, dO, dQ, dK, dV, dal, wsb,
                                                stream),
            "router_stage1": lambda: (
                S.sla2_soft_topk(p, q, k, wq, wk, 0.1, M, None, ws_r, stream),
                S.sla2_soft_topk_grad(p, M, dM, 0.1, dSg, stream),
                S.sla2_route_grad(p, q, k, wq, wk, dSg, dWq, dWk, wsg, stream)),
        }
        out["train"] = {}
        for name_, fn in legs.items():
            fn()
            torch.cuda.synchronize()
            S.timing_start(64 * reps + 64)
            ev0.record(stream)
            for _ in range(reps):
                fn()
            ev1.record(stream)
            torch.cuda.synchronize()
            stt = {n_: ms_ / c_ for n_, (ms_, c_) in S.timing_stop().items()}
            out["train"][name_] = {"ms": ev0.elapsed_time(ev1) / reps, "reps": reps,
                                   "stages_ms": stt}
        del wsb, wsg

    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(x, dense)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
