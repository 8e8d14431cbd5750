"""Throughput of the fused attention JVP (primal + tangent) on one MI355X.

One step = one ``attn_jvp_fwd`` call over the whole workload (every query tile
of every (batch, head)), inputs resident in HBM.  Default workload: the
chunk-wise teacher-forcing mask at causal Wan2.1-1.3B attention shapes
(B=1, H=12, D=128, 21 clean + 21 noisy latent frames of 1560 tokens in chunks
of 3 frames, N = 65,520), bf16.

Prints one JSON line on stdout; progress goes to stderr.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 3]
                  [--no-cpu-baseline] [--no-configs] [--copy-calibration]

Besides the headline workload, the line carries ``configs``: the JVP and the
primal-only kernel (tangents compiled out) on the other bf16 workloads, and
the latency of the tiny fp32 workload (median of 200 single calls).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_VALU_TFLOPS = 157.3
# sources that decide what the bf16 JVP launch does (kernel, launch map, params)
KERNEL_SOURCES = ["attention_jvp_causal_attn_amd/csrc/attn_jvp_bf16_wide.hip",
                  "attention_jvp_causal_attn_amd/csrc/internal.h",
                  "attention_jvp_causal_attn_amd/csrc/attn_jvp_api.cpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_jvp_bf16_chunkwise65k_traffic.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def visible_pairs(w):
    """Admissible pairs per (b, h) under the TF mask: 2F groups of C rows, the
    groups of unit u seeing (u + 1) C keys: C^2 F (F + 1)."""
    F, C = w.n_units, w.unit_tokens
    return C * C * F * (F + 1)


def kernel_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when it
    was taken on the current kernel source and this workload; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    wl = re.search(r"workload:\s*(\S+)", text)
    tb = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (src and wl and tb) or src.group(1) != kernel_hash() or wl.group(1) != workload_name:
        return None
    return float(tb.group(1))


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    total = ev[0].elapsed_time(ev[-1])
    return total / steps, per


def clock_under_load(fn, n_calls=60):
    """The GPU's current shader and memory clocks, as the driver reports them
    in sysfs (pp_dpm_sclk / pp_dpm_mclk, the line marked '*'), sampled every
    20 ms while untimed calls of ``fn`` keep the GPU busy (about a second of
    queued work): min / median / max in MHz.  None when the files are not
    readable."""
    import threading
    import torch
    try:
        pr = torch.cuda.get_device_properties(0)
        dev = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (pr.pci_domain_id, pr.pci_bus_id,
                                                         pr.pci_device_id)
    except Exception:  # noqa: BLE001 - no PCI address, no record
        return None
    files = {k: os.path.join(dev, "pp_dpm_" + k) for k in ("sclk", "mclk")}
    if not all(os.access(f, os.R_OK) for f in files.values()):
        return None

    def current(path):
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*mhz", line.lower())
                    return int(m.group(1)) if m else None
        return None

    samples = {k: [] for k in files}
    done = threading.Event()

    def sample():
        while not done.is_set():
            for k, path in files.items():
                try:
                    v = current(path)
                except OSError:
                    v = None
                if v is not None:
                    samples[k].append(v)
            done.wait(0.02)

    for _ in range(n_calls):
        fn()
    t = threading.Thread(target=sample)
    t.start()
    torch.cuda.synchronize()
    done.set()
    t.join()
    out = {"source": dev + "/pp_dpm_{sclk,mclk}, sampled during untimed JVP calls"}
    for k, v in samples.items():
        v = sorted(v)
        out[k + "_mhz"] = ({"min": v[0], "median": v[len(v) // 2], "max": v[-1], "samples": len(v)}
                           if v else None)
    return out


def blas_info():
    """(library name, thread count) of the BLAS numpy calls, if threadpoolctl
    can tell."""
    try:
        from threadpoolctl import threadpool_info
        blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        if blas:
            return blas[0].get("internal_api", "unknown"), int(blas[0].get("num_threads", 1))
    except Exception:  # noqa: BLE001 - report what is known
        pass
    return "unknown", None


def cpu_baseline(w, x, h=0):
    """The fp64 oracle (as it stands, untuned) on one complete (b, h) slice of
    the workload: every query row.  Every slice of a workload holds the same
    admissible pairs, so the whole call takes B * H times as long; the rate is
    scaled with the same 12 * D FLOP per admissible pair as the GPU figure."""
    from oracle import masked_attention_jvp, tf_allowed
    pred = tf_allowed(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    sl = {k: v[:1, :, h:h + 1] for k, v in x.items()}    # slice (b=0, h)
    pairs = visible_pairs(w)
    t0 = time.perf_counter()
    masked_attention_jvp(sl["q"], sl["k"], sl["v"], sl["dq"], sl["dk"], sl["dv"], pred)
    dt = time.perf_counter() - t0
    lib, threads = blas_info()
    cores = len(os.sched_getaffinity(0))
    return {"value": 12 * w.D * pairs / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle on one complete (b,h) slice of {w.name} "
                       f"({w.N} query rows, {pairs} admissible pairs) in {dt:.1f} s; the "
                       f"whole call is B*H = {w.B * w.H} such slices ({w.B * w.H * dt:.0f} s)"),
            "slice_s": round(dt, 2), "call_s_scaled": round(w.B * w.H * dt, 1),
            "blas": {"library": lib, "threads": threads}, "host_cpus_in_affinity": cores}


def bench_workload(wid, args, stream):
    """JVP and primal-only kernels on workload ``wid`` (bf16), timed like the
    headline: algorithmic TFLOP/s and the JVP/primal time ratio."""
    import torch
    import attention_jvp_causal_attn_amd as aj
    from attention_jvp_causal_attn_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS[wid]
    log(f"config {wid}: {w.describe()}")
    xd = {k: v.to("cuda") for k, v in make_inputs(w).items()}
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    pairs = mask.info()["n_visible_pairs"]
    assert pairs == visible_pairs(w)
    o, do = torch.empty_like(xd["q"]), torch.empty_like(xd["q"])
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")

    def jvp():
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask,
                        o=o, d_o=do, lse=lse, stream=stream)

    def primal():
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask, o=o, lse=lse,
                        stream=stream)

    flops = 12 * w.D * pairs * w.B * w.H
    ms, _ = time_calls(jvp, args.steps, args.warmup, stream)
    pms, _ = time_calls(primal, args.steps, args.warmup, stream)
    tf, ptf = flops / ms / 1e9, flops / 3 / pms / 1e9
    log(f"  JVP {ms:.3f} ms ({tf:.1f} TFLOP/s, {100 * tf / PEAK_BF16_TFLOPS:.1f} %), primal "
        f"{pms:.3f} ms ({ptf:.1f} TFLOP/s), JVP/primal {ms / pms:.2f}")
    out = {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "N": w.N,
           "visible_pairs_per_slice": pairs,
           "jvp": {"ms": round(ms, 4), "tflops": round(tf, 2),
                   "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)},
           "primal_only": {"ms": round(pms, 4), "tflops": round(ptf, 2),
                           "pct_of_bf16_peak": round(100 * ptf / PEAK_BF16_TFLOPS, 2)},
           "jvp_over_primal_time": round(ms / pms, 3)}
    del xd, o, do, lse
    mask.free()
    torch.cuda.empty_cache()
    return out


def bench_tiny_latency(stream, calls=200):
    """Latency of the tiny fp32 workload (B=1, H=2, D=64, 128 tokens): each of
    ``calls`` JVP calls timed alone with events, after warm-up; the median."""
    import torch
    import attention_jvp_causal_attn_amd as aj
    from attention_jvp_causal_attn_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS[1]
    xd = {k: v.to("cuda") for k, v in make_inputs(w).items()}
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    o, do = torch.empty_like(xd["q"]), torch.empty_like(xd["q"])
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device="cuda")

    def jvp():
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask,
                        o=o, d_o=do, lse=lse, stream=stream)

    for _ in range(20):
        jvp()
    torch.cuda.synchronize()
    per = []
    for _ in range(calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        jvp()
        e1.record(stream)
        e1.synchronize()
        per.append(1e3 * e0.elapsed_time(e1))
    per.sort()
    log(f"config 1 ({w.name}): median latency {per[len(per) // 2]:.1f} us over {calls} calls")
    return {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "N": w.N, "dtype": w.dtype,
            "calls": calls, "latency_us_median": round(per[len(per) // 2], 2),
            "latency_us_p10": round(per[len(per) // 10], 2),
            "latency_us_p90": round(per[(9 * len(per)) // 10], 2)}


def bench_split(w, args, stream):
    """The split-key launch where it matters: frame-wise generation with a KV
    cache, the last frame's queries (one frame of tokens) against the cached
    20 clean frames plus itself, every key admissible.  Few query tiles meet
    long key lists, so the unsplit grid leaves compute units idle."""
    import torch
    import attention_jvp_causal_attn_amd as aj
    from attention_jvp_causal_attn_amd.inputs import make_random
    n_q, n_k = w.tokens_per_frame, 21 * w.tokens_per_frame
    xq = make_random(1, n_q, w.H, w.D, dtype=w.dtype, seed=31, tangent_std=0.1, device="cuda")
    xk = make_random(1, n_k, w.H, w.D, dtype=w.dtype, seed=41, tangent_std=0.1, device="cuda")
    m = aj.attn_jvp_mask_rects(n_q, n_k, [0, n_q], [0, 1], [0], [n_k])
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    S = aj.attn_jvp_split_choose(xq["q"], xk["k"], m, n_cu)
    ws = torch.empty(max(16, aj.attn_jvp_fwd_split_workspace(xq["q"], xk["k"], m, S)),
                     dtype=torch.uint8, device="cuda")
    o, do = torch.empty_like(xq["q"]), torch.empty_like(xq["q"])
    lse = torch.empty(1, w.H, n_q, dtype=torch.float32, device="cuda")

    def run(splits):
        return lambda: aj.attn_jvp_fwd(xq["q"], xk["k"], xk["v"], xq["dq"], xk["dk"], xk["dv"],
                                       m, o=o, d_o=do, lse=lse, stream=stream,
                                       max_splits=splits, workspace=ws if splits > 1 else None)

    flops = 12 * w.D * n_q * n_k * w.H
    ums, _ = time_calls(run(1), args.steps, args.warmup, stream)
    sms, _ = time_calls(run(S), args.steps, args.warmup, stream)
    log(f"KV-cache last frame ({n_q} x {n_k}): unsplit {ums:.3f} ms, "
        f"max_splits={S} {sms:.3f} ms ({flops / sms / 1e9:.1f} TFLOP/s)")
    return {"n_q": n_q, "n_k": n_k, "H": w.H, "D": w.D, "max_splits": S,
            "unsplit_ms": round(ums, 4), "split_ms": round(sms, 4),
            "unsplit_tflops": round(flops / ums / 1e9, 2),
            "split_tflops": round(flops / sms / 1e9, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-primal", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-split", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (configs object)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip sampling the GPU clocks under load")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every (batch, head) slice is independent; see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_jvp_causal_attn_amd as aj
    from attention_jvp_causal_attn_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    log(f"workload: {w.describe()}")
    t0 = time.perf_counter()
    x = make_inputs(w)
    xd = {k: v.to("cuda") for k, v in x.items()}
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    mask = aj.attn_jvp_mask_tf(w.n_frames, w.tokens_per_frame, w.frames_per_chunk)
    pairs = mask.info()["n_visible_pairs"]
    assert pairs == visible_pairs(w)
    flops = 12 * w.D * pairs * w.B * w.H
    pflops = 4 * w.D * pairs * w.B * w.H
    B, N, H, D = xd["q"].shape
    o = torch.empty_like(xd["q"])
    do = torch.empty_like(xd["q"])
    lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def jvp():
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], xd["dq"], xd["dk"], xd["dv"], mask,
                        o=o, d_o=do, lse=lse, stream=stream)

    def primal():
        aj.attn_jvp_fwd(xd["q"], xd["k"], xd["v"], None, None, None, mask, o=o, lse=lse,
                        stream=stream)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.float16, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB device copies done")

    ms, per = time_calls(jvp, args.steps, args.warmup, stream)
    per_sorted = sorted(per)
    value = flops / (ms * 1e-3) / 1e12
    log(f"JVP: {ms:.3f} ms/call, {value:.1f} TFLOP/s "
        f"({100 * value / PEAK_BF16_TFLOPS:.1f}% of bf16 peak)")
    clocks = None if args.no_clocks else clock_under_load(jvp)
    log(f"clocks under load: {clocks}")
    res = {
        "metric": "attention-JVP TFLOP/s (primal+tangent) and % of bf16 MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q, K, V, tangents at Wan2.1-1.3B attention shapes)",
        "config": {"workload": w.name, "mask": w.describe(), "B": w.B, "H": w.H, "D": w.D,
                   "N": w.N, "visible_pairs_per_slice": pairs,
                   "algorithmic_flop_per_call": flops, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "ms_p10": round(per_sorted[len(per) // 10], 4),
        "ms_median": round(per_sorted[len(per) // 2], 4),
        "ms_p90": round(per_sorted[(9 * len(per)) // 10], 4),
        "gpu_clocks": clocks,
    }
    if not args.no_primal:
        pms, _ = time_calls(primal, args.steps, args.warmup, stream)
        pval = pflops / (pms * 1e-3) / 1e12
        log(f"primal only: {pms:.3f} ms/call, {pval:.1f} TFLOP/s; JVP/primal time {ms / pms:.2f}")
        res["primal_only"] = {"ms_per_step": round(pms, 4), "tflops": round(pval, 2),
                              "jvp_over_primal_time": round(ms / pms, 3)}
    if not args.no_backward:
        # gradients of the primal (dQ, dK, dV) from the forward's O and LSE:
        # 10*D algorithmic FLOP per admissible pair (S recomputed, dP, dV, dK, dQ)
        g = torch.randn(xd["q"].shape, generator=torch.Generator().manual_seed(77)).to(
            xd["q"].dtype).to("cuda")
        primal()
        gq, gk, gv = (torch.empty_like(xd["q"]) for _ in range(3))
        delta = torch.empty_like(lse)

        def backward():
            aj.attn_jvp_bwd(xd["q"], xd["k"], xd["v"], o, g, lse, mask, g_q=gq, g_k=gk, g_v=gv,
                            delta=delta, stream=stream)

        bms, _ = time_calls(backward, args.steps, args.warmup, stream)
        bval = 10 * w.D * pairs * w.B * w.H / (bms * 1e-3) / 1e12
        log(f"backward: {bms:.3f} ms/call, {bval:.1f} TFLOP/s (10*D FLOP per pair)")
        res["backward"] = {"ms_per_step": round(bms, 4), "tflops": round(bval, 2),
                           "flop_per_pair": 10 * w.D}
    if not args.no_split:
        res["kv_cache_last_frame"] = bench_split(w, args, stream)
    if not args.no_configs:
        del xd, o, do, lse
        torch.cuda.empty_cache()
        configs = {"1": bench_tiny_latency(stream)}
        for wid in (2, 3, 4, 5):
            if wid != args.workload:
                configs[str(wid)] = bench_workload(wid, args, stream)
        res["configs"] = configs
    traffic = measured_traffic(w.name)
    res["roofline"] = {"bound": "mfma", "achieved": round(value, 2), "peak": PEAK_BF16_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                       "traffic": traffic}
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on one complete (b, h) slice ...")
        res["cpu_baseline"] = cpu_baseline(w, x)
        log(f"cpu baseline: {res['cpu_baseline']}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
