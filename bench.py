"""Throughput of the K3-shape MXFP4 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--config b1|b2|b8|b64|stack12|prefill|prefill_fp4|prefill128|b1_stream|
                              int8_dequant|mfma_rate]

A step is one full pass of the layer (router GEMV + top-k, token->expert
plan, routed MXFP4 gate/up and down GEMVs, shared bf16 experts, weighted
combine) over one batch of synthetic tokens already resident in HBM.  Each
step takes fresh tokens (seed 1000 + i), so the routing and the set of
experts streamed change from step to step.  For batch 1 the layer is held in
several replicas at different addresses, used round-robin, so that no step
finds the previous step's weights in the 256 MB Infinity Cache (in a model
the other layers run in between).

b1_stream is the decode step with the experts NOT resident: their records sit
in pinned host memory and an HBM pool of 256 slots is filled on demand
(moe_pool_fetch, on a copy stream) after the router; the shared experts run
meanwhile and the routed experts wait for the copies (moe_forward_pooled), so
each step includes the host-to-device copies of the experts it misses.

Untimed warmup: the W warmup steps, repeated until they have run for at
least 0.2 s (the GPU's clocks reach their steady state under load).

Printed: one JSON line with tokens/s (value), ms per step, the expert-weight
HBM rate, the dominant kernel's roofline (HIP events around each kernel of
the library's own launches) and the float64 oracle timed on the host cores
on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MAT_BYTES = 7168 * 1536 // 2 + 7168 * 1536 // 32   # one MXFP4 matrix: 5,849,088 B
REC_BYTES = 3 * MAT_BYTES                          # one expert: 17,547,264 B
SHARED_MAT_BYTES = 7168 * 1536 * 2                 # one bf16 shared matrix
# kernels of one moe_layer call, in launch order (see moe_profile_events)
KERNELS_GEMV = ["router_shared_gateup", "select_shared_down", "routed_gateup", "routed_down_combine"]
# one token: the whole layer in one launch
KERNELS_GEMV_ONE = ["decode_front"]
# 2 to 8 tokens: the top-k runs in the router launch; the shared down beside the routed gate/up
KERNELS_GEMV_SMALL = ["router_shared_gateup_topk", "shared_down_routed_gateup", "routed_down_combine"]
KERNELS_MFMA = ["router_quant", "select_plan", "mx_gateup", "mx_down", "combine"]
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense MXFP8 (the FP4 x FP8 block-scaled MFMA rate)
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PCIE_PEAK_GBS = 64.0            # PCIe 5.0 x16, one direction
WARMUP_S = 0.2                  # least wall time of untimed warmup steps

CONFIGS = {
    "b1": dict(tokens=1, layers=1, replicas=8,
               desc="K3 MoE layer decode, batch 1 (H 7168, 896 experts x I 1536 MXFP4, top-16, 2 bf16 shared)"),
    "b2": dict(tokens=2, layers=1, replicas=8,
               desc="K3 MoE layer decode, batch 2 (the speculative-verify shape: the current "
                    "token and one drafted token)"),
    "b8": dict(tokens=8, layers=1, replicas=8,
               desc="K3 MoE layer decode, batch 8"),
    "b64": dict(tokens=64, layers=1, replicas=1,
                desc="K3 MoE layer batched decode, 64 tokens"),
    "stack12": dict(tokens=8, layers=12, replicas=1,
                    desc="12 stacked K3 MoE layers (RMSNorm -> MoE -> residual), batch 8"),
    "prefill128": dict(tokens=4096, layers=1, replicas=1, bias=True, favor=128, path="mfma",
                       steps=20, warmup=3,
                       desc="compute-bound diagnostic of the prefill kernels: 4096 tokens routed to "
                            "128 experts (512 tokens each) by +20 on their logit bias"),
    "b1_stream": dict(tokens=1, layers=1, replicas=1, pool_slots=256, steps=100, warmup=10,
                      desc="K3 MoE layer decode, batch 1, experts streamed from pinned host memory "
                           "into a 256-slot HBM pool (least recently used eviction)"),
    "int8_dequant": dict(kind="int8_dequant", rows=32768, cols=7168, steps=50, warmup=5,
                         desc="row-scaled int8 -> fp32 expansion of a dense weight matrix, "
                              "32768 x 7168 (235 MB int8 -> 940 MB fp32)"),
    "mfma_rate": dict(kind="mfma_rate", steps=10, warmup=3,
                      desc="issue rate of the block-scaled 16x16x128 MFMA: FP4 x FP4 vs FP4 x FP8 "
                           "(vs FP8 x FP8), register operands, 8 independent accumulators per wave"),
    "prefill128_fp4": dict(tokens=4096, layers=1, replicas=1, bias=True, favor=128,
                           path="mfma_fp4", steps=20, warmup=3,
                           desc="compute-bound diagnostic of the FP4 x FP4 prefill kernels: 4096 "
                                "tokens routed to 128 experts (512 tokens each), MXFP4 activations"),
    "prefill_fp4": dict(tokens=4096, layers=1, replicas=1, bias=True, path="mfma_fp4", steps=20,
                        warmup=3,
                        desc="K3 MoE layer prefill, 4096 tokens, per-expert logit bias N(0,0.5), "
                             "MXFP4 activations on block-scaled FP4 x FP4 MFMA"),
    "prefill": dict(tokens=4096, layers=1, replicas=1, bias=True, path="mfma", steps=20, warmup=3,
                    desc="K3 MoE layer prefill, 4096 tokens, per-expert logit bias N(0,0.5), "
                         "MXFP8 activations on block-scaled MFMA"),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="default 200 (prefill 20)")
    p.add_argument("--warmup", type=int, default=None, help="default 20 (prefill 3)")
    p.add_argument("--config", default="b1", choices=sorted(CONFIGS))
    p.add_argument("--replicas", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=1)
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/pmc_<kernel>_<config>.json from two rocprofv3 --pmc "
                        "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) and exit")
    p.add_argument("--stats-summary", metavar="KERNEL_STATS_CSV",
                   help="write profiles/kernel_stats_<config>.json from a rocprofv3 --stats "
                        "run_kernel_stats.csv of this config and exit")
    return p.parse_args()


# dominant launch per config: (HIP kernel name in traces, name in kernel_us)
PMC_KERNELS = {"b1": ("moe_decode_front", "decode_front"),
               "b64": ("moe_routed_gateup", "routed_gateup"),
               "prefill": ("moe_mx_gateup", "mx_gateup"),
               "int8_dequant": ("int8_row_dequant_kernel", "int8_row_dequant")}


def pmc_summary(args, out_dir=None):
    """HBM bytes per launch of the config's dominant kernel from FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch), each scaled by what the counter reads
    for the largest plain device copy in the same run (1 GiB read and
    1 GiB written)."""
    import collections
    import csv
    ksub, name = PMC_KERNELS[args.config]

    def per_kernel(path, counter):
        d = collections.defaultdict(list)
        copies = []  # (dispatch id, value) of the device copies
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                d[r["Kernel_Name"]].append(float(r["Counter_Value"]))
                if "copyBuffer" in r["Kernel_Name"]:
                    copies.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        # the calibration: the run's last three copies (1 GiB each; set-up
        # copies of other sizes come earlier)
        calib = float(np.median([v for _, v in sorted(copies)[-3:]]))
        return d, calib
    f, calib_f = per_kernel(args.pmc_summary[0], "FETCH_SIZE")
    w, calib_w = per_kernel(args.pmc_summary[1], "WRITE_SIZE")
    kf = [k for k in f if ksub in k and "copyBuffer" not in k]
    assert len(kf) == 1, kf
    copy_kib = (1 << 30) / 1024
    fs, wsc = copy_kib / calib_f, copy_kib / calib_w
    fetch = float(np.mean(f[kf[0]]))
    write = float(np.mean(w[kf[0]]))
    if args.config == "int8_dequant":
        c = CONFIGS["int8_dequant"]
        alg = c["rows"] * c["cols"] * 5 + c["rows"] * 4
    elif args.config == "prefill":  # 4096 tokens; every expert active at this routing
        alg = kernel_bytes(name, CONFIGS["prefill"]["tokens"], 16, 896, 2)
    elif args.config == "b64":
        # the counters average over every dispatch of the run, warmup included:
        # distinct experts at their expectation for 64 tokens routed uniformly
        T, k, E = CONFIGS["b64"]["tokens"], 16, 896
        alg = kernel_bytes(name, T, k, E * (1 - (1 - k / E) ** T), 2)
    else:
        alg = kernel_bytes(name, 1, 16, 16, 2)
    out = {"kernel": ksub, "bench_name": name, "config": args.config,
           "source_hash": source_hash(), "dispatches": len(f[kf[0]]),
           "fetch_kib_raw_mean": round(fetch, 1), "write_kib_raw_mean": round(write, 1),
           "calibration": {"copy_bytes": 1 << 30, "fetch_kib_raw": calib_f, "write_kib_raw": calib_w,
                           "fetch_scale": round(fs, 3), "write_scale": round(wsc, 3)},
           "fetch_bytes_per_launch": round(fetch * 1024 * fs),
           "write_bytes_per_launch": round(write * 1024 * wsc)}
    out["bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    out["algorithmic_bytes"] = round(alg)
    out["traffic_over_algorithmic"] = round(out["bytes_per_launch"] / alg, 4)
    # the config's other launches, same runs and scaling
    others = {}
    for n in config_kernels(args.config):
        hit = [kn for kn in f if HIP_KERNEL[n] in kn and "copyBuffer" not in kn]
        if len(hit) == 1 and hit[0] != kf[0] and hit[0] in w:
            others[n] = {"fetch_bytes_per_launch": round(float(np.mean(f[hit[0]])) * 1024 * fs),
                         "write_bytes_per_launch": round(float(np.mean(w[hit[0]])) * 1024 * wsc)}
    if others:
        out["other_launches"] = others
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"pmc_{name}_{args.config}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)
    return out


# the HIP kernel (a substring of its name in a kernel trace) of each timed launch
HIP_KERNEL = {"decode_front": "moe_decode_front", "routed_down_combine": "moe_routed_down_combine",
              "routed_gateup": "moe_routed_gateup", "shared_down_routed_gateup": "moe_routed_gateup",
              "router_shared_gateup": "moe_router_shared_gateup",
              "router_shared_gateup_topk": "moe_router_shared_gateup",
              "select_shared_down": "moe_select_shared_down", "select_plan": "moe_select_shared_down",
              "router_quant": "moe_router_mx_quant", "mx_gateup": "moe_mx_gateup",
              "mx_down": "moe_mx_down", "combine": "moe_combine(",
              "int8_row_dequant": "int8_row_dequant_kernel"}


def config_kernels(config):
    cfgd = CONFIGS[config]
    if cfgd.get("kind") == "int8_dequant":
        return ["int8_row_dequant"]
    T = cfgd["tokens"]
    return (KERNELS_MFMA if cfgd.get("path") in ("mfma", "mfma_fp4") else KERNELS_GEMV_ONE
            if T == 1 else KERNELS_GEMV_SMALL if T <= 8 else KERNELS_GEMV)


def stats_summary(args):
    """Average kernel durations of a rocprofv3 --kernel-trace --stats run of
    this config, per timed launch, with the hash of the kernel sources."""
    import csv
    rows = list(csv.DictReader(open(args.stats_summary)))
    out = {"config": args.config, "source_hash": source_hash(), "kernels": {}}
    for name in config_kernels(args.config):
        hit = [r for r in rows if HIP_KERNEL[name] in r["Name"]]
        assert len(hit) == 1, (name, [r["Name"] for r in hit])
        r = hit[0]
        out["kernels"][name] = {"calls": int(r["Calls"]),
                                "avg_us": round(float(r["AverageNs"]) / 1e3, 2),
                                "min_us": round(float(r["MinNs"]) / 1e3, 2),
                                "max_us": round(float(r["MaxNs"]) / 1e3, 2)}
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{args.config}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out), flush=True)


def rocprof_us(name, config):
    """A launch's average duration in the committed rocprofv3 summary of this
    config, or None once the kernel sources have changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{config}.json")
    if os.path.exists(path):
        d = json.load(open(path))
        if d.get("source_hash") == source_hash() and name in d["kernels"]:
            return d["kernels"][name]["avg_us"]
    return None


def pmc_traffic(name, config):
    """bytes_per_launch of a committed counter summary, or None once the
    kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{name}_{config}.json")
    if os.path.exists(path):
        pmc = json.load(open(path))
        if pmc.get("source_hash") == source_hash():
            return pmc.get("bytes_per_launch")
    return None


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_routed_expert_x896_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def kernel_bytes(name, T, k, D, S, H=7168, I=1536, E=896):
    """Algorithmic HBM bytes of one launch: weights read once, activations in
    and out; intermediates passed between launches counted once where they
    are written and once where they are read (h and the shared h as bf16
    hi + lo, 4 bytes per element; shared outputs fp32).  The routed
    partials that stay inside the down launch are not counted."""
    x = T * H * 2
    if name == "router_shared_gateup":
        return E * H * 2 + x + T * E * 4 + S * 2 * SHARED_MAT_BYTES + S * T * I * 4
    if name == "router_shared_gateup_topk":  # + logits read back, ids and weights written
        return (E * H * 2 + x + 2 * T * E * 4 + T * k * 8
                + S * 2 * SHARED_MAT_BYTES + S * T * I * 4)
    if name == "select_shared_down":
        return (T * E * 4 + T * k * 8 + T * k * 4 + E * 8
                + S * SHARED_MAT_BYTES + S * T * I * 4 + S * T * H * 4)
    if name == "routed_gateup":
        return D * 2 * MAT_BYTES + x + T * k * I * 4
    if name == "shared_down_routed_gateup":
        return (T * k * 4 + D * 2 * MAT_BYTES + x + T * k * I * 4
                + S * SHARED_MAT_BYTES + S * T * I * 4 + S * T * H * 4)
    if name == "routed_down_combine":
        return D * MAT_BYTES + T * k * I * 4 + T * k * 4 + S * T * H * 4 + x
    if name == "decode_front":  # the whole one-token layer: the three-launch sum
        return (kernel_bytes("router_shared_gateup_topk", T, k, D, S, H, I, E)
                + D * 2 * MAT_BYTES + T * k * 4 + T * k * I * 4
                + S * SHARED_MAT_BYTES + S * T * I * 4 + S * T * H * 4
                + kernel_bytes("routed_down_combine", T, k, D, S, H, I, E))
    # prefill (MFMA) path; MXFP8 rows are padded to multiples of 512 (exact at K3)
    xq = T * H * (1 + 1 / 32)
    hq = T * k * I * (1 + 1 / 32)
    if name == "router_quant":
        return E * H * 2 + x + xq + T * E * 4 + E * 4
    if name == "select_plan":
        return T * E * 4 + T * k * 8 + T * k * 4 * 2 + E * 8
    if name == "mx_gateup":
        return D * 2 * MAT_BYTES + S * 2 * SHARED_MAT_BYTES + xq + x + hq + S * T * I * 4
    if name == "mx_down":
        return D * MAT_BYTES + S * SHARED_MAT_BYTES + hq + S * T * I * 4 + T * k * H * 4 + S * T * H * 4
    if name == "combine":
        return T * k * H * 4 + T * k * 4 + S * T * H * 4 + T * H * 2
    raise KeyError(name)


def mfma_flops(name, T, k, S, H=7168, I=1536, E=896):
    """Matrix-core FLOPs of a prefill launch (routed on the scaled FP4 x FP8
    MFMA, shared experts and router on bf16; the shared down counts its hi
    and lo halves)."""
    if name == "mx_gateup":
        return 2 * 2 * T * k * H * I, 2 * 2 * S * T * H * I
    if name == "mx_down":
        return 2 * T * k * H * I, 2 * 2 * S * T * H * I
    if name == "router_quant":
        return 0, 2 * T * E * H
    return 0, 0


def cpu_baseline(cfg_name, n_tokens):
    """The float64 oracle on the host cores, on a bounded sample."""
    import synth
    from oracle import moe as M
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    c = synth.K3
    H, I = c["hidden"], c["inter"]
    cfg = CONFIGS[cfg_name]
    mx = cfg.get("path") == "mfma"
    mx4 = cfg.get("path") == "mfma_fp4"
    bias = synth.router_bias(0, 0, c["n_experts"]) if cfg.get("bias") else None
    if bias is not None and cfg.get("favor"):
        bias = bias.copy()
        bias[:cfg["favor"]] += 20.0
    layer = M.Layer(H, I, c["n_experts"], c["top_k"], synth.router_weight(0, 0, c["n_experts"], H),
                    expert_record=lambda e: synth.expert_record(0, 0, e, H, I),
                    shared=[synth.shared_expert(0, 0, s, H, I) for s in range(c["n_shared"])],
                    router_bias=bias)
    n_layers = cfg["layers"]
    t0 = time.perf_counter()
    done = 0
    for i in range(n_tokens):
        # one token of the workload's input through one layer (route + experts)
        M.moe_layer(synth.activations(1000 + i, 1, H), layer, act_mxfp8=mx, act_mxfp4=mx4)
        done += 1
        if time.perf_counter() - t0 > 30:
            break
    dt = time.perf_counter() - t0
    # a token of the stacked workload passes n_layers layers
    return {"value": round(done / dt / n_layers, 6), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} single-token layer call(s) of {cfg_name} through the float64 numpy "
                      f"oracle ({'MXFP8 activations, logit bias, ' if mx else ''}"
                      f"{'MXFP4 activations, logit bias, ' if mx4 else ''}"
                      f"router + 16 experts dequantised and applied + 2 shared"
                      f"{', scaled by 1/%d layers' % n_layers if n_layers > 1 else ''}), "
                      f"{dt:.1f} s; BLAS threads {threads}, host cpu_count {os.cpu_count()}"}


def mfma_rate_bench(args, cfgd):
    """Matrix-core rate of the block-scaled MFMA per operand-format pair, at 2
    and 4 waves per SIMD, timed by the launch-stamped events (interleaved
    order, median of `steps` launches per case)."""
    import ctypes
    import torch
    from mxfp4_routed_expert_x896_amd import binding as b
    steps = args.steps if args.steps is not None else cfgd["steps"]
    warmup = args.warmup if args.warmup is not None else cfgd["warmup"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cu = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4000
    pairs = [("fp4xfp4", 4, 4), ("fp4xfp8", 4, 0), ("fp8xfp8", 0, 0)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    arr = (ctypes.c_void_p * 2)(*[e.cuda_event for e in evs])
    res = {}
    for wps in (2, 4):
        blocks = cu * wps  # 4 waves per workgroup, one per SIMD
        out = torch.empty(blocks * 4, dtype=torch.float32, device=dev)
        flops = blocks * 4 * iters * 8 * 2 * 16 * 16 * 128
        times = {n: [] for n, _, _ in pairs}
        for _ in range(warmup):
            for n, af, bf in pairs:
                b.mfma_rate(af, bf, iters, blocks, out)
        torch.cuda.synchronize()
        b.profile_events(arr, 2)
        for i in range(steps):  # ABBA: alternate the order of the cases
            for n, af, bf in (pairs if i % 2 == 0 else pairs[::-1]):
                b.mfma_rate(af, bf, iters, blocks, out)
                torch.cuda.synchronize()
                times[n].append(evs[0].elapsed_time(evs[1]) * 1e-3)
        b.profile_events(None, 0)
        assert torch.isfinite(out).all()
        for n in times:
            res[f"{n}_tflops_{wps}w"] = round(flops / float(np.median(times[n])) / 1e12, 1)
    ratio = res["fp4xfp4_tflops_4w"] / res["fp4xfp8_tflops_4w"]
    out = {
        "metric": "block-scaled MFMA issue rate (diagnostic)",
        "value": res["fp4xfp4_tflops_4w"], "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "higher_is_better": True, "vs_baseline": None, "dtype": "fp4*fp4->f32",
        "data": "register operands", "config": {"workload": cfgd["desc"], "iters": iters},
        "rates_tflops": res, "fp4xfp4_over_fp4xfp8": round(ratio, 3),
        "peaks_tflops": {"fp4": FP4_MFMA_PEAK_TFLOPS, "fp8": FP8_MFMA_PEAK_TFLOPS},
        "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def int8_dequant_bench(args, cfgd):
    """One step = one row-scaled int8 -> fp32 expansion of the whole matrix.
    Bytes per element: 1 read + 4 written (+ 4 per row for the scale)."""
    import torch
    from mxfp4_routed_expert_x896_amd import binding as b
    R, C = cfgd["rows"], cfgd["cols"]
    steps = args.steps if args.steps is not None else cfgd["steps"]
    warmup = args.warmup if args.warmup is not None else cfgd["warmup"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(0)
    # two input copies used alternately, so a step does not find the previous
    # step's 235 MB of int8 in the 256 MB Infinity Cache
    qs = [torch.randint(-128, 128, (R, C), dtype=torch.int8, device=dev, generator=g)
          for _ in range(2)]
    ss = [(torch.rand(R, device=dev, generator=g) * 1e-3 + 1e-5).float() for _ in range(2)]
    out = torch.empty((R, C), dtype=torch.float32, device=dev)
    nbytes = R * C * (1 + 4) + R * 4
    for i in range(warmup):
        b.int8_row_dequant(qs[i % 2], ss[i % 2], out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        b.int8_row_dequant(qs[i % 2], ss[i % 2], out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the kernel alone: it stamps a pair of events with its own start and end
    # (moe_profile_events), on the stream it runs on
    import ctypes
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    arr = (ctypes.c_void_p * 2)(*[e.cuda_event for e in evs])
    b.profile_events(arr, 2)
    k = []
    for i in range(steps):
        b.int8_row_dequant(qs[i % 2], ss[i % 2], out)
        assert b.profile_count() == 2
        torch.cuda.synchronize()
        k.append(evs[0].elapsed_time(evs[1]) * 1e3)
    b.profile_events(None, 0)
    k_us = float(np.mean(k))
    achieved = nbytes / (k_us * 1e-6) / 1e9
    res = {
        "metric": "GB/s, row-scaled int8 -> fp32 expansion (int8 read + fp32 written)",
        "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8*f32->f32",
        "data": "synthetic (seeded; int8 uniform over -128..127, scales uniform 1e-5..1e-3)",
        "config": {"workload": cfgd["desc"], "rows": R, "cols": C},
        "kernel_us": {"int8_row_dequant": round(k_us, 2)},
        "roofline": {"kernel": "int8_row_dequant", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": pmc_traffic("int8_row_dequant", "int8_dequant"),
                     "algorithmic_bytes": nbytes},
    }
    del qs, ss, out
    if args.calib_copy:  # a plain 1 GiB device copy for the counter calibration
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        from oracle import spine as S
        rng = np.random.default_rng(0)
        rs = 2048
        q = rng.integers(-128, 128, size=(rs, C), dtype=np.int16).astype(np.int8)
        sc = (rng.random(rs) * 1e-3 + 1e-5).astype(np.float32)
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 10.0:
            S.int8_row_dequant(q, sc)
            n += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(n * (rs * C * 5 + rs * 4) / dt / 1e9, 3),
                               "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} calls of the float64 numpy oracle on {rs} x {C} "
                                         "(the same bytes per element), about 10 s"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design note, not a measured path)",
              file=sys.stderr)
        sys.exit(2)

    cfgd = CONFIGS[args.config]
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.stats_summary:
        stats_summary(args)
        return
    if cfgd.get("kind") == "int8_dequant":
        int8_dequant_bench(args, cfgd)
        return
    if cfgd.get("kind") == "mfma_rate":
        mfma_rate_bench(args, cfgd)
        return

    import torch
    import synth
    import synth.device as SD
    from mxfp4_routed_expert_x896_amd import binding as b

    T, n_layers = cfgd["tokens"], cfgd["layers"]
    if args.steps is None:
        args.steps = cfgd.get("steps", 200)
    if args.warmup is None:
        args.warmup = cfgd.get("warmup", 20)
    mfma = cfgd.get("path") in ("mfma", "mfma_fp4")
    fp4_act = cfgd.get("path") == "mfma_fp4"
    path = b.PATH_MFMA_FP4 if fp4_act else b.PATH_MFMA if mfma else b.PATH_GEMV
    KERNELS = config_kernels(args.config)
    replicas = args.replicas or cfgd["replicas"]
    c = synth.K3
    H, I, E, k, S = c["hidden"], c["inter"], c["n_experts"], c["top_k"], c["n_shared"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- layers resident in HBM
    t_setup = time.time()
    layers, keep = [], []
    n_distinct = n_layers
    for l in range(n_distinct):
        d = SD.upload_layer(c, seed=0, layer=l, bias=bool(cfgd.get("bias")))
        if cfgd.get("favor"):  # diagnostic: every token's top-16 among the favoured experts
            d["router_bias"][: cfgd["favor"]] += 20.0
        L = b.Layer.from_canonical(H, I, E, k, d["router_w"], d["experts"], d["shared_gate"],
                                   d["shared_up"], d["shared_down"], d["router_bias"])
        del d  # canonical copies are not needed once packed
        keep.append(L)
        layers.append(L)
        print(f"[bench] layer {l} resident ({time.time() - t_setup:.0f} s)", file=sys.stderr,
              flush=True)
    if n_layers == 1:
        for r in range(1, replicas):
            L0 = layers[0]
            t = {n: (getattr(L0, n).clone() if getattr(L0, n) is not None else None)
                 for n in ("router_w", "experts", "shared_gate", "shared_up", "shared_down")}
            layers.append(b.Layer(H, I, E, k, t["router_w"], t["experts"], t["shared_gate"],
                                  t["shared_up"], t["shared_down"]))
    torch.cuda.synchronize()
    gammas = [SD.upload_gamma(0, l, H)[1] for l in range(n_layers)]
    n_steps = args.warmup + args.steps
    xs = torch.stack([SD.upload_tokens(1000 + i, T, H)[1] for i in range(n_steps)])
    ids = torch.empty((n_steps, n_layers, T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((n_steps, n_layers, T, k), dtype=torch.float32, device=dev)
    y = torch.empty((n_layers + 1, T, H), dtype=torch.int16, device=dev)
    normed = torch.empty((T, H), dtype=torch.int16, device=dev)
    ws = layers[0].workspace(T)
    pool = pooled = copy_stream = ready = None
    if cfgd.get("pool_slots"):
        copy_stream = torch.cuda.Stream(device=dev)  # default priority
        ready = torch.cuda.Event()
        L0 = layers[0]
        host = torch.empty(L0.experts.shape, dtype=torch.uint8, pin_memory=True)
        host.copy_(L0.experts)
        pool = b.ExpertPool(host, cfgd["pool_slots"], device=dev)
        pooled = b.Layer(H, I, E, k, L0.router_w, pool.slots, L0.shared_gate, L0.shared_up,
                         L0.shared_down, L0.router_bias, pool=pool)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.time() - t_setup:.0f} s; {len(layers)} resident layer copies",
          file=sys.stderr, flush=True)

    def step(i):
        if pooled is not None:
            # the router picks the experts (a host round trip for the ids);
            # the pool copies their records on the copy stream while the
            # shared experts run; the routed experts wait for the copies
            b.route(pooled, xs[i], ids[i, 0], wts[i, 0], ws)
            ids_host = ids[i, 0].cpu().numpy()
            copy_stream.wait_stream(torch.cuda.current_stream())
            pool.fetch(ids_host, stream=copy_stream)
            ready.record(copy_stream)
            b.forward_pooled(pooled, xs[i], ids[i, 0], wts[i, 0], y[0], ws, ready, path=path)
        elif n_layers == 1:
            L = layers[i % len(layers)]
            b.moe_layer(L, xs[i], y[0], ids[i, 0], wts[i, 0], ws, path=path)
        else:
            cur = xs[i]
            for l in range(n_layers):
                b.rmsnorm(cur, gammas[l], 1e-6, normed)
                b.moe_layer(layers[l], normed, y[l + 1], ids[i, l], wts[i, l], ws,
                            residual=cur, path=path)
                cur = y[l + 1]

    # warmup: the W warmup steps, repeated until the GPU has run at least
    # WARMUP_S of them (after the idle setup the clocks need tens of
    # milliseconds of load to reach their steady state: the first 25 ms of
    # one-token steps ran 6% slower than the next)
    t_w = time.perf_counter()
    warmup_run = 0
    while True:
        for i in range(args.warmup):
            step(i)
        warmup_run += args.warmup
        torch.cuda.synchronize()
        if args.warmup == 0 or time.perf_counter() - t_w >= WARMUP_S:
            break
    pool_before = pool.stats() if pool is not None else None
    t0 = time.perf_counter()
    for i in range(args.warmup, n_steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)

    # distinct experts per (step, layer)
    id_np = ids[args.warmup:].cpu().numpy()
    D = np.array([[len(np.unique(id_np[s, l])) for l in range(n_layers)]
                  for s in range(args.steps)])
    exp_bytes = (D * REC_BYTES + S * 3 * SHARED_MAT_BYTES).sum(axis=1).mean()
    exp_gbs = exp_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- per-kernel durations: each of the library's kernels stamps a pair of
    # events with its own start and end (moe_profile_events)
    n_ev = 16
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    import ctypes
    arr = (ctypes.c_void_p * n_ev)(*[e.cuda_event for e in evs])
    b.profile_events(arr, n_ev)
    per_kernel = {name: [] for name in KERNELS}
    span = []
    prof_steps = min(args.steps, 100)
    for i in range(args.warmup, args.warmup + prof_steps):
        L = layers[i % len(layers)]
        b.moe_layer(L, xs[i], y[0], ids[i, 0], wts[i, 0], ws, path=path)
        cnt = b.profile_count()
        torch.cuda.synchronize()
        for j, name in enumerate(KERNELS[:cnt // 2]):
            per_kernel[name].append(evs[2 * j].elapsed_time(evs[2 * j + 1]) * 1e3)
        span.append(evs[0].elapsed_time(evs[cnt - 1]) * 1e3)
    b.profile_events(None, 0)
    kern_us = {n: float(np.mean(v)) for n, v in per_kernel.items() if v}
    dom = max(kern_us, key=kern_us.get)
    D0 = D[:prof_steps, 0]
    dom_bytes = float(np.mean([kernel_bytes(dom, T, k, d, S) for d in D0]))
    mfma_info = None
    if mfma:
        f8, f16 = mfma_flops(dom, T, k, S)
        t_dom = kern_us[dom] * 1e-6
        # the launch's bounding roof: its bytes at the HBM peak or its MFMA work
        # at the dense peaks (routed at the MXFP8 rate -- a FP4 x FP8 MFMA runs at
        # the FP8 rate -- or the FP4 rate on the FP4 x FP4 path, shared at bf16),
        # whichever is longer
        routed_peak = FP4_MFMA_PEAK_TFLOPS if fp4_act else FP8_MFMA_PEAK_TFLOPS
        t_bound = max(dom_bytes / (HBM_PEAK_GBS * 1e9),
                      f8 / (routed_peak * 1e12) + f16 / (BF16_MFMA_PEAK_TFLOPS * 1e12))
        name = "fp4xfp4_tflops" if fp4_act else "fp4xfp8_tflops"
        mfma_info = {"kernel": dom, name: round(f8 / t_dom / 1e12, 1),
                     "frac_of_fp8_peak": round(f8 / t_dom / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4),
                     "frac_of_fp4_peak": round(f8 / t_dom / 1e12 / FP4_MFMA_PEAK_TFLOPS, 4),
                     "bf16_tflops_same_launch": round(f16 / t_dom / 1e12, 1),
                     "bounding_roof_us": round(t_bound * 1e6, 1),
                     "frac_of_bounding_roof": round(t_bound / t_dom, 4)}
    achieved = dom_bytes / (kern_us[dom] * 1e-6) / 1e9

    traffic = pmc_traffic(dom, args.config)

    # the box's practical HBM ceiling: a plain 1 GiB device-to-device copy
    # (read + write bytes over its time), outside the timed region
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = round(5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
    del src, dst

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {
        "metric": "tokens/s & expert-weight HBM GB/s, K3-shape MXFP4 MoE layer (b=1/64/4096)",
        "value": round(T / (ms_per_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_run,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4*mxfp4->f32" if fp4_act else "mxfp4*mxfp8->f32" if mfma
                  else "mxfp4*bf16->f32"),
        "data": "synthetic (seeded; codes uniform, E8M0 118..126, N(0,0.02) bf16 router/shared, N(0,1) tokens"
                + ((", logit bias N(0,0.5)" + (f", +20 on experts 0..{cfgd['favor'] - 1}"
                                                  if cfgd.get("favor") else "") + ")")
                   if cfgd.get("bias") else ")"),
        "config": {"workload": cfgd["desc"], "tokens_per_step": T, "layers": n_layers,
                   "resident_copies": len(layers), "path": cfgd.get("path", "gemv")},
        "expert_weight_gbs": round(float(exp_gbs), 1),
        "expert_weight_hbm_frac": round(float(exp_gbs) / HBM_PEAK_GBS, 4),
        "distinct_experts_mean": round(float(D.mean()), 2),
        "kernel_us": {n: round(v, 2) for n, v in kern_us.items()},
        "layer_span_us_events": round(float(np.mean(span)), 2),
        "layer_span_us_median": round(float(np.median(span)), 2),
        "layer_span_us_iqr": [round(float(np.percentile(span, 25)), 2),
                              round(float(np.percentile(span, 75)), 2)],
        # median span per resident copy of the layer (step i runs copy i mod copies):
        # identical bytes at different addresses
        "layer_span_us_by_copy": ([round(float(np.median(span[(c - args.warmup) % len(layers)::len(layers)])), 2)
                                   for c in range(len(layers))]
                                  if n_layers == 1 and len(layers) > 1 and len(span) >= 2 * len(layers)
                                  else None),
        "hbm_copy_gbs": copy_gbs,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": round(dom_bytes),
                     "us_events": round(kern_us[dom], 2)},
    }
    rp = rocprof_us(dom, args.config)
    if rp is not None:  # the same launch in the committed rocprofv3 summary (its own timing)
        out["roofline"]["us_rocprof"] = rp
        out["roofline"]["frac_rocprof"] = round(dom_bytes / (rp * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    if mfma_info is not None:
        out["mfma"] = mfma_info
    if pool is not None:
        copied, resident = (a - c for a, c in zip(pool.stats(), pool_before))
        h2d = copied * REC_BYTES / args.steps
        out["stream"] = {
            "pool_slots": cfgd["pool_slots"],
            "records_copied_per_step": round(copied / args.steps, 2),
            "hit_rate": round(resident / max(copied + resident, 1), 4),
            "h2d_bytes_per_step": round(h2d),
            "h2d_gbs": round(h2d / (ms_per_step * 1e-3) / 1e9, 2),
            "pcie_peak_gbs": PCIE_PEAK_GBS,
            "copies_at_pcie_peak_us": round(h2d / (PCIE_PEAK_GBS * 1e9) * 1e6, 1),
            "note": "value includes the host-to-device copies; kernel_us and roofline are the "
                    "same kernels timed on the resident layer"}
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.config, args.cpu_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
