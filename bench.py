"""Benchmark of the MoE layer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic tokens:
moe_route -> moe_dispatch -> moe_expert_mlp -> moe_combine, each a C-ABI call
on one HIP stream, inputs and weights resident in HBM before timing starts.

Prints one JSON line.  `value` is whole-layer tokens/s (tokens per step /
step time).  The per-stage figures the metric names are reported beside it:
dispatch+combine tokens/s and HBM GB/s against the 8 TB/s peak, and the
expert GEMM's TFLOP/s against the 2.5 PFLOP/s dense bf16 MFMA peak.  The
`roofline` object is for the expert MLP (the dominant kernel pair), timed with
HIP events recorded on its own stream around every call inside the timed
region; its bound follows from the MLP's flops per algorithmic byte against
the ridge point (MFMA-bound above it, HBM-bound below, as the weight-streaming
decode shape is).  `cpu_baseline` is the fp64 CPU oracle timed on a bounded sample of
the same workload's tokens.

Usage: python bench.py [--gpus 1] [--steps 30] [--warmup 5] [--workload dsv3_prefill_ep]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

_ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, _ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
FP32_VALU_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(_ROOT, "profiles", "expert_mlp_dsv3_prefill_ep_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="dsv3_prefill_ep")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the graph-replay timing of the whole layer")
    p.add_argument("--no-cold", action="store_true",
                   help="skip the cold-cache dispatch/combine timing")
    p.add_argument("--no-mxfp8", action="store_true",
                   help="skip the block-scaled (MX-FP8 payload and gate/up) layer timing")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--write-traffic-record", metavar="DIR", default=None,
                   help="no GPU work: read the rocprofv3 counter CSVs under DIR (pmc_FETCH_SIZE, "
                        "pmc_WRITE_SIZE, pmc_copy_FETCH_SIZE, pmc_copy_WRITE_SIZE) and write the "
                        "expert-MLP HBM traffic record for the current kernel source")
    p.add_argument("--packed-weights", action="store_true",
                   help="expert weights in the packed layout (moe_pack_weights, "
                        "MOE_WEIGHTS_PACKED); the block-scaled leg is skipped")
    p.add_argument("--dbo", action="store_true",
                   help="only time the two-microbatch forward (moe_forward_dbo, compute + comm "
                        "streams) against the unsplit moe_forward on the same tokens")
    p.add_argument("--no-dbo", action="store_true",
                   help="skip the dual-microbatch leg of the default line")
    p.add_argument("--no-probes", action="store_true",
                   help="skip the achievable-peak probes (streaming copy, MFMA loops)")
    p.add_argument("--tokens", type=int, default=0,
                   help="override the workload's token count (ad-hoc measurements)")
    p.add_argument("--shared-beside-combine", action="store_true",
                   help="run the shared experts beside the combine (MOE_SHARED_BESIDE_COMBINE)")
    return p.parse_args()


def dbo_timings(args, layer, torch) -> dict:
    """Whole-layer time of moe_forward_dbo on two streams, on one stream, and of
    the unsplit moe_forward, on the same tokens (same outputs)."""
    compute, comm = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(compute)
        for _ in range(args.steps):
            fn()
        ev1.record(compute)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps

    unsplit = timed(lambda: layer.forward(stream=compute))
    ref = layer.out.clone()
    split = timed(lambda: layer.forward_dbo(compute=compute, comm=comm))
    torch.cuda.synchronize()
    same = bool(torch.equal(layer.out.view(torch.int16), ref.view(torch.int16)))
    one_stream = timed(lambda: layer.forward_dbo(compute=compute, comm=compute))
    graph_ms = None
    if not args.no_graph:
        g = layer.capture_forward(dbo=True)
        graph_ms = timed(lambda: g.launch(compute))
        g.destroy()
    return {"unsplit_ms": unsplit, "split_two_streams_ms": split,
            "split_one_stream_ms": one_stream, "overlap_gain": unsplit / split - 1.0,
            "bitwise_equal_to_unsplit": same, "split_graph_replay_ms": graph_ms}


def dbo_leg(args, layer, torch) -> dict:
    """The dual-microbatch workload (8192 tokens of the DeepSeek-V3-shaped share,
    split at the midpoint into two 4096-token microbatches) on the same device
    weights as the main workload."""
    from combine_router_softmax_top_amd import binding as B
    from combine_router_softmax_top_amd import workloads as W
    from combine_router_softmax_top_amd.layer import MoELayer
    cfg5 = W.CONFIGS["dsv3_dual_microbatch"]
    layer5 = MoELayer(cfg5, {"x": W.make_tokens(cfg5, seed=0)}, share_weights=layer)
    r = dbo_timings(args, layer5, torch)
    T = cfg5.num_tokens
    mid = B.dbo_split_point(T)
    r.update({"workload": cfg5.name, "tokens": T, "microbatches": [mid, T - mid],
              "tokens_per_s_two_streams": T / (r["split_two_streams_ms"] * 1e-3),
              "tokens_per_s_unsplit": T / (r["unsplit_ms"] * 1e-3)})
    del layer5
    torch.cuda.empty_cache()
    return r


def bench_dbo(args, cfg, layer, torch) -> dict:
    """The --dbo line: moe_forward_dbo vs moe_forward on the chosen workload."""
    from combine_router_softmax_top_amd import binding as B
    r = dbo_timings(args, layer, torch)
    T = cfg.num_tokens
    return {"metric": "dual-microbatch layer tokens/s (moe_forward_dbo, two HIP streams)",
            "value": T / (r["split_two_streams_ms"] * 1e-3), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["split_two_streams_ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
            "data": "synthetic (seeded)",
            "config": {"workload": cfg.name, "tokens": T, "microbatches": [
                B.dbo_split_point(T), T - B.dbo_split_point(T)]}, **r}


def achievable_peaks(torch, stream) -> dict:
    """What plain streaming kernels and register-only MFMA loops reach on this
    GPU (include/moe_probe.h), next to the nominal peaks the roofline uses."""
    from combine_router_softmax_top_amd import binding as B
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    sink = torch.empty(16384 * 256, dtype=torch.int32, device="cuda")

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    res = {"how": "1 GiB, 16-byte accesses in contiguous 16-32 KB blocks per workgroup, the best "
                  "of 1024-16384 workgroups of 256; MFMA loops: 256 workgroups of 8 waves, 8 "
                  "independent register-only MFMAs per round"}
    grids = (1024, 2048, 4096, 8192, 16384)
    for key, kind, moved in [("copy", B.PROBE_COPY, 2 * n), ("read", B.PROBE_READ, n),
                             ("write", B.PROBE_WRITE, n)]:
        best, best_wg = 0.0, 0
        for g in grids:
            t = timed(lambda: B.probe_stream(kind, n, dst=b if kind != B.PROBE_READ else None,
                                             src=a if kind != B.PROBE_WRITE else None,
                                             sink=sink if kind == B.PROBE_READ else None,
                                             workgroups=g, stream=stream))
            if moved / t / 1e9 > best:
                best, best_wg = moved / t / 1e9, g
        res[f"{key}_GB_per_s"] = best  # copy: bytes read + bytes written
        res[f"{key}_workgroups"] = best_wg
    del a, b
    out = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    for kind, key, iters in [(B.PROBE_MFMA_BF16, "mfma_bf16_TFLOP_per_s", 4000),
                             (B.PROBE_MFMA_FP8, "mfma_fp8_TFLOP_per_s", 2000)]:
        t = timed(lambda: B.probe_mfma(kind, 256, iters, out, stream=stream))
        res[key] = B.probe_mfma_flops(kind, 256, iters) / t / 1e12
    res["nominal"] = {"hbm_GB_per_s": HBM_PEAK_GBS, "bf16_TFLOP_per_s": BF16_MFMA_PEAK_TFLOPS,
                      "fp8_TFLOP_per_s": FP8_MFMA_PEAK_TFLOPS}
    return res


def library_dense_gemm(torch, stream, cfg, n_loc: int) -> dict:
    """The vendor library's bf16 GEMM (torch.nn.functional.linear, i.e. hipBLASLt)
    on dense matrices with the M x N x K of this layer's two expert GEMMs: the
    rows (routed, plus T per shared expert) as one [M, d] matrix times the
    stacked gate and up weights [2I, d], and [M, I] times the down weights
    [d, I].  One dense product per pass, no expert grouping: a reference for
    the grouped kernels, same flops."""
    d, inter = cfg.hidden, cfg.intermediate
    rows = n_loc + cfg.num_shared * cfg.num_tokens
    g = torch.Generator(device="cuda").manual_seed(7)
    out = {}
    for key, (m, n, k) in (("gate_up", (rows, 2 * inter, d)), ("down", (rows, d, inter))):
        a = (torch.randn(m, k, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
        w = (torch.randn(n, k, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        with torch.cuda.stream(stream):
            for _ in range(3):
                y = torch.nn.functional.linear(a, w)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                y = torch.nn.functional.linear(a, w)
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 10 * 1e3
        out[f"{key}_us"] = us
        out[f"{key}_TFLOP_per_s"] = 2.0 * m * n * k / (us * 1e-6) / 1e12
        del a, w, y
    out["both_us"] = out["gate_up_us"] + out["down_us"]
    out["shapes"] = {"gate_up": [rows, 2 * inter, d], "down": [rows, d, inter]}
    return out


def source_digest() -> str:
    """Digest of the bf16 expert-MLP kernel's source code (its file and the
    shared grouped-GEMM header): // comments and blank lines are left out, so
    a change to the comments alone keeps a traffic record valid and any change
    to the code voids it."""
    import re
    csrc = os.path.join(_ROOT, "combine_router_softmax_top_amd", "csrc")
    code = []
    for name in ("expert_mlp.hip", "grouped_gemm.h"):
        with open(os.path.join(csrc, name)) as f:
            lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in f.read().splitlines()]
        code.append("\n".join(ln for ln in lines if ln.strip()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def algorithmic(cfg, n_loc: int, t_touch: int) -> dict:
    """Minimum HBM bytes / flops of each stage (per call)."""
    T, d, E, K, I, b = (cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k,
                        cfg.intermediate, cfg.elem_bytes)
    S = cfg.num_shared
    route = T * d * b + E * d * b + T * K * 8 + (E * 4 if cfg.zipf_s is not None else 0)
    dispatch = t_touch * d * b + n_loc * d * b + n_loc * 4 + 2 * T * K * 4 + 2 * E * 4
    combine = n_loc * d * b + T * K * 8 + T * d * b + S * T * d * b
    flops = 6.0 * n_loc * d * I + 6.0 * S * T * d * I
    # Expert MLP: every local and shared expert's three weight matrices read
    # once (every local expert is taken to have rows), the rows read (x),
    # h written and read back, y written.
    rows = n_loc + S * T
    e_loc = cfg.expert_end - cfg.expert_begin
    gemm_bytes = (e_loc + S) * 3 * I * d * b + rows * (2 * d + 2 * I) * b
    return dict(route=route, dispatch=dispatch, combine=combine, gemm_flops=flops,
                gemm_bytes=gemm_bytes)


def mlp_roofline(cfg, alg: dict, mlp_ms: float) -> tuple:
    """The expert MLP's `expert_gemm` and `roofline` objects for a measured
    stage time (ms): both rates from the algorithmic flops and bytes, and the
    bound from the arithmetic intensity against the ridge point of the
    roofline (peak flops over 8 TB/s) -- below it the stage is HBM-bound."""
    peak = BF16_MFMA_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_VALU_PEAK_TFLOPS
    tflops = alg["gemm_flops"] / (mlp_ms * 1e-3) / 1e12
    gbs = alg["gemm_bytes"] / (mlp_ms * 1e-3) / 1e9
    ai = alg["gemm_flops"] / alg["gemm_bytes"]
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    expert_gemm = {"TFLOP_per_s": tflops, "frac_mfma_peak": tflops / peak, "flops": alg["gemm_flops"],
                   "algorithmic_bytes": alg["gemm_bytes"], "GB_per_s": gbs, "flop_per_byte": ai,
                   "ridge_flop_per_byte": ridge}
    if ai >= ridge:
        roofline = {"bound": "mfma" if cfg.dtype == "bf16" else "alu", "achieved": tflops,
                    "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak}
    else:
        roofline = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS}
    return expert_gemm, roofline


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, target_s: float) -> dict:
    """The fp64 oracle's whole-layer forward (oracle.forward) on the first n
    tokens of the workload with every host thread, n grown to about 60 % of
    target_s; then the same on fewer tokens with one thread; then the oracle's
    stages one by one (route, dispatch, expert MLP, combine) on a quarter of
    the sample with every thread."""
    import oracle
    threads = oracle.num_threads()

    def sample(n):
        sub = cfg.with_tokens(n)
        sub_inp = dict(inp)
        sub_inp["x"] = inp["x"][:n].contiguous()
        return sub, sub_inp

    def grow(budget):
        n = 8
        while True:
            sub, sub_inp = sample(n)
            t0 = time.perf_counter()
            oracle.forward(sub, sub_inp)
            dt = time.perf_counter() - t0
            if dt >= budget * 0.5 or n >= cfg.num_tokens:
                return n, dt, sub, sub_inp
            n = min(cfg.num_tokens, max(n * 2, int(n * budget / max(dt, 1e-3))))

    n, dt, sub, sub_inp = grow(0.6 * target_s)
    reps = 1
    if dt < target_s * 0.3:
        # The whole workload is quick: repeat it until about the budget.
        reps = max(2, int(0.6 * target_s / max(dt, 1e-4)))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.forward(sub, sub_inp)
        dt = time.perf_counter() - t0
    what = f"first {n} of the {cfg.num_tokens} tokens" if n < cfg.num_tokens else \
        f"all {n} tokens" + (f", {reps} times" if reps > 1 else "")
    res = {"value": n * reps / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{what} of the same workload, whole layer (route, dispatch, expert MLP, "
                     f"combine) in fp64, {dt:.1f} s",
           "cpu_model": _cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}
    # one thread, about a fifth of the budget
    budget1 = 0.2 * target_s
    n1 = max(1, min(n, int(budget1 * (n * reps / dt) / threads)))
    sub1, inp1 = sample(n1)
    oracle.set_threads(1)
    try:
        reps1, dt1 = 0, 0.0
        while dt1 < 0.5 * budget1 or reps1 == 0:
            t0 = time.perf_counter()
            oracle.forward(sub1, inp1)
            dt1 += time.perf_counter() - t0
            reps1 += 1
    finally:
        oracle.set_threads(threads)
    res["one_thread"] = {"value": n1 * reps1 / dt1, "unit": "tokens/s",
                         "sample": f"first {n1} tokens, whole layer"
                                   + (f", {reps1} times" if reps1 > 1 else "") + f", {dt1:.1f} s"}
    # stages, every thread
    ns = max(1, n // 4)
    subs, inps = sample(ns)
    K, E = cfg.top_k, cfg.num_experts
    st = {}
    t0 = time.perf_counter()
    ids, w, _ = oracle.route(inps["x"], inps["w_router"], inps["bias"], K, cfg.score,
                             cfg.renormalize)
    t1 = time.perf_counter()
    d = oracle.dispatch(ids, E, cfg.expert_begin, cfg.expert_end, x=inps["x"])
    t2 = time.perf_counter()
    off = d["offsets"]
    row_expert = oracle_row_experts(off, cfg.num_local)
    y = oracle.expert_mlp(d["x_sorted"], row_expert, inps["w_gate"], inps["w_up"], inps["w_down"])
    ysh = None
    if cfg.num_shared:
        import torch
        ysh = torch.stack([oracle.expert_mlp(inps["x"], torch.full((ns,), s, dtype=torch.int32),
                                             inps["ws_gate"], inps["ws_up"], inps["ws_down"])
                           for s in range(cfg.num_shared)])
    t3 = time.perf_counter()
    padded = y.new_zeros(ns * K, y.shape[1])
    padded[:y.shape[0]] = y
    oracle.combine(padded, d["row_of"], w, ns, K, y_shared=ysh)
    t4 = time.perf_counter()
    res["stages_s"] = {"tokens": ns, "route": t1 - t0, "dispatch": t2 - t1,
                       "expert_mlp": t3 - t2, "combine": t4 - t3}
    return res


def oracle_row_experts(offsets, n_loc: int):
    """Local expert index of every dispatched row, from the expert offsets."""
    import torch
    n = int(offsets[n_loc])
    re = torch.empty(n, dtype=torch.int32)
    for j in range(n_loc):
        re[int(offsets[j]):int(offsets[j + 1])] = j
    return re


def write_traffic_record(d: str, out_path: str = TRAFFIC_FILE) -> dict:
    """HBM bytes per expert-MLP call from FETCH_SIZE / WRITE_SIZE counter runs.

    Each counter (KiB per dispatch, averaged over dispatches) is scaled by what
    the same counter reads for a plain device copy of 1 GiB (which reads and
    writes 1 GiB), so the result is in real bytes.
    """
    import csv
    import glob
    import re

    def per_kernel(sub):
        f = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter CSV under {os.path.join(d, sub)}")
        acc = {}
        for r in csv.DictReader(open(f[0])):
            m = re.search(r"(\w+_kernel(<[^>]*>)?|__amd_rocclr_copyBuffer)", r["Kernel_Name"])
            if m:
                acc.setdefault(m.group(1), []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fetch, write = per_kernel("pmc_FETCH_SIZE"), per_kernel("pmc_WRITE_SIZE")
    copy_kib = float(1 << 20)
    ff = copy_kib / per_kernel("pmc_copy_FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    fw = copy_kib / per_kernel("pmc_copy_WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    g1 = (fetch["gemm_bf16_kernel<1>"] * ff + write["gemm_bf16_kernel<1>"] * fw) * 1024
    g0 = (fetch["gemm_bf16_kernel<0>"] * ff + write["gemm_bf16_kernel<0>"] * fw) * 1024
    rec = {"workload": "dsv3_prefill_ep", "source_digest": source_digest(),
           "hbm_bytes_per_launch": g1 + g0, "gate_up_bytes": g1, "down_bytes": g0,
           "fetch_factor": ff, "write_factor": fw,
           "per_kernel_hbm_mb": {k: {"read": fetch[k] * ff * 1024 / 1e6,
                                     "write": write.get(k, 0.0) * fw * 1024 / 1e6}
                                 for k in fetch if k != "__amd_rocclr_copyBuffer"},
           "note": "FETCH_SIZE/WRITE_SIZE per dispatch of the two expert-MLP kernels, "
                   "scaled by a 1 GiB device copy"}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def main():
    args = parse()
    if args.write_traffic_record:
        print(json.dumps(write_traffic_record(args.write_traffic_record)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_router_softmax_top_amd import binding as B
    from combine_router_softmax_top_amd import workloads as W
    from combine_router_softmax_top_amd.layer import MoELayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    cfg = W.CONFIGS[args.workload]
    if args.packed_weights:
        cfg = cfg.replace(packed_weights=True)
    if args.tokens:
        cfg = cfg.with_tokens(args.tokens)
    if args.shared_beside_combine:
        cfg = cfg.replace(shared_beside_combine=True)
    t_gen = time.perf_counter()
    inp = W.make_inputs(cfg, seed=0)
    t_gen = time.perf_counter() - t_gen
    layer = MoELayer(cfg, inp, device="cuda:0")
    if args.dbo:
        print(json.dumps(bench_dbo(args, cfg, layer, torch)), flush=True)
        return
    stream = torch.cuda.Stream()

    def step(evs=None):
        with torch.cuda.stream(stream):
            if evs is not None:
                evs[0].record(stream)
            layer.route(stream, with_logits=False)
            if evs is not None:
                evs[1].record(stream)
            layer.dispatch(stream)
            if evs is not None:
                evs[2].record(stream)
            layer.expert_mlp(stream)
            if evs is not None:
                evs[3].record(stream)
            layer.combine(stream)
            if evs is not None:
                evs[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_loc = layer.n_rows()
    ids = layer.topk_ids
    local = (ids >= cfg.expert_begin) & (ids < cfg.expert_end)
    t_touch = int(local.any(1).sum())
    alg = algorithmic(cfg, n_loc, t_touch)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage = {"route": 0.0, "dispatch": 0.0, "expert_mlp": 0.0, "combine": 0.0}
    names = list(stage)
    for ev in events:
        for j, nm in enumerate(names):
            stage[nm] += ev[j].elapsed_time(ev[j + 1]) / args.steps  # ms
    ms_per_step = wall * 1e3 / args.steps
    T = cfg.num_tokens

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    dc_ms = stage["dispatch"] + stage["combine"]
    dc_bytes = alg["dispatch"] + alg["combine"]
    bf16 = cfg.dtype == "bf16"
    gemm_tflops = alg["gemm_flops"] / (stage["expert_mlp"] * 1e-3) / 1e12
    expert_gemm, roofline = mlp_roofline(cfg, alg, stage["expert_mlp"])
    traffic = None
    if os.path.exists(TRAFFIC_FILE) and not cfg.packed_weights:  # counted on row-major weights
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_digest") == source_digest() and rec.get("workload") == cfg.name:
            traffic = rec.get("hbm_bytes_per_launch")
    result = {
        "metric": "dispatch+combine tokens/s & HBM GB/s (% peak); expert GEMM % MFMA peak",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s (whole layer step)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) expert weights, random router)",
        "config": {"workload": cfg.name, "tokens": T, "hidden": cfg.hidden,
                   "experts": cfg.num_experts,
                   "local_experts": f"{cfg.expert_begin}-{cfg.expert_end - 1}",
                   "top_k": cfg.top_k, "intermediate": cfg.intermediate,
                   "shared_experts": cfg.num_shared, "local_rows": n_loc,
                   "tokens_touching_local_experts": t_touch, "parallelism": "none (1 GPU)",
                   "weights": "packed" if cfg.packed_weights else "row-major"},
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
        "dispatch_combine": {
            "tokens_per_s": T / (dc_ms * 1e-3),
            "GB_per_s": gbs(dc_bytes, dc_ms),
            "frac_hbm_peak": gbs(dc_bytes, dc_ms) / HBM_PEAK_GBS,
            "dispatch_GB_per_s": gbs(alg["dispatch"], stage["dispatch"]),
            "combine_GB_per_s": gbs(alg["combine"], stage["combine"]),
            "algorithmic_bytes": dc_bytes},
        "route": {"GB_per_s": gbs(alg["route"], stage["route"]),
                  "frac_hbm_peak": gbs(alg["route"], stage["route"]) / HBM_PEAK_GBS,
                  "algorithmic_bytes": alg["route"]},
        "expert_gemm": expert_gemm,
        "roofline": roofline,
        "input_generation_s": round(t_gen, 1),
    }
    result["roofline"].update({"traffic": traffic,
                               "kernel": "moe_expert_mlp (gate/up SiLU GEMM + down GEMM)",
                               "avg_launch_us": stage["expert_mlp"] * 1e3})
    if not args.no_graph:
        result["graph_replay"] = graph_replay(args, layer, stream, torch)
    if not args.no_cold:
        cold = cold_dispatch_combine(layer, stream, torch, alg)
        w = cold_dispatch_combine(layer, stream, torch, alg, evict="write")
        cold["evicted_by_writing"] = {k: w[k] for k in ("dispatch_us", "combine_us", "frac_hbm_peak")}
        result["dispatch_combine_cold"] = cold
    if not args.no_mxfp8 and not cfg.packed_weights and cfg.dtype == "bf16" and cfg.num_shared == 0 and cfg.hidden % 512 == 0:
        result["mxfp8"] = mxfp8_leg(args, layer, stream, torch, alg, n_loc, t_touch)
    if not args.no_dbo and cfg.name == "dsv3_prefill_ep" and not cfg.packed_weights:
        result["dbo"] = dbo_leg(args, layer, torch)
    if not args.no_probes:
        peaks = achievable_peaks(torch, stream)
        peaks["expert_gemm_frac_of_mfma_loop"] = (
            gemm_tflops / peaks["mfma_bf16_TFLOP_per_s"] if bf16 else None)
        if bf16 and n_loc > 0:
            lib = library_dense_gemm(torch, stream, cfg, n_loc)
            lib["expert_mlp_us"] = stage["expert_mlp"] * 1e3
            peaks["library_dense_gemm_bf16"] = lib
        peaks["dispatch_combine_frac_of_copy"] = gbs(dc_bytes, dc_ms) / peaks["copy_GB_per_s"]
        result["achievable_peaks"] = peaks
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def mxfp8_leg(args, layer, stream, torch, alg, n_loc: int, t_touch: int) -> dict:
    """The same step with the block-scaled payload: route, moe_dispatch_mxfp8
    (MX-FP8 rows), moe_expert_mlp_mxfp8 (fp8 gate/up; the down projection in
    fp8 too when I is a multiple of 512, else in bf16), combine, on the same
    tokens and the same (encoded) weights, timed the same way."""
    from combine_router_softmax_top_amd import binding as B
    cfg = layer.cfg
    T, K, d, I, E = cfg.num_tokens, cfg.top_k, cfg.hidden, cfg.intermediate, cfg.num_experts
    ref = layer.out.clone()
    fp8_down = I % 512 == 0
    mx = layer.quantize_weights(down=fp8_down)
    xq = torch.empty(T * K, d, dtype=torch.uint8, device=layer.device)
    xs = torch.empty(T * K * d // 32, dtype=torch.uint8, device=layer.device)

    def step(evs=None):
        with torch.cuda.stream(stream):
            if evs is not None:
                evs[0].record(stream)
            layer.route(stream, with_logits=False)
            if evs is not None:
                evs[1].record(stream)
            B.moe_dispatch_mxfp8(layer.cs, layer.x, layer.topk_ids, layer.counts, layer.offsets,
                                 xq, xs, layer.src_index, layer.row_of, layer.ws_dispatch, stream)
            if evs is not None:
                evs[2].record(stream)
            B.moe_expert_mlp_mxfp8(layer.cs, xq, xs, layer.offsets, mx["wq_gate"],
                                   mx["wq_gate_scales"], mx["wq_up"], mx["wq_up_scales"],
                                   None if fp8_down else layer.w_down, layer.y_sorted,
                                   layer.ws_mlp, stream, wq_down=mx.get("wq_down"),
                                   wq_down_scales=mx.get("wq_down_scales"))
            if evs is not None:
                evs[3].record(stream)
            layer.combine(stream)
            if evs is not None:
                evs[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ["route", "dispatch", "expert_mlp", "combine"]
    stage = {nm: sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / args.steps
             for j, nm in enumerate(names)}
    ms = wall * 1e3 / args.steps
    # Algorithmic bytes of the block-scaled dispatch: bf16 token rows read once,
    # codes and scales written per local row, the maps as in the bf16 dispatch.
    disp = t_touch * d * 2 + n_loc * (d + d // 32) + n_loc * 4 + 2 * T * K * 4 + 2 * E * 4
    dc_ms = stage["dispatch"] + stage["combine"]
    dc = disp + alg["combine"]
    mlp_tf = alg["gemm_flops"] / (stage["expert_mlp"] * 1e-3) / 1e12
    out = layer.out.float()
    rel = float((out - ref.float()).norm() / ref.float().norm())
    return {
        "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms,
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
        "dispatch_GB_per_s": disp / (stage["dispatch"] * 1e-3) / 1e9,
        "dispatch_combine": {"tokens_per_s": T / (dc_ms * 1e-3),
                             "GB_per_s": dc / (dc_ms * 1e-3) / 1e9,
                             "frac_hbm_peak": dc / (dc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "algorithmic_bytes": dc},
        "expert_mlp_TFLOP_per_s": mlp_tf,
        "down_projection": "fp8" if fp8_down else "bf16",
        "expert_mlp_note": "gate/up on the fp8 scaled MFMA (dense peak 5.0 PFLOP/s); down on the "
                           + ("fp8 scaled MFMA with h encoded in the gate/up epilogue"
                              if fp8_down else "bf16 MFMA (2.5)")
                           + "; per-kernel split in the rocprofv3 summary",
        "rel_l2_vs_bf16_layer": rel}


def cold_dispatch_combine(layer, stream, torch, alg, iters: int = 10, evict: str = "read") -> dict:
    """Dispatch and combine with cold caches: right before each of them 1 GiB
    of an unrelated buffer is read (evict="read"), which replaces what L2 and
    the 256 MB Infinity Cache hold with clean lines, so the stage's reads come
    from HBM (the layer's own sequence leaves part of y_sorted in the cache).
    evict="write" fills the buffer instead: that leaves the caches full of
    dirty lines, whose write-back to HBM then runs during the stage."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    flush.fill_(1)
    sink = torch.empty((), dtype=torch.int64, device="cuda")

    def evict_caches(i):
        if evict == "read":
            torch.sum(flush.view(torch.int32), dim=0, out=sink)
        else:
            flush.fill_(i & 255)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(iters)]
    with torch.cuda.stream(stream):
        for i in range(iters):
            evict_caches(i)
            ev[i][0].record(stream)
            layer.dispatch(stream)
            ev[i][1].record(stream)
            layer.expert_mlp(stream)
            evict_caches(i + 1)
            ev[i][2].record(stream)
            layer.combine(stream)
            ev[i][3].record(stream)
    torch.cuda.synchronize()
    d = sum(e[0].elapsed_time(e[1]) for e in ev) / iters
    c = sum(e[2].elapsed_time(e[3]) for e in ev) / iters
    nbytes = alg["dispatch"] + alg["combine"]
    gbs = nbytes / ((d + c) * 1e-3) / 1e9
    del flush
    how = ("1 GiB of another buffer read before each stage (L2 and Infinity Cache refilled with "
           "clean lines), HIP events" if evict == "read" else
           "1 GiB written before each stage (caches left holding dirty lines), HIP events")
    return {"dispatch_us": d * 1e3, "combine_us": c * 1e3, "GB_per_s": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "how": how}


def graph_replay(args, layer, stream, torch) -> dict:
    """The whole layer (moe_forward) captured once as a HIP graph and replayed
    back to back on one stream: the step without per-launch host work."""
    g = layer.capture_forward()
    for _ in range(max(args.warmup, 1)):
        g.launch(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        g.launch(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    g.destroy()
    ms = e0.elapsed_time(e1) / args.steps
    return {"ms_per_step": ms, "tokens_per_s": layer.cfg.num_tokens / (ms * 1e-3),
            "how": "moe_graph_capture_forward once, moe_graph_launch per step, HIP events"}


if __name__ == "__main__":
    main()
