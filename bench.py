"""Benchmark of the fused "sum of partials + residual add + RMSNorm (+ fp8)" epilogue.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2]

One step is one call of the whole epilogue (sum, residual add, RMSNorm, optional fp8
epilogue) over one batch of the workload, with inputs already resident in HBM. The
default workload is the decode batch at hidden 4096 (P = 8 bf16 partials of
[80, 4096]). Buffer sets are rotated so that the inputs of a step are not left in the
256 MB last-level cache by the previous step (about 1 GiB of sets). The K timed steps
are captured as HIP graphs (launch overhead of the host excluded, as under graph
replay in serving) and bracketed by torch.cuda.synchronize().

Prints one JSON line with: throughput (algorithmic GB/s, the metric), tokens/s, a
roofline object for the fused kernel (algorithmic bytes per launch / average launch
time from HIP events on the launch stream, against 8 TB/s), the unfused PyTorch
sequence timed the same way, and the CPU oracle timed on a bounded sample of the same
workload.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30
CPU_SAMPLE_ELEMS = 1 << 23  # partial elements per oracle call in the CPU baseline


def kernel_sources_sha() -> str:
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "residual_add_rmsnorm_fp32_amd", "csrc", "*"))):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"far_vec_kernel_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_sources_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_sources_sha():
        return None
    return float(m_b.group(1))


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c2", help="c1..c5 (default c2: decode, hidden 4096)")
    ap.add_argument("--tokens", type=int, default=None, help="first T rows of the workload")
    ap.add_argument("--sets", type=int, default=None,
                    help="number of rotating input/output sets (default: enough for 1 GiB)")
    ap.add_argument("--eager", action="store_true", help="launch every step from the host")
    ap.add_argument("--no-rotate", action="store_true", help="one buffer set (cache-warm)")
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--plan", default=None, help="JSON launch plan to force")
    ap.add_argument("--quant", default=None, choices=["none", "static", "dynamic", "group", "tensor"],
                    help="override the workload's fp8 mode (the other forms of the op)")
    ap.add_argument("--no-residual", action="store_true", help="form without a residual input")
    ap.add_argument("--discard-residual", action="store_true", help="do not write the new residual")
    ap.add_argument("--no-copy", action="store_true", help="skip the device-copy ceiling")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of the step's byte count (for counters)")
    return ap.parse_args()


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures the kernel on one GPU; --gpus {args.gpus} is not supported "
              "(the cross-GPU exchange of partials is not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from residual_add_rmsnorm_fp32_amd import binding as B
    from residual_add_rmsnorm_fp32_amd import workloads as wk

    B.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = wk.WORKLOADS[args.workload]
    T = args.tokens or wl.T
    inp = wk.make_inputs(wl, T=T)
    P, H, dt = wl.P, wl.H, wl.dtype
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    quant = args.quant or wl.quant
    if quant == "static" and inp["scale"] is None:
        inp["scale"] = np.array([0.05], np.float32)
    with_norm = quant == "none"
    with_res = not args.no_residual
    with_res_out = not args.discard_residual
    algo_bytes = wk.algorithmic_bytes(P, T, H, 2, quant, with_norm, with_res, with_res_out)
    plan = json.loads(args.plan) if args.plan else None

    def dev_codes(c):
        return torch.from_numpy(np.ascontiguousarray(c).view(np.int16)).view(tdt).to(dev)

    base = {
        "partials": dev_codes(inp["partials"]),      # [P, T, H]
        "residual": dev_codes(inp["residual"]),
        "gamma": dev_codes(inp["gamma"]),
        "scale": (torch.from_numpy(inp["scale"]).to(dev) if inp["scale"] is not None else None),
    }
    n_sets = 1 if args.no_rotate else max(1, min(512, -(-ROTATE_BYTES // algo_bytes)))
    if args.sets:
        n_sets = args.sets

    n_scales = {"dynamic": T, "group": T * -(-H // B.FAR_FP8_GROUP), "tensor": 1}.get(quant, 0)
    ws_bytes = B.far_workspace_bytes(T, H, quant)

    def make_set():
        s = {"partials": base["partials"].clone(),
             "residual": base["residual"].clone() if with_res else None,
             "gamma": base["gamma"], "scale": base["scale"],
             "residual_out": torch.empty(T, H, dtype=tdt, device=dev) if with_res_out else None,
             "norm_out": torch.empty(T, H, dtype=tdt, device=dev) if with_norm else None,
             "quant_out": torch.empty(T, H, dtype=torch.uint8, device=dev) if quant != "none" else None,
             "scale_out": torch.empty(n_scales, dtype=torch.float32, device=dev) if n_scales else None,
             "workspace": torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None}
        return s

    sets = [make_set() for _ in range(n_sets)]
    shape = f"[{T},{H}]"

    def fused(s):
        B.far_fused_add_rmsnorm(s["partials"], s["residual"], s["gamma"], wl.eps, wl.weight_bias,
                                quant, s["scale"], s["norm_out"], s["residual_out"], s["quant_out"],
                                s["scale_out"], plan=plan, workspace=s["workspace"])

    def unfused(s):
        acc = s["partials"].float().sum(0)
        if s["residual"] is not None:
            acc = acc + s["residual"].float()
        new_res = acc.to(tdt)
        x = new_res.float()
        r = torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + wl.eps)
        y = x * r * (wl.weight_bias + s["gamma"].float())
        if quant == "none":
            return y.to(tdt), new_res
        if quant == "static":
            return (y / s["scale"]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn), new_res
        if quant == "group":
            yg = y.view(T, -1, B.FAR_FP8_GROUP) if H % B.FAR_FP8_GROUP == 0 else y.view(T, 1, H)
            amax = yg.abs().amax(-1, keepdim=True)
        elif quant == "tensor":
            amax = y.abs().amax()
            yg = y
        else:
            amax = y.abs().amax(-1, keepdim=True)
            yg = y
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
        return (yg / sc).clamp(-448.0, 448.0).to(torch.float8_e4m3fn), new_res, sc

    def time_steps(step_fn, K, W, eager, sets=sets):
        n_sets = len(sets)
        stream = torch.cuda.current_stream()
        for i in range(W):
            step_fn(sets[i % n_sets])
        torch.cuda.synchronize()
        graphs = []
        if not eager:
            # whole rotations, about 256 launches per graph, so the per-replay cost of a
            # graph is spread over many launches
            per_graph = min(K, n_sets * max(1, 256 // n_sets))
            full, rem = divmod(K, per_graph)
            def capture(n):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n):
                        step_fn(sets[i % n_sets])
                return g
            g_full = capture(per_graph) if full else None
            g_rem = capture(rem) if rem else None
            if g_full:
                g_full.replay()
            torch.cuda.synchronize()
            graphs = [g_full] * full + ([g_rem] if g_rem else [])
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        if eager:
            for i in range(K):
                step_fn(sets[i % n_sets])
        else:
            for g in graphs:
                g.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, start.elapsed_time(stop) / 1e3

    K, W = args.steps, args.warmup
    wall, ev = time_steps(fused, K, W, args.eager)
    ms_per_step = wall / K * 1e3
    launch_s = ev / K
    achieved = algo_bytes / launch_s / 1e9
    value = algo_bytes * K / wall / 1e9

    result = {
        "metric": "fused add+RMSNorm(+fp8) achieved HBM GB/s and % of peak; tokens/s at hidden=4096",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {wl.description}" + (f" (first {T} tokens)" if T != wl.T else "")
                        + (f" [quant {quant}]" if quant != wl.quant else "")
                        + (" [no residual input]" if not with_res else "")
                        + (" [new residual not written]" if not with_res_out else ""),
            "num_partials": P, "tokens": T, "hidden": H, "storage": dt, "quant": quant,
            "eps": wl.eps, "weight_bias": wl.weight_bias,
            "outputs": ("norm_out" if with_norm else "quant_out") + ("+new_residual" if with_res_out else "")
                       + ("+scale_out" if n_scales else ""),
            "residual_input": with_res,
            "launch": "eager" if args.eager else "hipGraph replay",
            "buffer_sets": n_sets, "plan": B.far_plan(T, H, P, tdt, quant) if plan is None else plan,
        },
        "tokens_per_s": round(T * K / wall, 1),
        "algorithmic_bytes_per_step": algo_bytes,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(wl.name if (T == wl.T and quant == wl.quant and with_res
                                                and with_res_out) else f"{wl.name}_other"),
            "avg_launch_us": round(launch_s * 1e6, 3),
            "kernel": ("far_vec_kernel" if B.far_plan(T, H, P, tdt, quant)["variant"] == "vector" else "far_generic_kernel")
                      + (" + far_tensor_scale_kernel + far_tensor_quant_kernel" if quant == "tensor" else ""),
        },
    }

    if not args.no_unfused:
        wall_u, ev_u = time_steps(unfused, max(K // 4, 1), W, args.eager)
        ku = max(K // 4, 1)
        result["unfused_torch"] = {
            "ms_per_step": round(wall_u / ku * 1e3, 6),
            "gbs_same_bytes": round(algo_bytes * ku / wall_u / 1e9, 2),
            "fused_speedup": round((wall_u / ku) / (wall / K), 3),
        }

    if not args.no_copy:
        # streaming ceiling: torch's device copy moving the same bytes (reads B/2 and
        # writes B/2), rotated over the same amount of memory and timed the same way
        half = algo_bytes // 2
        n_copy = max(1, min(512, -(-ROTATE_BYTES // algo_bytes))) if not args.no_rotate else 1
        del sets[1:]
        torch.cuda.empty_cache()
        pairs = [(torch.empty(half, dtype=torch.uint8, device=dev),
                  torch.empty(half, dtype=torch.uint8, device=dev)) for _ in range(n_copy)]
        for a_, b_ in pairs:
            a_.fill_(1)
        wall_c, ev_c = time_steps(lambda pr: pr[1].copy_(pr[0]), K, W, args.eager, sets=pairs)
        copy_gbs = 2 * half * K / ev_c / 1e9
        result["copy_ceiling"] = {
            "kind": "torch device copy of half the algorithmic bytes (same bytes moved)",
            "gbs": round(copy_gbs, 2),
            "fused_over_copy": round(achieved / copy_gbs, 4),
        }
        del pairs
        torch.cuda.empty_cache()

    if args.copy_calibration:
        src = torch.empty(algo_bytes // 2, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes_read"] = src.numel()

    if not args.no_cpu:
        from oracle import far_oracle as orc

        # a bounded sample: the first rows of the batch, about 2^23 partial elements per
        # call (the whole batch for the decode workloads)
        sample_rows = max(1, min(T, CPU_SAMPLE_ELEMS // (P * H)))
        parts = inp["partials"][:, :sample_rows]
        res = inp["residual"][:sample_rows] if with_res else None
        sample_bytes = wk.algorithmic_bytes(P, sample_rows, H, 2, quant, with_norm, with_res,
                                            with_res_out)
        calls = 0
        t0 = time.perf_counter()
        qid = {"none": 0, "static": 1, "dynamic": 2, "group": 3, "tensor": 4}[quant]
        while True:
            orc.fused_add_rmsnorm(parts, res, inp["gamma"], dt, wl.eps, wl.weight_bias,
                                  quant_mode=qid, scale=inp["scale"])
            calls += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        what = (f"the whole {shape} batch" if sample_rows == T
                else f"the first {sample_rows} of the {T} tokens of the {shape} batch")
        result["cpu_baseline"] = {
            "value": round(sample_bytes * calls / el / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{calls} calls on {what} (P={P}) through the numpy float64 oracle, "
                      f"{el:.1f} s, one host thread",
        }

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
