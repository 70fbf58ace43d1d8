#!/usr/bin/env python3
"""Benchmark of the gfx950 NHWC convolution library on one MI355X.

One step = one pass of the headline workload (the pointwise 1x1 dgrad,
N=32, H=W=56, K=256 -> C=64, fp16) through the C ABI, on inputs already
resident in HBM.  Steps rotate over enough copies of the operands that the
256 MB Infinity Cache cannot serve a step from the previous one.  HIP events
on the launch stream bracket exactly K steps after W warm-up steps; before
those, each workload first runs back to back for 60 ms (settle_ms), since the
GPU clock reaches its sustained value only after about 50 ms of load (a
3x3 dgrad timed from idle reads ~8 % slow, a 7x7 depthwise one ~13 %).

The JSON line also carries, per seeded workload of the method (forward, dgrad
and weight-gradient shapes), the measured time and its fraction of the binding MI355X roof
(HBM 8 TB/s, dense fp16/bf16 MFMA 2.5 PFLOP/s, fp32 vector 157.3 TFLOP/s), and
the fp64 CPU oracle timed on a bounded sample of the headline workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-shapes]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0      # dense fp16 / bf16
VALU_PEAK_TFLOPS = 157.3       # fp32 vector (two FMAs per lane per cycle)
HEADLINE = "c2_pointwise"
ROTATE_BYTES = 1 << 30         # >= 4x the Infinity Cache
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per launch read from rocprofv3 FETCH_SIZE / WRITE_SIZE counters,
# keyed by workload, with a hash of the kernel sources they were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", default=None, help="time one workload only (for profiling)")
    ap.add_argument("--no-shapes", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (scales the HBM byte counters)")
    ap.add_argument("--source-hash", nargs="+", metavar="FILE",
                    help="print the hash recorded with counter-based traffic for these sources")
    return ap.parse_args()


def metrics(name):
    """Algorithmic bytes, nominal and valid flops, and the binding roof of a workload.

    Every pass reads two of x, dY, W and writes the third once, and performs
    the same multiply-adds: the formulas hold for forward, dgrad and wgrad."""
    from convolution_nhwc_amd import synth
    wl = synth.WORKLOADS[name]
    p = wl["prob"]
    ho = (p["h"] + 2 * p["pad_h"] - p["r"]) // p["stride"] + 1
    wo = (p["w"] + 2 * p["pad_w"] - p["s"]) // p["stride"] + 1
    cg = p["c"] // p["groups"]
    act = p["n"] * p["h"] * p["w"] * p["c"] * 2
    res = p["n"] * ho * wo * p["k"] * 2
    wbytes = p["k"] * p["r"] * p["s"] * cg * 2
    alg_bytes = act + res + wbytes
    nominal = 2.0 * p["n"] * ho * wo * p["k"] * cg * p["r"] * p["s"]
    # valid flops: only taps that land inside the image
    def taps(size, out, pad, f, s):
        o = np.arange(out)[:, None] * s - pad + np.arange(f)[None, :]
        return ((o >= 0) & (o < size)).sum()
    valid = 2.0 * p["n"] * p["k"] * cg * taps(p["h"], ho, p["pad_h"], p["r"], p["stride"]) * \
        taps(p["w"], wo, p["pad_w"], p["s"], p["stride"])
    depthwise = p["groups"] == p["c"] == p["k"]
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_cmp = valid / ((VALU_PEAK_TFLOPS if depthwise else MFMA_PEAK_TFLOPS) * 1e12)
    bound = "hbm" if t_hbm >= t_cmp else ("alu" if depthwise else "mfma")
    return dict(bytes=alg_bytes, nominal_flops=nominal, valid_flops=valid, bound=bound,
                t_ideal_s=max(t_hbm, t_cmp))


def source_hash(paths):
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch from the committed counter runs, or None when there
    is no record or the kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            ent = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not ent:
        return None
    try:
        if source_hash(ent["sources"]) != ent["sources_sha256"]:
            return None
    except OSError:
        return None
    return ent["hbm_bytes_per_launch"]


class Workload:
    """Device operands of a seeded workload, replicated for cache rotation."""

    def __init__(self, name):
        import torch
        from convolution_nhwc_amd import api, synth
        self.name = name
        wl = synth.WORKLOADS[name]
        self.p = p = wl["prob"]
        self.op = wl["op"]
        ho, wo = api.cnhwc_out_dims(p)
        cg = p["c"] // p["groups"]
        x_shape, y_shape = (p["n"], p["h"], p["w"], p["c"]), (p["n"], ho, wo, p["k"])
        w_shape = (p["k"], p["r"], p["s"], cg)
        dev = "cuda"
        if self.op == "wgrad":
            # both operands are activations (x, dY) and rotate; the output is dW
            (ab, _), (bb, _) = synth.wgrad_operands(wl["seed"], x_shape, y_shape, p["dtype"])
            out_shape = w_shape
        else:
            act_shape = x_shape if self.op == "fwd" else y_shape
            out_shape = y_shape if self.op == "fwd" else x_shape
            (ab, _), (bb, _) = synth.operands(wl["seed"], act_shape, w_shape,
                                              p["dtype"], act_dist=("uniform", -1.0, 1.0),
                                              w_dist=wl.get("w_dist"), w_fan_in=wl["fan_in"])
        a0 = torch.from_numpy(ab.view(np.int16)).to(dev)
        b0 = torch.from_numpy(bb.view(np.int16)).to(dev)
        opc = {"fwd": api.OP_FWD, "dgrad": api.OP_DGRAD, "wgrad": api.OP_WGRAD}[self.op]
        self.opc = opc
        self.kernel, self.variant = api.cnhwc_plan(p, opc)
        self.ws_bytes = api.cnhwc_workspace_size(p, opc)
        rot_b = self.op == "wgrad"
        per_set = a0.numel() * 2 + (b0.numel() * 2 if rot_b else 0) + \
            int(np.prod(out_shape)) * 2 + self.ws_bytes
        nsets = int(max(1, min(64, -(-ROTATE_BYTES // per_set))))
        self.acts = [a0] + [a0.clone() for _ in range(nsets - 1)]
        self.bs = [b0] + [b0.clone() if rot_b else b0 for _ in range(nsets - 1)]
        self.outs = [torch.empty(out_shape, dtype=torch.int16, device=dev) for _ in range(nsets)]
        self.wss = [torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
                    for _ in range(nsets)]
        self.nsets = nsets
        self.stream = torch.cuda.current_stream().cuda_stream
        self.api = api
        self.i = 0

    def step(self):
        j = self.i % self.nsets
        self.i += 1
        f = {"fwd": self.api.cnhwc_fwd, "dgrad": self.api.cnhwc_dgrad,
             "wgrad": self.api.cnhwc_wgrad}[self.op]
        f(self.p, self.acts[j].data_ptr(), self.bs[j].data_ptr(), self.outs[j].data_ptr(),
          self.wss[j].data_ptr(), self.ws_bytes, self.stream)


SETTLE_S = 0.06


def settle(wk, seconds=SETTLE_S):
    """Run steps back to back for `seconds` of host time so the GPU clock is
    at its sustained value before warm-up and timing."""
    import torch
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(100):
            wk.step()
        torch.cuda.synchronize()


def time_steps(wk, steps, warmup):
    import torch
    settle(wk)
    for _ in range(warmup):
        wk.step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        wk.step()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per step


def cpu_baseline():
    """The fp64 oracle, untuned, on the headline workload, repeated for ~10 s."""
    import oracle
    from convolution_nhwc_amd import synth
    wl = synth.WORKLOADS[HEADLINE]
    p = wl["prob"]
    ho, wo = oracle.out_dims(p)
    (_, af), (_, wf) = synth.operands(wl["seed"], (p["n"], ho, wo, p["k"]),
                                      (p["k"], p["r"], p["s"], p["c"]), p["dtype"],
                                      w_fan_in=wl["fan_in"])
    oracle.conv_dgrad(af[:1], wf, dict(p, n=1))  # load / warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.conv_dgrad(af, wf, p)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0:
            break
    sec = el / reps
    full = metrics(HEADLINE)
    return {"value": round(full["bytes"] / sec / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "fp64 nested-loop oracle on the whole headline workload (32 images), "
                      "%d runs in %.1f s, %.3f s per run" % (reps, el, sec)}


def cpl_matrix(args):
    """The row-streaming depthwise dgrad kernel at every channels-per-lane
    count on the depthwise workloads (forced through the test override),
    beside the dispatcher's own pick; a refused count carries its reason."""
    import torch
    from convolution_nhwc_amd import api, synth
    out = []
    for name in ("c5_dw3x3", "c5_dw7x7", "c5_dw7x7_s2"):
        ent = {"workload": name}
        ent["dispatch"] = api.cnhwc_plan(synth.WORKLOADS[name]["prob"], api.OP_DGRAD)[0]
        for cpl in (1, 2, 4, 8):
            key = "cpl%d" % cpl
            try:
                with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=cpl):
                    wk = Workload(name)
                    t = time_steps(wk, max(10, args.steps // 4), 3)
                mm = metrics(name)
                ent[key] = {"us": round(t * 1e3, 2), "GB/s": round(mm["bytes"] / (t * 1e-3) / 1e9, 1)}
                del wk
                torch.cuda.empty_cache()
            except api.CnhwcError as e:
                ent[key] = {"refused": e.reason[:160]}
        out.append(ent)
        print("# cpl %s" % json.dumps(ent), file=sys.stderr, flush=True)
    return out


def copy_calibration():
    """A plain device copy of 1 GiB, to scale the HBM byte counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": 3}))


def main():
    args = parse()
    if args.source_hash:
        print(source_hash(args.source_hash))
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each image is independent; see the design notes on sharding over N).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    from convolution_nhwc_amd import api, synth
    api.lib()

    names = [args.only] if args.only else [HEADLINE]
    head = Workload(names[0])
    ms = time_steps(head, args.steps, args.warmup)
    m = metrics(head.name)
    gbs = m["bytes"] / (ms * 1e-3) / 1e9
    tflops = m["nominal_flops"] / (ms * 1e-3) / 1e12
    if m["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    elif m["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 3), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4)}
    else:
        vt = m["valid_flops"] / (ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": round(vt, 3), "peak": VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(vt / VALU_PEAK_TFLOPS, 4)}
    roof["traffic"] = recorded_traffic(head.name)
    roof["algorithmic_bytes"] = int(m["bytes"])
    line = {
        "metric": "effective conv TFLOP/s and HBM GB/s per shape, % of MI355X roofline",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": int(SETTLE_S * 1000), "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head.p["dtype"], "data": "synthetic",
        "config": {"workload": head.name, "op": head.op, "kernel": head.kernel,
                   **{k: head.p[k] for k in ("n", "h", "w", "c", "k", "r", "s", "stride",
                                             "pad_h", "pad_w", "groups")}},
        "effective_tflops": round(tflops, 3),
        "roofline": roof,
    }
    del head
    torch.cuda.empty_cache()
    if not args.no_shapes and not args.only:
        shapes = []
        for name in synth.WORKLOADS:
            if name == "c1_pointwise_tiny":
                continue
            try:
                wk = Workload(name)
                t = time_steps(wk, max(10, args.steps // 2), max(3, args.warmup // 2))
                mm = metrics(name)
                ent = {"workload": name, "op": wk.op, "kernel": wk.kernel, "dtype": wk.p["dtype"],
                       "ms": round(t, 5), "GB/s": round(mm["bytes"] / (t * 1e-3) / 1e9, 1),
                       "TFLOP/s": round(mm["nominal_flops"] / (t * 1e-3) / 1e12, 2),
                       "bound": mm["bound"], "roofline_frac": round(mm["t_ideal_s"] / (t * 1e-3), 4)}
                if mm["bound"] == "hbm":
                    ent["frac_of_peak"] = round(mm["bytes"] / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                elif mm["bound"] == "mfma":
                    ent["frac_of_peak"] = round(mm["nominal_flops"] / (t * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4)
                else:
                    ent["frac_of_peak"] = round(mm["valid_flops"] / (t * 1e-3) / 1e12 / VALU_PEAK_TFLOPS, 4)
                del wk
                torch.cuda.empty_cache()
            except Exception as e:  # a workload whose kernel is not available yet
                ent = {"workload": name, "error": str(e)[:200]}
            shapes.append(ent)
            print("# %s" % json.dumps(ent), file=sys.stderr, flush=True)
        line["shapes"] = shapes
        line["cpl_matrix"] = cpl_matrix(args)
    if not args.no_cpu_baseline and not args.only:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
