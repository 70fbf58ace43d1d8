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

Every operand rotates (activations, filter, output, workspace).

The JSON line also carries, per seeded workload of the method (forward, dgrad
and weight-gradient shapes), the measured time and its fraction of the binding
MI355X roof (HBM 8 TB/s, dense fp16/bf16 MFMA 2.5 PFLOP/s, fp32 vector
157.3 TFLOP/s) and of the same roof as measured on this GPU by the ceiling
microbenchmarks (libcnhwc_ceiling.so: HBM streams at the workload's
read:write share, MFMA and dot2 issue at their best occupancy), the HBM bytes
per launch from the committed rocprofv3 counter runs where the kernel source
still matches them, and the fp64 CPU oracle on the headline workload (whole
batch on every host thread, ~10 s of repeats; one thread on two images).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-shapes]
                    [--no-ceilings] [--ceilings-only] [--no-cpu-baseline]
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
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="back-to-back run before each workload's warm-up (GPU clock settling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured machine ceilings (fractions against the spec peaks only)")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="only measure and print the machine ceilings")
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
        # every operand rotates (activations, filter or second activation,
        # output, workspace), so no step finds its inputs in the Infinity Cache
        per_set = a0.numel() * 2 + b0.numel() * 2 + int(np.prod(out_shape)) * 2 + self.ws_bytes
        nsets = int(max(1, min(64, -(-ROTATE_BYTES // per_set))))
        self.acts = [a0] + [a0.clone() for _ in range(nsets - 1)]
        self.bs = [b0] + [b0.clone() for _ in range(nsets - 1)]
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


def settle(wk, seconds=None):
    """Run steps back to back for `seconds` of host time so the GPU clock is
    at its sustained value before warm-up and timing."""
    import torch
    seconds = SETTLE_S if seconds is None else seconds
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_runs(fn, budget_s, min_runs=3):
    """Run fn repeatedly for about budget_s; per-run wall times."""
    times, t_all = [], time.perf_counter()
    while len(times) < min_runs or time.perf_counter() - t_all < budget_s:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return times


def cpu_baseline():
    """The fp64 oracle, untuned, on the headline workload: the whole batch on
    every host thread OpenMP gives it (about 10 s of repeats), then one thread
    on a two-image sample (about 5 s), each reported as median and min."""
    import oracle
    from convolution_nhwc_amd import synth
    wl = synth.WORKLOADS[HEADLINE]
    p = wl["prob"]
    ho, wo = oracle.out_dims(p)
    (_, af), (_, wf) = synth.operands(wl["seed"], (p["n"], ho, wo, p["k"]),
                                      (p["k"], p["r"], p["s"], p["c"]), p["dtype"],
                                      w_fan_in=wl["fan_in"])
    oracle.conv_dgrad(af[:1], wf, dict(p, n=1))  # load / warm
    full_bytes = metrics(HEADLINE)["bytes"]
    threads = oracle.num_threads()
    multi = sorted(_time_runs(lambda: oracle.conv_dgrad(af, wf, p), 10.0))
    med = multi[len(multi) // 2]
    one_n = 2
    oracle.set_num_threads(1)
    try:
        single = sorted(_time_runs(lambda: oracle.conv_dgrad(af[:one_n], wf, dict(p, n=one_n)), 5.0))
    finally:
        oracle.set_num_threads(threads)
    smed = single[len(single) // 2]
    scale = one_n / p["n"]
    return {"value": round(full_bytes / med / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "fp64 nested-loop oracle on the whole headline workload (%d images), %d runs, "
                      "median %.4f s, min %.4f s per run" % (p["n"], len(multi), med, multi[0]),
            "median_s": round(med, 5), "min_s": round(multi[0], 5),
            "best_GB/s": round(full_bytes / multi[0] / 1e9, 4),
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(full_bytes * scale / smed / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": "%d of the %d images, %d runs" % (one_n, p["n"], len(single)),
                              "median_s": round(smed, 5), "min_s": round(single[0], 5)}}


# ---- measured machine ceilings -------------------------------------------------

CEILING_LIB = os.path.join(ROOT, "convolution_nhwc_amd", "libcnhwc_ceiling.so")


def _ceiling_lib():
    import ctypes
    if not os.path.exists(CEILING_LIB):
        raise RuntimeError("libcnhwc_ceiling.so is not built (%s); run "
                           "`python -m convolution_nhwc_amd.build`" % CEILING_LIB)
    L = ctypes.CDLL(CEILING_LIB)
    vp = ctypes.c_void_p
    L.ceiling_stream.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int64, ctypes.c_int, vp, vp]
    L.ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    L.ceiling_dot2.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    L.ceiling_lds.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    L.ceiling_empty.argtypes = [ctypes.c_int, vp]
    for f in (L.ceiling_stream, L.ceiling_mfma, L.ceiling_dot2, L.ceiling_lds, L.ceiling_empty):
        f.restype = ctypes.c_int
    return L


def _event_time_ms(launch, reps, settle_s=None):
    """Mean ms per launch over `reps` back-to-back launches, after the clock
    has settled under the same load."""
    import torch
    settle_s = SETTLE_S if settle_s is None else settle_s
    t0 = time.time()
    while time.time() - t0 < settle_s:
        for _ in range(10):
            launch()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        launch()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def ceilings():
    """What one MI355X delivers under the convolution kernels' kinds of load
    (libcnhwc_ceiling.so): HBM streams with R reads to one write and a
    read-only stream (best of three grid sizes), MFMA 16x16x32 f16 and dot2
    issue at 1, 2 and 4 waves per SIMD, LDS read bandwidth at 1, 2 and 4
    blocks of 4 waves a CU, and the back-to-back cost of an empty launch."""
    import torch
    L = _ceiling_lib()
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(16, dtype=torch.float32, device="cuda")
    out = {}
    chunk = 512 << 20
    bufs = [torch.empty(chunk, dtype=torch.uint8, device="cuda") for _ in range(5)]
    for b in bufs:
        b.fill_(1)
    n16 = chunk // 16
    ptr = [b.data_ptr() for b in bufs]
    stream = {}
    for reads in (0, 1, 2, 3, 4):
        if reads == 0:
            # read-only: the first four chunks' worth as one 2 GiB stream
            big = torch.empty(4 * chunk, dtype=torch.uint8, device="cuda")
            big.fill_(1)
            nb, args, moved = 4 * n16, (big.data_ptr(), 0, 0, 0, 0), 4 * chunk
        else:
            big = None
            nb, args, moved = n16, tuple(ptr[:reads]) + (0,) * (4 - reads) + (ptr[4],), (reads + 1) * chunk
        best = 0.0
        for blocks in (1024, 2048, 4096):
            def launch(a=args, nb=nb, blocks=blocks, reads=reads):
                rc = L.ceiling_stream(reads, *a, nb, blocks, sink.data_ptr(), st)
                if rc:
                    raise RuntimeError("ceiling_stream failed: %d" % rc)
            ms = _event_time_ms(launch, 10)
            best = max(best, moved / (ms * 1e-3) / 1e9)
        del big
        stream[reads] = round(best, 1)
    out["hbm_GBs"] = {"read_only": stream[0], "1r:1w": stream[1], "2r:1w": stream[2],
                      "3r:1w": stream[3], "4r:1w": stream[4]}
    del bufs
    torch.cuda.empty_cache()
    mf = {}
    iters = 2000
    for wps in (1, 2, 4):
        blocks = 256 * wps
        ms = _event_time_ms(lambda: L.ceiling_mfma(blocks, iters, sink.data_ptr(), st), 5)
        mf["%d_wave_per_simd" % wps] = round(blocks * 4 * iters * 8 * 16384 / (ms * 1e-3) / 1e12, 1)
    out["mfma_f16_TFLOPs"] = mf
    d2 = {}
    for wps in (1, 2, 4, 8):
        blocks = 256 * wps
        ms = _event_time_ms(lambda: L.ceiling_dot2(blocks, iters, sink.data_ptr(), st), 5)
        d2["%d_wave_per_simd" % wps] = round(blocks * 256 * iters * 8 * 4 / (ms * 1e-3) / 1e12, 1)
    out["dot2_TFLOPs"] = d2
    lds = {}
    for bpc in (1, 2, 4):
        blocks = 256 * bpc
        ms = _event_time_ms(lambda: L.ceiling_lds(blocks, iters, sink.data_ptr(), st), 5)
        gbs = blocks * 256 * iters * 8 * 16 / (ms * 1e-3) / 1e9
        lds["%d_block_per_cu" % bpc] = {"GB/s_per_CU": round(gbs / 256, 1),
                                         "B/clk_per_CU_at_2.4GHz": round(gbs / 256 / 2.4, 1)}
    out["lds_read"] = lds
    em = {}
    for blocks in (256, 1024):
        ms = _event_time_ms(lambda: L.ceiling_empty(blocks, st), 200)
        em["%d_blocks" % blocks] = round(ms * 1e3, 3)
    out["empty_launch_us"] = em
    return out


def hbm_ceiling_for(name, ceil):
    """Measured HBM ceiling at a workload's read share: piecewise linear in
    the read fraction between the measured streams (1:1, 2:1, 3:1, 4:1 reads
    to writes and read-only)."""
    from convolution_nhwc_amd import synth
    wl = synth.WORKLOADS[name]
    p = wl["prob"]
    ho = (p["h"] + 2 * p["pad_h"] - p["r"]) // p["stride"] + 1
    wo = (p["w"] + 2 * p["pad_w"] - p["s"]) // p["stride"] + 1
    act = p["n"] * p["h"] * p["w"] * p["c"] * 2
    res = p["n"] * ho * wo * p["k"] * 2
    wb = p["k"] * p["r"] * p["s"] * (p["c"] // p["groups"]) * 2
    written = {"fwd": res, "dgrad": act, "wgrad": wb}[wl["op"]]
    f = 1.0 - written / float(act + res + wb)
    pts = [(0.5, ceil["1r:1w"]), (2 / 3, ceil["2r:1w"]), (0.75, ceil["3r:1w"]), (0.8, ceil["4r:1w"]),
           (1.0, ceil["read_only"])]
    if f <= pts[0][0]:
        return pts[0][1]
    for (f0, v0), (f1, v1) in zip(pts, pts[1:]):
        if f <= f1:
            return v0 + (v1 - v0) * (f - f0) / (f1 - f0)
    return pts[-1][1]


def measured_ceiling(name, mm, ceil):
    """The measured ceiling of a workload's binding roof: HBM GB/s at its read
    share, or the best MFMA / dot2 TFLOP/s over the waves-per-SIMD counts."""
    if ceil is None:
        return None
    if mm["bound"] == "hbm":
        return round(hbm_ceiling_for(name, ceil["hbm_GBs"]), 1)
    if mm["bound"] == "mfma":
        return max(ceil["mfma_f16_TFLOPs"].values())
    return max(ceil["dot2_TFLOPs"].values())


def frac_of_ceiling(name, mm, t_s, ceil):
    """Achieved rate over the measured ceiling of the workload's binding roof
    (bytes for HBM, nominal flops for MFMA, valid flops for the vector ALUs)."""
    c = measured_ceiling(name, mm, ceil)
    if c is None:
        return None
    if mm["bound"] == "hbm":
        return round(mm["bytes"] / t_s / 1e9 / c, 4)
    if mm["bound"] == "mfma":
        return round(mm["nominal_flops"] / t_s / 1e12 / c, 4)
    return round(mm["valid_flops"] / t_s / 1e12 / c, 4)


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
    global SETTLE_S
    SETTLE_S = args.settle_ms / 1000.0
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
    if args.ceilings_only:
        print(json.dumps({"ceilings": ceilings()}), flush=True)
        return
    from convolution_nhwc_amd import api, synth
    api.lib()
    ceil = None if (args.no_ceilings or args.only) else ceilings()
    if ceil is not None:
        print("# ceilings %s" % json.dumps(ceil), file=sys.stderr, flush=True)

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
    if ceil is not None:
        roof["frac_of_measured_ceiling"] = frac_of_ceiling(head.name, m, ms * 1e-3, ceil)
        roof["measured_ceiling"] = measured_ceiling(head.name, m, ceil)
    line = {
        "metric": "effective conv TFLOP/s and HBM GB/s per shape, % of MI355X roofline",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": round(SETTLE_S * 1000, 1), "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": head.p["dtype"], "data": "synthetic",
        "config": {"workload": head.name, "op": head.op, "kernel": head.kernel,
                   **{k: head.p[k] for k in ("n", "h", "w", "c", "k", "r", "s", "stride",
                                             "pad_h", "pad_w", "groups")}},
        "effective_tflops": round(tflops, 3),
        "roofline": roof,
    }
    if ceil is not None:
        line["ceilings"] = ceil
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
                ent["frac_of_measured_ceiling"] = frac_of_ceiling(name, mm, t * 1e-3, ceil)
                ent["traffic"] = recorded_traffic(name)
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
