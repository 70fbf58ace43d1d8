"""Helpers for the GPU parity tests: seeded operands, device upload, NaN-poisoned
outputs, the call through the C ABI binding and the comparison with the oracle.

Tolerance: every element must satisfy |gpu - ref| <= 1e-2 * (1 + |ref|), where
ref is the fp64 oracle on the exact values of the same 16-bit inputs.
"""
import numpy as np

import oracle
from convolution_nhwc_amd import api, synth

TOL = 1e-2
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


def torch():
    import torch as t
    return t


def to_device(bits):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def poisoned(shape, dtype):
    t = torch()
    return t.full(shape, NAN_BITS[dtype] - (1 << 16) if NAN_BITS[dtype] >= 1 << 15 else NAN_BITS[dtype],
                  dtype=t.int16, device="cuda")


def from_device(x, dtype):
    bits = x.cpu().numpy().view(np.uint16)
    return synth.bits_to_f64(bits, dtype)


def operands(p, op, seed, exact=False):
    """(act_bits, act_f64, w_bits, w_f64) for problem p and pass op."""
    ho, wo = oracle.out_dims(p)
    act_shape = (p["n"], p["h"], p["w"], p["c"]) if op == "fwd" else (p["n"], ho, wo, p["k"])
    w_shape = (p["k"], p["r"], p["s"], p["c"] // p["groups"])
    if exact:
        rng = synth.generator(seed)
        a = synth.draw(rng, act_shape, ("ints", (-1.0, 0.0, 1.0)))
        w = synth.draw(rng, w_shape, ("ints", (-1.0, 0.0, 1.0)))
        (ab, af), (wb, wf) = synth.round_to(a, p["dtype"]), synth.round_to(w, p["dtype"])
    else:
        fan = p["c"] // p["groups"] * p["r"] * p["s"] if op == "fwd" else p["k"] // p["groups"] * p["r"] * p["s"]
        (ab, af), (wb, wf) = synth.operands(seed, act_shape, w_shape, p["dtype"], w_fan_in=fan)
    return ab, af, wb, wf


def run_gpu(p, op, act_bits, w_bits):
    """Run pass op through the C ABI on poisoned outputs; returns the output as f64."""
    t = torch()
    ho, wo = api.cnhwc_out_dims(p)
    a = to_device(act_bits)
    w = to_device(w_bits)
    if op == "fwd":
        out = poisoned((p["n"], ho, wo, p["k"]), p["dtype"])
        need = api.cnhwc_workspace_size(p, api.OP_FWD)
        ws = t.full((max(need, 16) // 4,), float("nan"), dtype=t.float32, device="cuda")
        api.cnhwc_fwd(p, a.data_ptr(), w.data_ptr(), out.data_ptr(), ws.data_ptr(), need,
                      t.cuda.current_stream().cuda_stream)
    else:
        out = poisoned((p["n"], p["h"], p["w"], p["c"]), p["dtype"])
        need = api.cnhwc_workspace_size(p, api.OP_DGRAD)
        ws = t.full((max(need, 16) // 4,), float("nan"), dtype=t.float32, device="cuda")
        api.cnhwc_dgrad(p, a.data_ptr(), w.data_ptr(), out.data_ptr(), ws.data_ptr() if need else None,
                        need, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return out


def reference(p, op, act_f64, w_f64):
    return oracle.conv_fwd(act_f64, w_f64, p) if op == "fwd" else oracle.conv_dgrad(act_f64, w_f64, p)


def check_close(got, ref, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: %d non-finite outputs (unwritten?)" % (what, int(np.sum(~np.isfinite(got))))
    err = np.abs(got - ref)
    bound = TOL * (1.0 + np.abs(ref))
    bad = err > bound
    assert not bad.any(), "%s: %d of %d outside tolerance, max err %.3g at %s (got %r want %r)" % (
        what, int(bad.sum()), bad.size, float(err.max()), np.unravel_index(np.argmax(err - bound), err.shape),
        float(got.flat[np.argmax(err - bound)]), float(ref.flat[np.argmax(err - bound)]))
    return float(err.max())


def parity(p, op, seed, exact=False):
    """Full-tensor parity of one problem; returns (max_err, gpu_bits_tensor)."""
    ab, af, wb, wf = operands(p, op, seed, exact)
    out = run_gpu(p, op, ab, wb)
    got = from_device(out, p["dtype"])
    ref = reference(p, op, af, wf)
    if exact:
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), "exact mode: %d mismatches" % int(np.sum(got != ref))
        return 0.0, out
    return check_close(got, ref, str(p)), out


def run_wgrad(p, xb, yb):
    """Weight gradient through the C ABI on a NaN-poisoned dw and a NaN-filled
    workspace."""
    t = torch()
    x, dy = to_device(xb), to_device(yb)
    dw = poisoned((p["k"], p["r"], p["s"], p["c"] // p["groups"]), p["dtype"])
    need = api.cnhwc_workspace_size(p, api.OP_WGRAD)
    ws = t.full((max(need, 16) // 4,), float("nan"), dtype=t.float32, device="cuda")
    api.cnhwc_wgrad(p, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), ws.data_ptr() if need else None,
                    need, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    return dw


def workload_operands(name):
    """The named workload's seeded operands exactly as the benchmark draws them:
    (problem, op, (act_bits, act_f64), (second_bits, second_f64))."""
    wl = synth.WORKLOADS[name]
    p, op = wl["prob"], wl["op"]
    ho, wo = oracle.out_dims(p)
    x_shape = (p["n"], p["h"], p["w"], p["c"])
    y_shape = (p["n"], ho, wo, p["k"])
    w_shape = (p["k"], p["r"], p["s"], p["c"] // p["groups"])
    if op == "wgrad":
        a, b = synth.wgrad_operands(wl["seed"], x_shape, y_shape, p["dtype"])
    else:
        kw = dict(w_dist=wl["w_dist"]) if wl.get("w_dist") else dict(w_fan_in=wl["fan_in"])
        a, b = synth.operands(wl["seed"], x_shape if op == "fwd" else y_shape, w_shape, p["dtype"], **kw)
    return p, op, a, b


def full_size_parity(name):
    """The named workload at its full size, in the launch configuration the
    benchmark times (automatic dispatch), compared with the oracle on every
    output element (every image, channel and filter tap); returns the output
    bits as a numpy uint16 array."""
    p, op, (ab, af), (bb, bf) = workload_operands(name)
    if op == "wgrad":
        out = run_wgrad(p, ab, bb)
        ref = oracle.conv_wgrad(af, bf, p)
    else:
        out = run_gpu(p, op, ab, bb)
        ref = reference(p, op, af, bf)
    bits = out.cpu().numpy().view(np.uint16)
    check_close(synth.bits_to_f64(bits, p["dtype"]), ref, name)
    return bits
