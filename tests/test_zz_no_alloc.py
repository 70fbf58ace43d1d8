"""GPU test of cnhwc_fwd_static_ws, the forward entry point that allocates
nothing: its workspace is the library's static device array.

Through the C ABI it must give the same bits as cnhwc_fwd with a
caller-allocated workspace (same dispatcher, kernels and split order), and
stay within the oracle's tolerance, on consecutive calls that share the array:
the split-C workload (12.8 MB of fp32 partial sums), then smaller problems on
the same leftover contents, among them the implicit-GEMM forward (its
transformed filter lives in the workspace) and one that needs no workspace.
After the first call on the device (whose look-up of the array loads the code
object holding it), the device's free memory must not change across a call.
"""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth

from gpu_util import check_close, from_device, poisoned, run_gpu, to_device, torch, workload_operands

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="bf16"):
    return synth.problem(n, h, w, c, k, r, s, stride, pad_h, pad_w, groups, dtype)


def static_fwd(p, xb, wb, check_mem=True):
    t = torch()
    ho, wo = api.cnhwc_out_dims(p)
    x, w = to_device(xb), to_device(wb)
    y = poisoned((p["n"], ho, wo, p["k"]), p["dtype"])
    t.cuda.synchronize()
    free0 = t.cuda.mem_get_info()[0]
    api.cnhwc_fwd_static_ws(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    if check_mem:
        assert t.cuda.mem_get_info()[0] == free0, "device memory changed across the call"
    return y


def compare(p, xb, xf, wb, wf, what, check_mem=True):
    need = api.cnhwc_workspace_size(p, api.OP_FWD)
    assert need <= api.STATIC_WS_BYTES
    ref_bits = run_gpu(p, "fwd", xb, wb)           # cnhwc_fwd, caller-allocated workspace
    got = static_fwd(p, xb, wb, check_mem)
    assert np.array_equal(got.cpu().numpy(), ref_bits.cpu().numpy()), what
    check_close(from_device(got, p["dtype"]), oracle.conv_fwd(xf, wf, p), what)
    return need


def test_static_workspace_matches_caller_workspace_on_consecutive_calls():
    # first call: the split-C workload at full size
    p, op, (xb, xf), (wb, wf) = workload_operands("c4a_splitc_fwd")
    assert api.cnhwc_plan(p, api.OP_FWD)[1] == api.VAR_FWD_SPLITC
    # (the first call on the device looks the array up, which loads the code
    # object that holds it: device memory may change there, and only there)
    first = compare(p, xb, xf, wb, wf, "c4a_splitc_fwd", check_mem=False)
    assert first > 0
    # then smaller problems on the array's leftover contents
    smaller = [
        P(2, 7, 7, 512, 128, 3, 3, 1, 1, 1),                      # split-C, fewer partials
        P(1, 9, 9, 256, 64, 3, 3, 1, 1, 1, dtype="f16"),          # split-C, f16, 9x9
        P(2, 14, 14, 64, 256, 1, 1, dtype="f16"),                 # implicit-GEMM forward
        P(1, 12, 12, 64, 64, 3, 3, 1, 1, 1),                      # no workspace
    ]
    for i, q in enumerate(smaller):
        (xb, xf), (wb, wf) = synth.operands(700 + i, (q["n"], q["h"], q["w"], q["c"]),
                                            (q["k"], q["r"], q["s"], q["c"] // q["groups"]), q["dtype"],
                                            w_fan_in=q["c"] * q["r"] * q["s"])
        need = compare(q, xb, xf, wb, wf, "smaller problem %d" % i)
        assert need < first


def test_static_workspace_refuses_a_larger_workspace():
    p = synth.WORKLOADS["c4a_splitc_fwd"]["prob"]
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=64):
        assert api.cnhwc_workspace_size(p, api.OP_FWD) > api.STATIC_WS_BYTES
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_fwd_static_ws(p, 16, 32, 48, None)
    assert e.value.status == api.WORKSPACE_TOO_SMALL and "static workspace" in e.value.reason
