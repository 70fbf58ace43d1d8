"""GPU parity of the plain fallback kernels (one output per lane) against the
fp64 oracle, through the C ABI.

The dispatcher sends dense problems here when a channel count per group is not
a multiple of 8 (a 3-channel stem, 12 -> 20 channels, 4 channels a group) or
the stride exceeds the implicit-GEMM class table (stride 5).  Each case checks
that the automatic plan is the plain kernel, then compares every element with
the oracle; a forced-variant block runs the same kernels on dense shapes the
tuned kernels also take, so the two can be compared bit for bit on exact
inputs.
"""
import numpy as np
import pytest

from convolution_nhwc_amd import api

from gpu_util import operands, parity, run_gpu

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=stride, pad_h=pad_h, pad_w=pad_w,
                groups=groups, dtype=dtype)


def ident(p):
    return "n{n}h{h}w{w}c{c}k{k}r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}{dtype}".format(**p)


STEM = P(2, 32, 30, 3, 64, 7, 7, 2, 3, 3)                    # RGB stem, 7x7 stride 2
DGRAD_AUTO = [
    STEM,
    dict(STEM, dtype="bf16"),
    P(2, 11, 13, 12, 20, 3, 3, 1, 1, 1),                     # 12 -> 20 channels
    P(1, 10, 9, 12, 20, 3, 3, 1, 1, 1, dtype="bf16"),
    P(1, 16, 16, 8, 8, 5, 5, 5, 2, 2),                       # stride 5
    P(1, 23, 21, 16, 24, 3, 3, 5, 0, 1),                     # stride 5, taps miss most pixels
    P(2, 14, 14, 32, 32, 3, 3, 2, 1, 1, groups=8),           # 4 channels a group, stride 2
    P(1, 9, 12, 12, 24, 2, 3, 3, 1, 0, groups=3),            # ragged grouped, even filter rows
]
FWD_AUTO = [
    STEM,
    dict(STEM, dtype="bf16"),
    P(2, 11, 13, 12, 20, 3, 3, 1, 1, 1),
    P(1, 10, 9, 12, 20, 3, 3, 1, 1, 1, dtype="bf16"),
    P(1, 13, 15, 20, 12, 5, 3, 1, 2, 1),                     # non-square, per-axis pad
    P(1, 9, 12, 12, 24, 2, 3, 3, 1, 0, groups=3),
]


@pytest.mark.parametrize("p", DGRAD_AUTO, ids=ident)
def test_dispatched_generic_dgrad_parity(p):
    assert api.cnhwc_plan(p, api.OP_DGRAD)[1] == api.VAR_DGRAD_GENERIC
    parity(p, "dgrad", 501)


@pytest.mark.parametrize("p", FWD_AUTO, ids=ident)
def test_dispatched_generic_fwd_parity(p):
    assert api.cnhwc_plan(p, api.OP_FWD)[1] == api.VAR_FWD_GENERIC
    parity(p, "fwd", 502)


DENSE = [
    P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1),
    P(1, 15, 13, 64, 32, 3, 3, 2, 1, 1, dtype="bf16"),
    P(2, 10, 10, 64, 64, 3, 3, 1, 1, 1, groups=8),
    P(1, 12, 14, 32, 32, 5, 3, 1, 2, 1, groups=32),          # depthwise, non-square
]


@pytest.mark.parametrize("p", DENSE, ids=ident)
def test_forced_generic_parity_on_dense_shapes(p):
    with api.override(variant=api.VAR_DGRAD_GENERIC):
        parity(p, "dgrad", 503)
    with api.override(variant=api.VAR_FWD_GENERIC):
        parity(p, "fwd", 504)


@pytest.mark.parametrize("p", DENSE[:3], ids=ident)
def test_generic_matches_tuned_kernels_on_exact_inputs(p):
    """Inputs in {-1, 0, 1}: every partial sum is exact, so the plain kernels
    and the dispatcher's tuned kernels agree bit for bit."""
    for op in ("dgrad", "fwd"):
        ab, _, wb, _ = operands(p, op, 505, exact=True)
        tuned = run_gpu(p, op, ab, wb).cpu().numpy()
        with api.override(variant=api.VAR_DGRAD_GENERIC if op == "dgrad" else api.VAR_FWD_GENERIC):
            plain = run_gpu(p, op, ab, wb).cpu().numpy()
        assert np.array_equal(tuned, plain), op
        parity(p, op, 505, exact=True)


def test_generic_chunked_equals_unchunked():
    p = P(5, 9, 9, 12, 20, 3, 3, 1, 1, 1)
    ab, _, wb, _ = operands(p, "dgrad", 506)
    whole = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(chunk_limit_bytes=2 * 9 * 9 * 20 * 2):
        assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [2, 2, 1]
        parts = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(whole, parts)
