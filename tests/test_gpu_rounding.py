"""Bit-exact pin of the single round-to-nearest-even rounding of every output,
on every kernel path, through the C ABI.

Inputs are integers (exact in fp16 / bf16) sized so that every product and
every partial sum is an integer below 2^24: the fp32 accumulators then hold the
exact result whatever the summation order, tiling or split.  The outputs are
large enough that most are NOT representable in the 16-bit type (integers
above 2048 for fp16, above 256 for bf16), so each must be rounded exactly once,
to nearest with ties to even.  The GPU bits must therefore equal the oracle's
exact fp64 result rounded once by the test's own RNE (``synth.round_to``).  A
truncating or round-half-away conversion, or a second rounding of partial sums
(a split-C, split-K or wgrad partial stored in 16 bits), changes some outputs;
each case also checks that its outputs include ties and values between the
grid points, so the comparison can see those mistakes.

The target statement's tolerance bounds an output's error; the pages' fast
path claims results equal to the general path ("perf(rocke/conv): add the
pointwise fast path dgrad was missing", Test Result: identical relative
error), which needs a fixed, single rounding.  fp16 overflow is not reached.
"""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth

from gpu_util import run_gpu, run_wgrad

pytestmark = pytest.mark.gpu

TARGET_STD = {"f16": 6000.0, "bf16": 3000.0}   # output spread, above the exact-integer range
MAX_INPUT = {"f16": 2048, "bf16": 256}          # integers exact in the storage type


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return synth.problem(n, h, w, c, k, r, s, stride, pad_h, pad_w, groups, dtype)


def reduction_length(p, op):
    ho, wo = oracle.out_dims(p)
    cg, kg = p["c"] // p["groups"], p["k"] // p["groups"]
    if op == "fwd":
        return cg * p["r"] * p["s"]
    if op == "dgrad":
        return kg * (-(-p["r"] // p["stride"])) * (-(-p["s"] // p["stride"]))
    return p["n"] * ho * wo


def int_bound(p, op):
    """Largest input magnitude A with sum spread near the target: the sum of L
    products of two uniform integers in [-A, A] has standard deviation
    sqrt(L) * A (A + 1) / 3."""
    L = reduction_length(p, op)
    want = TARGET_STD[p["dtype"]] * 3.0 / np.sqrt(L)
    a = int(max(1, np.floor((np.sqrt(1 + 4 * want) - 1) / 2)))
    a = min(a, MAX_INPUT[p["dtype"]])
    assert L * a * a < 2 ** 24, "partial sums would not be exact in fp32"
    return a


def int_operands(p, op, seed):
    ho, wo = oracle.out_dims(p)
    a = int_bound(p, op)
    dist = ("ints", tuple(float(v) for v in range(-a, a + 1)))
    x_shape = (p["n"], p["h"], p["w"], p["c"])
    y_shape = (p["n"], ho, wo, p["k"])
    w_shape = (p["k"], p["r"], p["s"], p["c"] // p["groups"])
    if op == "wgrad":
        return synth.wgrad_operands(seed, x_shape, y_shape, p["dtype"], dist)
    return synth.operands(seed, x_shape if op == "fwd" else y_shape, w_shape, p["dtype"],
                          act_dist=dist, w_dist=dist)


def grid_checks(ref, dtype):
    """The exact results must include values the 16-bit type cannot hold,
    among them ties (exactly halfway between two neighbours).  Returns the
    once-rounded bits."""
    bits, rounded = synth.round_to(ref, dtype)
    inexact = rounded != ref
    assert inexact.mean() > 0.3, "too few outputs need rounding (%.3f)" % inexact.mean()
    # the grid neighbour on the other side of the exact value: one bit pattern
    # up in magnitude when rounding went towards zero, one down otherwise
    step = np.where(np.abs(rounded) < np.abs(ref), 1, -1).astype(np.int32)
    other = synth.bits_to_f64((bits.astype(np.int32) + step).astype(np.uint16), dtype)
    ties = inexact & (np.abs(other - ref) == np.abs(rounded - ref))
    assert ties.sum() > 0, "no ties among the outputs"
    return bits


CASES = [
    # (id, pass, problem, override)
    ("dgrad_pointwise_rows", "dgrad", P(2, 14, 14, 64, 256, 1, 1), {}),
    ("dgrad_pointwise_bf16", "dgrad", P(2, 10, 10, 64, 128, 1, 1, dtype="bf16"), {}),
    ("dgrad_pointwise_ring", "dgrad", P(2, 10, 12, 128, 192, 1, 1), dict(tune=1)),
    ("dgrad_ring_s2", "dgrad", P(2, 14, 14, 64, 128, 3, 3, 2, 1, 1), dict(tune=1)),
    ("dgrad_window_s1", "dgrad", P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1), dict(tune=2)),
    ("dgrad_splitk_bf16", "dgrad", P(2, 7, 7, 256, 128, 3, 3, 1, 1, 1, dtype="bf16"),
     dict(variant=api.VAR_DGRAD_SPLITK, split_c=4)),
    ("dgrad_grouped_bf16", "dgrad", P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1, groups=8, dtype="bf16"), {}),
    ("dgrad_dw_tiled", "dgrad", P(2, 16, 16, 64, 64, 3, 3, 1, 1, 1, groups=64), {}),
    ("dgrad_dw_tiled_7x7_bf16", "dgrad", P(1, 14, 12, 32, 32, 7, 7, 1, 3, 3, groups=32, dtype="bf16"), {}),
    ("dgrad_dw_stream_s2", "dgrad", P(2, 20, 20, 32, 32, 7, 7, 2, 3, 3, groups=32), {}),
    ("dgrad_dw_rotated", "dgrad", P(1, 16, 16, 16, 16, 13, 5, 1, 6, 2, groups=16), {}),
    ("dgrad_generic", "dgrad", P(1, 9, 9, 12, 20, 3, 3, 1, 1, 1), {}),
    ("fwd_window_bf16", "fwd", P(2, 7, 7, 128, 64, 3, 3, 1, 1, 1, dtype="bf16"),
     dict(variant=api.VAR_FWD_DIRECT, tune=2)),
    ("fwd_staged_bf16", "fwd", P(2, 7, 7, 128, 64, 3, 3, 1, 1, 1, dtype="bf16"),
     dict(variant=api.VAR_FWD_DIRECT, tune=1)),
    ("fwd_splitc_bf16", "fwd", P(2, 7, 7, 512, 128, 3, 3, 1, 1, 1, dtype="bf16"),
     dict(variant=api.VAR_FWD_SPLITC, split_c=4)),
    ("fwd_splitc_f16", "fwd", P(1, 7, 7, 256, 64, 3, 3, 1, 1, 1),
     dict(variant=api.VAR_FWD_SPLITC, split_c=2)),
    ("fwd_grouped_bf16", "fwd", P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1, groups=8, dtype="bf16"), {}),
    ("fwd_igemm_pointwise", "fwd", P(2, 14, 14, 64, 256, 1, 1), dict(variant=api.VAR_FWD_IGEMM)),
    ("fwd_dw_tiled", "fwd", P(2, 16, 16, 64, 64, 3, 3, 1, 1, 1, groups=64), {}),
    ("fwd_dw_rotated", "fwd", P(1, 16, 16, 16, 16, 13, 13, 1, 6, 6, groups=16), {}),
    ("fwd_generic_bf16", "fwd", P(1, 9, 9, 12, 20, 3, 3, 1, 1, 1, dtype="bf16"), {}),
    ("wgrad_splitk", "wgrad", P(2, 12, 10, 64, 128, 3, 3, 1, 1, 1), {}),
    ("wgrad_splitk_many_splits", "wgrad", P(2, 12, 10, 64, 128, 3, 3, 1, 1, 1), dict(tune=40)),
    ("wgrad_pointwise", "wgrad", P(2, 14, 14, 64, 256, 1, 1), {}),
    ("wgrad_pointwise_bf16", "wgrad", P(2, 8, 8, 64, 64, 1, 1, dtype="bf16"), {}),
    ("wgrad_generic", "wgrad", P(2, 8, 8, 3, 5, 3, 3, 1, 1, 1), {}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_single_rne_rounding_bit_exact(case):
    _, op, p, ov = case
    (ab, af), (bb, bf) = int_operands(p, op, 601)
    if op == "wgrad":
        ref = oracle.conv_wgrad(af, bf, p)
    elif op == "fwd":
        ref = oracle.conv_fwd(af, bf, p)
    else:
        ref = oracle.conv_dgrad(af, bf, p)
    want = grid_checks(ref, p["dtype"])
    with api.override(**ov):
        out = run_wgrad(p, ab, bb) if op == "wgrad" else run_gpu(p, op, ab, bb)
    got = out.cpu().numpy().view(np.uint16)
    bad = got != want
    assert not bad.any(), "%d of %d outputs differ from the once-rounded exact result; first at %s: got %r want %r" % (
        int(bad.sum()), bad.size, np.unravel_index(np.argmax(bad), bad.shape),
        float(synth.bits_to_f64(got[bad][:1], p["dtype"])[0]), float(synth.bits_to_f64(want[bad][:1], p["dtype"])[0]))
