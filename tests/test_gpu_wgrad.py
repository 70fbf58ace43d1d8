"""GPU parity of the weight gradient (cnhwc_wgrad) against the fp64 oracle.

Every case calls the C ABI on NaN-poisoned dw and a NaN-filled workspace and
compares all K*R*S*Cg elements with oracle.conv_wgrad on the exact values of
the same 16-bit inputs, to |gpu - ref| <= 1e-2 * (1 + |ref|).  The full-size
workloads are checked the same way, every element, at their full size.
"""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth
from gpu_util import check_close, from_device, full_size_parity, run_wgrad

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return synth.problem(n, h, w, c, k, r, s, stride, pad_h, pad_w, groups, dtype)


def ident(p):
    return "n{n}h{h}w{w}c{c}k{k}r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}{dtype}".format(**p)


SPLITK = [
    P(2, 12, 10, 64, 128, 3, 3, 1, 1, 1),                  # 64-channel j block, one k block
    P(2, 9, 11, 128, 128, 3, 3, 1, 1, 1, dtype="bf16"),    # 128-channel j block
    P(3, 14, 13, 256, 136, 3, 3, 2, 1, 1),                 # stride 2, ragged k block (128 + 8)
    P(1, 11, 9, 72, 24, 5, 3, 1, 2, 1),                    # ragged j block, small K, 5x3
    P(2, 7, 7, 48, 64, 7, 7, 2, 3, 3, dtype="bf16"),       # 7x7 stride 2
    P(2, 10, 10, 64, 64, 3, 3, 1, 0, 0, groups=2),         # grouped, Cg = Kg = 32
    P(1, 5, 4, 32, 32, 3, 3, 1, 1, 1),                     # 20 output pixels: one partial stage
    P(2, 16, 16, 16, 16, 1, 1, 2),                         # 1x1 stride 2
    P(1, 9, 9, 24, 40, 4, 2, 3, 1, 0),                     # stride 3, even filter sizes
    P(1, 8, 9, 128, 256, 3, 3, 1, 1, 1, dtype="bf16"),     # 8-wave block: 256 k x 128 j
]
POINTWISE = [
    P(2, 14, 14, 64, 256, 1, 1),
    P(3, 7, 9, 200, 48, 1, 1, dtype="bf16"),               # ragged j blocks (128 + 72), 189 pixels
    P(1, 3, 5, 16, 16, 1, 1),                              # 15 pixels
    P(2, 8, 8, 64, 64, 1, 1, groups=4),                    # grouped pointwise, Cg = Kg = 16
    P(2, 6, 7, 128, 384, 1, 1),                            # 8-wave blocks, ragged second k block
]
GENERIC = [
    P(2, 8, 8, 3, 5, 3, 3, 1, 1, 1),
    P(2, 9, 9, 16, 16, 3, 3, 2, 1, 1, groups=16),          # depthwise
    P(1, 7, 6, 12, 20, 2, 3, 1, 1, 0, groups=2, dtype="bf16"),
]


def operands(p, seed, exact=False):
    ho, wo = oracle.out_dims(p)
    dist = ("ints", (-1.0, 0.0, 1.0)) if exact else ("uniform", -1.0, 1.0)
    return synth.wgrad_operands(seed, (p["n"], p["h"], p["w"], p["c"]), (p["n"], ho, wo, p["k"]),
                                p["dtype"], dist)


def parity(p, seed, exact=False, **ov):
    (xb, xf), (yb, yf) = operands(p, seed, exact)
    with api.override(**ov):
        out = run_wgrad(p, xb, yb)
    got = from_device(out, p["dtype"])
    ref = oracle.conv_wgrad(xf, yf, p)
    if exact:
        assert np.all(np.isfinite(got))
        assert np.array_equal(got, ref), "exact mode: %d mismatches" % int(np.sum(got != ref))
        return 0.0, out
    return check_close(got, ref, ident(p)), out


@pytest.mark.parametrize("p", SPLITK, ids=ident)
def test_wgrad_splitk_parity(p):
    assert api.cnhwc_plan(p, api.OP_WGRAD)[1] == api.VAR_WGRAD_SPLITK
    parity(p, 101)


@pytest.mark.parametrize("tune", [1, 3, 40])
@pytest.mark.parametrize("p", [SPLITK[0], SPLITK[2], POINTWISE[1]], ids=ident)
def test_wgrad_forced_split_counts(p, tune):
    """Any number of pixel splits (one, a few, more than the stages of a split)."""
    parity(p, 102, tune=tune)


@pytest.mark.parametrize("p", POINTWISE, ids=ident)
def test_wgrad_pointwise_parity(p):
    assert api.cnhwc_plan(p, api.OP_WGRAD)[1] == api.VAR_WGRAD_POINTWISE
    parity(p, 103)


@pytest.mark.parametrize("p", POINTWISE, ids=ident)
def test_pointwise_wgrad_is_bit_identical_to_splitk(p):
    """The pointwise kernel drops the per-row gather only: same splits, same
    reduction order, same rounding as the general kernel."""
    (xb, _), (yb, _) = operands(p, 104)
    with api.override(variant=api.VAR_WGRAD_POINTWISE):
        a = run_wgrad(p, xb, yb).cpu().numpy()
    with api.override(variant=api.VAR_WGRAD_SPLITK):
        b = run_wgrad(p, xb, yb).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("p", GENERIC, ids=ident)
def test_wgrad_generic_parity(p):
    assert api.cnhwc_plan(p, api.OP_WGRAD)[1] == api.VAR_WGRAD_GENERIC
    parity(p, 105)


@pytest.mark.parametrize("p", [SPLITK[0], SPLITK[4], POINTWISE[0]], ids=ident)
def test_wgrad_generic_forced_on_mfma_shapes(p):
    parity(p, 106, variant=api.VAR_WGRAD_GENERIC)


@pytest.mark.parametrize("p", [P(2, 8, 8, 64, 128, 3, 3, 1, 1, 1),
                               P(2, 8, 8, 128, 64, 1, 1, dtype="bf16"),
                               P(2, 8, 8, 8, 8, 3, 3, 1, 1, 1)], ids=ident)
def test_wgrad_exact_on_integer_inputs(p):
    """Inputs in {-1, 0, 1} and at most 128 pixels: every partial sum is an
    integer below 2^8, exact in fp32 and in both storage types, so the result
    must equal the oracle bit for bit whatever the summation order."""
    parity(p, 107, exact=True)


def test_wgrad_over_batch_chunks():
    """A chunk limit that splits the batch in three: each chunk adds its own
    pixel splits to the workspace and one reduce sums them all."""
    p = P(6, 10, 9, 64, 64, 3, 3, 1, 1, 1)
    img = 10 * 9 * 64 * 2
    with api.override(chunk_limit_bytes=img * 2):
        assert api.cnhwc_chunk_plan(p, api.OP_WGRAD) == [2, 2, 2]
    parity(p, 108, chunk_limit_bytes=img * 2)
    parity(dict(p, r=1, s=1, pad_h=0, pad_w=0), 109, chunk_limit_bytes=img * 2)


def test_wgrad_is_deterministic():
    p = SPLITK[2]
    (xb, _), (yb, _) = operands(p, 110)
    a = run_wgrad(p, xb, yb).cpu().numpy()
    b = run_wgrad(p, xb, yb).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["f3_wgrad_pointwise", "f3_wgrad_3x3"])
def test_wgrad_workload_full_size(name):
    """The benchmarked workloads at full size, in the launch configuration the
    benchmark times, every dW element against the oracle."""
    full_size_parity(name)
