"""CPU check of the inputs behind the GPU rounding pin (test_gpu_rounding.py):
every case's operands are integers exact in the storage type, the oracle's
results are integers small enough that fp32 holds every partial sum exactly
(and below fp16's largest finite value), and the once-rounded results differ
from both a truncating and a round-half-away conversion, so the GPU comparison
can tell the three apart."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import synth

import test_gpu_rounding as pin


def truncated(ref, dtype):
    """Round towards zero onto the 16-bit grid (the mistake to be caught)."""
    bits, rounded = synth.round_to(ref, dtype)
    over = np.abs(rounded) > np.abs(ref)
    return np.where(over, (bits.astype(np.int32) - 1).astype(np.uint16), bits)


def half_away(ref, dtype):
    """Round to nearest with ties away from zero (the other mistake)."""
    bits, rounded = synth.round_to(ref, dtype)
    step = np.where(np.abs(rounded) < np.abs(ref), 1, -1).astype(np.int32)
    other_bits = (bits.astype(np.int32) + step).astype(np.uint16)
    other = synth.bits_to_f64(other_bits, dtype)
    tie = (rounded != ref) & (np.abs(other - ref) == np.abs(rounded - ref))
    away = np.abs(other) > np.abs(rounded)
    return np.where(tie & away, other_bits, bits)


@pytest.mark.parametrize("case", pin.CASES, ids=[c[0] for c in pin.CASES])
def test_rounding_pin_inputs_are_exact_and_discriminating(case):
    _, op, p, _ = case
    (ab, af), (bb, bf) = pin.int_operands(p, op, 601)
    for v in (af, bf):
        assert np.array_equal(v, np.round(v)) and np.abs(v).max() <= pin.MAX_INPUT[p["dtype"]]
    fn = {"fwd": oracle.conv_fwd, "dgrad": oracle.conv_dgrad, "wgrad": oracle.conv_wgrad}[op]
    ref = fn(af, bf, p)
    assert np.array_equal(ref, np.round(ref)) and np.abs(ref).max() < min(2 ** 24, 65504)
    want = pin.grid_checks(ref, p["dtype"])
    assert (truncated(ref, p["dtype"]) != want).any()
    assert (half_away(ref, p["dtype"]) != want).any()


def test_tie_detection_on_known_values():
    """fp16 holds only even integers in [2048, 4096): 2049 is a tie that goes
    down to 2048 (even mantissa), 2051 a tie that goes up to 2052, 2050 exact;
    bf16 holds multiples of 2 in [256, 512): 257 -> 256, 259 -> 260."""
    ref = np.array([2049.0, 2051.0, 2050.0, -2049.0, -2051.0])
    bits, rounded = synth.round_to(ref, "f16")
    assert list(rounded) == [2048.0, 2052.0, 2050.0, -2048.0, -2052.0]
    assert list(synth.bits_to_f64(half_away(ref, "f16"), "f16")) == [2050.0, 2052.0, 2050.0, -2050.0, -2052.0]
    assert list(synth.bits_to_f64(truncated(ref, "f16"), "f16")) == [2048.0, 2050.0, 2050.0, -2048.0, -2050.0]
    ref = np.array([257.0, 259.0, 258.0])
    assert list(synth.round_to(ref, "bf16")[1]) == [256.0, 260.0, 258.0]
