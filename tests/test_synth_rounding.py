"""Pins of the seeded input generators (CPU): fp16 and bf16 rounding is to
nearest with ties to even, every 16-bit pattern survives the round trip through
its exact float64 value, the draws are reproducible from the seed, and the
distributions are the stated ones.  Both the GPU side and the oracle read these
bit patterns, so a mistake here would not show as a parity failure."""
import numpy as np
import pytest

from convolution_nhwc_amd import synth


def f32(x):
    return np.asarray(x, dtype=np.float32)


def test_bf16_ties_go_to_even_and_others_to_nearest():
    one = 1.0
    # bf16 keeps 7 fraction bits: ulp(1) = 2^-7, halfway = 2^-8
    cases = [
        (one + 2.0 ** -8, 0x3F80),                  # tie, 1.0 is even
        (one + 3 * 2.0 ** -8, 0x3F82),              # tie, 1 + 2^-6 is even
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),     # just above the tie
        (one + 2.0 ** -8 - 2.0 ** -20, 0x3F80),     # just below the tie
        (-(one + 2.0 ** -8), 0xBF80),
        (2.0 ** -149, 0x0000),                      # smallest float32 subnormal rounds to 0
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    got = synth.f32_to_bf16_bits(f32([c[0] for c in cases]))
    assert [int(g) for g in got] == [c[1] for c in cases]


def test_fp16_ties_go_to_even_and_overflow_at_the_tie_above_max():
    # fp16 keeps 10 fraction bits: ulp(1) = 2^-10, halfway = 2^-11
    vals = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -30, 65504.0, 65519.0, 65520.0]
    with np.errstate(over="ignore"):
        bits, exact = synth.round_to(np.array(vals), synth.F16)
    assert [int(b) for b in bits] == [0x3C00, 0x3C02, 0x3C01, 0x7BFF, 0x7BFF, 0x7C00]
    assert exact[0] == 1.0 and exact[1] == 1 + 2.0 ** -9 and exact[3] == 65504.0


def test_fp16_rounds_float64_once():
    # 3.0185546875 is the midpoint between fp16 3.017578125 (0x4209) and
    # 3.01953125 (0x420a); this float64 value lies just below it, so it rounds
    # down.  Rounding through float32 first would land on the midpoint and tie
    # up to 0x420a.
    x = 3.018554582379905
    assert x < 3.0185546875 and float(np.float32(x)) == 3.0185546875
    bits, exact = synth.round_to(np.array([x]), synth.F16)
    assert int(bits[0]) == 0x4209 and exact[0] == 3.017578125


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_every_finite_pattern_round_trips(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = synth.bits_to_f64(bits, dtype)
    fin = np.isfinite(vals)
    back, exact = synth.round_to(vals[fin], dtype)
    # -0.0 and +0.0 keep their own patterns; NaN/inf are never drawn
    assert np.array_equal(back, bits[fin])
    assert np.array_equal(exact, vals[fin])


@pytest.mark.parametrize("dtype", [synth.F16, synth.BF16])
def test_rounding_matches_torch_cpu(dtype):
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(5))
    # float32 values exactly halfway between two bf16 neighbours: a bf16
    # pattern in the high half, 0x8000 in the low half (odd and even patterns)
    hi = rng.integers(0x0080, 0x7F00, 2000).astype(np.uint32)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32).astype(np.float64)
    a = np.concatenate([rng.uniform(-4, 4, 50000), rng.normal(0, 1e-3, 50000), ties, -ties])
    if dtype == synth.F16:
        # torch converts float64 to half through float32; on float32-exact inputs
        # that extra step is exact, so both must round the same way
        a = a.astype(np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        bits, _ = synth.round_to(a, dtype)
    if dtype == synth.F16:
        ref = torch.from_numpy(a).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    else:
        # float64 -> float32 -> bf16, both steps to nearest even
        ref = torch.from_numpy(a).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)


def test_draws_are_reproducible_and_seed_dependent():
    a1, w1 = synth.operands(11, (2, 5, 5, 8), (8, 3, 3, 8), synth.F16, w_fan_in=72)
    a2, w2 = synth.operands(11, (2, 5, 5, 8), (8, 3, 3, 8), synth.F16, w_fan_in=72)
    a3, _ = synth.operands(12, (2, 5, 5, 8), (8, 3, 3, 8), synth.F16, w_fan_in=72)
    assert np.array_equal(a1[0], a2[0]) and np.array_equal(w1[0], w2[0])
    assert not np.array_equal(a1[0], a3[0])


def test_distributions_are_the_stated_ones():
    (ab, af), (wb, wf) = synth.operands(3, (200000,), (200000,), synth.BF16, w_fan_in=256)
    assert af.min() >= -1.0 and af.max() <= 1.0
    assert abs(af.mean()) < 0.01 and abs(af.var() - 1.0 / 3.0) < 0.01      # uniform[-1, 1]
    assert abs(wf.mean()) < 1e-3 and abs(wf.std() - 1.0 / 16.0) < 1e-3     # normal(0, 1/sqrt(256))
    ints = synth.draw(synth.generator(4), (1000,), ("ints", (-2.0, 0.5, 3.0)))
    assert set(np.unique(ints)) == {-2.0, 0.5, 3.0}
