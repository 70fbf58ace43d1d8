"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module only draws random numbers and rounds them to the 16-bit storage
types; it holds none of the convolution's arithmetic (no output sizes, no
index maps).  Callers pass every shape explicitly.

Draw order, distributions and seeds for the named workloads are in
``WORKLOADS``: activations first (x for forward, dY for dgrad), then weights
(for the weight gradient: x, then dY), from one
``numpy.random.Generator(PCG64(seed))``; activations are
uniform[-1, 1], weights normal with standard deviation 1/sqrt(fan_in).  Values
are drawn in float64 and rounded to fp16 (numpy's round-to-nearest-even) or to
bf16 (to float32 first, then to bf16, both round-to-nearest-even).  The same
16-bit patterns feed the GPU and, as exact float64 values, the oracle.
"""
import numpy as np

F16 = "f16"
BF16 = "bf16"


def generator(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


def draw(rng, shape, dist):
    """One float64 array of ``shape`` from ``dist``.

    dist: ("uniform", lo, hi) | ("normal", std) | ("ints", (v0, v1, ...)).
    """
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.normal(0.0, dist[1], size=shape)
    if kind == "ints":
        vals = np.asarray(dist[1], dtype=np.float64)
        return vals[rng.integers(0, len(vals), size=shape)]
    raise ValueError("unknown distribution %r" % (dist,))


def f32_to_bf16_bits(a32):
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits):
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits):
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_to(a64, dtype):
    """(uint16 bit pattern, exact float64 value of those bits) for fp16 or bf16."""
    if dtype == F16:
        bits = np.asarray(a64, dtype=np.float64).astype(np.float16).view(np.uint16)
        return bits, f16_bits_to_f64(bits)
    if dtype == BF16:
        bits = f32_to_bf16_bits(np.asarray(a64, dtype=np.float64).astype(np.float32))
        return bits, bf16_bits_to_f64(bits)
    raise ValueError(dtype)


def bits_to_f64(bits, dtype):
    return f16_bits_to_f64(bits) if dtype == F16 else bf16_bits_to_f64(bits)


def operands(seed, act_shape, w_shape, dtype, act_dist=("uniform", -1.0, 1.0),
             w_dist=None, w_fan_in=None):
    """Activation then weight operand, each as (bits, exact f64 values).

    ``w_dist`` defaults to normal(0, 1/sqrt(w_fan_in)).
    """
    rng = generator(seed)
    if w_dist is None:
        w_dist = ("normal", 1.0 / np.sqrt(float(w_fan_in)))
    a = draw(rng, act_shape, act_dist)
    w = draw(rng, w_shape, w_dist)
    return round_to(a, dtype), round_to(w, dtype)


def wgrad_operands(seed, x_shape, dy_shape, dtype, dist=("uniform", -1.0, 1.0)):
    """The two activation operands of the weight gradient, x then dY, each as
    (bits, exact f64 values), both drawn from ``dist``."""
    rng = generator(seed)
    x = draw(rng, x_shape, dist)
    dy = draw(rng, dy_shape, dist)
    return round_to(x, dtype), round_to(dy, dtype)


def problem(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype=F16):
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=stride, pad_h=pad_h,
                pad_w=pad_w, groups=groups, dtype=dtype)


# The seeded workloads: the five families of shapes the method is measured on.
# op is "dgrad", "fwd" or "wgrad"; fan_in sets the weight standard deviation.
WORKLOADS = {
    "c1_pointwise_tiny": dict(op="dgrad", seed=1, fan_in=None,
                              w_dist=("uniform", -1.0, 1.0),
                              prob=problem(1, 8, 8, 16, 16, 1, 1)),
    "c2_pointwise": dict(op="dgrad", seed=2, fan_in=256,
                         prob=problem(32, 56, 56, 64, 256, 1, 1)),
    "c3a_3x3_s1": dict(op="dgrad", seed=31, fan_in=9 * 256,
                       prob=problem(32, 28, 28, 256, 256, 3, 3, 1, 1, 1)),
    "c3b_3x3_s2": dict(op="dgrad", seed=32, fan_in=9 * 256,
                       prob=problem(32, 56, 56, 256, 256, 3, 3, 2, 1, 1)),
    "c4a_splitc_fwd": dict(op="fwd", seed=41, fan_in=2048 * 9,
                           prob=problem(8, 7, 7, 2048, 512, 3, 3, 1, 1, 1, dtype=BF16)),
    "c4b_grouped_fwd": dict(op="fwd", seed=42, fan_in=8 * 9,
                            prob=problem(32, 28, 28, 256, 256, 3, 3, 1, 1, 1, groups=32,
                                         dtype=BF16)),
    "c5_dw3x3": dict(op="dgrad", seed=51, fan_in=9,
                     prob=problem(16, 56, 56, 384, 384, 3, 3, 1, 1, 1, groups=384)),
    "c5_dw7x7": dict(op="dgrad", seed=52, fan_in=49,
                     prob=problem(16, 56, 56, 384, 384, 7, 7, 1, 3, 3, groups=384)),
    # the pages' stride-2 channel-packed cases (7x7) at the C5 shape: the
    # row-streaming kernel's dispatch case
    "c5_dw7x7_s2": dict(op="dgrad", seed=56, fan_in=49,
                        prob=problem(16, 56, 56, 384, 384, 7, 7, 2, 3, 3, groups=384)),
    "c5_dw31x31": dict(op="dgrad", seed=53, fan_in=961,
                       prob=problem(8, 32, 32, 256, 256, 31, 31, 1, 15, 15, groups=256)),
    "c5_dw51x5": dict(op="dgrad", seed=54, fan_in=255,
                      prob=problem(8, 32, 32, 256, 256, 51, 5, 1, 25, 2, groups=256)),
    "c5_dw5x51": dict(op="dgrad", seed=55, fan_in=255,
                      prob=problem(8, 32, 32, 256, 256, 5, 51, 1, 2, 25, groups=256)),
    # depthwise forward (the next row after the hot path): the C5 shapes, forward
    "f1_dwfwd3x3": dict(op="fwd", seed=61, fan_in=9,
                        prob=problem(16, 56, 56, 384, 384, 3, 3, 1, 1, 1, groups=384)),
    "f1_dwfwd31x31": dict(op="fwd", seed=63, fan_in=961,
                          prob=problem(8, 32, 32, 256, 256, 31, 31, 1, 15, 15, groups=256)),
    # grouped dgrad (the second next row): the grouped forward shape, backward
    "f2_grouped_dgrad": dict(op="dgrad", seed=71, fan_in=8 * 9,
                             prob=problem(32, 28, 28, 256, 256, 3, 3, 1, 1, 1, groups=32,
                                          dtype=BF16)),
    # weight gradient (the third next row): the pointwise and 3x3 dgrad shapes,
    # backward weights; x and dY both uniform[-1, 1] (wgrad_operands)
    "f3_wgrad_pointwise": dict(op="wgrad", seed=81, fan_in=None,
                               prob=problem(32, 56, 56, 64, 256, 1, 1)),
    "f3_wgrad_3x3": dict(op="wgrad", seed=82, fan_in=None,
                         prob=problem(32, 28, 28, 256, 256, 3, 3, 1, 1, 1)),
    # split-K dgrad (the fourth next row): the split-C forward's layer run
    # backward -- few output pixels (8 x 7 x 7) over a 512 x 9 deep reduction;
    # the weights keep that layer's distribution
    "f4_splitk_dgrad": dict(op="dgrad", seed=91, fan_in=2048 * 9,
                            prob=problem(8, 7, 7, 2048, 512, 3, 3, 1, 1, 1, dtype=BF16)),
    # implicit-GEMM forward (the same row): the pointwise dgrad layer run
    # forward, 64 -> 256 channels over 32 x 56 x 56 pixels
    "f4_igemm_fwd_pointwise": dict(op="fwd", seed=92, fan_in=64,
                                   prob=problem(32, 56, 56, 64, 256, 1, 1)),
}
