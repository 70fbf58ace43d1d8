"""Split-K implicit-GEMM dgrad against the fp64 oracle, through the C ABI.

Each output tile's reduction (filter taps of its phase class x 64-deep dY
channel chunks) is divided among blocks that write fp32 partials of dX; the
split reduce pass adds them in ascending split order and rounds once.
"""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth
from gpu_util import check_close, from_device, full_size_parity, operands, parity, run_gpu, to_device

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return synth.problem(n, h, w, c, k, r, s, stride, pad_h, pad_w, groups, dtype)


def ident(p):
    return "n%d_%dx%d_c%d_k%d_f%dx%d_s%d_p%dx%d_g%d_%s" % (
        p["n"], p["h"], p["w"], p["c"], p["k"], p["r"], p["s"], p["stride"], p["pad_h"], p["pad_w"],
        p["groups"], p["dtype"])


SHAPES = [
    P(2, 7, 7, 128, 512, 3, 3, 1, 1, 1),            # stride 1, one class, 72 steps
    P(1, 9, 11, 64, 256, 3, 3, 2, 1, 1),            # stride 2: four classes of 1/2/2/4 taps
    P(1, 7, 7, 96, 320, 3, 3, 1, 1, 1),             # K % 64 != 0 (ragged last chunk), C % 64 != 0
    P(2, 5, 6, 200, 136, 3, 3, 1, 1, 1),            # ragged channel tile
    P(1, 7, 7, 256, 1024, 1, 1),                    # 1x1: pointwise addressing
    P(1, 8, 8, 64, 256, 3, 3, 1, 1, 1, groups=2),   # grouped
    P(1, 7, 7, 128, 512, 5, 3, 1, 2, 0),            # non-square filter, per-axis padding
    P(1, 13, 13, 16, 32, 3, 3, 4, 1, 1),            # stride 4: classes with no taps write zeros
    P(2, 7, 7, 128, 512, 3, 3, 1, 1, 1, dtype="bf16"),
    P(1, 12, 12, 16, 32, 9, 9, 1, 4, 4),            # 81 taps: step ranges cross many taps
]


@pytest.mark.parametrize("split", [2, 3, 8])
@pytest.mark.parametrize("p", SHAPES, ids=ident)
def test_splitk_dgrad_parity(p, split):
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=split):
        parity(p, "dgrad", 120)


def test_more_splits_than_steps():
    """Splits beyond the reduction steps are empty: their partials are zeros
    and the sum is unchanged."""
    p = P(1, 6, 6, 64, 64, 1, 1)   # one 64-deep step per tile
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=5):
        parity(p, "dgrad", 121)


@pytest.mark.parametrize("p", [P(1, 7, 7, 64, 256, 3, 3, 1, 1, 1), P(1, 9, 9, 64, 128, 3, 3, 2, 1, 1),
                               P(1, 6, 6, 32, 128, 1, 1, dtype="bf16")], ids=ident)
def test_splitk_dgrad_exact_on_integer_inputs(p):
    """Inputs in {-1, 0, 1}: partial sums are small integers, exact in fp32,
    so the result equals the rounded oracle bit for bit."""
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=4):
        parity(p, "dgrad", 122, exact=True)


def test_splitk_dgrad_deterministic_and_chunked_equals_unchunked():
    p = P(5, 7, 7, 128, 512, 3, 3, 1, 1, 1)
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=4):
        _, a = parity(p, "dgrad", 123)
        _, b = parity(p, "dgrad", 123)
    ws_img = 4 * 7 * 7 * 128 * 4
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=4, chunk_limit_bytes=2 * ws_img):
        assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [2, 2, 1]
        _, c = parity(p, "dgrad", 123)
    a, b, c = (x.cpu().numpy() for x in (a, b, c))
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_splitk_dgrad_workload_full_size():
    """The benchmarked workload at full size, in the launch configuration the
    benchmark times (automatic split), every dX element against the oracle."""
    assert api.cnhwc_plan(synth.WORKLOADS["f4_splitk_dgrad"]["prob"], api.OP_DGRAD)[1] == api.VAR_DGRAD_SPLITK
    full_size_parity("f4_splitk_dgrad")


# split-K over a small map (stride 1, groups 1, 1x1 or 3x3): the
# filter-streaming kernel, the automatic choice for these shapes
DSTREAM = [
    P(2, 7, 7, 256, 512, 3, 3, 1, 1, 1, dtype="bf16"),
    P(3, 5, 6, 96, 256, 3, 3, 1, 1, 1),               # 90 pixels: ragged last tile, 3 channel tiles
    P(2, 7, 7, 256, 1024, 1, 1),                      # 1x1
    P(1, 8, 6, 64, 256, 3, 3, 1, 1, 0, dtype="bf16"), # per-axis padding
    P(8, 7, 7, 128, 256, 3, 3, 1, 1, 1, dtype="bf16"),# 392 pixels: two groups of 4 images
]


@pytest.mark.parametrize("p", DSTREAM, ids=ident)
def test_splitk_dgrad_filter_streaming_parity(p):
    name, var = api.cnhwc_plan(p, api.OP_DGRAD)
    assert var == api.VAR_DGRAD_SPLITK and name.startswith("dgrad_stream_splitk"), name
    parity(p, "dgrad", 124)


@pytest.mark.parametrize("p", DSTREAM[:3], ids=ident)
def test_splitk_dgrad_filter_streaming_matches_ring_kernel_on_exact_inputs(p):
    """Inputs in {-1, 0, 1}: exact partial sums, so the filter-streaming kernel
    and the ring kernel (tune 1) agree bit for bit at the same split count."""
    name = api.cnhwc_plan(p, api.OP_DGRAD)[0]
    split = int(name.split("splitk")[1].split("_")[0])
    ab, _, wb, _ = operands(p, "dgrad", 125, exact=True)
    stream = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=split, tune=1):
        assert api.cnhwc_plan(p, api.OP_DGRAD)[0].startswith("dgrad_splitk")
        ring = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(stream, ring)
    parity(p, "dgrad", 125, exact=True)
