"""Implicit-GEMM forward (stride 1): the dgrad kernels run on x with the filter
rotated by 180 degrees and transposed, at padding R-1-pad, against the fp64
oracle's forward, through the C ABI."""
import numpy as np
import pytest

from convolution_nhwc_amd import api, synth
from gpu_util import parity

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return synth.problem(n, h, w, c, k, r, s, stride, pad_h, pad_w, groups, dtype)


def ident(p):
    return "n%d_%dx%d_c%d_k%d_f%dx%d_p%dx%d_%s" % (p["n"], p["h"], p["w"], p["c"], p["k"], p["r"], p["s"],
                                                 p["pad_h"], p["pad_w"], p["dtype"])


SHAPES = [
    P(2, 14, 14, 64, 64, 3, 3, 1, 1, 1),        # 'same' 3x3: window kernel, C_d = 64
    P(1, 12, 13, 128, 256, 3, 3, 1, 1, 1),      # C_d = 256: two channel tiles
    P(2, 11, 10, 64, 96, 5, 3, 1, 2, 1),        # non-square, per-axis padding
    P(1, 9, 9, 64, 64, 3, 3, 1, 0, 0),          # no padding ('valid'): rotated padding R-1
    P(1, 10, 10, 48, 80, 3, 3, 1, 1, 0),        # channels not tile multiples
    P(2, 9, 9, 64, 64, 1, 1),                   # 1x1, C_d = K = 64: row-streamed pointwise kernel
    P(1, 8, 9, 96, 128, 1, 1),                  # 1x1, C_d = 128: ring kernel, pointwise addressing
    P(1, 10, 10, 16, 32, 9, 9, 1, 4, 4),        # 81 taps
    P(2, 14, 14, 64, 64, 3, 3, 1, 1, 1, dtype="bf16"),
]


@pytest.mark.parametrize("p", SHAPES, ids=ident)
def test_fwd_igemm_parity(p):
    with api.override(variant=api.VAR_FWD_IGEMM):
        assert api.cnhwc_workspace_size(p, api.OP_FWD) == p["k"] * p["r"] * p["s"] * p["c"] * 2
        parity(p, "fwd", 130)


@pytest.mark.parametrize("p", [P(1, 8, 8, 64, 64, 3, 3, 1, 1, 1), P(1, 6, 7, 32, 64, 1, 1, dtype="bf16")],
                         ids=ident)
def test_fwd_igemm_exact_on_integer_inputs(p):
    with api.override(variant=api.VAR_FWD_IGEMM):
        parity(p, "fwd", 131, exact=True)


def test_fwd_igemm_chunked_equals_unchunked():
    p = P(5, 8, 8, 64, 64, 3, 3, 1, 1, 1)
    img = 8 * 8 * 64 * 2
    with api.override(variant=api.VAR_FWD_IGEMM):
        _, a = parity(p, "fwd", 132)
    with api.override(variant=api.VAR_FWD_IGEMM, chunk_limit_bytes=2 * img):
        assert api.cnhwc_chunk_plan(p, api.OP_FWD) == [2, 2, 1]
        _, b = parity(p, "fwd", 132)
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


POINTWISE_ROWS = [
    P(2, 9, 9, 64, 256, 1, 1),                  # 162 pixels: ragged last block
    P(1, 7, 5, 32, 64, 1, 1),                   # 35 pixels: one wave, most rows past M
    P(3, 10, 11, 64, 128, 1, 1),
    P(2, 8, 8, 32, 256, 1, 1, dtype="bf16"),
    P(4, 28, 28, 64, 256, 1, 1, dtype="bf16"),  # several blocks a wave
]


@pytest.mark.parametrize("p", POINTWISE_ROWS, ids=ident)
def test_pointwise_row_kernel_parity_and_bitwise_equal_to_transform_path(p):
    """The pointwise forward row kernel (filter read as stored, no transform)
    against the oracle, and bit for bit against the filter transform followed
    by the dgrad kernels' pointwise path (tune 1), which run the same MFMA
    chain per output."""
    with api.override(variant=api.VAR_FWD_IGEMM):
        assert api.cnhwc_plan(p, api.OP_FWD)[0].startswith("fwd_pw_rows_")
        _, a = parity(p, "fwd", 133)
    with api.override(variant=api.VAR_FWD_IGEMM, tune=1):
        assert api.cnhwc_plan(p, api.OP_FWD)[0].startswith("fwd_igemm_")
        _, b = parity(p, "fwd", 133)
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_fwd_igemm_workload_full_size():
    """The benchmarked pointwise forward at full size, in the launch
    configuration the benchmark times (automatic dispatch), every output
    element against the oracle."""
    from gpu_util import full_size_parity
    assert api.cnhwc_plan(synth.WORKLOADS["f4_igemm_fwd_pointwise"]["prob"], api.OP_FWD)[1] == api.VAR_FWD_IGEMM
    full_size_parity("f4_igemm_fwd_pointwise")
