"""GPU parity of depthwise forward (stride 1) on the depthwise kernels -- the
LDS-tiled kernel with the filter rotated by 180 degrees at padding R-1-pad, and
the rotated-filter kernel with the filter as stored -- against the fp64 oracle's
forward convolution."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth

from gpu_util import check_close, from_device, full_size_parity, operands, parity, run_gpu

pytestmark = pytest.mark.gpu


def DW(n, h, w, c, r, s, pad_h=0, pad_w=0, dtype="f16"):
    return dict(n=n, h=h, w=w, c=c, k=c, r=r, s=s, stride=1, pad_h=pad_h, pad_w=pad_w,
                groups=c, dtype=dtype)


def ident(p):
    return "n{n}h{h}w{w}c{c}r{r}s{s}p{pad_h}x{pad_w}{dtype}".format(**p)


TILED = [
    DW(2, 19, 30, 64, 3, 3, 1, 1),             # 'same', ragged tiles
    DW(1, 17, 57, 72, 3, 3, 0, 1),             # valid rows, padded columns, C % 64 != 0
    DW(1, 12, 31, 24, 3, 3, 2, 2),             # pad = R-1 + 1: output larger than the input
    DW(1, 10, 13, 16, 3, 3, 3, 1),             # pad_h > R-1: negative dgrad-side padding
    DW(2, 23, 17, 32, 5, 5, 2, 2),
    DW(1, 20, 22, 64, 7, 7, 3, 3),
    DW(1, 9, 12, 16, 7, 7, 0, 0),              # output smaller than the tile
    DW(2, 19, 29, 64, 3, 3, 1, 1, dtype="bf16"),
    DW(1, 20, 22, 40, 7, 7, 3, 3, dtype="bf16"),
]

ROT = [
    DW(1, 40, 37, 16, 13, 13, 6, 6),
    DW(1, 32, 32, 16, 31, 31, 15, 15),
    DW(1, 32, 32, 8, 51, 5, 25, 2),
    DW(1, 32, 32, 8, 5, 51, 2, 25),
    DW(2, 20, 24, 16, 7, 5, 1, 4),             # per-axis padding, not 'same'
    DW(1, 18, 21, 8, 5, 5, 2, 0),
    DW(1, 70, 45, 8, 3, 9, 1, 4),              # several tiles, ragged
    DW(1, 9, 11, 8, 17, 15, 8, 7),             # filter larger than the image
    DW(1, 14, 16, 8, 5, 5, 6, 7),              # pad > R-1
    DW(1, 33, 30, 16, 31, 31, 15, 15, dtype="bf16"),
]


@pytest.mark.parametrize("p", TILED, ids=ident)
def test_fwd_tiled_parity(p):
    with api.override(variant=api.VAR_FWD_DW_TILED):
        assert "fwd_dw_tiled" in api.cnhwc_plan(p, api.OP_FWD)[0]
        parity(p, "fwd", 401)


def test_fwd_tiled_7x7_several_channel_blocks():
    """The depthwise forward at 7x7 over three channel blocks, the last one
    partial, in bf16."""
    p = DW(2, 30, 33, 136, 7, 7, 3, 3, dtype="bf16")
    with api.override(variant=api.VAR_FWD_DW_TILED):
        parity(p, "fwd", 402)


@pytest.mark.parametrize("p", [DW(2, 30, 33, 136, 7, 7, 3, 3), DW(1, 56, 56, 128, 7, 7, 2, 4, dtype="bf16")],
                         ids=ident)
def test_fwd_tiled_7x7_persistent_matches_one_tile_kernel_bitwise(p):
    """The forward 7x7 (rotated filter) on the persistent kernel equals the
    one-tile kernel (tune 1) bit for bit: same products in the same order."""
    ab, af, wb, wf = operands(p, "fwd", 403)
    with api.override(variant=api.VAR_FWD_DW_TILED):
        assert "dw_tiled_persist" in api.cnhwc_plan(p, api.OP_FWD)[0]
        a = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_FWD_DW_TILED, tune=1):
        assert "dw_tiled_persist" not in api.cnhwc_plan(p, api.OP_FWD)[0]
        b = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)
    parity(p, "fwd", 403)


@pytest.mark.parametrize("tune", [0, 1, 2], ids=["split", "onegroup", "wideslice"])
@pytest.mark.parametrize("p", ROT, ids=ident)
def test_fwd_rotated_parity(p, tune):
    with api.override(variant=api.VAR_FWD_DW_ROTATED, tune=tune):
        assert "fwd_dw_rot" in api.cnhwc_plan(p, api.OP_FWD)[0]
        parity(p, "fwd", 402)


@pytest.mark.parametrize("p", [DW(1, 21, 30, 64, 7, 7, 3, 3), DW(1, 20, 20, 16, 5, 5, 2, 2, dtype="bf16"),
                               DW(1, 20, 20, 8, 13, 9, 6, 2)], ids=ident)
def test_fwd_kernels_agree_on_exact_inputs(p):
    """Inputs in {-1, 0, 1}: every partial sum is exact in fp32, so the
    depthwise kernels and the plain one-output-per-lane kernel must agree bit
    for bit."""
    ab, _, wb, _ = operands(p, "fwd", 403, exact=True)
    auto = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_FWD_GENERIC):
        gen = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(auto, gen)
    parity(p, "fwd", 403, exact=True)


@pytest.mark.parametrize("name", ["f1_dwfwd3x3", "f1_dwfwd31x31"])
def test_full_size_all_images(name):
    full_size_parity(name)
