"""GPU parity of the depthwise dgrad kernels (row streaming with cpl channels
per lane; LDS-tiled for stride-1 3x3/5x5/7x7; rotated-filter tiled for large /
non-square filters with per-axis padding) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth

from gpu_util import check_close, from_device, full_size_parity, operands, parity, run_gpu

pytestmark = pytest.mark.gpu


def DW(n, h, w, c, r, s, stride=1, pad_h=0, pad_w=0, dtype="f16"):
    return dict(n=n, h=h, w=w, c=c, k=c, r=r, s=s, stride=stride, pad_h=pad_h, pad_w=pad_w,
                groups=c, dtype=dtype)


def ident(p):
    return "n{n}h{h}w{w}c{c}r{r}s{s}st{stride}p{pad_h}x{pad_w}{dtype}".format(**p)


STREAM = [
    (DW(2, 19, 21, 48, 3, 3, 1, 1, 1), 8), (DW(2, 19, 21, 48, 3, 3, 1, 1, 1), 4),
    (DW(2, 19, 21, 48, 3, 3, 1, 1, 1), 2), (DW(1, 19, 21, 24, 3, 3, 1, 1, 1), 1),
    (DW(1, 23, 17, 32, 5, 5, 1, 2, 2), 4), (DW(1, 23, 17, 32, 5, 5, 1, 2, 2), 2),
    (DW(1, 18, 20, 16, 5, 5, 1, 1, 3), 1),                       # pads differ, not 'same'
    (DW(1, 20, 22, 32, 7, 7, 1, 3, 3), 2), (DW(1, 17, 19, 16, 7, 7, 1, 3, 3), 1),
    (DW(1, 9, 12, 16, 7, 7, 1, 2, 5), 2),                         # short image, odd pads
    (DW(2, 20, 23, 48, 3, 3, 2, 1, 1), 8), (DW(1, 21, 20, 32, 3, 3, 2, 1, 1), 4),
    (DW(1, 21, 20, 32, 3, 3, 2, 0, 1), 2), (DW(1, 22, 19, 16, 3, 3, 2, 1, 0), 1),
    (DW(1, 25, 23, 32, 5, 5, 2, 2, 2), 4), (DW(1, 25, 23, 32, 5, 5, 2, 1, 2), 2),
    (DW(1, 18, 18, 16, 5, 5, 2, 2, 2), 1),
    (DW(1, 29, 27, 32, 7, 7, 2, 3, 3), 2), (DW(1, 29, 27, 16, 7, 7, 2, 3, 2), 1),
    (DW(2, 19, 21, 48, 3, 3, 1, 1, 1, dtype="bf16"), 8),
    (DW(1, 20, 22, 32, 7, 7, 1, 3, 3, dtype="bf16"), 2),
    (DW(1, 21, 20, 32, 5, 5, 2, 2, 2, dtype="bf16"), 4),
]


@pytest.mark.parametrize("p,cpl", STREAM, ids=["%s_cpl%d" % (ident(p), c) for p, c in STREAM])
def test_stream_parity(p, cpl):
    with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=cpl):
        assert "cpl%d" % cpl in api.cnhwc_plan(p, api.OP_DGRAD)[0]
        parity(p, "dgrad", 301)


ROT = [
    DW(1, 40, 37, 16, 13, 13, 1, 6, 6),
    DW(1, 32, 32, 16, 31, 31, 1, 15, 15),
    DW(1, 32, 32, 8, 51, 5, 1, 25, 2),
    DW(1, 32, 32, 8, 5, 51, 1, 2, 25),
    DW(2, 20, 24, 16, 7, 5, 1, 1, 4),          # per-axis padding, not 'same'
    DW(1, 18, 21, 8, 5, 5, 1, 2, 0),           # pad_w = 0
    DW(1, 70, 45, 8, 3, 9, 1, 1, 4),           # several tiles, ragged
    DW(1, 9, 11, 8, 17, 15, 1, 8, 7),          # filter larger than the image
    DW(1, 33, 30, 16, 31, 31, 1, 15, 15, dtype="bf16"),
    DW(1, 24, 24, 8, 51, 5, 1, 25, 2, dtype="bf16"),
    # filters narrower than 8 columns: one slice of exactly S columns
    DW(1, 30, 26, 8, 15, 1, 1, 7, 0),
    DW(1, 25, 27, 16, 13, 2, 1, 6, 1),
    DW(1, 40, 37, 8, 21, 3, 1, 10, 1),
    DW(1, 33, 35, 8, 12, 4, 1, 5, 2),          # even filter rows
    DW(2, 28, 30, 16, 9, 6, 1, 4, 3, dtype="bf16"),
    DW(1, 36, 34, 8, 19, 7, 1, 9, 3),
]


@pytest.mark.parametrize("tune", [0, 1, 2], ids=["split", "onegroup", "wideslice"])
@pytest.mark.parametrize("p", ROT, ids=ident)
def test_rotated_parity(p, tune):
    """The rotated-filter kernel with its filter steps split over two lane
    groups (default), with one group (tune 1), and with 8-column filter
    slices for every width (tune 2; by default a filter narrower than 8
    columns is one slice of its own width)."""
    with api.override(variant=api.VAR_DGRAD_DW_ROTATED, tune=tune):
        parity(p, "dgrad", 302)


TILED = [
    DW(2, 19, 30, 64, 3, 3, 1, 1, 1),          # ragged rows and columns of tiles
    DW(1, 8, 28, 128, 3, 3, 1, 1, 1),          # exactly one tile row / column
    DW(1, 17, 57, 72, 3, 3, 1, 0, 1),          # C not a multiple of 64, pads differ
    DW(2, 23, 17, 32, 5, 5, 1, 2, 2),
    DW(1, 12, 31, 24, 5, 5, 1, 4, 0),          # pad > R-1 on one axis
    DW(1, 20, 22, 64, 7, 7, 1, 3, 3),
    DW(1, 9, 33, 200, 3, 3, 1, 1, 1),          # several channel blocks, ragged last block
    DW(1, 13, 29, 136, 7, 7, 1, 3, 3, dtype="bf16"),
    DW(1, 9, 12, 16, 7, 7, 1, 2, 5),           # short image, odd pads
    DW(1, 5, 6, 8, 7, 7, 1, 3, 3),             # image smaller than the filter
    DW(2, 19, 29, 64, 3, 3, 1, 1, 1, dtype="bf16"),
    DW(1, 20, 22, 40, 7, 7, 1, 3, 3, dtype="bf16"),
]


@pytest.mark.parametrize("p", TILED, ids=ident)
def test_tiled_parity(p):
    with api.override(variant=api.VAR_DGRAD_DW_TILED):
        assert "dw_tiled" in api.cnhwc_plan(p, api.OP_DGRAD)[0]
        parity(p, "dgrad", 306)


def test_tiled_and_stream_agree_on_exact_inputs():
    p = DW(1, 21, 30, 64, 7, 7, 1, 3, 3)
    ab, af, wb, wf = operands(p, "dgrad", 307, exact=True)
    with api.override(variant=api.VAR_DGRAD_DW_TILED):
        a = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=2):
        b = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)


TILED7 = [
    DW(2, 37, 61, 200, 7, 7, 1, 3, 3),         # 5 x 3 tiles, 4 channel blocks (the last partial)
    DW(3, 16, 28, 64, 7, 7, 1, 3, 3),          # whole tiles only
    DW(1, 9, 12, 16, 7, 7, 1, 2, 5),           # one partial tile, odd pads
    DW(2, 30, 33, 136, 7, 7, 1, 3, 3, dtype="bf16"),
]


@pytest.mark.parametrize("p", TILED7, ids=ident)
def test_tiled_7x7(p):
    """7x7 over several tile rows, columns and channel blocks (the last one
    partial), with the filter staged per channel block."""
    with api.override(variant=api.VAR_DGRAD_DW_TILED):
        parity(p, "dgrad", 308)


# the persistent 7x7 kernel: runs of several tiles a block (the C5 shape at
# one image), a channel block with more blocks than tiles, ragged tiles
PERSIST7 = [
    DW(2, 37, 61, 200, 7, 7, 1, 3, 3),
    DW(1, 56, 56, 384, 7, 7, 1, 3, 3),
    DW(1, 9, 12, 16, 7, 7, 1, 2, 5),
    DW(3, 30, 33, 136, 7, 7, 1, 3, 3, dtype="bf16"),
]


@pytest.mark.parametrize("p", PERSIST7, ids=ident)
def test_tiled_7x7_persistent_matches_one_tile_kernel_bitwise(p):
    """The persistent kernel adds every product in the one-tile kernel's order
    (filter row pairs from the last, columns ascending), so the two agree bit
    for bit; both against the oracle."""
    ab, af, wb, wf = operands(p, "dgrad", 309)
    with api.override(variant=api.VAR_DGRAD_DW_TILED):
        assert "dw_tiled_persist" in api.cnhwc_plan(p, api.OP_DGRAD)[0]
        a = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_DGRAD_DW_TILED, tune=1):
        assert "dw_tiled_persist" not in api.cnhwc_plan(p, api.OP_DGRAD)[0]
        b = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)
    parity(p, "dgrad", 309)


@pytest.mark.parametrize("p,var,cpl", [(DW(1, 17, 19, 32, 3, 3, 1, 1, 1), api.VAR_DGRAD_DW_STREAM, 8),
                                       (DW(1, 17, 30, 64, 5, 5, 1, 2, 2), api.VAR_DGRAD_DW_TILED, 0),
                                       (DW(1, 17, 19, 32, 7, 7, 2, 3, 3), api.VAR_DGRAD_DW_STREAM, 2),
                                       (DW(1, 20, 20, 8, 13, 9, 1, 6, 2), api.VAR_DGRAD_DW_ROTATED, 0),
                                       (DW(1, 20, 20, 16, 5, 5, 1, 2, 2, dtype="bf16"), api.VAR_DGRAD_DW_STREAM, 4)],
                         ids=["s3x3", "t5x5", "s7x7st2", "rot13x9", "s5x5bf16"])
def test_exact_small_integers_bitwise(p, var, cpl):
    with api.override(variant=var, cpl=cpl):
        parity(p, "dgrad", 303, exact=True)


def test_stream_and_rotated_agree():
    """Two different kernels (different summation orders) on one problem both
    meet the tolerance, and on exact inputs agree bit for bit."""
    p = DW(1, 21, 19, 16, 5, 5, 1, 2, 2)
    ab, af, wb, wf = operands(p, "dgrad", 304, exact=True)
    with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=2):
        a = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_DGRAD_DW_ROTATED):
        b = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)


def test_cpl_matrix_on_the_3x3_and_7x7_workloads():
    """Every cpl the dispatcher admits for the two row-streaming workloads
    (on 2 of their 16 images); refusals must carry a register-budget reason."""
    for name in ("c5_dw3x3", "c5_dw7x7", "c5_dw7x7_s2"):
        p = dict(synth.WORKLOADS[name]["prob"], n=2)
        for cpl in (8, 4, 2):
            try:
                with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=cpl):
                    api.cnhwc_plan(p, api.OP_DGRAD)
            except api.CnhwcError as e:
                assert "register budget" in e.reason
                continue
            with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=cpl):
                parity(p, "dgrad", 305)


@pytest.mark.parametrize("name", ["c5_dw3x3", "c5_dw7x7", "c5_dw7x7_s2", "c5_dw31x31", "c5_dw51x5", "c5_dw5x51"])
def test_full_size_all_images(name):
    full_size_parity(name)
