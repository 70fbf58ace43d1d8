"""GPU parity of the direct LDS-halo forward kernels (unsplit, split-C with the
reduce pass, grouped block-diagonal merge) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth

from gpu_util import check_close, from_device, full_size_parity, operands, parity, run_gpu

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="bf16"):
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=stride, pad_h=pad_h, pad_w=pad_w,
                groups=groups, dtype=dtype)


def ident(p):
    return "n{n}h{h}w{w}c{c}k{k}r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}{dtype}".format(**p)


DIRECT = [
    P(2, 7, 7, 64, 64, 3, 3, 1, 1, 1),
    P(3, 7, 7, 128, 96, 3, 3, 1, 1, 1),            # 2 images per tile, ragged images and K
    P(1, 20, 20, 64, 64, 3, 3, 1, 1, 1),           # row tiles
    P(1, 30, 17, 72, 40, 3, 3, 2, 1, 1),           # stride 2, odd extents, C % 64 != 0
    P(2, 13, 11, 32, 64, 5, 3, 1, 2, 1),           # non-square, per-axis pad
    P(1, 9, 200, 16, 16, 3, 3, 1, 1, 1),           # wide rows: partial-row tiles
    P(1, 12, 12, 64, 64, 1, 1),                    # 1x1
    P(1, 14, 14, 64, 128, 7, 7, 2, 3, 3),          # 7x7 s2 stem-like
    P(2, 10, 10, 64, 64, 3, 3, 1, 1, 1, dtype="f16"),
    P(1, 12, 12, 128, 128, 3, 3, 1, 1, 1, groups=2),  # grouped, large groups: direct
]


# tune 1: the register-staged direct kernel; 2: the pipelined input-window kernel
KERNELS = pytest.mark.parametrize("tune", [1, 2], ids=["staged", "window"])


@KERNELS
@pytest.mark.parametrize("p", DIRECT, ids=ident)
def test_direct_parity(p, tune):
    with api.override(variant=api.VAR_FWD_DIRECT, tune=tune):
        parity(p, "fwd", 201)


SPLIT = [
    (P(2, 7, 7, 512, 128, 3, 3, 1, 1, 1), 4),
    (P(1, 7, 7, 256, 64, 3, 3, 1, 1, 1), 2),
    (P(2, 5, 9, 384, 64, 3, 3, 1, 1, 1), 3),          # C/split not a multiple of 64
    (P(1, 8, 8, 1024, 64, 3, 3, 2, 1, 1, dtype="f16"), 8),
]


@KERNELS
@pytest.mark.parametrize("p,split", SPLIT, ids=[ident(p) + "x%d" % s for p, s in SPLIT])
def test_split_c_parity(p, split, tune):
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=split, tune=tune):
        assert "splitc%d" % split in api.cnhwc_plan(p, api.OP_FWD)[0]
        parity(p, "fwd", 202)


STREAM = [
    P(2, 7, 7, 512, 128, 3, 3, 1, 1, 1),
    P(3, 5, 6, 256, 96, 3, 3, 1, 1, 1, dtype="f16"),    # 90 pixels: ragged last tile, K % 64 != 0
    P(2, 14, 14, 256, 64, 3, 3, 2, 1, 1, dtype="f16"),  # stride 2: 15 x 15 windows, one image a group
    P(4, 7, 7, 512, 64, 1, 1),                          # 1x1
    P(2, 9, 9, 256, 32, 3, 3, 1, 0, 0, dtype="f16"),    # no padding, one k tile
    P(1, 8, 6, 256, 32, 3, 3, 1, 1, 0),                 # per-axis padding
    P(6, 7, 7, 1024, 32, 3, 3, 1, 1, 1),                # 294 pixels: two groups of 3 images
    P(8, 7, 7, 256, 64, 3, 3, 1, 1, 1),                 # 392 pixels: two groups of 4 images
]


@pytest.mark.parametrize("p", STREAM, ids=ident)
def test_filter_streaming_split_c_parity(p):
    """Split-C over a small map on the filter-streaming kernel (the automatic
    choice for these shapes), every element against the oracle."""
    name, var = api.cnhwc_plan(p, api.OP_FWD)
    assert var == api.VAR_FWD_SPLITC and name.startswith("fwd_stream_"), name
    parity(p, "fwd", 204)


@pytest.mark.parametrize("split", [2, 4, 8, 16])
def test_filter_streaming_forced_splits(split):
    p = P(2, 7, 7, 1024, 64, 3, 3, 1, 1, 1)
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=split):
        assert api.cnhwc_plan(p, api.OP_FWD)[0].startswith("fwd_stream_splitc%d" % split)
        parity(p, "fwd", 205)


@pytest.mark.parametrize("p", STREAM[:3], ids=ident)
def test_filter_streaming_matches_window_kernel_on_exact_inputs(p):
    """Inputs in {-1, 0, 1}: exact partial sums, so the filter-streaming kernel
    and the input-window kernel (tune 3) agree bit for bit."""
    ab, _, wb, _ = operands(p, "fwd", 206, exact=True)
    stream = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    with api.override(tune=3):
        assert api.cnhwc_plan(p, api.OP_FWD)[0].startswith("fwd_direct_")
        window = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(stream, window)
    parity(p, "fwd", 206, exact=True)


def test_filter_streaming_reproducible_and_chunked():
    p = P(5, 7, 7, 512, 64, 3, 3, 1, 1, 1)
    ab, _, wb, _ = operands(p, "fwd", 207)
    a = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    b = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)
    split = int(api.cnhwc_plan(p, api.OP_FWD)[0].split("splitc")[1].split("_")[0])
    ws_img = split * 7 * 7 * 64 * 4
    with api.override(chunk_limit_bytes=2 * ws_img):
        assert api.cnhwc_chunk_plan(p, api.OP_FWD) == [2, 2, 1]
        c = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(a, c)


def test_split_c_reproducible_and_close_to_unsplit():
    p = P(2, 7, 7, 512, 64, 3, 3, 1, 1, 1)
    ab, af, wb, wf = operands(p, "fwd", 203)
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=4):
        a = run_gpu(p, "fwd", ab, wb).cpu().numpy()
        b = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)
    with api.override(variant=api.VAR_FWD_DIRECT):
        u = from_device(run_gpu(p, "fwd", ab, wb), "bf16")
    check_close(synth.bits_to_f64(a.view(np.uint16), "bf16"), oracle.conv_fwd(af, wf, p))
    check_close(u, oracle.conv_fwd(af, wf, p))


GROUPED = [
    P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1, groups=8),     # Cg = Kg = 8, 4 groups merged
    P(1, 14, 14, 32, 32, 3, 3, 1, 1, 1, groups=32),    # depthwise forward, 32 merged
    P(2, 10, 10, 64, 128, 3, 3, 2, 1, 1, groups=16),   # Cg 4, Kg 8 -> 8 merged, 64 wide
    P(1, 9, 9, 64, 64, 5, 5, 1, 2, 2, groups=4),       # Cg 16: 2 merged
    P(1, 11, 13, 64, 32, 3, 1, 1, 1, 0, groups=2),     # Cg 32: no merge
    P(2, 8, 8, 64, 64, 3, 3, 1, 1, 1, groups=8, dtype="f16"),
    P(2, 13, 11, 64, 64, 3, 3, 2, 1, 1, groups=8),     # whole-row kernel, stride 2
    P(1, 10, 10, 128, 128, 1, 1, 1, 0, 0, groups=8),   # whole-row kernel, 1x1, Cg 16
    P(1, 15, 13, 64, 128, 1, 1, 1, 0, 0, groups=4),    # whole-row kernel, 1x1, 64 wide
    P(1, 8, 8, 512, 512, 3, 3, 1, 1, 1, groups=64),    # whole-row kernel, 16 sets over 8 waves
    P(1, 30, 9, 128, 128, 3, 3, 1, 1, 0, groups=16, dtype="f16"),  # whole-row kernel, two row tiles
]


@pytest.mark.parametrize("tune", [0, 1], ids=["auto", "setkernel"])
@pytest.mark.parametrize("p", GROUPED, ids=ident)
def test_grouped_merge_parity(p, tune):
    """Both grouped kernels: the whole-row one (auto, where it applies) and the
    group-set one (tune 1, every shape)."""
    depthwise = p["groups"] == p["c"] == p["k"] and p["stride"] == 1
    # stride-1 depthwise forward is dispatched to the depthwise kernels; the
    # merge is run on it by override here
    assert api.cnhwc_plan(p, api.OP_FWD)[1] == (api.VAR_FWD_DW_TILED if depthwise else api.VAR_FWD_GROUPED)
    with api.override(tune=tune, variant=api.VAR_FWD_GROUPED):
        parity(p, "fwd", 204)


@pytest.mark.parametrize("p,var", [(P(2, 7, 7, 128, 64, 3, 3, 1, 1, 1), api.VAR_FWD_DIRECT),
                                   (P(2, 7, 7, 512, 64, 3, 3, 1, 1, 1), api.VAR_FWD_SPLITC),
                                   (P(1, 10, 10, 64, 64, 3, 3, 1, 1, 1, groups=8), api.VAR_FWD_GROUPED)],
                         ids=["direct", "splitc", "grouped"])
def test_exact_small_integers_bitwise(p, var):
    with api.override(variant=var, split_c=4 if var == api.VAR_FWD_SPLITC else 0):
        parity(p, "fwd", 205, exact=True)


def test_split_c_chunked_equals_unchunked():
    p = P(5, 7, 7, 256, 64, 3, 3, 1, 1, 1)
    ab, _, wb, _ = operands(p, "fwd", 206)
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=2):
        whole = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    ws_img = 2 * 7 * 7 * 64 * 4
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=2, chunk_limit_bytes=2 * ws_img):
        assert api.cnhwc_chunk_plan(p, api.OP_FWD) == [2, 2, 1]
        parts = run_gpu(p, "fwd", ab, wb).cpu().numpy()
    assert np.array_equal(whole, parts)


@pytest.mark.parametrize("name", ["c4a_splitc_fwd", "c4b_grouped_fwd"])
def test_full_size_all_images(name):
    full_size_parity(name)
