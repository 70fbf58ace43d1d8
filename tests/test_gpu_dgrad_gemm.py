"""GPU parity of the MFMA dgrad kernels (1x1 pointwise fast path and general
R x S strided implicit GEMM) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from convolution_nhwc_amd import api, synth

from gpu_util import check_close, from_device, full_size_parity, operands, parity, run_gpu

pytestmark = pytest.mark.gpu


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=stride, pad_h=pad_h, pad_w=pad_w,
                groups=groups, dtype=dtype)


def ident(p):
    return "n{n}h{h}w{w}c{c}k{k}r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}{dtype}".format(**p)


POINTWISE = [
    synth.WORKLOADS["c1_pointwise_tiny"]["prob"],
    P(2, 9, 7, 64, 256, 1, 1),            # M = 126: one ragged M tile
    P(3, 17, 13, 136, 72, 1, 1),          # C and K not multiples of the tiles
    P(1, 8, 8, 16, 16, 1, 1, dtype="bf16"),
    P(2, 20, 20, 192, 40, 1, 1, dtype="bf16"),
    P(2, 13, 11, 40, 128, 1, 1),          # row-streamed kernel, C < 64
    P(1, 7, 9, 64, 192, 1, 1, dtype="bf16"),
]


@pytest.mark.parametrize("p", POINTWISE, ids=ident)
def test_pointwise_parity(p):
    assert api.cnhwc_plan(p, api.OP_DGRAD)[1] == api.VAR_DGRAD_POINTWISE
    parity(p, "dgrad", 101)


GROUPED_POINTWISE = [
    P(1, 8, 8, 16, 16, 1, 1, groups=2),          # 8 channels a group
    P(2, 14, 14, 512, 512, 1, 1, groups=2),      # 256 a group: two channel tiles per group
    P(1, 9, 10, 96, 144, 1, 1, groups=3, dtype="bf16"),  # ragged K per group (48)
]


@pytest.mark.parametrize("p", GROUPED_POINTWISE, ids=ident)
def test_grouped_pointwise_parity_and_bitwise_equal_to_general(p):
    """Grouped 1x1 dgrad on the pointwise fast path (each group's dY channels
    by offset, C/groups as the filter row stride): within tolerance of the
    oracle and bit-identical to the general implicit-GEMM kernel."""
    assert api.cnhwc_plan(p, api.OP_DGRAD)[1] == api.VAR_DGRAD_POINTWISE
    _, fast = parity(p, "dgrad", 109)
    with api.override(variant=api.VAR_DGRAD_IGEMM):
        _, general = parity(p, "dgrad", 109)
    assert np.array_equal(fast.cpu().numpy(), general.cpu().numpy())


IGEMM = [
    P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1),
    P(2, 14, 14, 64, 128, 3, 3, 2, 1, 1),
    P(1, 15, 13, 128, 64, 3, 3, 2, 1, 1),          # odd extents, ragged classes
    P(2, 11, 10, 32, 48, 5, 3, 2, 2, 1),           # non-square filter, per-axis pad
    P(1, 16, 16, 64, 64, 3, 3, 3, 1, 1),           # stride 3: 9 classes
    P(1, 17, 19, 40, 24, 4, 2, 2, 0, 1),           # even filter
    P(1, 9, 9, 16, 16, 1, 1, 2, 0, 0),             # stride > filter: classes with no taps
    P(1, 13, 13, 16, 32, 3, 3, 4, 1, 1),           # stride 4: zero classes
    P(2, 10, 10, 64, 64, 3, 3, 1, 1, 1, groups=2),
    P(1, 12, 12, 48, 96, 3, 3, 2, 1, 1, groups=3),
    P(2, 12, 12, 200, 136, 3, 3, 1, 1, 1),         # C not a tile multiple, K % 64 != 0
    P(1, 10, 12, 64, 64, 7, 7, 1, 3, 3),
    P(2, 14, 14, 64, 64, 3, 3, 1, 1, 1, dtype="bf16"),
    P(1, 16, 16, 64, 64, 3, 3, 2, 1, 1, dtype="bf16"),
    P(1, 8, 8, 16, 16, 1, 1, 1, 1, 1),             # 1x1 padded: general path
    P(1, 12, 12, 16, 16, 9, 9, 1, 4, 4),           # 81 taps in one class (more than 64)
    P(1, 20, 20, 16, 16, 17, 17, 2, 8, 8),         # stride 2: classes of 81, 72, 72 and 64 taps
]


@pytest.mark.parametrize("p", IGEMM, ids=ident)
def test_igemm_parity(p):
    # stride-1 grouped shapes may be dispatched to the grouped merge instead,
    # few tiles over a deep reduction to split-K; this test runs the
    # implicit-GEMM kernel on every shape
    assert api.cnhwc_plan(p, api.OP_DGRAD)[1] in (api.VAR_DGRAD_IGEMM, api.VAR_DGRAD_GROUPED,
                                                  api.VAR_DGRAD_SPLITK)
    with api.override(variant=api.VAR_DGRAD_IGEMM):
        parity(p, "dgrad", 102)


@pytest.mark.parametrize("tune", [1, 2], ids=["ring", "window"])
@pytest.mark.parametrize("p", IGEMM, ids=ident)
def test_igemm_parity_both_kernels(p, tune):
    """Both implicit-GEMM dgrad kernels (every class on the ring kernel; or
    classes with two or more taps on the dY-window kernel) on every shape."""
    with api.override(variant=api.VAR_DGRAD_IGEMM, tune=tune):
        parity(p, "dgrad", 108)


PERSIST = [
    P(2, 14, 14, 256, 128, 3, 3, 2, 1, 1),             # few tiles: shorter tiles, one per block
    P(2, 15, 13, 256, 256, 3, 3, 2, 1, 1),             # odd extents: classes of different sizes
    P(1, 16, 17, 256, 128, 3, 3, 3, 1, 1),             # stride 3: 9 classes
    P(1, 12, 13, 256, 128, 5, 3, 2, 2, 1),             # non-square filter, per-axis padding
    P(2, 10, 10, 512, 256, 3, 3, 2, 1, 1, groups=2),   # two groups of 256 channels
    P(1, 14, 14, 512, 128, 3, 3, 2, 1, 1),             # two channel tiles
    P(1, 15, 15, 256, 128, 4, 4, 2, 1, 2),             # even filter
    P(1, 10, 10, 256, 384, 3, 3, 2, 1, 1),             # 12 reduction chunks per tap
    P(1, 5, 6, 256, 128, 3, 3, 2, 1, 1),               # classes of one or two rows
    P(2, 14, 14, 256, 256, 3, 3, 2, 1, 1, dtype="bf16"),
]


@pytest.mark.parametrize("p", PERSIST, ids=ident)
def test_persistent_parity_and_bitwise_equal_to_ring(p):
    """The persistent 8-wave strided kernel (the implicit-GEMM plan's choice
    for these shapes; small ones go to split-K by default): within tolerance
    of the oracle, and bit-identical to the 4-wave ring kernel, which runs the
    same MFMA chain per output."""
    with api.override(variant=api.VAR_DGRAD_IGEMM):
        assert api.cnhwc_plan(p, api.OP_DGRAD)[0].startswith("dgrad_persist_")
        _, got = parity(p, "dgrad", 112)
    with api.override(variant=api.VAR_DGRAD_IGEMM, tune=1):
        assert api.cnhwc_plan(p, api.OP_DGRAD)[0].startswith("dgrad_igemm_")
        _, ring = parity(p, "dgrad", 112)
    assert np.array_equal(got.cpu().numpy(), ring.cpu().numpy())


def test_persistent_forced_at_stride_1():
    """tune 5 runs the persistent kernel on a stride-1 problem (one class of
    nine taps)."""
    p = P(2, 12, 12, 256, 128, 3, 3, 1, 1, 1)
    with api.override(variant=api.VAR_DGRAD_IGEMM, tune=5):
        assert api.cnhwc_plan(p, api.OP_DGRAD)[0].startswith("dgrad_persist_")
        _, got = parity(p, "dgrad", 114)
    with api.override(variant=api.VAR_DGRAD_IGEMM, tune=1):
        _, ring = parity(p, "dgrad", 114)
    assert np.array_equal(got.cpu().numpy(), ring.cpu().numpy())


def test_persistent_multi_tile_blocks_bitwise_equal_to_ring():
    """The 3x3 stride-2 workload at full size (blocks of the lighter classes
    walk two or four tiles each): bit-identical to the ring kernel on the
    same random inputs (the oracle comparison runs in the full-size test)."""
    p = synth.WORKLOADS["c3b_3x3_s2"]["prob"]
    assert api.cnhwc_plan(p, api.OP_DGRAD)[0].startswith("dgrad_persist_")
    ab, _, wb, _ = operands(p, "dgrad", 113)
    out = run_gpu(p, "dgrad", ab, wb)
    assert np.isfinite(from_device(out, p["dtype"])).all()
    with api.override(variant=api.VAR_DGRAD_IGEMM, tune=1):
        ring = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(out.cpu().numpy(), ring)


@pytest.mark.parametrize("p", [P(1, 12, 12, 64, 64, 3, 3, 2, 1, 1), P(2, 8, 8, 32, 32, 1, 1),
                               P(1, 10, 10, 32, 64, 3, 3, 1, 1, 1, dtype="bf16")], ids=ident)
def test_exact_small_integers_bitwise(p):
    """Inputs in {-1, 0, 1}: every partial sum is exact in fp32, so the rounded
    result must equal the oracle bit for bit whatever the summation order."""
    parity(p, "dgrad", 103, exact=True)


@pytest.mark.parametrize("p", [synth.WORKLOADS["c2_pointwise"]["prob"] | dict(n=2),
                               P(2, 30, 30, 64, 256, 1, 1), P(1, 8, 8, 16, 16, 1, 1, dtype="bf16")],
                         ids=ident)
def test_pointwise_bit_identical_to_general(p):
    ab, _, wb, _ = operands(p, "dgrad", 104)
    fast = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_DGRAD_IGEMM):
        gen = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(fast.view(np.uint16), gen.view(np.uint16))


@pytest.mark.parametrize("tune", [0, 3, 16, 50], ids=["auto", "lds", "bm16", "bm50"])
@pytest.mark.parametrize("p", [P(8, 56, 56, 64, 256, 1, 1), P(3, 17, 13, 40, 72, 1, 1),
                               P(4, 20, 20, 56, 128, 1, 1, dtype="bf16"),
                               P(2, 10, 10, 32, 520, 1, 1), P(1, 5, 7, 8, 64, 1, 1),
                               P(3, 11, 9, 24, 192, 1, 1), P(1, 1, 3, 64, 256, 1, 1)], ids=ident)
def test_pointwise_persistent_matches_ring(p, tune):
    """The row-streamed pointwise kernel (auto for K = 64..256 in steps of 64:
    runs of pixels per wave with ragged last blocks, C from 8 to 64, tiny M)
    and the LDS-persistent one (tune 3 or a tile height; several tiles per
    block at small heights, ragged last tile, K % 64 != 0, the shallower ring
    beside a large filter) against the one-tile-per-block ring kernel, bit for
    bit."""
    ab, _, wb, _ = operands(p, "dgrad", 109)
    with api.override(tune=tune):
        pers = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(tune=1):
        ring = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(pers.view(np.uint16), ring.view(np.uint16))


GROUPED = [
    P(2, 12, 12, 64, 64, 3, 3, 1, 1, 1, groups=8),          # Cg = Kg = 8: 4 groups merged
    P(1, 10, 10, 128, 256, 3, 3, 1, 1, 1, groups=16),       # Cg 8, Kg 16: 2 groups merged
    P(1, 13, 11, 64, 64, 3, 3, 1, 0, 2, groups=8),          # per-axis padding
    P(1, 9, 11, 256, 128, 1, 1, 1, 0, 0, groups=16),        # 1x1, 64 merged outputs
    P(2, 28, 28, 256, 256, 3, 3, 1, 1, 1, groups=32, dtype="bf16"),
    P(1, 30, 9, 128, 128, 3, 3, 1, 1, 0, groups=16, dtype="bf16"),  # two row tiles
]


@pytest.mark.parametrize("p", GROUPED, ids=ident)
def test_grouped_dgrad_parity(p):
    """Grouped dgrad (stride 1) on the block-diagonal merge."""
    assert api.cnhwc_plan(p, api.OP_DGRAD)[1] == api.VAR_DGRAD_GROUPED
    parity(p, "dgrad", 110)


@pytest.mark.parametrize("p", [GROUPED[0], GROUPED[1], GROUPED[3]], ids=ident)
def test_grouped_dgrad_matches_igemm_on_exact_inputs(p):
    """Inputs in {-1, 0, 1}: exact partial sums, so the merged kernel and the
    implicit-GEMM kernel (one group per tile) agree bit for bit."""
    ab, _, wb, _ = operands(p, "dgrad", 111, exact=True)
    merged = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    with api.override(variant=api.VAR_DGRAD_IGEMM):
        ig = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(merged, ig)
    parity(p, "dgrad", 111, exact=True)


def test_reproducible_bitwise():
    p = P(2, 14, 14, 64, 128, 3, 3, 2, 1, 1)
    ab, _, wb, _ = operands(p, "dgrad", 105)
    a = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    b = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(a, b)


def test_chunked_equals_unchunked():
    p = P(5, 12, 12, 64, 64, 3, 3, 2, 1, 1)
    ab, _, wb, _ = operands(p, "dgrad", 106)
    whole = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    img = 12 * 12 * 64 * 2
    with api.override(chunk_limit_bytes=2 * img):
        assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [2, 2, 1]
        parts = run_gpu(p, "dgrad", ab, wb).cpu().numpy()
    assert np.array_equal(whole, parts)


def test_planted_stride_mistake_is_caught():
    """A dY stride mistake planted in the oracle (K+1 instead of K between
    pixels) must break parity; shows the comparison is sensitive to it."""
    p = P(1, 6, 6, 16, 16, 1, 1)
    ab, af, wb, wf = operands(p, "dgrad", 107)
    got = from_device(run_gpu(p, "dgrad", ab, wb), "f16")
    flat = af.reshape(-1)
    wrong = np.stack([flat[i * 17:i * 17 + 16] if i * 17 + 16 <= flat.size else np.zeros(16)
                      for i in range(36)]).reshape(af.shape)
    with pytest.raises(AssertionError):
        check_close(got, oracle.conv_dgrad(wrong, wf, p))


FULL = ["c2_pointwise", "c3a_3x3_s1", "c3b_3x3_s2", "f2_grouped_dgrad"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_all_images(name):
    """The workload at its full size in the benchmark's launch configuration,
    every output element against the oracle."""
    full_size_parity(name)
