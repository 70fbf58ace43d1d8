"""CPU tests of the C ABI's host logic: exports, validation order and reasons,
output extents, the dispatcher's choices, the batch-chunk planner, workspace
sizing and the pointer checks.  Nothing here launches a kernel."""
import os
import re

import pytest

import oracle
from convolution_nhwc_amd import api, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1, dtype="f16"):
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=stride, pad_h=pad_h, pad_w=pad_w,
                groups=groups, dtype=dtype)


def declared_symbols():
    syms = set()
    for name in os.listdir(os.path.join(ROOT, "include")):
        if name.endswith(".h"):
            text = open(os.path.join(ROOT, "include", name)).read()
            syms |= set(re.findall(r"^\s*(?:int|const char\*|void)\s+\**(cnhwc_\w+)\s*\(", text, re.M))
    return syms


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert {"cnhwc_fwd", "cnhwc_dgrad", "cnhwc_plan"} <= syms
    L = api.lib()
    for s in syms:
        assert hasattr(L, s), s
    assert set(api.SYMBOLS) >= syms


@pytest.mark.parametrize("p", [P(2, 9, 11, 8, 8, 3, 3, 1, 1, 1), P(1, 56, 56, 64, 64, 3, 3, 2, 1, 1),
                               P(3, 17, 13, 8, 16, 5, 3, 3, 2, 0), P(1, 32, 32, 8, 8, 51, 5, 1, 25, 2, 8),
                               P(1, 7, 7, 16, 16, 7, 7, 4, 0, 3), P(1, 24, 24, 8, 8, 3, 3, 1, 1, 0)])
def test_out_dims_match_oracle(p):
    assert api.cnhwc_out_dims(p) == oracle.out_dims(p)


REFUSALS = [
    (dict(groups=0), "groups must be >= 1"),
    (dict(groups=-4), "groups must be >= 1"),
    (dict(groups=3), "multiples of groups"),
    (dict(stride=0), "stride must be >= 1"),
    (dict(pad_h=-1), "padding must be >= 0"),
    (dict(pad_w=-2), "padding must be >= 0"),
    (dict(n=0), "n must be >= 1"),
    (dict(r=9, s=9), "filter larger than the padded input"),
    (dict(dtype=7), "dtype"),
]


@pytest.mark.parametrize("change,reason", REFUSALS, ids=[r for _, r in REFUSALS])
def test_validation_refuses_with_reason(change, reason):
    p = dict(P(1, 6, 6, 8, 8, 3, 3, 1, 1, 1), **change)
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_out_dims(p)
    assert e.value.status == api.INVALID_ARG
    assert reason in e.value.reason


def test_validation_order_reports_first_failure():
    p = dict(P(1, 6, 6, 8, 8, 3, 3), stride=0, groups=0)
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_out_dims(p)
    assert "stride" in e.value.reason


def test_reserved_field_must_be_zero():
    pr = api._problem(P(1, 6, 6, 8, 8, 3, 3))
    pr.reserved = 1
    with pytest.raises(api.CnhwcError):
        api.cnhwc_out_dims(pr)


def wl(name):
    return synth.WORKLOADS[name]


EXPECT = {
    "c1_pointwise_tiny": api.VAR_DGRAD_POINTWISE,
    "c2_pointwise": api.VAR_DGRAD_POINTWISE,
    "c3a_3x3_s1": api.VAR_DGRAD_IGEMM,
    "c3b_3x3_s2": api.VAR_DGRAD_IGEMM,
    "c4a_splitc_fwd": api.VAR_FWD_SPLITC,
    "c4b_grouped_fwd": api.VAR_FWD_GROUPED,
    "c5_dw3x3": api.VAR_DGRAD_DW_TILED,
    "c5_dw7x7": api.VAR_DGRAD_DW_TILED,
    "c5_dw7x7_s2": api.VAR_DGRAD_DW_STREAM,
    "c5_dw31x31": api.VAR_DGRAD_DW_ROTATED,
    "c5_dw51x5": api.VAR_DGRAD_DW_ROTATED,
    "c5_dw5x51": api.VAR_DGRAD_DW_ROTATED,
    "f1_dwfwd3x3": api.VAR_FWD_DW_TILED,
    "f1_dwfwd31x31": api.VAR_FWD_DW_ROTATED,
    "f2_grouped_dgrad": api.VAR_DGRAD_GROUPED,
    "f3_wgrad_pointwise": api.VAR_WGRAD_POINTWISE,
    "f3_wgrad_3x3": api.VAR_WGRAD_SPLITK,
    "f4_splitk_dgrad": api.VAR_DGRAD_SPLITK,
    "f4_igemm_fwd_pointwise": api.VAR_FWD_IGEMM,
}

OPC = {"fwd": api.OP_FWD, "dgrad": api.OP_DGRAD, "wgrad": api.OP_WGRAD}


@pytest.mark.parametrize("name", sorted(EXPECT))
def test_dispatcher_choice_per_workload(name):
    w = wl(name)
    kname, var = api.cnhwc_plan(w["prob"], OPC[w["op"]])
    assert var == EXPECT[name], (name, kname)


def test_depthwise_forward_dispatch():
    """Stride-1 depthwise forward runs on the depthwise kernels (small square
    filters tiled, large / non-square / uneven padding rotated); strided
    depthwise forward stays on the grouped merge."""
    dw = dict(n=1, h=20, w=20, c=32, k=32, groups=32, dtype="f16")
    assert api.cnhwc_plan(dict(dw, r=5, s=5, stride=1, pad_h=2, pad_w=2), api.OP_FWD)[1] == api.VAR_FWD_DW_TILED
    assert api.cnhwc_plan(dict(dw, r=13, s=13, stride=1, pad_h=6, pad_w=6), api.OP_FWD)[1] == api.VAR_FWD_DW_ROTATED
    assert api.cnhwc_plan(dict(dw, r=7, s=5, stride=1, pad_h=3, pad_w=2), api.OP_FWD)[1] == api.VAR_FWD_DW_ROTATED
    assert api.cnhwc_plan(dict(dw, r=3, s=3, stride=2, pad_h=1, pad_w=1), api.OP_FWD)[1] == api.VAR_FWD_GROUPED
    # a depthwise dgrad variant is not a forward kernel
    with api.override(variant=api.VAR_DGRAD_DW_TILED):
        with pytest.raises(Exception):
            api.cnhwc_plan(dict(dw, r=3, s=3, stride=1, pad_h=1, pad_w=1), api.OP_FWD)


def test_dispatcher_falls_back_to_generic():
    # channel counts that are not multiples of 8 go to the plain kernels
    assert api.cnhwc_plan(P(1, 8, 8, 3, 5, 3, 3, 1, 1, 1), api.OP_DGRAD)[1] == api.VAR_DGRAD_GENERIC
    assert api.cnhwc_plan(P(1, 8, 8, 3, 5, 3, 3, 1, 1, 1), api.OP_FWD)[1] == api.VAR_FWD_GENERIC
    # strides above 4 exceed the implicit-GEMM class table
    assert api.cnhwc_plan(P(1, 16, 16, 8, 8, 5, 5, 5, 2, 2), api.OP_DGRAD)[1] == api.VAR_DGRAD_GENERIC


def test_pointwise_only_for_its_shape_class():
    for p in [P(1, 8, 8, 16, 16, 1, 1, 2), P(1, 8, 8, 16, 16, 1, 1, 1, 1, 1),
              P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1)]:
        assert api.cnhwc_plan(p, api.OP_DGRAD)[1] != api.VAR_DGRAD_POINTWISE


def test_grouped_pointwise_dispatch():
    """Grouped 1x1 dgrad: the block-diagonal merge when its groups merge into
    one MFMA tile, else the pointwise fast path with the group offsets."""
    assert api.cnhwc_plan(P(1, 8, 8, 16, 16, 1, 1, groups=2), api.OP_DGRAD)[1] == api.VAR_DGRAD_POINTWISE
    assert api.cnhwc_plan(P(2, 14, 14, 512, 512, 1, 1, groups=2), api.OP_DGRAD)[1] == api.VAR_DGRAD_POINTWISE
    assert api.cnhwc_plan(P(1, 9, 11, 256, 128, 1, 1, groups=16), api.OP_DGRAD)[1] == api.VAR_DGRAD_GROUPED


def test_forced_variant_refusals_carry_reasons():
    p = P(1, 16, 16, 16, 16, 3, 3, 2, 1, 1, groups=16)
    with api.override(variant=api.VAR_DGRAD_DW_ROTATED):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(p, api.OP_DGRAD)
    assert e.value.status == api.UNSUPPORTED and "stride" in e.value.reason
    big = P(1, 70, 70, 16, 16, 65, 3, 1, 32, 1, groups=16)
    with api.override(variant=api.VAR_DGRAD_DW_ROTATED):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(big, api.OP_DGRAD)
    assert "64" in e.value.reason
    with api.override(variant=api.VAR_DGRAD_POINTWISE):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1), api.OP_DGRAD)
    assert "1x1" in e.value.reason
    with api.override(variant=api.VAR_FWD_DIRECT):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1), api.OP_DGRAD)
    assert "not a dgrad kernel" in e.value.reason


def test_override_rejects_bad_cpl():
    with pytest.raises(api.CnhwcError):
        api.cnhwc_set_override(cpl=3)
    api.cnhwc_clear_override()


def test_depthwise_stream_cpl_must_divide_channels():
    p = P(1, 16, 16, 12, 12, 3, 3, 1, 1, 1, groups=12)
    with api.override(variant=api.VAR_DGRAD_DW_STREAM, cpl=8):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(p, api.OP_DGRAD)
    assert "cpl" in e.value.reason


@pytest.mark.parametrize("n,limit_images", [(7, 3), (10, 4), (5, 1), (9, 9), (1, 1)])
def test_chunk_planner_is_balanced(n, limit_images):
    p = P(n, 8, 8, 16, 16, 3, 3, 1, 1, 1)
    per_image = 8 * 8 * 16 * 2
    with api.override(chunk_limit_bytes=per_image * limit_images):
        counts = api.cnhwc_chunk_plan(p, api.OP_DGRAD)
    chunks = -(-n // limit_images)
    assert len(counts) == chunks and sum(counts) == n
    assert max(counts) - min(counts) <= 1 and max(counts) <= limit_images
    assert counts == sorted(counts, reverse=True)


def test_chunk_planner_default_is_one_chunk_for_every_workload():
    for name, w in synth.WORKLOADS.items():
        assert api.cnhwc_chunk_plan(w["prob"], OPC[w["op"]]) == [w["prob"]["n"]], name


LARGE_BATCH = [("c5_dw3x3", api.VAR_DGRAD_DW_TILED), ("c5_dw7x7", api.VAR_DGRAD_DW_TILED),
               ("c5_dw7x7_s2", api.VAR_DGRAD_DW_STREAM), ("c5_dw31x31", api.VAR_DGRAD_DW_ROTATED),
               ("c5_dw51x5", api.VAR_DGRAD_DW_ROTATED), ("f1_dwfwd3x3", api.VAR_FWD_DW_TILED),
               ("f1_dwfwd31x31", api.VAR_FWD_DW_ROTATED), ("c4a_splitc_fwd", api.VAR_FWD_DIRECT),
               ("c4b_grouped_fwd", api.VAR_FWD_GROUPED), ("c3a_3x3_s1", api.VAR_DGRAD_IGEMM),
               ("c2_pointwise", api.VAR_DGRAD_POINTWISE)]


@pytest.mark.parametrize("name,var", LARGE_BATCH, ids=[n for n, _ in LARGE_BATCH])
def test_large_batch_keeps_the_kernel_and_chunks(name, var):
    """A batch past the 32-bit buffer range keeps the kernel its shape selects
    (the split-C layer has enough output tiles at that batch to run unsplit)
    and runs as balanced chunks: the per-kernel checks look at one image, the
    batch is the chunk planner's ("feat(rocke): split-C and grouped LDS-halo
    direct conv fwd kernels", supporting changes: balanced per-chunk launches)."""
    w = wl(name)
    p = dict(w["prob"])
    ho, wo = oracle.out_dims(p)
    per_image = max(p["h"] * p["w"] * p["c"], ho * wo * p["k"]) * 2
    n_one = (2 ** 31 - 1) // per_image
    p["n"] = 2 * n_one + 3
    assert api.cnhwc_plan(p, OPC[w["op"]])[1] == var
    counts = api.cnhwc_chunk_plan(p, OPC[w["op"]])
    assert len(counts) == 3 and sum(counts) == p["n"] and max(counts) <= n_one
    assert max(counts) - min(counts) <= 1


def test_dw3x3_at_1024_images_is_two_chunks_of_512():
    p = dict(wl("c5_dw3x3")["prob"], n=1024)
    assert api.cnhwc_plan(p, api.OP_DGRAD)[1] == api.VAR_DGRAD_DW_TILED
    assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [512, 512]
    f = dict(wl("f1_dwfwd3x3")["prob"], n=1024)
    assert api.cnhwc_plan(f, api.OP_FWD)[1] == api.VAR_FWD_DW_TILED
    assert api.cnhwc_chunk_plan(f, api.OP_FWD) == [512, 512]


def test_override_cannot_raise_the_chunk_limit():
    """A test limit above the 32-bit range is clamped to it."""
    p = dict(wl("c5_dw3x3")["prob"], n=1024)
    with api.override(chunk_limit_bytes=1 << 40):
        assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [512, 512]


def test_chunk_planner_refuses_an_oversized_image():
    p = P(2, 8, 8, 16, 16, 3, 3, 1, 1, 1)
    with api.override(chunk_limit_bytes=1000):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_chunk_plan(p, api.OP_DGRAD)
    assert e.value.status == api.UNSUPPORTED and "one image" in e.value.reason


def test_chunk_planner_uses_the_largest_view():
    # dgrad with stride 2: dx per image is 4x dy per image
    p = P(6, 16, 16, 8, 8, 3, 3, 2, 1, 1)
    dx_img = 16 * 16 * 8 * 2
    with api.override(chunk_limit_bytes=dx_img * 2):
        assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [2, 2, 2]


def test_workspace_only_for_split_c():
    w = wl("c4a_splitc_fwd")
    p = w["prob"]
    name, var = api.cnhwc_plan(p, api.OP_FWD)
    assert var == api.VAR_FWD_SPLITC
    split = int(re.search(r"splitc(\d+)", name).group(1))
    assert split >= 2
    assert api.cnhwc_workspace_size(p, api.OP_FWD) == split * 8 * 7 * 7 * 512 * 4
    assert api.cnhwc_workspace_size(wl("c3a_3x3_s1")["prob"], api.OP_DGRAD) == 0
    assert api.cnhwc_workspace_size(wl("c4b_grouped_fwd")["prob"], api.OP_FWD) == 0


def test_pointer_checks_precede_any_launch():
    p = P(1, 8, 8, 16, 16, 1, 1)
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_dgrad(p, None, None, None, None, 0, None)
    assert e.value.status == api.INVALID_ARG and "NULL" in e.value.reason
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_dgrad(p, 0x10008, 0x20000, 0x30000, None, 0, None)
    assert e.value.status == api.MISALIGNED
    with pytest.raises(api.CnhwcError) as e:  # dx overlaps dy
        api.cnhwc_dgrad(p, 0x100000, 0x200000, 0x100000 + 64, None, 0, None)
    assert e.value.status == api.INVALID_ARG and "overlaps" in e.value.reason


def test_split_c_workspace_checks():
    w = wl("c4a_splitc_fwd")
    p = w["prob"]
    need = api.cnhwc_workspace_size(p, api.OP_FWD)
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_fwd(p, 0x1000000, 0x4000000, 0x8000000, 0x10000000, need - 16, None)
    assert e.value.status == api.WORKSPACE_TOO_SMALL
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_fwd(p, 0x1000000, 0x4000000, 0x8000000, None, need, None)
    assert e.value.status == api.INVALID_ARG


def test_last_error_clears_after_success():
    with pytest.raises(api.CnhwcError):
        api.cnhwc_out_dims(P(0, 8, 8, 8, 8, 1, 1))
    assert api.last_error() != ""
    api.cnhwc_out_dims(P(1, 8, 8, 8, 8, 1, 1))
    assert api.last_error() == ""


def test_wgrad_dispatch():
    """1x1 stride-1 unpadded wgrad takes the pointwise kernel (grouped too),
    other shapes with 8-aligned channel groups of at least 16 the split-K
    kernel, everything else the plain kernel."""
    W = api.OP_WGRAD
    assert api.cnhwc_plan(P(2, 8, 8, 64, 32, 1, 1), W)[1] == api.VAR_WGRAD_POINTWISE
    assert api.cnhwc_plan(P(2, 8, 8, 64, 32, 1, 1, groups=2), W)[1] == api.VAR_WGRAD_POINTWISE
    for p in [P(1, 8, 8, 16, 16, 1, 1, 2), P(1, 8, 8, 16, 16, 1, 1, 1, 1, 1),
              P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1), P(2, 9, 7, 32, 64, 5, 3, 2, 2, 1, groups=2)]:
        assert api.cnhwc_plan(p, W)[1] == api.VAR_WGRAD_SPLITK, p
    for p in [P(1, 8, 8, 3, 5, 3, 3, 1, 1, 1), P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1, groups=16),
              P(1, 8, 8, 12, 16, 1, 1), P(1, 8, 8, 16, 8, 3, 3, 1, 1, 1)]:
        assert api.cnhwc_plan(p, W)[1] == api.VAR_WGRAD_GENERIC, p
    with api.override(variant=api.VAR_DGRAD_IGEMM):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1), W)
    assert "not a wgrad kernel" in e.value.reason
    with api.override(variant=api.VAR_WGRAD_POINTWISE):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1), W)
    assert "1x1" in e.value.reason
    with api.override(variant=api.VAR_WGRAD_GENERIC):
        with pytest.raises(api.CnhwcError):
            api.cnhwc_plan(P(1, 8, 8, 16, 16, 3, 3, 1, 1, 1), api.OP_DGRAD)


def test_wgrad_workspace_counts_every_chunks_splits():
    """Workspace = (pixel splits of all chunks) * K*R*S*Cg fp32 partials; the
    plain kernel needs none and runs as one launch."""
    p = P(6, 16, 16, 32, 64, 3, 3, 1, 1, 1)
    elems = 64 * 9 * 32
    with api.override(tune=5):
        assert api.cnhwc_workspace_size(p, api.OP_WGRAD) == 5 * elems * 4
    img = 16 * 16 * 64 * 2  # dy per image is the largest view
    with api.override(tune=5, chunk_limit_bytes=img * 2):
        assert api.cnhwc_chunk_plan(p, api.OP_WGRAD) == [2, 2, 2]
        assert api.cnhwc_workspace_size(p, api.OP_WGRAD) == 3 * 5 * elems * 4
    auto = api.cnhwc_workspace_size(p, api.OP_WGRAD)
    assert auto > 0 and auto % (elems * 4) == 0
    g = P(6, 16, 16, 3, 5, 3, 3, 1, 1, 1)
    assert api.cnhwc_workspace_size(g, api.OP_WGRAD) == 0
    with api.override(chunk_limit_bytes=16 * 16 * 5 * 2):
        assert api.cnhwc_chunk_plan(g, api.OP_WGRAD) == [6]


def test_wgrad_checks_precede_any_launch():
    p = P(2, 8, 8, 16, 16, 3, 3, 1, 1, 1)
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_wgrad(p, None, 0x200000, 0x300000, None, 0, None)
    assert e.value.status == api.INVALID_ARG and "x is NULL" in e.value.reason
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_wgrad(p, 0x100000, 0x200008, 0x300000, None, 0, None)
    assert e.value.status == api.MISALIGNED and "dy" in e.value.reason
    with pytest.raises(api.CnhwcError) as e:  # dw overlaps x
        api.cnhwc_wgrad(p, 0x100000, 0x200000, 0x100000 + 64, None, 0, None)
    assert e.value.status == api.INVALID_ARG and "overlaps" in e.value.reason
    need = api.cnhwc_workspace_size(p, api.OP_WGRAD)
    assert need > 0
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_wgrad(p, 0x100000, 0x200000, 0x300000, 0x1000000, need - 16, None)
    assert e.value.status == api.WORKSPACE_TOO_SMALL
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_wgrad(p, 0x100000, 0x200000, 0x300000, None, need, None)
    assert e.value.status == api.INVALID_ARG and "ws" in e.value.reason
    with pytest.raises(api.CnhwcError) as e:  # workspace overlaps dy
        api.cnhwc_wgrad(p, 0x100000, 0x200000, 0x300000, 0x200000 + 256, need, None)
    assert e.value.status == api.INVALID_ARG and "workspace overlaps" in e.value.reason
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_plan(p, 3)
    assert e.value.status == api.INVALID_ARG


def test_splitk_dgrad_dispatch_and_workspace():
    """Few output tiles over a deep reduction split the reduction; the
    workspace holds one fp32 partial of dX per split; the large-map dgrad
    workloads stay unsplit with no workspace."""
    w = wl("f4_splitk_dgrad")
    p = w["prob"]
    name, var = api.cnhwc_plan(p, api.OP_DGRAD)
    assert var == api.VAR_DGRAD_SPLITK
    split = int(re.search(r"splitk(\d+)", name).group(1))
    assert 2 <= split <= 64
    assert api.cnhwc_workspace_size(p, api.OP_DGRAD) == split * 8 * 7 * 7 * 2048 * 4
    for other in ("c2_pointwise", "c3a_3x3_s1", "c3b_3x3_s2"):
        assert api.cnhwc_workspace_size(wl(other)["prob"], api.OP_DGRAD) == 0
    # deep 1x1 with a small map splits too (the pointwise addressing inside)
    small_1x1 = P(1, 7, 7, 512, 2048, 1, 1)
    assert api.cnhwc_plan(small_1x1, api.OP_DGRAD)[1] == api.VAR_DGRAD_SPLITK
    # a short reduction does not split
    assert api.cnhwc_plan(P(1, 7, 7, 64, 64, 3, 3, 1, 1, 1), api.OP_DGRAD)[1] == api.VAR_DGRAD_IGEMM
    # depthwise never takes it
    dw = dict(n=1, h=7, w=7, c=512, k=512, r=3, s=3, stride=1, pad_h=1, pad_w=1, groups=512, dtype="f16")
    assert api.cnhwc_plan(dw, api.OP_DGRAD)[1] != api.VAR_DGRAD_SPLITK


def test_splitk_dgrad_forced_split_counts_and_refusals():
    p = P(2, 9, 9, 64, 256, 3, 3, 2, 1, 1)
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=5):
        name, var = api.cnhwc_plan(p, api.OP_DGRAD)
        assert var == api.VAR_DGRAD_SPLITK and "splitk5_" in name
        assert api.cnhwc_workspace_size(p, api.OP_DGRAD) == 5 * 2 * 9 * 9 * 64 * 4
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=1):
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_plan(p, api.OP_DGRAD)
        assert e.value.status == api.UNSUPPORTED and "2 reduction splits" in e.value.reason
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=4):
        with pytest.raises(api.CnhwcError) as e:   # channels not a multiple of 8
            api.cnhwc_plan(P(1, 8, 8, 12, 16, 3, 3, 1, 1, 1), api.OP_DGRAD)
        assert e.value.status == api.UNSUPPORTED and "multiple of 8" in e.value.reason


def test_splitk_dgrad_workspace_follows_the_largest_chunk_and_is_checked():
    p = P(5, 7, 7, 256, 1024, 3, 3, 1, 1, 1)
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=4):
        ws_img = 4 * 7 * 7 * 256 * 4
        full = api.cnhwc_workspace_size(p, api.OP_DGRAD)
        assert full == 5 * ws_img
    with api.override(variant=api.VAR_DGRAD_SPLITK, split_c=4, chunk_limit_bytes=2 * ws_img):
        assert api.cnhwc_chunk_plan(p, api.OP_DGRAD) == [2, 2, 1]
        need = api.cnhwc_workspace_size(p, api.OP_DGRAD)
        assert need == 2 * ws_img
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_dgrad(p, 0x1000000, 0x4000000, 0x8000000, 0x10000000, need - 16, None)
        assert e.value.status == api.WORKSPACE_TOO_SMALL
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_dgrad(p, 0x1000000, 0x4000000, 0x8000000, None, need, None)
        assert e.value.status == api.INVALID_ARG


def test_fwd_igemm_acceptance_and_workspace():
    """The implicit-GEMM forward takes stride-1 ungrouped problems whose padding
    leaves a non-negative rotated padding; its workspace is the transformed
    filter, independent of the batch."""
    p = P(4, 16, 16, 64, 96, 3, 3, 1, 1, 1)
    with api.override(variant=api.VAR_FWD_IGEMM):
        name, var = api.cnhwc_plan(p, api.OP_FWD)
        assert var == api.VAR_FWD_IGEMM and name.startswith("fwd_igemm_")
        assert api.cnhwc_workspace_size(p, api.OP_FWD) == 96 * 9 * 64 * 2
        assert api.cnhwc_workspace_size(dict(p, n=40), api.OP_FWD) == 96 * 9 * 64 * 2
        for bad, why in ((dict(p, stride=2), "stride 1"), (dict(p, pad_h=3), "R-1"),
                         (dict(p, groups=2), "groups")):
            with pytest.raises(api.CnhwcError) as e:
                api.cnhwc_plan(bad, api.OP_FWD)
            assert e.value.status == api.UNSUPPORTED and why in e.value.reason
        with pytest.raises(api.CnhwcError) as e:   # the workspace is required
            api.cnhwc_fwd(p, 0x1000000, 0x4000000, 0x8000000, None, 0, None)
        assert e.value.status == api.INVALID_ARG


def test_static_workspace_forward_refuses_before_any_device_call():
    """cnhwc_fwd_static_ws checks the workspace against its static array
    first: a split count whose partial sums exceed it is refused with the
    reason, without touching a device (this runs on the CPU)."""
    p = synth.WORKLOADS["c4a_splitc_fwd"]["prob"]
    with api.override(variant=api.VAR_FWD_SPLITC, split_c=64):
        assert api.cnhwc_workspace_size(p, api.OP_FWD) > api.STATIC_WS_BYTES
        with pytest.raises(api.CnhwcError) as e:
            api.cnhwc_fwd_static_ws(p, 16, 32, 48, None)
    assert e.value.status == api.WORKSPACE_TOO_SMALL and "static workspace" in e.value.reason
    # an invalid descriptor is refused by the shared validation
    with pytest.raises(api.CnhwcError) as e:
        api.cnhwc_fwd_static_ws(dict(p, groups=0), 16, 32, 48, None)
    assert e.value.status == api.INVALID_ARG
    # the default split of the workload fits the array
    assert api.cnhwc_workspace_size(p, api.OP_FWD) <= api.STATIC_WS_BYTES
