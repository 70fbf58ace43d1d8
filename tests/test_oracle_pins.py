"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin is independent of oracle.c's loops:
  * a dense-operator brute force built here, in Python, from the forward index
    relation (forward = A x, dgrad = A^T dy: dgrad is by definition the adjoint);
  * torch's CPU fp64 conv2d / conv2d_input (a library routine, cross-check only);
  * the GEMM identity of the 1x1 stride-1 dgrad ("perf(rocke/conv): add the
    pointwise fast path dgrad was missing": the tilde decomposition is the
    identity there and the offsets are m*K + k and k*C + c);
  * the adjoint inner-product identity (and, for the weight gradient, the
    same identity with the weight as the variable);
  * the rotated-filter identity of stride-1 depthwise dgrad ("feat(rocke):
    channel-packed and large-filter depthwise dgrad", Rotated-filter dgrad);
  * the textbook zero-insertion form of strided dgrad;
  * block-diagonal and channel-slice (split-C) decompositions ("feat(rocke):
    split-C and grouped LDS-halo direct conv fwd kernels");
  * closed forms (all-ones inputs count in-range taps) and impulses;
  * the per-axis output width the third page's review prints (22 vs 24).
The last test builds the oracle with deliberate mistakes and checks that every
one of them breaks at least one pin.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def P(n, h, w, c, k, r, s, stride=1, pad_h=0, pad_w=0, groups=1):
    return dict(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=stride, pad_h=pad_h,
                pad_w=pad_w, groups=groups)


def rand_operands(p, seed, op="fwd"):
    rng = np.random.default_rng(seed)
    ho, wo = oracle.out_dims(p)
    x = rng.standard_normal((p["n"], p["h"], p["w"], p["c"]))
    dy = rng.standard_normal((p["n"], ho, wo, p["k"]))
    w = rng.standard_normal((p["k"], p["r"], p["s"], p["c"] // p["groups"]))
    return x, dy, w


def dense_operator(p, w):
    """Matrix A with fwd(x) = A @ x.ravel(), filled element by element from the
    index relation: y[n,ho,wo,k] reads x[n, ho*s-ph+r, wo*s-pw+t, g*Cg+j]."""
    n_, h_, w_, c_, k_ = p["n"], p["h"], p["w"], p["c"], p["k"]
    R, S, s, ph, pw, G = p["r"], p["s"], p["stride"], p["pad_h"], p["pad_w"], p["groups"]
    Cg, Kg = c_ // G, k_ // G
    # output extent found by scanning, not by the floor formula
    ho_list = [o for o in range(h_ + 2 * ph) if o * s - ph >= -ph and o * s - ph + R - 1 <= h_ - 1 + ph]
    wo_list = [o for o in range(w_ + 2 * pw) if o * s - pw >= -pw and o * s - pw + S - 1 <= w_ - 1 + pw]
    Ho, Wo = len(ho_list), len(wo_list)
    A = np.zeros((n_ * Ho * Wo * k_, n_ * h_ * w_ * c_))
    for n, ho, wo, k in itertools.product(range(n_), range(Ho), range(Wo), range(k_)):
        row = ((n * Ho + ho) * Wo + wo) * k_ + k
        g = k // Kg
        for r, t, j in itertools.product(range(R), range(S), range(Cg)):
            hh, ww = ho * s - ph + r, wo * s - pw + t
            if 0 <= hh < h_ and 0 <= ww < w_:
                A[row, ((n * h_ + hh) * w_ + ww) * c_ + g * Cg + j] += w[k, r, t, j]
    return A, Ho, Wo


TINY = [
    P(1, 5, 6, 3, 2, 3, 3, 1, 1, 1),
    P(2, 7, 5, 4, 6, 3, 2, 2, 1, 0),
    P(1, 7, 7, 2, 3, 5, 3, 3, 2, 1),
    P(1, 6, 7, 4, 4, 2, 5, 2, 0, 2, 2),
    P(2, 5, 5, 4, 4, 3, 3, 1, 1, 1, 4),
    P(1, 7, 6, 6, 6, 4, 4, 2, 1, 3, 3),
    P(1, 4, 4, 8, 8, 1, 1, 1, 0, 0),
    P(1, 7, 7, 2, 4, 5, 5, 3, 0, 0, 2),
    P(1, 6, 5, 3, 3, 3, 1, 2, 2, 0, 3),
]


@pytest.mark.parametrize("p", TINY, ids=lambda p: "n{n}h{h}w{w}c{c}k{k}r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}".format(**p))
def test_brute_force_operator(p):
    x, dy, w = rand_operands(p, 11)
    A, Ho, Wo = dense_operator(p, w)
    assert (Ho, Wo) == oracle.out_dims(p)
    y_ref = (A @ x.ravel()).reshape(p["n"], Ho, Wo, p["k"])
    dx_ref = (A.T @ dy.ravel()).reshape(x.shape)
    np.testing.assert_allclose(oracle.conv_fwd(x, w, p), y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.conv_dgrad(dy, w, p), dx_ref, rtol=1e-12, atol=1e-12)


MEDIUM = [
    P(2, 9, 11, 8, 12, 3, 3, 1, 1, 1),
    P(2, 12, 10, 6, 4, 3, 5, 2, 1, 2),
    P(1, 13, 13, 8, 8, 7, 7, 1, 3, 3, 8),
    P(2, 10, 9, 12, 6, 2, 3, 3, 0, 1, 3),
    P(1, 16, 16, 4, 4, 9, 3, 1, 4, 1, 4),
    P(1, 8, 8, 16, 16, 1, 1, 2, 0, 0),
]


@pytest.mark.parametrize("p", MEDIUM, ids=lambda p: "h{h}w{w}c{c}k{k}r{r}s{s}st{stride}g{groups}".format(**p))
def test_torch_cpu_cross_check(p):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    x, dy, w = rand_operands(p, 12)
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)
    dyt = torch.from_numpy(dy).permute(0, 3, 1, 2)
    pad = (p["pad_h"], p["pad_w"])
    y_t = F.conv2d(xt, wt, stride=p["stride"], padding=pad, groups=p["groups"])
    dx_t = torch.nn.grad.conv2d_input(xt.shape, wt, dyt, stride=p["stride"], padding=pad,
                                      groups=p["groups"])
    np.testing.assert_allclose(oracle.conv_fwd(x, w, p), y_t.permute(0, 2, 3, 1).numpy(),
                               rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(oracle.conv_dgrad(dy, w, p), dx_t.permute(0, 2, 3, 1).numpy(),
                               rtol=1e-10, atol=1e-10)


def test_pointwise_dgrad_is_a_gemm():
    p = P(2, 6, 7, 24, 40, 1, 1)
    _, dy, w = rand_operands(p, 13)
    m = p["n"] * p["h"] * p["w"]
    ref = (dy.reshape(m, p["k"]) @ w.reshape(p["k"], p["c"])).reshape(p["n"], p["h"], p["w"], p["c"])
    np.testing.assert_allclose(oracle.conv_dgrad(dy, w, p), ref, rtol=1e-12, atol=1e-12)


ADJ = [
    P(2, 9, 8, 6, 4, 3, 3, 1, 1, 1),
    P(1, 11, 10, 4, 6, 3, 3, 2, 1, 1),
    P(1, 10, 11, 6, 6, 5, 2, 3, 2, 0, 3),
    P(2, 8, 8, 8, 8, 7, 7, 1, 3, 3, 8),
    P(1, 9, 12, 4, 8, 4, 6, 2, 3, 1, 2),
    P(1, 12, 12, 5, 5, 13, 3, 1, 6, 1, 5),
]


@pytest.mark.parametrize("p", ADJ, ids=lambda p: "r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}".format(**p))
def test_adjoint_identity(p):
    x, dy, w = rand_operands(p, 14)
    lhs = np.vdot(oracle.conv_fwd(x, w, p), dy)
    rhs = np.vdot(x, oracle.conv_dgrad(dy, w, p))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


ROT = [
    P(2, 9, 10, 5, 5, 3, 3, 1, 1, 1, 5),
    P(1, 12, 11, 4, 4, 7, 7, 1, 3, 3, 4),
    P(1, 16, 16, 3, 3, 13, 5, 1, 6, 2, 3),
    P(1, 14, 14, 2, 2, 5, 13, 1, 2, 6, 2),
    P(1, 10, 10, 3, 3, 7, 5, 1, 1, 4, 3),
    P(1, 9, 9, 2, 2, 5, 5, 1, 4, 0, 2),
]


@pytest.mark.parametrize("p", ROT, ids=lambda p: "r{r}s{s}p{pad_h}x{pad_w}".format(**p))
def test_depthwise_dgrad_is_rotated_forward(p):
    """Stride-1 depthwise dgrad equals forward correlation of dY with the filter
    turned by 180 degrees, at padding R-1-pad_h rows and S-1-pad_w columns."""
    _, dy, w = rand_operands(p, 15)
    ho, wo = oracle.out_dims(p)
    q = P(p["n"], ho, wo, p["c"], p["c"], p["r"], p["s"], 1, p["r"] - 1 - p["pad_h"],
          p["s"] - 1 - p["pad_w"], p["c"])
    assert oracle.out_dims(q) == (p["h"], p["w"])
    rot = w[:, ::-1, ::-1, :]
    np.testing.assert_allclose(oracle.conv_dgrad(dy, w, p), oracle.conv_fwd(dy, rot, q),
                               rtol=1e-12, atol=1e-12)


ZI = [
    P(2, 9, 9, 4, 6, 3, 3, 2, 1, 1),
    P(1, 10, 11, 3, 5, 3, 3, 2, 1, 1),
    P(1, 13, 12, 2, 3, 5, 3, 3, 2, 1),
    P(1, 8, 9, 4, 4, 4, 2, 2, 1, 0),
]


@pytest.mark.parametrize("p", ZI, ids=lambda p: "h{h}w{w}r{r}s{s}st{stride}".format(**p))
def test_strided_dgrad_is_zero_inserted_correlation(p):
    """Stride-s dgrad = stride-1 correlation of dY with s-1 zeros inserted between
    pixels, padded by R-1-pad_h on top and R-1-pad_h+((H+2pad_h-R) mod s) below
    (likewise for columns), with the rotated filter and its two channel axes swapped."""
    _, dy, w = rand_operands(p, 16)
    ho, wo = oracle.out_dims(p)
    s, R, S = p["stride"], p["r"], p["s"]
    eh = (p["h"] + 2 * p["pad_h"] - R) % s
    ew = (p["w"] + 2 * p["pad_w"] - S) % s
    top, left = R - 1 - p["pad_h"], S - 1 - p["pad_w"]
    up = np.zeros((p["n"], (ho - 1) * s + 1 + 2 * top + eh, (wo - 1) * s + 1 + 2 * left + ew, p["k"]))
    up[:, top:top + (ho - 1) * s + 1:s, left:left + (wo - 1) * s + 1:s, :] = dy
    w_t = np.ascontiguousarray(w[:, ::-1, ::-1, :].transpose(3, 1, 2, 0))  # [C,R,S,K]
    q = P(p["n"], up.shape[1], up.shape[2], p["k"], p["c"], R, S, 1, 0, 0)
    assert oracle.out_dims(q) == (p["h"], p["w"])
    np.testing.assert_allclose(oracle.conv_dgrad(dy, w, p), oracle.conv_fwd(up, w_t, q),
                               rtol=1e-12, atol=1e-12)


def _block_diag(w, p):
    G, Cg, Kg = p["groups"], p["c"] // p["groups"], p["k"] // p["groups"]
    big = np.zeros((p["k"], p["r"], p["s"], p["c"]))
    for g in range(G):
        big[g * Kg:(g + 1) * Kg, :, :, g * Cg:(g + 1) * Cg] = w[g * Kg:(g + 1) * Kg]
    return big


@pytest.mark.parametrize("p", [P(2, 8, 8, 16, 16, 3, 3, 1, 1, 1, 4),
                               P(1, 9, 7, 12, 6, 3, 3, 2, 1, 1, 3),
                               P(1, 7, 7, 6, 6, 5, 5, 1, 2, 2, 6)],
                         ids=["g4", "g3s2", "dw"])
def test_grouped_is_block_diagonal(p):
    x, dy, w = rand_operands(p, 17)
    q = dict(p, groups=1)
    big = _block_diag(w, p)
    np.testing.assert_allclose(oracle.conv_fwd(x, w, p), oracle.conv_fwd(x, big, q),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.conv_dgrad(dy, w, p), oracle.conv_dgrad(dy, big, q),
                               rtol=1e-12, atol=1e-12)


def test_split_channels_sum_to_forward():
    p = P(2, 7, 7, 32, 8, 3, 3, 1, 1, 1)
    x, _, w = rand_operands(p, 18)
    total = np.zeros_like(oracle.conv_fwd(x, w, p))
    for lo in range(0, 32, 8):
        q = dict(p, c=8)
        total += oracle.conv_fwd(x[..., lo:lo + 8], w[..., lo:lo + 8], q)
    np.testing.assert_allclose(oracle.conv_fwd(x, w, p), total, rtol=1e-12, atol=1e-12)


def _fwd_tap_count(o, s, pad, R, size):
    lo = o * s - pad
    return max(0, min(R, size - lo) - max(0, -lo))


def _dgrad_tap_count(i, s, pad, R, out):
    lo, hi = max(i + pad - R + 1, 0), min(i + pad, (out - 1) * s)
    if hi < lo:
        return 0
    return hi // s - (lo + s - 1) // s + 1


@pytest.mark.parametrize("p", [P(1, 9, 10, 6, 4, 3, 3, 1, 1, 1),
                               P(2, 11, 9, 4, 6, 5, 3, 2, 2, 1, 2),
                               P(1, 10, 10, 3, 3, 7, 7, 3, 3, 3, 3),
                               P(1, 12, 8, 2, 2, 13, 5, 1, 6, 2, 2)],
                         ids=["s1", "s2g2", "s3dw", "tall"])
def test_all_ones_closed_forms(p):
    ho, wo = oracle.out_dims(p)
    Cg, Kg = p["c"] // p["groups"], p["k"] // p["groups"]
    w = np.ones((p["k"], p["r"], p["s"], Cg))
    y = oracle.conv_fwd(np.ones((p["n"], p["h"], p["w"], p["c"])), w, p)
    for a, b in itertools.product(range(ho), range(wo)):
        want = Cg * _fwd_tap_count(a, p["stride"], p["pad_h"], p["r"], p["h"]) * \
            _fwd_tap_count(b, p["stride"], p["pad_w"], p["s"], p["w"])
        assert np.all(y[:, a, b, :] == want)
    dx = oracle.conv_dgrad(np.ones((p["n"], ho, wo, p["k"])), w, p)
    for a, b in itertools.product(range(p["h"]), range(p["w"])):
        want = Kg * _dgrad_tap_count(a, p["stride"], p["pad_h"], p["r"], ho) * \
            _dgrad_tap_count(b, p["stride"], p["pad_w"], p["s"], wo)
        assert np.all(dx[:, a, b, :] == want)


def test_impulses_fix_orientation_and_offsets():
    p = P(1, 9, 8, 4, 6, 3, 5, 2, 1, 2, 2)
    ho, wo = oracle.out_dims(p)
    Cg, Kg = 2, 3
    w = np.random.default_rng(19).standard_normal((6, 3, 5, Cg))
    h0, w0, c0 = 4, 3, 3
    x = np.zeros((1, 9, 8, 4))
    x[0, h0, w0, c0] = 1.0
    y = oracle.conv_fwd(x, w, p)
    for a, b, k in itertools.product(range(ho), range(wo), range(6)):
        r, t = h0 - a * 2 + 1, w0 - b * 2 + 2
        inside = 0 <= r < 3 and 0 <= t < 5 and k // Kg == c0 // Cg
        assert y[0, a, b, k] == (w[k, r, t, c0 % Cg] if inside else 0.0)
    a0, b0, k0 = 2, 1, 4
    dy = np.zeros((1, ho, wo, 6))
    dy[0, a0, b0, k0] = 1.0
    dx = oracle.conv_dgrad(dy, w, p)
    for hh, ww, c in itertools.product(range(9), range(8), range(4)):
        r, t = hh - (a0 * 2 - 1), ww - (b0 * 2 - 2)
        inside = 0 <= r < 3 and 0 <= t < 5 and c // Cg == k0 // Kg
        assert dx[0, hh, ww, c] == (w[k0, r, t, c % Cg] if inside else 0.0)


def test_per_axis_width_from_the_pages():
    with open(os.path.join(GOLDEN, "per_axis_padding_wo.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        p = P(1, 8, case["w"], 1, 1, 3, case["s"], case["stride"], case["pad"], case["pad_w"])
        assert oracle.out_dims(p)[1] == case["wo"]
        q = dict(p, pad_w=case["pad"])
        assert oracle.out_dims(q)[1] == case["wo_if_pad_used"]


def weight_operator(p, x):
    """Matrix B with fwd(x, w) = B @ w.ravel() for the fixed input x, filled
    from the same forward index relation as dense_operator, with the roles of
    x and w exchanged: the weight gradient is then B^T dy."""
    n_, h_, w_, c_, k_ = p["n"], p["h"], p["w"], p["c"], p["k"]
    R, S, s, ph, pw, G = p["r"], p["s"], p["stride"], p["pad_h"], p["pad_w"], p["groups"]
    Cg, Kg = c_ // G, k_ // G
    Ho, Wo = oracle.out_dims(p)
    B = np.zeros((n_ * Ho * Wo * k_, k_ * R * S * Cg))
    for n, ho, wo, k in itertools.product(range(n_), range(Ho), range(Wo), range(k_)):
        row = ((n * Ho + ho) * Wo + wo) * k_ + k
        g = k // Kg
        for r, t, j in itertools.product(range(R), range(S), range(Cg)):
            hh, ww = ho * s - ph + r, wo * s - pw + t
            if 0 <= hh < h_ and 0 <= ww < w_:
                B[row, ((k * R + r) * S + t) * Cg + j] += x[n, hh, ww, g * Cg + j]
    return B


@pytest.mark.parametrize("p", TINY, ids=lambda p: "h{h}w{w}c{c}k{k}r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}".format(**p))
def test_wgrad_matches_weight_operator_transpose(p):
    """Brute force: wgrad(x, dy) = B(x)^T dy, with B built here element by element."""
    x, dy, _ = rand_operands(p, 15)
    B = weight_operator(p, x)
    ref = (B.T @ dy.ravel()).reshape(p["k"], p["r"], p["s"], p["c"] // p["groups"])
    np.testing.assert_allclose(oracle.conv_wgrad(x, dy, p), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("p", ADJ + [TINY[3], TINY[7]], ids=lambda p: "r{r}s{s}st{stride}p{pad_h}x{pad_w}g{groups}".format(**p))
def test_wgrad_adjoint_identity(p):
    """wgrad is the weight gradient of the forward map: for every weight w,
    <fwd(x, w), dy> = <w, wgrad(x, dy)> (the forward map is linear in w).
    Three random weights pin three independent functionals."""
    x, dy, _ = rand_operands(p, 16)
    dw = oracle.conv_wgrad(x, dy, p)
    rng = np.random.default_rng(17)
    for _ in range(3):
        w = rng.standard_normal(dw.shape)
        lhs = np.vdot(oracle.conv_fwd(x, w, p), dy)
        rhs = np.vdot(w, dw)
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_pointwise_wgrad_is_a_gemm():
    """1x1 stride 1: dW[k, c] = sum over pixels of dY[m, k] x[m, c] = (dY^T X)[k, c]."""
    p = P(2, 6, 7, 24, 40, 1, 1)
    x, dy, _ = rand_operands(p, 18)
    m = p["n"] * p["h"] * p["w"]
    ref = (dy.reshape(m, p["k"]).T @ x.reshape(m, p["c"])).reshape(p["k"], 1, 1, p["c"])
    np.testing.assert_allclose(oracle.conv_wgrad(x, dy, p), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("p", MEDIUM, ids=lambda p: "h{h}w{w}c{c}k{k}r{r}s{s}st{stride}g{groups}".format(**p))
def test_wgrad_torch_cpu_cross_check(p):
    torch = pytest.importorskip("torch")
    x, dy, w = rand_operands(p, 19)
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    dyt = torch.from_numpy(dy).permute(0, 3, 1, 2)
    wshape = (p["k"], p["c"] // p["groups"], p["r"], p["s"])
    dw_t = torch.nn.grad.conv2d_weight(xt, wshape, dyt, stride=p["stride"],
                                       padding=(p["pad_h"], p["pad_w"]), groups=p["groups"])
    np.testing.assert_allclose(oracle.conv_wgrad(x, dy, p), dw_t.permute(0, 2, 3, 1).numpy(),
                               rtol=1e-10, atol=1e-10)


def test_refuses_invalid_descriptors():
    bad = [P(1, 4, 4, 4, 4, 3, 3, groups=0), P(1, 4, 4, 4, 4, 3, 3, groups=-4),
           P(1, 4, 4, 6, 4, 3, 3, groups=4), P(1, 4, 4, 4, 4, 3, 3, stride=0),
           P(1, 2, 2, 4, 4, 5, 5), P(1, 4, 4, 4, 4, 3, 3, pad_h=-1)]
    for p in bad:
        with pytest.raises(ValueError):
            oracle.out_dims(p)


# ---- every planted oracle mistake must break at least one pin ------------------

def _pins_hold(mutation):
    """Compact re-run of the independent pins against a (possibly mutated) oracle."""
    for p in [TINY[1], TINY[3], TINY[5], P(1, 6, 6, 4, 4, 3, 3, 1, 1, 0, 1)]:
        x, dy, w = rand_operands(p, 21)
        A, Ho, Wo = dense_operator(p, w)
        y = oracle.conv_fwd(x, w, p, mutation=mutation)
        dx = oracle.conv_dgrad(dy, w, p, mutation=mutation)
        if not np.allclose(y, (A @ x.ravel()).reshape(y.shape), rtol=1e-12, atol=1e-12):
            return False
        if not np.allclose(dx, (A.T @ dy.ravel()).reshape(dx.shape), rtol=1e-12, atol=1e-12):
            return False
        # weight gradient: <A(w) x, dy> is linear in w with coefficients wgrad(x, dy)
        dw = oracle.conv_wgrad(x, dy, p, mutation=mutation)
        if not np.isclose(np.vdot(y, dy), np.vdot(w, dw), rtol=1e-12, atol=1e-12):
            return False
    return True


def test_pins_catch_planted_mistakes():
    assert _pins_hold(0)
    for m in range(1, 8):
        assert not _pins_hold(m), "planted mistake %d went unnoticed" % m
