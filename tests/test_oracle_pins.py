"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against what the pages and the mathematics fix:
the lattice definition of the bilinear kernel, standard convolution and
unfold (zero offsets), exact shifts (integer offsets), exact reproduction of
bilinear (affine-in-each-axis) ramps, partition of unity, softmax invariances,
torch's grid_sample (aggregation coordinate convention), linearity and the
degenerate shapes. No expected value here comes from the GPU library.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl

f64 = torch.float64


def lattice_bilinear(X, y, x):
    """sum over every pixel q of G(q, p) X(q), with G(q,p) = g(qx,px) g(qy,py) and
    g(a,b) = max(0, 1-|a-b|) (the bilinear kernel of the DCNv1 page, section 2)."""
    H, W = X.shape
    s = 0.0
    for qy in range(H):
        gy = max(0.0, 1.0 - abs(qy - y))
        if gy == 0.0:
            continue
        for qx in range(W):
            gx = max(0.0, 1.0 - abs(qx - x))
            s += gy * gx * X[qy, qx]
    return s


# ---------------------------------------------------------------- bilinear --

def test_bilinear_equals_lattice_sum():
    r = np.random.default_rng(7)
    X = r.standard_normal((5, 6))
    H, W = X.shape
    special_y = [-2.0, -1.0, -0.75, -0.5, 0.0, 0.25, 1.0, 2.5, H - 1.5, H - 1.0, H - 0.5, H, H + 0.2]
    special_x = [-2.0, -1.0, -0.3, 0.0, 0.5, 3.0, W - 1.25, W - 1.0, W - 0.5, W, W + 1.0]
    pts = [(y, x) for y in special_y for x in special_x]
    pts += [tuple(p) for p in r.uniform([-2, -2], [H + 1, W + 1], size=(300, 2))]
    for y, x in pts:
        v, ab = oracle.bilinear(X, y, x)
        ref = lattice_bilinear(X, y, x)
        assert abs(v - ref) <= 1e-14, (y, x, v, ref)
        assert ab >= abs(v) - 1e-15


def test_bilinear_integer_position_reads_pixel():
    X = np.arange(20, dtype=np.float64).reshape(4, 5)
    for y in range(4):
        for x in range(5):
            assert oracle.bilinear(X, y, x)[0] == X[y, x]
    assert oracle.bilinear(X, -1, 2)[0] == 0.0
    assert oracle.bilinear(X, 4, 2)[0] == 0.0
    assert oracle.bilinear(X, 1, 5)[0] == 0.0
    # halfway between two pixels: the mean
    assert oracle.bilinear(X, 1.5, 2.5)[0] == np.mean([X[1, 2], X[1, 3], X[2, 2], X[2, 3]])


def test_bilinear_weights_sum_to_one_inside():
    X = np.ones((6, 7))
    r = np.random.default_rng(3)
    for y, x in r.uniform([0, 0], [5, 6], size=(200, 2)):
        assert abs(oracle.bilinear(X, y, x)[0] - 1.0) <= 1e-15


# ------------------------------------------------------- core: zero offsets --

CONV_CASES = [
    # N, H, W, G, C, kh, kw, stride, pad, dil
    (2, 7, 9, 2, 3, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 9, 8, 1, 4, 3, 3, (2, 2), (1, 1), (1, 1)),
    (1, 10, 11, 3, 2, 3, 3, (1, 1), (2, 2), (2, 2)),
    (1, 8, 12, 2, 2, 3, 5, (1, 2), (1, 2), (1, 1)),
    (2, 6, 6, 4, 1, 3, 3, (1, 1), (0, 0), (1, 1)),
    (1, 5, 7, 1, 1, 1, 1, (1, 1), (0, 0), (1, 1)),
]


def _nchw(x):
    return torch.from_numpy(np.ascontiguousarray(x)).permute(0, 3, 1, 2).contiguous()


@pytest.mark.parametrize("N,H,W,G,C,kh,kw,s,p,d", CONV_CASES)
def test_core_zero_offsets_unit_masks_is_depthwise_box_conv(N, H, W, G, C, kh, kw, s, p, d):
    r = np.random.default_rng(11)
    x = r.standard_normal((N, H, W, G * C))
    Ho, Wo = wl.out_size(H, kh, s[0], p[0], d[0]), wl.out_size(W, kw, s[1], p[1], d[1])
    off = np.zeros((N, Ho, Wo, G, kh * kw, 2))
    out, _ = oracle.dcn_core(x, off, None, kh=kh, kw=kw, stride=s, pad=p, dil=d)
    ref = F.conv2d(_nchw(x), torch.ones(G * C, 1, kh, kw, dtype=f64), stride=s, padding=p,
                   dilation=d, groups=G * C)
    np.testing.assert_allclose(out, ref.permute(0, 2, 3, 1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,H,W,G,C,kh,kw,s,p,d", CONV_CASES)
def test_core_zero_offsets_masks_match_unfold(N, H, W, G, C, kh, kw, s, p, d):
    r = np.random.default_rng(12)
    x = r.standard_normal((N, H, W, G * C))
    Ho, Wo = wl.out_size(H, kh, s[0], p[0], d[0]), wl.out_size(W, kw, s[1], p[1], d[1])
    K = kh * kw
    off = np.zeros((N, Ho, Wo, G, K, 2))
    m = r.random((N, Ho, Wo, G, K))
    out, _ = oracle.dcn_core(x, off, m, kh=kh, kw=kw, stride=s, pad=p, dil=d)
    cols = F.unfold(_nchw(x), (kh, kw), dilation=d, padding=p, stride=s)  # [N, GC*K, L]
    cols = cols.view(N, G, C, K, Ho, Wo)
    mt = torch.from_numpy(m).permute(0, 3, 4, 1, 2).unsqueeze(2)  # [N, G, 1, K, Ho, Wo]
    ref = (cols * mt).sum(3).view(N, G * C, Ho, Wo).permute(0, 2, 3, 1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_core_softmax_zero_offsets_matches_torch_softmax():
    r = np.random.default_rng(13)
    N, H, W, G, C, kh, kw = 2, 6, 7, 3, 2, 3, 3
    K = 9
    x = r.standard_normal((N, H, W, G * C))
    off = np.zeros((N, H, W, G, K, 2))
    lg = r.standard_normal((N, H, W, G, K)) * 2
    out, _ = oracle.dcn_core(x, off, lg, kh=kh, kw=kw, pad=(1, 1), softmax=True)
    m = torch.softmax(torch.from_numpy(lg), dim=-1)
    cols = F.unfold(_nchw(x), (3, 3), padding=1).view(N, G, C, K, H, W)
    ref = (cols * m.permute(0, 3, 4, 1, 2).unsqueeze(2)).sum(3).view(N, G * C, H, W)
    np.testing.assert_allclose(out, ref.permute(0, 2, 3, 1).numpy(), rtol=0, atol=1e-12)


def test_softmax_primitive():
    r = np.random.default_rng(1)
    l = r.standard_normal(37) * 5
    m = oracle.softmax(l)
    np.testing.assert_allclose(m, torch.softmax(torch.from_numpy(l), 0).numpy(), rtol=1e-14)
    assert abs(m.sum() - 1) < 1e-14
    # large logits do not overflow (max subtraction)
    m2 = oracle.softmax(np.array([1000.0, 1000.0, 999.0]))
    assert np.all(np.isfinite(m2)) and abs(m2.sum() - 1) < 1e-15


# -------------------------------------------- core: exact closed forms ------

def _grid_base(Ho, Wo, kh, kw, s, p, d):
    """Grid base (without offsets) of every (ho, wo, k): arrays [Ho, Wo, K]."""
    ho = np.arange(Ho)[:, None, None]
    wo = np.arange(Wo)[None, :, None]
    i = (np.arange(kh * kw) // kw)[None, None, :]
    j = (np.arange(kh * kw) % kw)[None, None, :]
    by = ho * s[0] - p[0] + i * d[0]
    bx = wo * s[1] - p[1] + j * d[1]
    shape = (Ho, Wo, kh * kw)
    return np.broadcast_to(by, shape), np.broadcast_to(bx, shape)


@pytest.mark.parametrize("ramp", ["full", "x_only", "y_only"])
def test_core_reproduces_bilinear_ramps(ramp):
    """For X(h,w) = a + b*w + c*h + e*h*w bilinear sampling is exact wherever all four
    corners are inside; a ramp along one axis exposes a swapped (dx, dy) pair."""
    r = np.random.default_rng(21)
    N, H, W, G, C, kh, kw = 1, 12, 13, 2, 3, 3, 3
    s, p, d = (1, 1), (1, 1), (1, 1)
    K = 9
    a, b, c, e = (r.integers(-8, 9, size=(4, G * C)) / 8.0)
    if ramp == "x_only":
        c[:] = 0; e[:] = 0
    elif ramp == "y_only":
        b[:] = 0; e[:] = 0
    hh = np.arange(H)[:, None, None]
    ww = np.arange(W)[None, :, None]
    x = (a + b * ww + c * hh + e * hh * ww)[None]  # [1, H, W, GC]
    off = r.integers(-16, 17, size=(N, H, W, G, K, 2)) / 16.0
    m = r.integers(0, 9, size=(N, H, W, G, K)) / 8.0
    out, _ = oracle.dcn_core(x, off, m, kh=kh, kw=kw, stride=s, pad=p, dil=d)
    by, bx = _grid_base(H, W, kh, kw, s, p, d)
    yy = by[None, :, :, None, :] + off[..., 1]  # [N, Ho, Wo, G, K]
    xx = bx[None, :, :, None, :] + off[..., 0]
    inside = ((yy >= 0) & (yy <= H - 1) & (xx >= 0) & (xx <= W - 1)).all(axis=(3, 4))
    assert inside.sum() > 40
    for gi in range(G):
        for ci in range(C):
            ch = gi * C + ci
            val = a[ch] + b[ch] * xx[..., gi, :] + c[ch] * yy[..., gi, :] + e[ch] * yy[..., gi, :] * xx[..., gi, :]
            ref = (m[..., gi, :] * val).sum(-1)
            np.testing.assert_allclose(out[..., ch][inside], ref[inside], rtol=0, atol=1e-12)


def test_core_integer_offsets_are_exact_shifts():
    r = np.random.default_rng(22)
    N, H, W, G, C, kh, kw = 2, 7, 8, 2, 3, 3, 3
    s, p, d = (1, 1), (1, 1), (1, 1)
    K = 9
    x = r.integers(-4, 5, size=(N, H, W, G * C)).astype(np.float64)
    off = r.integers(-3, 4, size=(N, H, W, G, K, 2)).astype(np.float64)
    out, _ = oracle.dcn_core(x, off, None, kh=kh, kw=kw, stride=s, pad=p, dil=d)
    by, bx = _grid_base(H, W, kh, kw, s, p, d)
    ref = np.zeros_like(out)
    for n in range(N):
        for ho in range(H):
            for wo in range(W):
                for g in range(G):
                    for k in range(K):
                        yy = by[ho, wo, k] + int(off[n, ho, wo, g, k, 1])
                        xx = bx[ho, wo, k] + int(off[n, ho, wo, g, k, 0])
                        if 0 <= yy < H and 0 <= xx < W:
                            ref[n, ho, wo, g * C:(g + 1) * C] += x[n, yy, xx, g * C:(g + 1) * C]
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("softmax", [False, True])
def test_core_partition_of_unity(softmax):
    r = np.random.default_rng(23)
    N, H, W, G, C = 1, 16, 16, 3, 2
    K = 9
    x = np.ones((N, H, W, G * C))
    off = r.uniform(-1, 1, size=(N, H, W, G, K, 2))
    m = r.standard_normal((N, H, W, G, K)) if softmax else r.random((N, H, W, G, K))
    out, _ = oracle.dcn_core(x, off, m, kh=3, kw=3, pad=(1, 1), softmax=softmax)
    inner = out[:, 2:-2, 2:-2]  # every tap of these pixels is fully inside
    if softmax:
        np.testing.assert_allclose(inner, 1.0, rtol=0, atol=1e-14)
    else:
        ref = np.repeat(m.sum(-1), C, axis=-1)[:, 2:-2, 2:-2]
        np.testing.assert_allclose(inner, ref, rtol=0, atol=1e-13)


def test_core_softmax_invariances():
    r = np.random.default_rng(24)
    N, H, W, G, C = 1, 9, 10, 2, 3
    K = 9
    x = r.standard_normal((N, H, W, G * C))
    off = r.standard_normal((N, H, W, G, K, 2)) * 1.5
    lg = r.standard_normal((N, H, W, G, K))
    o1, _ = oracle.dcn_core(x, off, lg, kh=3, kw=3, pad=(1, 1), softmax=True)
    shift = r.standard_normal((N, H, W, G, 1)) * 10
    o2, _ = oracle.dcn_core(x, off, lg + shift, kh=3, kw=3, pad=(1, 1), softmax=True)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    # constant logits = the mean over the K points
    o3, _ = oracle.dcn_core(x, off, np.full_like(lg, 0.3), kh=3, kw=3, pad=(1, 1), softmax=True)
    o4, _ = oracle.dcn_core(x, off, None, kh=3, kw=3, pad=(1, 1))
    np.testing.assert_allclose(o3, o4 / K, rtol=0, atol=1e-13)


def test_core_out_of_image_taps_contribute_nothing():
    c = wl.core_case(N=2, H=9, W=11, G=2, C=3, dtype="f32", offset_std=2.0, mask="uniform",
                     oob_frac=0.3, seed=5)
    kw_ = dict(kh=3, kw=3, pad=(1, 1))
    o1, _ = oracle.dcn_core(c["x"], c["offset"], c["mask"], **kw_)
    m2 = c["mask"].clone().numpy()
    r = np.random.default_rng(0)
    m2[c["oob"]] = r.random(int(c["oob"].sum())) * 100
    o2, _ = oracle.dcn_core(c["x"], c["offset"], m2, **kw_)
    assert c["oob"].mean() > 0.2
    assert np.array_equal(o1, o2)


def test_core_linearity_and_null_mask():
    r = np.random.default_rng(25)
    N, H, W, G, C = 1, 8, 9, 2, 2
    K = 9
    x1, x2 = r.standard_normal((2, N, H, W, G * C))
    off = r.standard_normal((N, H, W, G, K, 2)) * 2
    m1, m2 = r.random((2, N, H, W, G, K))
    kw_ = dict(kh=3, kw=3, pad=(1, 1))
    o = lambda x, m: oracle.dcn_core(x, off, m, **kw_)[0]
    np.testing.assert_allclose(o(1.5 * x1 - 0.25 * x2, m1), 1.5 * o(x1, m1) - 0.25 * o(x2, m1), atol=1e-12)
    np.testing.assert_allclose(o(x1, 2 * m1 + m2), 2 * o(x1, m1) + o(x1, m2), atol=1e-12)
    assert np.array_equal(o(x1, None), o(x1, np.ones_like(m1)))


def test_core_degenerate_shapes():
    r = np.random.default_rng(26)
    # 1x1 image, 3x3 window with padding 1: only the centre tap can read the pixel
    x = r.standard_normal((1, 1, 1, 4))
    off = np.zeros((1, 1, 1, 2, 9, 2))
    m = r.random((1, 1, 1, 2, 9))
    out, _ = oracle.dcn_core(x, off, m, kh=3, kw=3, pad=(1, 1))
    ref = np.concatenate([m[0, 0, 0, 0, 4] * x[0, 0, 0, :2], m[0, 0, 0, 1, 4] * x[0, 0, 0, 2:]])
    np.testing.assert_allclose(out[0, 0, 0], ref, atol=1e-15)
    # K = 1 and zero offset: out = m * x
    x = r.standard_normal((2, 5, 6, 3))
    off = np.zeros((2, 5, 6, 3, 1, 2))
    m = r.random((2, 5, 6, 3, 1))
    out, _ = oracle.dcn_core(x, off, m, kh=1, kw=1)
    np.testing.assert_allclose(out, m[..., 0] * x, atol=1e-15)
    # a sample selection returns the same rows as the full output
    c = wl.core_case(N=2, H=6, W=7, G=2, C=2, dtype="f32", seed=9)
    full, _ = oracle.dcn_core(c["x"], c["offset"], c["mask"], kh=3, kw=3, pad=(1, 1))
    sel = [0, 5, 41, 83]
    part, _ = oracle.dcn_core(c["x"], c["offset"], c["mask"], kh=3, kw=3, pad=(1, 1), pix=sel)
    assert np.array_equal(part, full.reshape(-1, 4)[sel])


# ------------------------------------------------------------------- DCNv2 --

V2_CASES = [
    # N, Cin, H, W, Cout, kh, kw, stride, pad, dil, dg
    (2, 4, 6, 7, 5, 3, 3, (1, 1), (1, 1), (1, 1), 1),
    (1, 6, 9, 8, 3, 3, 3, (2, 2), (1, 1), (1, 1), 2),
    (1, 4, 10, 10, 2, 3, 3, (1, 1), (2, 2), (2, 2), 1),
    (1, 3, 7, 9, 4, 1, 3, (1, 1), (0, 1), (1, 1), 3),
]


@pytest.mark.parametrize("N,Cin,H,W,Cout,kh,kw,s,p,d,dg", V2_CASES)
def test_v2_zero_offsets_unit_masks_is_conv2d(N, Cin, H, W, Cout, kh, kw, s, p, d, dg):
    r = np.random.default_rng(31)
    x = r.standard_normal((N, Cin, H, W))
    w = r.standard_normal((Cout, Cin, kh, kw))
    Ho, Wo = wl.out_size(H, kh, s[0], p[0], d[0]), wl.out_size(W, kw, s[1], p[1], d[1])
    off = np.zeros((N, dg * kh * kw * 2, Ho, Wo))
    out, _ = oracle.dcn_v2(x, off, None, w, stride=s, pad=p, dil=d)
    ref = F.conv2d(torch.from_numpy(x), torch.from_numpy(w), stride=s, padding=p, dilation=d)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,Cin,H,W,Cout,kh,kw,s,p,d,dg", V2_CASES)
def test_v2_zero_offsets_masks_match_unfold(N, Cin, H, W, Cout, kh, kw, s, p, d, dg):
    r = np.random.default_rng(32)
    x = r.standard_normal((N, Cin, H, W))
    w = r.standard_normal((Cout, Cin, kh, kw))
    K = kh * kw
    Ho, Wo = wl.out_size(H, kh, s[0], p[0], d[0]), wl.out_size(W, kw, s[1], p[1], d[1])
    off = np.zeros((N, dg * K * 2, Ho, Wo))
    m = r.random((N, dg * K, Ho, Wo))
    out, _ = oracle.dcn_v2(x, off, m, w, stride=s, pad=p, dil=d)
    cols = F.unfold(torch.from_numpy(x), (kh, kw), dilation=d, padding=p, stride=s)  # [N, Cin*K, L]
    cols = cols.view(N, dg, Cin // dg, K, Ho * Wo)
    mt = torch.from_numpy(m).view(N, dg, 1, K, Ho * Wo)
    colm = (cols * mt).view(N, Cin * K, Ho * Wo)
    ref = (torch.from_numpy(w).view(Cout, Cin * K) @ colm).view(N, Cout, Ho, Wo)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)
    # the column stage on its own
    col_o = oracle.dcn_v2_columns(x, off, m, kh=kh, kw=kw, stride=s, pad=p, dil=d)
    np.testing.assert_allclose(col_o, colm.permute(0, 2, 1).reshape(-1, Cin * K).numpy(),
                               rtol=0, atol=1e-13)


def test_v2_integer_offsets_are_exact_shifts():
    r = np.random.default_rng(33)
    N, Cin, H, W, Cout = 1, 3, 6, 7, 2
    K = 9
    x = r.integers(-4, 5, size=(N, Cin, H, W)).astype(np.float64)
    w = r.integers(-2, 3, size=(Cout, Cin, 3, 3)).astype(np.float64)
    off = r.integers(-2, 3, size=(N, K * 2, H, W)).astype(np.float64)
    out, _ = oracle.dcn_v2(x, off, None, w, pad=(1, 1))
    ref = np.zeros((N, Cout, H, W))
    for ho in range(H):
        for wo in range(W):
            for ci in range(Cin):
                for k in range(K):
                    i, j = divmod(k, 3)
                    yy = ho - 1 + i + int(off[0, 2 * k + 1, ho, wo])
                    xx = wo - 1 + j + int(off[0, 2 * k, ho, wo])
                    if 0 <= yy < H and 0 <= xx < W:
                        ref[0, :, ho, wo] += w[:, ci, i, j] * x[0, ci, yy, xx]
    assert np.array_equal(out, ref)


def test_v2_ramp_and_pair_order():
    """Per-channel ramp along x only: a swapped (dx, dy) pair would read the y offset."""
    r = np.random.default_rng(34)
    N, Cin, H, W, Cout, K = 1, 2, 10, 12, 1, 9
    b = np.array([0.5, -0.25])
    x = np.broadcast_to(b[:, None, None] * np.arange(W)[None, None, :], (Cin, H, W))[None].copy()
    w = np.zeros((Cout, Cin, 3, 3))
    w[0, 0, 1, 2] = 1.0   # channel 0, tap (1, 2): k = 5
    w[0, 1, 2, 0] = 2.0   # channel 1, tap (2, 0): k = 6
    off = r.integers(-8, 9, size=(N, 2 * K, H, W)) / 8.0
    out, _ = oracle.dcn_v2(x, off, None, w, pad=(1, 1))
    wo = np.arange(W)[None, :]
    x5 = wo - 1 + 2 + off[0, 10]
    x6 = wo - 1 + 0 + off[0, 12]
    ref = 1.0 * b[0] * x5 + 2.0 * b[1] * x6
    inside = (x5 >= 0) & (x5 <= W - 1) & (x6 >= 0) & (x6 <= W - 1)
    y5 = np.arange(H)[:, None] + off[0, 11]
    y6 = np.arange(H)[:, None] + 1 + off[0, 13]
    inside &= (y5 >= 0) & (y5 <= H - 1) & (y6 >= 0) & (y6 <= H - 1)
    assert inside.sum() > 30
    np.testing.assert_allclose(out[0, 0][inside], ref[inside], rtol=0, atol=1e-12)


def test_v2_deformable_groups_split_channels():
    """With dg groups the result is the sum of dg single-group convolutions, each over
    its own channel slice with its own offsets and masks."""
    c = wl.v2_case(N=1, Cin=6, H=7, W=8, Cout=4, dg=3, dtype="f32", seed=35, mask="uniform")
    out, _ = oracle.dcn_v2(c["x"], c["offset"], c["mask"], c["weight"], pad=(1, 1))
    K = 9
    acc = np.zeros_like(out)
    for g in range(3):
        sl = slice(2 * g, 2 * g + 2)
        o_g, _ = oracle.dcn_v2(c["x"][:, sl], c["offset"][:, g * 2 * K:(g + 1) * 2 * K],
                               c["mask"][:, g * K:(g + 1) * K], c["weight"][:, sl], pad=(1, 1))
        acc += o_g
    np.testing.assert_allclose(out, acc, rtol=0, atol=1e-12)


def test_v2_mask_none_and_softmax():
    c = wl.v2_case(N=1, Cin=4, H=6, W=6, Cout=3, dg=2, dtype="f32", seed=36, mask="logits")
    o_none, _ = oracle.dcn_v2(c["x"], c["offset"], None, c["weight"], pad=(1, 1))
    o_one, _ = oracle.dcn_v2(c["x"], c["offset"], torch.ones_like(c["mask"]), c["weight"], pad=(1, 1))
    assert np.array_equal(o_none, o_one)
    o_sm, _ = oracle.dcn_v2(c["x"], c["offset"], c["mask"], c["weight"], pad=(1, 1), softmax=True)
    msm = torch.softmax(c["mask"].double().view(1, 2, 9, 6, 6), dim=2).view(1, 18, 6, 6)
    o_ref, _ = oracle.dcn_v2(c["x"], c["offset"], msm, c["weight"], pad=(1, 1))
    np.testing.assert_allclose(o_sm, o_ref, rtol=0, atol=1e-12)


def test_v2_softmax_without_mask_is_uniform_modulation():
    """softmax over the K points with no mask tensor: the implied logits are all equal,
    so every point gets 1/K. That is the unmasked result divided by K (the sum is
    linear in the modulation), and the same as passing any constant logits; with zero
    offsets it is conv2d / K."""
    c = wl.v2_case(N=2, Cin=4, H=6, W=7, Cout=3, dg=2, dtype="f32", seed=37, mask="logits")
    K = 9
    o_sm, _ = oracle.dcn_v2(c["x"], c["offset"], None, c["weight"], pad=(1, 1), softmax=True)
    o_plain, _ = oracle.dcn_v2(c["x"], c["offset"], None, c["weight"], pad=(1, 1))
    np.testing.assert_allclose(o_sm, o_plain / K, rtol=0, atol=1e-13)
    for v in (0.0, 3.7):
        o_c, _ = oracle.dcn_v2(c["x"], c["offset"], torch.full_like(c["mask"], v), c["weight"],
                               pad=(1, 1), softmax=True)
        np.testing.assert_allclose(o_sm, o_c, rtol=0, atol=1e-13)
    off0 = torch.zeros_like(c["offset"])
    o0, _ = oracle.dcn_v2(c["x"], off0, None, c["weight"], pad=(1, 1), softmax=True)
    ref = F.conv2d(c["x"].double(), c["weight"].double(), padding=1) / K
    np.testing.assert_allclose(o0, ref.numpy(), rtol=0, atol=1e-13)
    # the column stage alone
    col_sm = oracle.dcn_v2_columns(c["x"], c["offset"], None, kh=3, kw=3, pad=(1, 1), softmax=True)
    col_1 = oracle.dcn_v2_columns(c["x"], c["offset"], None, kh=3, kw=3, pad=(1, 1))
    np.testing.assert_allclose(col_sm, col_1 / K, rtol=0, atol=1e-14)


# ------------------------------------------------------------- aggregation --

def _grid_sample_maps(case, b, cam, s, u, v):
    """torch grid_sample (bilinear, zero padding, align_corners=False) of map (cam, s)
    of batch b at normalised (u, v): returns [n, G*Cg]."""
    H, W = case["spatial_shape"][cam, s]
    st = case["scale_start"][cam, s]
    fm = case["feat"][b, st:st + H * W].double().view(H, W, -1).permute(2, 0, 1)[None]
    grid = torch.stack([2 * torch.as_tensor(u, dtype=f64) - 1,
                        2 * torch.as_tensor(v, dtype=f64) - 1], -1).view(1, 1, -1, 2)
    smp = F.grid_sample(fm, grid, mode="bilinear", padding_mode="zeros", align_corners=False)
    return smp[0, :, 0, :].T.numpy()


def test_agg_single_tap_equals_grid_sample():
    c = wl.agg_case(B=1, shapes=[[(9, 13)]], A=64, pts=1, G=2, Cg=3, weights="ones", seed=41,
                    loc_lo=-0.2, loc_hi=1.2)
    # dyadic locations: u*W is exact in fp32, so the convention is checked exactly
    r = np.random.default_rng(4)
    loc = (r.integers(-128, 1153, size=(1, 64, 1, 1, 2)) / 1024.0).astype(np.float32)
    c["loc"] = torch.from_numpy(loc)
    out, ab = oracle.deform_agg(c["feat"], c["spatial_shape"], c["scale_start"], c["loc"], c["weights"])
    ref = _grid_sample_maps(c, 0, 0, 0, loc[0, :, 0, 0, 0], loc[0, :, 0, 0, 1])
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-13)
    assert np.all(ab >= np.abs(out) - 1e-15)


def test_agg_random_locations_within_fp32_coordinate_rounding():
    c = wl.agg_case(B=1, shapes=[[(31, 47)]], A=128, pts=1, G=1, Cg=4, weights="ones", seed=42)
    out, ab = oracle.deform_agg(c["feat"], c["spatial_shape"], c["scale_start"], c["loc"], c["weights"])
    u = c["loc"][0, :, 0, 0, 0].double().numpy()
    v = c["loc"][0, :, 0, 0, 1].double().numpy()
    ref = _grid_sample_maps(c, 0, 0, 0, u, v)
    # the oracle rounds u*W once to fp32 (<= 2^-19 px here); values are O(1)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-5)


@pytest.mark.parametrize("softmax", [False, True])
@pytest.mark.parametrize("cam_major", [True, False])
def test_agg_is_weighted_sum_of_grid_samples(softmax, cam_major):
    shapes = [[(6, 10), (3, 5)], [(4, 8), (2, 4)], [(5, 7), (3, 3)]]
    c = wl.agg_case(B=2, shapes=shapes, A=5, pts=3, G=2, Cg=3,
                    weights="logits" if softmax else "simplex", seed=43, cam_major=cam_major)
    r = np.random.default_rng(5)
    c["loc"] = torch.from_numpy((r.integers(-64, 1100, size=(2, 5, 3, 3, 2)) / 1024.0).astype(np.float32))
    out, _ = oracle.deform_agg(c["feat"], c["spatial_shape"], c["scale_start"], c["loc"],
                               c["weights"], softmax=softmax)
    B, A, pts, cams, scales, G, Cg = 2, 5, 3, 3, 2, 2, 3
    wts = c["weights"].double()
    if softmax:
        wts = torch.softmax(wts.view(B, A, pts * cams * scales, G), dim=2).view(B, A, pts, cams, scales, G)
    wts = wts.numpy()
    ref = np.zeros((B, A, G * Cg))
    loc = c["loc"].double().numpy()
    for b in range(B):
        for p in range(pts):
            for cam in range(cams):
                for s in range(scales):
                    smp = _grid_sample_maps(c, b, cam, s, loc[b, :, p, cam, 0], loc[b, :, p, cam, 1])
                    for g in range(G):
                        ref[b, :, g * Cg:(g + 1) * Cg] += wts[b, :, p, cam, s, g][:, None] * smp[:, g * Cg:(g + 1) * Cg]
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_agg_anchor_selection_and_linearity():
    c = wl.agg_case(B=2, shapes=[[(8, 12), (4, 6)]] * 2, A=7, pts=2, G=2, Cg=2,
                    weights="simplex", seed=44)
    args = (c["spatial_shape"], c["scale_start"], c["loc"])
    full, _ = oracle.deform_agg(c["feat"], *args, c["weights"])
    sel = [0, 3, 8, 13]
    part, _ = oracle.deform_agg(c["feat"], *args, c["weights"], anchors=sel)
    assert np.array_equal(part, full.reshape(14, -1)[sel])
    f2 = c["feat"].double() * 0.5 + 1.0
    o2, _ = oracle.deform_agg(f2, *args, c["weights"])
    o1, _ = oracle.deform_agg(torch.ones_like(f2), *args, c["weights"])
    np.testing.assert_allclose(o2, 0.5 * full + o1, atol=1e-12)


def test_agg_rejects_maps_beyond_feature_rows():
    c = wl.agg_case(B=1, shapes=[[(4, 4)]], A=2, pts=1, G=1, Cg=2, weights="ones", seed=45)
    st = c["scale_start"].copy()
    st[0, 0] = 1  # map would end one row past P_total
    with pytest.raises(ValueError):
        oracle.deform_agg(c["feat"], c["spatial_shape"], st, c["loc"], c["weights"])
