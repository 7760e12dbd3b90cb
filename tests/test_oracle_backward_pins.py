"""Pins of the oracle's DCNv3/v4 core backward to things other than itself (CPU only).

The pages print no backward pass; the oracle's gradients are the derivative of
the forward sum (grouped deformable sampling, DCNv4-in-YOLOv11 page, section
1.1; bilinear kernel, hands-on DCNv1 page, section 2). They are checked here
against:
  * brute force: the forward is linear in x, so grad_x[i] = <grad_out, F(e_i)>;
  * one-sided finite differences of the (pinned) forward in the offsets: inside
    one bilinear cell the sample is affine in each coordinate, so a step that
    stays in the cell gives the right derivative exactly (integer positions
    and out-of-image corners included);
  * finite differences in the modulation (exact without softmax, central with);
  * torch autograd through an independent fp64 formulation built on
    grid_sample (align_corners=True, zero padding), at non-integer positions;
  * zero offsets and unit modulation: autograd of a depthwise box conv2d and
    unfold;
  * softmax invariants (logit gradients sum to zero, shift invariance).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

f64 = torch.float64


def _case(seed, N, H, W, G, C, kh, kw, stride, pad, dil, grid=None, spread=1.5, mask=True):
    """Random x, offsets, modulation, grad_out. With grid=q the offsets are
    multiples of 1/q (fp32-exact, so scaled positions are exact too)."""
    r = np.random.default_rng(seed)
    Ho = oracle.out_size(H, kh, stride[0], pad[0], dil[0])
    Wo = oracle.out_size(W, kw, stride[1], pad[1], dil[1])
    K = kh * kw
    x = r.standard_normal((N, H, W, G * C))
    if grid:
        off = np.round(r.uniform(-spread * 2, spread * 2, (N, Ho, Wo, G, K, 2)) * grid) / grid
    else:
        off = r.standard_normal((N, Ho, Wo, G, K, 2)).astype(np.float32).astype(np.float64) * spread
    m = r.standard_normal((N, Ho, Wo, G, K)) if mask else None
    go = r.standard_normal((N, Ho, Wo, G * C))
    return x, off, m, go, (Ho, Wo)


def _fwd(x, off, m, kh, kw, stride, pad, dil, s, softmax):
    return oracle.dcn_core(x, off, m, kh=kh, kw=kw, stride=stride, pad=pad, dil=dil,
                           offset_scale=s, softmax=softmax)[0]


def _per_pair(go, out, G):
    """sum over each group's channels of grad_out * out -> [N,Ho,Wo,G]."""
    N, Ho, Wo, GC = go.shape
    return (go * out).reshape(N, Ho, Wo, G, GC // G).sum(-1)


SHAPES = [
    # N, H, W, G, C, kh, kw, stride, pad, dil
    (1, 4, 5, 2, 2, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 5, 4, 1, 3, 2, 3, (2, 1), (0, 2), (2, 1)),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("softmax", [False, True])
def test_grad_x_brute_force(shape, softmax):
    N, H, W, G, C, kh, kw, st, pd, dl = shape
    x, off, m, go, _ = _case(1, N, H, W, G, C, kh, kw, st, pd, dl)
    s = 1.0
    g = oracle.dcn_core_backward(x, off, m, go, kh=kh, kw=kw, stride=st, pad=pd, dil=dl,
                                 offset_scale=s, softmax=softmax)
    want = np.zeros_like(x)
    for i in range(x.size):
        e = np.zeros(x.size)
        e[i] = 1.0
        out = _fwd(e.reshape(x.shape), off, m, kh, kw, st, pd, dl, s, softmax)
        want.reshape(-1)[i] = (go * out).sum()
    assert np.abs(g["grad_x"] - want).max() <= 1e-12 * (1 + np.abs(want).max())
    assert np.all(g["grad_x_abs"] >= np.abs(g["grad_x"]) - 1e-12)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("s", [1.0, 0.5, 2.0])
@pytest.mark.parametrize("softmax", [False, True])
def test_grad_offset_one_sided_fd(shape, s, softmax):
    N, H, W, G, C, kh, kw, st, pd, dl = shape
    # positions on a 1/64 grid: many integer positions, cell edges and image borders
    x, off, m, go, _ = _case(2, N, H, W, G, C, kh, kw, st, pd, dl, grid=64, spread=2.0)
    g = oracle.dcn_core_backward(x, off, m, go, kh=kh, kw=kw, stride=st, pad=pd, dil=dl,
                                 offset_scale=s, softmax=softmax)
    base = _fwd(x, off, m, kh, kw, st, pd, dl, s, softmax)
    h = 2.0 ** -10 / s  # the position moves by 2^-10: stays inside its cell
    K = kh * kw
    for k in range(K):
        for comp in range(2):
            o2 = off.copy()
            o2[..., k, comp] += h
            fd = _per_pair(go, _fwd(x, o2, m, kh, kw, st, pd, dl, s, softmax) - base, G) / h
            got = g["grad_offset"][..., k, comp]
            tol = 1e-9 * (1 + g["grad_offset_abs"][..., k, comp])
            assert np.all(np.abs(got - fd) <= tol), (k, comp, np.abs(got - fd).max())


def test_grad_offset_integer_position_is_right_derivative():
    """At an integer position the derivative is the forward difference of the
    image (the cell to the right/below), times modulation and offset_scale."""
    H, W, C = 4, 5, 3
    r = np.random.default_rng(3)
    x = r.standard_normal((1, H, W, C))
    off = np.zeros((1, H, W, 1, 1, 2))
    m = r.standard_normal((1, H, W, 1, 1))
    go = r.standard_normal((1, H, W, C))
    g = oracle.dcn_core_backward(x, off, m, go, kh=1, kw=1, offset_scale=0.5)
    X = np.pad(x[0], ((0, 1), (0, 1), (0, 0)))  # zero beyond the last row/column
    ddx = X[:H, 1:W + 1] - X[:H, :W]
    ddy = X[1:H + 1, :W] - X[:H, :W]
    want_x = 0.5 * m[0, :, :, 0, 0] * (go[0] * ddx).sum(-1)
    want_y = 0.5 * m[0, :, :, 0, 0] * (go[0] * ddy).sum(-1)
    np.testing.assert_allclose(g["grad_offset"][0, :, :, 0, 0, 0], want_x, rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["grad_offset"][0, :, :, 0, 0, 1], want_y, rtol=0, atol=1e-13)


@pytest.mark.parametrize("shape", SHAPES)
def test_grad_offset_scale_not_power_of_two(shape):
    """offset_scale 0.3: the fp32 rounding of the scaled offset perturbs the
    difference quotient by ~1e-4 relative; the derivative carries the factor s."""
    N, H, W, G, C, kh, kw, st, pd, dl = shape
    x, off, m, go, _ = _case(4, N, H, W, G, C, kh, kw, st, pd, dl)
    s = 0.3
    g = oracle.dcn_core_backward(x, off, m, go, kh=kh, kw=kw, stride=st, pad=pd, dil=dl,
                                 offset_scale=s, softmax=False)
    h = 1e-3
    for k in range(kh * kw):
        for comp in range(2):
            o1, o2 = off.copy(), off.copy()
            o1[..., k, comp] += h
            o2[..., k, comp] -= h
            fd = _per_pair(go, _fwd(x, o1, m, kh, kw, st, pd, dl, s, False)
                           - _fwd(x, o2, m, kh, kw, st, pd, dl, s, False), G) / (2 * h)
            got = g["grad_offset"][..., k, comp]
            # random positions: a cell edge inside [d-h, d+h] is improbable but
            # possible; require agreement on nearly all pairs
            ok = np.abs(got - fd) <= 2e-3 * (1 + g["grad_offset_abs"][..., k, comp])
            assert ok.mean() > 0.97, (k, comp)


@pytest.mark.parametrize("shape", SHAPES)
def test_grad_mask_linear_and_softmax_fd(shape):
    N, H, W, G, C, kh, kw, st, pd, dl = shape
    x, off, m, go, _ = _case(5, N, H, W, G, C, kh, kw, st, pd, dl)
    K = kh * kw
    for softmax in (False, True):
        g = oracle.dcn_core_backward(x, off, m, go, kh=kh, kw=kw, stride=st, pad=pd, dil=dl,
                                     softmax=softmax)
        for k in range(K):
            if softmax:  # central difference in the logit, error O(h^2)
                h = 1e-5
                m1, m2 = m.copy(), m.copy()
                m1[..., k] += h
                m2[..., k] -= h
                fd = _per_pair(go, _fwd(x, off, m1, kh, kw, st, pd, dl, 1.0, True)
                               - _fwd(x, off, m2, kh, kw, st, pd, dl, 1.0, True), G) / (2 * h)
                tol = 1e-7 * (1 + g["grad_mask_abs"][..., k])
            else:  # the output is linear in the modulation: a unit step is exact
                m1 = m.copy()
                m1[..., k] += 1.0
                fd = _per_pair(go, _fwd(x, off, m1, kh, kw, st, pd, dl, 1.0, False)
                               - _fwd(x, off, m, kh, kw, st, pd, dl, 1.0, False), G)
                tol = 1e-11 * (1 + g["grad_mask_abs"][..., k])
            assert np.all(np.abs(g["grad_mask"][..., k] - fd) <= tol), (softmax, k)


def _torch_core(x, off, m, G, kh, kw, stride, pad, dil, s, softmax):
    """Independent fp64 formulation: one grid_sample per kernel point.
    x [N,H,W,G*C], off [N,Ho,Wo,G,K,2] ((dx, dy) pairs), m [N,Ho,Wo,G,K]."""
    N, H, W, GC = x.shape
    C = GC // G
    _, Ho, Wo, _, K, _ = off.shape
    img = x.reshape(N, H, W, G, C).permute(0, 3, 4, 1, 2).reshape(N * G, C, H, W)
    wgt = torch.softmax(m, -1) if softmax else m
    wgt = wgt.permute(0, 3, 1, 2, 4).reshape(N * G, Ho, Wo, K)
    o = off.permute(0, 3, 1, 2, 4, 5).reshape(N * G, Ho, Wo, K, 2)
    ys = (torch.arange(Ho, dtype=f64) * stride[0] - pad[0]).view(1, Ho, 1)
    xs = (torch.arange(Wo, dtype=f64) * stride[1] - pad[1]).view(1, 1, Wo)
    out = 0
    for i in range(kh):
        for j in range(kw):
            k = i * kw + j
            py = ys + i * dil[0] + s * o[..., k, 1]
            px = xs + j * dil[1] + s * o[..., k, 0]
            grid = torch.stack([2 * px / (W - 1) - 1, 2 * py / (H - 1) - 1], -1)
            smp = F.grid_sample(img, grid, mode="bilinear", padding_mode="zeros",
                                align_corners=True)  # [N*G, C, Ho, Wo]
            out = out + smp * wgt[..., k].unsqueeze(1)
    return out.reshape(N, G, C, Ho, Wo).permute(0, 3, 4, 1, 2).reshape(N, Ho, Wo, GC)


AUTOGRAD = [
    # N, H, W, G, C, kh, kw, stride, pad, dil, s, softmax
    (1, 6, 7, 2, 3, 3, 3, (1, 1), (1, 1), (1, 1), 1.0, False),
    (2, 5, 6, 3, 2, 3, 3, (1, 1), (1, 1), (1, 1), 0.5, True),
    (1, 7, 6, 1, 4, 3, 2, (2, 1), (2, 0), (2, 2), 0.25, False),
    (1, 4, 4, 2, 1, 1, 1, (1, 1), (0, 0), (1, 1), 1.0, True),
]


@pytest.mark.parametrize("case", AUTOGRAD)
def test_matches_autograd_of_grid_sample_formulation(case):
    N, H, W, G, C, kh, kw, st, pd, dl, s, softmax = case
    x, off, m, go, _ = _case(6, N, H, W, G, C, kh, kw, st, pd, dl, spread=2.0)
    tx = torch.tensor(x, requires_grad=True)
    to = torch.tensor(off, requires_grad=True)
    tm = torch.tensor(m, requires_grad=True)
    out = _torch_core(tx, to, tm, G, kh, kw, st, pd, dl, s, softmax)
    # the forward itself agrees (scaled offsets are fp32-exact here)
    ref = _fwd(x, off, m, kh, kw, st, pd, dl, s, softmax)
    np.testing.assert_allclose(out.detach().numpy(), ref, rtol=0, atol=1e-12)
    out.backward(torch.tensor(go))
    g = oracle.dcn_core_backward(x, off, m, go, kh=kh, kw=kw, stride=st, pad=pd, dil=dl,
                                 offset_scale=s, softmax=softmax)
    for name, t in (("grad_x", tx), ("grad_offset", to), ("grad_mask", tm)):
        d = np.abs(g[name] - t.grad.numpy())
        assert np.all(d <= 1e-10 * (1 + g[name + "_abs"])), (name, d.max())


@pytest.mark.parametrize("st,pd,dl", [((1, 1), (1, 1), (1, 1)), ((2, 2), (1, 0), (1, 2))])
def test_zero_offsets_unit_mask_is_box_conv_backward(st, pd, dl):
    N, H, W, G, C, kh, kw = 2, 6, 5, 2, 3, 3, 3
    r = np.random.default_rng(7)
    x = r.standard_normal((N, H, W, G * C))
    Ho, Wo = oracle.out_size(H, kh, st[0], pd[0], dl[0]), oracle.out_size(W, kw, st[1], pd[1], dl[1])
    off = np.zeros((N, Ho, Wo, G, kh * kw, 2))
    go = r.standard_normal((N, Ho, Wo, G * C))
    g = oracle.dcn_core_backward(x, off, None, go, kh=kh, kw=kw, stride=st, pad=pd, dil=dl, G=G)
    tx = torch.tensor(x).permute(0, 3, 1, 2).contiguous().requires_grad_(True)
    out = F.conv2d(tx, torch.ones(G * C, 1, kh, kw, dtype=f64), stride=st, padding=pd,
                   dilation=dl, groups=G * C)
    out.backward(torch.tensor(go).permute(0, 3, 1, 2))
    np.testing.assert_allclose(g["grad_x"], tx.grad.permute(0, 2, 3, 1).numpy(), rtol=0,
                               atol=1e-12)
    # modulation gradient: per tap, the group's channels of grad_out dotted with
    # the unfolded input
    cols = F.unfold(torch.tensor(x).permute(0, 3, 1, 2), (kh, kw), dilation=dl, padding=pd,
                    stride=st).reshape(N, G, C, kh * kw, Ho, Wo).numpy()
    want = np.einsum("nhwgc,ngckhw->nhwgk", go.reshape(N, Ho, Wo, G, C), cols)
    np.testing.assert_allclose(g["grad_mask"], want, rtol=0, atol=1e-12)


def test_softmax_logit_gradients_sum_to_zero_and_shift_invariant():
    x, off, m, go, _ = _case(8, 1, 5, 5, 2, 3, 3, 3, (1, 1), (1, 1), (1, 1))
    kw = dict(kh=3, kw=3, pad=(1, 1), softmax=True)
    g = oracle.dcn_core_backward(x, off, m, go, **kw)
    assert np.abs(g["grad_mask"].sum(-1)).max() <= 1e-12 * (1 + g["grad_mask_abs"].sum(-1).max())
    g2 = oracle.dcn_core_backward(x, off, m + 3.75, go, **kw)
    for name in ("grad_x", "grad_offset", "grad_mask"):
        np.testing.assert_allclose(g2[name], g[name], rtol=0, atol=1e-12)


def test_null_mask_means_unit_modulation_or_zero_logits():
    x, off, m, go, _ = _case(9, 1, 5, 4, 2, 2, 3, 3, (1, 1), (1, 1), (1, 1))
    kw = dict(kh=3, kw=3, pad=(1, 1))
    ones = np.ones_like(m)
    for softmax, ref in ((False, ones), (True, 0 * ones)):
        a = oracle.dcn_core_backward(x, off, None, go, softmax=softmax, G=2, **kw)
        b = oracle.dcn_core_backward(x, off, ref, go, softmax=softmax, **kw)
        for name in ("grad_x", "grad_offset", "grad_mask"):
            np.testing.assert_array_equal(a[name], b[name])


def test_gradients_are_linear_in_grad_out_and_zero_for_zero_mask():
    x, off, m, go, _ = _case(10, 1, 5, 6, 2, 2, 3, 3, (1, 1), (1, 1), (1, 1))
    kw = dict(kh=3, kw=3, pad=(1, 1))
    a = oracle.dcn_core_backward(x, off, m, go, **kw)
    b = oracle.dcn_core_backward(x, off, m, -2.0 * go, **kw)
    for name in ("grad_x", "grad_offset", "grad_mask"):
        np.testing.assert_allclose(b[name], -2.0 * a[name], rtol=0, atol=1e-12)
    z = oracle.dcn_core_backward(x, off, 0 * m, go, **kw)
    assert not z["grad_x"].any() and not z["grad_offset"].any()
    np.testing.assert_array_equal(z["grad_mask"], a["grad_mask"])


def test_degenerate_shapes():
    # 1x1 kernel, zero offsets: identity map, so grad_x = grad_out * m
    r = np.random.default_rng(11)
    x = r.standard_normal((1, 3, 4, 2))
    m = r.standard_normal((1, 3, 4, 2, 1))
    go = r.standard_normal((1, 3, 4, 2))
    g = oracle.dcn_core_backward(x, np.zeros((1, 3, 4, 2, 1, 2)), m, go, kh=1, kw=1)
    np.testing.assert_allclose(g["grad_x"], go * m[..., 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(g["grad_mask"][..., 0], go * x, rtol=0, atol=1e-15)
    # empty batch
    e = oracle.dcn_core_backward(np.zeros((0, 3, 4, 2)), np.zeros((0, 3, 4, 2, 1, 2)),
                                 None, np.zeros((0, 3, 4, 2)), kh=1, kw=1)
    assert e["grad_x"].shape == (0, 3, 4, 2)
    # every tap far outside: all gradients zero
    off = np.full((1, 3, 4, 2, 1, 2), 100.0)
    g = oracle.dcn_core_backward(x, off, m, go, kh=1, kw=1)
    assert not g["grad_x"].any() and not g["grad_offset"].any() and not g["grad_mask"].any()
