"""Pins of the oracle's aggregation backward to things other than itself (CPU only).

The Sparse4D deformable_aggregation page (section 2.1) names gradients of the
features, the sampling locations and the weights; the oracle takes them as the
derivative of the forward sum. They are checked here against brute force (the
forward is linear in the features and, without softmax, in the weights), exact
one-sided differences of the pinned forward in the locations (dyadic locations,
power-of-two maps: the step stays inside one bilinear cell), central differences
through the softmax, and torch autograd of an independent fp64 formulation built
on grid_sample (align_corners=False, zero padding).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

f64 = torch.float64


def _case(seed, B=1, A=3, pts=2, cams=2, shapes=((8, 16), (4, 8)), G=2, Cg=3, dyadic=False):
    r = np.random.default_rng(seed)
    scales = len(shapes)
    ss = np.array([[list(hw) for hw in shapes]] * cams, np.int32)
    sizes = [h * w for h, w in shapes] * cams
    st = np.cumsum([0] + sizes[:-1]).reshape(cams, scales).astype(np.int32)
    P = int(sum(sizes)) + 3
    feat = r.standard_normal((B, P, G * Cg))
    if dyadic:  # multiples of 1/256 inside (0, 1): u*W exact, fractions on a 1/64 grid
        loc = r.integers(1, 255, (B, A, pts, cams, 2)) / 256.0
    else:       # fp32 values: u*W exact for power-of-two W, positions almost never integer
        loc = r.uniform(-0.1, 1.1, (B, A, pts, cams, 2)).astype(np.float32).astype(np.float64)
    w = r.standard_normal((B, A, pts, cams, scales, G))
    go = r.standard_normal((B, A, G * Cg))
    return feat, ss, st, loc, w, go


def _fwd(feat, ss, st, loc, w, softmax):
    return oracle.deform_agg(feat, ss, st, loc, w, softmax=softmax)[0]


@pytest.mark.parametrize("softmax", [False, True])
def test_grad_feat_brute_force(softmax):
    feat, ss, st, loc, w, go = _case(1, A=2)
    g = oracle.deform_agg_backward(feat, ss, st, loc, w, go, softmax=softmax)
    want = np.zeros_like(feat)
    for i in range(feat.size):
        e = np.zeros(feat.size)
        e[i] = 1.0
        want.reshape(-1)[i] = (go * _fwd(e.reshape(feat.shape), ss, st, loc, w, softmax)).sum()
    assert np.abs(g["grad_feat"] - want).max() <= 1e-12 * (1 + np.abs(want).max())


def test_grad_weights_linear_and_softmax_fd():
    feat, ss, st, loc, w, go = _case(2)
    base = {sm: _fwd(feat, ss, st, loc, w, sm) for sm in (False, True)}
    gs = {sm: oracle.deform_agg_backward(feat, ss, st, loc, w, go, softmax=sm) for sm in (False, True)}
    for idx in np.ndindex(w.shape):
        w1 = w.copy()
        w1[idx] += 1.0  # linear without softmax: a unit step is exact
        fd = (go * (_fwd(feat, ss, st, loc, w1, False) - base[False])).sum()
        assert abs(gs[False]["grad_weights"][idx] - fd) <= 1e-11 * (1 + gs[False]["grad_weights_abs"][idx])
        h = 1e-5
        w1 = w.copy(); w1[idx] += h
        w2 = w.copy(); w2[idx] -= h
        fd = (go * (_fwd(feat, ss, st, loc, w1, True) - _fwd(feat, ss, st, loc, w2, True))).sum() / (2 * h)
        assert abs(gs[True]["grad_weights"][idx] - fd) <= 1e-7 * (1 + gs[True]["grad_weights_abs"][idx])


@pytest.mark.parametrize("softmax", [False, True])
def test_grad_loc_one_sided_fd(softmax):
    feat, ss, st, loc, w, go = _case(3, dyadic=True)
    g = oracle.deform_agg_backward(feat, ss, st, loc, w, go, softmax=softmax)
    base = _fwd(feat, ss, st, loc, w, softmax)
    h = 2.0 ** -12  # moves x by W*h <= 1/256: stays inside the cell (fractions on a 1/64 grid)
    for idx in np.ndindex(loc.shape):
        l1 = loc.copy()
        l1[idx] += h
        fd = (go * (_fwd(feat, ss, st, l1, w, softmax) - base)).sum() / h
        tol = 1e-9 * (1 + g["grad_loc_abs"][idx])
        assert abs(g["grad_loc"][idx] - fd) <= tol, (idx, g["grad_loc"][idx], fd)


def _torch_agg(feat, ss, st, loc, w, G, softmax):
    """Independent formulation: one grid_sample per (camera, scale)."""
    B, P, GC = feat.shape
    Cg = GC // G
    _, A, pts, cams, _ = loc.shape
    scales = w.shape[4]
    wt = w
    if softmax:
        wt = torch.softmax(w.permute(0, 1, 5, 2, 3, 4).reshape(B, A, G, -1), -1)
        wt = wt.reshape(B, A, G, pts, cams, scales).permute(0, 1, 3, 4, 5, 2)
    out = 0
    for cam in range(cams):
        for sc in range(scales):
            H, W = int(ss[cam, sc, 0]), int(ss[cam, sc, 1])
            s0 = int(st[cam, sc])
            fm = feat[:, s0:s0 + H * W].reshape(B, H, W, G, Cg).permute(0, 3, 4, 1, 2).reshape(B * G, Cg, H, W)
            grid = (2 * loc[:, :, :, cam] - 1).unsqueeze(1).expand(B, G, A, pts, 2).reshape(B * G, A, pts, 2)
            smp = F.grid_sample(fm, grid, mode="bilinear", padding_mode="zeros", align_corners=False)
            smp = smp.reshape(B, G, Cg, A, pts)  # [B, G, Cg, A, pts]
            ww = wt[:, :, :, cam, sc, :].permute(0, 3, 1, 2).unsqueeze(2)  # [B, G, 1, A, pts]
            out = out + (smp * ww).sum(-1)
    return out.permute(0, 3, 1, 2).reshape(B, A, G * Cg)


@pytest.mark.parametrize("softmax", [False, True])
def test_matches_autograd_of_grid_sample_formulation(softmax):
    G = 2
    feat, ss, st, loc, w, go = _case(4, A=4, pts=3, cams=2, G=G, Cg=4)
    tf = torch.tensor(feat, requires_grad=True)
    tl = torch.tensor(loc, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    out = _torch_agg(tf, ss, st, tl, tw, G, softmax)
    np.testing.assert_allclose(out.detach().numpy(), _fwd(feat, ss, st, loc, w, softmax), rtol=0,
                               atol=1e-12)
    out.backward(torch.tensor(go))
    g = oracle.deform_agg_backward(feat, ss, st, loc, w, go, softmax=softmax)
    for name, t in (("grad_feat", tf), ("grad_loc", tl), ("grad_weights", tw)):
        d = np.abs(g[name] - t.grad.numpy())
        assert np.all(d <= 1e-10 * (1 + g[name + "_abs"])), (name, d.max())


def test_softmax_logit_gradients_sum_to_zero_and_zero_weights():
    feat, ss, st, loc, w, go = _case(5)
    g = oracle.deform_agg_backward(feat, ss, st, loc, w, go, softmax=True)
    sums = g["grad_weights"].sum(axis=(2, 3, 4))
    assert np.abs(sums).max() <= 1e-12 * (1 + g["grad_weights_abs"].sum(axis=(2, 3, 4)).max())
    z = oracle.deform_agg_backward(feat, ss, st, loc, 0 * w, go, softmax=False)
    assert not z["grad_feat"].any() and not z["grad_loc"].any()
    # locations far outside every map: no gradient reaches the features or the locations
    far = oracle.deform_agg_backward(feat, ss, st, loc + 5.0, w, go, softmax=False)
    assert not far["grad_feat"].any() and not far["grad_loc"].any() and not far["grad_weights"].any()


def test_rows_outside_the_maps_get_no_gradient_and_linearity():
    feat, ss, st, loc, w, go = _case(6)
    g = oracle.deform_agg_backward(feat, ss, st, loc, w, go)
    n_used = int(sum(h * wd for h, wd in ss.reshape(-1, 2)))
    assert not g["grad_feat"][:, n_used:].any()  # the 3 spare rows after the last map
    g2 = oracle.deform_agg_backward(feat, ss, st, loc, w, -3.0 * go)
    for k in ("grad_feat", "grad_loc", "grad_weights"):
        np.testing.assert_allclose(g2[k], -3.0 * g[k], rtol=0, atol=1e-12)
