"""Pins of the oracle's DCNv2 backward to things other than itself (CPU only).

No page prints a backward pass; the oracle takes the derivative of the DCNv2 sum
(modulated sampling, DCNv2-in-YOLOv5 page, section 1; bilinear kernel, hands-on
DCNv1 page, section 2). Checked against:
  * brute force: the forward is linear in x and in the weight, so each gradient
    entry is <grad_out, F(e_i)>;
  * exact unit steps in the modulation (linear without softmax) and central
    differences through the softmax;
  * one-sided differences in the offsets on a dyadic grid (a step that stays in
    the bilinear cell gives the derivative exactly);
  * torch autograd of an independent fp64 formulation (grid_sample with
    align_corners=True in pixel-index coordinates, zero padding, then a
    contraction with the weight), with deformable groups, stride, padding and
    dilation;
  * zero offsets and unit modulation: autograd of torch's conv2d.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

f64 = torch.float64


def _case(seed, N, Cin, H, W, Cout, kh, kw, stride, pad, dil, dg, grid=None, mask=True):
    r = np.random.default_rng(seed)
    Ho = oracle.out_size(H, kh, stride[0], pad[0], dil[0])
    Wo = oracle.out_size(W, kw, stride[1], pad[1], dil[1])
    K = kh * kw
    x = r.standard_normal((N, Cin, H, W))
    if grid:
        off = np.round(r.uniform(-3, 3, (N, dg * K * 2, Ho, Wo)) * grid) / grid
    else:
        off = r.standard_normal((N, dg * K * 2, Ho, Wo)) * 1.5
    m = r.standard_normal((N, dg * K, Ho, Wo)) if mask else None
    w = r.standard_normal((Cout, Cin, kh, kw))
    go = r.standard_normal((N, Cout, Ho, Wo))
    return x, off, m, w, go


def _fwd(x, off, m, w, st, pd, dl, softmax):
    return oracle.dcn_v2(x, off, m, w, stride=st, pad=pd, dil=dl, softmax=softmax)[0]


def _bwd(x, off, m, w, go, st, pd, dl, softmax):
    return oracle.dcn_v2_backward(x, off, m, w, go, stride=st, pad=pd, dil=dl, softmax=softmax)


SHAPES = [
    # N, Cin, H, W, Cout, kh, kw, stride, pad, dil, dg
    (1, 2, 4, 5, 3, 3, 3, (1, 1), (1, 1), (1, 1), 1),
    (2, 4, 5, 4, 2, 2, 3, (2, 1), (0, 2), (2, 1), 2),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("softmax", [False, True])
def test_grad_x_and_weight_brute_force(shape, softmax):
    N, Cin, H, W, Cout, kh, kw, st, pd, dl, dg = shape
    x, off, m, w, go = _case(1, N, Cin, H, W, Cout, kh, kw, st, pd, dl, dg)
    g = _bwd(x, off, m, w, go, st, pd, dl, softmax)
    for name, arr, fwd in (("grad_x", x, lambda e: _fwd(e, off, m, w, st, pd, dl, softmax)),
                           ("grad_weight", w, lambda e: _fwd(x, off, m, e, st, pd, dl, softmax))):
        want = np.zeros_like(arr)
        for i in range(arr.size):
            e = np.zeros(arr.size)
            e[i] = 1.0
            want.reshape(-1)[i] = (go * fwd(e.reshape(arr.shape))).sum()
        assert np.abs(g[name] - want).max() <= 1e-12 * (1 + np.abs(want).max()), name
        assert np.all(g[name + "_abs"] >= np.abs(g[name]) - 1e-12), name


@pytest.mark.parametrize("shape", SHAPES)
def test_grad_mask_unit_steps_and_softmax_fd(shape):
    N, Cin, H, W, Cout, kh, kw, st, pd, dl, dg = shape
    x, off, m, w, go = _case(2, N, Cin, H, W, Cout, kh, kw, st, pd, dl, dg)
    g0 = _bwd(x, off, m, w, go, st, pd, dl, False)
    g1 = _bwd(x, off, m, w, go, st, pd, dl, True)
    base = _fwd(x, off, m, w, st, pd, dl, False)
    r = np.random.default_rng(3)
    for idx in map(tuple, r.integers(0, m.shape, size=(25, 4))):
        m1 = m.copy()
        m1[idx] += 1.0
        fd = (go * (_fwd(x, off, m1, w, st, pd, dl, False) - base)).sum()
        assert abs(g0["grad_mask"][idx] - fd) <= 1e-11 * (1 + g0["grad_mask_abs"][idx])
        h = 1e-5
        m1 = m.copy(); m1[idx] += h
        m2 = m.copy(); m2[idx] -= h
        fd = (go * (_fwd(x, off, m1, w, st, pd, dl, True) - _fwd(x, off, m2, w, st, pd, dl, True))).sum() / (2 * h)
        assert abs(g1["grad_mask"][idx] - fd) <= 1e-7 * (1 + g1["grad_mask_abs"][idx])


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("softmax", [False, True])
def test_grad_offset_one_sided_fd(shape, softmax):
    N, Cin, H, W, Cout, kh, kw, st, pd, dl, dg = shape
    x, off, m, w, go = _case(4, N, Cin, H, W, Cout, kh, kw, st, pd, dl, dg, grid=64)
    g = _bwd(x, off, m, w, go, st, pd, dl, softmax)
    base = _fwd(x, off, m, w, st, pd, dl, softmax)
    hstep = 2.0 ** -12  # positions on a 1/64 grid: the step stays inside the cell
    for idx in np.ndindex(off.shape):
        o1 = off.copy()
        o1[idx] += hstep
        fd = (go * (_fwd(x, o1, m, w, st, pd, dl, softmax) - base)).sum() / hstep
        assert abs(g["grad_offset"][idx] - fd) <= 1e-9 * (1 + g["grad_offset_abs"][idx]), idx


def _torch_v2(x, off, m, w, st, pd, dl, dg, softmax):
    """Independent formulation: one grid_sample per (kernel point, deformable group)."""
    N, Cin, H, W = x.shape
    Cout, _, kh, kw = w.shape
    K = kh * kw
    Ho, Wo = off.shape[2], off.shape[3]
    cpg = Cin // dg
    ho = torch.arange(Ho, dtype=f64).view(Ho, 1)
    wo = torch.arange(Wo, dtype=f64).view(1, Wo)
    if m is None:
        m = torch.ones((N, dg * K, Ho, Wo), dtype=f64)
    mm = m.view(N, dg, K, Ho, Wo)
    if softmax:
        mm = torch.softmax(mm, 2)
    samples = []  # [N, Cin, K, Ho, Wo]
    for k in range(K):
        i, j = k // kw, k % kw
        per_g = []
        for g in range(dg):
            dx = off[:, (g * K + k) * 2]
            dy = off[:, (g * K + k) * 2 + 1]
            py = ho * st[0] - pd[0] + i * dl[0] + dy
            px = wo * st[1] - pd[1] + j * dl[1] + dx
            grid = torch.stack([2 * px / (W - 1) - 1, 2 * py / (H - 1) - 1], -1)
            s = F.grid_sample(x[:, g * cpg:(g + 1) * cpg], grid, mode="bilinear",
                              padding_mode="zeros", align_corners=True)
            per_g.append(s * mm[:, g, k].unsqueeze(1))
        samples.append(torch.cat(per_g, 1))
    cols = torch.stack(samples, 2)  # [N, Cin, K, Ho, Wo]
    return torch.einsum("oik,nikhw->nohw", w.reshape(Cout, Cin, K), cols)


@pytest.mark.parametrize("softmax", [False, True])
@pytest.mark.parametrize("mask", [True, False])
def test_matches_autograd_of_grid_sample_formulation(softmax, mask):
    st, pd, dl, dg = (2, 1), (1, 2), (1, 2), 2
    x, off, m, w, go = _case(5, 2, 4, 7, 8, 3, 3, 2, st, pd, dl, dg, mask=mask)
    tx = torch.tensor(x, requires_grad=True)
    to = torch.tensor(off, requires_grad=True)
    tm = torch.tensor(m, requires_grad=True) if mask else None
    tw = torch.tensor(w, requires_grad=True)
    out = _torch_v2(tx, to, tm, tw, st, pd, dl, dg, softmax)
    np.testing.assert_allclose(out.detach().numpy(), _fwd(x, off, m, w, st, pd, dl, softmax),
                               rtol=0, atol=1e-11)
    out.backward(torch.tensor(go))
    g = _bwd(x, off, m, w, go, st, pd, dl, softmax)
    pairs = [("grad_x", tx), ("grad_offset", to), ("grad_weight", tw)]
    if mask:
        pairs.append(("grad_mask", tm))
    for name, t in pairs:
        d = np.abs(g[name] - t.grad.numpy())
        assert np.all(d <= 1e-10 * (1 + g[name + "_abs"])), (name, d.max())


def test_zero_offsets_unit_mask_is_conv2d():
    st, pd, dl = (1, 2), (1, 1), (2, 1)
    x, off, m, w, go = _case(6, 2, 3, 6, 7, 4, 3, 3, st, pd, dl, 1)
    off[:] = 0.0
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    out = F.conv2d(tx, tw, stride=st, padding=pd, dilation=dl)
    out.backward(torch.tensor(go))
    g = _bwd(x, off, None, w, go, st, pd, dl, False)
    assert np.abs(g["grad_x"] - tx.grad.numpy()).max() <= 1e-12 * (1 + np.abs(tx.grad.numpy()).max())
    assert np.abs(g["grad_weight"] - tw.grad.numpy()).max() <= 1e-12 * (1 + np.abs(tw.grad.numpy()).max())
    # the unit modulation's gradient: <grad_out, the tap's contribution>
    Ho, Wo = go.shape[2:]
    outs = [oracle.dcn_v2(x, off, (np.arange(9) == k).astype(np.float64)[None, :, None, None]
                          * np.ones((2, 9, Ho, Wo)), w, stride=st, pad=pd, dil=dl)[0] for k in range(9)]
    for k in range(9):
        np.testing.assert_allclose(g["grad_mask"][:, k], (go * outs[k]).sum(1), rtol=0, atol=1e-11)


def test_softmax_logit_gradients_sum_to_zero_and_linearity():
    st, pd, dl, dg = (1, 1), (1, 1), (1, 1), 2
    x, off, m, w, go = _case(7, 1, 4, 5, 6, 2, 3, 3, st, pd, dl, dg)
    g = _bwd(x, off, m, w, go, st, pd, dl, True)
    sums = g["grad_mask"].reshape(1, dg, 9, 5, 6).sum(2)
    scale = g["grad_mask_abs"].reshape(1, dg, 9, 5, 6).sum(2)
    assert np.all(np.abs(sums) <= 1e-12 * (1 + scale))
    g2 = _bwd(x, off, m, w, -2.5 * go, st, pd, dl, True)
    for k in ("grad_x", "grad_offset", "grad_mask", "grad_weight"):
        np.testing.assert_allclose(g2[k], -2.5 * g[k], rtol=0, atol=1e-11)


def test_softmax_without_mask_is_zero_logits():
    """softmax with no mask tensor differentiates w.r.t. the implied (equal) logits: the
    same gradients as explicit zero logits; grad_x, grad_offset and grad_weight are the
    unmodulated ones divided by K (every point has modulation 1/K)."""
    st, pd, dl, dg = (1, 1), (1, 1), (1, 1), 2
    x, off, m, w, go = _case(8, 2, 4, 5, 6, 3, 3, 3, st, pd, dl, dg)
    g = _bwd(x, off, None, w, go, st, pd, dl, True)
    gz = _bwd(x, off, np.zeros_like(m), w, go, st, pd, dl, True)
    for k in ("grad_x", "grad_offset", "grad_mask", "grad_weight"):
        np.testing.assert_allclose(g[k], gz[k], rtol=0, atol=1e-12)
    g1 = _bwd(x, off, None, w, go, st, pd, dl, False)
    for k in ("grad_x", "grad_offset", "grad_weight"):
        np.testing.assert_allclose(g[k], g1[k] / 9.0, rtol=0, atol=1e-12)
    # logits' gradient: m_k (g_k - sum_j m_j g_j) with m = 1/9 and g_k the unit
    # modulation's gradient
    gm = g1["grad_mask"].reshape(2, dg, 9, *go.shape[2:]) / 9.0
    want = (gm - gm.sum(2, keepdims=True) / 9.0).reshape(g["grad_mask"].shape)
    np.testing.assert_allclose(g["grad_mask"], want, rtol=0, atol=1e-12)
