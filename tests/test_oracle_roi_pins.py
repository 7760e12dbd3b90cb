"""Pins of the oracle's deformable RoI pooling (CPU only).

The DCNv1 page (section 3) gives per-bin offsets normalised by the RoI size,
dp_ij = gamma * dp^_ij o (w, h), bilinear sampling and pooling; the sampling grid
inside a bin and the coordinate convention are readings (see oracle.c). Checked
against: an independent fp64 formulation on torch's grid_sample (align_corners=True
in pixel-index coordinates, zero padding); the lattice definition of the bilinear
kernel; exact reproduction of bilinear ramps (closed form at the mean sample
position); integer offset shifts equal to shifted RoIs (the (w, h) scaling and the
(dx, dy) order); batch index, spatial_scale and NULL offsets.

Sample positions are, by the oracle's stated reading, a fixed sequence of fp32
operations. Where every step is exact (dyadic RoIs, offsets and gamma, k and S powers
of two) the oracle equals the fp64 formulation exactly; elsewhere it differs from it by
the fp32 rounding of the position only, and a unit ramp image, which returns the sample
position itself, pins that sequence against numpy float32 arithmetic.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

f64 = torch.float64


def _rois(r, R, N, H, W, scale=1.0):
    x1 = r.uniform(-2, W * 0.7, R)
    y1 = r.uniform(-2, H * 0.7, R)
    x2 = x1 + r.uniform(0.5, W * 0.6, R)
    y2 = y1 + r.uniform(0.5, H * 0.6, R)
    b = r.integers(0, N, R)
    return np.stack([b, x1 / scale, y1 / scale, x2 / scale, y2 / scale], 1)


def _torch_roi(x, rois, off, k, S, scale, gamma):
    """grid_sample formulation: all k*k*S*S sample positions of a RoI at once."""
    N, H, W, C = x.shape
    img = torch.tensor(x).permute(0, 3, 1, 2)
    outs = []
    for r in range(rois.shape[0]):
        b, x1, y1, x2, y2 = rois[r]
        x1, y1 = x1 * scale, y1 * scale
        w, h = (x2 * scale - x1), (y2 * scale - y1)
        ii = torch.arange(k, dtype=f64).view(k, 1, 1, 1)
        jj = torch.arange(k, dtype=f64).view(1, k, 1, 1)
        sy = ((torch.arange(S, dtype=f64) + 0.5) / S).view(1, 1, S, 1)
        sx = ((torch.arange(S, dtype=f64) + 0.5) / S).view(1, 1, 1, S)
        dx = torch.zeros(k, k, dtype=f64) if off is None else torch.tensor(off[r, :, :, 0])
        dy = torch.zeros(k, k, dtype=f64) if off is None else torch.tensor(off[r, :, :, 1])
        py = y1 + (ii + sy) * (h / k) + (gamma * dy * h).view(k, k, 1, 1)
        px = x1 + (jj + sx) * (w / k) + (gamma * dx * w).view(k, k, 1, 1)
        py, px = torch.broadcast_tensors(py, px)
        grid = torch.stack([2 * px / (W - 1) - 1, 2 * py / (H - 1) - 1], -1).reshape(1, k * k, S * S, 2)
        smp = F.grid_sample(img[int(b):int(b) + 1], grid, mode="bilinear", padding_mode="zeros",
                            align_corners=True)  # [1, C, k*k, S*S]
        outs.append(smp.mean(-1).reshape(C, k, k).permute(1, 2, 0))
    return torch.stack(outs).numpy()


def _dyadic(v, bits=6):
    return np.round(np.asarray(v) * 2.0 ** bits) / 2.0 ** bits


@pytest.mark.parametrize("k,S,scale,gamma", [(4, 2, 1.0, 0.125), (2, 4, 0.5, 0.25), (8, 1, 0.25, 1.0)])
def test_matches_grid_sample_formulation_exactly_at_dyadic_inputs(k, S, scale, gamma):
    """Every fp32 step of the position is exact here, so the oracle must equal the fp64
    grid_sample formulation to rounding of the fp64 sums."""
    r = np.random.default_rng(k * 10 + S)
    N, H, W, C = 2, 13, 17, 3
    x = r.standard_normal((N, H, W, C))
    rois = _rois(r, 6, N, H, W, scale)
    rois[:, 1:] = _dyadic(rois[:, 1:] * scale, 4) / scale
    off = _dyadic(r.standard_normal((6, k, k, 2)), 5)
    o, ab = oracle.deform_roi_pool(x, rois, off, k=k, S=S, spatial_scale=scale, gamma=gamma)
    want = _torch_roi(x, rois, off, k, S, scale, gamma)
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-12)
    assert np.all(ab >= np.abs(o) - 1e-12)
    o0, _ = oracle.deform_roi_pool(x, rois, None, k=k, S=S, spatial_scale=scale, gamma=gamma)
    np.testing.assert_allclose(o0, _torch_roi(x, rois, None, k, S, scale, gamma), rtol=0, atol=1e-12)


@pytest.mark.parametrize("k,S,scale,gamma", [(3, 2, 1.0, 0.1), (7, 1, 0.5, 0.2), (2, 3, 0.25, 1.0)])
def test_matches_grid_sample_formulation(k, S, scale, gamma):
    """General inputs: the fp32 position differs from the fp64 one by a few roundings of
    coordinates below 2^6 (< 6 * 2^-19 px), and a position error delta moves a sample by at
    most delta * (sum of its |corners|); for N(0,1) maps that is below 1e-4."""
    r = np.random.default_rng(k * 10 + S)
    N, H, W, C = 2, 13, 17, 3
    x = r.standard_normal((N, H, W, C))
    rois = _rois(r, 6, N, H, W, scale).astype(np.float32).astype(np.float64)
    off = r.standard_normal((6, k, k, 2)).astype(np.float32).astype(np.float64)
    o, ab = oracle.deform_roi_pool(x, rois, off, k=k, S=S, spatial_scale=scale, gamma=gamma)
    g32 = float(np.float32(gamma))
    want = _torch_roi(x, rois, off, k, S, np.float32(scale), g32)
    err = np.abs(o - want)
    assert err.max() < 1e-4, err.max()
    assert np.all(ab >= np.abs(o) - 1e-12)


def _f32_positions(roi, off, k, S, scale, gamma, axis):
    """Sample positions along one axis (0: x, 1: y) of every bin by the stated fp32
    operation sequence, in numpy float32 arithmetic: [k, k, S] per bin row/column."""
    f = np.float32
    s, gm = f(scale), f(gamma)
    a1, a2 = (f(roi[1]), f(roi[3])) if axis == 0 else (f(roi[2]), f(roi[4]))
    start = f(a1 * s)
    ext = f(f(a2 - a1) * s)
    b = f(ext / f(k))
    pos = np.zeros((k, k, S))
    for i in range(k):
        for j in range(k):
            d = f(0.0) if off is None else f(f(gm * f(off[i, j, axis])) * ext)
            idx = j if axis == 0 else i
            for t in range(S):
                u = f(f(2 * (idx * S + t) + 1) / f(2 * S))
                pos[i, j, t] = f(f(start + f(u * b)) + d)
    return pos


@pytest.mark.parametrize("k,S,scale,gamma", [(7, 2, 0.0625, 0.1), (3, 3, 0.5, 0.3), (5, 1, 1.0, 0.7),
                                          (3, 3, 0.3, 0.2)])
def test_fp32_position_sequence_on_unit_ramps(k, S, scale, gamma):
    """X(h, w) = w returns the sample's x position exactly (fp64 sums of a ramp), and
    X(h, w) = h its y position: the pooled value is the mean of the fp32 positions."""
    r = np.random.default_rng(20 + k)
    H, W = 64, 72
    yy, xx = np.meshgrid(np.arange(H, dtype=np.float64), np.arange(W, dtype=np.float64), indexing="ij")
    X = np.stack([xx, yy], -1)[None]  # channel 0: x ramp, channel 1: y ramp
    R = 12
    x1 = r.uniform(12, 30, R) / scale
    y1 = r.uniform(12, 24, R) / scale
    rois = np.stack([np.zeros(R), x1, y1, x1 + r.uniform(0.3, 14, R) / scale,
                     y1 + r.uniform(0.3, 14, R) / scale], 1).astype(np.float32).astype(np.float64)
    off = r.uniform(-1, 1, (R, k, k, 2)).astype(np.float32).astype(np.float64)
    # RoIs starting near the origin and reaching far: x2 - x1 then needs more bits than
    # fp32 holds, so its rounding is a step of its own (no offsets: samples stay inside)
    x1 = r.uniform(0.01, 0.4, R) / scale
    y1 = r.uniform(0.01, 0.4, R) / scale
    near = np.stack([np.zeros(R), x1, y1, x1 + r.uniform(30, 60, R) / scale,
                     y1 + r.uniform(30, 55, R) / scale], 1).astype(np.float32).astype(np.float64)
    for rois, offs in ((rois, off), (rois, None), (near, None)):
        o, _ = oracle.deform_roi_pool(X, rois, offs, k=k, S=S, spatial_scale=scale, gamma=gamma)
        for ri in range(R):
            px = _f32_positions(rois[ri], None if offs is None else offs[ri], k, S, scale, gamma, 0)
            py = _f32_positions(rois[ri], None if offs is None else offs[ri], k, S, scale, gamma, 1)
            want_x = px.mean(-1)                       # each row of samples shares x
            want_y = py.mean(-1)
            np.testing.assert_allclose(o[ri, :, :, 0], want_x, rtol=0, atol=1e-10)
            np.testing.assert_allclose(o[ri, :, :, 1], want_y, rtol=0, atol=1e-10)


def lattice(X, y, x):
    H, W = X.shape
    return sum(max(0.0, 1 - abs(qy - y)) * max(0.0, 1 - abs(qx - x)) * X[qy, qx]
               for qy in range(H) for qx in range(W))


def test_single_sample_is_lattice_bilinear():
    """k = S = 1: one sample at the RoI centre, fl(fl(y1 + fl(fl(1/2) * h)) + 0)."""
    r = np.random.default_rng(1)
    X = r.standard_normal((7, 9))
    f = np.float32
    for _ in range(20):
        x1, y1 = f(r.uniform(-2, 9)), f(r.uniform(-2, 7))
        w, h = f(r.uniform(0, 3)), f(r.uniform(0, 3))
        x2, y2 = f(x1 + w), f(y1 + h)
        rois = np.array([[0, x1, y1, x2, y2]], dtype=np.float64)
        o, _ = oracle.deform_roi_pool(X[None, :, :, None], rois, None, k=1, S=1)
        py = f(y1 + f(f(0.5) * f(y2 - y1)))
        px = f(x1 + f(f(0.5) * f(x2 - x1)))
        assert abs(o[0, 0, 0, 0] - lattice(X, float(py), float(px))) < 1e-12


def test_bilinear_ramp_reproduced_at_mean_position():
    H, W = 20, 24
    yy, xx = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    a, b, c, e = 0.3, -1.25, 0.75, 0.0625
    X = (a + b * xx + c * yy + e * xx * yy)[None, :, :, None]
    rois = np.array([[0, 3.25, 2.5, 14.0, 11.75], [0, 1.0, 1.0, 9.5, 13.0]])
    k, S, gamma = 4, 2, 0.125  # dyadic: every fp32 step of the positions is exact
    r = np.random.default_rng(2)
    off = np.round(r.uniform(-1, 1, (2, k, k, 2)) * 64) / 64
    o, _ = oracle.deform_roi_pool(X, rois, off, k=k, S=S, gamma=gamma)
    for ri, (_, x1, y1, x2, y2) in enumerate(rois):
        w, h = x2 - x1, y2 - y1
        for i in range(k):
            for j in range(k):
                ym = y1 + (i + 0.5) * h / k + gamma * off[ri, i, j, 1] * h
                xm = x1 + (j + 0.5) * w / k + gamma * off[ri, i, j, 0] * w
                assert abs(o[ri, i, j, 0] - (a + b * xm + c * ym + e * xm * ym)) < 1e-10


def test_integer_offset_shifts_equal_shifted_rois():
    """gamma * dx * w = 2 and gamma * dy * h = -1 px move every sample of the bin by
    (2, -1): the same as pooling a RoI moved by that much (where all bins move)."""
    r = np.random.default_rng(3)
    x = r.standard_normal((1, 16, 20, 4))
    k, S, gamma = 2, 2, 0.5
    roi = np.array([[0, 4.0, 6.0, 12.0, 10.0]])  # w = 8, h = 4
    off = np.zeros((1, k, k, 2))
    off[..., 0] = 2.0 / (gamma * 8.0)
    off[..., 1] = -1.0 / (gamma * 4.0)
    o, _ = oracle.deform_roi_pool(x, roi, off, k=k, S=S, gamma=gamma)
    moved = roi + np.array([[0, 2.0, -1.0, 2.0, -1.0]])
    o2, _ = oracle.deform_roi_pool(x, moved, None, k=k, S=S, gamma=gamma)
    np.testing.assert_array_equal(o, o2)


def test_batch_index_scale_and_constant_image():
    r = np.random.default_rng(4)
    x = r.standard_normal((3, 8, 8, 2))
    roi = np.array([[2, 2.0, 2.0, 10.0, 10.0]])
    o, _ = oracle.deform_roi_pool(x, roi, None, k=2, S=2, spatial_scale=0.5)
    o2, _ = oracle.deform_roi_pool(x[2:3], np.array([[0, 1.0, 1.0, 5.0, 5.0]]), None, k=2, S=2)
    np.testing.assert_array_equal(o, o2)
    ones = np.ones((1, 10, 10, 1))
    o, _ = oracle.deform_roi_pool(ones, np.array([[0, 2.0, 2.0, 7.0, 6.0]]),
                                  r.uniform(-1, 1, (1, 3, 3, 2)), k=3, S=2, gamma=0.1)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)  # all samples inside: partition of unity
