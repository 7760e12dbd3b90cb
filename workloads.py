"""Seeded synthetic inputs for the deformable-sampling ops.

This module is shared by the tests, the smoke check and the bench. It only draws
random numbers and lays them out; it holds none of the sampling arithmetic
(no bilinear weights, no positions, no softmax of the op), so neither the oracle
nor the GPU path can lean on it for a result.

Draws come from NumPy ``Generator(PCG64(seed))`` in float64, in a fixed order
(features, offsets/locations, masks/logits, out-of-bounds selection, weights),
and are then rounded once (round-to-nearest-even) to the tensor's dtype by torch.
Everything returned is a CPU torch tensor, except from the ``*_device`` functions,
whose multi-GB inputs are drawn on the GPU by torch's seeded generator.

Named workloads (see ``WORKLOADS``) mirror the shapes and value distributions of
the ops' typical uses: a DCNv4 block on a 32x32 map, a DCNv3 stage on 56x56
maps, a DCNv4 layer at the stride-8 (80x80) level of a 640-pixel detector, a
DCNv2 layer on 40x40 maps and a six-camera, four-scale aggregation with 900
anchors. Real datasets (COCO, VisDrone, nuScenes, KITTI) are not used; these
inputs stand in for them with the same tensor shapes.
"""
from __future__ import annotations

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _t(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 numpy -> torch tensor of the named dtype (one RNE rounding)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(DTYPES[dtype]).contiguous()


def out_size(n, k, s, p, d):
    """Output extent of a strided, padded, dilated window (shape bookkeeping only)."""
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def _force_oob(r, offset, frac, H, W, pad_h, pad_w, ax_x=0, ax_y=1):
    """Push a Bernoulli(frac) subset of taps fully outside the image.

    A chosen tap gets, on a random side, an offset component of magnitude
    (extent + pad + U(1, 8)) pixels: whatever the tap's grid base is (it lies in
    [-pad, extent + pad - 1]), the sample then lands at least one pixel beyond
    the image on that side, so all four bilinear corners are outside. The other
    component keeps its normal draw. offset[..., 0] is dx, offset[..., 1] is dy.
    """
    shape = offset.shape[:-1]
    pick = r.random(shape) < frac
    side = r.integers(0, 4, size=shape)
    dist = r.uniform(1.0, 8.0, size=shape)
    top = pick & (side == 0)
    bot = pick & (side == 1)
    lef = pick & (side == 2)
    rig = pick & (side == 3)
    offset[..., ax_y][top] = -(H + pad_h + dist[top])
    offset[..., ax_y][bot] = (H + pad_h + dist[bot])
    offset[..., ax_x][lef] = -(W + pad_w + dist[lef])
    offset[..., ax_x][rig] = (W + pad_w + dist[rig])
    return pick


def core_case(*, N, H, W, G, C, kh=3, kw=3, stride=(1, 1), pad=(1, 1), dil=(1, 1),
              dtype="f32", offset_std=2.0, mask="uniform", oob_frac=0.0, seed=0,
              x_kind="normal"):
    """Inputs of the channels-last DCNv3/v4 core.

    x      [N, H, W, G*C] of ``dtype``, N(0,1) (or small integers for x_kind="int")
    offset [N, Ho, Wo, G, K, 2] fp32 (dx, dy) ~ N(0, offset_std) pixels
    mask   [N, Ho, Wo, G, K] fp32: "uniform" U(0,1), "logits" N(0,1), "ones", None
    """
    r = rng(seed)
    Ho, Wo = out_size(H, kh, stride[0], pad[0], dil[0]), out_size(W, kw, stride[1], pad[1], dil[1])
    K = kh * kw
    if x_kind == "int":
        x = r.integers(-4, 5, size=(N, H, W, G * C)).astype(np.float64)
    else:
        x = r.standard_normal((N, H, W, G * C))
    off = r.standard_normal((N, Ho, Wo, G, K, 2)) * offset_std
    if mask == "uniform":
        m = r.random((N, Ho, Wo, G, K))
    elif mask == "logits":
        m = r.standard_normal((N, Ho, Wo, G, K))
    elif mask == "ones":
        m = np.ones((N, Ho, Wo, G, K))
    else:
        m = None
    oob = None
    if oob_frac > 0:
        oob = _force_oob(r, off, oob_frac, H, W, pad[0], pad[1])
    return dict(
        x=_t(x, dtype), offset=_t(off, "f32"), mask=None if m is None else _t(m, "f32"),
        oob=oob, N=N, H=H, W=W, G=G, C=C, kh=kh, kw=kw, stride=tuple(stride), pad=tuple(pad),
        dil=tuple(dil), Ho=Ho, Wo=Wo, dtype=dtype, softmax=(mask == "logits"))


def core_grad_out(c, seed=0, kind="normal"):
    """An upstream gradient for the core's output [N, Ho, Wo, G*C] in x's dtype:
    N(0,1) draws (or small integers for kind="int") from their own seeded stream."""
    r = rng(seed + 7919)
    shape = (c["N"], c["Ho"], c["Wo"], c["G"] * c["C"])
    if kind == "int":
        g = r.integers(-3, 4, size=shape).astype(np.float64)
    else:
        g = r.standard_normal(shape)
    return _t(g, c["dtype"])


def v2_case(*, N, Cin, H, W, Cout, kh=3, kw=3, stride=(1, 1), pad=(1, 1), dil=(1, 1),
            dg=1, dtype="bf16", offset_std=2.0, mask="sigmoid", w_std=0.02, seed=0,
            x_kind="normal"):
    """Inputs of the NCHW DCNv2 (modulated deformable convolution).

    x      [N, Cin, H, W] dtype ~ N(0,1)
    offset [N, dg*K*2, Ho, Wo] fp32 ~ N(0, offset_std); channel (g*K+k)*2 is dx, +1 is dy
    mask   [N, dg*K, Ho, Wo] fp32: "sigmoid" = sigmoid of N(0,1) draws (the module
           applies the sigmoid before the op), "uniform", "ones", "logits" or None
    weight [Cout, Cin, kh, kw] dtype ~ N(0, w_std)
    """
    r = rng(seed)
    Ho, Wo = out_size(H, kh, stride[0], pad[0], dil[0]), out_size(W, kw, stride[1], pad[1], dil[1])
    K = kh * kw
    if x_kind == "int":
        x = r.integers(-4, 5, size=(N, Cin, H, W)).astype(np.float64)
    else:
        x = r.standard_normal((N, Cin, H, W))
    off = r.standard_normal((N, dg * K * 2, Ho, Wo)) * offset_std
    if mask == "sigmoid":
        m = 1.0 / (1.0 + np.exp(-r.standard_normal((N, dg * K, Ho, Wo))))
    elif mask == "uniform":
        m = r.random((N, dg * K, Ho, Wo))
    elif mask == "logits":
        m = r.standard_normal((N, dg * K, Ho, Wo))
    elif mask == "ones":
        m = np.ones((N, dg * K, Ho, Wo))
    else:
        m = None
    if x_kind == "int":
        w = r.integers(-2, 3, size=(Cout, Cin, kh, kw)).astype(np.float64)
    else:
        w = r.standard_normal((Cout, Cin, kh, kw)) * w_std
    return dict(
        x=_t(x, dtype), offset=_t(off, "f32"), mask=None if m is None else _t(m, "f32"),
        weight=_t(w, dtype), N=N, Cin=Cin, H=H, W=W, Cout=Cout, kh=kh, kw=kw,
        stride=tuple(stride), pad=tuple(pad), dil=tuple(dil), dg=dg, Ho=Ho, Wo=Wo,
        dtype=dtype, softmax=(mask == "logits"))


def v2_grad_out(c, seed=0, kind="normal"):
    """An upstream gradient for the DCNv2 output [N, Cout, Ho, Wo] in x's dtype: N(0,1)
    draws (or small integers for kind="int") from their own seeded stream."""
    r = rng(seed + 7927)
    shape = (c["N"], c["Cout"], c["Ho"], c["Wo"])
    if kind == "int":
        g = r.integers(-3, 4, size=shape).astype(np.float64)
    else:
        g = r.standard_normal(shape)
    return _t(g, c["dtype"])


def agg_case(*, B, shapes, A, pts, G, Cg, dtype="f32", weights="logits", seed=0,
             cam_major=True, loc_lo=0.0, loc_hi=1.0):
    """Inputs of the multi-camera multi-scale aggregation.

    shapes       list over cameras of lists over scales of (H, W)
    feat         [B, P_total, G*Cg] ~ N(0,1); maps flattened cam-major (cam, scale,
                 h, w) when cam_major, else scale-major (scale, cam, h, w)
    spatial_shape int32 [cams, scales, 2] (H, W); scale_start int32 [cams, scales]
    loc          [B, A, pts, cams, 2] (u, v) ~ U(loc_lo, loc_hi)
    weights      [B, A, pts, cams, scales, G]: "logits" N(0,1) (for the op's softmax),
                 "simplex" = normalised Exp(1) draws (a uniform point of the simplex
                 per (b, a, g), for runs without the softmax) or "ones"
    """
    r = rng(seed)
    cams, scales = len(shapes), len(shapes[0])
    ss = np.array(shapes, dtype=np.int32).reshape(cams, scales, 2)
    st = np.zeros((cams, scales), np.int32)
    pos = 0
    order = [(c, s) for c in range(cams) for s in range(scales)] if cam_major else \
            [(c, s) for s in range(scales) for c in range(cams)]
    for c, s in order:
        st[c, s] = pos
        pos += int(ss[c, s, 0]) * int(ss[c, s, 1])
    P_total = pos
    feat = r.standard_normal((B, P_total, G * Cg))
    loc = r.uniform(loc_lo, loc_hi, size=(B, A, pts, cams, 2))
    if weights == "logits":
        w = r.standard_normal((B, A, pts, cams, scales, G))
    elif weights == "simplex":
        e = r.exponential(1.0, size=(B, A, pts, cams, scales, G))
        w = e / e.sum(axis=(2, 3, 4), keepdims=True)
    else:
        w = np.ones((B, A, pts, cams, scales, G))
    return dict(
        feat=_t(feat, dtype), spatial_shape=ss, scale_start=st, loc=_t(loc, "f32"),
        weights=_t(w, "f32"), B=B, P_total=P_total, A=A, pts=pts, cams=cams, scales=scales,
        G=G, Cg=Cg, dtype=dtype, softmax=(weights == "logits"))


# ------------------------------------------------------ device-side draws --
#
# For inputs of several GB (the tests at the 2-GiB buffer limits) the draws are made
# on the GPU with torch's seeded generator (Philox) instead: NumPy would need minutes
# and tens of GB of host memory. The tests copy the windows the oracle needs back to
# the host, so both sides still see the same values.

def _dgen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def core_case_device(*, N, H, W, G, C, dtype="f16", offset_range=4.0, seed=0, device="cuda"):
    """Core inputs drawn on `device`: x ~ N(0,1) in dtype [N,H,W,G*C]; offsets
    ~ U(-offset_range, offset_range) fp32 [N,H,W,G,9,2] (3x3 window, stride 1, pad 1);
    masks ~ U(0,1) fp32 [N,H,W,G,9]."""
    g = _dgen(seed, device)
    x = torch.randn((N, H, W, G * C), generator=g, device=device, dtype=torch.float32).to(DTYPES[dtype])
    off = torch.rand((N, H, W, G, 9, 2), generator=g, device=device) * (2 * offset_range) - offset_range
    m = torch.rand((N, H, W, G, 9), generator=g, device=device)
    return dict(x=x, offset=off, mask=m, N=N, H=H, W=W, G=G, C=C, dtype=dtype)


def v2_case_device(*, N, Cin, H, W, Cout, dtype="bf16", offset_range=4.0, w_std=0.02, seed=0,
                   device="cuda"):
    """DCNv2 inputs drawn on `device` (3x3 window, stride 1, pad 1, one deformable
    group): x ~ N(0,1) [N,Cin,H,W]; offsets ~ U(-r, r) [N,18,H,W]; masks ~ U(0,1)
    [N,9,H,W]; weight ~ N(0, w_std^2) [Cout,Cin,3,3]."""
    g = _dgen(seed, device)
    x = torch.randn((N, Cin, H, W), generator=g, device=device, dtype=torch.float32).to(DTYPES[dtype])
    off = torch.rand((N, 18, H, W), generator=g, device=device) * (2 * offset_range) - offset_range
    m = torch.rand((N, 9, H, W), generator=g, device=device)
    w = (torch.randn((Cout, Cin, 3, 3), generator=g, device=device) * w_std).to(DTYPES[dtype])
    return dict(x=x, offset=off, mask=m, weight=w, N=N, Cin=Cin, H=H, W=W, Cout=Cout, dtype=dtype)


def agg_case_device(*, B, shapes, A, pts, G, Cg, seed=0, device="cuda"):
    """Aggregation inputs drawn on `device`, fp32: feat ~ N(0,1) [B,P_total,G*Cg] with
    maps flattened camera-major; loc ~ U(0,1) [B,A,pts,cams,2]; weight logits ~ N(0,1)
    [B,A,pts,cams,scales,G] (for the op's softmax). spatial_shape and scale_start are
    host int32 arrays."""
    cams, scales = len(shapes), len(shapes[0])
    ss = np.array(shapes, dtype=np.int32).reshape(cams, scales, 2)
    st = np.zeros((cams, scales), np.int32)
    pos = 0
    for c in range(cams):
        for s in range(scales):
            st[c, s] = pos
            pos += int(ss[c, s, 0]) * int(ss[c, s, 1])
    g = _dgen(seed, device)
    feat = torch.randn((B, pos, G * Cg), generator=g, device=device)
    loc = torch.rand((B, A, pts, cams, 2), generator=g, device=device)
    w = torch.randn((B, A, pts, cams, scales, G), generator=g, device=device)
    return dict(feat=feat, spatial_shape=ss, scale_start=st, loc=loc, weights=w, B=B, P_total=pos,
                A=A, pts=pts, cams=cams, scales=scales, G=G, Cg=Cg, dtype="f32", softmax=True)


# Named workloads: the five shapes the ops are exercised and measured on.
SPARSE4D_SHAPES = [[(64, 176), (32, 88), (16, 44), (8, 22)]] * 6

def agg_grad_out(c, seed=0):
    """An upstream gradient for the aggregation output [B, A, G*Cg] in feat's dtype:
    N(0,1) draws from their own seeded stream."""
    r = rng(seed + 104729)
    return _t(r.standard_normal((c["B"], c["A"], c["G"] * c["Cg"])), c["dtype"])


def roi_case(*, N, H, W, C, R, k=7, S=2, spatial_scale=1.0 / 16, gamma=0.1, dtype="f32",
             offsets=True, seed=0):
    """Inputs of deformable RoI pooling.

    x       [N, H, W, C] of dtype ~ N(0,1) (channels-last)
    rois    [R, 5] fp32 (batch, x1, y1, x2, y2) in input coordinates (the map times
            1/spatial_scale): batch uniform, box centre uniform over the input, width
            and height log-uniform between 1/16 and 1/2 of the input size
    offset  [R, k, k, 2] fp32 normalised (dx, dy) ~ N(0, 1), or None
    """
    r = rng(seed)
    x = r.standard_normal((N, H, W, C))
    Wi, Hi = W / spatial_scale, H / spatial_scale
    cx = r.uniform(0, Wi, R)
    cy = r.uniform(0, Hi, R)
    bw = Wi * np.exp(r.uniform(np.log(1 / 16), np.log(1 / 2), R))
    bh = Hi * np.exp(r.uniform(np.log(1 / 16), np.log(1 / 2), R))
    b = r.integers(0, N, R).astype(np.float64)
    rois = np.stack([b, cx - bw / 2, cy - bh / 2, cx + bw / 2, cy + bh / 2], 1)
    off = r.standard_normal((R, k, k, 2)) if offsets else None
    return dict(x=_t(x, dtype), rois=_t(rois, "f32"), offset=None if off is None else _t(off, "f32"),
                N=N, H=H, W=W, C=C, R=R, k=k, S=S, spatial_scale=spatial_scale, gamma=gamma,
                dtype=dtype)


WORKLOADS = {
    # DCNv4 block, fp32, one 32x32 map with 4 groups of 16 channels.
    "dcnv4_f32_n1_32x32_g4c16": dict(
        op="core", seed=1001,
        args=dict(N=1, H=32, W=32, G=4, C=16, dtype="f32", offset_std=2.0, mask="uniform")),
    # DCNv3 stage, fp32, batch 8 of 56x56 maps, softmax over the 9 points.
    "dcnv3_f32_n8_56x56_g4c16_softmax": dict(
        op="core", seed=1002,
        args=dict(N=8, H=56, W=56, G=4, C=16, dtype="f32", offset_std=1.5, mask="logits")),
    # DCNv4 at the stride-8 level of a 640-pixel detector: fp16 x [16,80,80,256].
    "dcnv4_f16_n16_80x80_g16c16": dict(
        op="core", seed=1003,
        args=dict(N=16, H=80, W=80, G=16, C=16, dtype="f16", offset_std=3.0, mask="uniform",
                  oob_frac=0.05)),
    # DCNv2 modulated deformable conv, bf16, 8x256x40x40 -> 8x256x40x40.
    "dcnv2_bf16_n8_c256_40x40": dict(
        op="v2", seed=1004,
        args=dict(N=8, Cin=256, H=40, W=40, Cout=256, dtype="bf16", offset_std=2.0,
                  mask="sigmoid", w_std=0.02)),
    # Deformable RoI pooling on the stride-16 map of a 1024x1024 input: fp32 x
    # [2,64,64,256], 512 RoIs, 7x7 bins of 2x2 samples, gamma 0.1.
    "droi_f32_n2_64x64_c256_r512_k7": dict(
        op="roi", seed=1006,
        args=dict(N=2, H=64, W=64, C=256, R=512, k=7, S=2, spatial_scale=1.0 / 16, gamma=0.1,
                  dtype="f32")),
    # Six-camera, four-scale aggregation, 900 anchors x 13 points, 8 groups of 32.
    "agg_f32_6cam_4scale_a900p13_g8c32": dict(
        op="agg", seed=1005,
        args=dict(B=1, shapes=SPARSE4D_SHAPES, A=900, pts=13, G=8, Cg=32, dtype="f32",
                  weights="logits")),
}


def make(name: str, **override):
    """Build a named workload (optionally overriding some of its arguments)."""
    spec = WORKLOADS[name]
    args = dict(spec["args"])
    args.update(override)
    seed = args.pop("seed", spec["seed"])
    fn = {"core": core_case, "v2": v2_case, "agg": agg_case, "roi": roi_case}[spec["op"]]
    case = fn(seed=seed, **args)
    case["op"] = spec["op"]
    case["name"] = name
    return case
