"""CPU oracle for deformable sampling — TEST INFRASTRUCTURE ONLY.

Plain fp64 loop nests in ``oracle.c`` (built with gcc, OpenMP), wrapped with
ctypes. Only ``tests/``, the smoke check and the bench's ``cpu_baseline`` leg
may import this package; the GPU library never does, and the two share no code.

Every array is widened exactly to float64 before the call (fp16/bf16/fp32 ->
fp64 is exact), so the oracle sees the very values the GPU reads.

Functions (each follows the page/section cited in ``oracle.c``):
  bilinear     — one bilinear sample, zero outside the image
  softmax      — fp64 max-subtracted softmax
  dcn_core     — DCNv3/v4 core forward, channels-last
  dcn_core_backward — gradients of dcn_core w.r.t. x, offsets and modulation
  dcn_v2_columns, dcn_v2 — DCNv2 deform-im2col and modulated deformable conv
  deform_agg   — multi-camera multi-scale deformable aggregation
  deform_agg_backward — gradients of deform_agg w.r.t. features, locations, weights
  deform_roi_pool — deformable RoI pooling (per-bin offsets scaled by the RoI size)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Mutation testing loads a deliberately broken build of oracle.c from here.
_LIB_OVERRIDE = os.environ.get("DS_ORACLE_LIB")

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and (not os.path.exists(_LIB)
                                  or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(path)
        lib.oracle_bilinear.restype = ctypes.c_double
        lib.oracle_bilinear.argtypes = [_dp, _i64, _i64, _i64, ctypes.c_double,
                                        ctypes.c_double, _dp]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_set_threads.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_softmax.restype = None
        lib.oracle_softmax.argtypes = [_dp, _i64, _dp]
        lib.oracle_dcn_core.restype = ctypes.c_int
        lib.oracle_dcn_core.argtypes = [_dp, _dp, _dp, _dp, _dp] + [_i64] * 13 + [
            ctypes.c_float, ctypes.c_int, _i64p, _i64]
        lib.oracle_dcn_core_backward.restype = ctypes.c_int
        lib.oracle_dcn_core_backward.argtypes = [_dp] * 10 + [_i64] * 13 + [
            ctypes.c_float, ctypes.c_int]
        lib.oracle_dcn_v2_columns.restype = ctypes.c_int
        lib.oracle_dcn_v2_columns.argtypes = [_dp, _dp, _dp, _dp] + [_i64] * 13 + [
            ctypes.c_int, _i64p, _i64]
        lib.oracle_dcn_v2.restype = ctypes.c_int
        lib.oracle_dcn_v2.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp] + [_i64] * 14 + [
            ctypes.c_int, _i64p, _i64]
        lib.oracle_dcn_v2_backward.restype = ctypes.c_int
        lib.oracle_dcn_v2_backward.argtypes = [_dp] * 13 + [_i64] * 14 + [ctypes.c_int]
        lib.oracle_deform_agg.restype = ctypes.c_int
        lib.oracle_deform_agg.argtypes = [_dp, _i32p, _i32p, _dp, _dp, _dp, _dp] + [
            _i64] * 8 + [ctypes.c_int, _i64p, _i64]
        lib.oracle_deform_agg_backward.restype = ctypes.c_int
        lib.oracle_deform_agg_backward.argtypes = [_dp, _i32p, _i32p, _dp, _dp, _dp] + [_dp] * 6 + [
            _i64] * 8 + [ctypes.c_int]
        lib.oracle_deform_roi_pool.restype = ctypes.c_int
        lib.oracle_deform_roi_pool.argtypes = [_dp] * 5 + [_i64] * 7 + [ctypes.c_double] * 2
        _lib = lib
    return _lib


def _f64(a):
    """Exact widening of a numpy array or torch CPU tensor to contiguous fp64."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor (fp16/bf16/fp32): widen in torch, exact
        import torch
        a = a.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, t=_dp):
    return None if a is None else a.ctypes.data_as(t)


def _idx(sel):
    if sel is None:
        return None, 0
    s = np.ascontiguousarray(np.asarray(sel, dtype=np.int64).reshape(-1))
    return s, int(s.size)


def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Set the OpenMP thread count of the oracle's loops (for single-thread timings)."""
    _load().oracle_set_threads(int(n))


def out_size(n, k, s, p, d):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def bilinear(X, y, x):
    """Sample the 2-D map X[H, W] at (y, x); zero outside. Returns (value, absum)."""
    X = _f64(X)
    H, W = X.shape
    ab = ctypes.c_double(0.0)
    v = _load().oracle_bilinear(_ptr(X), H, W, 1, float(y), float(x), ctypes.byref(ab))
    return v, ab.value


def softmax(l):
    l = _f64(l).reshape(-1)
    m = np.empty_like(l)
    _load().oracle_softmax(_ptr(l), l.size, _ptr(m))
    return m


def dcn_core(x, offset, mask, *, kh, kw, stride=(1, 1), pad=(0, 0), dil=(1, 1),
             offset_scale=1.0, softmax=False, pix=None):
    """DCNv3/v4 core forward. x [N,H,W,G,C] (or [N,H,W,G*C] with offset giving G),
    offset [N,Ho,Wo,G,K,2], mask [N,Ho,Wo,G,K] or None.
    Returns (out, absum), each [N,Ho,Wo,G*C] (or [len(pix), G*C])."""
    x = _f64(x)
    offset = _f64(offset)
    mask = _f64(mask)
    N, H, W = x.shape[:3]
    G = offset.shape[3]
    GC = int(np.prod(x.shape[3:]))
    C = GC // G
    Ho, Wo = out_size(H, kh, stride[0], pad[0], dil[0]), out_size(W, kw, stride[1], pad[1], dil[1])
    sel, nsel = _idx(pix)
    rows = nsel if sel is not None else N * Ho * Wo
    out = np.zeros((rows, GC), np.float64)
    ab = np.zeros((rows, GC), np.float64)
    rc = _load().oracle_dcn_core(_ptr(x), _ptr(offset), _ptr(mask), _ptr(out), _ptr(ab),
                                 N, H, W, G, C, kh, kw, stride[0], stride[1], pad[0], pad[1],
                                 dil[0], dil[1], float(offset_scale), int(bool(softmax)),
                                 _ptr(sel, _i64p), nsel)
    if rc:
        raise ValueError("oracle_dcn_core rejected its arguments (%d)" % rc)
    if sel is None:
        out = out.reshape(N, Ho, Wo, GC)
        ab = ab.reshape(N, Ho, Wo, GC)
    return out, ab


def dcn_core_backward(x, offset, mask, grad_out, *, kh, kw, stride=(1, 1), pad=(0, 0),
                      dil=(1, 1), offset_scale=1.0, softmax=False, G=None):
    """Gradients of dcn_core. Shapes as dcn_core; grad_out [N,Ho,Wo,G*C].

    Returns a dict with grad_x [N,H,W,G*C], grad_offset (offset's shape),
    grad_mask (mask's shape, or [N,Ho,Wo,G,K] when mask is None: the gradient
    w.r.t. the unit modulation), and the matching *_abs arrays of summed
    |product terms| for error bounds."""
    x, offset, mask, gout = _f64(x), _f64(offset), _f64(mask), _f64(grad_out)
    N, H, W = x.shape[:3]
    G = offset.shape[3] if G is None else G
    GC = int(np.prod(x.shape[3:]))
    C = GC // G
    K = kh * kw
    Ho, Wo = out_size(H, kh, stride[0], pad[0], dil[0]), out_size(W, kw, stride[1], pad[1], dil[1])
    if gout.size != N * Ho * Wo * GC or offset.size != N * Ho * Wo * G * K * 2:
        raise ValueError("dcn_core_backward: shape mismatch")
    gx = np.zeros((N, H, W, GC)); gxa = np.zeros_like(gx)
    goff = np.zeros((N, Ho, Wo, G, K, 2)); goffa = np.zeros_like(goff)
    gm = np.zeros((N, Ho, Wo, G, K)); gma = np.zeros_like(gm)
    rc = _load().oracle_dcn_core_backward(
        _ptr(x), _ptr(offset), _ptr(mask), _ptr(gout), _ptr(gx), _ptr(goff), _ptr(gm),
        _ptr(gxa), _ptr(goffa), _ptr(gma), N, H, W, G, C, kh, kw, stride[0], stride[1],
        pad[0], pad[1], dil[0], dil[1], float(offset_scale), int(bool(softmax)))
    if rc:
        raise ValueError("oracle_dcn_core_backward rejected its arguments (%d)" % rc)
    return dict(grad_x=gx, grad_offset=goff, grad_mask=gm,
                grad_x_abs=gxa, grad_offset_abs=goffa, grad_mask_abs=gma)


def _v2_dims(x, offset, kh, kw, stride, pad, dil):
    N, Cin, H, W = x.shape
    Ho, Wo = out_size(H, kh, stride[0], pad[0], dil[0]), out_size(W, kw, stride[1], pad[1], dil[1])
    dg = offset.shape[1] // (2 * kh * kw)
    return N, Cin, H, W, Ho, Wo, dg


def dcn_v2_columns(x, offset, mask, *, kh, kw, stride=(1, 1), pad=(0, 0), dil=(1, 1),
                   softmax=False, pix=None):
    """Deform-im2col columns, [npix, Cin*K] with element ci*K + k."""
    x, offset, mask = _f64(x), _f64(offset), _f64(mask)
    N, Cin, H, W, Ho, Wo, dg = _v2_dims(x, offset, kh, kw, stride, pad, dil)
    sel, nsel = _idx(pix)
    rows = nsel if sel is not None else N * Ho * Wo
    cols = np.zeros((rows, Cin * kh * kw), np.float64)
    rc = _load().oracle_dcn_v2_columns(_ptr(x), _ptr(offset), _ptr(mask), _ptr(cols),
                                       N, Cin, H, W, kh, kw, stride[0], stride[1],
                                       pad[0], pad[1], dil[0], dil[1], dg, int(bool(softmax)),
                                       _ptr(sel, _i64p), nsel)
    if rc:
        raise ValueError("oracle_dcn_v2_columns rejected its arguments (%d)" % rc)
    return cols


def dcn_v2(x, offset, mask, weight, *, stride=(1, 1), pad=(0, 0), dil=(1, 1),
           softmax=False, pix=None):
    """DCNv2 forward, NCHW. Returns (out, absum): [N,Cout,Ho,Wo] or [npix, Cout]."""
    x, offset, mask, weight = _f64(x), _f64(offset), _f64(mask), _f64(weight)
    Cout, _, kh, kw = weight.shape
    N, Cin, H, W, Ho, Wo, dg = _v2_dims(x, offset, kh, kw, stride, pad, dil)
    sel, nsel = _idx(pix)
    rows = nsel if sel is not None else N * Ho * Wo
    out = np.zeros((rows, Cout), np.float64)
    ab = np.zeros((rows, Cout), np.float64)
    rc = _load().oracle_dcn_v2(_ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(out),
                               _ptr(ab), N, Cin, H, W, Cout, kh, kw, stride[0], stride[1],
                               pad[0], pad[1], dil[0], dil[1], dg, int(bool(softmax)),
                               _ptr(sel, _i64p), nsel)
    if rc:
        raise ValueError("oracle_dcn_v2 rejected its arguments (%d)" % rc)
    if sel is None:
        out = out.reshape(N, Ho, Wo, Cout).transpose(0, 3, 1, 2).copy()
        ab = ab.reshape(N, Ho, Wo, Cout).transpose(0, 3, 1, 2).copy()
    return out, ab


def dcn_v2_backward(x, offset, mask, weight, grad_out, *, stride=(1, 1), pad=(0, 0), dil=(1, 1),
                    softmax=False):
    """Gradients of dcn_v2. Returns a dict with grad_x [N,Cin,H,W], grad_offset
    [N,dg*K*2,Ho,Wo], grad_mask [N,dg*K,Ho,Wo] (w.r.t. the mask argument; the implied
    unit modulation when mask is None), grad_weight [Cout,Cin,kh,kw] and the matching
    *_abs arrays of summed |product terms|."""
    x, offset, mask, weight, gout = _f64(x), _f64(offset), _f64(mask), _f64(weight), _f64(grad_out)
    Cout, _, kh, kw = weight.shape
    N, Cin, H, W, Ho, Wo, dg = _v2_dims(x, offset, kh, kw, stride, pad, dil)
    K = kh * kw
    if gout.shape != (N, Cout, Ho, Wo) or offset.shape != (N, dg * K * 2, Ho, Wo):
        raise ValueError("dcn_v2_backward: shape mismatch")
    gx = np.zeros_like(x); gxa = np.zeros_like(x)
    goff = np.zeros_like(offset); goffa = np.zeros_like(offset)
    gm = np.zeros((N, dg * K, Ho, Wo)); gma = np.zeros_like(gm)
    gw = np.zeros_like(weight); gwa = np.zeros_like(weight)
    rc = _load().oracle_dcn_v2_backward(
        _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(gout), _ptr(gx), _ptr(goff),
        _ptr(gm), _ptr(gw), _ptr(gxa), _ptr(goffa), _ptr(gma), _ptr(gwa), N, Cin, H, W, Cout,
        kh, kw, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1], dg, int(bool(softmax)))
    if rc:
        raise ValueError("oracle_dcn_v2_backward rejected its arguments (%d)" % rc)
    return dict(grad_x=gx, grad_offset=goff, grad_mask=gm, grad_weight=gw,
                grad_x_abs=gxa, grad_offset_abs=goffa, grad_mask_abs=gma, grad_weight_abs=gwa)


def deform_agg(feat, spatial_shape, scale_start, loc, weights, *, softmax=False, anchors=None):
    """Aggregation forward. feat [B,P_total,G*Cg], spatial_shape int [cams,scales,2] (H,W),
    scale_start int [cams,scales], loc [B,A,pts,cams,2] (u,v), weights
    [B,A,pts,cams,scales,G]. Returns (out, absum): [B,A,G*Cg] or [len(anchors), G*Cg]."""
    feat, loc, weights = _f64(feat), _f64(loc), _f64(weights)
    ss = np.ascontiguousarray(np.asarray(spatial_shape, dtype=np.int32))
    st = np.ascontiguousarray(np.asarray(scale_start, dtype=np.int32))
    B, P_total, GC = feat.shape
    _, A, pts, cams, _ = loc.shape
    scales, G = weights.shape[4], weights.shape[5]
    Cg = GC // G
    sel, nsel = _idx(anchors)
    rows = nsel if sel is not None else B * A
    out = np.zeros((rows, GC), np.float64)
    ab = np.zeros((rows, GC), np.float64)
    rc = _load().oracle_deform_agg(_ptr(feat), _ptr(ss, _i32p), _ptr(st, _i32p), _ptr(loc),
                                   _ptr(weights), _ptr(out), _ptr(ab), B, P_total, A, pts,
                                   cams, scales, G, Cg, int(bool(softmax)), _ptr(sel, _i64p), nsel)
    if rc:
        raise ValueError("oracle_deform_agg rejected its arguments (%d)" % rc)
    if sel is None:
        out = out.reshape(B, A, GC)
        ab = ab.reshape(B, A, GC)
    return out, ab


def deform_agg_backward(feat, spatial_shape, scale_start, loc, weights, grad_out, *,
                        softmax=False):
    """Gradients of deform_agg. grad_out [B,A,G*Cg]. Returns a dict with grad_feat
    (feat's shape), grad_loc (loc's shape), grad_weights (weights' shape) and the
    matching *_abs arrays (sums of |product terms|)."""
    feat, loc, weights, gout = _f64(feat), _f64(loc), _f64(weights), _f64(grad_out)
    ss = np.ascontiguousarray(np.asarray(spatial_shape, dtype=np.int32))
    st = np.ascontiguousarray(np.asarray(scale_start, dtype=np.int32))
    B, P_total, GC = feat.shape
    _, A, pts, cams, _ = loc.shape
    scales, G = weights.shape[4], weights.shape[5]
    Cg = GC // G
    if gout.size != B * A * GC:
        raise ValueError("deform_agg_backward: grad_out must be [B,A,G*Cg]")
    gf, gfa = np.zeros_like(feat), np.zeros_like(feat)
    gl, gla = np.zeros_like(loc), np.zeros_like(loc)
    gw, gwa = np.zeros_like(weights), np.zeros_like(weights)
    rc = _load().oracle_deform_agg_backward(
        _ptr(feat), _ptr(ss, _i32p), _ptr(st, _i32p), _ptr(loc), _ptr(weights), _ptr(gout),
        _ptr(gf), _ptr(gl), _ptr(gw), _ptr(gfa), _ptr(gla), _ptr(gwa), B, P_total, A, pts, cams,
        scales, G, Cg, int(bool(softmax)))
    if rc:
        raise ValueError("oracle_deform_agg_backward rejected its arguments (%d)" % rc)
    return dict(grad_feat=gf, grad_loc=gl, grad_weights=gw, grad_feat_abs=gfa,
                grad_loc_abs=gla, grad_weights_abs=gwa)


def deform_roi_pool(x, rois, offset, *, k, S, spatial_scale=1.0, gamma=0.1):
    """Deformable RoI pooling. x [N,H,W,C] channels-last, rois [R,5] (batch, x1, y1, x2,
    y2), offset [R,k,k,2] (dx, dy) or None. Sample positions follow the fixed fp32
    operation sequence stated in oracle.c. Returns (out, absum), each [R,k,k,C]."""
    x, rois, offset = _f64(x), _f64(rois), _f64(offset)
    N, H, W, C = x.shape
    R = rois.shape[0]
    out = np.zeros((R, k, k, C))
    ab = np.zeros((R, k, k, C))
    rc = _load().oracle_deform_roi_pool(_ptr(x), _ptr(rois), _ptr(offset), _ptr(out), _ptr(ab),
                                        N, H, W, C, R, k, S, float(spatial_scale), float(gamma))
    if rc:
        raise ValueError("oracle_deform_roi_pool rejected its arguments (%d)" % rc)
    return out, ab

