"""deformable_sampling_amd — MI355X (gfx950) deformable sampling.

Thin ctypes binding over the C ABI of ``libdcn.so`` (declared in ``include/dcn.h``).
Each function below has the name of the C entry point it calls and only marshals
arguments: it checks device, dtype and contiguity of torch tensors, passes their
device pointers and torch's current HIP stream, and raises on a non-OK status.
Every step of the computation runs in the library's HIP kernels; there is no
CPU or PyTorch fallback, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcn.so")

DCN_F32, DCN_F16, DCN_BF16 = 0, 1, 2
_DTYPE_ID = {torch.float32: DCN_F32, torch.float16: DCN_F16, torch.bfloat16: DCN_BF16}

# alternative backward kernel paths (dcn_bwd_path flags; 0 = the library's choice)
DCN_BWD_DEFAULT, DCN_BWD_ATOMIC, DCN_BWD_PAIR_PASS = 0, 1, 2
DCN_BWD_PAIR_PASS_RECORDS, DCN_BWD_UNSTAGED_GATHER, DCN_BWD_GENERAL_MAIN = 4, 8, 16

STATUS = {0: "DCN_OK", 1: "DCN_ERR_NULL", 2: "DCN_ERR_SHAPE", 3: "DCN_ERR_PARAM",
          4: "DCN_ERR_DTYPE", 5: "DCN_ERR_ALIGN", 6: "DCN_ERR_WORKSPACE", 7: "DCN_ERR_HIP",
          8: "DCN_ERR_SCRATCH"}
DCN_V2_NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/dcn.h declares
EXPORTS = ("dcn_core_forward", "dcn_core_forward_packed", "dcn_core_backward_workspace_bytes", "dcn_core_backward",
           "dcn_v2_workspace_bytes", "dcn_v2_forward", "dcn_v2_im2col",
           "dcn_v2_backward_workspace_bytes", "dcn_v2_backward",
           "deform_agg_forward", "deform_agg_backward_workspace_bytes", "deform_agg_backward",
           "deform_roi_pool_forward",
           "dcn_core_backward_workspace_bytes_path", "dcn_core_backward_path",
           "deform_agg_backward_workspace_bytes_path", "deform_agg_backward_path",
           "dcn_v2_noalloc_bytes", "dcn_v2_forward_noalloc",
           "dcn_v2_packed_weight_bytes", "dcn_v2_pack_weight", "dcn_v2_forward_prepacked",
           "dcn_mfma_probe", "dcn_status_string", "dcn_last_hip_error")


class DcnError(RuntimeError):
    def __init__(self, fn, status, lib):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = "%s failed: %s (%s)" % (fn, self.name, lib.dcn_status_string(status).decode())
        if status == 7:
            msg += ", hipError %d" % lib.dcn_last_hip_error()
        super().__init__(msg)


_lib = None
_c = ctypes


def load(path: str | None = None):
    """Load libdcn.so (built by ``deformable_sampling_amd.build``); raise if missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            "libdcn.so not found at %s; build it with `python -m deformable_sampling_amd.build`" % p)
    lib = ctypes.CDLL(p)
    i, f, vp = _c.c_int, _c.c_float, _c.c_void_p
    lib.dcn_core_forward.restype = i
    lib.dcn_core_forward.argtypes = [vp, vp, vp, vp] + [i] * 13 + [f, i, i, vp]
    lib.dcn_core_forward_packed.restype = i
    lib.dcn_core_forward_packed.argtypes = [vp] * 3 + [i] * 13 + [f, i, i, i, i, vp]
    lib.dcn_core_backward_workspace_bytes.restype = _c.c_size_t
    lib.dcn_core_backward_workspace_bytes.argtypes = [i] * 14
    lib.dcn_core_backward.restype = i
    lib.dcn_core_backward.argtypes = [vp] * 8 + [_c.c_size_t] + [i] * 13 + [f, i, i, vp]
    lib.dcn_v2_workspace_bytes.restype = _c.c_size_t
    lib.dcn_v2_workspace_bytes.argtypes = [i] * 13 + [i]
    lib.dcn_v2_forward.restype = i
    lib.dcn_v2_forward.argtypes = [vp, vp, vp, vp, vp, vp, _c.c_size_t] + [i] * 15 + [i, vp]
    lib.dcn_v2_backward_workspace_bytes.restype = _c.c_size_t
    lib.dcn_v2_backward_workspace_bytes.argtypes = [i] * 15
    lib.dcn_v2_backward.restype = i
    lib.dcn_v2_backward.argtypes = [vp] * 10 + [_c.c_size_t] + [i] * 16 + [vp]
    lib.dcn_v2_im2col.restype = i
    lib.dcn_v2_im2col.argtypes = [vp, vp, vp, vp, _c.c_size_t] + [i] * 15 + [i, vp]
    lib.deform_agg_forward.restype = i
    lib.deform_agg_forward.argtypes = [vp, vp, vp, vp, vp, vp] + [i] * 9 + [i, vp]
    lib.deform_agg_backward_workspace_bytes.restype = _c.c_size_t
    lib.deform_agg_backward_workspace_bytes.argtypes = [i] * 9
    lib.deform_agg_backward.restype = i
    lib.deform_agg_backward.argtypes = [vp] * 10 + [_c.c_size_t] + [i] * 9 + [i, vp]
    u = _c.c_uint
    lib.dcn_core_backward_workspace_bytes_path.restype = _c.c_size_t
    lib.dcn_core_backward_workspace_bytes_path.argtypes = [i] * 14 + [u]
    lib.dcn_core_backward_path.restype = i
    lib.dcn_core_backward_path.argtypes = [vp] * 8 + [_c.c_size_t] + [i] * 13 + [f, i, i, u, vp]
    lib.deform_agg_backward_workspace_bytes_path.restype = _c.c_size_t
    lib.deform_agg_backward_workspace_bytes_path.argtypes = [i] * 9 + [u]
    lib.deform_agg_backward_path.restype = i
    lib.deform_agg_backward_path.argtypes = [vp] * 10 + [_c.c_size_t] + [i] * 9 + [i, u, vp]
    lib.dcn_v2_noalloc_bytes.restype = _c.c_size_t
    lib.dcn_v2_noalloc_bytes.argtypes = [i] * 15
    lib.dcn_v2_forward_noalloc.restype = i
    lib.dcn_v2_forward_noalloc.argtypes = [vp] * 5 + [i] * 15 + [i, vp]
    lib.dcn_v2_packed_weight_bytes.restype = _c.c_size_t
    lib.dcn_v2_packed_weight_bytes.argtypes = [i] * 4
    lib.dcn_v2_pack_weight.restype = i
    lib.dcn_v2_pack_weight.argtypes = [vp, vp, _c.c_size_t] + [i] * 4 + [i, vp]
    lib.dcn_v2_forward_prepacked.restype = i
    lib.dcn_v2_forward_prepacked.argtypes = [vp, vp, vp, vp, _c.c_size_t, vp, vp, _c.c_size_t] + [i] * 15 + [i, vp]
    lib.dcn_mfma_probe.restype = i
    lib.dcn_mfma_probe.argtypes = [vp, i, i, vp]
    lib.deform_roi_pool_forward.restype = i
    lib.deform_roi_pool_forward.argtypes = [vp] * 4 + [i] * 7 + [f, f, i, vp]
    lib.dcn_status_string.restype = _c.c_char_p
    lib.dcn_status_string.argtypes = [i]
    lib.dcn_last_hip_error.restype = i
    lib.dcn_last_hip_error.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return int(stream)
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(t, name, dtype=None, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))


def _pair(v):
    return (v, v) if isinstance(v, int) else tuple(v)


def out_size(n, k, s, p, d):
    return (n + 2 * p - d * (k - 1) - 1) // s + 1


def _call(fn, *args):
    lib = load()
    st = getattr(lib, fn)(*args)
    if st != 0:
        raise DcnError(fn, st, lib)


def dcn_core_forward(x, offset, mask, out=None, *, kernel=(3, 3), stride=1, pad=1, dilation=1,
                     offset_scale=1.0, softmax=False, stream=None):
    """DCNv3/v4 core. x [N,H,W,G*C]; offset [N,Ho,Wo,G,K,2] fp32 (dx,dy); mask
    [N,Ho,Wo,G,K] fp32 or None (logits if softmax). Returns out [N,Ho,Wo,G*C]."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    N, H, W, GC = x.shape
    G = offset.shape[3]
    if offset.dim() != 6 or offset.shape[4] != kh * kw or offset.shape[5] != 2 or GC % G:
        raise ValueError("offset must be [N,Ho,Wo,G,K,2] with G dividing the channels")
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape[:3]) != (N, Ho, Wo):
        raise ValueError("offset spatial shape %s != %s" % (tuple(offset.shape[:3]), (N, Ho, Wo)))
    if mask is not None and tuple(mask.shape) != (N, Ho, Wo, G, kh * kw):
        raise ValueError("mask must be [N,Ho,Wo,G,K]")
    if out is None:
        out = torch.empty((N, Ho, Wo, GC), dtype=x.dtype, device=x.device)
    _check(out, "out", x.dtype)
    _call("dcn_core_forward", _ptr(x), _ptr(offset), _ptr(mask), _ptr(out), N, H, W, G, GC // G,
          kh, kw, sh, sw, ph, pw, dh, dw, float(offset_scale), int(bool(softmax)),
          _DTYPE_ID[x.dtype], _stream(stream))
    return out


def pack_offset_mask(offset, mask, dtype=torch.float16, pixel_stride=None):
    """DCNv4's packed layout [N,Ho,Wo,pixel_stride]: per group K (dx, dy) pairs then K
    masks (ones when mask is None), padded rows zero. Layout helper for callers and
    tests (plain torch reshaping, no sampling arithmetic)."""
    N, Ho, Wo, G, K, _ = offset.shape
    m = torch.ones((N, Ho, Wo, G, K), dtype=offset.dtype, device=offset.device) if mask is None else mask
    rows = torch.cat([offset.reshape(N, Ho, Wo, G, 2 * K), m], -1).reshape(N, Ho, Wo, G * 3 * K)
    stride = G * 3 * K if pixel_stride is None else int(pixel_stride)
    if stride > G * 3 * K:
        rows = torch.nn.functional.pad(rows, (0, stride - G * 3 * K))
    return rows.to(dtype).contiguous()


def dcn_core_forward_packed(x, offset_mask, *, groups, kernel=(3, 3), stride=1, pad=1, dilation=1,
                            offset_scale=1.0, softmax=False, out=None, stream=None):
    """DCNv4 core with the packed offset+mask tensor [N,Ho,Wo,stride >= G*3K] (fp32/fp16/
    bf16; per group K (dx, dy) pairs then K masks). Returns out [N,Ho,Wo,G*C]."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(offset_mask, "offset_mask")
    if offset_mask.dtype not in _DTYPE_ID:
        raise ValueError("offset_mask must be fp32, fp16 or bf16")
    N, H, W, GC = x.shape
    G = int(groups)
    if GC % G:
        raise ValueError("groups must divide the channels")
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if offset_mask.dim() != 4 or tuple(offset_mask.shape[:3]) != (N, Ho, Wo):
        raise ValueError("offset_mask must be [N,Ho,Wo,stride]")
    if out is None:
        out = torch.empty((N, Ho, Wo, GC), dtype=x.dtype, device=x.device)
    _check(out, "out", x.dtype)
    _call("dcn_core_forward_packed", _ptr(x), _ptr(offset_mask), _ptr(out), N, H, W, G, GC // G,
          kh, kw, sh, sw, ph, pw, dh, dw, float(offset_scale), int(bool(softmax)),
          offset_mask.shape[3], _DTYPE_ID[offset_mask.dtype], _DTYPE_ID[x.dtype], _stream(stream))
    return out


def dcn_core_backward_workspace_bytes(N, H, W, G, C, kernel=(3, 3), stride=1, pad=1,
                                      dilation=1, dtype=torch.float16, path=DCN_BWD_DEFAULT):
    """Workspace bytes of dcn_core_backward (of dcn_core_backward_path when path != 0)."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    if path:
        return int(load().dcn_core_backward_workspace_bytes_path(
            N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, _DTYPE_ID[dtype], int(path)))
    return int(load().dcn_core_backward_workspace_bytes(N, H, W, G, C, kh, kw, sh, sw, ph, pw,
                                                        dh, dw, _DTYPE_ID[dtype]))


def dcn_core_backward(x, offset, mask, grad_out, *, kernel=(3, 3), stride=1, pad=1, dilation=1,
                      offset_scale=1.0, softmax=False, need=("x", "offset", "mask"),
                      grad_x=None, grad_offset=None, grad_mask=None, workspace=None,
                      path=DCN_BWD_DEFAULT, stream=None):
    """Gradients of dcn_core_forward w.r.t. x, offset and mask (the names in `need`).
    grad_out [N,Ho,Wo,G*C] in x's dtype. Returns (grad_x, grad_offset, grad_mask),
    None for a gradient not asked for; grad_mask is w.r.t. the mask argument (the
    unit modulation / zero logits when mask is None). path != 0 calls
    dcn_core_backward_path with those DCN_BWD_* flags."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    _check(grad_out, "grad_out", x.dtype)
    N, H, W, GC = x.shape
    G = offset.shape[3]
    K = kh * kw
    if offset.dim() != 6 or offset.shape[4] != K or offset.shape[5] != 2 or GC % G:
        raise ValueError("offset must be [N,Ho,Wo,G,K,2] with G dividing the channels")
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape[:3]) != (N, Ho, Wo):
        raise ValueError("offset spatial shape %s != %s" % (tuple(offset.shape[:3]), (N, Ho, Wo)))
    if mask is not None and tuple(mask.shape) != (N, Ho, Wo, G, K):
        raise ValueError("mask must be [N,Ho,Wo,G,K]")
    if tuple(grad_out.shape) != (N, Ho, Wo, GC):
        raise ValueError("grad_out must be [N,Ho,Wo,G*C]")
    dev = x.device
    if "x" in need and grad_x is None:
        grad_x = torch.empty_like(x)
    if "offset" in need and grad_offset is None:
        grad_offset = torch.empty_like(offset)
    if "mask" in need and grad_mask is None:
        grad_mask = torch.empty((N, Ho, Wo, G, K), dtype=torch.float32, device=dev)
    _check(grad_x, "grad_x", x.dtype, allow_none=True)
    _check(grad_offset, "grad_offset", torch.float32, allow_none=True)
    _check(grad_mask, "grad_mask", torch.float32, allow_none=True)
    wsb = dcn_core_backward_workspace_bytes(N, H, W, G, GC // G, kernel, stride, pad, dilation,
                                            x.dtype, path) if grad_x is not None else 0
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    args = [_ptr(x), _ptr(offset), _ptr(mask), _ptr(grad_out), _ptr(grad_x), _ptr(grad_offset),
            _ptr(grad_mask), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            N, H, W, G, GC // G, kh, kw, sh, sw, ph, pw, dh, dw, float(offset_scale),
            int(bool(softmax)), _DTYPE_ID[x.dtype]]
    if path:
        _call("dcn_core_backward_path", *args, int(path), _stream(stream))
    else:
        _call("dcn_core_backward", *args, _stream(stream))
    return grad_x, grad_offset, grad_mask


def dcn_v2_workspace_bytes(N, Cin, H, W, Cout, kernel=(3, 3), stride=1, pad=1, dilation=1,
                           dtype=torch.bfloat16):
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    return int(load().dcn_v2_workspace_bytes(N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw,
                                             _DTYPE_ID[dtype]))


def dcn_v2_forward(x, offset, mask, weight, out=None, workspace=None, *, stride=1, pad=1,
                   dilation=1, deform_groups=None, softmax=False, stream=None):
    """DCNv2. x [N,Cin,H,W] bf16/fp16; offset [N,dg*K*2,Ho,Wo] fp32; mask [N,dg*K,Ho,Wo]
    fp32 or None; weight [Cout,Cin,kh,kw]. Returns out [N,Cout,Ho,Wo]."""
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(weight, "weight", x.dtype)
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    N, Cin, H, W = x.shape
    Cout, Cin_w, kh, kw = weight.shape
    if Cin_w != Cin:
        raise ValueError("weight has %d input channels, x has %d" % (Cin_w, Cin))
    K = kh * kw
    dg = deform_groups if deform_groups is not None else offset.shape[1] // (2 * K)
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape) != (N, dg * K * 2, Ho, Wo):
        raise ValueError("offset must be [N, dg*K*2, Ho, Wo]")
    if mask is not None and tuple(mask.shape) != (N, dg * K, Ho, Wo):
        raise ValueError("mask must be [N, dg*K, Ho, Wo]")
    if out is None:
        out = torch.empty((N, Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    _check(out, "out", x.dtype)
    need = dcn_v2_workspace_bytes(N, Cin, H, W, Cout, (kh, kw), (sh, sw), (ph, pw), (dh, dw), x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _call("dcn_v2_forward", _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(out),
          _ptr(workspace), workspace.numel() * workspace.element_size(), N, Cin, H, W, Cout, kh, kw,
          sh, sw, ph, pw, dh, dw, dg, int(bool(softmax)), _DTYPE_ID[x.dtype], _stream(stream))
    return out


def dcn_v2_packed_weight_bytes(Cout, Cin, kernel=(3, 3)):
    """Bytes of the packed weight of a DCNv2 layer (0 if the sizes are invalid)."""
    kh, kw = _pair(kernel)
    return int(load().dcn_v2_packed_weight_bytes(Cout, Cin, kh, kw))


def dcn_v2_pack_weight(weight, packed=None, stream=None):
    """Permute weight [Cout,Cin,kh,kw] (bf16/fp16) once into the order the fused DCNv2
    kernel reads; returns the packed buffer (uint8 device tensor) for
    dcn_v2_forward_prepacked."""
    _check(weight, "weight")
    Cout, Cin, kh, kw = weight.shape
    need = dcn_v2_packed_weight_bytes(Cout, Cin, (kh, kw))
    if packed is None:
        packed = torch.empty(max(need, 1), dtype=torch.uint8, device=weight.device)
    _check(packed, "packed")
    _call("dcn_v2_pack_weight", _ptr(weight), _ptr(packed), packed.numel() * packed.element_size(),
          Cout, Cin, kh, kw, _DTYPE_ID[weight.dtype], _stream(stream))
    return packed


def dcn_v2_forward_prepacked(x, offset, mask, packed_weight, Cout, out=None, workspace=None, *,
                             kernel=(3, 3), stride=1, pad=1, dilation=1, deform_groups=None,
                             softmax=False, stream=None):
    """dcn_v2_forward with a weight packed by dcn_v2_pack_weight (for Cout output channels
    and the given kernel size). Returns out [N,Cout,Ho,Wo]."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(packed_weight, "packed_weight")
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    N, Cin, H, W = x.shape
    K = kh * kw
    dg = deform_groups if deform_groups is not None else offset.shape[1] // (2 * K)
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape) != (N, dg * K * 2, Ho, Wo):
        raise ValueError("offset must be [N, dg*K*2, Ho, Wo]")
    if mask is not None and tuple(mask.shape) != (N, dg * K, Ho, Wo):
        raise ValueError("mask must be [N, dg*K, Ho, Wo]")
    if out is None:
        out = torch.empty((N, Cout, Ho, Wo), dtype=x.dtype, device=x.device)
    _check(out, "out", x.dtype)
    need = dcn_v2_workspace_bytes(N, Cin, H, W, Cout, (kh, kw), (sh, sw), (ph, pw), (dh, dw), x.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _call("dcn_v2_forward_prepacked", _ptr(x), _ptr(offset), _ptr(mask), _ptr(packed_weight),
          packed_weight.numel() * packed_weight.element_size(), _ptr(out), _ptr(workspace),
          workspace.numel() * workspace.element_size(), N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw,
          dh, dw, dg, int(bool(softmax)), _DTYPE_ID[x.dtype], _stream(stream))
    return out


def dcn_v2_noalloc_bytes(N, Cin, H, W, Cout, kernel=(3, 3), stride=1, pad=1, dilation=1,
                         deform_groups=1, dtype=torch.bfloat16):
    """Static-scratch bytes dcn_v2_forward_noalloc needs for these sizes (0 if invalid)."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    return int(load().dcn_v2_noalloc_bytes(N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw,
                                           deform_groups, _DTYPE_ID[dtype]))


def dcn_v2_forward_noalloc(x, offset, mask, weight, out, *, stride=1, pad=1, dilation=1,
                           deform_groups=None, softmax=False, stream=None):
    """dcn_v2_forward with the library's static workspace: allocates nothing, so `out`
    [N,Cout,Ho,Wo] must be passed in. Overlapping calls on one GPU race."""
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(weight, "weight", x.dtype)
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    _check(out, "out", x.dtype)
    N, Cin, H, W = x.shape
    Cout, Cin_w, kh, kw = weight.shape
    if Cin_w != Cin:
        raise ValueError("weight has %d input channels, x has %d" % (Cin_w, Cin))
    K = kh * kw
    dg = deform_groups if deform_groups is not None else offset.shape[1] // (2 * K)
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape) != (N, dg * K * 2, Ho, Wo):
        raise ValueError("offset must be [N, dg*K*2, Ho, Wo]")
    if mask is not None and tuple(mask.shape) != (N, dg * K, Ho, Wo):
        raise ValueError("mask must be [N, dg*K, Ho, Wo]")
    if tuple(out.shape) != (N, Cout, Ho, Wo):
        raise ValueError("out must be [N, Cout, Ho, Wo]")
    _call("dcn_v2_forward_noalloc", _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(out),
          N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, dg, int(bool(softmax)),
          _DTYPE_ID[x.dtype], _stream(stream))
    return out


def dcn_v2_backward_workspace_bytes(N, Cin, H, W, Cout, kernel=(3, 3), stride=1, pad=1,
                                    dilation=1, deform_groups=1, dtype=torch.bfloat16):
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    return int(load().dcn_v2_backward_workspace_bytes(N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw,
                                                      dh, dw, int(deform_groups), _DTYPE_ID[dtype]))


def dcn_v2_backward(x, offset, mask, weight, grad_out, *, stride=1, pad=1, dilation=1,
                    deform_groups=None, softmax=False, need=("x", "offset", "mask", "weight"),
                    workspace=None, stream=None):
    """Gradients of dcn_v2_forward. Returns a dict with the requested entries of
    grad_x [N,Cin,H,W] (x's dtype), grad_offset, grad_mask (fp32, shaped as offset and
    mask; mask's shape [N,dg*K,Ho,Wo] when mask is None) and grad_weight (fp32)."""
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(weight, "weight", x.dtype)
    _check(grad_out, "grad_out", x.dtype)
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    N, Cin, H, W = x.shape
    Cout, Cin_w, kh, kw = weight.shape
    if Cin_w != Cin:
        raise ValueError("weight has %d input channels, x has %d" % (Cin_w, Cin))
    K = kh * kw
    dg = deform_groups if deform_groups is not None else offset.shape[1] // (2 * K)
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape) != (N, dg * K * 2, Ho, Wo):
        raise ValueError("offset must be [N, dg*K*2, Ho, Wo]")
    if mask is not None and tuple(mask.shape) != (N, dg * K, Ho, Wo):
        raise ValueError("mask must be [N, dg*K, Ho, Wo]")
    if tuple(grad_out.shape) != (N, Cout, Ho, Wo):
        raise ValueError("grad_out must be [N, Cout, Ho, Wo]")
    dev = x.device
    res = {}
    if "x" in need:
        res["grad_x"] = torch.empty_like(x)
    if "offset" in need:
        res["grad_offset"] = torch.empty((N, dg * K * 2, Ho, Wo), dtype=torch.float32, device=dev)
    if "mask" in need:
        res["grad_mask"] = torch.empty((N, dg * K, Ho, Wo), dtype=torch.float32, device=dev)
    if "weight" in need:
        res["grad_weight"] = torch.empty((Cout, Cin, kh, kw), dtype=torch.float32, device=dev)
    nbytes = dcn_v2_backward_workspace_bytes(N, Cin, H, W, Cout, (kh, kw), (sh, sw), (ph, pw),
                                             (dh, dw), dg, x.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _call("dcn_v2_backward", _ptr(x), _ptr(offset), _ptr(mask), _ptr(weight), _ptr(grad_out),
          _ptr(res.get("grad_x")), _ptr(res.get("grad_offset")), _ptr(res.get("grad_mask")),
          _ptr(res.get("grad_weight")), _ptr(workspace), workspace.numel() * workspace.element_size(),
          N, Cin, H, W, Cout, kh, kw, sh, sw, ph, pw, dh, dw, dg, int(bool(softmax)),
          _DTYPE_ID[x.dtype], _stream(stream))
    return res


def dcn_v2_im2col(x, offset, mask, Cout, workspace, *, kernel=(3, 3), stride=1, pad=1,
                  dilation=1, deform_groups=None, softmax=False, stream=None):
    """The deform-im2col stage of DCNv2 alone: x channels-last and the columns
    [P_pad][Rp] land in `workspace` (laid out as for dcn_v2_forward with this Cout).
    Returns `workspace`."""
    kh, kw = _pair(kernel)
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dilation)
    _check(x, "x")
    _check(offset, "offset", torch.float32)
    _check(mask, "mask", torch.float32, allow_none=True)
    N, Cin, H, W = x.shape
    K = kh * kw
    dg = deform_groups if deform_groups is not None else offset.shape[1] // (2 * K)
    Ho, Wo = out_size(H, kh, sh, ph, dh), out_size(W, kw, sw, pw, dw)
    if tuple(offset.shape) != (N, dg * K * 2, Ho, Wo):
        raise ValueError("offset must be [N, dg*K*2, Ho, Wo]")
    if mask is not None and tuple(mask.shape) != (N, dg * K, Ho, Wo):
        raise ValueError("mask must be [N, dg*K, Ho, Wo]")
    _call("dcn_v2_im2col", _ptr(x), _ptr(offset), _ptr(mask), _ptr(workspace),
          workspace.numel() * workspace.element_size(), N, Cin, H, W, Cout, kh, kw,
          sh, sw, ph, pw, dh, dw, dg, int(bool(softmax)), _DTYPE_ID[x.dtype], _stream(stream))
    return workspace


def deform_agg_forward(feat, spatial_shape, scale_start, loc, weights, out=None, *, softmax=False,
                       stream=None):
    """Aggregation. feat [B,P_total,G*Cg]; spatial_shape int [cams,scales,2] (host);
    scale_start int [cams,scales] (host); loc [B,A,pts,cams,2] fp32; weights
    [B,A,pts,cams,scales,G] fp32. Returns out [B,A,G*Cg]."""
    import numpy as np
    _check(feat, "feat")
    _check(loc, "loc", torch.float32)
    _check(weights, "weights", torch.float32)
    ss = np.ascontiguousarray(np.asarray(
        spatial_shape.cpu() if hasattr(spatial_shape, "cpu") else spatial_shape, dtype=np.int32))
    st = np.ascontiguousarray(np.asarray(
        scale_start.cpu() if hasattr(scale_start, "cpu") else scale_start, dtype=np.int32))
    B, P_total, GC = feat.shape
    _, A, pts, cams, two = loc.shape
    scales, G = weights.shape[4], weights.shape[5]
    if two != 2 or tuple(weights.shape) != (B, A, pts, cams, scales, G) or GC % G:
        raise ValueError("loc must be [B,A,pts,cams,2] and weights [B,A,pts,cams,scales,G]")
    if ss.shape != (cams, scales, 2) or st.shape != (cams, scales):
        raise ValueError("spatial_shape must be [cams,scales,2] and scale_start [cams,scales]")
    if out is None:
        out = torch.empty((B, A, GC), dtype=feat.dtype, device=feat.device)
    _check(out, "out", feat.dtype)
    _call("deform_agg_forward", _ptr(feat), ss.ctypes.data, st.ctypes.data, _ptr(loc),
          _ptr(weights), _ptr(out), B, P_total, A, pts, cams, scales, G, GC // G,
          int(bool(softmax)), _DTYPE_ID[feat.dtype], _stream(stream))
    return out


def deform_agg_backward_workspace_bytes(B, P_total, A, pts, cams, scales, G, Cg,
                                        dtype=torch.float32, path=DCN_BWD_DEFAULT):
    """Workspace bytes of deform_agg_backward (of deform_agg_backward_path when path != 0)."""
    if path:
        return int(load().deform_agg_backward_workspace_bytes_path(
            B, P_total, A, pts, cams, scales, G, Cg, _DTYPE_ID[dtype], int(path)))
    return int(load().deform_agg_backward_workspace_bytes(B, P_total, A, pts, cams, scales, G,
                                                          Cg, _DTYPE_ID[dtype]))


def deform_agg_backward(feat, spatial_shape, scale_start, loc, weights, grad_out, *,
                        softmax=False, need=("feat", "loc", "weights"), workspace=None,
                        path=DCN_BWD_DEFAULT, stream=None):
    """Gradients of deform_agg_forward w.r.t. feat, loc and weights (the names in
    `need`). Returns (grad_feat, grad_loc, grad_weights), None where not asked.
    workspace: a device buffer, None to allocate one, or False to pass none (allowed
    when only the weights' gradient is asked). path != 0 calls deform_agg_backward_path
    with those DCN_BWD_* flags."""
    _check(feat, "feat")
    _check(loc, "loc", torch.float32)
    _check(weights, "weights", torch.float32)
    import numpy as np
    _check(grad_out, "grad_out", feat.dtype)
    ss = np.ascontiguousarray(np.asarray(
        spatial_shape.cpu() if hasattr(spatial_shape, "cpu") else spatial_shape, dtype=np.int32))
    st = np.ascontiguousarray(np.asarray(
        scale_start.cpu() if hasattr(scale_start, "cpu") else scale_start, dtype=np.int32))
    B, P_total, GC = feat.shape
    _, A, pts, cams, _ = loc.shape
    scales, G = weights.shape[4], weights.shape[5]
    if GC % G or tuple(weights.shape[:4]) != (B, A, pts, cams) or ss.shape != (cams, scales, 2):
        raise ValueError("inconsistent aggregation shapes")
    if tuple(grad_out.shape) != (B, A, GC):
        raise ValueError("grad_out must be [B, A, G*Cg]")
    gf = torch.empty_like(feat) if "feat" in need else None
    gl = torch.empty_like(loc) if "loc" in need else None
    gw = torch.empty_like(weights) if "weights" in need else None
    wsb = deform_agg_backward_workspace_bytes(B, P_total, A, pts, cams, scales, G, GC // G,
                                              feat.dtype, path)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=feat.device)
    elif workspace is False:
        workspace = None
    args = [_ptr(feat), ss.ctypes.data, st.ctypes.data, _ptr(loc), _ptr(weights), _ptr(grad_out),
            _ptr(gf), _ptr(gl), _ptr(gw), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            B, P_total, A, pts, cams, scales, G, GC // G, int(bool(softmax)),
            _DTYPE_ID[feat.dtype]]
    if path:
        _call("deform_agg_backward_path", *args, int(path), _stream(stream))
    else:
        _call("deform_agg_backward", *args, _stream(stream))
    return gf, gl, gw


def deform_roi_pool_forward(x, rois, offset, *, output_size, sampling_ratio=2, spatial_scale=1.0,
                            gamma=0.1, out=None, stream=None):
    """Deformable RoI pooling. x [N,H,W,C] channels-last; rois [R,5] fp32 (batch, x1, y1,
    x2, y2); offset [R,k,k,2] fp32 (dx, dy) or None. Returns out [R,k,k,C]."""
    k = int(output_size)
    _check(x, "x")
    _check(rois, "rois", torch.float32)
    _check(offset, "offset", torch.float32, allow_none=True)
    N, H, W, C = x.shape
    R = rois.shape[0]
    if rois.dim() != 2 or rois.shape[1] != 5:
        raise ValueError("rois must be [R, 5]")
    if offset is not None and tuple(offset.shape) != (R, k, k, 2):
        raise ValueError("offset must be [R, k, k, 2]")
    if out is None:
        out = torch.empty((R, k, k, C), dtype=x.dtype, device=x.device)
    _check(out, "out", x.dtype)
    _call("deform_roi_pool_forward", _ptr(x), _ptr(rois), _ptr(offset), _ptr(out), N, H, W, C, R, k,
          int(sampling_ratio), float(spatial_scale), float(gamma), _DTYPE_ID[x.dtype],
          _stream(stream))
    return out

