"""C ABI of libdcn.so on the CPU: exports and host-side argument validation.

Every rejected call returns its status before any HIP call, so these run without
a GPU. No call here passes validation with real work (that would launch kernels).
"""
import ctypes
import os
import re

import pytest

import deformable_sampling_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcn.h")

OK, NULL, SHAPE, PARAM, DTYPE, ALIGN, WORKSPACE, HIP, SCRATCH = range(9)
A = 0x10000  # a 256-byte aligned fake device address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"#[^\n]*", "", text)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\(", text)
    return sorted(set(n for n in names if n.startswith(("dcn_", "deform_"))))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        from deformable_sampling_amd import build
        build.build()
    return dsa.load()


def test_library_exports_every_declared_function(lib):
    declared = header_functions()
    assert set(declared) == set(dsa.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(9):
        s = lib.dcn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.dcn_status_string(99).decode() == "unknown status"
    assert lib.dcn_last_hip_error() == 0


def core(lib, x=A, off=A, mask=A, out=A, N=1, H=8, W=8, G=2, C=4, kh=3, kw=3, sh=1, sw=1,
         ph=1, pw=1, dh=1, dw=1, scale=1.0, softmax=0, dtype=0):
    return lib.dcn_core_forward(x, off, mask, out, N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw,
                                scale, softmax, dtype, None)


def test_core_validation(lib):
    assert core(lib, dtype=7) == DTYPE
    assert core(lib, N=-1) == SHAPE
    assert core(lib, H=0) == SHAPE
    assert core(lib, W=-3) == SHAPE
    assert core(lib, G=0) == SHAPE
    assert core(lib, C=0) == SHAPE
    assert core(lib, kh=0) == SHAPE
    assert core(lib, kh=5, kw=13) == SHAPE          # K = 65 > 64
    assert core(lib, sh=0) == PARAM
    assert core(lib, dw=0) == PARAM
    assert core(lib, pw=-1) == PARAM
    assert core(lib, H=2, kh=5, ph=0) == SHAPE      # Ho <= 0
    assert core(lib, H=40000, W=40000, G=2, C=4) == SHAPE  # image > 2^31 elements
    assert core(lib, N=0) == OK                      # empty batch: nothing to do
    assert core(lib, N=0, x=None, off=None, out=None) == OK
    assert core(lib, x=None) == NULL
    assert core(lib, off=None) == NULL
    assert core(lib, out=None) == NULL
    assert core(lib, x=A + 2, dtype=0) == ALIGN      # fp32 x on a 2-byte boundary
    assert core(lib, out=A + 1, dtype=1) == ALIGN    # fp16 out on an odd address
    assert core(lib, off=A + 2) == ALIGN
    assert core(lib, mask=A + 1) == ALIGN
    assert lib.dcn_last_hip_error() == 0


def core_bwd(lib, x=A, off=A, mask=A, go=A, gx=A, goff=A, gm=A, ws=A, wsb=1 << 40, N=1, H=8,
             W=8, G=2, C=4, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, scale=1.0, softmax=0,
             dtype=1):
    return lib.dcn_core_backward(x, off, mask, go, gx, goff, gm, ws, wsb, N, H, W, G, C, kh, kw,
                                 sh, sw, ph, pw, dh, dw, scale, softmax, dtype, None)


def bwd_ws(lib, N, H, W, G, C, kh=3, kw=3, s=1, p=1, d=1, dtype=1):
    return lib.dcn_core_backward_workspace_bytes(N, H, W, G, C, kh, kw, s, s, p, p, d, d, dtype)


def test_core_backward_workspace_bytes(lib):
    # binned: counts + fill cursors, starts (256-B aligned), 16-B records per sample
    N, H, W, G, C = 16, 80, 80, 16, 16
    nb = N * G * (80 // 16 + 1) ** 2 * 4
    a256 = lambda v: (v + 255) // 256 * 256
    head = a256((nb * 4 + 4 + 15) // 16 * 16 + nb * 4)
    starts = a256(nb * 4 + 4)
    assert bwd_ws(lib, N, H, W, G, C) == a256(head + starts + N * 80 * 80 * G * 9 * 16)
    assert bwd_ws(lib, 1, 3, 5, 1, 3, dtype=0) > 0            # fp32 binned too
    assert bwd_ws(lib, 1, 0, 5, 1, 3) == 0                    # invalid
    assert bwd_ws(lib, 1, 3, 5, 1, 3, dtype=9) == 0           # bad dtype
    assert bwd_ws(lib, 1, 3, 5, 1, 3, s=0) == 0               # stride 0
    assert bwd_ws(lib, 1, 2, 2, 1, 3, kh=5, kw=5, p=0) == 0   # Ho <= 0


def bwd_ws_path(lib, N, H, W, G, C, path, dtype=1):
    return lib.dcn_core_backward_workspace_bytes_path(N, H, W, G, C, 3, 3, 1, 1, 1, 1, 1, 1,
                                                      dtype, path)


def test_core_backward_workspace_bytes_atomic_fallback(lib):
    assert bwd_ws_path(lib, 16, 80, 80, 16, 16, 1) == 16 * 80 * 80 * 256 * 4
    assert bwd_ws_path(lib, 1, 3, 5, 1, 3, 1, dtype=2) == 256   # 45 floats -> 256 B
    assert bwd_ws_path(lib, 1, 3, 5, 1, 3, 1, dtype=0) == 0     # fp32: in place
    # the flags that keep the sorted path leave its size unchanged; unknown bits give 0
    for path in (0, 2, 4, 8, 16, 2 | 4 | 8):
        assert bwd_ws_path(lib, 16, 80, 80, 16, 16, path) == bwd_ws(lib, 16, 80, 80, 16, 16)
    assert bwd_ws_path(lib, 16, 80, 80, 16, 16, 32) == 0
    assert bwd_ws_path(lib, 16, 80, 80, 16, 16, 1 << 31) == 0


def test_core_backward_validation(lib):
    assert core_bwd(lib, dtype=7) == DTYPE
    assert core_bwd(lib, N=-1) == SHAPE
    assert core_bwd(lib, C=0) == SHAPE
    assert core_bwd(lib, kh=5, kw=13) == SHAPE
    assert core_bwd(lib, sh=0) == PARAM
    assert core_bwd(lib, H=2, kh=5, ph=0) == SHAPE
    assert core_bwd(lib, H=40000, W=40000) == SHAPE
    assert core_bwd(lib, N=0, x=None, off=None, go=None) == OK
    assert core_bwd(lib, x=None) == NULL
    assert core_bwd(lib, off=None) == NULL
    assert core_bwd(lib, go=None) == NULL
    assert core_bwd(lib, go=A + 1) == ALIGN          # fp16 grad_out on an odd address
    assert core_bwd(lib, gx=A + 1) == ALIGN
    assert core_bwd(lib, goff=A + 2) == ALIGN
    assert core_bwd(lib, gm=A + 2) == ALIGN
    assert core_bwd(lib, ws=None) == WORKSPACE       # fp16 grad_x needs the accumulator
    assert core_bwd(lib, ws=A + 128) == WORKSPACE    # not 256-byte aligned
    assert core_bwd(lib, wsb=bwd_ws(lib, 1, 8, 8, 2, 4) - 1) == WORKSPACE
    assert core_bwd(lib, gx=None, goff=None, gm=None, ws=None) == OK  # nothing asked for
    assert lib.dcn_last_hip_error() == 0


def v2(lib, x=A, off=A, mask=A, w=A, out=A, ws=A, wsb=1 << 40, N=1, Cin=16, H=8, W=8, Cout=8,
       kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, dg=1, softmax=0, dtype=2):
    return lib.dcn_v2_forward(x, off, mask, w, out, ws, wsb, N, Cin, H, W, Cout, kh, kw, sh, sw,
                              ph, pw, dh, dw, dg, softmax, dtype, None)


def test_v2_workspace_bytes(lib):
    # 8x256x40x40, 3x3: channels-last copy + permuted weight + columns, 256-B aligned
    n = lib.dcn_v2_workspace_bytes(8, 256, 40, 40, 256, 3, 3, 1, 1, 1, 1, 1, 1, 2)
    xt = 8 * 40 * 40 * 256 * 2
    wp = 256 * 2304 * 2
    col = 12800 * 2304 * 2
    assert n == xt + wp + col
    assert lib.dcn_v2_workspace_bytes(1, 3, 5, 5, 2, 3, 3, 1, 1, 1, 1, 1, 1, 1) > 0
    assert lib.dcn_v2_workspace_bytes(1, 3, 5, 5, 2, 3, 3, 1, 1, 1, 1, 1, 1, 0) == 0  # fp32
    assert lib.dcn_v2_workspace_bytes(1, 3, 5, 5, 2, 3, 3, 0, 1, 1, 1, 1, 1, 2) == 0  # stride 0
    assert lib.dcn_v2_workspace_bytes(1, 3, 2, 2, 2, 5, 5, 1, 1, 0, 0, 1, 1, 2) == 0  # Ho <= 0


def test_v2_validation(lib):
    assert v2(lib, dtype=0) == DTYPE                 # MFMA path is bf16/fp16
    assert v2(lib, dtype=9) == DTYPE
    assert v2(lib, N=-1) == SHAPE
    assert v2(lib, Cin=0) == SHAPE
    assert v2(lib, Cout=0) == SHAPE
    assert v2(lib, kh=9, kw=9) == SHAPE              # K = 81 > 64
    assert v2(lib, sh=0) == PARAM
    assert v2(lib, dg=0) == PARAM
    assert v2(lib, Cin=16, dg=3) == PARAM            # dg must divide Cin
    assert v2(lib, Cin=24, dg=2) == PARAM            # 12 channels per group: not a multiple of 8
    assert v2(lib, H=2, kh=5, ph=0) == SHAPE
    assert v2(lib, N=0) == OK
    assert v2(lib, x=None) == NULL
    assert v2(lib, w=None) == NULL
    assert v2(lib, ws=None) == WORKSPACE
    assert v2(lib, ws=A + 16) == WORKSPACE           # workspace must be 256-B aligned
    need = lib.dcn_v2_workspace_bytes(1, 16, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 2)
    assert v2(lib, wsb=need - 1) == WORKSPACE
    assert v2(lib, x=A + 1) == ALIGN
    assert v2(lib, off=A + 2) == ALIGN


def agg(lib, feat=A, ss=None, st=None, loc=A, w=A, out=A, B=1, P=1000, Anc=4, pts=2, cams=2,
        scales=2, G=2, Cg=8, softmax=0, dtype=0, shapes=None, starts=None):
    shapes = shapes if shapes is not None else [(10, 20)] * (cams * scales)
    starts = starts if starts is not None else [0] * (cams * scales)
    ssa = (ctypes.c_int32 * (2 * len(shapes)))(*[v for hw in shapes for v in hw])
    sta = (ctypes.c_int32 * len(starts))(*starts)
    ss = ssa if ss is None else ss
    st = sta if st is None else st
    return lib.deform_agg_forward(feat, ctypes.cast(ss, ctypes.c_void_p) if ss else None,
                                  ctypes.cast(st, ctypes.c_void_p) if st else None, loc, w, out,
                                  B, P, Anc, pts, cams, scales, G, Cg, softmax, dtype, None)


def test_agg_validation(lib):
    assert agg(lib, dtype=3) == DTYPE
    assert agg(lib, B=-1) == SHAPE
    assert agg(lib, P=0) == SHAPE
    assert agg(lib, pts=0) == SHAPE
    assert agg(lib, G=0) == SHAPE
    assert agg(lib, cams=9, scales=8) == SHAPE       # 72 maps > 64
    assert agg(lib, ss=False) == NULL
    assert agg(lib, st=False) == NULL
    assert agg(lib, starts=[0, 0, 0, 801]) == SHAPE  # 801 + 200 rows > P_total
    assert agg(lib, shapes=[(10, 20), (0, 5), (10, 20), (10, 20)]) == SHAPE
    assert agg(lib, starts=[0, -1, 0, 0]) == SHAPE
    assert agg(lib, starts=[0, 0, 0, 800], B=0) == OK  # exactly fits: passes the map check
    assert agg(lib, Anc=0) == OK
    assert agg(lib, B=0) == OK
    assert agg(lib, feat=None) == NULL
    assert agg(lib, w=None) == NULL
    assert agg(lib, loc=A + 4) == ALIGN              # (u, v) pairs need 8-byte alignment
    assert agg(lib, feat=A + 2, dtype=0) == ALIGN
    assert lib.dcn_last_hip_error() == 0             # nothing above reached a launch


def agg_bwd(lib, feat=A, ss=None, st=None, loc=A, w=A, go=A, gf=A, gl=A, gw=A, ws=A, wsb=1 << 40,
            B=1, P=100, An=4, pts=2, cams=2, scales=2, G=2, Cg=8, softmax=0, dtype=0):
    ss = (ctypes.c_int32 * 8)(5, 5, 2, 3, 5, 5, 2, 3) if ss is None else ss
    st = (ctypes.c_int32 * 4)(0, 25, 31, 56) if st is None else st
    return lib.deform_agg_backward(feat, ss, st, loc, w, go, gf, gl, gw, ws, wsb, B, P, An, pts,
                                   cams, scales, G, Cg, softmax, dtype, None)


def test_agg_backward_workspace_and_validation(lib):
    a256 = lambda v: (v + 255) // 256 * 256
    n = lib.deform_agg_backward_workspace_bytes(1, 89760, 900, 13, 6, 4, 8, 32, 0)
    T = 13 * 6 * 4
    assert n == (a256(8 * 900 * 13 * 6 * 2 * 4)      # grad_loc partials per group
                 + a256(900 * T * 8 * 4)             # per-sample g_t
                 + a256(3 * 8 * 900 * 4)             # per-(anchor, group) max, 1/sum, sum wt g_t
                 + a256(900 * T * 8 * 4)             # normalised weights
                 + a256(89760 * 2 * 4) + a256(89760 * 4)  # bucket counts + cursors, starts
                 + a256((89760 + 4095) // 4096 * 4)  # scan block sums
                 + a256(900 * T * 4 * 8))            # entries: one per corner
    assert lib.deform_agg_backward_workspace_bytes(1, 89760, 900, 13, 6, 4, 8, 32, 1) == n
    assert lib.deform_agg_backward_workspace_bytes(1, 0, 9, 1, 1, 1, 1, 8, 0) == 0
    assert agg_bwd(lib, dtype=5) == DTYPE
    assert agg_bwd(lib, Cg=513) == SHAPE                              # channel rounds limit
    assert agg_bwd(lib, cams=9, scales=8) == SHAPE                    # > 64 maps
    assert agg_bwd(lib, st=(ctypes.c_int32 * 4)(0, 25, 31, 96)) == SHAPE  # map past P_total
    assert agg_bwd(lib, B=0, feat=None, loc=None, w=None, go=None) == OK
    assert agg_bwd(lib, go=None) == NULL
    assert agg_bwd(lib, gl=A + 2) == ALIGN
    assert agg_bwd(lib, loc=A + 4) == ALIGN                            # (u, v) pairs: 8-byte aligned
    assert agg_bwd(lib, ws=None) == WORKSPACE                          # grad_loc needs partials
    assert agg_bwd(lib, wsb=16) == WORKSPACE
    assert agg_bwd(lib, gf=None, gl=None, gw=None, ws=None) == OK     # nothing asked for
    assert lib.dcn_last_hip_error() == 0


def roi(lib, x=A, rois=A, off=A, out=A, N=1, H=8, W=8, C=16, R=4, k=3, S=2, dtype=0):
    return lib.deform_roi_pool_forward(x, rois, off, out, N, H, W, C, R, k, S, 1.0, 0.1, dtype, None)


def test_roi_pool_validation(lib):
    assert roi(lib, dtype=4) == DTYPE
    assert roi(lib, N=0) == SHAPE
    assert roi(lib, C=0) == SHAPE
    assert roi(lib, R=-1) == SHAPE
    assert roi(lib, k=0) == PARAM
    assert roi(lib, S=0) == PARAM
    assert roi(lib, S=65) == PARAM
    assert roi(lib, H=50000, W=50000) == SHAPE
    assert roi(lib, R=0, x=None, rois=None, out=None) == OK
    assert roi(lib, x=None) == NULL
    assert roi(lib, rois=None) == NULL
    assert roi(lib, out=None) == NULL
    assert roi(lib, off=A + 4) == ALIGN            # (dx, dy) pairs: 8-byte aligned
    assert roi(lib, x=A + 2, dtype=0) == ALIGN
    assert lib.dcn_last_hip_error() == 0


def core_packed(lib, x=A, om=A, out=A, N=1, H=8, W=8, G=2, C=4, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1,
                dh=1, dw=1, stride=54, om_dtype=1, dtype=1):
    return lib.dcn_core_forward_packed(x, om, out, N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw,
                                       1.0, 0, stride, om_dtype, dtype, None)


def test_core_packed_validation(lib):
    assert core_packed(lib, om_dtype=9) == DTYPE
    assert core_packed(lib, dtype=9) == DTYPE
    assert core_packed(lib, stride=53) == PARAM          # G*3K = 54 elements per pixel
    assert core_packed(lib, kh=0) == SHAPE
    assert core_packed(lib, N=0, x=None, om=None, out=None) == OK
    assert core_packed(lib, om=None) == NULL
    assert core_packed(lib, om=A + 1) == ALIGN           # fp16 offsets on an odd address
    assert core_packed(lib, om=A + 2, om_dtype=0) == ALIGN
    assert lib.dcn_last_hip_error() == 0



def v2b(lib, x=A, off=A, mask=A, w=A, go=A, gx=A, goff=A, gm=A, gw=A, ws=A, wsb=1 << 40, N=1,
        Cin=16, H=8, W=8, Cout=8, kh=3, kw=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, dg=1, softmax=0,
        dtype=2):
    return lib.dcn_v2_backward(x, off, mask, w, go, gx, goff, gm, gw, ws, wsb, N, Cin, H, W, Cout,
                               kh, kw, sh, sw, ph, pw, dh, dw, dg, softmax, dtype, None)


def test_v2_backward_workspace_bytes(lib):
    a256 = lambda v: (v + 255) // 256 * 256
    n = lib.dcn_v2_backward_workspace_bytes(8, 256, 40, 40, 256, 3, 3, 1, 1, 1, 1, 1, 1, 1, 2)
    P, R, D = 12800, 2304, 8 * 40 * 40
    splits = 7  # 2 x 18 output tiles of the weight gradient -> 256 // 36 splits over 200 K steps
    want = (a256(8 * 40 * 40 * 256 * 2) + a256(2304 * 256 * 2) + a256(P * 256 * 2)
            + a256(256 * P * 2) + a256(2304 * P * 2) + a256(P * R * 4) + a256(splits * 256 * R * 4)
            + a256(D * 8) + a256(D * 4) + a256(P * 9 * 4 * 8))
    assert n == want
    assert lib.dcn_v2_backward_workspace_bytes(1, 3, 5, 5, 2, 3, 3, 1, 1, 1, 1, 1, 1, 1, 1) > 0
    assert lib.dcn_v2_backward_workspace_bytes(1, 3, 5, 5, 2, 3, 3, 1, 1, 1, 1, 1, 1, 1, 0) == 0
    assert lib.dcn_v2_backward_workspace_bytes(1, 16, 5, 5, 2, 3, 3, 1, 1, 1, 1, 1, 1, 3, 2) == 0


def test_v2_backward_validation(lib):
    assert v2b(lib, dtype=0) == DTYPE
    assert v2b(lib, N=-1) == SHAPE
    assert v2b(lib, kh=9, kw=9) == SHAPE
    assert v2b(lib, dg=3) == PARAM
    assert v2b(lib, Cin=24, dg=2) == PARAM
    assert v2b(lib, N=0) == OK
    assert v2b(lib, x=None) == NULL
    assert v2b(lib, go=None) == NULL
    assert v2b(lib, gx=None, goff=None, gm=None, gw=None) == OK  # nothing requested
    assert v2b(lib, ws=None) == WORKSPACE
    need = lib.dcn_v2_backward_workspace_bytes(1, 16, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 1, 2)
    assert v2b(lib, wsb=need - 1) == WORKSPACE
    assert v2b(lib, gx=A + 1) == ALIGN
    assert v2b(lib, gw=A + 2) == ALIGN
    assert lib.dcn_last_hip_error() == 0


def test_agg_backward_workspace_atomic_fallback(lib):
    n = lib.deform_agg_backward_workspace_bytes_path(1, 89760, 900, 13, 6, 4, 8, 32, 0, 1)
    a256 = lambda v: (v + 255) // 256 * 256
    T = 13 * 6 * 4
    assert n == (a256(8 * 900 * 13 * 6 * 2 * 4)                     # fp32: loc partials,
                 + a256(900 * T * 8 * 4) + a256(3 * 8 * 900 * 4))    # g_t and unit sums only
    n16 = lib.deform_agg_backward_workspace_bytes_path(1, 89760, 900, 13, 6, 4, 8, 32, 1, 1)
    assert n16 == n + 89760 * 256 * 4                                # + fp32 feature accumulator
    dflt = lib.deform_agg_backward_workspace_bytes(1, 89760, 900, 13, 6, 4, 8, 32, 0)
    assert lib.deform_agg_backward_workspace_bytes_path(1, 89760, 900, 13, 6, 4, 8, 32, 0, 16) == dflt
    assert lib.deform_agg_backward_workspace_bytes_path(1, 89760, 900, 13, 6, 4, 8, 32, 0, 64) == 0


def test_backward_path_variants_validate_their_flags(lib):
    """The *_path entry points reject unknown flag bits before any HIP call and otherwise
    validate exactly as the default entry points (a rejected size is rejected by both)."""
    args = (A, A, A, A, A, A, A, A, 1 << 40, 1, 8, 8, 2, 4, 3, 3, 1, 1, 1, 1, 1, 1, 1.0, 0, 1)
    assert lib.dcn_core_backward_path(*args, 32, None) == PARAM
    assert lib.dcn_core_backward_path(*args, 1 << 31, None) == PARAM
    bad = (A, A, A, A, A, A, A, A, 1 << 40, 1, 8, 8, 2, 4, 3, 3, 0, 1, 1, 1, 1, 1, 1.0, 0, 1)
    assert lib.dcn_core_backward_path(*bad, 1, None) == PARAM      # stride 0
    assert lib.dcn_core_backward_path(*args[:-1], 7, 2, None) == DTYPE
    ss = (ctypes.c_int32 * 8)(5, 5, 2, 3, 5, 5, 2, 3)
    st = (ctypes.c_int32 * 4)(0, 25, 31, 56)
    aargs = (A, ss, st, A, A, A, A, A, A, A, 1 << 40, 1, 100, 4, 2, 2, 2, 2, 8, 0, 0)
    assert lib.deform_agg_backward_path(*aargs, 64, None) == PARAM
    st_bad = (ctypes.c_int32 * 4)(0, 25, 31, 99)                  # map past P_total
    aargs_bad = (A, ss, st_bad) + aargs[3:]
    assert lib.deform_agg_backward_path(*aargs_bad, 1, None) == SHAPE
    assert lib.dcn_last_hip_error() == 0


def test_v2_noalloc_sizes_and_validation(lib):
    """dcn_v2_forward_noalloc: scratch need per call (fused shapes: channels-last x plus
    the permuted weight; others also the columns), a call beyond the static array is
    refused with DCN_ERR_SCRATCH before any HIP call, and bad arguments give the same
    status as dcn_v2_forward."""
    a256 = lambda v: (v + 255) // 256 * 256
    # 8x256x40x40, Cout 256, bf16: fused (Cin % 64 == 0)
    need = lib.dcn_v2_noalloc_bytes(8, 256, 40, 40, 256, 3, 3, 1, 1, 1, 1, 1, 1, 1, 2)
    assert need == a256(8 * 40 * 40 * 256 * 2) + a256(256 * 2304 * 2)
    assert need < dsa.DCN_V2_NOALLOC_SCRATCH_BYTES
    # Cin 16: two-stage, the columns too
    full = lib.dcn_v2_workspace_bytes(2, 16, 9, 11, 24, 3, 3, 1, 1, 1, 1, 1, 1, 2)
    assert lib.dcn_v2_noalloc_bytes(2, 16, 9, 11, 24, 3, 3, 1, 1, 1, 1, 1, 1, 1, 2) == full
    assert lib.dcn_v2_noalloc_bytes(2, 16, 9, 11, 24, 3, 3, 0, 1, 1, 1, 1, 1, 1, 2) == 0

    def call(N=1, Cin=16, H=8, W=8, Cout=8, x=A, off=A, m=A, w=A, out=A, dg=1, dtype=2):
        return lib.dcn_v2_forward_noalloc(x, off, m, w, out, N, Cin, H, W, Cout, 3, 3, 1, 1, 1,
                                          1, 1, 1, dg, 0, dtype, None)
    # 4 x 256 x 160 x 160 (Cin not a multiple of 64 -> columns): far beyond 64 MiB
    big = lib.dcn_v2_noalloc_bytes(4, 200, 160, 160, 64, 3, 3, 1, 1, 1, 1, 1, 1, 1, 2)
    assert big > dsa.DCN_V2_NOALLOC_SCRATCH_BYTES
    assert call(N=4, Cin=200, H=160, W=160, Cout=64) == SCRATCH
    assert call(dtype=0) == DTYPE
    assert call(dtype=9) == DTYPE
    assert call(Cin=0) == SHAPE
    assert call(dg=3) == PARAM
    assert call(x=None) == NULL
    assert call(w=None) == NULL
    assert call(out=A + 1) == ALIGN
    assert call(N=0) == OK
    assert lib.dcn_last_hip_error() == 0


def test_v2_packed_weight_sizes_and_validation(lib):
    """dcn_v2_pack_weight / dcn_v2_forward_prepacked: packed size (Cout rounded up to
    128 rows of Rp = K*Cin_pad rounded up to 64 values), and every rejected call's
    status before any HIP call; the prepacked forward only takes layers that form their
    columns on chip (Cin a multiple of 64)."""
    assert lib.dcn_v2_packed_weight_bytes(256, 256, 3, 3) == 256 * 2304 * 2
    assert lib.dcn_v2_packed_weight_bytes(24, 16, 3, 3) == 128 * 192 * 2
    assert lib.dcn_v2_packed_weight_bytes(300, 128, 3, 3) == 384 * 1152 * 2
    assert lib.dcn_v2_packed_weight_bytes(0, 16, 3, 3) == 0
    assert lib.dcn_v2_packed_weight_bytes(8, 16, 9, 9) == 0  # K > 64
    need = lib.dcn_v2_packed_weight_bytes(8, 64, 3, 3)

    def pack(w=A, p=A, nbytes=need, Cout=8, Cin=64, kh=3, kw=3, dtype=2):
        return lib.dcn_v2_pack_weight(w, p, nbytes, Cout, Cin, kh, kw, dtype, None)
    assert pack(dtype=0) == DTYPE
    assert pack(dtype=5) == DTYPE
    assert pack(Cout=0) == SHAPE
    assert pack(kh=0) == SHAPE
    assert pack(w=None) == NULL
    assert pack(p=None) == NULL
    assert pack(w=A + 1) == ALIGN
    assert pack(p=A + 8) == ALIGN
    assert pack(nbytes=need - 1) == WORKSPACE

    ws = lib.dcn_v2_workspace_bytes(1, 64, 8, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 2)

    def fwd(N=1, Cin=64, Cout=8, x=A, off=A, m=A, pw=A, pbytes=need, out=A, w=A, wbytes=ws, dg=1,
            dtype=2):
        return lib.dcn_v2_forward_prepacked(x, off, m, pw, pbytes, out, w, wbytes, N, Cin, 8, 8, Cout,
                                            3, 3, 1, 1, 1, 1, 1, 1, dg, 0, dtype, None)
    assert fwd(dtype=0) == DTYPE
    assert fwd(Cin=0) == SHAPE
    assert fwd(dg=3) == PARAM
    assert fwd(Cin=16, pbytes=lib.dcn_v2_packed_weight_bytes(8, 16, 3, 3)) == PARAM  # two-stage layer
    assert fwd(x=None) == NULL
    assert fwd(pw=None) == NULL
    assert fwd(out=A + 1) == ALIGN
    assert fwd(pw=A + 8) == ALIGN
    assert fwd(pbytes=need - 1) == WORKSPACE
    assert fwd(wbytes=ws - 1) == WORKSPACE
    assert fwd(w=None) == WORKSPACE
    assert fwd(N=0) == OK
    assert lib.dcn_last_hip_error() == 0


def test_mfma_probe_validation(lib):
    assert lib.dcn_mfma_probe(A, 0, 10, None) == PARAM
    assert lib.dcn_mfma_probe(A, 4, -1, None) == PARAM
    assert lib.dcn_mfma_probe(None, 4, 10, None) == NULL
    assert lib.dcn_mfma_probe(A + 2, 4, 10, None) == ALIGN
    assert lib.dcn_last_hip_error() == 0
