"""GPU parity of the aggregation backward (deform_agg_backward through the C ABI)
against the CPU oracle's fp64 gradients.

Tolerances as the core backward: every fp32 gradient within 1e-5 of the oracle's
sum of |product terms| for that element; an fp16/bf16 grad_feat additionally within
half an ulp of its value. The full six-camera, four-scale workload is checked whole.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import oracle
import workloads as wl
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

REL = 1e-5
HALF_ULP = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
HALF_TINY = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def _say(*a):
    print(*a, flush=True)


def run(c, go, softmax=None, need=("feat", "loc", "weights"), workspace=None,
        path=dsa.DCN_BWD_DEFAULT):
    sm = c["softmax"] if softmax is None else softmax
    r = dsa.deform_agg_backward(dev(c["feat"]), c["spatial_shape"], c["scale_start"],
                                dev(c["loc"]), dev(c["weights"]), dev(go), softmax=sm, need=need,
                                workspace=workspace, path=path)
    torch.cuda.synchronize()
    return r


def ref(c, go, softmax=None):
    sm = c["softmax"] if softmax is None else softmax
    return oracle.deform_agg_backward(c["feat"], c["spatial_shape"], c["scale_start"], c["loc"],
                                      c["weights"], go, softmax=sm)


def check_grad(g, o, ab, dtype, what):
    g = np.asarray(g, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.all(np.isfinite(g)), what + ": non-finite"
    err = np.abs(g - o)
    bound = REL * ab
    if dtype in HALF_ULP:
        bound = bound + HALF_ULP[dtype] * np.abs(o) + HALF_TINY[dtype]
    bad = err > bound
    assert not bad.any(), "%s: %d of %d beyond bound (worst err %.3g where bound %.3g)" % (
        what, int(bad.sum()), bad.size, float(err[bad].max()), float(bound[bad][np.argmax(err[bad])]))
    return float(err.max(initial=0.0))


def check_all(r, o, dtype, what):
    gf, gl, gw = r
    out = {}
    if gf is not None:
        out["feat"] = check_grad(host(gf), o["grad_feat"], o["grad_feat_abs"], dtype, what + " grad_feat")
    if gl is not None:
        out["loc"] = check_grad(host(gl), o["grad_loc"], o["grad_loc_abs"], "f32", what + " grad_loc")
    if gw is not None:
        out["w"] = check_grad(host(gw), o["grad_weights"], o["grad_weights_abs"], "f32",
                              what + " grad_weights")
    return out


TWO_CAM = [[(12, 20), (6, 10)]] * 2
SWEEP = [
    ("f32_cg32_softmax", dict(B=1, shapes=TWO_CAM, A=16, pts=3, G=4, Cg=32), {}),
    ("f32_cg32_plain", dict(B=1, shapes=TWO_CAM, A=16, pts=3, G=4, Cg=32, weights="simplex"), {}),
    ("f32_cg8_z8", dict(B=2, shapes=TWO_CAM, A=9, pts=2, G=2, Cg=8), {}),
    ("f32_cg5_idle_lanes", dict(B=1, shapes=TWO_CAM, A=7, pts=2, G=3, Cg=5), {}),
    ("f32_cg64_one_slice", dict(B=1, shapes=TWO_CAM, A=6, pts=2, G=2, Cg=64), {}),
    ("f32_cg96_two_rounds", dict(B=1, shapes=TWO_CAM, A=5, pts=2, G=1, Cg=96), {}),
    ("f16_cg32", dict(B=1, shapes=TWO_CAM, A=12, pts=3, G=4, Cg=32, dtype="f16"), {}),
    ("bf16_cg16", dict(B=1, shapes=TWO_CAM, A=12, pts=3, G=4, Cg=16, dtype="bf16"), {}),
    ("f32_three_scales_63_records", dict(B=1, shapes=[[(9, 13), (5, 7), (3, 4)]] * 3, A=8, pts=7,
                                         G=2, Cg=16), {}),
    ("f32_one_scale_64_pairs", dict(B=1, shapes=[[(10, 12)]] * 5, A=6, pts=13, G=2, Cg=16), {}),
    ("f32_locations_outside", dict(B=1, shapes=TWO_CAM, A=10, pts=3, G=2, Cg=32, loc_lo=-0.3,
                                   loc_hi=1.3), {}),
    ("f32_scale_major_layout", dict(B=1, shapes=TWO_CAM, A=8, pts=2, G=2, Cg=32, cam_major=False), {}),
]


@pytest.mark.parametrize("name,args,extra", SWEEP, ids=[s[0] for s in SWEEP])
def test_agg_backward_sweep(gpu, name, args, extra):
    c = wl.agg_case(seed=500 + len(name), **args)
    go = wl.agg_grad_out(c, seed=len(name))
    _say("agg backward sweep", name)
    r = run(c, go, **extra)
    o = ref(c, go, **extra)
    _say(name, check_all(r, o, c["dtype"], name))


def test_agg_backward_six_camera_workload(gpu):
    """The full 6-camera x 4-scale, 900-anchor x 13-point, 8x32-channel workload."""
    name = "agg_f32_6cam_4scale_a900p13_g8c32"
    c = wl.make(name)
    go = wl.agg_grad_out(c, seed=3)
    _say("agg backward full", name)
    r = run(c, go)
    o = ref(c, go)
    _say(name, check_all(r, o, "f32", name))


def test_agg_backward_subsets_and_determinism(gpu):
    c = wl.agg_case(B=1, shapes=TWO_CAM, A=20, pts=3, G=4, Cg=32, seed=41)
    go = wl.agg_grad_out(c, seed=41)
    full = run(c, go)
    again = run(c, go)
    assert torch.equal(full[1], again[1]) and torch.equal(full[2], again[2])
    only_w = run(c, go, need=("weights",))
    only_l = run(c, go, need=("loc",))
    only_f = run(c, go, need=("feat",))
    assert only_w[0] is None and only_w[1] is None
    assert torch.equal(only_w[2], full[2]) and torch.equal(only_l[1], full[1])
    o = ref(c, go)
    check_grad(host(only_f[0]), o["grad_feat"], o["grad_feat_abs"], "f32", "grad_feat alone")


GENERAL = [
    ("f32_cg32_softmax", dict(B=1, shapes=TWO_CAM, A=16, pts=3, G=4, Cg=32)),
    ("f16_cg32", dict(B=1, shapes=TWO_CAM, A=12, pts=3, G=4, Cg=32, dtype="f16")),
    ("bf16_cg16", dict(B=1, shapes=TWO_CAM, A=12, pts=3, G=4, Cg=16, dtype="bf16")),
    ("f32_three_scales_63_records", dict(B=1, shapes=[[(9, 13), (5, 7), (3, 4)]] * 3, A=8, pts=7,
                                         G=2, Cg=16)),
]


@pytest.mark.parametrize("name,args", GENERAL, ids=[s[0] for s in GENERAL])
def test_agg_backward_general_main_kernel(gpu, name, args):
    """The general main kernel on the bucketed path (channel vectors of 4 elements, no
    load pipelining), which 16-byte-vector groups otherwise leave to the pipelined
    kernel; selected through deform_agg_backward_path(DCN_BWD_GENERAL_MAIN)."""
    c = wl.agg_case(seed=900 + len(name), **args)
    go = wl.agg_grad_out(c, seed=len(name))
    _say("agg backward general main kernel", name)
    r = run(c, go, path=dsa.DCN_BWD_GENERAL_MAIN)
    o = ref(c, go)
    _say(name, check_all(r, o, c["dtype"], name))


@pytest.mark.parametrize("softmax", [True, False])
def test_agg_backward_weights_without_workspace(gpu, softmax):
    """grad_weights alone with no workspace (the general kernel) against the oracle and
    against the same call with a workspace (the pipelined kernel and finishing pass)."""
    c = wl.agg_case(B=1, shapes=TWO_CAM, A=20, pts=3, G=4, Cg=32, seed=43)
    go = wl.agg_grad_out(c, seed=43)
    _say("agg backward weights without workspace, softmax", softmax)
    bare = run(c, go, softmax=softmax, need=("weights",), workspace=False)
    full = run(c, go, softmax=softmax, need=("weights",))
    o = ref(c, go, softmax=softmax)
    for r, what in ((bare, "no workspace"), (full, "workspace")):
        assert r[0] is None and r[1] is None
        check_grad(host(r[2]), o["grad_weights"], o["grad_weights_abs"], "f32", what)


FALLBACK = [
    ("f32_cg32_softmax", dict(B=1, shapes=TWO_CAM, A=16, pts=3, G=4, Cg=32)),
    ("bf16_cg16", dict(B=2, shapes=TWO_CAM, A=9, pts=3, G=4, Cg=16, dtype="bf16")),
    ("f32_cg5_outside", dict(B=1, shapes=TWO_CAM, A=7, pts=2, G=3, Cg=5, loc_lo=-0.3, loc_hi=1.3)),
]


@pytest.mark.parametrize("name,args", FALLBACK, ids=[s[0] for s in FALLBACK])
def test_agg_backward_atomic_fallback(gpu, name, args):
    """The fp32-atomic feature gradient (used past the bucket limits), selected here at
    small sizes through deform_agg_backward_path(DCN_BWD_ATOMIC)."""
    c = wl.agg_case(seed=700 + len(name), **args)
    go = wl.agg_grad_out(c, seed=len(name))
    _say("agg backward atomic fallback", name)
    r = run(c, go, path=dsa.DCN_BWD_ATOMIC)
    o = ref(c, go)
    _say(name, check_all(r, o, c["dtype"], name))


def test_agg_backward_hot_rows(gpu):
    """Every sample of 64 anchors on one 3x4 map: hundreds of corners per feature row
    (long buckets, merged per block in LDS)."""
    c = wl.agg_case(B=1, shapes=[[(3, 4)]] * 2, A=64, pts=8, G=2, Cg=32, seed=45)
    go = wl.agg_grad_out(c, seed=46)
    r = run(c, go)
    o = ref(c, go)
    _say("hot rows", check_all(r, o, "f32", "hot rows"))


def test_agg_backward_spare_rows_and_unaligned_grad_out(gpu):
    """Feature rows outside every map get exact zeros; a grad_out whose address is only
    4-byte aligned takes the one-channel gather."""
    c = wl.agg_case(B=1, shapes=TWO_CAM, A=10, pts=3, G=4, Cg=32, seed=43)
    go = wl.agg_grad_out(c, seed=44)
    buf = torch.zeros(go.numel() + 4, device="cuda")
    buf[1:1 + go.numel()] = dev(go).view(-1)
    go_mis = buf[1:1 + go.numel()].view(go.shape)
    r = dsa.deform_agg_backward(dev(c["feat"]), c["spatial_shape"], c["scale_start"], dev(c["loc"]),
                                dev(c["weights"]), go_mis, softmax=True)
    torch.cuda.synchronize()
    o = ref(c, go, softmax=True)
    check_all(r, o, "f32", "unaligned grad_out")
    used = int(sum(h * w for h, w in np.asarray(c["spatial_shape"]).reshape(-1, 2)))
    assert not host(r[0])[:, used:].any()


def test_agg_backward_empty(gpu):
    c = wl.agg_case(B=1, shapes=TWO_CAM, A=0, pts=3, G=4, Cg=32, seed=1)
    go = torch.zeros((1, 0, 128))
    gf, gl, gw = run(c, go)
    assert gf.shape == c["feat"].shape and gl.numel() == 0 and gw.numel() == 0
