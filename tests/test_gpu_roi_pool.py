"""GPU parity of deformable RoI pooling (deform_roi_pool_forward through the C ABI)
against the CPU oracle.

Both sides form every sample position by the same fixed sequence of fp32 operations
(each rounded once; stated with the oracle), so they sample at identical positions and
differ only by the fp32 accumulation of the weighted corners and the mean. Bound per
element: 1e-5 of the oracle's sum of |product terms|; fp16/bf16 outputs add half an ulp
of the value.
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


def run(c):
    out = dsa.deform_roi_pool_forward(dev(c["x"]), dev(c["rois"]), dev(c["offset"]),
                                      output_size=c["k"], sampling_ratio=c["S"],
                                      spatial_scale=c["spatial_scale"], gamma=c["gamma"])
    torch.cuda.synchronize()
    return host(out)


def check(c, g, what):
    o, ab = oracle.deform_roi_pool(c["x"], c["rois"], c["offset"], k=c["k"], S=c["S"],
                                   spatial_scale=c["spatial_scale"], gamma=c["gamma"])
    assert g.shape == o.shape
    assert np.all(np.isfinite(g)), what
    err = np.abs(g - o)
    bound = REL * ab
    if c["dtype"] in HALF_ULP:
        bound = bound + HALF_ULP[c["dtype"]] * np.abs(o) + HALF_TINY[c["dtype"]]
    bad = err > bound
    assert not bad.any(), "%s: %d beyond bound (worst %.3g)" % (what, int(bad.sum()), float(err.max()))
    return float(err.max())


SWEEP = [
    ("f32_c64_k7_s2", dict(N=2, H=20, W=24, C=64, R=24, k=7, S=2, spatial_scale=0.25)),
    ("f32_c5_scalar", dict(N=1, H=9, W=11, C=5, R=10, k=3, S=2, spatial_scale=1.0)),
    ("f32_c6_vec2", dict(N=1, H=12, W=10, C=6, R=8, k=2, S=3, spatial_scale=0.5)),
    ("f16_c32_vec8", dict(N=2, H=16, W=16, C=32, R=16, k=7, S=2, spatial_scale=0.125, dtype="f16")),
    ("bf16_c128_four_bins_per_wave", dict(N=1, H=14, W=18, C=128, R=12, k=4, S=1, dtype="bf16",
                                         spatial_scale=0.5)),
    ("f32_c320_rounds", dict(N=1, H=8, W=9, C=320, R=5, k=2, S=2, spatial_scale=1.0)),
    ("f32_no_offsets", dict(N=2, H=20, W=20, C=16, R=20, k=5, S=2, spatial_scale=0.25, offsets=False)),
    ("f32_gamma_one_far_samples", dict(N=1, H=16, W=16, C=16, R=16, k=3, S=2, gamma=1.0,
                                       spatial_scale=0.5)),
    ("f32_k1_s1", dict(N=1, H=7, W=7, C=8, R=9, k=1, S=1, spatial_scale=1.0)),
]


@pytest.mark.parametrize("name,args", SWEEP, ids=[s[0] for s in SWEEP])
def test_roi_pool_sweep(gpu, name, args):
    c = wl.roi_case(seed=700 + len(name), **args)
    _say("roi pool sweep", name)
    _say(name, check(c, run(c), name))


def test_roi_pool_named_workload(gpu):
    c = wl.make("droi_f32_n2_64x64_c256_r512_k7")
    _say("roi pool full workload")
    _say("droi", check(c, run(c), "droi_f32_n2_64x64_c256_r512_k7"))


def test_roi_pool_bad_batch_index_and_degenerate_rois(gpu):
    """A RoI naming no image pools to zeros; zero-size and inverted RoIs sample one
    point (or mirror) exactly as the oracle says; deterministic (no atomics)."""
    c = wl.roi_case(N=2, H=10, W=12, C=8, R=6, k=2, S=2, spatial_scale=1.0, seed=9)
    rois = c["rois"].clone()
    rois[0, 0] = 5.0                      # no such image
    rois[1, 3:] = rois[1, 1:3]            # zero width and height
    rois[2, [1, 3]] = rois[2, [3, 1]]     # inverted x
    c["rois"] = rois
    g = run(c)
    assert not g[0].any()
    c_ok = dict(c, rois=rois[1:], offset=c["offset"][1:], R=5)
    check(c_ok, g[1:], "degenerate rois")
    assert np.array_equal(g, run(c))
