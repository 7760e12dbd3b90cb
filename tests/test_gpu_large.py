"""GPU parity at the 2-GiB limits of one buffer resource.

Each op addresses an input through 32-bit buffer offsets when it fits in 2 GiB and
switches to 64-bit global addresses beyond that; these tests run the larger form:
  - the core forward on an fp16 image of exactly 2 GiB (1 x 2048 x 2048 x 256): the
    tile kernel stages its regions with global-address copies;
  - DCNv2 on a bf16 input of 2 GiB (1 x 256 x 2048 x 2048): the channels-last copy no
    longer fits a buffer, so the columns go through the workspace (19 GB of them) and
    the two-stage GEMM;
  - the aggregation over 2.7 GB of fp32 features: the kernel without buffer loads.
Inputs are seeded draws made on the GPU (workloads.*_device). The core and DCNv2
results are checked by translation: the op on a 76 x 76 crop of the input (a small
image, the well-tested buffer path) gives the same outputs, bit for bit, wherever the
crop holds every tap (offsets are drawn within +-4 px, the crop keeps a 6-px margin),
and sampled pixels of those windows are checked against the oracle on the crop. The
aggregation is checked against the oracle on every anchor.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import oracle
import workloads as wl
from gpu_util import check, host

pytestmark = pytest.mark.gpu

CROP = 76
MARGIN = 6  # taps of a pixel reach at most 5 px beyond it with |offset| < 4


def _say(*a):
    print(*a, flush=True)


def _windows(H, W):
    # a corner window (taps leaving the image), one inside, and the opposite corner
    return [(0, 0), (H // 2 - 37, W // 2 - 29), (H - CROP, W - CROP)]


def _interior(y0, x0, H, W):
    """Rows/columns of a crop whose pixels' taps all stay inside the crop (a crop edge
    on an image edge needs no margin: the taps beyond it are outside both)."""
    ylo = 0 if y0 == 0 else MARGIN
    yhi = CROP if y0 + CROP == H else CROP - MARGIN
    xlo = 0 if x0 == 0 else MARGIN
    xhi = CROP if x0 + CROP == W else CROP - MARGIN
    return ylo, yhi, xlo, xhi


def _sample(ylo, yhi, xlo, xhi, n, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    ys = r.integers(ylo, yhi, n)
    xs = r.integers(xlo, xhi, n)
    return np.unique(ys * CROP + xs)


def test_core_fp16_image_of_2gib(gpu):
    N, H, W, G, C = 1, 2048, 2048, 16, 16
    _say("core 2 GiB: drawing inputs")
    c = wl.core_case_device(N=N, H=H, W=W, G=G, C=C, dtype="f16", offset_range=4.0, seed=31)
    assert c["x"].numel() * c["x"].element_size() == 1 << 31
    out = dsa.dcn_core_forward(c["x"], c["offset"], c["mask"])
    torch.cuda.synchronize()
    _say("core 2 GiB: full launch done")
    for i, (y0, x0) in enumerate(_windows(H, W)):
        sl = (slice(None), slice(y0, y0 + CROP), slice(x0, x0 + CROP))
        xc = c["x"][sl].contiguous()
        oc = c["offset"][sl].contiguous()
        mc = c["mask"][sl].contiguous()
        outc = dsa.dcn_core_forward(xc, oc, mc)
        torch.cuda.synchronize()
        ylo, yhi, xlo, xhi = _interior(y0, x0, H, W)
        assert torch.equal(outc[:, ylo:yhi, xlo:xhi], out[:, y0 + ylo:y0 + yhi, x0 + xlo:x0 + xhi]), (y0, x0)
        pix = _sample(ylo, yhi, xlo, xhi, 300, seed=40 + i)
        o, ab = oracle.dcn_core(xc.cpu(), oc.cpu(), mc.cpu(), kh=3, kw=3, stride=(1, 1), pad=(1, 1),
                                dil=(1, 1), pix=pix)
        st = check(host(out[sl].contiguous()).reshape(-1, G * C)[pix], o, ab, "f16", "core 2GiB window %d" % i)
        _say("core 2 GiB window", (y0, x0), len(pix), "pixels", st)


def test_dcn_v2_bf16_input_of_2gib(gpu):
    N, Cin, H, W, Cout = 1, 256, 2048, 2048, 32
    _say("dcnv2 2 GiB: drawing inputs")
    c = wl.v2_case_device(N=N, Cin=Cin, H=H, W=W, Cout=Cout, dtype="bf16", offset_range=4.0,
                          w_std=1.0 / np.sqrt(Cin * 9), seed=32)
    assert c["x"].numel() * c["x"].element_size() == 1 << 31
    need = dsa.dcn_v2_workspace_bytes(N, Cin, H, W, Cout, dtype=torch.bfloat16)
    _say("dcnv2 2 GiB: workspace %.1f GB" % (need / 1e9))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = dsa.dcn_v2_forward(c["x"], c["offset"], c["mask"], c["weight"], workspace=ws)
    torch.cuda.synchronize()
    del ws
    _say("dcnv2 2 GiB: full call done")
    for i, (y0, x0) in enumerate(_windows(H, W)):
        sl = (slice(None), slice(None), slice(y0, y0 + CROP), slice(x0, x0 + CROP))
        xc = c["x"][sl].contiguous()
        oc = c["offset"][sl].contiguous()
        mc = c["mask"][sl].contiguous()
        outc = dsa.dcn_v2_forward(xc, oc, mc, c["weight"])  # Cin % 64 == 0: columns on chip
        torch.cuda.synchronize()
        ylo, yhi, xlo, xhi = _interior(y0, x0, H, W)
        assert torch.equal(outc[:, :, ylo:yhi, xlo:xhi], out[:, :, y0 + ylo:y0 + yhi, x0 + xlo:x0 + xhi]), (y0, x0)
        pix = _sample(ylo, yhi, xlo, xhi, 200, seed=50 + i)
        o, ab = oracle.dcn_v2(xc.cpu(), oc.cpu(), mc.cpu(), c["weight"].cpu(), stride=(1, 1), pad=(1, 1),
                              dil=(1, 1), pix=pix)
        g = host(out[sl].contiguous())  # [1, Cout, CROP, CROP]
        g = g.reshape(Cout, CROP * CROP).T[pix]
        st = check(g, o, ab, "bf16", "dcnv2 2GiB window %d" % i, operand_rounding=True)
        _say("dcnv2 2 GiB window", (y0, x0), len(pix), "pixels", st)


def test_aggregation_features_over_2gib(gpu):
    shapes = [[(512, 640), (256, 320), (128, 160), (64, 80)]] * 6
    _say("aggregation 2.7 GB: drawing inputs")
    c = wl.agg_case_device(B=1, shapes=shapes, A=48, pts=13, G=8, Cg=32, seed=33)
    assert c["feat"].numel() * 4 > (1 << 31)
    out = dsa.deform_agg_forward(c["feat"], c["spatial_shape"], c["scale_start"], c["loc"],
                                 c["weights"], softmax=True)
    torch.cuda.synchronize()
    _say("aggregation 2.7 GB: launch done; oracle")
    o, ab = oracle.deform_agg(c["feat"].cpu(), c["spatial_shape"], c["scale_start"], c["loc"].cpu(),
                              c["weights"].cpu(), softmax=True)
    st = check(host(out), o, ab, "f32", "aggregation 2.7 GB")
    _say("aggregation 2.7 GB", st)
