"""dcn_v2_forward_noalloc (the library's static workspace) against dcn_v2_forward (a
caller workspace) through the C ABI: the same kernels on the same inputs, so the outputs
must be bit-identical, and both meet the oracle's bound. Calls in a row with different
shapes reuse the one static array: a large fused call, then smaller ones (the two-stage
path, whose columns pass through the array, and a small fused call), then the large one
again.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import oracle
import workloads as wl
from gpu_util import check, dev, host

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(c):
    x, off, m, w = dev(c["x"]), dev(c["offset"]), dev(c["mask"]), dev(c["weight"])
    kw_ = dict(stride=c["stride"], pad=c["pad"], dilation=c["dil"], deform_groups=c["dg"],
               softmax=c["softmax"])
    ref = dsa.dcn_v2_forward(x, off, m, w, **kw_)
    out = torch.full_like(ref, float("nan"))
    dsa.dcn_v2_forward_noalloc(x, off, m, w, out, **kw_)
    torch.cuda.synchronize()
    return out, ref


def _oracle_check(c, g, pix=None):
    o, ab = oracle.dcn_v2(c["x"], c["offset"], c["mask"], c["weight"], stride=c["stride"],
                          pad=c["pad"], dil=c["dil"], softmax=c["softmax"], pix=pix)
    if pix is None:  # the oracle returns [N, Cout, Ho, Wo]
        return check(g, o, ab, c["dtype"], "noalloc", operand_rounding=True)
    Cout = c["weight"].shape[0]
    gp = g.transpose(0, 2, 3, 1).reshape(-1, Cout)[pix]  # the oracle: [npix, Cout]
    return check(gp, o, ab, c["dtype"], "noalloc", operand_rounding=True)


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row(gpu):
    big = wl.make("dcnv2_bf16_n8_c256_40x40")
    small = wl.v2_case(N=2, Cin=16, H=9, W=11, Cout=24, dtype="bf16", seed=501, w_std=0.08)
    small_fused = wl.v2_case(N=1, Cin=64, H=10, W=11, Cout=40, dg=2, mask=None, dtype="f16",
                             seed=502, w_std=0.04)
    small_fused["softmax"] = True
    need = [dsa.dcn_v2_noalloc_bytes(c["N"], c["Cin"], c["H"], c["W"], c["weight"].shape[0],
                                     deform_groups=c["dg"], dtype=c["x"].dtype)
            for c in (big, small, small_fused)]
    assert need[1] < need[0] and need[2] < need[0], need
    for i, (name, c) in enumerate((("8x256x40x40 fused", big), ("2x16x9x11 two-stage", small),
                                   ("1x64x10x11 fused softmax", small_fused),
                                   ("8x256x40x40 fused again", big))):
        _say("noalloc call", i, name)
        out, ref = _both(c)
        assert torch.equal(out, ref), name
        g = host(out)
        if c is big:
            pix = np.random.default_rng(i).integers(0, 8 * 40 * 40, 200)
            _say(name, _oracle_check(c, g, pix))
        else:
            _say(name, _oracle_check(c, g))
