"""GPU parity of dcn_core_forward_packed: DCNv4's packed offset+mask tensor in fp32,
fp16 or bf16 (per group K (dx, dy) pairs then K masks, pixel rows possibly padded).

Half-precision offsets and masks are widened exactly, so the oracle takes the same
values widened to fp64 and the bars are those of the unpacked forward. With fp32
values the packed call runs the same arithmetic as dcn_core_forward and must equal
it bit for bit, on the LDS-tiled path and on the direct path.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import workloads as wl
from gpu_util import check, dev, host, oracle_core, run_core, sample_pixels

pytestmark = pytest.mark.gpu

OMT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _say(*a):
    print(*a, flush=True)


def _quantise(c, om):
    """The case with its offsets and masks rounded to the packed element type."""
    t = OMT[om]
    q = dict(c)
    q["offset"] = c["offset"].to(t).float()
    q["mask"] = None if c["mask"] is None else c["mask"].to(t).float()
    return q


def _run_packed(c, om, stride=None, offset_scale=1.0, softmax=None):
    sm = c["softmax"] if softmax is None else softmax
    packed = dsa.pack_offset_mask(dev(c["offset"]), dev(c["mask"]), dtype=OMT[om], pixel_stride=stride)
    out = dsa.dcn_core_forward_packed(dev(c["x"]), packed, groups=c["G"], kernel=(c["kh"], c["kw"]),
                                      stride=c["stride"], pad=c["pad"], dilation=c["dil"],
                                      offset_scale=offset_scale, softmax=sm)
    torch.cuda.synchronize()
    return out


PACKED = [
    # name, core_case args, packed dtype, pixel stride padding (elements), extra
    ("tile_f32_om_f16", dict(N=2, H=13, W=17, G=3, C=8, dtype="f32"), "f16", 0, {}),
    ("tile_f32_om_bf16", dict(N=1, H=12, W=11, G=2, C=16, dtype="f32"), "bf16", 0, {}),
    ("tile_f16_om_f16_pad6", dict(N=2, H=11, W=10, G=4, C=16, dtype="f16"), "f16", 6, {}),
    ("tile_bf16_om_bf16", dict(N=1, H=12, W=9, G=2, C=32, dtype="bf16"), "bf16", 0, {}),
    ("tile_f16_om_f32_pad2", dict(N=1, H=10, W=12, G=2, C=16, dtype="f16"), "f32", 2, {}),
    ("tile_f32_softmax_om_f16", dict(N=2, H=9, W=10, G=2, C=8, mask="logits", dtype="f32"), "f16", 0, {}),
    ("tile_f32_nomask_om_f16", dict(N=1, H=9, W=10, G=2, C=8, mask=None, dtype="f32"), "f16", 0, {}),
    ("tile_f32_far_om_f16", dict(N=1, H=10, W=12, G=2, C=8, offset_std=20.0, dtype="f32"), "f16", 0, {}),
    ("tile_f32_scale_om_bf16", dict(N=1, H=10, W=11, G=2, C=8, offset_std=3.0, dtype="f32"), "bf16", 0,
     {"offset_scale": 0.37}),
    ("direct_f32_c5_om_f16", dict(N=1, H=9, W=11, G=2, C=5, dtype="f32"), "f16", 0, {}),
    ("direct_f32_k3x5_om_bf16", dict(N=1, H=11, W=16, G=2, C=4, kh=3, kw=5, pad=(1, 2), dtype="f32"),
     "bf16", 3, {}),
    ("direct_f32_stride2_om_f16", dict(N=2, H=15, W=14, G=2, C=8, stride=(2, 2), dtype="f32"), "f16", 0, {}),
    ("direct_bf16_c3_softmax_om_f16", dict(N=1, H=6, W=7, G=5, C=3, mask="logits", dtype="bf16"), "f16", 1,
     {}),
    ("direct_f32_wide_c320_om_f16", dict(N=1, H=5, W=6, G=1, C=320, dtype="f32"), "f16", 0, {}),
]


@pytest.mark.parametrize("name,args,om,padding,extra", PACKED, ids=[p[0] for p in PACKED])
def test_packed_sweep(gpu, name, args, om, padding, extra):
    c = _quantise(wl.core_case(seed=300 + len(name), **args), om)
    K = c["kh"] * c["kw"]
    _say("packed", name)
    g = host(_run_packed(c, om, stride=c["G"] * 3 * K + padding, **extra))
    o, ab = oracle_core(c, **extra)
    _say(name, check(g, o, ab, c["dtype"], name))


@pytest.mark.parametrize("args", [dict(N=2, H=13, W=17, G=3, C=8, dtype="f32", mask="logits"),
                                  dict(N=1, H=9, W=11, G=2, C=5, dtype="f32")],
                         ids=["tile", "direct"])
def test_packed_f32_equals_unpacked_bitwise(gpu, args):
    c = wl.core_case(seed=41, offset_std=4.0, **args)
    a = host(run_core(c))
    b = host(_run_packed(c, "f32", stride=c["G"] * 3 * 9 + 5))
    assert np.array_equal(a, b)


def test_packed_headline_fp16_sampled(gpu):
    """The detector P3 workload with a packed fp16 offset+mask tensor, rows padded to
    a multiple of 8 elements (16 * 27 = 432 already is), sampled against the oracle."""
    c = _quantise(wl.make("dcnv4_f16_n16_80x80_g16c16"), "f16")
    _say("packed headline")
    g = host(_run_packed(c, "f16"))
    pix = sample_pixels(16, 80, 80, 2000, seed=11)
    o, ab = oracle_core(c, pix=pix)
    _say("packed headline", check(g.reshape(-1, 256)[pix], o, ab, "f16", "packed headline"))
    # same values through the unpacked call: identical output
    assert np.array_equal(g, host(run_core(c)))


def test_packed_empty_and_misaligned(gpu):
    x = torch.zeros((0, 4, 4, 8), device="cuda")
    om = torch.zeros((0, 4, 4, 54), device="cuda", dtype=torch.float16)
    out = dsa.dcn_core_forward_packed(x, om, groups=2)
    assert out.shape == (0, 4, 4, 8)
    c = _quantise(wl.core_case(N=1, H=6, W=7, G=2, C=8, dtype="f32", seed=3), "f16")
    packed = dsa.pack_offset_mask(dev(c["offset"]), dev(c["mask"]), dtype=torch.float16)
    n = packed.numel()
    buf = torch.zeros(n + 8, device="cuda", dtype=torch.float16)
    buf[1:1 + n] = packed.view(-1)
    shifted = buf[1:1 + n].view(packed.shape)  # 2-byte aligned only: scalar loads on every path
    out = dsa.dcn_core_forward_packed(dev(c["x"]), shifted, groups=2)
    torch.cuda.synchronize()
    o, ab = oracle_core(c)
    check(host(out), o, ab, "f32", "2-byte aligned packed")
