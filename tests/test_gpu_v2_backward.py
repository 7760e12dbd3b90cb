"""GPU parity of the DCNv2 backward (dcn_v2_backward through the C ABI) against the
CPU oracle's fp64 derivative.

Bounds per element, from the arithmetic: grad_offset and grad_mask within 1e-5 of
the oracle's sum of |product terms| (fp32 throughout); grad_x within the same plus
half an ulp of its dtype (one output rounding); grad_weight contracts grad_out with
the forward's columns rounded to the dtype, so each product term carries one more
relative error of at most the dtype's unit roundoff u (2^-8 bf16, 2^-11 fp16):
within (u + 1e-5) of its sum of |terms|.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import oracle
import workloads as wl
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}  # unit roundoff: 8- and 11-bit significands
TINY = {"bf16": 2.0 ** -134, "f16": 2.0 ** -25}
REL = 1e-5


def _say(*a):
    print(*a, flush=True)


def run(c, go, need=("x", "offset", "mask", "weight")):
    r = dsa.dcn_v2_backward(dev(c["x"]), dev(c["offset"]), dev(c["mask"]), dev(c["weight"]), dev(go),
                            stride=c["stride"], pad=c["pad"], dilation=c["dil"],
                            deform_groups=c["dg"], softmax=c["softmax"], need=need)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in r.items()}


def ref(c, go):
    return oracle.dcn_v2_backward(c["x"], c["offset"], c["mask"], c["weight"], go, stride=c["stride"],
                                  pad=c["pad"], dil=c["dil"], softmax=c["softmax"])


def compare(g, o, dtype, what):
    stats = {}
    for name in g:
        err = np.abs(g[name] - o[name])
        ab = o[name + "_abs"]
        if name == "grad_weight":
            bound = (UNIT[dtype] + REL) * ab
        elif name == "grad_x":
            bound = REL * ab + UNIT[dtype] * np.abs(o[name]) + TINY[dtype]
        else:
            bound = REL * ab
        assert np.all(np.isfinite(g[name])), (what, name)
        bad = err > bound
        assert not bad.any(), "%s %s: %d beyond bound (worst err %.3g)" % (
            what, name, int(bad.sum()), float(err.max()))
        stats[name] = float(err.max())
    return stats


SWEEP = [
    ("bf16_small", dict(N=2, Cin=16, H=9, W=11, Cout=24, dtype="bf16")),
    ("f16_small", dict(N=2, Cin=16, H=9, W=11, Cout=24, dtype="f16")),
    ("bf16_cin3_pad", dict(N=1, Cin=3, H=12, W=10, Cout=5, dtype="bf16")),
    ("bf16_cin20_cout130", dict(N=1, Cin=20, H=7, W=13, Cout=130, dtype="bf16")),
    ("bf16_dg2", dict(N=2, Cin=32, H=8, W=9, Cout=16, dg=2, dtype="bf16")),
    ("f16_dg4_c128", dict(N=1, Cin=128, H=8, W=9, Cout=64, dg=4, dtype="f16")),
    ("bf16_stride2", dict(N=1, Cin=16, H=15, W=14, Cout=16, stride=(2, 2), dtype="bf16")),
    ("bf16_dil2", dict(N=1, Cin=16, H=12, W=12, Cout=16, pad=(2, 2), dil=(2, 2), dtype="bf16")),
    ("bf16_k1x3", dict(N=1, Cin=8, H=9, W=10, Cout=8, kh=1, kw=3, pad=(0, 1), dtype="bf16")),
    ("bf16_mask_none", dict(N=1, Cin=16, H=8, W=8, Cout=8, mask=None, dtype="bf16")),
    ("bf16_softmax", dict(N=1, Cin=16, H=8, W=8, Cout=8, mask="logits", dtype="bf16")),
    ("f16_softmax_dg2", dict(N=2, Cin=32, H=7, W=9, Cout=20, dg=2, mask="logits", dtype="f16")),
    ("bf16_far_offsets", dict(N=1, Cin=16, H=10, W=11, Cout=16, offset_std=12.0, dtype="bf16")),
    ("bf16_c320_many_pixels", dict(N=2, Cin=320, H=13, W=17, Cout=72, dtype="bf16")),
    ("bf16_1x1_image", dict(N=3, Cin=8, H=1, W=1, Cout=8, dtype="bf16")),
    # Cin a multiple of 64: the weight gradient with the columns formed on chip (several
    # pixel splits, grad_out channels past one 256-row block, tiny pixel counts, softmax)
    ("bf16_c64_stride2", dict(N=2, Cin=64, H=11, W=13, Cout=40, stride=(2, 2), dtype="bf16")),
    ("f16_c128_softmax", dict(N=1, Cin=128, H=7, W=9, Cout=24, mask="logits", dtype="f16")),
    ("bf16_c64_cout300", dict(N=1, Cin=64, H=6, W=7, Cout=300, dtype="bf16")),
    ("bf16_c64_1x1_image", dict(N=3, Cin=64, H=1, W=1, Cout=8, dtype="bf16")),
    ("bf16_c128_dg2", dict(N=1, Cin=128, H=8, W=9, Cout=32, dg=2, dtype="bf16")),  # 64 channels per group
]


@pytest.mark.parametrize("name,args", SWEEP, ids=[s[0] for s in SWEEP])
def test_v2_backward_sweep(gpu, name, args):
    K = args.get("kh", 3) * args.get("kw", 3)
    c = wl.v2_case(seed=500 + len(name), w_std=1.0 / np.sqrt(args["Cin"] * K), **args)
    go = wl.v2_grad_out(c, seed=501)
    _say("v2 backward", name)
    g = run(c, go)
    _say(name, compare(g, ref(c, go), c["dtype"], name))


def test_v2_backward_named_workload(gpu):
    """The 8x256x40x40 bf16 layer, every gradient element against the oracle."""
    name = "dcnv2_bf16_n8_c256_40x40"
    c = wl.make(name)
    go = wl.v2_grad_out(c, seed=502)
    _say("v2 backward", name)
    g = run(c, go)
    _say("oracle ...")
    o = ref(c, go)
    _say(name, compare(g, o, "bf16", name))


def test_v2_backward_subsets_and_repeat(gpu):
    """Requesting a subset of the gradients gives the same values; offset, mask and
    weight gradients are bitwise reproducible."""
    c = wl.v2_case(N=2, Cin=32, H=9, W=10, Cout=24, dg=2, dtype="bf16", seed=77,
                   w_std=1.0 / np.sqrt(32 * 9))
    go = wl.v2_grad_out(c, seed=78)
    full = run(c, go)
    again = run(c, go)
    for k in ("grad_offset", "grad_mask", "grad_weight"):
        assert np.array_equal(full[k], again[k]), k
    o = ref(c, go)
    for need in (("x",), ("weight",), ("offset", "mask"), ("mask",)):
        part = run(c, go, need=need)
        assert set(part) == {"grad_" + n for n in need}
        compare(part, o, "bf16", "subset %s" % (need,))
        for k in part:
            if k != "grad_x":
                assert np.array_equal(part[k], full[k]), k


def test_v2_backward_integer_inputs_bit_exact(gpu):
    """Small-integer x, weight and grad_out with integer offsets and no mask: every
    product and sum is an exact integer in fp32, so all four gradients equal the
    oracle's bit for bit (grad_x after its bf16 rounding)."""
    c = wl.v2_case(N=2, Cin=8, H=9, W=10, Cout=12, dtype="bf16", mask=None, seed=9, x_kind="int")
    c["offset"] = torch.round(c["offset"])
    go = wl.v2_grad_out(c, seed=10, kind="int")
    g = run(c, go)
    o = ref(c, go)
    assert np.array_equal(g["grad_x"], torch.from_numpy(o["grad_x"]).bfloat16().double().numpy())
    for k in ("grad_offset", "grad_mask", "grad_weight"):
        assert np.array_equal(g[k], o[k]), k


def test_v2_backward_empty_batch(gpu):
    c = wl.v2_case(N=1, Cin=8, H=6, W=6, Cout=8, dtype="bf16", seed=1)
    x = torch.zeros((0, 8, 6, 6), dtype=torch.bfloat16, device="cuda")
    off = torch.zeros((0, 18, 6, 6), device="cuda")
    go = torch.zeros((0, 8, 6, 6), dtype=torch.bfloat16, device="cuda")
    r = dsa.dcn_v2_backward(x, off, None, dev(c["weight"]), go)
    assert r["grad_x"].shape == (0, 8, 6, 6)
