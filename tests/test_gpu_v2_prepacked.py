"""dcn_v2_pack_weight and dcn_v2_forward_prepacked through the C ABI.

The packed buffer is checked element by element against the layout the header states,
built here on the host by plain indexing of the weight; the prepacked forward runs the
same fused kernel as dcn_v2_forward on the same values, so its output must be
bit-identical to dcn_v2_forward's (which the parity tests check against the oracle),
also when one packed weight serves several calls in a row.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import workloads as wl
from gpu_util import dev

pytestmark = pytest.mark.gpu

CASES = [
    # the 8x256x40x40 bf16 layer
    ("layer_bf16", dict(N=8, Cin=256, H=40, W=40, Cout=256, dtype="bf16")),
    ("f16_cin64", dict(N=2, Cin=64, H=11, W=13, Cout=40, dtype="f16")),
    # Cout over one 256-row block: rows past Cout are padding
    ("cout300", dict(N=1, Cin=128, H=9, W=10, Cout=300, dtype="bf16")),
    ("dg2_softmax", dict(N=2, Cin=256, H=7, W=9, Cout=32, dg=2, mask="logits", dtype="bf16")),
    ("k1x3_stride2", dict(N=1, Cin=64, H=12, W=15, Cout=24, kh=1, kw=3, pad=(0, 1), stride=(2, 2),
                          dtype="f16")),
]


def packed_reference(w):
    """The packed order on the host: weight [Cout, Cin, kh, kw] -> 16-bit words; value
    (co, ci, k) has K index r = k*Cin_pad + ci, and the 8 values (co, 16q + 8h .. +7)
    fill 16-byte slot ((co//32 * Rp//16 + q)*2 + h)*32 + co%32. Padding is zero."""
    Cout, Cin, kh, kw = w.shape
    K = kh * kw
    cin_pad = -(-Cin // 8) * 8
    rp = -(-(K * cin_pad) // 64) * 64
    mp = -(-Cout // 128) * 128
    rows = np.zeros((mp, rp), np.uint16)  # [co][r], tap-major
    wb = w.reshape(Cout, Cin, K)
    for k in range(K):
        rows[:Cout, k * cin_pad:k * cin_pad + Cin] = wb[:, :, k]
    out = np.zeros(mp * rp, np.uint16)
    for co in range(mp):
        for c8 in range(rp // 8):
            q, h = c8 // 2, c8 % 2
            slot = ((co // 32 * (rp // 16) + q) * 2 + h) * 32 + co % 32
            out[slot * 8:slot * 8 + 8] = rows[co, c8 * 8:c8 * 8 + 8]
    return out


@pytest.mark.parametrize("name,args", CASES, ids=[c[0] for c in CASES])
def test_prepacked_matches_forward(gpu, name, args):
    c = wl.v2_case(seed=300 + len(name), w_std=1.0 / np.sqrt(args["Cin"] * 9), **args)
    x, off, w = dev(c["x"]), dev(c["offset"]), dev(c["weight"])
    m = dev(c["mask"]) if c["mask"] is not None else None
    Cout, Cin, kh, kw = w.shape
    print(name, tuple(x.shape), Cout, flush=True)
    kw_ = dict(stride=c["stride"], pad=c["pad"], dilation=c["dil"], deform_groups=c["dg"],
               softmax=c["softmax"])
    packed = dsa.dcn_v2_pack_weight(w)
    ref = dsa.dcn_v2_forward(x, off, m, w, **kw_)
    out = torch.full_like(ref, float("nan"))
    dsa.dcn_v2_forward_prepacked(x, off, m, packed, Cout, out, kernel=(kh, kw), **kw_)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), name
    # the packed layout, element by element (host copy of the weight as 16-bit words)
    wbits = w.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    want = packed_reference(wbits)
    got = packed.cpu().numpy().view(np.uint16)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_prepacked_reused_across_calls(gpu):
    """One packed weight, three inputs in a row (the second with another batch size)."""
    args = dict(Cin=128, H=10, W=12, Cout=64, dtype="bf16")
    w = None
    packed = None
    for i, N in enumerate((3, 1, 3)):
        c = wl.v2_case(N=N, seed=400 + i, w_std=0.05, **args)
        if w is None:
            w = dev(c["weight"])
            packed = dsa.dcn_v2_pack_weight(w)
        x, off, m = dev(c["x"]), dev(c["offset"]), dev(c["mask"])
        print("reuse", i, N, flush=True)
        ref = dsa.dcn_v2_forward(x, off, m, w)
        out = dsa.dcn_v2_forward_prepacked(x, off, m, packed, args["Cout"])
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i


def test_prepacked_rejects_two_stage_layers(gpu):
    """Cin not a multiple of 64: the layer's columns pass through the workspace, so
    the fused kernel's packed weight does not apply (DCN_ERR_PARAM)."""
    c = wl.v2_case(N=1, Cin=16, H=8, W=8, Cout=8, dtype="bf16", seed=5)
    x, off, m, w = dev(c["x"]), dev(c["offset"]), dev(c["mask"]), dev(c["weight"])
    packed = dsa.dcn_v2_pack_weight(w)
    with pytest.raises(dsa.DcnError) as e:
        dsa.dcn_v2_forward_prepacked(x, off, m, packed, 8)
    assert e.value.name == "DCN_ERR_PARAM"
