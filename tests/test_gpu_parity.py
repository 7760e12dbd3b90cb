"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Seeded synthetic inputs; fp32 within 1e-5 of the sum of |product terms| A_i (and of
max|out| globally); fp16/bf16 outputs within 1e-5 * A_i plus one rounding to the type
(and, for DCNv2, one more rounding of the sampled columns per product term: u * A_i),
and within 2e-2 absolute everywhere; integer cases bit-exact. Full-size workloads are
compared on sampled outputs the oracle computes one by one, in the same launch
configuration the bench times.
"""
import numpy as np
import pytest
import torch

import deformable_sampling_amd as dsa
import oracle
import workloads as wl
from gpu_util import (check, dev, host, oracle_core, run_core, sample_pixels,
                      v2_workspace_layout)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ core ----

@pytest.mark.parametrize("name", ["dcnv4_f32_n1_32x32_g4c16", "dcnv3_f32_n8_56x56_g4c16_softmax"])
def test_core_named_workload_full(gpu, name):
    c = wl.make(name)
    _say("core full", name)
    g = host(run_core(c))
    o, ab = oracle_core(c)
    st = check(g, o, ab, c["dtype"], name)
    _say(name, st)


def test_core_detector_p3_fp16_sampled(gpu):
    name = "dcnv4_f16_n16_80x80_g16c16"
    c = wl.make(name)
    _say("core sampled", name)
    g = host(run_core(c))
    assert g.shape == (16, 80, 80, 256)
    pix = sample_pixels(16, 80, 80, 3000, seed=7)
    o, ab = oracle_core(c, pix=pix)
    st = check(g.reshape(-1, 256)[pix], o, ab, "f16", name)
    _say(name, len(pix), "pixels", st)
    # forced out-of-image taps contribute exactly nothing: changing their masks
    # leaves the GPU output bit-identical
    m2 = c["mask"].clone()
    m2[torch.from_numpy(c["oob"])] = 7.0
    g2 = host(run_core(c, mask=m2))
    assert np.array_equal(g, g2)


CORE_SWEEP = [
    # name, dict(core_case args), extra
    ("f32_vec4_tails", dict(N=2, H=13, W=17, G=3, C=8, dtype="f32"), {}),
    ("f32_scalar_c5", dict(N=1, H=9, W=11, G=2, C=5, dtype="f32"), {}),
    ("f32_vec2_c6", dict(N=1, H=7, W=9, G=2, C=6, dtype="f32"), {}),
    ("f16_vec8", dict(N=2, H=11, W=10, G=4, C=16, dtype="f16"), {}),
    ("f16_vec4_c12", dict(N=1, H=10, W=12, G=2, C=12, dtype="f16"), {}),
    ("bf16_vec8", dict(N=1, H=12, W=9, G=2, C=32, dtype="bf16"), {}),
    ("bf16_scalar_c3", dict(N=1, H=6, W=7, G=5, C=3, dtype="bf16"), {}),
    ("f32_stride2", dict(N=2, H=15, W=14, G=2, C=8, stride=(2, 2), dtype="f32"), {}),
    ("f32_dil2_pad2", dict(N=1, H=12, W=13, G=2, C=8, pad=(2, 2), dil=(2, 2), dtype="f32"), {}),
    ("f32_pad0", dict(N=1, H=10, W=10, G=1, C=4, pad=(0, 0), dtype="f32"), {}),
    ("f32_k3x5", dict(N=1, H=11, W=16, G=2, C=4, kh=3, kw=5, pad=(1, 2), dtype="f32"), {}),
    ("f32_k1", dict(N=2, H=6, W=5, G=3, C=4, kh=1, kw=1, pad=(0, 0), dtype="f32"), {}),
    ("f32_k5x5", dict(N=1, H=9, W=9, G=2, C=8, kh=5, kw=5, pad=(2, 2), dtype="f32"), {}),
    ("f32_1x1_image", dict(N=3, H=1, W=1, G=2, C=4, dtype="f32"), {}),
    ("f32_g1_c1", dict(N=1, H=8, W=8, G=1, C=1, dtype="f32"), {}),
    ("f32_mask_none", dict(N=1, H=9, W=10, G=2, C=8, mask=None, dtype="f32"), {}),
    ("f32_softmax", dict(N=2, H=9, W=10, G=2, C=8, mask="logits", dtype="f32"), {}),
    ("f32_softmax_c5_s5", dict(N=1, H=7, W=8, G=3, C=5, mask="logits", dtype="f32"), {}),
    ("f32_softmax_nomask", dict(N=1, H=6, W=6, G=2, C=4, mask=None, dtype="f32"), {"softmax": True}),
    ("f16_softmax", dict(N=1, H=10, W=9, G=4, C=16, mask="logits", dtype="f16"), {}),
    ("f32_far_offsets", dict(N=1, H=10, W=12, G=2, C=8, offset_std=20.0, dtype="f32"), {}),
    ("f32_oob_30pct", dict(N=1, H=10, W=12, G=2, C=8, oob_frac=0.3, dtype="f32"), {}),
    ("f32_offset_scale", dict(N=1, H=10, W=11, G=2, C=8, offset_std=3.0, dtype="f32"), {"offset_scale": 0.37}),
    ("f32_wide_c320", dict(N=1, H=5, W=6, G=1, C=320, dtype="f32"), {}),
    ("f16_many_groups", dict(N=1, H=8, W=8, G=32, C=8, dtype="f16"), {}),
    # more tiles than compute units, several tile rows per column: the band kernel
    # (persistent blocks carrying window rows from band to band), 20- and 16-wide tiles,
    # partial last bands and columns, softmax, no mask, far offsets, offset_scale, fp32
    ("f16_bands_tw20", dict(N=12, H=70, W=60, G=8, C=16, dtype="f16", oob_frac=0.05,
                            offset_std=3.0), {}),
    ("f16_bands_tw16_softmax", dict(N=10, H=50, W=45, G=8, C=16, mask="logits", dtype="f16"), {}),
    ("f16_bands_far_nomask", dict(N=12, H=34, W=41, G=8, C=16, offset_std=6.0, mask=None,
                                  dtype="f16"), {"offset_scale": 0.7}),
    ("f32_bands_c8", dict(N=12, H=40, W=40, G=8, C=8, dtype="f32", offset_std=3.0,
                          oob_frac=0.05), {}),
]


@pytest.mark.parametrize("name,args,extra", CORE_SWEEP, ids=[s[0] for s in CORE_SWEEP])
def test_core_sweep(gpu, name, args, extra):
    c = wl.core_case(seed=100 + len(name), **args)
    _say("core sweep", name)
    g = host(run_core(c, **extra))
    o, ab = oracle_core(c, **extra)
    st = check(g, o, ab, c["dtype"], name)
    _say(name, st)


def test_core_integer_inputs_bit_exact(gpu):
    """Small-integer x, integer offsets, unit masks: every product and partial sum is
    an exact integer in fp32, so the GPU must equal the oracle bit for bit."""
    c = wl.core_case(N=2, H=12, W=13, G=3, C=8, dtype="f32", mask="ones", seed=5, x_kind="int")
    c["offset"] = torch.round(c["offset"] * 2)
    g = host(run_core(c))
    o, _ = oracle_core(c)
    assert np.array_equal(g, o)
    c16 = dict(c, x=c["x"].half(), dtype="f16")
    g16 = host(run_core(c16))
    assert np.array_equal(g16, torch.from_numpy(o).half().double().numpy())


def test_core_deterministic_and_guard_region(gpu):
    """Two runs are bit-identical (no atomics); NaN sentinels around x are never read;
    a 4-byte-aligned (not 16-byte) x takes the scalar path with the same result."""
    c = wl.core_case(N=2, H=10, W=11, G=2, C=8, dtype="f32", offset_std=6.0, seed=8)
    n = c["x"].numel()
    buf = torch.full((n + 64,), float("nan"), device="cuda")
    buf[1:1 + n] = dev(c["x"]).view(-1)
    x_mis = buf[1:1 + n].view(c["x"].shape)  # 4-byte aligned only, NaN on both sides
    o_dev = dev(c["offset"])
    m_dev = dev(c["mask"])
    kw_ = dict(kernel=(3, 3), stride=1, pad=1, dilation=1)
    a = dsa.dcn_core_forward(dev(c["x"]), o_dev, m_dev, **kw_)
    b = dsa.dcn_core_forward(dev(c["x"]), o_dev, m_dev, **kw_)
    s = dsa.dcn_core_forward(x_mis, o_dev, m_dev, **kw_)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.isfinite(s).all()
    o, ab = oracle_core(c)
    check(host(s), o, ab, "f32", "scalar path")
    check(host(a), o, ab, "f32", "vector path")


def test_core_empty_batch(gpu):
    x = torch.zeros((0, 4, 4, 8), device="cuda")
    off = torch.zeros((0, 4, 4, 2, 9, 2), device="cuda")
    out = dsa.dcn_core_forward(x, off, None)
    assert out.shape == (0, 4, 4, 8)


# -------------------------------------------------------------------- v2 ----

def run_v2(c, workspace=None):
    out = dsa.dcn_v2_forward(dev(c["x"]), dev(c["offset"]), dev(c["mask"]), dev(c["weight"]),
                             workspace=workspace, stride=c["stride"], pad=c["pad"],
                             dilation=c["dil"], deform_groups=c["dg"], softmax=c["softmax"])
    torch.cuda.synchronize()
    return out


def oracle_v2(c, pix=None):
    return oracle.dcn_v2(c["x"], c["offset"], c["mask"], c["weight"], stride=c["stride"],
                         pad=c["pad"], dil=c["dil"], softmax=c["softmax"], pix=pix)


def test_v2_named_workload_sampled(gpu):
    name = "dcnv2_bf16_n8_c256_40x40"
    c = wl.make(name)
    _say("v2 sampled", name)
    N, Cin, H, W, Cout = 8, 256, 40, 40, 256
    need = dsa.dcn_v2_workspace_bytes(N, Cin, H, W, Cout, dtype=torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    g = host(run_v2(c, workspace=ws))
    pix = sample_pixels(N, 40, 40, 400, seed=9)
    o, ab = oracle_v2(c, pix=pix)
    assert np.abs(o).max() < 4.0  # bf16 output rounding stays below 2e-2
    g_pix = g.transpose(0, 2, 3, 1).reshape(-1, Cout)[pix]
    st = check(g_pix, o, ab, "bf16", name, operand_rounding=True)
    _say(name, "out", st)
    # the deform-im2col stage on its own: columns in the workspace vs the oracle's
    ws.zero_()
    dsa.dcn_v2_im2col(dev(c["x"]), dev(c["offset"]), dev(c["mask"]), Cout, ws)
    torch.cuda.synchronize()
    lay = v2_workspace_layout(N, Cin, H, W, Cout, 3, 3, 40, 40)
    col = ws[lay["off_col"]:lay["off_col"] + 12800 * lay["Rp"] * 2].view(torch.bfloat16)
    col = col.view(12800, lay["Rp"])[:, :lay["R"]].reshape(12800, 9, lay["cin_pad"])[:, :, :Cin]
    col_g = host(col[torch.from_numpy(pix).cuda()].permute(0, 2, 1).reshape(len(pix), Cin * 9))
    col_o = oracle.dcn_v2_columns(c["x"], c["offset"], c["mask"], kh=3, kw=3, pad=(1, 1), pix=pix)
    cerr = np.abs(col_g - col_o)
    assert (cerr <= 2.0 ** -8 * np.abs(col_o) + 1e-6).all(), float(cerr.max())
    _say(name, "columns max err", float(cerr.max()))


V2_SWEEP = [
    ("bf16_small", dict(N=2, Cin=16, H=9, W=11, Cout=24, dtype="bf16")),
    ("f16_small", dict(N=2, Cin=16, H=9, W=11, Cout=24, dtype="f16")),
    ("bf16_cin3_pad", dict(N=1, Cin=3, H=12, W=10, Cout=5, dtype="bf16")),
    ("bf16_cin20", dict(N=1, Cin=20, H=7, W=13, Cout=130, dtype="bf16")),
    ("bf16_dg2", dict(N=2, Cin=32, H=8, W=9, Cout=16, dg=2, dtype="bf16")),
    ("bf16_stride2", dict(N=1, Cin=16, H=15, W=14, Cout=16, stride=(2, 2), dtype="bf16")),
    ("bf16_dil2", dict(N=1, Cin=16, H=12, W=12, Cout=16, pad=(2, 2), dil=(2, 2), dtype="bf16")),
    ("bf16_k1x3", dict(N=1, Cin=8, H=9, W=10, Cout=8, kh=1, kw=3, pad=(0, 1), dtype="bf16")),
    ("bf16_mask_none", dict(N=1, Cin=16, H=8, W=8, Cout=8, mask=None, dtype="bf16")),
    ("bf16_softmax", dict(N=1, Cin=16, H=8, W=8, Cout=8, mask="logits", dtype="bf16")),
    # softmax with no mask tensor: every kernel point gets the uniform modulation 1/K
    ("bf16_softmax_mask_none", dict(N=1, Cin=16, H=8, W=8, Cout=8, mask=None, dtype="bf16"),
     dict(softmax=True)),
    ("bf16_many_pixels", dict(N=3, Cin=64, H=23, W=29, Cout=96, dtype="bf16")),
    # Cin a multiple of 64: columns formed inside the GEMM. Pixel counts that are not
    # multiples of the 64-pixel block, Cout over one 256-channel block, groups, softmax
    ("fused_f16", dict(N=2, Cin=64, H=11, W=13, Cout=40, dtype="f16")),
    ("fused_cout300", dict(N=1, Cin=128, H=9, W=10, Cout=300, dtype="bf16")),
    ("fused_dg4", dict(N=2, Cin=128, H=8, W=9, Cout=64, dg=4, dtype="bf16")),
    ("fused_softmax_stride2", dict(N=1, Cin=64, H=15, W=14, Cout=32, stride=(2, 2),
                                   mask="logits", dtype="bf16")),
    ("fused_mask_none_dil2", dict(N=1, Cin=64, H=12, W=12, Cout=16, pad=(2, 2), dil=(2, 2),
                                  mask=None, dtype="f16")),
    ("fused_k1x3", dict(N=1, Cin=64, H=9, W=10, Cout=8, kh=1, kw=3, pad=(0, 1), dtype="bf16")),
    ("fused_softmax_mask_none", dict(N=2, Cin=64, H=10, W=11, Cout=24, dg=2, mask=None,
                                     dtype="bf16"), dict(softmax=True)),
    # Cin of 128 and 256: two and four 64-channel K steps per tap, with two groups of
    # 128 channels, a 1x3 window (an odd number of steps) and the softmax
    ("fused_wide_dg2", dict(N=1, Cin=256, H=7, W=9, Cout=32, dg=2, dtype="bf16")),
    ("fused_wide_f16_k1x3", dict(N=1, Cin=128, H=6, W=10, Cout=48, kh=1, kw=3, pad=(0, 1),
                                 dtype="f16")),
    ("fused_wide_softmax", dict(N=2, Cin=128, H=9, W=8, Cout=72, mask="logits", dtype="bf16")),
    # 3x3 at stride 1 and dilation 1 with one group: the staged-region kernel (8x8 pixel
    # tiles, partial at the image edge; 1, 2, 3 and 5 channel blocks), other paddings, no
    # mask, softmax without mask, and offsets wide enough that many taps leave the
    # +-6-px region and are read from memory
    ("region_pad0_mask_none", dict(N=1, Cin=64, H=13, W=17, Cout=40, pad=(0, 0), mask=None,
                                   dtype="bf16")),
    ("region_softmax_mask_none_f16", dict(N=2, Cin=128, H=9, W=12, Cout=24, mask=None, dtype="f16"),
     dict(softmax=True)),
    ("region_far_taps_pad21", dict(N=1, Cin=64, H=20, W=21, Cout=32, pad=(2, 1), offset_std=6.0,
                                   dtype="bf16")),
    ("region_cin192", dict(N=1, Cin=192, H=10, W=9, Cout=16, dtype="bf16")),
    ("region_cin320_softmax", dict(N=1, Cin=320, H=6, W=7, Cout=8, mask="logits", dtype="f16")),
]
V2_SWEEP = [s if len(s) == 3 else s + ({},) for s in V2_SWEEP]


@pytest.mark.parametrize("name,args,extra", V2_SWEEP, ids=[s[0] for s in V2_SWEEP])
def test_v2_sweep(gpu, name, args, extra):
    K = args.get("kh", 3) * args.get("kw", 3)
    c = wl.v2_case(seed=200 + len(name), w_std=1.0 / np.sqrt(args["Cin"] * K), **args)
    c.update(extra)
    _say("v2 sweep", name)
    g = host(run_v2(c))
    o, ab = oracle_v2(c)
    assert np.abs(o).max() < 4.0
    st = check(g, o, ab, c["dtype"], name, operand_rounding=True)
    _say(name, st)


def test_v2_integer_inputs_bit_exact(gpu):
    c = wl.v2_case(N=2, Cin=8, H=9, W=10, Cout=12, dtype="bf16", mask=None, seed=6, x_kind="int")
    c["offset"] = torch.round(c["offset"])
    g = host(run_v2(c))
    o, _ = oracle_v2(c)
    # exact integer sums, rounded once to bf16 on both sides
    assert np.array_equal(g, torch.from_numpy(o).bfloat16().double().numpy())


# ------------------------------------------------------------ aggregation ----

def run_agg(c, softmax=None):
    sm = c["softmax"] if softmax is None else softmax
    out = dsa.deform_agg_forward(dev(c["feat"]), c["spatial_shape"], c["scale_start"],
                                 dev(c["loc"]), dev(c["weights"]), softmax=sm)
    torch.cuda.synchronize()
    return out


def oracle_agg(c, softmax=None, anchors=None):
    sm = c["softmax"] if softmax is None else softmax
    return oracle.deform_agg(c["feat"], c["spatial_shape"], c["scale_start"], c["loc"],
                             c["weights"], softmax=sm, anchors=anchors)


@pytest.mark.parametrize("weights", ["logits", "simplex"])
def test_agg_named_workload(gpu, weights):
    name = "agg_f32_6cam_4scale_a900p13_g8c32"
    c = wl.make(name, weights=weights)
    _say("agg", name, weights)
    g = host(run_agg(c))
    anchors = np.arange(0, 900, 3)
    o, ab = oracle_agg(c, anchors=anchors)
    st = check(g[0][anchors], o, ab, "f32", name)
    _say(name, weights, st)


AGG_SWEEP = [
    ("f32_small", dict(B=2, shapes=[[(9, 13), (5, 7)], [(6, 10), (3, 5)]], A=37, pts=3, G=2, Cg=8)),
    ("f32_scale_major", dict(B=1, shapes=[[(9, 13), (5, 7)], [(6, 10), (3, 5)]], A=21, pts=2, G=2,
                             Cg=8, cam_major=False)),
    ("f32_cg5_scalar", dict(B=1, shapes=[[(7, 9)]] * 3, A=19, pts=4, G=3, Cg=5)),
    ("f32_cg24_nonpow2", dict(B=1, shapes=[[(8, 12), (4, 6)]], A=10, pts=5, G=2, Cg=24)),
    ("f32_cg320_wide", dict(B=1, shapes=[[(5, 6)]], A=6, pts=2, G=1, Cg=320)),
    ("f32_loc_outside", dict(B=1, shapes=[[(10, 16), (5, 8)]] * 2, A=40, pts=3, G=4, Cg=8,
                             loc_lo=-0.3, loc_hi=1.3)),
    ("f16_small", dict(B=1, shapes=[[(9, 13), (5, 7)]] * 2, A=33, pts=3, G=2, Cg=16, dtype="f16")),
    ("bf16_small", dict(B=1, shapes=[[(9, 13), (5, 7)]] * 2, A=33, pts=3, G=2, Cg=16, dtype="bf16")),
    # group channels of 64/128/256 bytes: the pipelined paths with 4/8/16 lanes per slice
    # (camera-phased where a camera's taps, scales x points, fit one 64-tap chunk);
    # T = pts*cams*scales below one 64-tap chunk, just over one, and several with a tail
    ("f32_cg16_s4_t12", dict(B=2, shapes=[[(9, 13), (5, 7)], [(6, 10), (3, 5)]], A=37, pts=3,
                             G=2, Cg=16)),
    ("f32_cg32_s8_t81", dict(B=1, shapes=[[(12, 20), (6, 10), (3, 5)]] * 3, A=45, pts=9, G=3,
                             Cg=32)),
    ("f32_cg64_s16_t68", dict(B=1, shapes=[[(8, 11), (4, 6)]] * 2, A=13, pts=17, G=2, Cg=64)),
    ("f32_cg32_s8_t312", dict(B=1, shapes=[[(6, 9), (3, 5), (2, 3), (1, 2)]] * 6, A=9, pts=13,
                              G=2, Cg=32)),
    ("f16_cg32_s4_t130", dict(B=2, shapes=[[(10, 14)]] * 5, A=11, pts=26, G=3, Cg=32,
                              dtype="f16")),
    ("bf16_cg64_s8_t40", dict(B=1, shapes=[[(9, 13), (5, 7)]] * 4, A=27, pts=5, G=2, Cg=64,
                              dtype="bf16")),
    ("bf16_cg128_s16_t24", dict(B=1, shapes=[[(7, 9), (4, 5), (2, 3)]] * 2, A=7, pts=4, G=1,
                                Cg=128, dtype="bf16")),
    # the camera-phased grid over more units than one round (9003 units: a full round of
    # four units per wavefront, then 811 split unevenly over the eight XCD ranges)
    ("f32_cg32_s8_rounds", dict(B=1, shapes=[[(6, 8), (3, 4)]] * 2, A=3001, pts=2, G=3, Cg=32)),
    # 80 taps per camera (scales x points > 64): the unit-at-a-time pipelined kernel
    ("f32_cg32_s8_sp80", dict(B=1, shapes=[[(6, 9), (3, 5), (2, 3), (1, 2)]] * 2, A=9, pts=20,
                              G=2, Cg=32)),
    ("bf16_cg64_s8_sp72", dict(B=2, shapes=[[(9, 13), (5, 7), (3, 4)]] * 3, A=5, pts=24, G=2,
                               Cg=64, dtype="bf16")),
]


@pytest.mark.parametrize("softmax", [True, False])
@pytest.mark.parametrize("name,args", AGG_SWEEP, ids=[s[0] for s in AGG_SWEEP])
def test_agg_sweep(gpu, name, args, softmax):
    c = wl.agg_case(seed=300 + len(name), weights="logits" if softmax else "simplex", **args)
    _say("agg sweep", name, softmax)
    g = host(run_agg(c))
    o, ab = oracle_agg(c)
    st = check(g, o, ab, c["dtype"], name)
    _say(name, softmax, st)


@pytest.mark.parametrize("Cg", [8, 32])
def test_agg_masked_logits(gpu, Cg):
    # -inf logits (masked taps) get softmax weight 0. Anchor 0 has every tap of its
    # first 64 (camera-major) masked, so the running maximum starts at -inf; anchor 1 is
    # masked everywhere except one tap; elsewhere 30% of the logits are masked.
    c = wl.agg_case(B=1, shapes=[[(6, 9), (3, 5), (2, 3), (1, 2)]] * 6, A=12, pts=13, G=2,
                    Cg=Cg, seed=77)
    w = c["weights"].clone()  # [B, A, pts, cams, scales, G]
    rng = np.random.default_rng(5)
    w[torch.from_numpy(rng.random(w.shape) < 0.3)] = -float("inf")
    w[0, 0, :, :3] = -float("inf")  # cameras 0-2 of anchor 0: its first 156 camera-major taps
    w[0, 1] = -float("inf")
    w[0, 1, 7, 4, 2] = 0.5
    c["weights"] = w
    _say("agg masked logits", Cg)
    g = host(run_agg(c))
    o, ab = oracle_agg(c)
    assert np.isfinite(o).all()
    st = check(g, o, ab, c["dtype"], "agg masked Cg=%d" % Cg)
    _say(Cg, st)


def test_agg_deterministic(gpu):
    c = wl.agg_case(B=1, shapes=[[(16, 20), (8, 10)]] * 3, A=50, pts=4, G=4, Cg=8, seed=17)
    a = run_agg(c)
    b = run_agg(c)
    assert torch.equal(a, b)
