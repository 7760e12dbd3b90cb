"""GPU parity of the core backward (dcn_core_backward through the C ABI) against
the CPU oracle's fp64 gradients.

Tolerances: every fp32 result (grad_offset, grad_mask, and grad_x for fp32 x)
within 1e-5 of the oracle's sum of |product terms| for that element; an fp16/bf16
grad_x additionally within half an ulp of its value (one rounding of the fp32
accumulator). Integer inputs are bit-exact. The full-size detector workload is
launched whole and checked on two of its images (each image's gradients depend on
that image alone).
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


def run_bwd(c, go, offset_scale=1.0, softmax=None, mask="keep", need=("x", "offset", "mask"),
            path=dsa.DCN_BWD_DEFAULT):
    sm = c["softmax"] if softmax is None else softmax
    m = c["mask"] if mask == "keep" else mask
    r = dsa.dcn_core_backward(dev(c["x"]), dev(c["offset"]), dev(m), dev(go),
                              kernel=(c["kh"], c["kw"]), stride=c["stride"], pad=c["pad"],
                              dilation=c["dil"], offset_scale=offset_scale, softmax=sm, need=need,
                              path=path)
    torch.cuda.synchronize()
    return r


def oracle_bwd(c, go, offset_scale=1.0, softmax=None, mask="keep", images=None):
    sm = c["softmax"] if softmax is None else softmax
    m = c["mask"] if mask == "keep" else mask
    x, off = c["x"], c["offset"]
    if images is not None:
        x, off, go = x[images], off[images], go[images]
        m = None if m is None else m[images]
    return oracle.dcn_core_backward(x, off, m, go, kh=c["kh"], kw=c["kw"], stride=c["stride"],
                                    pad=c["pad"], dil=c["dil"], offset_scale=offset_scale,
                                    softmax=sm, G=c["G"])


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


def check_all(r, o, dtype, what, images=None):
    gx, goff, gm = r
    sel = (lambda t: t) if images is None else (lambda t: t[images])
    out = {}
    if gx is not None:
        out["x"] = check_grad(host(sel(gx)), o["grad_x"], o["grad_x_abs"], dtype, what + " grad_x")
    if goff is not None:
        out["off"] = check_grad(host(sel(goff)), o["grad_offset"], o["grad_offset_abs"], "f32",
                                what + " grad_offset")
    if gm is not None:
        out["mask"] = check_grad(host(sel(gm)), o["grad_mask"], o["grad_mask_abs"], "f32",
                                 what + " grad_mask")
    return out


BWD_SWEEP = [
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
    ("f32_k8x8_lds_cap", dict(N=1, H=12, W=12, G=2, C=4, kh=8, kw=8, pad=(3, 3), dtype="f32"), {}),
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
    ("f16_wide_c1024_two_rounds", dict(N=1, H=4, W=5, G=1, C=1024, dtype="f16"), {}),
    ("f16_many_groups", dict(N=1, H=8, W=8, G=32, C=8, dtype="f16"), {}),
    ("f16_c1040_uneven_rounds", dict(N=1, H=3, W=4, G=1, C=1040, dtype="f16"), {}),
    ("f32_tiles_exact_32x48", dict(N=1, H=32, W=48, G=2, C=4, offset_std=6.0, dtype="f32"), {}),
    ("bf16_tiles_ragged_37x21", dict(N=2, H=37, W=21, G=2, C=16, offset_std=4.0, dtype="bf16"), {}),
    ("f32_c48_three_gather_rounds", dict(N=1, H=18, W=17, G=1, C=48, dtype="f32"), {}),
]


@pytest.mark.parametrize("name,args,extra", BWD_SWEEP, ids=[s[0] for s in BWD_SWEEP])
def test_backward_sweep(gpu, name, args, extra):
    c = wl.core_case(seed=300 + len(name), **args)
    go = wl.core_grad_out(c, seed=len(name))
    _say("core backward sweep", name)
    r = run_bwd(c, go, **extra)
    o = oracle_bwd(c, go, **extra)
    _say(name, check_all(r, o, c["dtype"], name))


@pytest.mark.parametrize("name", ["dcnv4_f32_n1_32x32_g4c16", "dcnv3_f32_n8_56x56_g4c16_softmax"])
def test_backward_named_workload_full(gpu, name):
    c = wl.make(name)
    go = wl.core_grad_out(c, seed=11)
    _say("core backward full", name)
    r = run_bwd(c, go)
    o = oracle_bwd(c, go)
    _say(name, check_all(r, o, c["dtype"], name))


def test_backward_detector_p3_fp16_two_images(gpu):
    """fp16 x [16,80,80,256], G=16, C=16, 3x3, 5% of taps outside the image: the
    whole batch in one launch; images 0 and 15 checked against the oracle."""
    name = "dcnv4_f16_n16_80x80_g16c16"
    c = wl.make(name)
    go = wl.core_grad_out(c, seed=12)
    _say("core backward sampled", name)
    r = run_bwd(c, go)
    for img in (0, 15):
        o = oracle_bwd(c, go, images=[img])
        _say(name, "image", img, check_all(r, o, "f16", name, images=[img]))


def test_backward_integer_inputs_bit_exact(gpu):
    """Small-integer x and grad_out, integer offsets, unit modulation: all products
    and sums are exact integers in fp32 whatever the summation order, and integer
    positions take the right derivative on both sides, so all three gradients equal
    the oracle bit for bit (fp16 grad_x too: the integers are representable)."""
    c = wl.core_case(N=2, H=12, W=13, G=3, C=8, dtype="f32", mask="ones", seed=5, x_kind="int")
    c["offset"] = torch.round(c["offset"] * 2)
    go = wl.core_grad_out(c, seed=5, kind="int")
    o = oracle_bwd(c, go)
    for dt in ("f32", "f16"):
        cc = dict(c, x=c["x"].to(wl.DTYPES[dt]), dtype=dt)
        r = run_bwd(cc, go.to(wl.DTYPES[dt]))
        assert np.array_equal(host(r[0]), o["grad_x"]), dt
        assert np.array_equal(host(r[1]), o["grad_offset"]), dt
        assert np.array_equal(host(r[2]), o["grad_mask"]), dt


def test_backward_subsets_and_determinism(gpu):
    """Asking for one gradient gives the same values as asking for all; grad_offset
    and grad_mask are bitwise reproducible; grad_x agrees within fp32 rounding."""
    c = wl.core_case(N=2, H=10, W=11, G=2, C=16, dtype="f16", offset_std=4.0, seed=9)
    go = wl.core_grad_out(c, seed=9)
    full = run_bwd(c, go)
    again = run_bwd(c, go)
    assert torch.equal(full[1], again[1]) and torch.equal(full[2], again[2])
    only_x = run_bwd(c, go, need=("x",))
    only_off = run_bwd(c, go, need=("offset",))
    only_m = run_bwd(c, go, need=("mask",))
    assert only_x[1] is None and only_x[2] is None
    assert torch.equal(only_off[1], full[1]) and torch.equal(only_m[2], full[2])
    o = oracle_bwd(c, go)
    check_grad(host(only_x[0]), o["grad_x"], o["grad_x_abs"], "f16", "grad_x alone")


def test_backward_one_tile_receives_every_sample(gpu):
    """Every sample of a 48x48 map lands inside input tile (1, 1): that tile's gather
    walks its records in several LDS chunks, all other tiles have none."""
    c = wl.core_case(N=1, H=48, W=48, G=2, C=8, dtype="f32", seed=21)
    r = np.random.default_rng(21)
    Ho, Wo, K = c["Ho"], c["Wo"], 9
    ho = np.arange(Ho).reshape(Ho, 1, 1, 1)
    wo = np.arange(Wo).reshape(1, Wo, 1, 1)
    ki = (np.arange(K) // 3).reshape(1, 1, 1, K)
    kj = (np.arange(K) % 3).reshape(1, 1, 1, K)
    ty = r.uniform(16.0, 31.0, (Ho, Wo, 2, K))
    tx = r.uniform(16.0, 31.0, (Ho, Wo, 2, K))
    off = np.stack([tx - (wo - 1 + kj), ty - (ho - 1 + ki)], -1)[None]
    c["offset"] = torch.from_numpy(off).float().contiguous()
    go = wl.core_grad_out(c, seed=21)
    res = run_bwd(c, go)
    o = oracle_bwd(c, go)
    gx = host(res[0])
    assert not gx[:, :16].any() and not gx[:, 32:].any() and not gx[:, :, :16].any()
    _say("one tile", check_all(res, o, "f32", "one tile"))


FALLBACK_CASES = [s for s in BWD_SWEEP if s[0] in (
    "f32_vec4_tails", "f16_vec8", "bf16_scalar_c3", "f32_softmax", "f32_k5x5",
    "f16_c1040_uneven_rounds")]


@pytest.mark.parametrize("name,args,extra", FALLBACK_CASES, ids=[s[0] for s in FALLBACK_CASES])
def test_backward_atomic_fallback(gpu, name, args, extra):
    """The fp32-atomic fallback (used beyond the record packing's limits), selected
    here at small sizes through dcn_core_backward_path(DCN_BWD_ATOMIC)."""
    c = wl.core_case(seed=300 + len(name), **args)
    go = wl.core_grad_out(c, seed=len(name))
    _say("core backward atomic fallback", name)
    r = run_bwd(c, go, path=dsa.DCN_BWD_ATOMIC, **extra)
    o = oracle_bwd(c, go, **extra)
    _say(name, check_all(r, o, c["dtype"], name))


PAIR_GRADS = ["f32_vec4_tails", "f16_vec8", "f32_far_offsets", "f32_softmax", "f16_many_groups"]


@pytest.mark.parametrize("name", PAIR_GRADS)
def test_backward_pair_pass_gradients(gpu, name):
    """grad_offset / grad_mask from the pair pass (DCN_BWD_PAIR_PASS) on shapes whose
    default path computes them in the LDS-tiled kernel: both paths meet the bound."""
    args, extra = {n: (a, e) for n, a, e in BWD_SWEEP}[name]
    c = wl.core_case(seed=100 + len(name), **args)
    go = wl.core_grad_out(c, seed=len(name))
    _say("core backward pair-pass gradients", name)
    r = run_bwd(c, go, path=dsa.DCN_BWD_PAIR_PASS, **extra)
    o = oracle_bwd(c, go, **extra)
    _say(name, check_all(r, o, c["dtype"], name))


@pytest.mark.parametrize("name", ["f32_vec4_tails", "f16_vec8", "f16_many_groups", "f32_far_offsets"])
def test_backward_unstaged_gather(gpu, name):
    """grad_x through the gather that reads grad_out per visit (DCN_BWD_UNSTAGED_GATHER)
    on shapes whose default gather stages each record's grad_out slice in LDS."""
    args, extra = {n: (a, e) for n, a, e in BWD_SWEEP}[name]
    c = wl.core_case(seed=100 + len(name), **args)
    go = wl.core_grad_out(c, seed=len(name))
    _say("core backward unstaged gather", name)
    r = run_bwd(c, go, path=dsa.DCN_BWD_UNSTAGED_GATHER, **extra)
    o = oracle_bwd(c, go, **extra)
    _say(name, check_all(r, o, c["dtype"], name))


@pytest.mark.parametrize("name", ["f32_vec4_tails", "f16_vec8", "f32_far_offsets", "f32_softmax"])
def test_backward_pair_pass_records(gpu, name):
    """grad_x records filed by the pair pass (DCN_BWD_PAIR_PASS_RECORDS) while the tiled
    kernel computes grad_offset / grad_mask: the default files them in the tiled kernel
    on these shapes."""
    args, extra = {n: (a, e) for n, a, e in BWD_SWEEP}[name]
    c = wl.core_case(seed=100 + len(name), **args)
    go = wl.core_grad_out(c, seed=len(name))
    _say("core backward pair-pass records", name)
    r = run_bwd(c, go, path=dsa.DCN_BWD_PAIR_PASS_RECORDS, **extra)
    o = oracle_bwd(c, go, **extra)
    _say(name, check_all(r, o, c["dtype"], name))


def test_backward_empty_batch(gpu):
    x = torch.zeros((0, 4, 4, 8), device="cuda")
    off = torch.zeros((0, 4, 4, 2, 9, 2), device="cuda")
    go = torch.zeros((0, 4, 4, 8), device="cuda")
    gx, goff, gm = dsa.dcn_core_backward(x, off, None, go)
    assert gx.shape == (0, 4, 4, 8) and goff.shape == off.shape and gm.shape == (0, 4, 4, 2, 9)
