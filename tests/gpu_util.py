"""Helpers for the GPU parity tests: run the library on seeded inputs and compare
with the CPU oracle under the stated tolerances."""
import numpy as np
import torch

import deformable_sampling_amd as dsa
import oracle

FP32_REL = 1e-5   # fp32 accumulation: |g - o| <= 1e-5 * (sum of |product terms|), and vs max|o|
HALF_ABS = 2e-2   # fp16/bf16 outputs: also within 2e-2 absolute everywhere
# unit roundoff of one round-to-nearest-even to the storage type (half an ulp, relative)
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# half the spacing of the type's subnormals (the absolute floor of a rounding)
HALF_TINY = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}
_KEYS = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def dev(t):
    return None if t is None else t.to("cuda").contiguous()


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def half_bound(o, ab, key, operand_rounding=False):
    """Elementwise bound for an fp16/bf16 output computed with fp32 accumulation and
    rounded once to the type: the fp32 sum is within 1e-5 * A_i of the exact value o_i,
    and rounding that sum moves it by at most u times its magnitude. With
    operand_rounding, the operands of the contraction (DCNv2's sampled columns) were
    themselves rounded to the type first, which moves the sum by at most u * A_i more."""
    u = UNIT_ROUNDOFF[key]
    ab = np.asarray(ab, np.float64)
    b = FP32_REL * ab * (1.0 + u) + u * np.abs(o) + HALF_TINY[key]
    if operand_rounding:
        b = b + u * (1.0 + u) * ab
    return b


def check(g, o, ab, dtype, what="", operand_rounding=False):
    """g: GPU result (fp64 numpy), o: oracle fp64, ab: oracle sum of |terms|.
    Returns a dict of error statistics; raises AssertionError beyond tolerance."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    assert np.all(np.isfinite(g)), what + ": non-finite GPU output"
    key = _KEYS.get(dtype, dtype)
    err = np.abs(g - o)
    stats = dict(max_abs=float(err.max(initial=0.0)), max_out=float(np.abs(o).max(initial=0.0)))
    if key == "f32":
        bound = FP32_REL * np.asarray(ab, np.float64)
    else:
        bound = half_bound(o, ab, key, operand_rounding)
    bad = err > bound
    stats["max_err_over_bound"] = float((err / np.maximum(bound, 1e-300)).max(initial=0.0))
    assert not bad.any(), "%s: %d elements beyond the bound (worst err %.3g where the bound is %.3g)" % (
        what, int(bad.sum()), float(err[bad].max()), float(bound[bad][np.argmax(err[bad])]))
    if key == "f32":
        assert stats["max_abs"] <= FP32_REL * max(stats["max_out"], 1e-300), (what, stats)
    else:
        assert stats["max_abs"] <= HALF_ABS, (what, stats)
    return stats


def run_core(c, offset_scale=1.0, softmax=None, mask="keep"):
    sm = c["softmax"] if softmax is None else softmax
    m = c["mask"] if mask == "keep" else mask
    out = dsa.dcn_core_forward(dev(c["x"]), dev(c["offset"]), dev(m), kernel=(c["kh"], c["kw"]),
                               stride=c["stride"], pad=c["pad"], dilation=c["dil"],
                               offset_scale=offset_scale, softmax=sm)
    torch.cuda.synchronize()
    return out


def oracle_core(c, offset_scale=1.0, softmax=None, mask="keep", pix=None):
    sm = c["softmax"] if softmax is None else softmax
    m = c["mask"] if mask == "keep" else mask
    return oracle.dcn_core(c["x"], c["offset"], m, kh=c["kh"], kw=c["kw"], stride=c["stride"],
                           pad=c["pad"], dil=c["dil"], offset_scale=offset_scale, softmax=sm,
                           pix=pix)


def sample_pixels(N, Ho, Wo, n, seed):
    """n random output pixels plus every image's four corners and its first/last rows."""
    r = np.random.default_rng(seed)
    sel = set(r.integers(0, N * Ho * Wo, size=n).tolist())
    for img in range(N):
        base = img * Ho * Wo
        sel.update(base + np.arange(Wo))
        sel.update(base + (Ho - 1) * Wo + np.arange(Wo))
        sel.update(base + np.arange(Ho) * Wo)
        sel.update(base + np.arange(Ho) * Wo + Wo - 1)
    return np.array(sorted(sel), dtype=np.int64)


def v2_workspace_layout(N, Cin, H, W, Cout, kh, kw, Ho, Wo):
    """Offsets (bytes) and row length (elements) of the DCNv2 workspace regions, as
    documented with dcn_v2_workspace_bytes: channels-last x, permuted weight, columns."""
    a256 = lambda v: (v + 255) // 256 * 256
    rup = lambda v, m: (v + m - 1) // m * m
    cin_pad = rup(Cin, 8)
    R = kh * kw * cin_pad
    Rp = rup(R, 64)
    Mp = rup(Cout, 128)
    off_wp = a256(N * H * W * cin_pad * 2)
    off_col = off_wp + a256(Mp * Rp * 2)
    return dict(cin_pad=cin_pad, R=R, Rp=Rp, off_col=off_col)
