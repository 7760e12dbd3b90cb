"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle.c (a swapped pair, a wrong sign
or index, a dropped term, a transposed operand), builds it with gcc into a
temporary library, and runs the pin suite against it in a subprocess. The pins
must fail for every mutant; the unmodified source must pass.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, occurrence to replace: 1-based)
MUTANTS = [
    ("core_swap_dx_dy", "fl32_mul(offset_scale, om[2 * k + 1])", "fl32_mul(offset_scale, om[2 * k + 0])", 1),
    ("core_pad_sign", "(double)(ho * sh - ph + i * dh)", "(double)(ho * sh + ph + i * dh)", 1),
    ("core_no_dilation", "(double)(wo * sw - pw + j * dw)", "(double)(wo * sw - pw + j)", 1),
    ("core_point_order_col_major", "int64_t k = i * kw + j;", "int64_t k = j * kh + i;", 1),
    ("core_group_channel_base", "x + n * H * W * GC + g * C + c", "x + n * H * W * GC + c", 1),
    ("core_mask_group_stride", "mask + (p * G + g) * K", "mask + p * K", 1),
    ("bilinear_weights_transposed", "double wx[2] = {1.0 - fx, fx};", "double wx[2] = {fx, 1.0 - fx};", 1),
    ("bilinear_drop_corner", "for (int dx = 0; dx < 2; ++dx)", "for (int dx = 0; dx < 1; ++dx)", 1),
    ("bilinear_edge_off_by_one", "qy >= (double)H", "qy > (double)H", 1),
    ("softmax_no_max_shift", "m[i] = exp(l[i * lstride] - mx);", "m[i] = exp(l[i * lstride]);", 1),
    ("softmax_no_normalise", "for (int64_t i = 0; i < n; ++i) m[i] /= den;", "", 1),
    ("v2_swap_dx_dy", "double dx = offset[(oc + 0) * HWo + r];", "double dx = offset[(oc + 1) * HWo + r];", 1),
    ("v2_mask_ignores_group", "mask[(n * dg * K + g * K + k) * HWo + r]", "mask[(n * dg * K + k) * HWo + r]", 1),
    ("v2_weight_transposed", "s += wr[rr] * col[rr];", "s += weight[(rr % Cout) * R + rr / Cout] * col[rr];", 1),
    ("v2_point_order_col_major", "int64_t k = i * kw + j;", "int64_t k = j * kh + i;", 3),
    ("v2_softmax_null_mask_unit", "for (int64_t k = 0; k < K; ++k) m[k] = 1.0 / (double)K;",
     "for (int64_t k = 0; k < K; ++k) m[k] = 1.0;", 1),
    ("agg_no_half_pixel", "(double)(float)(uv[0] * (double)Ws) - 0.5", "(double)(float)(uv[0] * (double)Ws)", 1),
    ("agg_uv_swapped", "double yy = (double)(float)(uv[1] * (double)Hs) - 0.5;",
     "double yy = (double)(float)(uv[0] * (double)Hs) - 0.5;", 1),
    ("agg_weight_order", "w[(p * cams + cam) * scales + sc]", "w[(sc * cams + cam) * pts + p]", 1),
    ("agg_ignores_scale_start", "(b * P_total + scale_start[cs]) * GC", "(b * P_total) * GC", 1),
    ("agg_weight_group_stride", "weights + ba * T * G + g;", "weights + ba * T * G;", 1),
]

# Mistakes in the core backward (oracle_dcn_core_backward), caught by its own pins.
BWD_MUTANTS = [
    ("bwd_swap_dx_dy", "fl32_mul(offset_scale, om[2 * k + 1])", "fl32_mul(offset_scale, om[2 * k + 0])", 2),
    ("bwd_pad_sign", "(double)(ho * sh - ph + i * dh)", "(double)(ho * sh + ph + i * dh)", 2),
    ("bwd_dy_weights_use_fy", "double dwy[2][2] = {{-(1.0 - fx), -fx}, {1.0 - fx, fx}};",
     "double dwy[2][2] = {{-(1.0 - fy), -fy}, {1.0 - fy, fy}};", 1),
    ("bwd_dx_sign", "double dwx[2][2] = {{-(1.0 - fy), 1.0 - fy}, {-fy, fy}};",
     "double dwx[2][2] = {{(1.0 - fy), -(1.0 - fy)}, {fy, -fy}};", 1),
    ("bwd_offset_pair_swapped", "goff[pg * K * 2 + 2 * k + 0] = s * m[k] * sx;",
     "goff[pg * K * 2 + 2 * k + 0] = s * m[k] * sy;", 1),
    ("bwd_no_offset_scale", "goff[pg * K * 2 + 2 * k + 1] = s * m[k] * sy;",
     "goff[pg * K * 2 + 2 * k + 1] = m[k] * sy;", 1),
    ("bwd_offset_no_modulation", "goff[pg * K * 2 + 2 * k + 0] = s * m[k] * sx;",
     "goff[pg * K * 2 + 2 * k + 0] = s * sx;", 1),
    ("bwd_grad_x_no_modulation", "gx[idx[a][b] + c] += m[k] * w[a][b] * gc;",
     "gx[idx[a][b] + c] += w[a][b] * gc;", 1),
    ("bwd_grad_x_transposed_corner", "((n * H + (int64_t)qy) * W + (int64_t)qx) * GC + g * C",
     "((n * H + (int64_t)qx) * W + (int64_t)qy) * GC + g * C", 1),
    ("bwd_grad_x_wrong_group", "((n * H + (int64_t)qy) * W + (int64_t)qx) * GC + g * C",
     "((n * H + (int64_t)qy) * W + (int64_t)qx) * GC", 1),
    ("bwd_softmax_no_centering", "double v = softmax ? m[k] * (gm[k] - dot) : gm[k];",
     "double v = softmax ? m[k] * gm[k] : gm[k];", 1),
    ("bwd_softmax_dot_unweighted", "dot += m[k] * gm[k];", "dot += gm[k];", 1),
    ("bwd_mask_grad_times_m", "double v = softmax ? m[k] * (gm[k] - dot) : gm[k];",
     "double v = softmax ? m[k] * (gm[k] - dot) : m[k] * gm[k];", 1),
    ("bwd_mask_grad_group_stride", "const double *Gv = gout + ((n * Ho + ho) * Wo + wo) * GC + g * C;",
     "const double *Gv = gout + ((n * Ho + ho) * Wo + wo) * GC;", 1),
]

# Mistakes in the aggregation backward (oracle_deform_agg_backward), caught by its pins.
AGG_BWD_MUTANTS = [
    ("aggbwd_loc_scale_factor", "lg[0] += w[t] * (double)Ws * sx;", "lg[0] += w[t] * (double)Hs * sx;", 1),
    ("aggbwd_loc_uv_swapped", "lg[1] += w[t] * (double)Hs * sy;", "lg[1] += w[t] * (double)Hs * sx;", 1),
    ("aggbwd_loc_no_weight", "lg[0] += w[t] * (double)Ws * sx;", "lg[0] += (double)Ws * sx;", 1),
    ("aggbwd_feat_no_weight", "gfeat[row * GC + g * Cg + c] += w[t] * wb[a][bb] * Gv[c];",
     "gfeat[row * GC + g * Cg + c] += wb[a][bb] * Gv[c];", 1),
    ("aggbwd_feat_ignores_scale_start",
     "int64_t row = b * P_total + scale_start[cs] + (int64_t)qy * Ws + (int64_t)qx;",
     "int64_t row = b * P_total + (int64_t)qy * Ws + (int64_t)qx;", 1),
    ("aggbwd_softmax_no_centering", "double v = softmax ? w[t] * (gt[t] - dot) : gt[t];",
     "double v = softmax ? w[t] * gt[t] : gt[t];", 1),
    ("aggbwd_weights_layout", "if (gw) gw[(ba * T + t) * G + g] = v;", "if (gw) gw[(ba * G + g) * T + t] = v;", 1),
    ("aggbwd_dx_sign", "double dwx[2][2] = {{-(1.0 - fy), 1.0 - fy}, {-fy, fy}};",
     "double dwx[2][2] = {{(1.0 - fy), -(1.0 - fy)}, {fy, -fy}};", 3),
    ("aggbwd_grad_out_group_stride", "const double *Gv = gout + ba * GC + g * Cg;",
     "const double *Gv = gout + ba * GC;", 1),
]

# Mistakes in the DCNv2 backward (oracle_dcn_v2_backward), caught by its pins.
V2_BWD_MUTANTS = [
    ("v2bwd_weight_tap_major", "s += weight[co * R + rr] * go;",
     "s += weight[co * R + (rr % K) * Cin + rr / K] * go;", 1),
    ("v2bwd_gout_batch_channel_swapped", "double go = gout[(n * Cout + co) * HWo + r];",
     "double go = gout[(co * N + n) * HWo + r];", 1),
    ("v2bwd_weight_grad_from_column_grad", "s += go * col[p * R + rr];", "s += go * gc[p * R + rr];", 1),
    ("v2bwd_grad_x_no_modulation", "if (gx && w[a][b] != 0.0) gx[xi] += m[k] * w[a][b] * u;",
     "if (gx && w[a][b] != 0.0) gx[xi] += w[a][b] * u;", 1),
    ("v2bwd_offset_pair_swapped", "goff[(oc + 0) * HWo + r] = m[k] * sx;",
     "goff[(oc + 0) * HWo + r] = m[k] * sy;", 1),
    ("v2bwd_column_grad_tap_major", "double u = gc[p * R + ci * K + k], ua = gca[p * R + ci * K + k];",
     "double u = gc[p * R + k * Cin + ci], ua = gca[p * R + k * Cin + ci];", 1),
    ("v2bwd_softmax_no_centering", "double v = softmax ? m[k] * (gm[k] - dot) : gm[k];",
     "double v = softmax ? m[k] * gm[k] : gm[k];", 2),
    ("v2bwd_softmax_null_mask_unit", "for (int64_t k = 0; k < K; ++k) m[k] = 1.0 / (double)K;",
     "for (int64_t k = 0; k < K; ++k) m[k] = 1.0;", 2),
    ("v2bwd_dy_sign", "double dwy[2][2] = {{-(1.0 - fx), -fx}, {1.0 - fx, fx}};",
     "double dwy[2][2] = {{(1.0 - fx), fx}, {-(1.0 - fx), -fx}};", 2),
]

# Mistakes in deformable RoI pooling (oracle_deform_roi_pool), caught by its pins.
ROI_MUTANTS = [
    ("roi_swap_dx_dy", "* 2 + 0])) * w);", "* 2 + 1])) * w);", 1),
    ("roi_offset_scaled_by_h", "* 2 + 0])) * w);", "* 2 + 0])) * h);", 1),
    ("roi_no_gamma", "dy = fl32(fl32(gm * fl32(offset[", "dy = fl32(fl32(fl32(offset[", 1),
    ("roi_no_half_sample", "double tx = fl32((double)(2 * (j * S + sx) + 1) / (double)(2 * S));",
     "double tx = fl32((double)(2 * (j * S + sx)) / (double)(2 * S));", 1),
    ("roi_bins_transposed", "double bw = fl32(w / (double)k), bh = fl32(h / (double)k);",
     "double bw = fl32(h / (double)k), bh = fl32(w / (double)k);", 1),
    ("roi_mean_over_S", "o[c] = sum / (double)(S * S);", "o[c] = sum / (double)S;", 1),
    ("roi_ignores_batch", "const double *X = x + n * H * W * C;", "const double *X = x;", 1),
    ("roi_scale_x1_only", "double x1 = fl32(rx1 * s), y1 = fl32(ry1 * s);",
     "double x1 = rx1, y1 = fl32(ry1 * s);", 1),
    # the fp32 position sequence itself
    ("roi_bin_width_unrounded", "double bw = fl32(w / (double)k)", "double bw = w / (double)k", 1),
    ("roi_position_single_rounding", "double xx = fl32(fl32(x1 + fl32(tx * bw)) + dx);",
     "double xx = fl32(x1 + tx * bw + dx);", 1),
    ("roi_extent_unrounded", "h = fl32(fl32(ry2 - ry1) * s);", "h = fl32((ry2 - ry1) * s);", 1),
]


def _replace_nth(text, old, new, n):
    idx = -1
    for _ in range(n):
        idx = text.find(old, idx + 1)
        assert idx >= 0, "mutation anchor not found: %r (occurrence %d)" % (old, n)
    return text[:idx] + new + text[idx + len(old):]


def _build(src_text, tmp_path, name):
    c = tmp_path / (name + ".c")
    so = tmp_path / ("lib" + name + ".so")
    c.write_text(src_text)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
                    "-o", str(so), str(c), "-lm"], check=True)
    return str(so)


def _run_pins(lib, pins="test_oracle_pins.py"):
    env = dict(os.environ, DS_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", pins)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_oracle_passes_pins(tmp_path):
    lib = _build(open(SRC).read(), tmp_path, "orig")
    res = _run_pins(lib)
    assert res.returncode == 0, res.stdout[-3000:]
    res = _run_pins(lib, "test_oracle_backward_pins.py")
    assert res.returncode == 0, res.stdout[-3000:]
    res = _run_pins(lib, "test_oracle_agg_backward_pins.py")
    assert res.returncode == 0, res.stdout[-3000:]
    res = _run_pins(lib, "test_oracle_roi_pins.py")
    assert res.returncode == 0, res.stdout[-3000:]
    res = _run_pins(lib, "test_oracle_v2_backward_pins.py")
    assert res.returncode == 0, res.stdout[-3000:]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, nth):
    text = _replace_nth(open(SRC).read(), old, new, nth)
    lib = _build(text, tmp_path, name)
    res = _run_pins(lib)
    assert res.returncode != 0, "mutant %s survived the pins" % name


@pytest.mark.parametrize("name,old,new,nth", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_pins_catch_mutant(tmp_path, name, old, new, nth):
    text = _replace_nth(open(SRC).read(), old, new, nth)
    lib = _build(text, tmp_path, name)
    res = _run_pins(lib, "test_oracle_backward_pins.py")
    assert res.returncode != 0, "mutant %s survived the backward pins" % name


@pytest.mark.parametrize("name,old,new,nth", AGG_BWD_MUTANTS, ids=[m[0] for m in AGG_BWD_MUTANTS])
def test_agg_backward_pins_catch_mutant(tmp_path, name, old, new, nth):
    text = _replace_nth(open(SRC).read(), old, new, nth)
    lib = _build(text, tmp_path, name)
    res = _run_pins(lib, "test_oracle_agg_backward_pins.py")
    assert res.returncode != 0, "mutant %s survived the aggregation backward pins" % name


@pytest.mark.parametrize("name,old,new,nth", ROI_MUTANTS, ids=[m[0] for m in ROI_MUTANTS])
def test_roi_pins_catch_mutant(tmp_path, name, old, new, nth):
    text = _replace_nth(open(SRC).read(), old, new, nth)
    lib = _build(text, tmp_path, name)
    res = _run_pins(lib, "test_oracle_roi_pins.py")
    assert res.returncode != 0, "mutant %s survived the RoI pooling pins" % name


@pytest.mark.parametrize("name,old,new,nth", V2_BWD_MUTANTS, ids=[m[0] for m in V2_BWD_MUTANTS])
def test_v2_backward_pins_catch_mutant(tmp_path, name, old, new, nth):
    text = _replace_nth(open(SRC).read(), old, new, nth)
    lib = _build(text, tmp_path, name)
    res = _run_pins(lib, "test_oracle_v2_backward_pins.py")
    assert res.returncode != 0, "mutant %s survived the DCNv2 backward pins" % name
