"""Benchmark of the deformable-sampling forward path on one MI355X.

One step = one DCNv4 core forward (dcn_core_forward) over the detector stride-8
workload: fp16 x [16, 80, 80, 256] (16 groups of 16 channels), 3x3 window, fp32
offsets ~ N(0, 3) px with 5% of taps forced outside the image, fp32 masks ~ U(0,1),
fp32 arithmetic and accumulation, fp16 output. Inputs are resident in HBM before
the timed region.

Printed (one JSON line): bilinear taps/s (whole job), ms per step, the roofline
object of the core kernel (algorithmic bytes per launch / HIP-event launch time vs
8 TB/s), the CPU oracle's rate on a bounded sample, and side measurements of the
other ops (DCNv4/DCNv3 small maps, the core backward, DCNv2 im2col + MFMA GEMM and
the deform-im2col stage alone, aggregation forward and backward, deformable RoI
pooling).

  python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--only core|c1|c2|packed|bwd|v2|v2p|v2col|v2bwd|agg|aggbwd|roi|mfma]
  python bench.py --calib-copy     # plain copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
METRIC = "bilinear taps/sec + achieved HBM GB/s (% roofline), DCNv4 core fwd"
HEADLINE = "dcnv4_f16_n16_80x80_g16c16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dcn_core_f16_n16_80x80_hbm_traffic.txt")
CORE_SOURCES = ["dcn_core.hip", "dcn_core_tile.hip", "dcn_common.hpp", "internal.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "deformable_sampling_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the core kernel from the committed counter summary,
    or None if it is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != source_hash(CORE_SOURCES):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on torch's current stream (the stream every launch below uses)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, iters, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) / iters, e0.elapsed_time(e1) / 1e3 / iters

    def run_cold(self, fn, iters, warmup, flush):
        """Each launch timed alone (HIP events around it) after flush() has streamed a
        buffer larger than the 256 MB last-level cache through the device, so that the
        launch finds none of its inputs cached. Returns (median, p10, p90) seconds."""
        torch = self.torch
        for _ in range(warmup):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(iters):
            flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) / 1e3 for a, b in evs)
        q = lambda f: ts[min(len(ts) - 1, int(f * len(ts)))]
        return q(0.5), q(0.1), q(0.9)


class Flush:
    """Streams 2 x 512 MiB (read one buffer, write the other) between cold launches."""

    def __init__(self, torch, mib=512):
        n = mib * (1 << 20) // 4
        self.a = torch.ones(n, device="cuda")
        self.b = torch.empty_like(self.a)

    def __call__(self):
        self.b.copy_(self.a)


def cold_fields(timer, call, flush, nbytes, iters=50, warmup=3):
    """Cold-cache timing of one op: median and spread, and its HBM rate."""
    med, p10, p90 = timer.run_cold(call, iters, warmup, flush)
    return dict(cold_kernel_us=round(med * 1e6, 2), cold_p10_us=round(p10 * 1e6, 2),
                cold_p90_us=round(p90 * 1e6, 2), cold_gbs=nbytes / med / 1e9,
                cold_frac=nbytes / med / 1e9 / HBM_PEAK_GBS)


def measure_copy(torch, timer, mib=1024):
    """Sustained device copy bandwidth (read + write bytes / time) of a plain copy of
    mib MiB: the measured counterpart of the published HBM peak."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    _, kern = timer.run(lambda: b.copy_(a), 20, 5)
    return 2.0 * n * 4 / kern / 1e9


def measure_mfma(dsa, torch, timer, iters=4096):
    """Sustained dense bf16 MFMA rate of dcn_mfma_probe (register operands only) over
    two blocks of four waves per compute unit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    sink = torch.empty(blocks * 256, device="cuda")
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream

    def call():
        st = lib.dcn_mfma_probe(sink.data_ptr(), blocks, iters, stream)
        if st:
            raise RuntimeError("dcn_mfma_probe status %d" % st)
    _, kern = timer.run(call, 10, 2)
    flops = blocks * 4.0 * iters * 4 * 32768
    return flops / kern / 1e12


def raw_core_call(lib, c, x, off, mask, out, stream, softmax):
    """Argument tuple of the C entry point, prepared once (the timed loop then only
    crosses the ctypes boundary)."""
    N, H, W, GC = x.shape
    G = off.shape[3]
    dt = {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]]
    args = (x.data_ptr(), off.data_ptr(), None if mask is None else mask.data_ptr(),
            out.data_ptr(), N, H, W, G, GC // G, c["kh"], c["kw"], c["stride"][0],
            c["stride"][1], c["pad"][0], c["pad"][1], c["dil"][0], c["dil"][1],
            ctypes.c_float(1.0), int(bool(softmax)), dt, stream)
    fn = lib.dcn_core_forward

    def call():
        st = fn(*args)
        if st:
            raise RuntimeError("dcn_core_forward status %d" % st)
    return call


def headline_tensors(torch, c):
    """Device copies of a core case's x, offsets, masks and an output buffer."""
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, off, m = dev(c["x"]), dev(c["offset"]), dev(c["mask"])
    out = torch.empty((c["N"], c["Ho"], c["Wo"], c["G"] * c["C"]), dtype=x.dtype, device="cuda")
    return x, off, m, out


def bench_core(dsa, torch, timer, name, iters, warmup, flush=None):
    import workloads as wl
    c = wl.make(name)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, off, m = dev(c["x"]), dev(c["offset"]), dev(c["mask"])
    out = torch.empty((c["N"], c["Ho"], c["Wo"], c["G"] * c["C"]), dtype=x.dtype, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    call = raw_core_call(dsa.load(), c, x, off, m, out, stream, c["softmax"])
    wall, kern = timer.run(call, iters, warmup)
    taps = c["N"] * c["Ho"] * c["Wo"] * c["G"] * c["kh"] * c["kw"]
    nbytes = (x.numel() * x.element_size() + off.numel() * 4 + (m.numel() * 4 if m is not None else 0)
              + out.numel() * out.element_size())
    r = dict(workload=name, taps=taps, channel_taps=taps * c["C"], algo_bytes=nbytes,
             wall_s=wall, kernel_s=kern, taps_per_s=taps / kern,
             gbs=nbytes / kern / 1e9, frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)
    if flush is not None:
        r.update(cold_fields(timer, call, flush, nbytes))
    return r, c


def bench_core_packed(dsa, torch, timer, name, iters, warmup):
    """dcn_core_forward_packed on a core workload with DCNv4's packed offset+mask
    tensor in fp16 (the same values rounded to fp16): offsets and masks in 6 bytes
    per tap instead of 12."""
    import workloads as wl
    c = wl.make(name)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x = dev(c["x"])
    om = dsa.pack_offset_mask(dev(c["offset"]), dev(c["mask"]), dtype=torch.float16)
    out = torch.empty((c["N"], c["Ho"], c["Wo"], c["G"] * c["C"]), dtype=x.dtype, device="cuda")
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    dt = {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]]
    N, H, W, GC = x.shape
    G = c["G"]
    args = (x.data_ptr(), om.data_ptr(), out.data_ptr(), N, H, W, G, GC // G, c["kh"], c["kw"],
            c["stride"][0], c["stride"][1], c["pad"][0], c["pad"][1], c["dil"][0], c["dil"][1],
            ctypes.c_float(1.0), int(bool(c["softmax"])), om.shape[3], 1, dt, stream)

    def call():
        st = lib.dcn_core_forward_packed(*args)
        if st:
            raise RuntimeError("dcn_core_forward_packed status %d" % st)
    wall, kern = timer.run(call, iters, warmup)
    taps = c["N"] * c["Ho"] * c["Wo"] * c["G"] * c["kh"] * c["kw"]
    nbytes = (x.numel() + out.numel()) * x.element_size() + om.numel() * 2
    return dict(workload=name + " packed fp16 offset+mask", taps=taps, channel_taps=taps * c["C"],
                algo_bytes=nbytes, wall_s=wall, kernel_s=kern, taps_per_s=taps / kern,
                gbs=nbytes / kern / 1e9, frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)


def bench_core_bwd(dsa, torch, timer, name, iters, warmup):
    """dcn_core_backward (grad_x, grad_offset, grad_mask) on a core workload: the
    whole call (bin count, scan, pair pass with the sample records, tile gather)."""
    import workloads as wl
    c = wl.make(name)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, off, m = dev(c["x"]), dev(c["offset"]), dev(c["mask"])
    go = dev(wl.core_grad_out(c, seed=1))
    gx = torch.empty_like(x)
    goff = torch.empty_like(off)
    gm = torch.empty_like(m) if m is not None else torch.empty(
        (c["N"], c["Ho"], c["Wo"], c["G"], c["kh"] * c["kw"]), device="cuda")
    N, H, W, GC = x.shape
    G = c["G"]
    dt = {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]]
    lib = dsa.load()
    wsb = lib.dcn_core_backward_workspace_bytes(N, H, W, G, GC // G, c["kh"], c["kw"],
                                                c["stride"][0], c["stride"][1], c["pad"][0],
                                                c["pad"][1], c["dil"][0], c["dil"][1], dt)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), off.data_ptr(), None if m is None else m.data_ptr(), go.data_ptr(),
            gx.data_ptr(), goff.data_ptr(), gm.data_ptr(), ws.data_ptr(), wsb, N, H, W, G,
            GC // G, c["kh"], c["kw"], c["stride"][0], c["stride"][1], c["pad"][0], c["pad"][1],
            c["dil"][0], c["dil"][1], ctypes.c_float(1.0), int(bool(c["softmax"])), dt, stream)
    fn = lib.dcn_core_backward

    def call():
        st = fn(*args)
        if st:
            raise RuntimeError("dcn_core_backward status %d" % st)
    wall, kern = timer.run(call, iters, warmup)
    taps = c["N"] * c["Ho"] * c["Wo"] * G * c["kh"] * c["kw"]
    es = x.element_size()
    # read x, offsets, masks, grad_out; write grad_x, grad_offset, grad_mask
    nbytes = (2 * x.numel() * es + 2 * off.numel() * 4 + 2 * gm.numel() * 4
              + go.numel() * es)
    return dict(workload=name + " backward", taps=taps, algo_bytes=nbytes, wall_s=wall,
                kernel_s=kern, taps_per_s=taps / kern, gbs=nbytes / kern / 1e9,
                frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)


def bench_v2(dsa, torch, timer, iters, warmup, flush=None, prepacked=False):
    """dcn_v2_forward on the 8x256x40x40 bf16 layer (prepacked: dcn_v2_forward_prepacked
    with the weight packed once before the timed calls, as an inference layer whose
    weight does not change would run)."""
    import workloads as wl
    name = "dcnv2_bf16_n8_c256_40x40"
    c = wl.make(name)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, off, m, w = dev(c["x"]), dev(c["offset"]), dev(c["mask"]), dev(c["weight"])
    N, Cin, H, W, Cout = c["N"], c["Cin"], c["H"], c["W"], c["Cout"]
    need = dsa.dcn_v2_workspace_bytes(N, Cin, H, W, Cout, dtype=torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty((N, Cout, c["Ho"], c["Wo"]), dtype=torch.bfloat16, device="cuda")
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), off.data_ptr(), m.data_ptr(), w.data_ptr(), out.data_ptr(), ws.data_ptr(),
            need, N, Cin, H, W, Cout, 3, 3, 1, 1, 1, 1, 1, 1, 1, 0, 2, stream)

    if prepacked:
        packed = dsa.dcn_v2_pack_weight(w)
        pargs = (x.data_ptr(), off.data_ptr(), m.data_ptr(), packed.data_ptr(), packed.numel(),
                 out.data_ptr(), ws.data_ptr(), need, N, Cin, H, W, Cout, 3, 3, 1, 1, 1, 1, 1, 1, 1, 0, 2,
                 stream)

        def call():
            st = lib.dcn_v2_forward_prepacked(*pargs)
            if st:
                raise RuntimeError("dcn_v2_forward_prepacked status %d" % st)
    else:
        def call():
            st = lib.dcn_v2_forward(*args)
            if st:
                raise RuntimeError("dcn_v2_forward status %d" % st)
    wall, kern = timer.run(call, iters, warmup)
    P = N * c["Ho"] * c["Wo"]
    flops = 2.0 * Cout * Cin * 9 * P
    nbytes = x.numel() * 2 + off.numel() * 4 + m.numel() * 4 + w.numel() * 2 + out.numel() * 2
    r = dict(workload=name + (" prepacked weight" if prepacked else ""), taps=P * 9,
             channel_taps=P * 9 * Cin, algo_bytes=nbytes,
             flops=flops, wall_s=wall, kernel_s=kern, tflops=flops / kern / 1e12,
             mfma_frac=flops / kern / 1e12 / MFMA_BF16_PEAK_TFLOPS,
             note=("two launches: x to channels-last, deform-im2col fused into the MFMA GEMM "
                   "(weight packed once, outside the timed calls)" if prepacked else
                   "two launches: layout prep (x and weight), deform-im2col fused into the MFMA GEMM"))
    if flush is not None:
        r.update(cold_fields(timer, call, flush, nbytes))
        r["cold_tflops"] = flops / (r["cold_kernel_us"] * 1e-6) / 1e12
    return r


def bench_v2_im2col(dsa, torch, timer, iters, warmup, flush=None):
    """dcn_v2_im2col on the 8x256x40x40 bf16 layer: the deform-im2col stage alone (x to
    channels-last, then the K-contiguous bf16 columns [P][K*Cin] into the workspace),
    against the HBM roofline of x, offsets and masks read once and the columns written
    once."""
    import workloads as wl
    name = "dcnv2_bf16_n8_c256_40x40"
    c = wl.make(name)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, off, m = dev(c["x"]), dev(c["offset"]), dev(c["mask"])
    N, Cin, H, W, Cout = c["N"], c["Cin"], c["H"], c["W"], c["Cout"]
    need = dsa.dcn_v2_workspace_bytes(N, Cin, H, W, Cout, dtype=torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), off.data_ptr(), m.data_ptr(), ws.data_ptr(), need, N, Cin, H, W, Cout,
            3, 3, 1, 1, 1, 1, 1, 1, 1, 0, 2, stream)

    def call():
        st = lib.dcn_v2_im2col(*args)
        if st:
            raise RuntimeError("dcn_v2_im2col status %d" % st)
    wall, kern = timer.run(call, iters, warmup)
    P = N * c["Ho"] * c["Wo"]
    cols = P * 9 * Cin * 2
    nbytes = x.numel() * 2 + off.numel() * 4 + m.numel() * 4 + cols
    r = dict(workload=name + " deform-im2col", taps=P * 9, channel_taps=P * 9 * Cin, algo_bytes=nbytes,
             wall_s=wall, kernel_s=kern, taps_per_s=P * 9 / kern, gbs=nbytes / kern / 1e9,
             frac=nbytes / kern / 1e9 / HBM_PEAK_GBS,
             note="two launches: x to channels-last, then the column kernel")
    if flush is not None:
        r.update(cold_fields(timer, call, flush, nbytes))
    return r


def bench_v2_bwd(dsa, torch, timer, iters, warmup):
    """dcn_v2_backward (grad x, offsets, masks, weight) on the 8x256x40x40 bf16 layer:
    the whole call (layouts, transposed columns, two MFMA GEMMs, bucket count/scan,
    sample pass, destination gather, NCHW grad_x)."""
    import workloads as wl
    name = "dcnv2_bf16_n8_c256_40x40"
    c = wl.make(name)
    dev = lambda t: None if t is None else t.to("cuda").contiguous()
    x, off, m, w = dev(c["x"]), dev(c["offset"]), dev(c["mask"]), dev(c["weight"])
    go = dev(wl.v2_grad_out(c, seed=502))
    N, Cin, H, W, Cout = c["N"], c["Cin"], c["H"], c["W"], c["Cout"]
    Ho, Wo = c["Ho"], c["Wo"]
    need = dsa.dcn_v2_backward_workspace_bytes(N, Cin, H, W, Cout, dtype=torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    gx = torch.empty_like(x)
    goff = torch.empty_like(off)
    gm = torch.empty_like(m)
    gw = torch.empty((Cout, Cin, 3, 3), dtype=torch.float32, device="cuda")
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), off.data_ptr(), m.data_ptr(), w.data_ptr(), go.data_ptr(), gx.data_ptr(),
            goff.data_ptr(), gm.data_ptr(), gw.data_ptr(), ws.data_ptr(), need, N, Cin, H, W, Cout,
            3, 3, 1, 1, 1, 1, 1, 1, 1, 0, 2, stream)

    def call():
        st = lib.dcn_v2_backward(*args)
        if st:
            raise RuntimeError("dcn_v2_backward status %d" % st)
    wall, kern = timer.run(call, iters, warmup)
    P = N * Ho * Wo
    flops = 2 * 2.0 * Cout * Cin * 9 * P  # column gradient + weight gradient
    # inputs read once (x, offsets, masks, weight, grad_out), gradients written once
    nbytes = (2 * x.numel() * 2 + 2 * off.numel() * 4 + 2 * m.numel() * 4 + w.numel() * 2
              + gw.numel() * 4 + go.numel() * 2)
    return dict(workload=name + " backward", taps=P * 9, algo_bytes=nbytes, flops=flops,
                wall_s=wall, kernel_s=kern, tflops=flops / kern / 1e12,
                mfma_frac=flops / kern / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                gbs=nbytes / kern / 1e9, frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)


def bench_agg(dsa, torch, timer, iters, warmup, softmax=True, flush=None):
    import workloads as wl
    name = "agg_f32_6cam_4scale_a900p13_g8c32"
    c = wl.make(name, weights="logits" if softmax else "simplex")
    dev = lambda t: t.to("cuda").contiguous()
    feat, loc, wts = dev(c["feat"]), dev(c["loc"]), dev(c["weights"])
    out = torch.empty((c["B"], c["A"], c["G"] * c["Cg"]), dtype=feat.dtype, device="cuda")
    import numpy as np
    ss = np.ascontiguousarray(c["spatial_shape"], dtype=np.int32)
    st = np.ascontiguousarray(c["scale_start"], dtype=np.int32)
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    args = (feat.data_ptr(), ss.ctypes.data, st.ctypes.data, loc.data_ptr(), wts.data_ptr(),
            out.data_ptr(), c["B"], c["P_total"], c["A"], c["pts"], c["cams"], c["scales"], c["G"],
            c["Cg"], int(softmax), 0, stream)

    def call():
        s = lib.deform_agg_forward(*args)
        if s:
            raise RuntimeError("deform_agg_forward status %d" % s)
    wall, kern = timer.run(call, iters, warmup)
    taps = c["B"] * c["A"] * c["pts"] * c["cams"] * c["scales"] * c["G"]
    nbytes = feat.numel() * 4 + loc.numel() * 4 + wts.numel() * 4 + out.numel() * 4
    r = dict(workload=name + ("_softmax" if softmax else ""), taps=taps,
             channel_taps=taps * c["Cg"], algo_bytes=nbytes, wall_s=wall, kernel_s=kern,
             taps_per_s=taps / kern, gbs=nbytes / kern / 1e9,
             frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)
    if flush is not None:
        r.update(cold_fields(timer, call, flush, nbytes))
    return r


def bench_agg_bwd(dsa, torch, timer, iters, warmup):
    """deform_agg_backward (features, locations, weights) on the six-camera workload,
    softmax weights: the whole call (clear, gradient kernel, grad_loc reduction)."""
    import numpy as np
    import workloads as wl
    name = "agg_f32_6cam_4scale_a900p13_g8c32"
    c = wl.make(name)
    dev = lambda t: t.to("cuda").contiguous()
    feat, loc, wts = dev(c["feat"]), dev(c["loc"]), dev(c["weights"])
    go = dev(wl.agg_grad_out(c, seed=1))
    gf, gl, gw = torch.empty_like(feat), torch.empty_like(loc), torch.empty_like(wts)
    ss = np.ascontiguousarray(c["spatial_shape"], dtype=np.int32)
    st = np.ascontiguousarray(c["scale_start"], dtype=np.int32)
    lib = dsa.load()
    wsb = lib.deform_agg_backward_workspace_bytes(c["B"], c["P_total"], c["A"], c["pts"],
                                                  c["cams"], c["scales"], c["G"], c["Cg"], 0)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    args = (feat.data_ptr(), ss.ctypes.data, st.ctypes.data, loc.data_ptr(), wts.data_ptr(),
            go.data_ptr(), gf.data_ptr(), gl.data_ptr(), gw.data_ptr(), ws.data_ptr(), wsb,
            c["B"], c["P_total"], c["A"], c["pts"], c["cams"], c["scales"], c["G"], c["Cg"], 1, 0,
            stream)

    def call():
        s = lib.deform_agg_backward(*args)
        if s:
            raise RuntimeError("deform_agg_backward status %d" % s)
    wall, kern = timer.run(call, iters, warmup)
    taps = c["B"] * c["A"] * c["pts"] * c["cams"] * c["scales"] * c["G"]
    # read feat, loc, weights, grad_out; write grad_feat, grad_loc, grad_weights
    nbytes = 2 * feat.numel() * 4 + 2 * loc.numel() * 4 + 2 * wts.numel() * 4 + go.numel() * 4
    return dict(workload=name + "_softmax backward", taps=taps, algo_bytes=nbytes, wall_s=wall,
                kernel_s=kern, taps_per_s=taps / kern, gbs=nbytes / kern / 1e9,
                frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)


def bench_roi(dsa, torch, timer, iters, warmup):
    """deform_roi_pool_forward on the 512-RoI, 7x7-bin workload."""
    import workloads as wl
    name = "droi_f32_n2_64x64_c256_r512_k7"
    c = wl.make(name)
    dev = lambda t: t.to("cuda").contiguous()
    x, rois, off = dev(c["x"]), dev(c["rois"]), dev(c["offset"])
    out = torch.empty((c["R"], c["k"], c["k"], c["C"]), dtype=x.dtype, device="cuda")
    lib = dsa.load()
    stream = torch.cuda.current_stream().cuda_stream
    dt = {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]]
    args = (x.data_ptr(), rois.data_ptr(), off.data_ptr(), out.data_ptr(), c["N"], c["H"], c["W"],
            c["C"], c["R"], c["k"], c["S"], ctypes.c_float(c["spatial_scale"]),
            ctypes.c_float(c["gamma"]), dt, stream)

    def call():
        s = lib.deform_roi_pool_forward(*args)
        if s:
            raise RuntimeError("deform_roi_pool_forward status %d" % s)
    wall, kern = timer.run(call, iters, warmup)
    samples = c["R"] * c["k"] * c["k"] * c["S"] * c["S"]
    # the feature map once, RoIs, offsets, output
    nbytes = (x.numel() + out.numel()) * x.element_size() + rois.numel() * 4 + off.numel() * 4
    return dict(workload=name, taps=samples, algo_bytes=nbytes, wall_s=wall, kernel_s=kern,
                taps_per_s=samples / kern, gbs=nbytes / kern / 1e9,
                frac=nbytes / kern / 1e9 / HBM_PEAK_GBS)


def cpu_baseline(case, target_s=10.0, max_reps=200):
    """The oracle (as it stands, fp64 C with OpenMP) timed on the headline workload.

    The sample is bounded to about target_s seconds of CPU work: a random subset of
    the output pixels if the full workload would take longer, otherwise the full
    workload repeated. Returns taps/s over everything the oracle computed."""
    import numpy as np
    import oracle
    xs = oracle._f64(case["x"])
    off = oracle._f64(case["offset"])
    m = oracle._f64(case["mask"])
    npix_all = case["N"] * case["Ho"] * case["Wo"]
    per_pix_taps = case["G"] * case["kh"] * case["kw"]
    r = np.random.default_rng(123)

    def run(pix):
        t0 = time.perf_counter()
        oracle.dcn_core(xs, off, m, kh=case["kh"], kw=case["kw"], stride=case["stride"],
                        pad=case["pad"], dil=case["dil"], pix=pix)
        return time.perf_counter() - t0

    probe = np.sort(r.choice(npix_all, size=min(1024, npix_all), replace=False))
    t_probe = run(probe)
    est_full = t_probe * npix_all / len(probe)
    if est_full >= target_s:
        n = int(max(len(probe), npix_all * target_s / est_full))
        pix = np.sort(r.choice(npix_all, size=n, replace=False))
        t = run(pix)
        taps = n * per_pix_taps
        sample = "%d of %d output pixels (x %d groups x %d taps), %.1f s" % (
            n, npix_all, case["G"], case["kh"] * case["kw"], t)
    else:
        reps, t = 0, 0.0
        while t < target_s and reps < max_reps:
            t += run(None)
            reps += 1
        taps = reps * npix_all * per_pix_taps
        sample = "full workload (%d output pixels x %d groups x %d taps) x %d runs, %.1f s" % (
            npix_all, case["G"], case["kh"] * case["kw"], reps, t)
    out = dict(value=taps / t, unit="taps/s", cores=oracle.threads(), kind="oracle", sample=sample,
               cores_affinity=len(os.sched_getaffinity(0)))
    out["single_thread"] = oracle_single_thread()
    return out


def oracle_single_thread(target_s=1.0):
    """The oracle on one thread over the two small core workloads (whole, repeated to
    about target_s each): taps/s."""
    import oracle
    import workloads as wl
    res = []
    n0 = oracle.threads()
    oracle.set_threads(1)
    try:
        for name in ("dcnv4_f32_n1_32x32_g4c16", "dcnv3_f32_n8_56x56_g4c16_softmax"):
            c = wl.make(name)
            xs, off = oracle._f64(c["x"]), oracle._f64(c["offset"])
            m = oracle._f64(c["mask"])
            taps = c["N"] * c["Ho"] * c["Wo"] * c["G"] * c["kh"] * c["kw"]
            reps, t = 0, 0.0
            while t < target_s and reps < 1000:
                t0 = time.perf_counter()
                oracle.dcn_core(xs, off, m, kh=c["kh"], kw=c["kw"], stride=c["stride"],
                                pad=c["pad"], dil=c["dil"], softmax=c["softmax"])
                t += time.perf_counter() - t0
                reps += 1
            res.append(dict(workload=name, value=taps * reps / t, unit="taps/s", threads=1,
                            runs=reps, seconds=round(t, 3)))
    finally:
        oracle.set_threads(n0)
    return res


def calib_copy(torch, mb=1024, iters=5):
    """A plain device copy of known size, to scale FETCH_SIZE/WRITE_SIZE counters."""
    n = mb * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(iters):
        b.copy_(a)
    torch.cuda.synchronize()
    log("calib copy: %d launches of %d bytes read + %d bytes written" % (iters, n * 4, n * 4))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["core", "all", "bwd", "aggbwd", "v2bwd", "c1", "c2", "v2", "v2p",
                                       "agg", "packed", "roi", "mfma", "v2col"], default="all")
    ap.add_argument("--calib-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no cross-GPU exchange (it shards "
              "by image with nothing to exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import deformable_sampling_amd as dsa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dsa.load()
    if args.calib_copy:
        calib_copy(torch)
        return
    timer = Timer(torch)

    # one op alone (for profiling its kernels)
    if args.only in ("c1", "c2"):
        nm = {"c1": "dcnv4_f32_n1_32x32_g4c16", "c2": "dcnv3_f32_n8_56x56_g4c16_softmax"}[args.only]
        r, _ = bench_core(dsa, torch, timer, nm, args.steps, args.warmup)
        log("%s: %.2f us/launch" % (nm, r["kernel_s"] * 1e6))
        return
    if args.only == "v2col":
        r = bench_v2_im2col(dsa, torch, timer, args.steps, args.warmup)
        log("dcnv2 deform-im2col: %.2f us/call, %.0f GB/s" % (r["kernel_s"] * 1e6, r["gbs"]))
        return
    if args.only in ("v2", "v2p"):
        r = bench_v2(dsa, torch, timer, args.steps, args.warmup, prepacked=args.only == "v2p")
        log("dcnv2: %.2f us/call, %.0f TFLOP/s" % (r["kernel_s"] * 1e6, r["tflops"]))
        return
    if args.only == "agg":
        r = bench_agg(dsa, torch, timer, args.steps, args.warmup, softmax=True)
        log("aggregation: %.2f us/launch" % (r["kernel_s"] * 1e6))
        return
    if args.only == "packed":
        r = bench_core_packed(dsa, torch, timer, HEADLINE, args.steps, args.warmup)
        log("packed core: %.2f us/launch" % (r["kernel_s"] * 1e6))
        return
    if args.only == "roi":
        r = bench_roi(dsa, torch, timer, args.steps, args.warmup)
        log("roi pooling: %.2f us/launch" % (r["kernel_s"] * 1e6))
        return
    if args.only == "mfma":
        log("mfma probe: %.0f TFLOP/s; copy %.0f GB/s" % (measure_mfma(dsa, torch, timer),
                                                        measure_copy(torch, timer)))
        return
    if args.only == "v2bwd":  # the DCNv2 backward alone (for profiling)
        r = bench_v2_bwd(dsa, torch, timer, args.steps, args.warmup)
        log("dcnv2 backward: %.2f us/call" % (r["kernel_s"] * 1e6))
        return
    if args.only == "aggbwd":  # the aggregation backward alone (for profiling)
        r = bench_agg_bwd(dsa, torch, timer, args.steps, args.warmup)
        log("aggregation backward: %.2f us/call" % (r["kernel_s"] * 1e6))
        return
    if args.only == "bwd":  # the core backward alone (for profiling)
        r = bench_core_bwd(dsa, torch, timer, HEADLINE, args.steps, args.warmup)
        log("core backward: %.2f us/call" % (r["kernel_s"] * 1e6))
        return
    log("headline: %s, warmup %d, steps %d" % (HEADLINE, args.warmup, args.steps))
    head, case = bench_core(dsa, torch, timer, HEADLINE, args.steps, args.warmup)
    log("headline done: %.2f us/launch" % (head["kernel_s"] * 1e6))
    extra = []
    ceilings = None
    head_cold = None
    if args.only == "all":
        flush = Flush(torch)
        head_cold = cold_fields(timer, raw_core_call(dsa.load(), case, *headline_tensors(torch, case),
                                                     torch.cuda.current_stream().cuda_stream,
                                                     case["softmax"]),
                                flush, head["algo_bytes"])
        ceilings = dict(copy_gbs=measure_copy(torch, timer), mfma_bf16_tflops=measure_mfma(dsa, torch, timer),
                        note="measured: a 1 GiB device copy (read + write bytes / time) and "
                             "dcn_mfma_probe (dense bf16 MFMAs on register operands)")
        log("ceilings: copy %.0f GB/s, mfma %.0f TFLOP/s" % (ceilings["copy_gbs"],
                                                             ceilings["mfma_bf16_tflops"]))
        for nm in ["dcnv4_f32_n1_32x32_g4c16", "dcnv3_f32_n8_56x56_g4c16_softmax"]:
            r, _ = bench_core(dsa, torch, timer, nm, 200, 20, flush=flush)
            extra.append(r)
            log("%s done" % nm)
        extra.append(bench_core_packed(dsa, torch, timer, HEADLINE, 200, 20))
        log("packed offset+mask done")
        extra.append(bench_core_bwd(dsa, torch, timer, HEADLINE, 100, 10))
        log("core backward done")
        for pre in (False, True):
            r = bench_v2(dsa, torch, timer, 100, 10, flush=flush, prepacked=pre)
            r["mfma_frac_of_probe"] = r["tflops"] / ceilings["mfma_bf16_tflops"]
            extra.append(r)
        extra.append(bench_v2_im2col(dsa, torch, timer, 100, 10, flush=flush))
        log("dcnv2 done")
        extra.append(bench_v2_bwd(dsa, torch, timer, 50, 5))
        log("dcnv2 backward done")
        extra.append(bench_agg(dsa, torch, timer, 100, 10, softmax=True, flush=flush))
        extra.append(bench_agg(dsa, torch, timer, 100, 10, softmax=False, flush=flush))
        extra.append(bench_agg_bwd(dsa, torch, timer, 20, 3))
        log("aggregation done")
        extra.append(bench_roi(dsa, torch, timer, 100, 10))
        log("roi pooling done")
        for r in extra:
            r["kernel_us"] = round(r.pop("kernel_s") * 1e6, 2)
            r["wall_us"] = round(r.pop("wall_s") * 1e6, 2)
            if "gbs" in r:
                r["frac_of_measured_copy"] = r["gbs"] / ceilings["copy_gbs"]
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(case)
        log("cpu baseline done: %s" % cpu["sample"])

    achieved = head["algo_bytes"] / head["kernel_s"] / 1e9
    traffic = read_traffic()
    line = {
        "metric": METRIC,
        "value": head["taps"] / head["wall_s"],
        "unit": "taps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["wall_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the workload, no dataset)",
        "config": {"workload": HEADLINE, "op": "dcn_core_forward", "N": 16, "H": 80, "W": 80,
                   "groups": 16, "group_channels": 16, "kernel": "3x3", "stride": 1, "pad": 1,
                   "dilation": 1, "storage": "x/out fp16, offsets/masks fp32",
                   "taps_per_step": head["taps"], "kernel_us": round(head["kernel_s"] * 1e6, 2),
                   "kernel_taps_per_s": head["taps_per_s"],
                   "cold": head_cold},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "algo_bytes_per_launch": head["algo_bytes"],
                     "kernel": "dcn_core_tile_kernel (fp16, 3x3, 16x16-pixel x 2-group LDS halo tiles)",
                     "source_hash": source_hash(CORE_SOURCES)},
        "ceilings": ceilings,
        "roofline_vs_measured_copy": (achieved / ceilings["copy_gbs"]) if ceilings else None,
        "cpu_baseline": cpu,
        "other_ops": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
