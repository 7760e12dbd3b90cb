// C ABI of libdcn: argument validation on the host, then dispatch to the kernels.
// Every check below runs before any HIP API call, so a rejected call has no effect
// (this also lets the checks be exercised on a machine without a GPU).
#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "dcn.h"
#include "internal.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr long long kI32 = 2147483647LL;
constexpr unsigned kBwdPathMask = DCN_BWD_ATOMIC | DCN_BWD_PAIR_PASS | DCN_BWD_PAIR_PASS_RECORDS |
                                  DCN_BWD_UNSTAGED_GATHER | DCN_BWD_GENERAL_MAIN;

bool valid_dtype(dcn_dtype d) { return d == DCN_F32 || d == DCN_F16 || d == DCN_BF16; }
size_t dtype_size(dcn_dtype d) { return d == DCN_F32 ? 4 : 2; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

long long out_extent(int in, int k, int s, int p, int d) {
    return ((long long)in + 2LL * p - (long long)d * (k - 1) - 1) / s + 1;
}

dcn_status hip_status(hipError_t e) {
    if (e == hipSuccess) return DCN_OK;
    g_last_hip_error = (int)e;
    return DCN_ERR_HIP;
}

// Shared window checks of the core and DCNv2 paths.
dcn_status check_window(int kh, int kw, int sh, int sw, int ph, int pw, int dh, int dw) {
    if (kh <= 0 || kw <= 0) return DCN_ERR_SHAPE;
    if ((long long)kh * kw > 64) return DCN_ERR_SHAPE;
    if (sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0 || ph < 0 || pw < 0) return DCN_ERR_PARAM;
    return DCN_OK;
}

}  // namespace

// dcn_v2_forward_noalloc: the workspace is this file's static device array instead of a
// caller buffer, for callers that cannot allocate. Each device holds its own copy of the
// array; its address on a device comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the first call there and kept. Host code uses only that
// address, never the array's name. Nothing in it needs clearing between calls: every
// byte a call reads was written earlier in the same call.
static __device__ __align__(256) unsigned char scratch[DCN_V2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of `scratch` (hipGetSymbolAddress once per device).
hipError_t scratch_address(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_acquire);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}
}  // namespace

extern "C" {

const char *dcn_status_string(dcn_status s) {
    switch (s) {
        case DCN_OK: return "ok";
        case DCN_ERR_NULL: return "null pointer";
        case DCN_ERR_SHAPE: return "invalid shape or size limit exceeded";
        case DCN_ERR_PARAM: return "invalid parameter";
        case DCN_ERR_DTYPE: return "unsupported dtype";
        case DCN_ERR_ALIGN: return "misaligned pointer";
        case DCN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case DCN_ERR_HIP: return "HIP launch error";
        case DCN_ERR_SCRATCH: return "the call needs more than the library's static scratch";
    }
    return "unknown status";
}

int dcn_last_hip_error(void) { return g_last_hip_error; }

dcn_status dcn_core_forward(const void *x, const float *offset, const float *mask, void *out,
                            int N, int H, int W, int G, int C, int kh, int kw, int stride_h,
                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                            float offset_scale, int softmax, dcn_dtype dtype, hipStream_t stream) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (N < 0 || H <= 0 || W <= 0 || G <= 0 || C <= 0) return DCN_ERR_SHAPE;
    dcn_status st = check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w);
    if (st != DCN_OK) return st;
    const long long Ho = out_extent(H, kh, stride_h, pad_h, dil_h);
    const long long Wo = out_extent(W, kw, stride_w, pad_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return DCN_ERR_SHAPE;
    // index limits of the kernels (32-bit pair and in-image element offsets)
    if ((long long)(H + 1) * (W + 1) * G * C > kI32) return DCN_ERR_SHAPE;
    if ((long long)N * Ho * Wo * G > kI32) return DCN_ERR_SHAPE;
    if (N == 0) return DCN_OK;
    if (!x || !offset || !out) return DCN_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned(x, es) || !aligned(out, es) || !aligned(offset, 4) ||
        (mask && !aligned(mask, 4)))
        return DCN_ERR_ALIGN;

    dcn::CoreLaunch a;
    a.x = x; a.offset = offset; a.mask = mask; a.out = out;
    a.N = N; a.H = H; a.W = W; a.G = G; a.C = C; a.kh = kh; a.kw = kw;
    a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w; a.dh = dil_h; a.dw = dil_w;
    a.Ho = (int)Ho; a.Wo = (int)Wo;
    a.offset_scale = offset_scale;
    a.softmax = softmax;
    a.dtype = dtype;
    const int K = kh * kw;
    a.om_dtype = DCN_F32;
    a.off_grp = 2 * K; a.off_pix = G * 2 * K; a.mask_grp = K; a.mask_pix = G * K;
    a.om_plain = true;
    return hip_status(dcn::launch_dcn_core(a, stream));
}

dcn_status dcn_core_forward_packed(const void *x, const void *offset_mask, void *out, int N, int H,
                                   int W, int G, int C, int kh, int kw, int stride_h, int stride_w,
                                   int pad_h, int pad_w, int dil_h, int dil_w, float offset_scale,
                                   int softmax, int om_pixel_stride, dcn_dtype om_dtype,
                                   dcn_dtype dtype, hipStream_t stream) {
    if (!valid_dtype(dtype) || !valid_dtype(om_dtype)) return DCN_ERR_DTYPE;
    if (N < 0 || H <= 0 || W <= 0 || G <= 0 || C <= 0) return DCN_ERR_SHAPE;
    dcn_status st = check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w);
    if (st != DCN_OK) return st;
    const long long Ho = out_extent(H, kh, stride_h, pad_h, dil_h);
    const long long Wo = out_extent(W, kw, stride_w, pad_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return DCN_ERR_SHAPE;
    const int K = kh * kw;
    if ((long long)om_pixel_stride < (long long)G * 3 * K) return DCN_ERR_PARAM;
    if ((long long)(H + 1) * (W + 1) * G * C > kI32) return DCN_ERR_SHAPE;
    if ((long long)N * Ho * Wo * G > kI32) return DCN_ERR_SHAPE;
    if (N == 0) return DCN_OK;
    if (!x || !offset_mask || !out) return DCN_ERR_NULL;
    if (!aligned(x, dtype_size(dtype)) || !aligned(out, dtype_size(dtype)) ||
        !aligned(offset_mask, dtype_size(om_dtype)))
        return DCN_ERR_ALIGN;
    const size_t oe = dtype_size(om_dtype);
    dcn::CoreLaunch a;
    a.x = x; a.offset = offset_mask;
    a.mask = static_cast<const char *>(offset_mask) + (size_t)2 * K * oe;
    a.out = out;
    a.N = N; a.H = H; a.W = W; a.G = G; a.C = C; a.kh = kh; a.kw = kw;
    a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w; a.dh = dil_h; a.dw = dil_w;
    a.Ho = (int)Ho; a.Wo = (int)Wo;
    a.offset_scale = offset_scale;
    a.softmax = softmax;
    a.dtype = dtype;
    a.om_dtype = om_dtype;
    a.off_grp = 3 * K; a.off_pix = om_pixel_stride; a.mask_grp = 3 * K; a.mask_pix = om_pixel_stride;
    a.om_plain = false;
    return hip_status(dcn::launch_dcn_core(a, stream));
}

static bool valid_path(unsigned path) { return (path & ~kBwdPathMask) == 0; }

size_t dcn_core_backward_workspace_bytes_path(int N, int H, int W, int G, int C, int kh, int kw,
                                              int stride_h, int stride_w, int pad_h, int pad_w,
                                              int dil_h, int dil_w, dcn_dtype dtype,
                                              unsigned path) {
    if (!valid_path(path)) return 0;
    if (!valid_dtype(dtype) || N < 0 || H <= 0 || W <= 0 || G <= 0 || C <= 0) return 0;
    if (check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w) != DCN_OK) return 0;
    const long long Ho = out_extent(H, kh, stride_h, pad_h, dil_h);
    const long long Wo = out_extent(W, kw, stride_w, pad_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return 0;
    if ((long long)(H + 1) * (W + 1) * G * C > kI32 || (long long)N * Ho * Wo * G > kI32) return 0;
    dcn::CoreBwdPlan plan;
    dcn::plan_core_bwd(N, H, W, G, C, (int)Ho, (int)Wo, kh * kw, dtype,
                       (path & DCN_BWD_ATOMIC) != 0, plan);
    return plan.total;
}

size_t dcn_core_backward_workspace_bytes(int N, int H, int W, int G, int C, int kh, int kw,
                                         int stride_h, int stride_w, int pad_h, int pad_w,
                                         int dil_h, int dil_w, dcn_dtype dtype) {
    return dcn_core_backward_workspace_bytes_path(N, H, W, G, C, kh, kw, stride_h, stride_w,
                                                  pad_h, pad_w, dil_h, dil_w, dtype, 0u);
}

dcn_status dcn_core_backward_path(const void *x, const float *offset, const float *mask,
                                  const void *grad_out, void *grad_x, float *grad_offset,
                                  float *grad_mask, void *workspace, size_t workspace_bytes, int N,
                                  int H, int W, int G, int C, int kh, int kw, int stride_h,
                                  int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                                  float offset_scale, int softmax, dcn_dtype dtype, unsigned path,
                                  hipStream_t stream) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (!valid_path(path)) return DCN_ERR_PARAM;
    if (N < 0 || H <= 0 || W <= 0 || G <= 0 || C <= 0) return DCN_ERR_SHAPE;
    dcn_status st = check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w);
    if (st != DCN_OK) return st;
    const long long Ho = out_extent(H, kh, stride_h, pad_h, dil_h);
    const long long Wo = out_extent(W, kw, stride_w, pad_w, dil_w);
    if (Ho <= 0 || Wo <= 0) return DCN_ERR_SHAPE;
    if ((long long)(H + 1) * (W + 1) * G * C > kI32) return DCN_ERR_SHAPE;
    if ((long long)N * Ho * Wo * G > kI32) return DCN_ERR_SHAPE;
    if (N == 0) return DCN_OK;
    if (!x || !offset || !grad_out) return DCN_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned(x, es) || !aligned(grad_out, es) || !aligned(grad_x, es) ||
        !aligned(offset, 4) || (mask && !aligned(mask, 4)) || !aligned(grad_offset, 4) ||
        !aligned(grad_mask, 4))
        return DCN_ERR_ALIGN;
    dcn::CoreBwdPlan plan;
    dcn::plan_core_bwd(N, H, W, G, C, (int)Ho, (int)Wo, kh * kw, dtype,
                       (path & DCN_BWD_ATOMIC) != 0, plan);
    if (grad_x && plan.total > 0) {
        if (!workspace || !aligned(workspace, 256) || workspace_bytes < plan.total)
            return DCN_ERR_WORKSPACE;
    }
    if (!grad_x && !grad_offset && !grad_mask) return DCN_OK;

    dcn::CoreBwdLaunch a;
    a.x = x; a.offset = offset; a.mask = mask; a.grad_out = grad_out;
    a.grad_x = grad_x; a.grad_offset = grad_offset; a.grad_mask = grad_mask;
    a.workspace = workspace;
    a.N = N; a.H = H; a.W = W; a.G = G; a.C = C; a.kh = kh; a.kw = kw;
    a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w; a.dh = dil_h; a.dw = dil_w;
    a.Ho = (int)Ho; a.Wo = (int)Wo;
    a.offset_scale = offset_scale;
    a.softmax = softmax;
    a.dtype = dtype;
    a.path = path;
    return hip_status(dcn::launch_dcn_core_bwd(a, plan, stream));
}

dcn_status dcn_core_backward(const void *x, const float *offset, const float *mask,
                             const void *grad_out, void *grad_x, float *grad_offset,
                             float *grad_mask, void *workspace, size_t workspace_bytes, int N,
                             int H, int W, int G, int C, int kh, int kw, int stride_h, int stride_w,
                             int pad_h, int pad_w, int dil_h, int dil_w, float offset_scale,
                             int softmax, dcn_dtype dtype, hipStream_t stream) {
    return dcn_core_backward_path(x, offset, mask, grad_out, grad_x, grad_offset, grad_mask,
                                  workspace, workspace_bytes, N, H, W, G, C, kh, kw, stride_h,
                                  stride_w, pad_h, pad_w, dil_h, dil_w, offset_scale, softmax,
                                  dtype, 0u, stream);
}

size_t dcn_v2_workspace_bytes(int N, int Cin, int H, int W, int Cout, int kh, int kw, int stride_h,
                              int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                              dcn_dtype dtype) {
    if (check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w) != DCN_OK) return 0;
    if (H <= 0 || W <= 0) return 0;
    dcn::V2Plan plan;
    if (!dcn::plan_dcn_v2(N, Cin, H, W, Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h,
                          dil_w, dtype, plan))
        return 0;
    return plan.total;
}

// Argument checks shared by dcn_v2_forward, dcn_v2_forward_noalloc and dcn_v2_im2col
// (columns_only: no weight and no out). On DCN_OK with N > 0, `a` is ready to launch
// except for its workspace; all checks here precede any HIP call.
static dcn_status v2_check(const void *x, const float *offset, const float *mask,
                           const void *weight, void *out, int N, int Cin, int H, int W, int Cout,
                           int kh, int kw, int stride_h, int stride_w, int pad_h, int pad_w,
                           int dil_h, int dil_w, int deform_groups, int softmax, dcn_dtype dtype,
                           bool columns_only, dcn::V2Launch &a) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (dtype == DCN_F32) return DCN_ERR_DTYPE;
    if (N < 0 || Cin <= 0 || H <= 0 || W <= 0 || Cout <= 0) return DCN_ERR_SHAPE;
    dcn_status st = check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w);
    if (st != DCN_OK) return st;
    if (deform_groups <= 0 || Cin % deform_groups != 0) return DCN_ERR_PARAM;
    if (deform_groups > 1 && (Cin / deform_groups) % 8 != 0) return DCN_ERR_PARAM;
    dcn::V2Plan plan;
    if (!dcn::plan_dcn_v2(N, Cin, H, W, Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h,
                          dil_w, dtype, plan))
        return DCN_ERR_SHAPE;
    // 32-bit limits of the kernels' in-image offsets and pixel counts
    if ((long long)(H + 1) * (W + 1) * plan.Cin_pad > kI32) return DCN_ERR_SHAPE;
    if (plan.Pp > kI32 || (long long)N * Cin * H * W > (1LL << 40)) return DCN_ERR_SHAPE;
    if (N == 0) return DCN_OK;
    if (!x || !offset || (!columns_only && (!weight || !out))) return DCN_ERR_NULL;
    if (!aligned(x, 2) || !aligned(weight, 2) || !aligned(out, 2) || !aligned(offset, 4) ||
        (mask && !aligned(mask, 4)))
        return DCN_ERR_ALIGN;
    if (columns_only) {
        weight = nullptr;
        out = nullptr;
    }
    a.x = x; a.offset = offset; a.mask = mask; a.weight = weight; a.out = out;
    a.packed_weight = nullptr;
    a.workspace = nullptr;
    a.N = N; a.Cin = Cin; a.H = H; a.W = W; a.Cout = Cout; a.kh = kh; a.kw = kw;
    a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w; a.dh = dil_h; a.dw = dil_w;
    a.dg = deform_groups;
    a.softmax = softmax;
    a.dtype = dtype;
    a.plan = plan;
    return DCN_OK;
}

// Shared by dcn_v2_forward and dcn_v2_im2col (weight == out == NULL: columns only).
static dcn_status v2_call(const void *x, const float *offset, const float *mask, const void *weight,
                          void *out, void *workspace, size_t workspace_bytes, int N, int Cin, int H,
                          int W, int Cout, int kh, int kw, int stride_h, int stride_w, int pad_h,
                          int pad_w, int dil_h, int dil_w, int deform_groups, int softmax,
                          dcn_dtype dtype, hipStream_t stream, bool columns_only) {
    dcn::V2Launch a;
    const dcn_status st = v2_check(x, offset, mask, weight, out, N, Cin, H, W, Cout, kh, kw,
                                   stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, deform_groups,
                                   softmax, dtype, columns_only, a);
    if (st != DCN_OK || N == 0) return st;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < a.plan.total)
        return DCN_ERR_WORKSPACE;
    a.workspace = workspace;
    return hip_status(dcn::launch_dcn_v2(a, stream));
}

dcn_status dcn_v2_forward(const void *x, const float *offset, const float *mask, const void *weight,
                          void *out, void *workspace, size_t workspace_bytes, int N, int Cin, int H,
                          int W, int Cout, int kh, int kw, int stride_h, int stride_w, int pad_h,
                          int pad_w, int dil_h, int dil_w, int deform_groups, int softmax,
                          dcn_dtype dtype, hipStream_t stream) {
    return v2_call(x, offset, mask, weight, out, workspace, workspace_bytes, N, Cin, H, W, Cout, kh,
                   kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, deform_groups, softmax,
                   dtype, stream, false);
}

// The weight dimensions of a DCNv2 layer (Cin_pad, K, Rp, Mp) as plan_dcn_v2 sets them:
// the plan of a one-pixel layer with the same weight.
static bool v2_weight_plan(int Cout, int Cin, int kh, int kw, dcn::V2Plan &plan) {
    if (Cout <= 0 || Cin <= 0 || kh <= 0 || kw <= 0 || kh * kw > 64) return false;
    return dcn::plan_dcn_v2(1, Cin, kh, kw, Cout, kh, kw, 1, 1, 0, 0, 1, 1, DCN_BF16, plan);
}

size_t dcn_v2_packed_weight_bytes(int Cout, int Cin, int kh, int kw) {
    dcn::V2Plan plan;
    if (!v2_weight_plan(Cout, Cin, kh, kw, plan)) return 0;
    return (size_t)plan.Mp * plan.Rp * 2;
}

dcn_status dcn_v2_pack_weight(const void *weight, void *packed, size_t packed_bytes, int Cout, int Cin,
                              int kh, int kw, dcn_dtype dtype, hipStream_t stream) {
    if (!valid_dtype(dtype) || dtype == DCN_F32) return DCN_ERR_DTYPE;
    dcn::V2Plan plan;
    if (!v2_weight_plan(Cout, Cin, kh, kw, plan)) return DCN_ERR_SHAPE;
    if ((long long)plan.Mp * plan.Rp * 2 >= (1LL << 31)) return DCN_ERR_SHAPE;
    if (!weight || !packed) return DCN_ERR_NULL;
    if (!aligned(weight, 2) || !aligned(packed, 16)) return DCN_ERR_ALIGN;
    if (packed_bytes < (size_t)plan.Mp * plan.Rp * 2) return DCN_ERR_WORKSPACE;
    return hip_status(dcn::launch_dcn_v2_pack_weight(weight, packed, Cout, Cin, plan, stream));
}

dcn_status dcn_v2_forward_prepacked(const void *x, const float *offset, const float *mask,
                                    const void *packed_weight, size_t packed_bytes, void *out,
                                    void *workspace, size_t workspace_bytes, int N, int Cin, int H,
                                    int W, int Cout, int kh, int kw, int stride_h, int stride_w,
                                    int pad_h, int pad_w, int dil_h, int dil_w, int deform_groups,
                                    int softmax, dcn_dtype dtype, hipStream_t stream) {
    dcn::V2Launch a;
    const dcn_status st = v2_check(x, offset, mask, packed_weight, out, N, Cin, H, W, Cout, kh, kw,
                                   stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, deform_groups,
                                   softmax, dtype, false, a);
    if (st != DCN_OK || N == 0) return st;
    if (!dcn::v2_fused_applies(a.plan, deform_groups, true)) return DCN_ERR_PARAM;
    if (!aligned(packed_weight, 16)) return DCN_ERR_ALIGN;
    if (packed_bytes < (size_t)a.plan.Mp * a.plan.Rp * 2) return DCN_ERR_WORKSPACE;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < a.plan.total)
        return DCN_ERR_WORKSPACE;
    a.packed_weight = packed_weight;
    a.workspace = workspace;
    return hip_status(dcn::launch_dcn_v2(a, stream));
}

dcn_status dcn_v2_im2col(const void *x, const float *offset, const float *mask, void *workspace,
                         size_t workspace_bytes, int N, int Cin, int H, int W, int Cout, int kh,
                         int kw, int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                         int dil_w, int deform_groups, int softmax, dcn_dtype dtype,
                         hipStream_t stream) {
    return v2_call(x, offset, mask, nullptr, nullptr, workspace, workspace_bytes, N, Cin, H, W,
                   Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, deform_groups,
                   softmax, dtype, stream, true);
}

size_t dcn_v2_noalloc_bytes(int N, int Cin, int H, int W, int Cout, int kh, int kw, int stride_h,
                            int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                            int deform_groups, dcn_dtype dtype) {
    if (check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w) != DCN_OK) return 0;
    if (H <= 0 || W <= 0 || deform_groups <= 0) return 0;
    dcn::V2Plan plan;
    if (!dcn::plan_dcn_v2(N, Cin, H, W, Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h,
                          dil_w, dtype, plan))
        return 0;
    return dcn::v2_fused_applies(plan, deform_groups, true) ? plan.off_col : plan.total;
}

dcn_status dcn_v2_forward_noalloc(const void *x, const float *offset, const float *mask,
                                  const void *weight, void *out, int N, int Cin, int H, int W,
                                  int Cout, int kh, int kw, int stride_h, int stride_w, int pad_h,
                                  int pad_w, int dil_h, int dil_w, int deform_groups, int softmax,
                                  dcn_dtype dtype, hipStream_t stream) {
    dcn::V2Launch a;
    const dcn_status st = v2_check(x, offset, mask, weight, out, N, Cin, H, W, Cout, kh, kw,
                                   stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, deform_groups,
                                   softmax, dtype, false, a);
    if (st != DCN_OK || N == 0) return st;
    const size_t need = dcn::v2_fused_applies(a.plan, deform_groups, true) ? a.plan.off_col
                                                                            : a.plan.total;
    if (need > (size_t)DCN_V2_NOALLOC_SCRATCH_BYTES) return DCN_ERR_SCRATCH;
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return hip_status(e);
    a.workspace = ws;
    return hip_status(dcn::launch_dcn_v2(a, stream));
}

// Shape checks and plan of the DCNv2 backward (the forward's limits).
static dcn_status v2_bwd_plan(int N, int Cin, int H, int W, int Cout, int kh, int kw, int stride_h,
                              int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                              int deform_groups, dcn_dtype dtype, dcn::V2BwdPlan &plan) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (dtype == DCN_F32) return DCN_ERR_DTYPE;
    if (N < 0 || Cin <= 0 || H <= 0 || W <= 0 || Cout <= 0) return DCN_ERR_SHAPE;
    dcn_status st = check_window(kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w);
    if (st != DCN_OK) return st;
    if (deform_groups <= 0 || Cin % deform_groups != 0) return DCN_ERR_PARAM;
    if (deform_groups > 1 && (Cin / deform_groups) % 8 != 0) return DCN_ERR_PARAM;
    if (!dcn::plan_dcn_v2_bwd(N, Cin, H, W, Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h,
                              dil_w, deform_groups, dtype, plan))
        return DCN_ERR_SHAPE;
    // 32-bit limits: in-image offsets, pixel counts, bucket entries and sample ids
    if ((long long)(H + 1) * (W + 1) * plan.Cin_pad > kI32) return DCN_ERR_SHAPE;
    if (plan.Pp > kI32 || plan.entries > kI32 || plan.D > kI32) return DCN_ERR_SHAPE;
    if ((long long)N * Cin * H * W > (1LL << 40)) return DCN_ERR_SHAPE;
    return DCN_OK;
}

size_t dcn_v2_backward_workspace_bytes(int N, int Cin, int H, int W, int Cout, int kh, int kw,
                                       int stride_h, int stride_w, int pad_h, int pad_w, int dil_h,
                                       int dil_w, int deform_groups, dcn_dtype dtype) {
    dcn::V2BwdPlan plan;
    if (v2_bwd_plan(N, Cin, H, W, Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h, dil_w,
                    deform_groups, dtype, plan) != DCN_OK)
        return 0;
    return plan.total;
}

dcn_status dcn_v2_backward(const void *x, const float *offset, const float *mask, const void *weight,
                           const void *grad_out, void *grad_x, float *grad_offset, float *grad_mask,
                           float *grad_weight, void *workspace, size_t workspace_bytes, int N,
                           int Cin, int H, int W, int Cout, int kh, int kw, int stride_h,
                           int stride_w, int pad_h, int pad_w, int dil_h, int dil_w,
                           int deform_groups, int softmax, dcn_dtype dtype, hipStream_t stream) {
    dcn::V2BwdPlan plan;
    dcn_status st = v2_bwd_plan(N, Cin, H, W, Cout, kh, kw, stride_h, stride_w, pad_h, pad_w, dil_h,
                                dil_w, deform_groups, dtype, plan);
    if (st != DCN_OK) return st;
    if (N == 0) return DCN_OK;
    if (!x || !offset || !weight || !grad_out) return DCN_ERR_NULL;
    if (!grad_x && !grad_offset && !grad_mask && !grad_weight) return DCN_OK;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < plan.total)
        return DCN_ERR_WORKSPACE;
    if (!aligned(x, 2) || !aligned(weight, 2) || !aligned(grad_out, 2) || !aligned(grad_x, 2) ||
        !aligned(offset, 4) || (mask && !aligned(mask, 4)) || !aligned(grad_offset, 4) ||
        !aligned(grad_mask, 4) || !aligned(grad_weight, 4))
        return DCN_ERR_ALIGN;
    dcn::V2BwdLaunch a;
    a.x = x; a.offset = offset; a.mask = mask; a.weight = weight; a.grad_out = grad_out;
    a.grad_x = grad_x; a.grad_offset = grad_offset; a.grad_mask = grad_mask;
    a.grad_weight = grad_weight;
    a.workspace = workspace;
    a.N = N; a.Cin = Cin; a.H = H; a.W = W; a.Cout = Cout; a.kh = kh; a.kw = kw;
    a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w; a.dh = dil_h; a.dw = dil_w;
    a.dg = deform_groups;
    a.softmax = softmax;
    a.dtype = dtype;
    a.plan = plan;
    return hip_status(dcn::launch_dcn_v2_bwd(a, stream));
}

dcn_status deform_agg_forward(const void *feat, const int32_t *spatial_shape,
                              const int32_t *scale_start, const float *loc, const float *weights,
                              void *out, int B, int P_total, int A, int pts, int cams, int scales,
                              int G, int Cg, int softmax, dcn_dtype dtype, hipStream_t stream) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (B < 0 || A < 0 || P_total <= 0 || pts <= 0 || cams <= 0 || scales <= 0 || G <= 0 ||
        Cg <= 0)
        return DCN_ERR_SHAPE;
    if ((long long)cams * scales > dcn::kAggMaxMaps) return DCN_ERR_SHAPE;
    if ((long long)B * P_total * G * Cg > kI32) return DCN_ERR_SHAPE;
    if ((long long)B * A * G > kI32) return DCN_ERR_SHAPE;
    if ((long long)pts * cams * scales * G > kI32) return DCN_ERR_SHAPE;
    if (!spatial_shape || !scale_start) return DCN_ERR_NULL;
    dcn::AggLaunch a;
    for (int i = 0; i < cams * scales; ++i) {
        const int h = spatial_shape[2 * i], w = spatial_shape[2 * i + 1], s0 = scale_start[i];
        if (h <= 0 || w <= 0 || s0 < 0) return DCN_ERR_SHAPE;
        if ((long long)s0 + (long long)h * w > P_total) return DCN_ERR_SHAPE;
        a.maps.H[i] = h;
        a.maps.W[i] = w;
        a.maps.start[i] = s0;
    }
    if (B == 0 || A == 0) return DCN_OK;
    if (!feat || !loc || !weights || !out) return DCN_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned(feat, es) || !aligned(out, es) || !aligned(loc, 8) || !aligned(weights, 4))
        return DCN_ERR_ALIGN;
    a.feat = feat; a.loc = loc; a.weights = weights; a.out = out;
    a.B = B; a.P_total = P_total; a.A = A; a.pts = pts; a.cams = cams; a.scales = scales;
    a.G = G; a.Cg = Cg; a.softmax = softmax;
    a.dtype = dtype;
    return hip_status(dcn::launch_deform_agg(a, stream));
}

size_t deform_agg_backward_workspace_bytes_path(int B, int P_total, int A, int pts, int cams,
                                                int scales, int G, int Cg, dcn_dtype dtype,
                                                unsigned path) {
    if (!valid_path(path)) return 0;
    if (!valid_dtype(dtype) || B < 0 || A < 0 || P_total <= 0 || pts <= 0 || cams <= 0 ||
        scales <= 0 || G <= 0 || Cg <= 0)
        return 0;
    dcn::AggBwdPlan plan;
    dcn::plan_agg_bwd(B, P_total, A, pts, cams, scales, G, Cg, dtype, (path & DCN_BWD_ATOMIC) != 0,
                      plan);
    return plan.total;
}

size_t deform_agg_backward_workspace_bytes(int B, int P_total, int A, int pts, int cams,
                                           int scales, int G, int Cg, dcn_dtype dtype) {
    return deform_agg_backward_workspace_bytes_path(B, P_total, A, pts, cams, scales, G, Cg, dtype,
                                                    0u);
}

dcn_status deform_agg_backward_path(const void *feat, const int32_t *spatial_shape,
                                    const int32_t *scale_start, const float *loc,
                                    const float *weights, const void *grad_out, void *grad_feat,
                                    float *grad_loc, float *grad_weights, void *workspace,
                                    size_t workspace_bytes, int B, int P_total, int A, int pts,
                                    int cams, int scales, int G, int Cg, int softmax,
                                    dcn_dtype dtype, unsigned path, hipStream_t stream) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (!valid_path(path)) return DCN_ERR_PARAM;
    if (B < 0 || A < 0 || P_total <= 0 || pts <= 0 || cams <= 0 || scales <= 0 || G <= 0 ||
        Cg <= 0)
        return DCN_ERR_SHAPE;
    if ((long long)cams * scales > dcn::kAggMaxMaps) return DCN_ERR_SHAPE;
    if (Cg > 512) return DCN_ERR_SHAPE;  // channel rounds of the backward kernel
    if ((long long)B * P_total * G * Cg > kI32) return DCN_ERR_SHAPE;
    if ((long long)B * A * G > kI32) return DCN_ERR_SHAPE;
    if ((long long)pts * cams * scales * G > kI32) return DCN_ERR_SHAPE;
    if ((long long)B * A * pts * cams * scales * G > kI32) return DCN_ERR_SHAPE;
    if (!spatial_shape || !scale_start) return DCN_ERR_NULL;
    dcn::AggBwdLaunch a;
    for (int i = 0; i < cams * scales; ++i) {
        const int h = spatial_shape[2 * i], w = spatial_shape[2 * i + 1], s0 = scale_start[i];
        if (h <= 0 || w <= 0 || s0 < 0) return DCN_ERR_SHAPE;
        if ((long long)s0 + (long long)h * w > P_total) return DCN_ERR_SHAPE;
        a.maps.H[i] = h;
        a.maps.W[i] = w;
        a.maps.start[i] = s0;
    }
    if (B == 0) return DCN_OK;
    if (A == 0 && !grad_feat) return DCN_OK;  // with A == 0 grad_feat is all zeros
    if (!feat || (A > 0 && (!loc || !weights || !grad_out))) return DCN_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned(feat, es) || !aligned(grad_out, es) || !aligned(grad_feat, es) ||
        !aligned(loc, 8) || !aligned(weights, 4) || !aligned(grad_loc, 4) ||
        !aligned(grad_weights, 4))
        return DCN_ERR_ALIGN;
    dcn::AggBwdPlan plan;
    dcn::plan_agg_bwd(B, P_total, A, pts, cams, scales, G, Cg, dtype, (path & DCN_BWD_ATOMIC) != 0,
                      plan);
    const bool needs_ws =
        (grad_loc || (grad_feat && (plan.binned || dtype != DCN_F32))) && plan.total > 0;
    if (needs_ws && (!workspace || !aligned(workspace, 256) || workspace_bytes < plan.total))
        return DCN_ERR_WORKSPACE;
    if (!grad_feat && !grad_loc && !grad_weights) return DCN_OK;
    a.feat = feat; a.loc = loc; a.weights = weights; a.grad_out = grad_out;
    a.grad_feat = grad_feat; a.grad_loc = grad_loc; a.grad_weights = grad_weights;
    a.workspace = workspace;
    a.B = B; a.P_total = P_total; a.A = A; a.pts = pts; a.cams = cams; a.scales = scales;
    a.G = G; a.Cg = Cg; a.softmax = softmax;
    a.dtype = dtype;
    a.path = path;
    return hip_status(dcn::launch_deform_agg_bwd(a, plan, stream));
}

dcn_status deform_agg_backward(const void *feat, const int32_t *spatial_shape,
                               const int32_t *scale_start, const float *loc, const float *weights,
                               const void *grad_out, void *grad_feat, float *grad_loc,
                               float *grad_weights, void *workspace, size_t workspace_bytes, int B,
                               int P_total, int A, int pts, int cams, int scales, int G, int Cg,
                               int softmax, dcn_dtype dtype, hipStream_t stream) {
    return deform_agg_backward_path(feat, spatial_shape, scale_start, loc, weights, grad_out,
                                    grad_feat, grad_loc, grad_weights, workspace, workspace_bytes,
                                    B, P_total, A, pts, cams, scales, G, Cg, softmax, dtype, 0u,
                                    stream);
}


dcn_status deform_roi_pool_forward(const void *x, const float *rois, const float *offset, void *out,
                                   int N, int H, int W, int C, int R, int k, int sampling_ratio,
                                   float spatial_scale, float gamma, dcn_dtype dtype,
                                   hipStream_t stream) {
    if (!valid_dtype(dtype)) return DCN_ERR_DTYPE;
    if (N <= 0 || H <= 0 || W <= 0 || C <= 0 || R < 0) return DCN_ERR_SHAPE;
    if (k <= 0 || sampling_ratio <= 0 || sampling_ratio > 64) return DCN_ERR_PARAM;
    if ((long long)(H + 1) * (W + 1) * C > kI32) return DCN_ERR_SHAPE;
    if ((long long)R * k * k * C > kI32) return DCN_ERR_SHAPE;
    if (R == 0) return DCN_OK;
    if (!x || !rois || !out) return DCN_ERR_NULL;
    const size_t es = dtype_size(dtype);
    if (!aligned(x, es) || !aligned(out, es) || !aligned(rois, 4) || !aligned(offset, 8))
        return DCN_ERR_ALIGN;
    dcn::RoiLaunch a;
    a.x = x; a.rois = rois; a.offset = offset; a.out = out;
    a.N = N; a.H = H; a.W = W; a.C = C; a.R = R; a.k = k; a.S = sampling_ratio;
    a.spatial_scale = spatial_scale; a.gamma = gamma;
    a.dtype = dtype;
    return hip_status(dcn::launch_deform_roi_pool(a, stream));
}

dcn_status dcn_mfma_probe(float *sink, int blocks, int iters, hipStream_t stream) {
    if (blocks <= 0 || iters < 0) return DCN_ERR_PARAM;
    if (!sink) return DCN_ERR_NULL;
    if (!aligned(sink, 4)) return DCN_ERR_ALIGN;
    return hip_status(dcn::launch_mfma_probe(sink, blocks, iters, stream));
}

}  // extern "C"
