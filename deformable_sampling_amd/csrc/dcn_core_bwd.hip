// DCNv3/v4 core backward, channels-last, for gfx950.
//
// The gradients of the core's deformable sum ("DCNv4 in YOLOv11", lpnh.cn, section
// 1.1; bilinear kernel from "Hands-on DCNv1 in PyTorch", agent.csdn.net, section 2).
// The pages give no backward pass; these are the derivatives of that sum. For one
// (pixel, group) pair and tap k at (y0 + fy, x0 + fx), with corners X_ab (a along y,
// b along x; a corner outside the image is 0) and G the pair's C channels of
// grad_out, let D_ab = sum_c G_c X_ab,c (one dot product per corner). Then
//   grad_m_k   = (1-fy)((1-fx) D_00 + fx D_01) + fy((1-fx) D_10 + fx D_11)
//   d/dy       = (1-fx)(D_10 - D_00) + fx (D_11 - D_01)
//   d/dx       = (1-fy)(D_01 - D_00) + fy (D_11 - D_10)
//   grad_off_k = offset_scale * m_k * (d/dx, d/dy)
//   grad_x[corner ab, c] += m_k * w_ab * G_c          (w_ab the bilinear weights)
// and with the DCNv3 softmax, grad_logit_k = m_k (grad_m_k - sum_j m_j grad_m_j).
// Derivatives at integer positions are taken from the right (the cell the
// position's floor selects), where a zero-weight corner still enters d/dx, d/dy.
//
// Mapping (the forward's): the unit is a (pixel, group) pair; a pair's C channels
// are spread over S lanes of V channels each (16-byte vectors where alignment
// allows), Q = 64/S pairs per wavefront, PB = 4Q pairs per 256-thread block.
//   1. offsets and modulation of the block's pairs -> LDS (coalesced), softmax;
//   2. per lane and tap: four corner vector loads, the four partial dots D_ab over
//      the lane's channels, and the grad_x scatter as fp32 atomic adds (corners
//      inside the image with nonzero weight only); the partial dots are summed over
//      the pair's S lanes and kept in LDS;
//   3. per pair: grad_offset and grad_mask from the dots, written over the staged
//      offsets and modulation in LDS, then stored with coalesced writes.
// grad_x accumulates in fp32: in the caller's buffer for fp32, in the workspace
// for fp16/bf16 (then rounded once into grad_x by a conversion kernel). The
// accumulator is cleared by a fill kernel first. Atomic order varies, so grad_x is
// not bitwise reproducible run to run; grad_offset and grad_mask are.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

constexpr int kThreads = 256;

struct BwdParams {
    int N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo;
    float offset_scale;
    int softmax, has_mask, vec_io;
    int want_x, want_off, want_mask;
    int npairs, S, Q, nchunk, PB, nblocks;
};

// Copy n floats between global memory and LDS with the whole block (float4 when
// both ends are 16-byte aligned).
__device__ __forceinline__ void block_copy(float *dst, const float *src, int n, bool vec) {
    const int tid = threadIdx.x;
    int done = 0;
    if (vec) {
        const int n4 = n >> 2;
        const float4 *s4 = reinterpret_cast<const float4 *>(src);
        float4 *d4 = reinterpret_cast<float4 *>(dst);
        for (int i = tid; i < n4; i += kThreads) d4[i] = s4[i];
        done = n4 << 2;
    }
    for (int i = done + tid; i < n; i += kThreads) dst[i] = src[i];
}

// Sum over the S lanes of segment q (lanes q*S .. q*S+S-1); every lane of the
// segment receives the total.
__device__ __forceinline__ float seg_total(float v, int S, int q) {
    if ((S & (S - 1)) == 0) return seg_sum_pow2(v, S);
    float r = 0.0f;
    for (int j = 0; j < S; ++j) r += __shfl(v, q * S + j, 64);
    return r;
}
__device__ __forceinline__ float seg_max(float v, int S, int q) {
    if ((S & (S - 1)) == 0) return seg_max_pow2(v, S);
    float r = -INFINITY;
    for (int j = 0; j < S; ++j) r = fmaxf(r, __shfl(v, q * S + j, 64));
    return r;
}

// Corner geometry of one tap: integer corner (y0, x0), fractions f and their
// complements u = 1 - f, and which of the four corners lie inside the image.
struct TapGeo {
    int y0, x0;
    float fy, fx, uy, ux;
    bool vy0, vy1, vx0, vx1;
};

// base + t -> corner c0 = base + floor(t), f = t - floor(t), u = (floor(t) + 1) - t.
// Each of f and u is exact whenever it is below 1/2 (f = 1 + t rounds only for t in
// (-1/2, 0), where u = -t is exact; u = 1 - t rounds only for t in (0, 1/2), where f
// = t is exact), so both bilinear weight factors carry a relative error of at most
// one rounding. Deriving u as 1 - f instead would give a small u an absolute error
// of up to 2^-25, and a large relative one. |t| is clamped at 2^24 px as in the
// forward.
__device__ __forceinline__ void split_coord_fu(int base, float t, int &c0, float &f, float &u) {
    t = fminf(fmaxf(t, -16777216.0f), 16777216.0f);
    const float fl = floorf(t);
    f = t - fl;
    u = (fl + 1.0f) - t;
    c0 = base + (int)fl;
}

__device__ __forceinline__ TapGeo tap_geo(int by, int bx, float2 d, float s, int H, int W) {
    TapGeo t;
    split_coord_fu(by, __fmul_rn(s, d.y), t.y0, t.fy, t.uy);
    split_coord_fu(bx, __fmul_rn(s, d.x), t.x0, t.fx, t.ux);
    t.vy0 = (unsigned)t.y0 < (unsigned)H;
    t.vy1 = (unsigned)(t.y0 + 1) < (unsigned)H;
    t.vx0 = (unsigned)t.x0 < (unsigned)W;
    t.vx1 = (unsigned)(t.x0 + 1) < (unsigned)W;
    return t;
}

template <class E, int V, int KH, int KW>
__global__ __launch_bounds__(kThreads) void dcn_core_bwd_kernel(
    const typename E::bits *__restrict__ x, const float *__restrict__ offset,
    const float *__restrict__ mask, const typename E::bits *__restrict__ gout,
    float *__restrict__ gacc, float *__restrict__ goff, float *__restrict__ gmask, BwdParams p) {
    extern __shared__ float smem[];
    const int kh = KH > 0 ? KH : p.kh;
    const int kw = KW > 0 ? KW : p.kw;
    const int K = kh * kw;
    float *s_off = smem;               // [PB][K][2] offsets, later grad_offset
    float *s_m = s_off + p.PB * K * 2; // [PB][K] modulation m_k, later grad_mask
    float *s_d = s_m + p.PB * K;       // [PB][K][4] corner dots D_ab

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int pair0 = blk * p.PB;
    const int npb = min(p.PB, p.npairs - pair0);

    // 1. offsets and modulation of pairs [pair0, pair0 + npb) -> LDS
    block_copy(s_off, offset + (size_t)pair0 * K * 2, npb * K * 2, p.vec_io);
    if (p.has_mask) {
        block_copy(s_m, mask + (size_t)pair0 * K, npb * K, p.vec_io);
    } else {
        for (int i = threadIdx.x; i < npb * K; i += kThreads) s_m[i] = p.softmax ? 0.0f : 1.0f;
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane / p.S, s = lane - q * p.S;
    const int lp = wave * p.Q + q;
    const bool active = (q < p.Q) && (lp < npb);

    if (p.softmax) {  // DCNv3: softmax over the K logits of each pair, in place
        float *ml = s_m + lp * K;
        float mx = -INFINITY;
        if (active)
            for (int k = s; k < K; k += p.S) mx = fmaxf(mx, ml[k]);
        mx = seg_max(mx, p.S, q);
        float sum = 0.0f;
        if (active)
            for (int k = s; k < K; k += p.S) sum += expf(ml[k] - mx);
        sum = seg_total(sum, p.S, q);
        if (active) {
            const float inv = 1.0f / sum;
            for (int k = s; k < K; k += p.S) ml[k] = expf(ml[k] - mx) * inv;
        }
        __syncthreads();
    }

    const int e = pair0 + lp;
    const int pix = e / p.G;
    const int g = e - pix * p.G;
    const int wo = pix % p.Wo;
    const int t2 = pix / p.Wo;
    const int ho = t2 % p.Ho;
    const int n = t2 / p.Ho;
    const int GC = p.G * p.C;
    float *so = s_off + lp * K * 2;
    float *sm = s_m + lp * K;
    float *sd = s_d + lp * K * 4;
    const int by0 = ho * p.sh - p.ph, bx0 = wo * p.sw - p.pw;

    // 2. corner dots and the grad_x scatter
    if (active) {
        const size_t img_base = (size_t)n * p.H * p.W * GC + (size_t)g * p.C;
        const typename E::bits *img = x + img_base;
        float *acc = p.want_x ? gacc + img_base : nullptr;
        const typename E::bits *gp = gout + (size_t)pix * GC + g * p.C;
        int round = 0;
        for (int ch = s; ch < p.nchunk; ch += p.S, ++round) {
            float gv[V];
            load_f32<E, V>(gp + ch * V, gv);
            const typename E::bits *imgc = img + ch * V;
            auto tap = [&](int i, int j) {
                const int k = i * kw + j;
                const float2 d = *reinterpret_cast<const float2 *>(so + 2 * k);
                const TapGeo t = tap_geo(by0 + i * p.dh, bx0 + j * p.dw, d, p.offset_scale, p.H, p.W);
                const int yc0 = min(max(t.y0, 0), p.H - 1), yc1 = min(max(t.y0 + 1, 0), p.H - 1);
                const int xc0 = min(max(t.x0, 0), p.W - 1), xc1 = min(max(t.x0 + 1, 0), p.W - 1);
                const int o00 = (yc0 * p.W + xc0) * GC, o01 = (yc0 * p.W + xc1) * GC;
                const int o10 = (yc1 * p.W + xc0) * GC, o11 = (yc1 * p.W + xc1) * GC;
                float a[V], b[V], c[V], dd[V];
                load_f32<E, V>(imgc + o00, a);
                load_f32<E, V>(imgc + o01, b);
                load_f32<E, V>(imgc + o10, c);
                load_f32<E, V>(imgc + o11, dd);
                float D00 = 0.0f, D01 = 0.0f, D10 = 0.0f, D11 = 0.0f;
#pragma unroll
                for (int u = 0; u < V; ++u) {
                    D00 = fmaf(gv[u], a[u], D00);
                    D01 = fmaf(gv[u], b[u], D01);
                    D10 = fmaf(gv[u], c[u], D10);
                    D11 = fmaf(gv[u], dd[u], D11);
                }
                if (acc) {
                    const float m = sm[k];
                    const float gy0 = t.vy0 ? t.uy * m : 0.0f;
                    const float gy1 = t.vy1 ? t.fy * m : 0.0f;
                    const float gx0 = t.vx0 ? t.ux : 0.0f;
                    const float gx1 = t.vx1 ? t.fx : 0.0f;
                    const float w[4] = {gy0 * gx0, gy0 * gx1, gy1 * gx0, gy1 * gx1};
                    const int o[4] = {o00, o01, o10, o11};
                    float *accc = acc + ch * V;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (w[r] != 0.0f) {
#pragma unroll
                            for (int u = 0; u < V; ++u) unsafeAtomicAdd(accc + o[r] + u, w[r] * gv[u]);
                        }
                    }
                }
                D00 = seg_total(D00, p.S, q);
                D01 = seg_total(D01, p.S, q);
                D10 = seg_total(D10, p.S, q);
                D11 = seg_total(D11, p.S, q);
                if (s == 0) {
                    float4 *dst = reinterpret_cast<float4 *>(sd + 4 * k);
                    float4 v = make_float4(D00, D01, D10, D11);
                    if (round > 0) {
                        const float4 o = *dst;
                        v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
                    }
                    *dst = v;
                }
            };
            if constexpr (KH > 0) {
#pragma unroll
                for (int i = 0; i < KH; ++i)
#pragma unroll
                    for (int j = 0; j < KW; ++j) tap(i, j);
            } else {
                for (int i = 0; i < kh; ++i)
                    for (int j = 0; j < kw; ++j) tap(i, j);
            }
        }
    }
    if (!p.want_off && !p.want_mask) return;  // uniform over the grid
    __syncthreads();

    // 3. grad_offset and grad_mask of each pair from its dots
    float dot = 0.0f;
    if (active) {
        for (int k = s; k < K; k += p.S) {
            const int i = k / kw, j = k - (k / kw) * kw;
            const float2 d = *reinterpret_cast<const float2 *>(so + 2 * k);
            const TapGeo t = tap_geo(by0 + i * p.dh, bx0 + j * p.dw, d, p.offset_scale, p.H, p.W);
            const float4 D = *reinterpret_cast<const float4 *>(sd + 4 * k);
            const float D00 = (t.vy0 && t.vx0) ? D.x : 0.0f;
            const float D01 = (t.vy0 && t.vx1) ? D.y : 0.0f;
            const float D10 = (t.vy1 && t.vx0) ? D.z : 0.0f;
            const float D11 = (t.vy1 && t.vx1) ? D.w : 0.0f;
            // weights applied outside the differences, so each corner's rounding
            // error is scaled by that corner's own weight
            const float ux = t.ux, uy = t.uy;
            const float gm = uy * (ux * D00 + t.fx * D01) + t.fy * (ux * D10 + t.fx * D11);
            const float ddy = ux * (D10 - D00) + t.fx * (D11 - D01);
            const float ddx = uy * (D01 - D00) + t.fy * (D11 - D10);
            const float m = sm[k];
            const float sc = p.offset_scale * m;
            so[2 * k] = sc * ddx;
            so[2 * k + 1] = sc * ddy;
            sd[4 * k] = gm;
            dot = fmaf(m, gm, dot);
        }
    }
    if (p.softmax) dot = seg_total(dot, p.S, q);
    if (active) {
        for (int k = s; k < K; k += p.S) {
            const float gm = sd[4 * k];
            sm[k] = p.softmax ? sm[k] * (gm - dot) : gm;
        }
    }
    __syncthreads();
    if (p.want_off) block_copy(goff + (size_t)pair0 * K * 2, s_off, npb * K * 2, p.vec_io);
    if (p.want_mask) block_copy(gmask + (size_t)pair0 * K, s_m, npb * K, p.vec_io);
}

// Clear n floats (vectorised when dst is 16-byte aligned).
__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ dst, long long n, int vec) {
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long done = 0;
    if (vec) {
        const long long n4 = n >> 2;
        float4 *d4 = reinterpret_cast<float4 *>(dst);
        for (long long i = tid; i < n4; i += stride) d4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        done = n4 << 2;
    }
    for (long long i = done + tid; i < n; i += stride) dst[i] = 0.0f;
}

// Round the fp32 accumulator into the fp16/bf16 gradient, 8 elements per step
// where both ends allow it.
template <class E>
__global__ __launch_bounds__(256) void round_out_kernel(const float *__restrict__ src,
                                                        typename E::bits *__restrict__ dst,
                                                        long long n, int vec) {
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long stride = (long long)gridDim.x * blockDim.x;
    long long done = 0;
    if (vec) {
        const long long n8 = n >> 3;
        for (long long i = tid; i < n8; i += stride) {
            const float4 a = reinterpret_cast<const float4 *>(src)[2 * i];
            const float4 b = reinterpret_cast<const float4 *>(src)[2 * i + 1];
            const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            store_f32<E, 8>(dst + 8 * i, f);
        }
        done = n8 << 3;
    }
    for (long long i = done + tid; i < n; i += stride) dst[i] = from_f32(E{}, src[i]);
}

int elementwise_blocks(long long n) {
    const long long b = (n / 4 + 255) / 256;
    return (int)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

template <class E, int V>
hipError_t launch_v(const CoreBwdLaunch &a, const BwdParams &p, float *gacc, hipStream_t stream) {
    const int K = a.kh * a.kw;
    const size_t lds = (size_t)p.PB * K * 7 * sizeof(float);
    const dim3 grid(p.nblocks), block(kThreads);
    using B = typename E::bits;
    const B *x = static_cast<const B *>(a.x);
    const B *go = static_cast<const B *>(a.grad_out);
    if (a.kh == 3 && a.kw == 3)
        hipLaunchKernelGGL((dcn_core_bwd_kernel<E, V, 3, 3>), grid, block, lds, stream, x,
                           a.offset, a.mask, go, gacc, a.grad_offset, a.grad_mask, p);
    else
        hipLaunchKernelGGL((dcn_core_bwd_kernel<E, V, 0, 0>), grid, block, lds, stream, x,
                           a.offset, a.mask, go, gacc, a.grad_offset, a.grad_mask, p);
    return hipGetLastError();
}

template <class E>
hipError_t launch_e(const CoreBwdLaunch &a, hipStream_t stream) {
    constexpr int elt = (int)sizeof(typename E::bits);
    // Widest vector that divides C and that x and grad_out are aligned to.
    int V = 16 / elt;
    while (V > 1 && (a.C % V != 0 || ((uintptr_t)a.x % (V * elt)) != 0 ||
                     ((uintptr_t)a.grad_out % (V * elt)) != 0))
        V >>= 1;
    BwdParams p;
    p.N = a.N; p.H = a.H; p.W = a.W; p.G = a.G; p.C = a.C; p.kh = a.kh; p.kw = a.kw;
    p.sh = a.sh; p.sw = a.sw; p.ph = a.ph; p.pw = a.pw; p.dh = a.dh; p.dw = a.dw;
    p.Ho = a.Ho; p.Wo = a.Wo;
    p.offset_scale = a.offset_scale;
    p.softmax = a.softmax ? 1 : 0;
    p.has_mask = a.mask != nullptr;
    p.want_x = a.grad_x != nullptr;
    p.want_off = a.grad_offset != nullptr;
    p.want_mask = a.grad_mask != nullptr;
    auto a16 = [](const void *ptr) { return ptr == nullptr || (uintptr_t)ptr % 16 == 0; };
    p.vec_io = a16(a.offset) && a16(a.mask) && a16(a.grad_offset) && a16(a.grad_mask);
    p.npairs = a.N * a.Ho * a.Wo * a.G;
    p.nchunk = a.C / V;
    p.S = p.nchunk < 64 ? p.nchunk : 64;
    const int K = a.kh * a.kw;
    p.Q = 64 / p.S;
    // the block's LDS (7 floats per pair and tap) stays <= 64 KB
    const int qcap = 65536 / (4 * K * 7 * (int)sizeof(float));
    if (p.Q > qcap) p.Q = qcap > 0 ? qcap : 1;
    p.PB = 4 * p.Q;
    p.nblocks = (p.npairs + p.PB - 1) / p.PB;

    const long long nx = (long long)a.N * a.H * a.W * a.G * a.C;
    float *gacc = nullptr;
    if (a.grad_x) {
        gacc = (E::id == DCN_F32) ? static_cast<float *>(a.grad_x) : static_cast<float *>(a.workspace);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(elementwise_blocks(nx)), dim3(256), 0, stream,
                           gacc, nx, (int)((uintptr_t)gacc % 16 == 0));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipError_t err = hipErrorInvalidValue;
    switch (V) {
        case 8: if constexpr (elt == 2) err = launch_v<E, 8>(a, p, gacc, stream); break;
        case 4: err = launch_v<E, 4>(a, p, gacc, stream); break;
        case 2: err = launch_v<E, 2>(a, p, gacc, stream); break;
        default: err = launch_v<E, 1>(a, p, gacc, stream); break;
    }
    if (err != hipSuccess) return err;
    if constexpr (E::id != DCN_F32) {
        if (!a.grad_x) return err;
        using B = typename E::bits;
        B *dst = static_cast<B *>(a.grad_x);
        const int vec = ((uintptr_t)dst % 16 == 0) && ((uintptr_t)gacc % 16 == 0);
        hipLaunchKernelGGL((round_out_kernel<E>), dim3(elementwise_blocks(nx)), dim3(256), 0,
                           stream, gacc, dst, nx, vec);
        err = hipGetLastError();
    }
    return err;
}

}  // namespace

size_t core_bwd_workspace_bytes(long long x_elems, dcn_dtype dtype) {
    if (dtype == DCN_F32) return 0;
    return (size_t)((x_elems * 4 + 255) / 256 * 256);
}

hipError_t launch_dcn_core_bwd(const CoreBwdLaunch &a, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_e<EF32>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        case DCN_BF16: return launch_e<EBF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
