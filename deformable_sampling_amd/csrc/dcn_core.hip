// DCNv3/v4 core forward, channels-last, for gfx950.
//
// Operation ("DCNv4 in YOLOv11", lpnh.cn, sections 1.1 and 3.2; bilinear kernel and
// deformable sum from "Hands-on DCNv1 in PyTorch", agent.csdn.net, sections 1-2):
//   out[n,ho,wo,g*C+c] = sum_k m_k * bilinear(x[n,:,:,g*C+c], base_k + offset_scale*d_k)
// with m_k the raw mask (DCNv4) or its softmax over the K points (DCNv3).
//
// Mapping. The unit of work is a (pixel, group) pair: the pair index e = pixel*G + g
// runs over [0, N*Ho*Wo*G), and the offsets [.., G, K, 2] and masks [.., G, K] of
// consecutive pairs are consecutive in memory (other layouts and fp16/bf16 offsets
// and masks, such as DCNv4's packed per-group rows of K (dx, dy) pairs then K masks,
// are staged element by element and widened to fp32). A pair's C channels are covered by S
// lanes, each holding V channels (16 bytes when alignment allows), so a wavefront
// works on Q = 64/S pairs and every corner read of a tap is one contiguous vector
// per lane (the channel-fastest mapping of the DCNv3 kernel page, widened to 16 B).
// A 256-thread block takes PB = 4*Q consecutive pairs:
//   1. stages the block's offsets and masks (two contiguous ranges) into LDS with
//      coalesced 16-byte loads;
//   2. DCNv3 only: softmax over K per pair in LDS, the S lanes of a pair splitting
//      the K logits and combining max and sum with wavefront shuffles;
//   3. per lane: for each tap, corner positions from LDS, four 16-byte corner loads
//      (clamped inside the image, zero weight outside), fp32 FMAs with the mask
//      folded into the bilinear weights; one store per lane.
// Blocks are remapped so each XCD processes a contiguous range of pixels (its L2
// then holds the input rows those pixels sample).
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

struct CoreParams {
    int N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo;
    float offset_scale;
    int softmax, has_mask, vec_stage;
    int off_pix, off_grp, mask_pix, mask_grp, om_plain;  // offset/mask addressing
    int npairs;  // N*Ho*Wo*G (< 2^31, checked by the host)
    int S;       // lanes per pair
    int Q;       // pairs per wavefront
    int nchunk;  // C / V vector chunks per pair
    int PB;      // pairs per block (4*Q)
    int nblocks;
};

constexpr int kThreads = 256;

__device__ __forceinline__ void stage_range(float *dst, const float *src, int n, bool vec) {
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

// Reduction over the S lanes of this lane's segment [q*S, q*S + S).
template <bool MAX>
__device__ __forceinline__ float seg_reduce(float v, int S, int q) {
    if ((S & (S - 1)) == 0) {
        for (int o = 1; o < S; o <<= 1) {
            const float u = __shfl_xor(v, o, 64);
            v = MAX ? fmaxf(v, u) : v + u;
        }
        return v;
    }
    float r = MAX ? -INFINITY : 0.0f;
    for (int j = 0; j < S; ++j) {
        const float u = __shfl(v, q * S + j, 64);
        r = MAX ? fmaxf(r, u) : r + u;
    }
    return r;
}

// Offsets/masks of pairs [pair0, pair0 + npb) -> LDS as fp32, for any layout and
// element type (the plain fp32 layout takes stage_range instead): element r of pair
// e = pixel*G + g sits at base + pixel*pix + g*grp + r.
template <class OM>
__device__ __forceinline__ void stage_strided(float *dst, const typename OM::bits *src, int pair0,
                                              int npb, int per, int pix_stride, int grp_stride,
                                              int G) {
    for (int idx = threadIdx.x; idx < npb * per; idx += kThreads) {
        const int lq = idx / per, r = idx - lq * per;
        const int e = pair0 + lq;
        const int pixel = e / G, g = e - pixel * G;
        dst[idx] = to_f32(OM{}, src[(size_t)pixel * pix_stride + (size_t)g * grp_stride + r]);
    }
}

template <class E, class OM, int V, int KH, int KW>
__global__ __launch_bounds__(kThreads) void dcn_core_kernel(const typename E::bits *__restrict__ x,
                                                            const typename OM::bits *__restrict__ offset,
                                                            const typename OM::bits *__restrict__ mask,
                                                            typename E::bits *__restrict__ out,
                                                            CoreParams p) {
    extern __shared__ float smem[];
    const int kh = KH > 0 ? KH : p.kh;
    const int kw = KW > 0 ? KW : p.kw;
    const int K = kh * kw;
    float *s_off = smem;                // [PB][K][2]
    float *s_m = smem + p.PB * K * 2;   // [PB][K]

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int pair0 = blk * p.PB;
    const int npb = min(p.PB, p.npairs - pair0);

    // 1. offsets and masks of pairs [pair0, pair0 + npb) -> LDS
    if (p.om_plain) {  // fp32 [.., G, K, 2] and [.., G, K]: two contiguous ranges
        const float *of = reinterpret_cast<const float *>(offset);
        stage_range(s_off, of + (size_t)pair0 * K * 2, npb * K * 2, p.vec_stage);
    } else {
        stage_strided<OM>(s_off, offset, pair0, npb, 2 * K, p.off_pix, p.off_grp, p.G);
    }
    if (p.has_mask) {
        if (p.om_plain)
            stage_range(s_m, reinterpret_cast<const float *>(mask) + (size_t)pair0 * K, npb * K,
                        p.vec_stage);
        else
            stage_strided<OM>(s_m, mask, pair0, npb, K, p.mask_pix, p.mask_grp, p.G);
    } else {
        for (int i = threadIdx.x; i < npb * K; i += kThreads) s_m[i] = 1.0f;
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane / p.S, s = lane - q * p.S;
    const int lp = wave * p.Q + q;
    const bool active = (q < p.Q) && (lp < npb);

    // 2. DCNv3: softmax over the K points of each pair, in place in LDS.
    if (p.softmax) {
        float *ml = s_m + lp * K;
        float mx = -INFINITY;
        if (active)
            for (int k = s; k < K; k += p.S) mx = fmaxf(mx, ml[k]);
        mx = seg_reduce<true>(mx, p.S, q);
        float sum = 0.0f;
        if (active)
            for (int k = s; k < K; k += p.S) sum += expf(ml[k] - mx);
        sum = seg_reduce<false>(sum, p.S, q);
        if (active) {
            const float inv = 1.0f / sum;
            for (int k = s; k < K; k += p.S) ml[k] = expf(ml[k] - mx) * inv;
        }
        __syncthreads();
    }

    if (!active) return;

    // 3. gather and accumulate
    const int e = pair0 + lp;
    const int pix = e / p.G;
    const int g = e - pix * p.G;
    const int wo = pix % p.Wo;
    const int t2 = pix / p.Wo;
    const int ho = t2 % p.Ho;
    const int n = t2 / p.Ho;
    const int GC = p.G * p.C;
    const typename E::bits *img = x + (size_t)n * p.H * p.W * GC + g * p.C;
    const float *so = s_off + lp * K * 2;
    const float *sm = s_m + lp * K;
    const int by0 = ho * p.sh - p.ph, bx0 = wo * p.sw - p.pw;

    for (int ch = s; ch < p.nchunk; ch += p.S) {
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.0f;
        const typename E::bits *imgc = img + ch * V;
        auto tap = [&](int i, int j) {
            const int k = i * kw + j;
            const float2 d = *reinterpret_cast<const float2 *>(so + 2 * k);
            int y0, x0;
            float fy, fx;
            split_coord(by0 + i * p.dh, mul_rn(p.offset_scale, d.y), y0, fy);
            split_coord(bx0 + j * p.dw, mul_rn(p.offset_scale, d.x), x0, fx);
            const Tap t = make_tap(y0, x0, fy, fx, sm[k], p.H, p.W, GC);
            accumulate_tap<E, V>(imgc, t, acc);
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
        store_f32<E, V>(out + (size_t)pix * GC + g * p.C + ch * V, acc);
    }
}

template <class E, class OM, int V>
hipError_t launch_om(const CoreLaunch &a, CoreParams &p, hipStream_t stream) {
    const int K = a.kh * a.kw;
    const size_t lds = (size_t)p.PB * K * 3 * sizeof(float);
    const dim3 grid(p.nblocks), block(kThreads);
    using B = typename E::bits;
    using OB = typename OM::bits;
    const B *x = static_cast<const B *>(a.x);
    const OB *off = static_cast<const OB *>(a.offset);
    const OB *msk = static_cast<const OB *>(a.mask);
    B *out = static_cast<B *>(a.out);
    if (a.kh == 3 && a.kw == 3)
        hipLaunchKernelGGL((dcn_core_kernel<E, OM, V, 3, 3>), grid, block, lds, stream, x, off, msk,
                           out, p);
    else
        hipLaunchKernelGGL((dcn_core_kernel<E, OM, V, 0, 0>), grid, block, lds, stream, x, off, msk,
                           out, p);
    return hipGetLastError();
}

template <class E, int V>
hipError_t launch_v(const CoreLaunch &a, CoreParams &p, hipStream_t stream) {
    switch (a.om_dtype) {
        case DCN_F32: return launch_om<E, EF32, V>(a, p, stream);
        case DCN_F16: return launch_om<E, EF16, V>(a, p, stream);
        case DCN_BF16: return launch_om<E, EBF16, V>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

template <class E>
hipError_t launch_e(const CoreLaunch &a, hipStream_t stream) {
    constexpr int elt = (int)sizeof(typename E::bits);
    // Widest vector (16, 8, 4 or 2 bytes) that divides the group's channels and
    // that both x and out are aligned to.
    int V = 16 / elt;
    while (V > 1 && (a.C % V != 0 || ((uintptr_t)a.x % (V * elt)) != 0 ||
                     ((uintptr_t)a.out % (V * elt)) != 0))
        V >>= 1;
    CoreParams p;
    p.N = a.N; p.H = a.H; p.W = a.W; p.G = a.G; p.C = a.C; p.kh = a.kh; p.kw = a.kw;
    p.sh = a.sh; p.sw = a.sw; p.ph = a.ph; p.pw = a.pw; p.dh = a.dh; p.dw = a.dw;
    p.Ho = a.Ho; p.Wo = a.Wo;
    p.offset_scale = a.offset_scale;
    p.softmax = a.softmax ? 1 : 0;
    p.has_mask = a.mask != nullptr;
    p.vec_stage = ((uintptr_t)a.offset % 16 == 0) && (a.mask == nullptr || (uintptr_t)a.mask % 16 == 0);
    p.off_pix = a.off_pix; p.off_grp = a.off_grp; p.mask_pix = a.mask_pix; p.mask_grp = a.mask_grp;
    p.om_plain = a.om_plain ? 1 : 0;
    p.npairs = a.N * a.Ho * a.Wo * a.G;
    p.nchunk = a.C / V;
    p.S = p.nchunk < 64 ? p.nchunk : 64;
    // pairs per wavefront; capped so the block's offset/mask tile stays <= 64 KB of LDS
    const int K = a.kh * a.kw;
    p.Q = 64 / p.S;
    const int qcap = 65536 / (4 * K * 3 * (int)sizeof(float));
    if (p.Q > qcap) p.Q = qcap > 0 ? qcap : 1;
    p.PB = 4 * p.Q;
    p.nblocks = (p.npairs + p.PB - 1) / p.PB;
    switch (V) {
        case 8: if constexpr (elt == 2) return launch_v<E, 8>(a, p, stream); break;
        case 4: return launch_v<E, 4>(a, p, stream);
        case 2: return launch_v<E, 2>(a, p, stream);
        default: return launch_v<E, 1>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dcn_core(const CoreLaunch &a, hipStream_t stream) {
    CoreTilePlan tp;
    if (plan_core_tile(a, tp)) return launch_dcn_core_tile(a, tp, stream);
    switch (a.dtype) {
        case DCN_F32: return launch_e<EF32>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        case DCN_BF16: return launch_e<EBF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
