// Deformable RoI pooling, channels-last, for gfx950.
//
// Operation ("Hands-on DCNv1 in PyTorch", agent.csdn.net, section 3: per-bin offsets
// normalised by the RoI size, dp_ij = gamma * dp^_ij o (w, h), bilinear sampling,
// pooling; bilinear kernel from section 2). For RoI r = (batch, x1, y1, x2, y2)
// scaled by spatial_scale, w = (x2 - x1)*scale, h = (y2 - y1)*scale, bin (i, j) of
// the k x k grid averages S x S bilinear samples at
//   (y1s + (i + (sy + 1/2)/S) h/k + gamma*dy_ij*h,  x1s + (j + (sx + 1/2)/S) w/k + gamma*dx_ij*w)
// in pixel-index coordinates, zero outside the image per corner.
//
// Mapping: a bin's C channels are spread over L lanes of V channels (16-byte vectors
// where alignment allows); a wavefront takes Z = 64/L bins. Every lane forms the
// sample positions itself and gathers the four corner vectors of each sample; the
// average is stored once.
//
// Sample positions are a fixed sequence of fp32 operations, each rounded once to
// nearest even and never fused with a neighbour (explicit mul_rn, correctly rounded
// division, additions in the order written):
//   x1s = fl(x1*s), w = fl(fl(x2 - x1)*s), bw = fl(w/k), dx = fl(fl(gamma*dx^)*w),
//   tx = fl((2(j*S + sx) + 1) / (2S)), px = fl(fl(x1s + fl(tx*bw)) + dx),
// and likewise for y; the corner/fraction split of px is exact. Two implementations
// that follow this sequence sample at bit-identical positions.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

constexpr int kThreads = 256;

struct RoiParams {
    int N, H, W, C, R, k, S;
    float scale, gamma;
    int L, Z, nchunk;  // lanes per bin, bins per wavefront, V-chunks per bin
    int nbins, nblocks;
    int has_offset;
};

template <class E, int V>
__global__ __launch_bounds__(kThreads) void roi_pool_kernel(const typename E::bits *__restrict__ x,
                                                            const float *__restrict__ rois,
                                                            const float *__restrict__ offset,
                                                            typename E::bits *__restrict__ out,
                                                            RoiParams p) {
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int wave = blk * (kThreads / 64) + (int)(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int z = lane / p.L, l = lane - z * p.L;
    const int bin = wave * p.Z + z;
    if (z >= p.Z || bin >= p.nbins) return;  // no barrier in this kernel
    const int kk = p.k * p.k;
    const int r = bin / kk, ij = bin - r * kk;
    const int i = ij / p.k, j = ij - i * p.k;
    const float *ro = rois + (size_t)r * 5;
    const int n = (int)ro[0];
    const int C = p.C;
    typename E::bits *o = out + (size_t)bin * C;
    if (n < 0 || n >= p.N) {  // a RoI naming no image of the batch pools to zero
        for (int ch = l; ch < p.nchunk; ch += p.L) {
            float z0[V];
#pragma unroll
            for (int u = 0; u < V; ++u) z0[u] = 0.0f;
            store_f32<E, V>(o + ch * V, z0);
        }
        return;
    }
    const float rx1 = ro[1], ry1 = ro[2], rx2 = ro[3], ry2 = ro[4];
    const float x1 = mul_rn(rx1, p.scale), y1 = mul_rn(ry1, p.scale);
    const float w = mul_rn(rx2 - rx1, p.scale), h = mul_rn(ry2 - ry1, p.scale);
    const float bw = __fdiv_rn(w, (float)p.k), bh = __fdiv_rn(h, (float)p.k);
    float dx = 0.0f, dy = 0.0f;
    if (p.has_offset) {
        const float2 d = reinterpret_cast<const float2 *>(offset)[bin];
        dx = mul_rn(mul_rn(p.gamma, d.x), w);
        dy = mul_rn(mul_rn(p.gamma, d.y), h);
    }
    const typename E::bits *img = x + (size_t)n * p.H * p.W * C;
    const float den = (float)(2 * p.S);
    const float inv_n = 1.0f / (float)(p.S * p.S);
    for (int ch = l; ch < p.nchunk; ch += p.L) {
        float acc[V];
#pragma unroll
        for (int u = 0; u < V; ++u) acc[u] = 0.0f;
        const typename E::bits *imgc = img + ch * V;
        for (int sy = 0; sy < p.S; ++sy) {
            const float ty = __fdiv_rn((float)(2 * (i * p.S + sy) + 1), den);
            const float yy = (y1 + mul_rn(ty, bh)) + dy;
            for (int sx = 0; sx < p.S; ++sx) {
                const float tx = __fdiv_rn((float)(2 * (j * p.S + sx) + 1), den);
                const float xx = (x1 + mul_rn(tx, bw)) + dx;
                int y0, x0;
                float fy, fx;
                split_coord(0, yy, y0, fy);
                split_coord(0, xx, x0, fx);
                const Tap t = make_tap(y0, x0, fy, fx, 1.0f, p.H, p.W, C);
                accumulate_tap<E, V>(imgc, t, acc);
            }
        }
#pragma unroll
        for (int u = 0; u < V; ++u) acc[u] *= inv_n;
        store_f32<E, V>(o + ch * V, acc);
    }
}

template <class E>
hipError_t launch_e(const RoiLaunch &a, hipStream_t stream) {
    constexpr int elt = (int)sizeof(typename E::bits);
    int V = 16 / elt;
    while (V > 1 && (a.C % V != 0 || ((uintptr_t)a.x % (V * elt)) != 0 ||
                     ((uintptr_t)a.out % (V * elt)) != 0))
        V >>= 1;
    RoiParams p;
    p.N = a.N; p.H = a.H; p.W = a.W; p.C = a.C; p.R = a.R; p.k = a.k; p.S = a.S;
    p.scale = a.spatial_scale; p.gamma = a.gamma;
    p.nchunk = a.C / V;
    p.L = p.nchunk < 64 ? p.nchunk : 64;
    p.Z = 64 / p.L;
    p.nbins = a.R * a.k * a.k;
    const int waves = (p.nbins + p.Z - 1) / p.Z;
    p.nblocks = (waves + 3) / 4;
    p.has_offset = a.offset != nullptr;
    using B = typename E::bits;
    const B *x = static_cast<const B *>(a.x);
    B *out = static_cast<B *>(a.out);
    const dim3 grid(p.nblocks), block(kThreads);
    switch (V) {
        case 8:
            if constexpr (elt == 2)
                hipLaunchKernelGGL((roi_pool_kernel<E, 8>), grid, block, 0, stream, x, a.rois, a.offset, out, p);
            break;
        case 4: hipLaunchKernelGGL((roi_pool_kernel<E, 4>), grid, block, 0, stream, x, a.rois, a.offset, out, p); break;
        case 2: hipLaunchKernelGGL((roi_pool_kernel<E, 2>), grid, block, 0, stream, x, a.rois, a.offset, out, p); break;
        default: hipLaunchKernelGGL((roi_pool_kernel<E, 1>), grid, block, 0, stream, x, a.rois, a.offset, out, p); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_deform_roi_pool(const RoiLaunch &a, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_e<EF32>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        case DCN_BF16: return launch_e<EBF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
