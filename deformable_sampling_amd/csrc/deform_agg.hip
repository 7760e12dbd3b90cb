// Multi-camera, multi-scale deformable aggregation (Sparse4D) for gfx950.
//
// Operation ("Sparse4D deformable_aggregation", mlqm.cn, sections 2.1-2.2 and 7;
// bilinear kernel from "Hands-on DCNv1 in PyTorch", agent.csdn.net, section 2):
//   out[b,a,g*Cg+c] = sum_{p,cam,s} w[b,a,p,cam,s,g] * bilinear(map_{cam,s}, y, x),
//   x = fl32(u*W_s) - 0.5, y = fl32(v*H_s) - 0.5,
// with the weights optionally softmax-normalised over all (p, cam, s) of (b, a, g).
//
// Mapping. One wavefront per (anchor, group) unit. S = Cg/V lanes hold the group's
// channels (V per lane, 16 bytes for fp32), and the Z = 64/S lane slices split the
// unit's (point, camera) pairs, each slice running all scales of its pairs; the Z
// partial sums are combined with shuffles at the end. The sampling location is
// shared by all groups, the weight is per group. Units are ordered group-major, and
// blocks are remapped so that each XCD processes a contiguous range of units: with 8
// groups each XCD then serves one group, and its L2 only has to hold that group's
// 1/8 slice of every feature map.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

struct AggParams {
    int B, P_total, A, pts, cams, scales, G, Cg, softmax;
    int S, Z, nchunk;  // lanes per slice, slices per wave, V-chunks per group
    int BA;            // B*A
    int nunits;        // B*A*G
    int group_major;
    int nblocks;
    AggMaps maps;
};

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <class E, int V>
__global__ __launch_bounds__(kThreads) void deform_agg_kernel(const typename E::bits *__restrict__ feat,
                                                              const float *__restrict__ loc,
                                                              const float *__restrict__ weights,
                                                              typename E::bits *__restrict__ out,
                                                              const AggParams p) {
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int unit = blk * kWaves + (int)(threadIdx.x >> 6);
    if (unit >= p.nunits) return;  // whole wavefronts leave together
    const int lane = threadIdx.x & 63;
    const int z = lane / p.S, s = lane - z * p.S;

    int ba, g;
    if (p.group_major) {
        g = unit / p.BA;
        ba = unit - g * p.BA;
    } else {
        ba = unit / p.G;
        g = unit - ba * p.G;
    }
    const int b = ba / p.A;
    const int T = p.pts * p.cams * p.scales;
    const float *wrow = weights + (size_t)ba * T * p.G + g;  // tap t at wrow[t*G]

    float mx = 0.0f, inv = 1.0f;
    if (p.softmax) {  // softmax over the unit's T taps: all 64 lanes split the logits
        float m = -INFINITY;
        for (int t = lane; t < T; t += 64) m = fmaxf(m, wrow[(size_t)t * p.G]);
        mx = wave_max(m);
        float sum = 0.0f;
        for (int t = lane; t < T; t += 64) sum += expf(wrow[(size_t)t * p.G] - mx);
        inv = 1.0f / wave_sum(sum);
    }

    const int GC = p.G * p.Cg;
    const typename E::bits *fb = feat + (size_t)b * p.P_total * GC + g * p.Cg;
    const float *lrow = loc + (size_t)ba * p.pts * p.cams * 2;
    const int npc = p.pts * p.cams;
    const bool lane_on = z < p.Z;

    for (int ch0 = 0; ch0 < p.nchunk; ch0 += p.S) {
        const int ch = ch0 + s;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.0f;
        if (lane_on && ch < p.nchunk) {
            const typename E::bits *fc = fb + ch * V;
            for (int pc = z; pc < npc; pc += p.Z) {  // (point, camera) pairs of this slice
                const float2 uv = *reinterpret_cast<const float2 *>(lrow + 2 * pc);
                const int cam = pc % p.cams;
                float pacc[V];
#pragma unroll
                for (int i = 0; i < V; ++i) pacc[i] = 0.0f;
                for (int sc = 0; sc < p.scales; ++sc) {
                    const int cs = cam * p.scales + sc;
                    const int Hs = p.maps.H[cs], Ws = p.maps.W[cs];
                    float w = wrow[(size_t)(pc * p.scales + sc) * p.G];
                    if (p.softmax) w = expf(w - mx) * inv;
                    // one fp32 rounding of u*W, then the half-pixel shift
                    const float xf = __fsub_rn(__fmul_rn(uv.x, (float)Ws), 0.5f);
                    const float yf = __fsub_rn(__fmul_rn(uv.y, (float)Hs), 0.5f);
                    int x0, y0;
                    float fx, fy;
                    split_coord(0, xf, x0, fx);
                    split_coord(0, yf, y0, fy);
                    const Tap t = make_tap(y0, x0, fy, fx, w, Hs, Ws, GC);
                    accumulate_tap<E, V>(fc + (size_t)p.maps.start[cs] * GC, t, pacc);
                }
#pragma unroll
                for (int i = 0; i < V; ++i) acc[i] += pacc[i];
            }
        }
        // combine the Z slices (lanes s, s+S, s+2S, ...)
        if ((p.S & (p.S - 1)) == 0) {
            for (int o = p.S; o < 64; o <<= 1)
#pragma unroll
                for (int i = 0; i < V; ++i) acc[i] += __shfl_xor(acc[i], o, 64);
        } else {
            float tot[V];
#pragma unroll
            for (int i = 0; i < V; ++i) tot[i] = 0.0f;
            for (int zz = 0; zz < p.Z; ++zz)
#pragma unroll
                for (int i = 0; i < V; ++i) tot[i] += __shfl(acc[i], zz * p.S + s, 64);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = tot[i];
        }
        if (z == 0 && ch < p.nchunk)
            store_f32<E, V>(out + (size_t)ba * GC + g * p.Cg + ch * V, acc);
    }
}

template <class E, int V>
hipError_t launch_v(const AggLaunch &a, AggParams &p, hipStream_t stream) {
    using Bt = typename E::bits;
    hipLaunchKernelGGL((deform_agg_kernel<E, V>), dim3(p.nblocks), dim3(kThreads), 0, stream,
                       static_cast<const Bt *>(a.feat), a.loc, a.weights, static_cast<Bt *>(a.out),
                       p);
    return hipGetLastError();
}

template <class E>
hipError_t launch_e(const AggLaunch &a, hipStream_t stream) {
    constexpr int elt = (int)sizeof(typename E::bits);
    int V = 16 / elt;
    while (V > 1 && (a.Cg % V != 0 || ((uintptr_t)a.feat % (V * elt)) != 0 ||
                     ((uintptr_t)a.out % (V * elt)) != 0))
        V >>= 1;
    AggParams p;
    p.B = a.B; p.P_total = a.P_total; p.A = a.A; p.pts = a.pts; p.cams = a.cams;
    p.scales = a.scales; p.G = a.G; p.Cg = a.Cg; p.softmax = a.softmax ? 1 : 0;
    p.nchunk = a.Cg / V;
    p.S = p.nchunk < 64 ? p.nchunk : 64;
    p.Z = 64 / p.S;
    p.BA = a.B * a.A;
    p.nunits = p.BA * a.G;
    p.group_major = 1;
    p.nblocks = (p.nunits + kWaves - 1) / kWaves;
    p.maps = a.maps;
    switch (V) {
        case 8: if constexpr (elt == 2) return launch_v<E, 8>(a, p, stream); break;
        case 4: return launch_v<E, 4>(a, p, stream);
        case 2: return launch_v<E, 2>(a, p, stream);
        default: return launch_v<E, 1>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_deform_agg(const AggLaunch &a, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_e<EF32>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        case DCN_BF16: return launch_e<EBF16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
