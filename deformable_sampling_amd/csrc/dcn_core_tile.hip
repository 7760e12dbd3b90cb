// DCNv3/v4 core forward, LDS halo-tile variant (gfx950).
//
// Same operation as dcn_core.hip ("DCNv4 in YOLOv11", lpnh.cn, sections 1.1 and 3.2;
// bilinear kernel of "Hands-on DCNv1 in PyTorch", agent.csdn.net, section 2).
//
// Why: with channels-last x, one group's channel vector at one pixel is 32-64 bytes,
// a fraction of a 128-byte cache line whose other bytes belong to groups that sample
// elsewhere. Gathering corners straight from global memory moves a whole line from
// L2 for nearly every corner, so L2->L1 traffic, not HBM, bounds that kernel. Here
// each block owns an output tile (TH x TW pixels) of GB groups whose channels form
// one contiguous slice of SB bytes per pixel, and first copies the input region
// those pixels reach with offsets up to +-halo pixels into LDS (zeros outside the
// image). Corners are then read from LDS; only taps that leave the region (and
// still touch the image) read global memory.
//
// Per block:
//   1. each lane loads its (pixel, group)'s K offsets and K masks into registers;
//   2. the block stages the input region [RH x RW pixels x SB bytes] into LDS;
//   3. DCNv3: softmax over K per pair; the S lanes of a pair split the exponentials
//      and exchange sum and values with wavefront shuffles;
//   4. per tap: fraction/corner split once per lane, 4*NC 16-byte LDS reads (or the
//      global fallback), fp32 FMAs with the mask folded into the weights.
// A lane holds NC 16-byte chunks (32 bytes when the group's channels allow), so the
// position and weight arithmetic of a tap is shared by as many channels as possible.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

using TileParams = CoreTilePlan;

template <class E, int V>
__device__ __forceinline__ void unpack(const uint4 &r, float (&f)[V]) {
    using B = typename E::bits;
    B b[V];
    __builtin_memcpy(b, &r, 16);
#pragma unroll
    for (int i = 0; i < V; ++i) f[i] = to_f32(E{}, b[i]);
}

constexpr int kStageBatch = 8;  // 16-byte staging loads kept in flight per thread

template <class E, int KH, int KW, int S, int NC>
__global__ __launch_bounds__(1024) void dcn_core_tile_kernel(const typename E::bits *__restrict__ x,
                                                             const float *__restrict__ offset,
                                                             const float *__restrict__ mask,
                                                             typename E::bits *__restrict__ out,
                                                             const TileParams p) {
    using Bt = typename E::bits;
    constexpr int V = 16 / (int)sizeof(Bt);
    constexpr int K = KH * KW;
    extern __shared__ uint4 lds[];  // [RH][RW][cpp]

    // block -> (image, tile row, tile column, group block), group block fastest: the
    // group blocks of one tile share every input cache line, so they run on the same
    // XCD (contiguous logical ranges per XCD) and the line is fetched into one L2.
    int t = xcd_remap((int)blockIdx.x, p.nblocks);
    const int gb = t % p.gblocks;
    t /= p.gblocks;
    const int tx = t % p.tiles_x;
    t /= p.tiles_x;
    const int ty = t % p.tiles_y;
    const int n = t / p.tiles_y;
    const int ho0 = ty * p.TH, wo0 = tx * p.TW, g0 = gb * p.GB;
    const int ry0 = ho0 * p.sh - p.ph - p.halo;
    const int rx0 = wo0 * p.sw - p.pw - p.halo;

    // thread -> (pixel in tile, group in block, lane s of the pair)
    const int tid = threadIdx.x;
    const int lp = tid % p.lpp;  // lane within the pixel = gl*S + s
    const int s = lp % S;
    const int gl = lp / S;
    const int q = tid / p.lpp;
    const int qy = q / p.TW, qx = q - qy * p.TW;
    const int ho = ho0 + qy, wo = wo0 + qx;
    const bool active = q < p.TH * p.TW && ho < p.Ho && wo < p.Wo;
    const int g = g0 + gl;
    const int GC = p.G * p.C;
    const Bt *ximg = x + (size_t)n * p.H * p.W * GC;

    // 1. this pair's offsets and masks -> registers (in flight during staging)
    float d[2 * K], m[K];
    {
        const size_t pr = active ? (((size_t)n * p.Ho + ho) * p.Wo + wo) * p.G + g : 0;
        const float2 *o2 = reinterpret_cast<const float2 *>(offset + pr * K * 2);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float2 v = o2[k];
            d[2 * k] = v.x;
            d[2 * k + 1] = v.y;
        }
        if (p.has_mask) {
            const float *mm = mask + pr * K;
#pragma unroll
            for (int k = 0; k < K; ++k) m[k] = mm[k];
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) m[k] = 1.0f;
        }
    }

    // 2. stage the input region: chunk i -> region pixel i >> log2(cpp), chunk i & (cpp-1)
    {
        const Bt *img = ximg + (size_t)g0 * p.C;
        const int total = p.RH * p.RW * p.cpp;
        const int nt = blockDim.x;
        for (int i0 = tid; i0 < total; i0 += kStageBatch * nt) {
            uint4 v[kStageBatch];
#pragma unroll
            for (int u = 0; u < kStageBatch; ++u) {
                const int i = i0 + u * nt;
                v[u] = make_uint4(0, 0, 0, 0);
                const int r = i >> p.cpp_log2;
                const int c = i & (p.cpp - 1);
                const int ry = __float2int_rz(((float)r + 0.5f) * p.inv_rw);  // exact r / RW
                const int yy = ry0 + ry, xx = rx0 + (r - ry * p.RW);
                if (i < total && (unsigned)yy < (unsigned)p.H && (unsigned)xx < (unsigned)p.W)
                    v[u] = *reinterpret_cast<const uint4 *>(
                        img + __umul24(__umul24(yy, p.W) + xx, GC) + c * V);
            }
#pragma unroll
            for (int u = 0; u < kStageBatch; ++u) {
                const int i = i0 + u * nt;
                if (i < total) lds[i] = v[u];
            }
        }
    }
    __syncthreads();

    // 3. DCNv3 softmax over the K points: lane s of the pair's S lanes takes the
    //    exponentials of k = s, s+S, ...; the sum and the values are exchanged with
    //    wavefront shuffles inside the pair's aligned S-lane segment.
    if (p.softmax) {
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < K; ++k) mx = fmaxf(mx, m[k]);
        constexpr int J = (K + S - 1) / S;
        float e[J];
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int k = j * S + s;
            float mk = m[0];
#pragma unroll
            for (int kk = 1; kk < K; ++kk) mk = (kk == k) ? m[kk] : mk;
            e[j] = k < K ? expf(mk - mx) : 0.0f;
            sum += e[j];
        }
#pragma unroll
        for (int o = 1; o < S; o <<= 1) sum += __shfl_xor(sum, o, 64);
        const float inv = 1.0f / sum;
        const int seg = (threadIdx.x & 63) - s;  // first lane of this pair's segment
#pragma unroll
        for (int k = 0; k < K; ++k) m[k] = __shfl(e[k / S], seg + k % S, 64) * inv;
    }
    if (!active) return;

    // 4. taps. Region coordinates of a tap are (ly, lx); taps whose 2x2 corners are
    //    not all inside the staged region get weight 0 here and are recorded in `far`
    //    for the global pass below (taps wholly outside the image read the region's
    //    zeros or are skipped there).
    float acc[NC][V];
#pragma unroll
    for (int u = 0; u < NC; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[u][i] = 0.0f;
    const int rowc = p.RW * p.cpp;
    // chunk order alternates with the pixel's parity so that lanes of neighbouring
    // pixels start on different LDS banks; acc[uu] accumulates chunk uu ^ flip and the
    // swap is undone once at the store
    const int slot0 = lp * NC;
    const int flip = (NC == 2) ? (q & 1) : 0;
    const int by0 = ho * p.sh - p.ph, bx0 = wo * p.sw - p.pw;
    unsigned far = 0;
#pragma unroll
    for (int i = 0; i < KH; ++i) {
#pragma unroll
        for (int j = 0; j < KW; ++j) {
            const int k = i * KW + j;
            int y0, x0;
            float fy, fx;
            split_coord(by0 + i * p.dh, __fmul_rn(p.offset_scale, d[2 * k + 1]), y0, fy);
            split_coord(bx0 + j * p.dw, __fmul_rn(p.offset_scale, d[2 * k]), x0, fx);
            const int ly = y0 - ry0, lx = x0 - rx0;
            const bool inreg = (unsigned)ly <= (unsigned)(p.RH - 2) && (unsigned)lx <= (unsigned)(p.RW - 2);
            far |= inreg ? 0u : (1u << k);
            const float mk = inreg ? m[k] : 0.0f;
            const int cell = (int)__umul24((unsigned)ly, (unsigned)rowc) + (lx << p.cpp_log2);
            const int base = (inreg ? cell : 0) + slot0;
            const float gy0 = (1.0f - fy) * mk, gy1 = fy * mk;
            const float w00 = gy0 * (1.0f - fx), w01 = gy0 * fx;
            const float w10 = gy1 * (1.0f - fx), w11 = gy1 * fx;
#pragma unroll
            for (int uu = 0; uu < NC; ++uu) {
                const int u = uu ^ flip;
                float a[V], b[V], c[V], e[V];
                unpack<E, V>(lds[base + u], a);
                unpack<E, V>(lds[base + p.cpp + u], b);
                unpack<E, V>(lds[base + rowc + u], c);
                unpack<E, V>(lds[base + rowc + p.cpp + u], e);
#pragma unroll
                for (int z = 0; z < V; ++z) {
                    acc[uu][z] = fmaf(w00, a[z], acc[uu][z]);
                    acc[uu][z] = fmaf(w01, b[z], acc[uu][z]);
                    acc[uu][z] = fmaf(w10, c[z], acc[uu][z]);
                    acc[uu][z] = fmaf(w11, e[z], acc[uu][z]);
                }
            }
        }
    }
    // global pass for taps that left the region (rare): corners read from x with the
    // per-corner image bounds; taps wholly outside the image contribute nothing
    if (far) {
        const Bt *imgc = ximg + (size_t)g * p.C + s * NC * V;
        while (far) {
            const int k = __builtin_ctz(far);
            far &= far - 1;
            float dx = d[0], dy = d[1], mk = m[0];
#pragma unroll
            for (int kk = 1; kk < K; ++kk) {
                dx = (kk == k) ? d[2 * kk] : dx;
                dy = (kk == k) ? d[2 * kk + 1] : dy;
                mk = (kk == k) ? m[kk] : mk;
            }
            const int i = k / KW, j = k - (k / KW) * KW;
            int y0, x0;
            float fy, fx;
            split_coord(by0 + i * p.dh, __fmul_rn(p.offset_scale, dy), y0, fy);
            split_coord(bx0 + j * p.dw, __fmul_rn(p.offset_scale, dx), x0, fx);
            if (y0 < -1 || y0 >= p.H || x0 < -1 || x0 >= p.W) continue;
            const Tap tp = make_tap(y0, x0, fy, fx, mk, p.H, p.W, GC);
#pragma unroll
            for (int uu = 0; uu < NC; ++uu) accumulate_tap<E, V>(imgc + (uu ^ flip) * V, tp, acc[uu]);
        }
    }
    if (NC == 2 && flip) {
#pragma unroll
        for (int z = 0; z < V; ++z) {
            const float tmp = acc[0][z];
            acc[0][z] = acc[NC - 1][z];
            acc[NC - 1][z] = tmp;
        }
    }
    Bt *o = out + (((size_t)n * p.Ho + ho) * p.Wo + wo) * GC + (size_t)g * p.C + s * NC * V;
#pragma unroll
    for (int u = 0; u < NC; ++u) store_f32<E, V>(o + u * V, acc[u]);
}

// Tile shape knobs: threads per block, tile width, LDS bytes per block (two blocks
// fit in the 160 KB of a CU at <= 80 KB), the largest halo tried and the target
// slice bytes per region pixel.
#ifndef DCN_TILE_THREADS
#define DCN_TILE_THREADS 512
#endif
#ifndef DCN_TILE_LDS_BYTES
#define DCN_TILE_LDS_BYTES (78 * 1024)
#endif
#ifndef DCN_TILE_MAX_HALO
#define DCN_TILE_MAX_HALO 12
#endif
#ifndef DCN_TILE_TW
#define DCN_TILE_TW 16
#endif
#ifndef DCN_TILE_SLICE
#define DCN_TILE_SLICE 64
#endif

template <class E, int S, int NC>
hipError_t launch_tile(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    using Bt = typename E::bits;
    auto kern = dcn_core_tile_kernel<E, 3, 3, S, NC>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
        DCN_TILE_LDS_BYTES);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(kern, dim3(p.nblocks), dim3(p.threads), p.lds_bytes, stream,
                       static_cast<const Bt *>(a.x), a.offset, a.mask, static_cast<Bt *>(a.out), p);
    return hipGetLastError();
}

template <class E, int NC>
hipError_t launch_tile_s(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    switch (p.S) {
        case 1: return launch_tile<E, 1, NC>(a, p, stream);
        case 2: return launch_tile<E, 2, NC>(a, p, stream);
        case 4: return launch_tile<E, 4, NC>(a, p, stream);
        case 8: return launch_tile<E, 8, NC>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

template <class E>
hipError_t launch_tile_e(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    if constexpr (E::id == DCN_BF16) {
        return launch_tile_s<E, 1>(a, p, stream);
    } else {
        return p.NC == 2 ? launch_tile_s<E, 2>(a, p, stream) : launch_tile_s<E, 1>(a, p, stream);
    }
}

int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

}  // namespace

// Choose a tile for the LDS path; false if this call should use the direct kernel
// (window other than 3x3, channel slice not a multiple of 16 bytes or over 256
// bytes, misaligned pointers, image too large for 24-bit offsets, or no useful halo
// fits in LDS).
bool plan_core_tile(const CoreLaunch &a, TileParams &p) {
    if (!(a.kh == 3 && a.kw == 3)) return false;
    const int elt = a.dtype == DCN_F32 ? 4 : 2;
    const int cbytes = a.C * elt;
    if (cbytes % 16 != 0 || cbytes > 256) return false;
    if ((uintptr_t)a.x % 16 || (uintptr_t)a.out % 16 || (uintptr_t)a.offset % 8) return false;
    if ((long long)a.H * a.W >= (1LL << 24) || (long long)a.G * a.C >= (1LL << 24)) return false;
    // 16-byte chunks per lane: two where the channels allow, except for bf16, whose
    // widening (no mixed-precision FMA) would need twice the registers
    const int NC = (cbytes % 32 == 0 && a.dtype != DCN_BF16) ? 2 : 1;
    const int S = cbytes / (16 * NC);         // lanes per (pixel, group): 1, 2, 4 or 8
    if (S & (S - 1)) return false;
    int GB = 1;  // groups per block: a power of two dividing G, slice <= DCN_TILE_SLICE
    while (a.G % (2 * GB) == 0 && 2 * GB * cbytes <= DCN_TILE_SLICE) GB *= 2;
    const int cpp = GB * cbytes / 16;  // chunks per region pixel (a power of two)
    const int lpp = GB * S;            // lanes per output pixel
    const int pix = DCN_TILE_THREADS / lpp;
    if (pix < 1) return false;
    int TW = DCN_TILE_TW < pix ? DCN_TILE_TW : pix;
    if (TW > a.Wo) TW = a.Wo;
    int TH = pix / TW;
    if (TH > a.Ho) TH = a.Ho;
    if (TH < 1) return false;
    const size_t sb = (size_t)cpp * 16;
    int halo = -1;
    for (int h = DCN_TILE_MAX_HALO; h >= 1; --h) {
        const size_t rh = (size_t)(TH - 1) * a.sh + (size_t)(a.kh - 1) * a.dh + 2 + 2 * h;
        const size_t rw = (size_t)(TW - 1) * a.sw + (size_t)(a.kw - 1) * a.dw + 2 + 2 * h;
        if (rh * rw * sb <= DCN_TILE_LDS_BYTES) { halo = h; break; }
    }
    if (halo < 2) return false;
    p.N = a.N; p.H = a.H; p.W = a.W; p.G = a.G; p.C = a.C; p.kh = a.kh; p.kw = a.kw;
    p.sh = a.sh; p.sw = a.sw; p.ph = a.ph; p.pw = a.pw; p.dh = a.dh; p.dw = a.dw;
    p.Ho = a.Ho; p.Wo = a.Wo;
    p.offset_scale = a.offset_scale;
    p.softmax = a.softmax ? 1 : 0;
    p.has_mask = a.mask != nullptr;
    p.GB = GB; p.S = S; p.NC = NC; p.cpp = cpp; p.cpp_log2 = ilog2(cpp); p.lpp = lpp;
    p.TH = TH; p.TW = TW; p.halo = halo;
    p.RH = (TH - 1) * a.sh + (a.kh - 1) * a.dh + 2 + 2 * halo;
    p.RW = (TW - 1) * a.sw + (a.kw - 1) * a.dw + 2 + 2 * halo;
    p.inv_rw = 1.0f / (float)p.RW;
    p.tiles_x = (a.Wo + TW - 1) / TW;
    p.tiles_y = (a.Ho + TH - 1) / TH;
    p.gblocks = a.G / GB;
    const long long nb = (long long)p.gblocks * a.N * p.tiles_y * p.tiles_x;
    if (nb > 0x7fffffffLL) return false;
    p.nblocks = (int)nb;
    p.threads = TH * TW * lpp;
    p.lds_bytes = (size_t)p.RH * p.RW * sb;
    return true;
}

hipError_t launch_dcn_core_tile(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_tile_e<EF32>(a, p, stream);
        case DCN_F16: return launch_tile_e<EF16>(a, p, stream);
        case DCN_BF16: return launch_tile_e<EBF16>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
