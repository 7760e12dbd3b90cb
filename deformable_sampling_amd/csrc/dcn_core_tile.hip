// DCNv3/v4 core forward, LDS halo-tile kernels (gfx950).
//
// Same operation as dcn_core.hip ("DCNv4 in YOLOv11", lpnh.cn, sections 1.1 and 3.2;
// bilinear kernel of "Hands-on DCNv1 in PyTorch", agent.csdn.net, section 2).
//
// Why: with channels-last x, one group's channel vector at one pixel is 32-64 bytes,
// a fraction of a 128-byte cache line whose other bytes belong to groups that sample
// elsewhere. Gathering corners straight from global memory moves a whole line from
// L2 for nearly every corner, so L2->L1 traffic, not HBM, bounds that kernel. Here a
// tile is TH x TW output pixels of GB groups whose channels form one contiguous
// slice of SB bytes per pixel; the input region those pixels reach with offsets up
// to +-halo pixels is copied into LDS (zeros outside the image), corners are read
// from LDS, and only taps that leave the region (and still touch the image) read
// global memory, in a deferred pass.
//
// One tile per block: the region is staged with direct-to-LDS loads (16 bytes per
// lane, buffer- or global-address form); while they are in flight each lane turns its
// pair's offsets into tap cells and weights. Two 8-wave blocks share a CU, so one
// block's staging also overlaps the other's compute.
// Per tile: DCNv3 softmax over K per pair (the S lanes of a pair split the
// exponentials and exchange sum and values with wavefront shuffles); per tap the
// fraction/corner split once per lane, 4*NC 16-byte LDS reads, fp32 FMAs with the
// mask folded into the four bilinear weights; one store per 16-byte chunk.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {

// 16 zero bytes: the source of direct-to-LDS loads for region pixels outside the image.
__device__ __attribute__((aligned(16))) uint4 g_dcn_zero_chunk[1];

namespace {

using TileParams = CoreTilePlan;

#include "core_bwd_bins.hpp"

// Bin grid of the grad_x records in the terms the bin helpers use.
struct RecGrid {
    int H, W, G, TY, TX, sh, sw, ph, pw;
};
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Tile t -> (image, tile row, tile column, group block), group block fastest: the
// group blocks of one tile share every input cache line, so consecutive tiles (which
// run on one XCD) fetch each line into one L2.
struct TileAt {
    int n, ho0, wo0, g0, ry0, rx0;
};
__device__ __forceinline__ TileAt tile_at(int t, const TileParams &p) {
    TileAt a;
    const int gb = t % p.gblocks;
    t /= p.gblocks;
    const int tx = t % p.tiles_x;
    t /= p.tiles_x;
    const int ty = t % p.tiles_y;
    a.n = t / p.tiles_y;
    a.ho0 = ty * p.TH;
    a.wo0 = tx * p.TW;
    a.g0 = gb * p.GB;
    a.ry0 = a.ho0 * p.sh - p.ph - p.halo;
    a.rx0 = a.wo0 * p.sw - p.pw - p.halo;
    return a;
}

// This lane's (pixel, group) within a tile: lane lp of the pixel is gl*S + s.
// LPP_/TW_ != 0 give lanes per pixel and tile width at compile time (the 16x16,
// 512-thread plan has 2 and 16), so the lane's indices are shifts and masks.
struct LaneAt {
    int s, gl, q, ho, wo, g;
    unsigned pix, pr;  // output pixel (n*Ho + ho)*Wo + wo and pair pix*G + g; 0 if idle
    bool active;
};
template <int S, int LPP_ = 0, int TW_ = 0>
__device__ __forceinline__ LaneAt lane_at(const TileAt &a, const TileParams &p) {
    LaneAt l;
    const int tid = threadIdx.x;
    const int lpp = LPP_ ? LPP_ : p.lpp;
    const int tw = TW_ ? TW_ : p.TW;
    const int lp = tid % lpp;
    l.s = lp % S;
    l.gl = lp / S;
    l.q = tid / lpp;
    const int qy = l.q / tw, qx = l.q - qy * tw;
    l.ho = a.ho0 + qy;
    l.wo = a.wo0 + qx;
    l.active = l.q < p.TH * p.TW && l.ho < p.Ho && l.wo < p.Wo;
    l.g = a.g0 + l.gl;
    // 24-bit multiplies: the plan keeps N*Ho, Wo and Wo*G below 2^24 and the pair count
    // below 2^31
    const unsigned row = __umul24((unsigned)a.n, (unsigned)p.Ho) + (unsigned)l.ho;
    l.pix = l.active ? __umul24(row, (unsigned)p.Wo) + (unsigned)l.wo : 0u;
    l.pr = l.active ? __umul24(row, (unsigned)(p.Wo * p.G)) + __umul24((unsigned)l.wo, (unsigned)p.G) +
                          (unsigned)l.g
                    : 0u;
    return l;
}

// Corner/fraction split of base + t as split_coord does, with the fraction taken by
// v_fract_f32 (t - floor(t), held below 1) and the corner by v_cvt_flr_i32_f32 (one
// instruction for floor and convert, exact for the clamped |t| <= 2^24; the compiler
// emits a floor and a convert). The offsets reaching here are already scaled by
// offset_scale (see scale_offsets).
__device__ __forceinline__ void split_coord_fast(int base, float t, int &c0, float &f) {
    t = __builtin_amdgcn_fmed3f(t, -16777216.0f, 16777216.0f);
    f = __builtin_amdgcn_fractf(t);
    int fl;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(fl) : "v"(t));
    c0 = base + fl;
}

// fl32(offset_scale * d) for every offset, once per pair (skipped when the scale is 1,
// which leaves every value unchanged).
template <int K>
__device__ __forceinline__ void scale_offsets(float (&d)[2 * K], float scale) {
    if (scale != 1.0f) {
#pragma unroll
        for (int i = 0; i < 2 * K; ++i) d[i] = mul_rn(scale, d[i]);
    }
}

// Offset/mask element tags: the plain fp32 layout of dcn_core_forward ([.., G, K, 2]
// offsets, [.., G, K] masks) is a type of its own so that its addressing and 8-byte
// (dx, dy) loads are compiled in; EF32/EF16/EBF16 name DCNv4's packed rows (pixel and
// group strides from the parameters) of that element type.
struct OMPlain : EF32 {};
template <class OM> constexpr bool kOmPlain = false;
template <> constexpr bool kOmPlain<OMPlain> = true;

// The pair's K (dx, dy) offsets and K masks into registers as fp32 (pair 0 for idle
// lanes). The plain layout takes the tap's pair as one 8-byte load; packed rows, and
// fp16/bf16 values, are read element by element and widened exactly.
template <int K, class OM>
__device__ __forceinline__ void load_dm(float (&d)[2 * K], float (&m)[K], const TileAt &a,
                                        const LaneAt &l, const typename OM::bits *offset,
                                        const typename OM::bits *mask, const TileParams &p) {
    if constexpr (kOmPlain<OM>) {
        const size_t pr = l.pr;
        const float2 *o2 = reinterpret_cast<const float2 *>(offset + pr * K * 2);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float2 v = o2[k];
            d[2 * k] = v.x;
            d[2 * k + 1] = v.y;
        }
        if (p.has_mask) {
            const typename OM::bits *mm = mask + pr * K;
#pragma unroll
            for (int k = 0; k < K; ++k) m[k] = to_f32(OM{}, mm[k]);
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) m[k] = 1.0f;
        }
    } else {
        const size_t pixel = l.pix;
        const int g = l.active ? l.g : 0;
        const typename OM::bits *od = offset + pixel * p.off_pix + (size_t)g * p.off_grp;
#pragma unroll
        for (int i = 0; i < 2 * K; ++i) d[i] = to_f32(OM{}, od[i]);
        if (p.has_mask) {
            const typename OM::bits *mm = mask + pixel * p.mask_pix + (size_t)g * p.mask_grp;
#pragma unroll
            for (int k = 0; k < K; ++k) m[k] = to_f32(OM{}, mm[k]);
        } else {
#pragma unroll
            for (int k = 0; k < K; ++k) m[k] = 1.0f;
        }
    }
}

// DCNv3 softmax over the K points: lane s of the pair's S lanes takes the
// exponentials of k = s, s+S, ...; the sum and the values are exchanged with
// wavefront shuffles inside the pair's aligned S-lane segment. All lanes call it.
template <int K, int S>
__device__ __forceinline__ void softmax_k(float (&m)[K], int s) {
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
    if constexpr (S == 1) {
        const float inv = 1.0f / sum;
#pragma unroll
        for (int k = 0; k < K; ++k) m[k] = e[k] * inv;
    } else if constexpr (S == 2) {
        // the pair's two lanes are neighbours: a DPP swap (quad_perm 1,0,3,2) instead of
        // LDS permutes
        auto swap = [](float v) {
            return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, false));
        };
        sum += swap(sum);
        const float inv = 1.0f / sum;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const float o = swap(e[j]);  // the other lane's exponential of point 2j + (1 - s)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int k = 2 * j + t;
                if (k < K) m[k] = (t == s ? e[j] : o) * inv;
            }
        }
    } else {
#pragma unroll
        for (int o = 1; o < S; o <<= 1) sum += __shfl_xor(sum, o, 64);
        const float inv = 1.0f / sum;
        const int seg = (threadIdx.x & 63) - s;  // first lane of this pair's segment
#pragma unroll
        for (int k = 0; k < K; ++k) m[k] = __shfl(e[k / S], seg + k % S, 64) * inv;
    }
}

// The taps of one lane in two steps. make_taps turns the pair's offsets and masks into
// each tap's region cell and four weights; it needs no LDS, so it runs while the
// region is still being copied in. taps_run then reads the corners from the staged
// region `buf`, accumulates and stores. Taps whose 2x2 corners are not all inside the
// region get weight 0 in the LDS pass; those that still touch the image (bits of
// `far`) are redone from global memory in the deferred pass.
// CPP_ and RW_ fix the chunks per region pixel and the region width at compile time
// (0: taken from p): the four corners of a chunk are then one address plus constant
// offsets that the LDS reads encode as immediates.
struct TapW {
    int cell;  // region chunk index of the (y0, x0) corner, chunk 0 (0 for weight-0 taps)
    float w00, w01, w10, w11;
};

template <class E, int KH, int KW, int S, int NC, int CPP_ = 0, int RW_ = 0>
__device__ __forceinline__ void make_taps(TapW (&tw)[KH * KW], unsigned &far, float (&d)[2 * KH * KW],
                                          const float (&m)[KH * KW], const TileAt &a,
                                          const LaneAt &l, const TileParams &p) {
    constexpr int K = KH * KW;
    scale_offsets<K>(d, p.offset_scale);
    const int cpp = CPP_ ? CPP_ : p.cpp;
    const int rw = RW_ ? RW_ : p.RW;
    const int rowc = rw * cpp;
    const int lby = __mul24(l.ho, p.sh) - p.ph - a.ry0, lbx = __mul24(l.wo, p.sw) - p.pw - a.rx0;
    // grid base of the output pixel relative to the region origin; the image bounds
    // test adds the origin back (y0 + 1 = ly + ry0 + 1)
    const int ty = a.ry0 + 1, tx = a.rx0 + 1;
    far = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int i = k / KW, j = k - (k / KW) * KW;
        int ly, lx;
        float fy, fx;
        split_coord_fast(lby + i * p.dh, d[2 * k + 1], ly, fy);
        split_coord_fast(lbx + j * p.dw, d[2 * k], lx, fx);
        const bool inreg = (unsigned)ly <= (unsigned)(p.RH - 2) && (unsigned)lx <= (unsigned)(rw - 2);
        const bool touch = (unsigned)(ly + ty) <= (unsigned)p.H && (unsigned)(lx + tx) <= (unsigned)p.W;
        // some corner inside the image: y0 in [-1, H-1] and x0 in [-1, W-1]
        far |= (!inreg && touch) ? (1u << k) : 0u;
        const float mk = inreg ? m[k] : 0.0f;
        const int cell = (int)__umul24((unsigned)ly, (unsigned)rowc) + lx * cpp;
        TapW &t = tw[k];
        t.cell = inreg ? cell : 0;
        const float gy1 = fy * mk, gy0 = mk - gy1;
        t.w01 = gy0 * fx;
        t.w00 = gy0 - t.w01;
        t.w11 = gy1 * fx;
        t.w10 = gy1 - t.w11;
    }
}

// coff: this pair's 2K offsets in memory (re-read for taps of the deferred pass).
template <class E, class OM, int KH, int KW, int S, int NC, int CPP_ = 0, int RW_ = 0>
__device__ __forceinline__ void taps_run(const uint4 *buf, const typename E::bits *x,
                                         typename E::bits *out, const TapW (&tw)[KH * KW], unsigned far,
                                         const float (&m)[KH * KW], const TileAt &a,
                                         const LaneAt &l, const TileParams &p,
                                         const typename OM::bits *coff) {
    using Bt = typename E::bits;
    constexpr int V = 16 / (int)sizeof(Bt);
    constexpr int K = KH * KW;
    const int GC = p.G * p.C;
    float acc[NC][V];
#pragma unroll
    for (int u = 0; u < NC; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[u][i] = 0.0f;
    const int cpp = CPP_ ? CPP_ : p.cpp;
    const int rw = RW_ ? RW_ : p.RW;
    const int rowc = rw * cpp;
    const int lp = l.gl * S + l.s;
    // chunk order alternates with the pixel's parity so that lanes of neighbouring
    // pixels start on different LDS banks; acc[uu] accumulates chunk uu ^ flip and the
    // swap is undone at the store
    const int flip = (NC == 2) ? (l.q & 1) : 0;
    int slot[NC];
#pragma unroll
    for (int uu = 0; uu < NC; ++uu) slot[uu] = lp * NC + (uu ^ flip);
    // Units (tap k, chunk uu) in order; unit n + 1's four corner reads are written
    // before unit n's multiply-adds.
    constexpr int NU = K * NC;
    uint4 buf4[2][4];
    auto issue = [&](int n) __attribute__((always_inline)) {
        const int k = n / NC, uu = n % NC;
        const uint4 *q = buf + tw[k].cell + slot[uu];
        buf4[n & 1][0] = q[0];
        buf4[n & 1][1] = q[cpp];
        buf4[n & 1][2] = q[rowc];
        buf4[n & 1][3] = q[rowc + cpp];
    };
    auto accum = [&](int n) __attribute__((always_inline)) {
        const int k = n / NC, uu = n % NC;
        float va[V], vb[V], vc[V], ve[V];
        unpack<E, V>(buf4[n & 1][0], va);
        unpack<E, V>(buf4[n & 1][1], vb);
        unpack<E, V>(buf4[n & 1][2], vc);
        unpack<E, V>(buf4[n & 1][3], ve);
#pragma unroll
        for (int z = 0; z < V; ++z) {
            acc[uu][z] = fmaf(tw[k].w00, va[z], acc[uu][z]);
            acc[uu][z] = fmaf(tw[k].w01, vb[z], acc[uu][z]);
            acc[uu][z] = fmaf(tw[k].w10, vc[z], acc[uu][z]);
            acc[uu][z] = fmaf(tw[k].w11, ve[z], acc[uu][z]);
        }
    };
#pragma unroll
    for (int n = 0; n <= NU; ++n) {
        if (n < NU) issue(n);
        if (n >= 1) accum(n - 1);
    }
    const int by0 = l.ho * p.sh - p.ph, bx0 = l.wo * p.sw - p.pw;
    const Bt *ximg = x + (size_t)a.n * p.H * p.W * GC;
    if (far) {  // deferred global pass (rare)
        const Bt *imgc = ximg + (size_t)l.g * p.C + l.s * NC * V;
        while (far) {
            const int k = __builtin_ctz(far);
            far &= far - 1;
            // the tap's offsets again from memory (the pair's row, just read, is in
            // cache): no offset register stays live through the LDS pass
            float dx, dy;
            if constexpr (kOmPlain<OM>) {
                const float2 dv = reinterpret_cast<const float2 *>(coff)[k];
                dx = dv.x;
                dy = dv.y;
            } else {
                dx = to_f32(OM{}, coff[2 * k]);
                dy = to_f32(OM{}, coff[2 * k + 1]);
            }
            if (p.offset_scale != 1.0f) {
                dx = mul_rn(p.offset_scale, dx);
                dy = mul_rn(p.offset_scale, dy);
            }
            float mk = m[0];
#pragma unroll
            for (int kk = 1; kk < K; ++kk) mk = (kk == k) ? m[kk] : mk;
            const int i = k / KW, j = k - (k / KW) * KW;
            int y0, x0;
            float fy, fx;
            split_coord_fast(by0 + i * p.dh, dy, y0, fy);
            split_coord_fast(bx0 + j * p.dw, dx, x0, fx);
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
    Bt *o = out + (size_t)l.pr * p.C + l.s * NC * V;
#pragma unroll
    for (int u = 0; u < NC; ++u) store_f32<E, V>(o + u * V, acc[u]);
}

// Stage the tile's region with direct global->LDS copies: each wave moves 64
// consecutive 16-byte chunks per instruction (lane order = LDS order); chunks outside
// the image copy the zero chunk. Thread t always moves chunk t & (cpp-1) of region
// pixels r = t >> log2(cpp), r + dr, ... with the row/column advanced incrementally.
// The caller waits (barrier) before reading.
template <class E>
__device__ __forceinline__ void stage_region(uint4 *lds, const typename E::bits *__restrict__ x,
                                             const TileAt &a, const TileParams &p) {
    using Bt = typename E::bits;
    constexpr int V = 16 / (int)sizeof(Bt);
    const int tid = threadIdx.x;
    const int GC = p.G * p.C;
    const Bt *img = x + (size_t)a.n * p.H * p.W * GC + (size_t)a.g0 * p.C + (tid & (p.cpp - 1)) * V;
    const int total = p.RH * p.RW * p.cpp;
    const int nt = blockDim.x;
    const int dr = nt >> p.cpp_log2;
    const int ddy = dr / p.RW, ddx = dr - ddy * p.RW;
    int r = tid >> p.cpp_log2;
    int ry = r / p.RW, rx = r - ry * p.RW;
    for (int i0 = tid & ~63; i0 < total; i0 += nt) {
        const int yy = a.ry0 + ry, xx = a.rx0 + rx;
        const bool ok = i0 + (tid & 63) < total && (unsigned)yy < (unsigned)p.H && (unsigned)xx < (unsigned)p.W;
        const void *src = ok ? (const void *)(img + __umul24(__umul24(yy, p.W) + xx, GC))
                             : (const void *)g_dcn_zero_chunk;
        __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)(lds + i0), 16, 0, 0);
        rx += ddx;
        ry += ddy;
        if (rx >= p.RW) { rx -= p.RW; ++ry; }
    }
}

// stage_region for a region of RH x RW pixels and a block of NT threads known at
// compile time: an unrolled sequence of copies per wave (the last one only where
// chunks remain). The copies go through a buffer resource over the image: a chunk
// outside the image gets an offset past the resource's end, which reads as zeros.
// Unlike the global-address form, buffer-form copies let the compiler wait for the
// pair's offset/mask loads (issued before) without waiting for the copies, so the
// tap arithmetic runs while the region is in flight. The image must be < 2 GiB.
template <class E, int RW, int CPP, int RH, int NT>
__device__ __forceinline__ void stage_region_fixed(uint4 *lds, const typename E::bits *__restrict__ x,
                                                   const TileAt &a, const TileParams &p) {
    using Bt = typename E::bits;
    constexpr int V = 16 / (int)sizeof(Bt);
    constexpr int elt = (int)sizeof(Bt);
    constexpr int total = RH * RW * CPP;
    constexpr int NIT = (total + NT - 1) / NT;
    const int tid = threadIdx.x;
    const int GC = p.G * p.C;
    const unsigned img_bytes = (unsigned)(p.H * p.W * GC * elt);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(x + (size_t)a.n * p.H * p.W * GC, img_bytes);
    const int cb = ((a.g0 * p.C) + (tid & (CPP - 1)) * V) * elt;
    const int w0 = __builtin_amdgcn_readfirstlane(tid & ~63);
    const int lane = tid & 63;
    // region pixel of this lane's first copy, then advanced by NT / CPP pixels per copy
    static_assert(NT % CPP == 0, "whole pixels per step");
    constexpr int DY = (NT / CPP) / RW, DX = (NT / CPP) % RW;
    const int r0 = (w0 + lane) / CPP;
    int ry = r0 / RW, rx = r0 - ry * RW;
    const int GCe = GC * elt;
    // Byte offset of the lane's region pixel in the image, advanced by a constant per copy
    // (DY rows and DX columns, one more row and RW columns back on a wrap): no multiply
    // in the loop. Unsigned arithmetic wraps; offsets of pixels outside the image are
    // never used, and those inside are below img_bytes < 2^31.
    const unsigned rowb = (unsigned)(p.W * GCe);
    int yy = a.ry0 + ry, xx = a.rx0 + rx;
    unsigned off = (unsigned)yy * rowb + (unsigned)(xx * GCe + cb);
    const int xend = a.rx0 + RW;
    const unsigned step = (unsigned)DY * rowb + (unsigned)(DX * GCe);
    const unsigned wrap = rowb - (unsigned)(RW * GCe);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i0 = w0 + it * NT;
        if (it < NIT - 1 || i0 < total) {
            // only the last step can pass the region's end
            const bool in = it < NIT - 1 || i0 + lane < total;
            const bool ok = in && (unsigned)yy < (unsigned)p.H && (unsigned)xx < (unsigned)p.W;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds + i0), 16,
                                                     ok ? (int)off : (int)img_bytes, 0, 0, 0);
        }
        xx += DX;
        yy += DY;
        off += step;
        if (xx >= xend) {
            xx -= RW;
            ++yy;
            off += wrap;
        }
    }
}

// ---------------------------------------------------------- one tile/block --

template <class E, class OM, int KH, int KW, int S, int NC, int CPP_, int RW_, int RH_>
__global__ __launch_bounds__(1024) void dcn_core_tile_kernel(const typename E::bits *__restrict__ x,
                                                             const typename OM::bits *__restrict__ offset,
                                                             const typename OM::bits *__restrict__ mask,
                                                             typename E::bits *__restrict__ out,
                                                             const TileParams p) {
    constexpr int K = KH * KW;
    extern __shared__ uint4 lds[];  // [RH][RW][cpp]

    const TileAt a = tile_at(xcd_remap((int)blockIdx.x, p.nblocks), p);
    // the compiled-in staging plan (RH_ != 0) has 16-pixel rows of 2 lanes per pixel
    const LaneAt l = lane_at<S, RH_ ? 2 : 0, RH_ ? 16 : 0>(a, p);

    float d[2 * K], m[K];
    load_dm<K, OM>(d, m, a, l, offset, mask, p);

    if constexpr (RH_ != 0)
        stage_region_fixed<E, RW_, CPP_, RH_, 512>(lds, x, a, p);
    else
        stage_region<E>(lds, x, a, p);
    if (p.softmax) softmax_k<K, S>(m, l.s);
    TapW tw[K];
    unsigned far;
    make_taps<E, KH, KW, S, NC, CPP_, RW_>(tw, far, d, m, a, l, p);
    // the empty asm statements take the tap values as operands, so they are computed
    // here, before the barrier, instead of being sunk behind it into the active-lane
    // branch
#pragma unroll
    for (int k = 0; k < K; ++k)
        asm volatile("" ::"v"(tw[k].cell), "v"(tw[k].w00), "v"(tw[k].w01), "v"(tw[k].w10), "v"(tw[k].w11));
    asm volatile("" ::"v"(far));
    __syncthreads();
    if (!l.active) return;
    const typename OM::bits *coff = kOmPlain<OM> ? offset + (size_t)l.pr * K * 2
                                                 : offset + (size_t)l.pix * p.off_pix + (size_t)l.g * p.off_grp;
    taps_run<E, OM, KH, KW, S, NC, CPP_, RW_>(lds, x, out, tw, far, m, a, l, p, coff);
}

// ------------------------------------------------- backward: tap gradients --
//
// grad_offset and grad_mask of the core backward with the forward's tile structure
// (one lane per (pixel, group) pair: S = 1): the region is staged in LDS as in the
// forward, the lane holds the pair's grad_out channels, and per tap the four corner
// dots D_ab = sum_c grad_out_c X_ab,c come from LDS (corners outside the image are the
// staged zeros); taps leaving the region are redone from global memory afterwards.
// With exact complements u = (floor + 1) - t (split_coord_fu):
//   g_k = uy (ux D00 + fx D01) + fy (ux D10 + fx D11)
//   grad_offset_k = s m_k (uy (D01 - D00) + fy (D11 - D10), ux (D10 - D00) + fx (D11 - D01))
//   grad_mask_k = g_k, or m_k (g_k - sum_j m_j g_j) with the softmax.
template <class E, int NC>
__device__ __forceinline__ void dots4(const uint4 (&c)[NC][4], const float (&gv)[NC][16 / sizeof(typename E::bits)],
                                      float &d00, float &d01, float &d10, float &d11) {
    constexpr int V = 16 / (int)sizeof(typename E::bits);
#pragma unroll
    for (int uu = 0; uu < NC; ++uu) {
        float va[V], vb[V], vc[V], ve[V];
        unpack<E, V>(c[uu][0], va);
        unpack<E, V>(c[uu][1], vb);
        unpack<E, V>(c[uu][2], vc);
        unpack<E, V>(c[uu][3], ve);
#pragma unroll
        for (int z = 0; z < V; ++z) {
            d00 = fmaf(gv[uu][z], va[z], d00);
            d01 = fmaf(gv[uu][z], vb[z], d01);
            d10 = fmaf(gv[uu][z], vc[z], d10);
            d11 = fmaf(gv[uu][z], ve[z], d11);
        }
    }
}

template <class E, int NC, int CPP_, int RW_>
__global__ __launch_bounds__(1024) void dcn_core_bwd_tile_kernel(const typename E::bits *__restrict__ x,
                                                                 const float *__restrict__ offset,
                                                                 const float *__restrict__ mask,
                                                                 const typename E::bits *__restrict__ gout,
                                                                 float *__restrict__ goff,
                                                                 float *__restrict__ gmask,
                                                                 const TileParams p,
                                                                 const CoreRecArgs ra) {
    using Bt = typename E::bits;
    constexpr int V = 16 / (int)sizeof(Bt);
    constexpr int K = 9;
    extern __shared__ uint4 lds[];  // [RH][RW][cpp]

    const TileAt a = tile_at(xcd_remap((int)blockIdx.x, p.nblocks), p);
    const LaneAt l = lane_at<1>(a, p);
    const int GC = p.G * p.C;

    float d[2 * K], m[K];
    load_dm<K, OMPlain>(d, m, a, l, reinterpret_cast<const uint32_t *>(offset),
                        reinterpret_cast<const uint32_t *>(mask), p);
    stage_region<E>(lds, x, a, p);
    const size_t pixel = l.pix;
    float gv[NC][V];  // this pair's grad_out channels
    {
        const Bt *gp = gout + pixel * GC + (size_t)l.g * p.C;
#pragma unroll
        for (int uu = 0; uu < NC; ++uu) load_f32<E, V>(gp + uu * V, gv[uu]);
    }
    __syncthreads();
    if (p.softmax) softmax_k<K, 1>(m, 0);
    scale_offsets<K>(d, p.offset_scale);

    const int cpp = CPP_ ? CPP_ : p.cpp;
    const int rw = RW_ ? RW_ : p.RW;
    const int rowc = rw * cpp;
    const int lby = l.ho * p.sh - p.ph - a.ry0, lbx = l.wo * p.sw - p.pw - a.rx0;
    const int ty = a.ry0 + 1, tx = a.rx0 + 1;
    const size_t pair = pixel * p.G + l.g;
    unsigned far = 0;
    float dot = 0.0f;  // sum_k m_k g_k (softmax)
    // With the region geometry compiled in, a pair's 27 results wait in registers and
    // leave through LDS in coalesced runs; the generic variant (more address registers)
    // stores each tap's results directly.
    constexpr bool kStage = CPP_ != 0;
    float rg[K];   // g_k, then grad_mask_k (kStage)
    float2 ro[K];  // grad_offset_k (kStage)
    float2 *go = reinterpret_cast<float2 *>(goff) + pair * K;
    float *gmp = gmask ? gmask + pair * K : nullptr;
    // g_k and grad_offset_k of tap k (a compile-time index) from its corner dots
    auto grads = [&](int k, float mk, float uy, float fy, float ux, float fx, float d00, float d01,
                     float d10, float d11) __attribute__((always_inline)) {
        const float gk = uy * (ux * d00 + fx * d01) + fy * (ux * d10 + fx * d11);
        dot = fmaf(mk, gk, dot);
        const float sc = p.offset_scale * mk;
        const float2 o = make_float2(sc * (uy * (d01 - d00) + fy * (d11 - d10)),
                                     sc * (ux * (d10 - d00) + fx * (d11 - d01)));
        if constexpr (kStage) {
            rg[k] = gk;
            ro[k] = o;
        } else {
            if (gmp) gmp[k] = gk;
            if (goff) go[k] = o;
        }
    };
    if (l.active) {
        // units (tap k, chunk uu) in order, the next unit's four corner reads issued
        // before this unit's dots; a tap's dots are complete after its last chunk
        struct TapG {
            float fy, uy, fx, ux;
            bool inreg;
        };
        constexpr int NU = K * NC;
        TapG tg[2];
        int cellk[2];
        uint4 cb[2][4];
        auto issue = [&](int n) __attribute__((always_inline)) {
            const int k = n / NC, uu = n % NC;
            TapG &t = tg[k & 1];
            if (uu == 0) {
                const int i = k / 3, j = k - (k / 3) * 3;
                int ly, lx;
                split_coord_fu(lby + i * p.dh, d[2 * k + 1], ly, t.fy, t.uy);
                split_coord_fu(lbx + j * p.dw, d[2 * k], lx, t.fx, t.ux);
                t.inreg = (unsigned)ly <= (unsigned)(p.RH - 2) && (unsigned)lx <= (unsigned)(rw - 2);
                const bool touch = (unsigned)(ly + ty) <= (unsigned)p.H && (unsigned)(lx + tx) <= (unsigned)p.W;
                far |= (!t.inreg && touch) ? (1u << k) : 0u;
                cellk[k & 1] = t.inreg ? (int)__umul24((unsigned)ly, (unsigned)rowc) + lx * cpp : 0;
            }
            const uint4 *q = lds + cellk[k & 1] + l.gl * NC + uu;
            cb[n & 1][0] = q[0];
            cb[n & 1][1] = q[cpp];
            cb[n & 1][2] = q[rowc];
            cb[n & 1][3] = q[rowc + cpp];
        };
        float d00 = 0.0f, d01 = 0.0f, d10 = 0.0f, d11 = 0.0f;
        auto accum = [&](int n) __attribute__((always_inline)) {
            const int k = n / NC, uu = n % NC;
            float va[V], vb[V], vc[V], ve[V];
            unpack<E, V>(cb[n & 1][0], va);
            unpack<E, V>(cb[n & 1][1], vb);
            unpack<E, V>(cb[n & 1][2], vc);
            unpack<E, V>(cb[n & 1][3], ve);
#pragma unroll
            for (int z = 0; z < V; ++z) {
                d00 = fmaf(gv[uu][z], va[z], d00);
                d01 = fmaf(gv[uu][z], vb[z], d01);
                d10 = fmaf(gv[uu][z], vc[z], d10);
                d11 = fmaf(gv[uu][z], ve[z], d11);
            }
            if (uu == NC - 1) {
                const TapG &t = tg[k & 1];
                if (!t.inreg) d00 = d01 = d10 = d11 = 0.0f;  // outside the image, or redone below
                grads(k, m[k], t.uy, t.fy, t.ux, t.fx, d00, d01, d10, d11);
                d00 = d01 = d10 = d11 = 0.0f;
            }
        };
        issue(0);
#pragma unroll
        for (int n = 0; n < NU; ++n) {
            if (n + 1 < NU) issue(n + 1);
            accum(n);
        }
        if (far) {  // deferred global pass (rare): taps leaving the region
            const Bt *img = x + (size_t)a.n * p.H * p.W * GC + (size_t)l.g * p.C;
            const float2 *coff = reinterpret_cast<const float2 *>(offset) + pair * K;
            const int by0 = l.ho * p.sh - p.ph, bx0 = l.wo * p.sw - p.pw;
            while (far) {
                const int k = __builtin_ctz(far);
                far &= far - 1;
                const float2 dv = coff[k];
                float dx = dv.x, dy = dv.y;
                if (p.offset_scale != 1.0f) {
                    dx = mul_rn(p.offset_scale, dx);
                    dy = mul_rn(p.offset_scale, dy);
                }
                const int i = k / 3, j = k - (k / 3) * 3;
                int y0, x0;
                float fy, uy, fx, ux;
                split_coord_fu(by0 + i * p.dh, dy, y0, fy, uy);
                split_coord_fu(bx0 + j * p.dw, dx, x0, fx, ux);
                const bool vy0 = (unsigned)y0 < (unsigned)p.H, vy1 = (unsigned)(y0 + 1) < (unsigned)p.H;
                const bool vx0 = (unsigned)x0 < (unsigned)p.W, vx1 = (unsigned)(x0 + 1) < (unsigned)p.W;
                const int yc0 = min(max(y0, 0), p.H - 1), yc1 = min(max(y0 + 1, 0), p.H - 1);
                const int xc0 = min(max(x0, 0), p.W - 1), xc1 = min(max(x0 + 1, 0), p.W - 1);
                const Bt *r0 = img + (size_t)yc0 * p.W * GC, *r1 = img + (size_t)yc1 * p.W * GC;
                uint4 c[NC][4];
#pragma unroll
                for (int uu = 0; uu < NC; ++uu) {
                    c[uu][0] = *reinterpret_cast<const uint4 *>(r0 + (size_t)xc0 * GC + uu * V);
                    c[uu][1] = *reinterpret_cast<const uint4 *>(r0 + (size_t)xc1 * GC + uu * V);
                    c[uu][2] = *reinterpret_cast<const uint4 *>(r1 + (size_t)xc0 * GC + uu * V);
                    c[uu][3] = *reinterpret_cast<const uint4 *>(r1 + (size_t)xc1 * GC + uu * V);
                }
                float e00 = 0.0f, e01 = 0.0f, e10 = 0.0f, e11 = 0.0f;
                dots4<E, NC>(c, gv, e00, e01, e10, e11);
                if (!(vy0 && vx0)) e00 = 0.0f;
                if (!(vy0 && vx1)) e01 = 0.0f;
                if (!(vy1 && vx0)) e10 = 0.0f;
                if (!(vy1 && vx1)) e11 = 0.0f;
                // results go to registers: select the tap at compile time (its LDS pass
                // added 0 to dot)
#pragma unroll
                for (int kk = 0; kk < K; ++kk)
                    if (kk == k) grads(kk, m[kk], uy, fy, ux, fx, e00, e01, e10, e11);
            }
        }
        if (p.softmax) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if constexpr (kStage) rg[k] = m[k] * (rg[k] - dot);
                else if (gmp) gmp[k] = m[k] * (gmp[k] - dot);
            }
        }
    }
    if constexpr (!kStage) return;
    // Stores through LDS (the region is no longer read): each pair's 27 results in a
    // staging row, then the block writes every pixel's run of GB pairs (GB*18 floats of
    // grad_offset, GB*9 of grad_mask, contiguous in memory) with consecutive lanes on
    // consecutive 8- or 4-byte pieces.
    __syncthreads();
    float *stg = reinterpret_cast<float *>(lds);
    const int tid = threadIdx.x;
    if (l.active) {
        float *row = stg + (size_t)tid * 27;  // tid = q * GB + gl (one lane per pair)
#pragma unroll
        for (int k = 0; k < K; ++k) {
            row[2 * k] = ro[k].x;
            row[2 * k + 1] = ro[k].y;
            row[18 + k] = rg[k];
        }
    }
    __syncthreads();
    const int npix = p.TH * p.TW, GB = p.GB;
    const int run2 = GB * K;  // float2 pieces of grad_offset per pixel (= grad_mask floats)
    for (int t = tid; t < npix * run2; t += blockDim.x) {
        const int q = t / run2, j = t - q * run2;
        const int qy = q / p.TW, qx = q - qy * p.TW;
        const int ho = a.ho0 + qy, wo = a.wo0 + qx;
        if (ho >= p.Ho || wo >= p.Wo) continue;
        const int gl = j / K, k = j - gl * K;
        const float *row = stg + (size_t)(q * GB + gl) * 27;
        const size_t pr = (((size_t)a.n * p.Ho + ho) * p.Wo + wo) * p.G + a.g0 + gl;
        if (goff) reinterpret_cast<float2 *>(goff)[pr * K + k] = make_float2(row[2 * k], row[2 * k + 1]);
        if (gmask) gmask[pr * K + k] = row[18 + k];
    }
    if (!ra.rec) return;  // uniform over the grid

    // grad_x records (the record pass of the core backward, done here while the
    // offsets are in cache): one 16-byte record per sample with a cell inside the
    // image, filed in its home bin. Bins in the window around this tile (per group
    // of the block) are ranked with plain LDS atomics, others through a hash table;
    // then one range per bin and block is reserved and the records are written.
    unsigned *s_key = reinterpret_cast<unsigned *>(stg + (size_t)blockDim.x * 27);
    unsigned *s_hcnt = s_key + kHash, *s_hbase = s_hcnt + kHash, *s_hlim = s_hbase + kHash;
    unsigned *s_wcnt = s_hlim + kHash;                 // [GB][kWinSlots]
    unsigned *s_wbase = s_wcnt + GB * kWinSlots, *s_wlim = s_wbase + GB * kWinSlots;
    for (int i = tid; i < kHash; i += blockDim.x) {
        s_key[i] = kEmpty;
        s_hcnt[i] = 0;
    }
    for (int i = tid; i < GB * kWinSlots; i += blockDim.x) s_wcnt[i] = 0;
    __syncthreads();
    RecGrid rg2;
    rg2.H = p.H; rg2.W = p.W; rg2.G = p.G; rg2.TY = ra.TY; rg2.TX = ra.TX;
    rg2.sh = p.sh; rg2.sw = p.sw; rg2.ph = p.ph; rg2.pw = p.pw;
    const BinWin win = bin_window(a.ho0, a.wo0, rg2);
    unsigned code[K];
    float2 dk[K];
    const int by0 = l.ho * p.sh - p.ph, bx0 = l.wo * p.sw - p.pw;
    const unsigned pix_in_image = (unsigned)(l.ho * p.Wo + l.wo);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        code[k] = 0xffffffffu;
        dk[k] = make_float2(0.0f, 0.0f);
        if (!l.active) continue;
        float2 dv = reinterpret_cast<const float2 *>(offset)[pair * K + k];
        if (p.offset_scale != 1.0f) {
            dv.x = mul_rn(p.offset_scale, dv.x);
            dv.y = mul_rn(p.offset_scale, dv.y);
        }
        dk[k] = dv;
        const int i = k / 3, j = k - (k / 3) * 3;
        int y0, x0;
        float f, u;
        split_coord_fu(by0 + i * p.dh, dv.y, y0, f, u);
        split_coord_fu(bx0 + j * p.dw, dv.x, x0, f, u);
        unsigned bin, local, rank = 0;
        if (!home_bin(y0, x0, a.n, l.g, rg2, bin, local)) continue;
        const int ws = win_slot(y0, x0, win);
        if (ws >= 0) {
            const int slot = l.gl * kWinSlots + ws;
            rank = atomicAdd(&s_wcnt[slot], 1u);
            code[k] = ((unsigned)(kHash + slot) << 20) | (local << 12) | rank;
        } else {
            const int slot = block_bin_slot(s_key, s_hcnt, bin, rank);
            if (slot < kHash) {
                code[k] = ((unsigned)slot << 20) | (local << 12) | rank;
            } else {  // table full: reserve directly
                const unsigned at = ra.starts[bin] + atomicAdd(&ra.fill[bin], 1u);
                if (at < ra.starts[bin + 1])
                    ra.rec[at] = make_uint4((pix_in_image << 8) | local, __float_as_uint(dv.y),
                                            __float_as_uint(dv.x), __float_as_uint(m[k]));
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < kHash; i += blockDim.x) {
        if (s_hcnt[i]) {
            const unsigned key = s_key[i];
            s_hbase[i] = ra.starts[key] + atomicAdd(&ra.fill[key], s_hcnt[i]);
            s_hlim[i] = ra.starts[key + 1];
        }
    }
    for (int i = tid; i < GB * kWinSlots; i += blockDim.x) {
        if (s_wcnt[i]) {
            const unsigned key = win_bin(i % kWinSlots, a.n, a.g0 + i / kWinSlots, win, rg2);
            s_wbase[i] = ra.starts[key] + atomicAdd(&ra.fill[key], s_wcnt[i]);
            s_wlim[i] = ra.starts[key + 1];
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const unsigned c = code[k];
        if (c == 0xffffffffu) continue;
        const int slot = (int)(c >> 20);
        const unsigned base = slot < kHash ? s_hbase[slot] : s_wbase[slot - kHash];
        const unsigned lim = slot < kHash ? s_hlim[slot] : s_wlim[slot - kHash];
        const unsigned at = base + (c & 0xfffu);
        if (at < lim)
            ra.rec[at] = make_uint4((pix_in_image << 8) | ((c >> 12) & 0xffu), __float_as_uint(dk[k].y),
                                    __float_as_uint(dk[k].x), __float_as_uint(m[k]));
    }
}

// --------------------------------------------------------------- launching --

// Tile knobs of the one-tile kernel: threads per block, tile width, LDS bytes per
// block (two blocks fit in a CU's 160 KB at <= 80 KB), largest halo tried, target
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

template <class E, class OM, int S, int NC>
hipError_t launch_tile(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    using Bt = typename E::bits;
    using OB = typename OM::bits;
    const Bt *x = static_cast<const Bt *>(a.x);
    const OB *off = static_cast<const OB *>(a.offset);
    const OB *msk = static_cast<const OB *>(a.mask);
    Bt *out = static_cast<Bt *>(a.out);
    auto go = [&](auto kern) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
            DCN_TILE_LDS_BYTES);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(kern, dim3(p.nblocks), dim3(p.threads), p.lds_bytes, stream, x, off, msk,
                           out, p);
        return hipGetLastError();
    };
    // 16x16-pixel tiles with halo 8 (region width 35) of 64-byte slices: the common
    // plan, with its region geometry compiled in; with region height 35, 512 threads
    // and an image under 2 GiB, also the staging (RH_ = 35: buffer-form copies)
    const bool fixed = p.RH == 35 && p.threads == 512 && p.lpp == 2 && p.TW == 16 &&
                       (size_t)p.H * p.W * p.G * p.C * sizeof(Bt) < (size_t(1) << 31);

    if (p.cpp == 4 && p.RW == 35 && fixed) return go(dcn_core_tile_kernel<E, OM, 3, 3, S, NC, 4, 35, 35>);
    if (p.cpp == 4 && p.RW == 35) return go(dcn_core_tile_kernel<E, OM, 3, 3, S, NC, 4, 35, 0>);
    if (p.cpp == 2 && p.RW == 35 && fixed) return go(dcn_core_tile_kernel<E, OM, 3, 3, S, NC, 2, 35, 35>);
    if (p.cpp == 2 && p.RW == 35) return go(dcn_core_tile_kernel<E, OM, 3, 3, S, NC, 2, 35, 0>);
    return go(dcn_core_tile_kernel<E, OM, 3, 3, S, NC, 0, 0, 0>);
}

template <class E, int S, int NC>
hipError_t launch_tile_om(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    if (a.om_plain) return launch_tile<E, OMPlain, S, NC>(a, p, stream);
    switch (a.om_dtype) {
        case DCN_F32: return launch_tile<E, EF32, S, NC>(a, p, stream);
        case DCN_F16: return launch_tile<E, EF16, S, NC>(a, p, stream);
        case DCN_BF16: return launch_tile<E, EBF16, S, NC>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

template <class E, int NC>
hipError_t launch_tile_s(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    switch (p.S) {
        case 1: return launch_tile_om<E, 1, NC>(a, p, stream);
        case 2: return launch_tile_om<E, 2, NC>(a, p, stream);
        case 4: return launch_tile_om<E, 4, NC>(a, p, stream);
        case 8: return launch_tile_om<E, 8, NC>(a, p, stream);
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

// LDS bytes of a region: whole 1 KB blocks, since every wave's direct-to-LDS copy
// writes 64 consecutive 16-byte chunks.
size_t region_bytes(size_t rh, size_t rw, size_t sb) { return (rh * rw * sb + 1023) / 1024 * 1024; }

int pick_halo(const CoreLaunch &a, int TH, int TW, size_t sb, size_t budget) {
    for (int h = DCN_TILE_MAX_HALO; h >= 1; --h) {
        const size_t rh = (size_t)(TH - 1) * a.sh + (size_t)(a.kh - 1) * a.dh + 2 + 2 * h;
        const size_t rw = (size_t)(TW - 1) * a.sw + (size_t)(a.kw - 1) * a.dw + 2 + 2 * h;
        if (region_bytes(rh, rw, sb) <= budget) return h;
    }
    return -1;
}

}  // namespace

// Choose a tile for the LDS kernels; false if this call should use the direct kernel
// (window other than 3x3, channel slice not a multiple of 16 bytes or over 256
// bytes, misaligned pointers, image too large for 24-bit offsets, or no useful halo
// fits in LDS).
bool plan_core_tile(const CoreLaunch &a, TileParams &p) {
    if (!(a.kh == 3 && a.kw == 3)) return false;
    const int elt = a.dtype == DCN_F32 ? 4 : 2;
    const int cbytes = a.C * elt;
    if (cbytes % 16 != 0 || cbytes > 256) return false;
    if ((uintptr_t)a.x % 16 || (uintptr_t)a.out % 16) return false;
    if (a.om_plain && (uintptr_t)a.offset % 8) return false;  // 8-byte (dx, dy) loads
    if ((long long)a.H * a.W >= (1LL << 24) || (long long)a.G * a.C >= (1LL << 24)) return false;
    // lane indices use 24-bit multiplies (the pair count is below 2^31 by validation)
    if ((long long)a.N * a.Ho >= (1LL << 24) || (long long)a.Wo * a.G >= (1LL << 24)) return false;
    // 16-byte chunks per lane: two where the channels allow, except for bf16, whose
    // widening (no mixed-precision FMA) would need twice the registers
    const int NC = (cbytes % 32 == 0 && a.dtype != DCN_BF16) ? 2 : 1;
    const int S = cbytes / (16 * NC);  // lanes per (pixel, group): 1, 2, 4 or 8
    if (S & (S - 1)) return false;
    int GB = 1;  // groups per tile: a power of two dividing G, slice <= DCN_TILE_SLICE
    while (a.G % (2 * GB) == 0 && 2 * GB * cbytes <= DCN_TILE_SLICE) GB *= 2;
    const int cpp = GB * cbytes / 16;  // chunks per region pixel (a power of two)
    const int lpp = GB * S;            // lanes per output pixel
    const size_t sb = (size_t)cpp * 16;

    const int pix = DCN_TILE_THREADS / lpp;
    if (pix < 1) return false;
    int TW = DCN_TILE_TW < pix ? DCN_TILE_TW : pix;
    if (TW > a.Wo) TW = a.Wo;
    int TH = pix / TW;
    if (TH > a.Ho) TH = a.Ho;
    if (TH < 1) return false;
    if ((TH * TW) % NC != 0) return false;  // staging needs blockDim % cpp == 0
    const int halo = pick_halo(a, TH, TW, sb, DCN_TILE_LDS_BYTES);
    if (halo < 2) return false;
    p.N = a.N; p.H = a.H; p.W = a.W; p.G = a.G; p.C = a.C; p.kh = a.kh; p.kw = a.kw;
    p.sh = a.sh; p.sw = a.sw; p.ph = a.ph; p.pw = a.pw; p.dh = a.dh; p.dw = a.dw;
    p.Ho = a.Ho; p.Wo = a.Wo;
    p.offset_scale = a.offset_scale;
    p.softmax = a.softmax ? 1 : 0;
    p.has_mask = a.mask != nullptr;
    p.off_pix = a.off_pix; p.off_grp = a.off_grp; p.mask_pix = a.mask_pix; p.mask_grp = a.mask_grp;
    p.GB = GB; p.S = S; p.NC = NC; p.cpp = cpp; p.cpp_log2 = ilog2(cpp); p.lpp = lpp;
    p.TH = TH; p.TW = TW; p.halo = halo;
    p.RH = (TH - 1) * a.sh + (a.kh - 1) * a.dh + 2 + 2 * halo;
    p.RW = (TW - 1) * a.sw + (a.kw - 1) * a.dw + 2 + 2 * halo;
    p.tiles_x = (a.Wo + TW - 1) / TW;
    p.tiles_y = (a.Ho + TH - 1) / TH;
    p.gblocks = a.G / GB;
    const long long nt = (long long)p.gblocks * a.N * p.tiles_y * p.tiles_x;
    if (nt > 0x7fffffffLL) return false;
    p.nblocks = (int)nt;  // tiles
    p.threads = TH * TW * lpp;
    p.lds_bytes = region_bytes(p.RH, p.RW, sb);
    return true;
}

template <class E, int NC>
hipError_t launch_bwd_tile_nc(const CoreLaunch &a, const TileParams &p, float *goff, float *gmask,
                              const CoreRecArgs *ra, bool *rec_done, hipStream_t stream) {
    // the variants with the region geometry compiled in also file the grad_x records
    CoreRecArgs rec = {};
    const bool staged = p.RW == 35 && (p.cpp == 4 || p.cpp == 2);
    if (ra && staged) rec = *ra;
    if (rec_done) *rec_done = rec.rec != nullptr;
    using Bt = typename E::bits;
    const Bt *x = static_cast<const Bt *>(a.x);
    const Bt *gout = static_cast<const Bt *>(a.out);
    const float *off = static_cast<const float *>(a.offset);
    const float *msk = static_cast<const float *>(a.mask);
    auto go = [&](auto kern) {
        static const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
            DCN_TILE_LDS_BYTES);
        if (attr != hipSuccess) return attr;
        // one staging row per pair, then the record pass's hash table and bin windows
        const size_t stage = (size_t)p.threads * 27 * sizeof(float) +
                             (size_t)(4 * kHash + 3 * p.GB * kWinSlots) * sizeof(unsigned);
        const size_t lds = p.lds_bytes > stage ? p.lds_bytes : stage;
        hipLaunchKernelGGL(kern, dim3(p.nblocks), dim3(p.threads), lds, stream, x, off, msk, gout,
                           goff, gmask, p, rec);
        return hipGetLastError();
    };
    if (p.cpp == 4 && p.RW == 35) return go(dcn_core_bwd_tile_kernel<E, NC, 4, 35>);
    if (p.cpp == 2 && p.RW == 35) return go(dcn_core_bwd_tile_kernel<E, NC, 2, 35>);
    return go(dcn_core_bwd_tile_kernel<E, NC, 0, 0>);
}

template <class E>
hipError_t launch_bwd_tile_e(const CoreLaunch &a, const TileParams &p, float *goff, float *gmask,
                             const CoreRecArgs *ra, bool *rec_done, hipStream_t stream) {
    if constexpr (E::id == DCN_BF16) {
        return launch_bwd_tile_nc<E, 1>(a, p, goff, gmask, ra, rec_done, stream);
    } else {
        return p.NC == 2 ? launch_bwd_tile_nc<E, 2>(a, p, goff, gmask, ra, rec_done, stream)
                         : launch_bwd_tile_nc<E, 1>(a, p, goff, gmask, ra, rec_done, stream);
    }
}

hipError_t launch_dcn_core_tile(const CoreLaunch &a, const TileParams &p, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_tile_e<EF32>(a, p, stream);
        case DCN_F16: return launch_tile_e<EF16>(a, p, stream);
        case DCN_BF16: return launch_tile_e<EBF16>(a, p, stream);
    }
    return hipErrorInvalidValue;
}

// grad_offset / grad_mask of the core backward on the tile plan p (S == 1, fp32 plain
// offsets): a.out carries grad_out.
hipError_t launch_dcn_core_bwd_tile(const CoreLaunch &a, const TileParams &p, float *goff, float *gmask,
                                    const CoreRecArgs *ra, bool *rec_done, hipStream_t stream) {
    if (rec_done) *rec_done = false;
    if (p.S != 1 || a.kh != 3 || a.kw != 3) return hipErrorInvalidValue;
    switch (a.dtype) {
        case DCN_F32: return launch_bwd_tile_e<EF32>(a, p, goff, gmask, ra, rec_done, stream);
        case DCN_F16: return launch_bwd_tile_e<EF16>(a, p, goff, gmask, ra, rec_done, stream);
        case DCN_BF16: return launch_bwd_tile_e<EBF16>(a, p, goff, gmask, ra, rec_done, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
