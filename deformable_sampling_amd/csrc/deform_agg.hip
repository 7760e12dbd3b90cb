// Multi-camera, multi-scale deformable aggregation (Sparse4D) for gfx950.
//
// Operation ("Sparse4D deformable_aggregation", mlqm.cn, sections 2.1-2.2 and 7;
// bilinear kernel from "Hands-on DCNv1 in PyTorch", agent.csdn.net, section 2):
//   out[b,a,g*Cg+c] = sum_{p,cam,s} w[b,a,p,cam,s,g] * bilinear(map_{cam,s}, y, x),
//   x = fl32(u*W_s) - 0.5, y = fl32(v*H_s) - 0.5,
// with the weights optionally softmax-normalised over all (p, cam, s) of (b, a, g).
//
// Mapping. One wavefront per (anchor, group) unit. The unit's T taps are taken in
// chunks of 64. For a chunk, each lane first turns one tap into a record in LDS:
// its four corner offsets and four bilinear weights with the tap weight folded in
// (the softmax numerator exp(l - max) when normalising; the division by the sum
// is applied once at the end). Then S = Cg/V lanes hold the group's channels (V per
// lane, 16 bytes for fp32) and the Z = 64/S lane slices share out the chunk's
// records: per record, 4 corner loads and 4V fused multiply-adds. The Z partial sums
// are combined with shuffles at the end.
//
// Locality. Taps are visited camera-major (camera, scale, point), units are ordered
// group-major and blocks are remapped so each XCD runs a contiguous range of units.
// With 8 groups each XCD serves one group, and as its wavefronts advance through the
// cameras roughly together, its L2 holds one camera's maps of one group at a time
// (about 2 MB for 6 cameras x 4 scales of 64x176..8x22, 32 fp32 channels) instead of
// that group's slice of every map. Where a camera's taps fit one 64-tap chunk, the
// camera-phased kernel (deform_agg_cam_kernel) goes further: a persistent grid in
// which each wavefront holds up to four units and visits camera c of all of them
// before camera c + 1, so that every unit of an XCD's range passes through a camera
// while its maps are in L2, not only the units resident at one time.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

struct AggParams {
    int B, P_total, A, pts, cams, scales, G, Cg, softmax;
    int S, Z, nchunk;  // lanes per slice, slices per wave, V-chunks per group
    int BA;            // B*A
    int nunits;        // B*A*G
    int nblocks;
    AggMaps maps;
};

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Records gathered per unrolled step of a slice, and the occupancy the register
// allocation aims for (waves per SIMD).
#ifndef DCN_AGG_UNROLL
#define DCN_AGG_UNROLL 4
#endif
#ifndef DCN_AGG_WAVES_PER_EU
#define DCN_AGG_WAVES_PER_EU 2
#endif
constexpr int kU = DCN_AGG_UNROLL;

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
// The same maximum without LDS permutes (every lane active): row_shr DPP steps leave
// each 16-lane row's maximum in the row's last lane (lanes without a source keep -inf),
// and four lane reads combine the rows.
__device__ __forceinline__ float wave_max_dpp(float v) {
    const int ninf = __float_as_int(-INFINITY);
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x111, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x112, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x114, 0xf, 0xf, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x118, 0xf, 0xf, false)));
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 47));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 63));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// One sampling tap: offsets of the 4 corners from the group's feature base (bytes
// for buffer loads, elements otherwise) and their weights (bilinear x tap weight; 0 for corners outside the map).
struct alignas(16) TapRec {
    int o00, o01, o10, o11;
    float w00, w01, w10, w11;
};

template <class E, int V, bool BUF>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DCN_AGG_WAVES_PER_EU)))
void deform_agg_kernel(const typename E::bits *__restrict__ feat,
                                                              const float *__restrict__ loc,
                                                              const float *__restrict__ weights,
                                                              typename E::bits *__restrict__ out,
                                                              const AggParams p) {
    __shared__ int s_h[kAggMaxMaps], s_w[kAggMaxMaps], s_start[kAggMaxMaps];
    __shared__ TapRec s_rec[kWaves][64];

    const int nmaps = p.cams * p.scales;
    for (int i = threadIdx.x; i < nmaps; i += kThreads) {
        s_h[i] = p.maps.H[i];
        s_w[i] = p.maps.W[i];
        s_start[i] = p.maps.start[i];
    }
    __syncthreads();

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int unit = blk * kWaves + wv;
    if (unit >= p.nunits) return;  // whole wavefronts leave together; no barrier follows
    const int lane = threadIdx.x & 63;
    const int z = lane / p.S, s = lane - z * p.S;
    const bool lane_on = z < p.Z;

#ifndef DCN_AGG_ORDER
#define DCN_AGG_ORDER 0
#endif
#if DCN_AGG_ORDER == 0
    const int g = unit / p.BA, ba = unit - g * p.BA;  // group-major
#elif DCN_AGG_ORDER == 1
    const int ba = unit / p.G, g = unit - ba * p.G;  // anchor-major
#else
    // XCD x (contiguous eighth of the units) serves groups 2*(x/2)..+1, alternating
    const int h = unit / (2 * p.BA), rem = unit - h * 2 * p.BA;
    const int ba = rem >> 1, g = 2 * h + (rem & 1);
#endif
    const int b = ba / p.A;
    const int T = p.pts * p.cams * p.scales;
    const int sp = p.scales * p.pts;
    const float *wrow = weights + (size_t)ba * T * p.G + g;  // natural tap tn at wrow[tn*G]
    const float *lrow = loc + (size_t)ba * p.pts * p.cams * 2;
    const int GC = p.G * p.Cg;
    const typename E::bits *fb = feat + (size_t)b * p.P_total * GC + g * p.Cg;
    constexpr int elt = (int)sizeof(typename E::bits);
    constexpr int kOffScale = BUF ? elt : 1;  // record offsets: bytes (buffer) or elements
    // buffer view of this batch's features from the group's first channel; the
    // hardware returns 0 for any read past its end
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)fb, (short)0, BUF ? (int)((unsigned)((size_t)p.P_total * GC - g * p.Cg) * elt) : 0,
        0x00020000);
    TapRec *rec = s_rec[wv];

    float mx = 0.0f;
    if (p.softmax) {
        float m = -INFINITY;
        for (int t = lane; t < T; t += 64) m = fmaxf(m, wrow[(size_t)t * p.G]);
        mx = wave_max(m);
    }

    for (int ch0 = 0; ch0 < p.nchunk; ch0 += p.S) {
        const int ch = ch0 + s;
        const bool ch_on = lane_on && ch < p.nchunk;
        const typename E::bits *fc = fb + ch * V;
        float acc[V];
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = 0.0f;
        float esum = 0.0f;

        // tap weight (logit) and location of the lane's tap in chunk t0
        auto fetch = [&](int t0, float &w, float2 &uv) {
            const int t = t0 + lane;
            if (t < T) {
                const int cam = t / sp, rem = t - cam * sp;
                const int sc = rem / p.pts, pt = rem - sc * p.pts;
                w = wrow[(size_t)((pt * p.cams + cam) * p.scales + sc) * p.G];
                uv = *reinterpret_cast<const float2 *>(lrow + 2 * (pt * p.cams + cam));
            }
        };
        float w_nx = 0.0f;
        float2 uv_nx = make_float2(0.0f, 0.0f);
        fetch(0, w_nx, uv_nx);

        for (int t0 = 0; t0 < T; t0 += 64) {
            // ---- records: lane l describes tap t0 + l (camera, scale, point order)
            const int t = t0 + lane;
            float w = w_nx;
            const float2 uv = uv_nx;
            if (t0 + 64 < T) fetch(t0 + 64, w_nx, uv_nx);  // in flight during the gathers
            TapRec r;
            if (t < T) {
                const int cam = t / sp, rem = t - cam * sp;
                const int sc = rem / p.pts;
                const int cs = cam * p.scales + sc;
                if (p.softmax) {
                    w = expf(w - mx);
                    esum += w;
                }
                const int Hs = s_h[cs], Ws = s_w[cs];
                // one fp32 rounding of u*W, then the half-pixel shift
                const float xf = __fsub_rn(mul_rn(uv.x, (float)Ws), 0.5f);
                const float yf = __fsub_rn(mul_rn(uv.y, (float)Hs), 0.5f);
                int x0, y0;
                float fx, fy;
                split_coord(0, xf, x0, fx);
                split_coord(0, yf, y0, fy);
                const Tap tp = make_tap(y0, x0, fy, fx, w, Hs, Ws, GC);
                const int base = s_start[cs] * GC;
                r.o00 = (base + tp.o00) * kOffScale; r.o01 = (base + tp.o01) * kOffScale;
                r.o10 = (base + tp.o10) * kOffScale; r.o11 = (base + tp.o11) * kOffScale;
                r.w00 = tp.w00; r.w01 = tp.w01; r.w10 = tp.w10; r.w11 = tp.w11;
            } else {  // padding record: weight 0, reads pixel 0 of the first map
                r.o00 = r.o01 = r.o10 = r.o11 = 0;
                r.w00 = r.w01 = r.w10 = r.w11 = 0.0f;
            }
            rec[lane] = r;  // this wavefront's own records: LDS keeps a wave's accesses in order

            // ---- gathers: slice z takes records z, z+Z, ...; U records per batch, all
            // 4U corner loads issued before the first multiply-add
            const int nt = min(64, T - t0);
            if (ch_on) {
                using R = typename Raw<V * elt>::t;
                const int lane_off = ch * V * elt;
                auto ld = [&](int off) -> R {
                    if constexpr (BUF) {
                        return buffer_load<R>(rsrc, off + lane_off);
                    } else {
                        return *reinterpret_cast<const R *>(fc + off);
                    }
                };
                for (int jb = 0; jb < nt; jb += kU * p.Z) {
                    TapRec q[kU];
                    R d[kU][4];
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const int j = jb + u * p.Z + z;
                        q[u] = rec[j < 64 ? j : 63];
                        if (j >= nt) q[u].w00 = q[u].w01 = q[u].w10 = q[u].w11 = 0.0f;
                    }
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        d[u][0] = ld(q[u].o00);
                        d[u][1] = ld(q[u].o01);
                        d[u][2] = ld(q[u].o10);
                        d[u][3] = ld(q[u].o11);
                    }
#pragma unroll
                    for (int u = 0; u < kU; ++u) {
                        const float wc[4] = {q[u].w00, q[u].w01, q[u].w10, q[u].w11};
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            float f[V];
                            load_f32<E, V>(reinterpret_cast<const typename E::bits *>(&d[u][c]), f);
#pragma unroll
                            for (int i = 0; i < V; ++i) acc[i] = fmaf(wc[c], f[i], acc[i]);
                        }
                    }
                }
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
        if (p.softmax) {
            const float inv = 1.0f / wave_sum(esum);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] *= inv;
        }
        if (z == 0 && ch < p.nchunk)
            store_f32<E, V>(out + (size_t)ba * GC + g * p.Cg + ch * V, acc);
    }
}

// Software-pipelined form for the common shapes: a group's channels are exactly S
// 16-byte lane chunks (S = 4, 8 or 16), with feature slabs addressable by buffer
// loads. A slice takes U records per batch; batch k+1's 4U corner loads are issued
// before batch k is consumed, so each wavefront always has loads in flight, and the
// next chunk's records are built (into the other of two LDS record buffers) while
// the current chunk's first loads are outstanding.
#ifndef DCN_AGG_PIPE_U
#define DCN_AGG_PIPE_U 1
#endif
// Dynamic LDS reserved per block of the pipelined kernel, only to cap residency
// (about 77 KB per block with the static records: 2 blocks, 8 wavefronts per CU).
// For these random 128-byte gathers more resident wavefronts do not add bandwidth:
// with a group's lines confined to one eighth of the L2 sets (pixel stride = 8
// lines), more lines in flight mostly evict each other.
#ifndef DCN_AGG_LDS_RESERVE
#define DCN_AGG_LDS_RESERVE 61440
#endif

template <class E, int S, int U>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DCN_AGG_WAVES_PER_EU)))
void deform_agg_pipe_kernel(const typename E::bits *__restrict__ feat,
                            const float *__restrict__ loc, const float *__restrict__ weights,
                            typename E::bits *__restrict__ out, const AggParams p) {
    constexpr int elt = (int)sizeof(typename E::bits);
    constexpr int V = 16 / elt;
    constexpr int Z = 64 / S;    // slices per wavefront
    constexpr int NB = S / U;    // batches per slice per 64-record chunk
    static_assert(S * Z == 64 && NB * U == S && NB % 2 == 0, "pipeline shape");
    using R = uint4;

    __shared__ int s_h[kAggMaxMaps], s_w[kAggMaxMaps], s_start[kAggMaxMaps];
    __shared__ TapRec s_rec[kWaves][2][64];

    const int nmaps = p.cams * p.scales;
    for (int i = threadIdx.x; i < nmaps; i += kThreads) {
        s_h[i] = p.maps.H[i];
        s_w[i] = p.maps.W[i];
        s_start[i] = p.maps.start[i];
    }
    __syncthreads();

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int unit = blk * kWaves + wv;
    if (unit >= p.nunits) return;  // whole wavefronts leave together; no barrier follows
    const int lane = threadIdx.x & 63;
    const int z = lane / S, s = lane % S;

    const int g = unit / p.BA, ba = unit - g * p.BA;  // group-major
    const int b = ba / p.A;
    const int T = p.pts * p.cams * p.scales;
    const int sp = p.scales * p.pts;
    const float *wrow = weights + (size_t)ba * T * p.G + g;  // natural tap tn at wrow[tn*G]
    const float *lrow = loc + (size_t)ba * p.pts * p.cams * 2;
    const int GC = p.G * p.Cg;
    const typename E::bits *fb = feat + (size_t)b * p.P_total * GC + g * p.Cg;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)fb, (short)0, (int)((unsigned)((size_t)p.P_total * GC - g * p.Cg) * elt),
        0x00020000);
    const int lane_off = s * 16;

    // Softmax without a separate pass over the logits: records of a chunk carry
    // exp(l - m) for the running maximum m as of that chunk (m_run, wave-uniform);
    // esum is kept relative to m_run, and the accumulators are rescaled by
    // exp(m_old - m_new) where consumption enters the next chunk (f_next).
    float m_run = -INFINITY, f_next = 1.0f;

    // ---- records: lane l describes tap t0 + l (camera, scale, point order)
    float w_nx = 0.0f, esum = 0.0f;
    float2 uv_nx = make_float2(0.0f, 0.0f);
    auto fetch = [&](int t0) __attribute__((always_inline)) {
        const int t = t0 + lane;
        if (t < T) {
            const int cam = t / sp, rem = t - cam * sp;
            const int sc = rem / p.pts, pt = rem - sc * p.pts;
            w_nx = wrow[(size_t)((pt * p.cams + cam) * p.scales + sc) * p.G];
            uv_nx = *reinterpret_cast<const float2 *>(lrow + 2 * (pt * p.cams + cam));
        }
    };
    auto build = [&](int t0, TapRec *buf) __attribute__((always_inline)) {
        const int t = t0 + lane;
        float w = w_nx;
        const float2 uv = uv_nx;
        if (t0 + 64 < T) fetch(t0 + 64);  // in flight until the next build
        if (p.softmax) {
            const float l = t < T ? w : -INFINITY;
            const float m_new = fmaxf(m_run, wave_max(l));
            f_next = m_new == -INFINITY ? 1.0f : expf(m_run - m_new);
            esum *= f_next;
            m_run = m_new;
            w = l == -INFINITY ? 0.0f : expf(l - m_new);
            esum += w;
        }
        TapRec r;
        if (t < T) {
            const int cam = t / sp, rem = t - cam * sp;
            const int cs = cam * p.scales + rem / p.pts;
            const int Hs = s_h[cs], Ws = s_w[cs];
            // one fp32 rounding of u*W, then the half-pixel shift
            const float xf = __fsub_rn(mul_rn(uv.x, (float)Ws), 0.5f);
            const float yf = __fsub_rn(mul_rn(uv.y, (float)Hs), 0.5f);
            int x0, y0;
            float fx, fy;
            split_coord(0, xf, x0, fx);
            split_coord(0, yf, y0, fy);
            const Tap tp = make_tap(y0, x0, fy, fx, w, Hs, Ws, GC);
            const int base = s_start[cs] * GC;
            r.o00 = (base + tp.o00) * elt; r.o01 = (base + tp.o01) * elt;
            r.o10 = (base + tp.o10) * elt; r.o11 = (base + tp.o11) * elt;
            r.w00 = tp.w00; r.w01 = tp.w01; r.w10 = tp.w10; r.w11 = tp.w11;
        } else {  // padding record: weight 0, reads the group's first pixel
            r.o00 = r.o01 = r.o10 = r.o11 = 0;
            r.w00 = r.w01 = r.w10 = r.w11 = 0.0f;
        }
        buf[lane] = r;  // this wavefront's own records: LDS keeps a wave's accesses in order
    };

    // ---- gathers: batch bb of chunk c = records (bb*U + u)*Z + z, u < U
    struct Batch {
        R d[U][4];
        float w[U][4];
    };
    auto issue = [&](int c, int bb, Batch &B) __attribute__((always_inline)) {
        const TapRec *rc = s_rec[wv][c & 1];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const TapRec q = rc[(bb * U + u) * Z + z];
            B.w[u][0] = q.w00; B.w[u][1] = q.w01; B.w[u][2] = q.w10; B.w[u][3] = q.w11;
            B.d[u][0] = buffer_load<R>(rsrc, q.o00 + lane_off);
            B.d[u][1] = buffer_load<R>(rsrc, q.o01 + lane_off);
            B.d[u][2] = buffer_load<R>(rsrc, q.o10 + lane_off);
            B.d[u][3] = buffer_load<R>(rsrc, q.o11 + lane_off);
        }
    };
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    auto consume = [&](const Batch &B) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float f[V];
                load_f32<E, V>(reinterpret_cast<const typename E::bits *>(&B.d[u][k]), f);
#pragma unroll
                for (int i = 0; i < V; ++i) acc[i] = fmaf(B.w[u][k], f[i], acc[i]);
            }
        // Empty volatile asm reading and writing the accumulators: the batch's
        // multiply-adds complete here, before the loads that follow in program order,
        // instead of being sunk to the end of the chunk (which would keep every
        // batch's data live in registers at once).
#pragma unroll
        for (int i = 0; i < V; ++i) asm volatile("" : "+v"(acc[i]));
    };

    const int nch = (T + 63) / 64;
    fetch(0);
    build(0, s_rec[wv][0]);
    Batch A, B2;
    issue(0, 0, A);
    for (int c = 0; c < nch; ++c) {
        const bool more = c + 1 < nch;
        if (p.softmax)  // chunk c's records are relative to the maximum as of chunk c
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] *= f_next;
        if (more) build((c + 1) * 64, s_rec[wv][(c + 1) & 1]);
#pragma unroll
        for (int bb = 0; bb < NB; bb += 2) {  // A holds batch bb, B2 takes bb + 1
            issue(c, bb + 1, B2);
            consume(A);
            if (bb + 2 < NB) issue(c, bb + 2, A);
            else if (more) issue(c + 1, 0, A);
            consume(B2);
        }
    }

    // combine the Z slices (lanes s, s+S, s+2S, ...)
#pragma unroll
    for (int o = S; o < 64; o <<= 1)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] += __shfl_xor(acc[i], o, 64);
    if (p.softmax) {
        const float inv = 1.0f / wave_sum(esum);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] *= inv;
    }
    if (z == 0) store_f32<E, V>(out + (size_t)ba * GC + g * p.Cg + s * V, acc);
}

// ------------------------------------------------------ camera-phased --
//
// The pipelined kernel with the units of an XCD processed camera by camera. In the
// kernel above a wavefront takes one unit from start to end, so the 256 wavefronts an
// XCD holds at a time pass through the cameras together, but the ~3.5 rounds of
// units that follow each fetch every camera's maps of their group into L2 again:
// about 3.5 x 6 x 1.9 MB of fills per group, where one camera's maps of one group
// (1.9 MB for 64x176..8x22 and 32 fp32 channels) fit the 4 MB L2. Here the grid is
// persistent (two blocks per CU, all resident): the units of a round are split into
// eight XCD ranges, wavefront j of an XCD owns units j, j + W, j + 2W, ... (up to MU,
// W = wavefronts per XCD), and a wavefront visits camera 0 of each of its units,
// then camera 1, and so on. A camera's maps are then fetched about once per round
// for all units of the XCD. A chunk is one unit's taps of one camera (scales x
// points <= 64); the softmax keeps a running maximum, a sum and a rescale factor per
// unit, as above. Records, gathers and the one-batch-ahead pipeline are those of the
// kernel above.
template <class E, int S, int U, int MU>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DCN_AGG_WAVES_PER_EU)))
void deform_agg_cam_kernel(const typename E::bits *__restrict__ feat,
                           const float *__restrict__ loc, const float *__restrict__ weights,
                           typename E::bits *__restrict__ out, const AggParams p) {
    constexpr int elt = (int)sizeof(typename E::bits);
    constexpr int V = 16 / elt;
    constexpr int Z = 64 / S;    // slices per wavefront
    constexpr int NB = S / U;    // batches per slice per 64-record chunk
    static_assert(S * Z == 64 && NB * U == S && NB % 2 == 0, "pipeline shape");
    using R = uint4;

    __shared__ int s_h[kAggMaxMaps], s_w[kAggMaxMaps], s_start[kAggMaxMaps];
    __shared__ TapRec s_rec[kWaves][2][64];

    const int nmaps = p.cams * p.scales;
    for (int i = threadIdx.x; i < nmaps; i += kThreads) {
        s_h[i] = p.maps.H[i];
        s_w[i] = p.maps.W[i];
        s_start[i] = p.maps.start[i];
    }
    __syncthreads();

    // block b runs on XCD b % 8 (the dispatcher's round robin); p.nblocks is a
    // multiple of 8
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int xcd = (int)blockIdx.x % 8;
    const int wpx = (p.nblocks / 8) * kWaves;  // wavefronts per XCD
    const int j = ((int)blockIdx.x / 8) * kWaves + wv;
    const int lane = threadIdx.x & 63;
    const int z = lane / S, s = lane % S;
    const int sp = p.scales * p.pts;  // taps of one camera (<= 64)
    const int GC = p.G * p.Cg;
    const int lane_off = s * 16;
    const int per_round = 8 * wpx * MU;
    const int nch = p.cams * MU;

    for (int r0 = 0; r0 < p.nunits; r0 += per_round) {
        const int nr = min(per_round, p.nunits - r0);
        const int q = (nr + 7) / 8;
        const int u_beg = r0 + xcd * q, u_end = min(r0 + (xcd + 1) * q, r0 + nr);
        if (u_beg + j >= u_end) continue;  // no unit for this wavefront in this round

        bool ok[MU];
        int ba_k[MU], g_k[MU];
        const float *wrow[MU];
        const float *lrow[MU];
        __amdgpu_buffer_rsrc_t rs[MU];
#pragma unroll
        for (int k = 0; k < MU; ++k) {
            const int unit = u_beg + j + k * wpx;
            ok[k] = unit < u_end;
            const int uu = ok[k] ? unit : u_beg + j;
            const int g = uu / p.BA, ba = uu - g * p.BA;  // group-major
            const int b = ba / p.A;
            ba_k[k] = ba;
            g_k[k] = g;
            wrow[k] = weights + (size_t)ba * (sp * p.cams) * p.G + g;
            lrow[k] = loc + (size_t)ba * p.pts * p.cams * 2;
            const typename E::bits *fb = feat + (size_t)b * p.P_total * GC + g * p.Cg;
            rs[k] = __builtin_amdgcn_make_buffer_rsrc(
                (void *)fb, (short)0, (int)((unsigned)((size_t)p.P_total * GC - g * p.Cg) * elt), 0x00020000);
        }

        float m_run[MU], esum[MU], fk[MU];
        float acc[MU][V];
#pragma unroll
        for (int k = 0; k < MU; ++k) {
            m_run[k] = -INFINITY;
            esum[k] = 0.0f;
            fk[k] = 1.0f;
#pragma unroll
            for (int i = 0; i < V; ++i) acc[k][i] = 0.0f;
        }

        // lane l < sp describes tap (cam, scale l / pts, point l % pts) of its unit
        float w_nx = 0.0f;
        float2 uv_nx = make_float2(0.0f, 0.0f);
        auto fetch = [&](int cam, int k) __attribute__((always_inline)) {
            if (ok[k] && lane < sp) {
                const int sc = lane / p.pts, pt = lane - sc * p.pts;
                w_nx = wrow[k][(size_t)((pt * p.cams + cam) * p.scales + sc) * p.G];
                uv_nx = *reinterpret_cast<const float2 *>(lrow[k] + 2 * (pt * p.cams + cam));
            }
        };
        // records of chunk (cam, k) into buf; then the inputs of chunk (cam2, k2)
        auto build = [&](int cam, int k, TapRec *buf, int cam2, int k2) __attribute__((always_inline)) {
            const bool valid = ok[k] && lane < sp;
            float w = w_nx;
            const float2 uv = uv_nx;
            if (cam2 < p.cams) fetch(cam2, k2);  // in flight until the next build
            if (p.softmax) {
                const float l = valid ? w : -INFINITY;
                const float m_new = fmaxf(m_run[k], wave_max_dpp(l));
                fk[k] = m_new == -INFINITY ? 1.0f : expf(m_run[k] - m_new);
                esum[k] *= fk[k];
                m_run[k] = m_new;
                w = l == -INFINITY ? 0.0f : expf(l - m_new);
                esum[k] += w;
            }
            TapRec r;
            if (valid) {
                const int cs = cam * p.scales + lane / p.pts;
                const int Hs = s_h[cs], Ws = s_w[cs];
                // one fp32 rounding of u*W, then the half-pixel shift
                const float xf = __fsub_rn(mul_rn(uv.x, (float)Ws), 0.5f);
                const float yf = __fsub_rn(mul_rn(uv.y, (float)Hs), 0.5f);
                int x0, y0;
                float fx, fy;
                split_coord(0, xf, x0, fx);
                split_coord(0, yf, y0, fy);
                const Tap tp = make_tap(y0, x0, fy, fx, w, Hs, Ws, GC);
                const int base = s_start[cs] * GC;
                r.o00 = (base + tp.o00) * elt; r.o01 = (base + tp.o01) * elt;
                r.o10 = (base + tp.o10) * elt; r.o11 = (base + tp.o11) * elt;
                r.w00 = tp.w00; r.w01 = tp.w01; r.w10 = tp.w10; r.w11 = tp.w11;
            } else {  // padding record: weight 0, no loads (see issue)
                r.o00 = r.o01 = r.o10 = r.o11 = 0;
                r.w00 = r.w01 = r.w10 = r.w11 = 0.0f;
            }
            buf[lane] = r;  // this wavefront's own records: LDS keeps a wave's accesses in order
        };

        struct Batch {
            R d[U][4];
            float w[U][4];
        };
        // batch bb of the chunk in buffer cb for unit k: records (bb*U + u)*Z + z; the
        // corners of padding records (index >= the chunk's tap count) are not loaded
        auto issue = [&](int k, int cb, int bb, Batch &B) __attribute__((always_inline)) {
            const TapRec *rc = s_rec[wv][cb];
            const int nval = ok[k] ? sp : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ri = (bb * U + u) * Z + z;
                const TapRec q = rc[ri];
                B.w[u][0] = q.w00; B.w[u][1] = q.w01; B.w[u][2] = q.w10; B.w[u][3] = q.w11;
                if (ri < nval) {
                    B.d[u][0] = buffer_load<R>(rs[k], q.o00 + lane_off);
                    B.d[u][1] = buffer_load<R>(rs[k], q.o01 + lane_off);
                    B.d[u][2] = buffer_load<R>(rs[k], q.o10 + lane_off);
                    B.d[u][3] = buffer_load<R>(rs[k], q.o11 + lane_off);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) B.d[u][c] = make_uint4(0, 0, 0, 0);
                }
            }
        };
        auto consume = [&](const Batch &B, float (&ac)[V]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float f[V];
                    load_f32<E, V>(reinterpret_cast<const typename E::bits *>(&B.d[u][c]), f);
#pragma unroll
                    for (int i = 0; i < V; ++i) ac[i] = fmaf(B.w[u][c], f[i], ac[i]);
                }
            // the batch's multiply-adds complete here (see the kernel above)
#pragma unroll
            for (int i = 0; i < V; ++i) asm volatile("" : "+v"(ac[i]));
        };

        // chunk n = cam * MU + k sits in record buffer n & 1 = k & 1 (MU even)
        static_assert(MU % 2 == 0, "record buffer of a chunk from its unit index");
        fetch(0, 0);
        build(0, 0, s_rec[wv][0], 0, 1);
        Batch A, B2;
        issue(0, 0, 0, A);
        for (int cam = 0; cam < p.cams; ++cam) {
#pragma unroll
            for (int k = 0; k < MU; ++k) {
                const int n = cam * MU + k;
                const bool more = n + 1 < nch;
                const int k1 = (k + 1) % MU, cam1 = cam + (k + 1) / MU;
                const int k2 = (k + 2) % MU, cam2 = cam + (k + 2) / MU;
                if (p.softmax)  // chunk n's records are relative to its unit's maximum as of chunk n
#pragma unroll
                    for (int i = 0; i < V; ++i) acc[k][i] *= fk[k];
                if (more) build(cam1, k1, s_rec[wv][k1 & 1], cam2, k2);
#pragma unroll
                for (int bb = 0; bb < NB; bb += 2) {  // A holds batch bb, B2 takes bb + 1
                    issue(k, k & 1, bb + 1, B2);
                    consume(A, acc[k]);
                    if (bb + 2 < NB) issue(k, k & 1, bb + 2, A);
                    else if (more) issue(k1, k1 & 1, 0, A);
                    consume(B2, acc[k]);
                }
            }
        }

#pragma unroll
        for (int k = 0; k < MU; ++k) {
            // combine the Z slices (lanes s, s+S, s+2S, ...)
#pragma unroll
            for (int o = S; o < 64; o <<= 1)
#pragma unroll
                for (int i = 0; i < V; ++i) acc[k][i] += __shfl_xor(acc[k][i], o, 64);
            if (p.softmax) {
                const float inv = 1.0f / wave_sum(esum[k]);
#pragma unroll
                for (int i = 0; i < V; ++i) acc[k][i] *= inv;
            }
            if (ok[k] && z == 0) store_f32<E, V>(out + (size_t)ba_k[k] * GC + g_k[k] * p.Cg + s * V, acc[k]);
        }
    }
}

// Blocks of the persistent grid: two per CU of the current device (rounded up to a
// multiple of the 8 XCDs), looked up once per device.
#ifndef DCN_AGG_CAM_BPC
#define DCN_AGG_CAM_BPC 2
#endif
#ifndef DCN_AGG_CAM_MU
#define DCN_AGG_CAM_MU 4
#endif
int persistent_blocks() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu < 1)
            cu = 256;
        cache[dev] = (DCN_AGG_CAM_BPC * cu + 7) / 8 * 8;
    }
    return cache[dev];
}

template <class E, int V>
hipError_t launch_v(const AggLaunch &a, AggParams &p, hipStream_t stream) {
    using Bt = typename E::bits;
    const Bt *feat = static_cast<const Bt *>(a.feat);
    Bt *out = static_cast<Bt *>(a.out);
    // byte offsets within one batch's feature slab must fit a buffer's 32-bit range
    const bool buf = (unsigned long long)a.P_total * a.G * a.Cg * sizeof(Bt) < (1ull << 31);
    if (buf)
        hipLaunchKernelGGL((deform_agg_kernel<E, V, true>), dim3(p.nblocks), dim3(kThreads), 0,
                           stream, feat, a.loc, a.weights, out, p);
    else
        hipLaunchKernelGGL((deform_agg_kernel<E, V, false>), dim3(p.nblocks), dim3(kThreads), 0,
                           stream, feat, a.loc, a.weights, out, p);
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
    p.nblocks = (p.nunits + kWaves - 1) / kWaves;
    p.maps = a.maps;
    using Bt = typename E::bits;
    const bool buf = (unsigned long long)a.P_total * a.G * a.Cg * elt < (1ull << 31);
    if (buf && V * elt == 16) {
        auto pipe = [&](auto kern) {
            hipLaunchKernelGGL(kern, dim3(p.nblocks), dim3(kThreads), DCN_AGG_LDS_RESERVE, stream,
                               static_cast<const Bt *>(a.feat), a.loc, a.weights,
                               static_cast<Bt *>(a.out), p);
            return hipGetLastError();
        };
        constexpr int U = DCN_AGG_PIPE_U;
        if (p.scales * p.pts <= 64 && (p.nchunk == 8 || p.nchunk == 16 || (p.nchunk == 4 && U <= 2))) {
            // camera-phased persistent grid: two blocks per CU, a multiple of 8
            p.nblocks = persistent_blocks();
            constexpr int MU = DCN_AGG_CAM_MU;
            // dynamic LDS that leaves room for DCN_AGG_CAM_BPC blocks per CU and no more
            constexpr size_t res = 163840 / DCN_AGG_CAM_BPC - (sizeof(TapRec) * kWaves * 2 * 64 + 3 * 4 * kAggMaxMaps) - 1024;
            auto cam = [&](auto kern) {
                hipLaunchKernelGGL(kern, dim3(p.nblocks), dim3(kThreads), res, stream,
                                   static_cast<const Bt *>(a.feat), a.loc, a.weights,
                                   static_cast<Bt *>(a.out), p);
                return hipGetLastError();
            };
            if (p.nchunk == 8) return cam(deform_agg_cam_kernel<E, 8, U, MU>);
            if (p.nchunk == 16) return cam(deform_agg_cam_kernel<E, 16, U, MU>);
            return cam(deform_agg_cam_kernel<E, 4, (U < 2 ? U : 2), MU>);
        }
        if (p.nchunk == 8) return pipe(deform_agg_pipe_kernel<E, 8, U>);
        if (p.nchunk == 16) return pipe(deform_agg_pipe_kernel<E, 16, U>);
        if (p.nchunk == 4 && U <= 2) return pipe(deform_agg_pipe_kernel<E, 4, (U < 2 ? U : 2)>);
    }
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
