// Backward of the multi-camera, multi-scale deformable aggregation, for gfx950.
//
// The Sparse4D deformable_aggregation page ("Sparse4D deformable_aggregation",
// mlqm.cn, section 2.1) names gradients of the features, the sampling locations and
// the weights; these are the derivatives of the forward sum (sections 2.1-2.2 and 7;
// bilinear kernel from "Hands-on DCNv1 in PyTorch", agent.csdn.net, section 2). With
// G the (anchor, group)'s grad_out, wt the (softmax-normalised) weight of sample
// t = (point, camera, scale) at x = fl32(u*W_s) - 0.5, y = fl32(v*H_s) - 0.5, and
// D_ab = sum_c G_c X_ab,c the dot products of G with the four corners:
//   grad_feat[corner ab] += wt * w_ab * G                       (inside the map)
//   g_t    = sum_ab w_ab D_ab        grad_weight_t = g_t, or wt (g_t - sum_j wj g_j)
//   grad_u += wt * W_s * ((1-fy)(D_01 - D_00) + fy (D_11 - D_10))  over scales, groups
//   grad_v += wt * H_s * ((1-fx)(D_10 - D_00) + fx (D_11 - D_01))
// (derivatives from the right at integer positions; d fl32(u*W)/du taken as W).
//
// Mapping: one wavefront per (anchor, group) unit, units group-major (as the
// forward). A round takes 64/scales (point, camera) pairs: each lane first turns one
// sample into an LDS record (clamped corner offsets, validity, fractions and their
// exact complements, wt); then slices of S lanes (V = 4, 2 or 1 channels per lane,
// S*V >= Cg, S a power of two) walk the records: four V-wide corner loads and the
// partial dots D_ab, summed over the slice into the sample's g_t, grad_u, grad_v in
// LDS. The owner lane of each (point, camera) sums its scales and stores that
// group's grad_loc partial. Where a group's channels are 2-16 vectors of 16 bytes
// and a workspace is given, agg_bwd_pipe_kernel does this with the corner loads one
// batch of records ahead (buffer loads, row_shr DPP sums), the unit's logits read
// once into registers (softmax from them, no further passes), and g_t stored
// contiguously per unit in the workspace with the unit's max, 1/sum and
// sum_t wt g_t; a finishing pass then writes grad_weights (g_t, or
// wt (g_t - sum_j wj g_j)) and the normalised weights along their [sample, G]
// layout. (Written from the group-major units directly, those 4-byte stores leave
// every line partly written by eight XCDs: 33 us of the main kernel's 189 us, and
// the two extra passes over the logits 55 us.) Otherwise agg_bwd_kernel takes the
// records one batch at a time, and the lane that built a sample stores its g_t (and,
// with softmax, rewrites it as wt (g_t - sum_j wj g_j) once the sum is known) and its
// normalised weight wt. A second kernel adds the G partials of grad_loc in group
// order.
//
// The feature gradient is a scatter (each sample adds to four feature rows); it runs
// as a gather. Sample corners are bucketed by destination feature row (shared by all
// groups, as the locations are): a count pass and a fill pass enumerate the samples
// map by map, so a block's samples fall on few rows of a small map, and merge them
// per row in an LDS hash table before touching the global counters (one atomic per
// row and block); a one-block scan turns counts into bucket starts. After the main
// kernel, one wavefront per (feature row, 16*V channels) sums wt[g] * w_ab * G over
// the bucket, four entries at a time in four 16-lane groups, and stores the row once
// in its dtype. No float atomics; the summation order within a bucket follows the
// fill order, so grad_feat's last bits may vary between runs, while grad_loc and
// grad_weights are deterministic. Past the bucket limits (or with the DCN_BWD_ATOMIC
// path of deform_agg_backward_path) the feature gradient is accumulated with fp32 atomic adds
// after each batch of records (half a wavefront per corner, 32 contiguous channels
// per half, G from LDS) into grad_feat (fp32) or a workspace accumulator rounded
// once at the end.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRounds = 8;  // channel rounds of 64 lanes: Cg <= 512
constexpr int kRegRounds = 8;  // sample rounds a lane of the pipelined kernel keeps: T <= 8 * 64

struct AggBwdParams {
    int B, P_total, A, pts, cams, scales, G, Cg, softmax;
    int S, Z, crounds;  // slice width, slices per wave, channel rounds (Cg > 64)
    int npc;            // (point, camera) pairs per round
    int BA, nunits, nblocks;
    int want_feat, want_loc, want_w;
    AggMaps maps;
};

struct alignas(16) AggRec {
    int o00, o01, o10, o11;  // element offsets of the corners (clamped into the map)
    float fy, fx, uy, ux;
    float wt, Ws, Hs;
    int valid;               // bit per corner: 1 = 00, 2 = 01, 4 = 10, 8 = 11
};

__device__ __forceinline__ float wsum(float v) {
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wmax(float v) {
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// base + t -> corner, fraction f and its complement u = (floor(t) + 1) - t; each
// of f and u is exact when below 1/2, so both weight factors have full relative
// precision.
__device__ __forceinline__ void split_fu(float t, int &c0, float &f, float &u) {
    t = fminf(fmaxf(t, -16777216.0f), 16777216.0f);
    const float fl = floorf(t);
    f = t - fl;
    u = (fl + 1.0f) - t;
    c0 = (int)fl;
}

template <class E, int V>
__global__ __launch_bounds__(kThreads) void agg_bwd_kernel(
    const typename E::bits *__restrict__ feat, const float *__restrict__ loc,
    const float *__restrict__ weights, const typename E::bits *__restrict__ gout,
    float *__restrict__ gacc, float *__restrict__ gloc_part, float *__restrict__ gw,
    float *__restrict__ wn, const AggBwdParams p) {
    __shared__ int s_h[kAggMaxMaps], s_w[kAggMaxMaps], s_start[kAggMaxMaps];
    __shared__ AggRec s_rec[kWaves][64];
    __shared__ float s_res[kWaves][64][3];  // g_t, grad_u, grad_v per record
    __shared__ float s_g[kWaves][64 * kMaxRounds];  // the unit's grad_out (atomic path)

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
    const int g = unit / p.BA, ba = unit - g * p.BA;  // group-major
    const int b = ba / p.A;
    const int T = p.pts * p.cams * p.scales;
    const int NPC = p.pts * p.cams;
    const int GC = p.G * p.Cg;
    const float *wrow = weights + (size_t)ba * T * p.G + g;  // sample t at wrow[t*G]
    const float *lrow = loc + (size_t)ba * NPC * 2;
    const typename E::bits *fb = feat + (size_t)b * p.P_total * GC + g * p.Cg;
    float *ab = gacc ? gacc + (size_t)b * p.P_total * GC + g * p.Cg : nullptr;
    AggRec *rec = s_rec[wv];
    float(*res)[3] = s_res[wv];

    // softmax over the unit's T logits
    float mx = 0.0f, inv = 1.0f;
    if (p.softmax) {
        float m = -INFINITY;
        for (int t = lane; t < T; t += 64) m = fmaxf(m, wrow[(size_t)t * p.G]);
        mx = wmax(m);
        float e = 0.0f;
        for (int t = lane; t < T; t += 64) e += expf(wrow[(size_t)t * p.G] - mx);
        inv = 1.0f / wsum(e);
    }
    // this lane's channels of G for the loads: channels (cr*S + s)*V + u; for the
    // atomic adds the whole of G waits in LDS
    constexpr int RM = kMaxRounds / V;  // Cg <= 512 = 64 * kMaxRounds
    float gc[RM][V];
#pragma unroll
    for (int r = 0; r < RM; ++r)
#pragma unroll
        for (int u = 0; u < V; ++u) {
            const int c = (r * p.S + s) * V + u;
            gc[r][u] = (r < p.crounds && c < p.Cg) ? to_f32(E{}, gout[(size_t)ba * GC + g * p.Cg + c]) : 0.0f;
        }
    float *sg = s_g[wv];
    if (ab)
        for (int c = lane; c < p.Cg; c += 64) sg[c] = to_f32(E{}, gout[(size_t)ba * GC + g * p.Cg + c]);

    const int per_round = p.npc * p.scales;  // records per round (<= 64)
    float dot = 0.0f;                        // sum_t wt g_t over this lane's samples
    for (int pc0 = 0; pc0 < NPC; pc0 += p.npc) {
        // ---- records: lane l < per_round describes sample (pc0 + l / scales, l % scales)
        const int lpc = lane / p.scales, lsc = lane - lpc * p.scales;
        const int pc = pc0 + lpc;
        const bool own = lane < per_round && pc < NPC;
        int t_nat = 0;
        float wt = 0.0f;
        if (own) {
            const int cam = pc % p.cams;
            const int cs = cam * p.scales + lsc;
            t_nat = pc * p.scales + lsc;  // (point, camera, scale) natural order
            const float l = wrow[(size_t)t_nat * p.G];
            wt = p.softmax ? expf(l - mx) * inv : l;
            const float2 uv = *reinterpret_cast<const float2 *>(lrow + 2 * pc);
            const int Hs = s_h[cs], Ws = s_w[cs];
            const float xf = __fsub_rn(mul_rn(uv.x, (float)Ws), 0.5f);
            const float yf = __fsub_rn(mul_rn(uv.y, (float)Hs), 0.5f);
            int x0, y0;
            AggRec r;
            split_fu(yf, y0, r.fy, r.uy);
            split_fu(xf, x0, r.fx, r.ux);
            const bool vy0 = (unsigned)y0 < (unsigned)Hs, vy1 = (unsigned)(y0 + 1) < (unsigned)Hs;
            const bool vx0 = (unsigned)x0 < (unsigned)Ws, vx1 = (unsigned)(x0 + 1) < (unsigned)Ws;
            const int yc0 = min(max(y0, 0), Hs - 1), yc1 = min(max(y0 + 1, 0), Hs - 1);
            const int xc0 = min(max(x0, 0), Ws - 1), xc1 = min(max(x0 + 1, 0), Ws - 1);
            const int base = s_start[cs];
            r.o00 = (base + yc0 * Ws + xc0) * GC;
            r.o01 = (base + yc0 * Ws + xc1) * GC;
            r.o10 = (base + yc1 * Ws + xc0) * GC;
            r.o11 = (base + yc1 * Ws + xc1) * GC;
            r.valid = (vy0 && vx0 ? 1 : 0) | (vy0 && vx1 ? 2 : 0) | (vy1 && vx0 ? 4 : 0) |
                      (vy1 && vx1 ? 8 : 0);
            r.wt = wt;
            r.Ws = (float)Ws;
            r.Hs = (float)Hs;
            rec[lane] = r;
        }
        const int nrec = min(per_round, (NPC - pc0) * p.scales);
        // ---- gathers: slice z takes records z, z + Z, ... (one channel per lane)
        for (int j0 = 0; j0 < nrec; j0 += p.Z) {
            const int j = j0 + z;
            const bool on = z < p.Z && j < nrec;
            const AggRec r = rec[on ? j : 0];
            float D00 = 0.0f, D01 = 0.0f, D10 = 0.0f, D11 = 0.0f;
            if (on) {
                const float w00 = ((r.valid & 1) ? r.uy * r.ux : 0.0f) * r.wt;
                const float w01 = ((r.valid & 2) ? r.uy * r.fx : 0.0f) * r.wt;
                const float w10 = ((r.valid & 4) ? r.fy * r.ux : 0.0f) * r.wt;
                const float w11 = ((r.valid & 8) ? r.fy * r.fx : 0.0f) * r.wt;
#pragma unroll
                for (int cr = 0; cr < RM; ++cr) {
                    if (cr >= p.crounds) break;
                    const int c = (cr * p.S + s) * V;
                    if (c < p.Cg) {  // Cg % V == 0: the whole vector is in range
                        float a[V], b[V], cc[V], d[V];
                        load_f32<E, V>(fb + r.o00 + c, a);
                        load_f32<E, V>(fb + r.o01 + c, b);
                        load_f32<E, V>(fb + r.o10 + c, cc);
                        load_f32<E, V>(fb + r.o11 + c, d);
#pragma unroll
                        for (int u = 0; u < V; ++u) {
                            const float G = gc[cr][u];
                            D00 = fmaf(G, a[u], D00);
                            D01 = fmaf(G, b[u], D01);
                            D10 = fmaf(G, cc[u], D10);
                            D11 = fmaf(G, d[u], D11);
                        }
                    }
                }
            }
            D00 = seg_sum_pow2(D00, p.S);
            D01 = seg_sum_pow2(D01, p.S);
            D10 = seg_sum_pow2(D10, p.S);
            D11 = seg_sum_pow2(D11, p.S);
            if (on && s == 0) {
                const float d00 = (r.valid & 1) ? D00 : 0.0f, d01 = (r.valid & 2) ? D01 : 0.0f;
                const float d10 = (r.valid & 4) ? D10 : 0.0f, d11 = (r.valid & 8) ? D11 : 0.0f;
                // weights applied outside the differences
                res[j][0] = r.uy * (r.ux * d00 + r.fx * d01) + r.fy * (r.ux * d10 + r.fx * d11);
                res[j][1] = r.wt * r.Ws * (r.uy * (d01 - d00) + r.fy * (d11 - d10));
                res[j][2] = r.wt * r.Hs * (r.ux * (d10 - d00) + r.fx * (d11 - d01));
            }
            // feature gradient of these Z records: per record two atomic instructions,
            // each covering two corners with 32 contiguous channels apiece
            if (ab) {
                const int half = lane >> 5, cl = lane & 31;
                for (int jj = 0; jj < p.Z; ++jj) {
                    const int jr = j0 + jj;
                    if (jr >= nrec) break;
                    const AggRec q = rec[jr];
                    const float wy = half ? q.fy : q.uy;
                    const bool va = (q.valid >> (2 * half)) & 1, vb = (q.valid >> (2 * half + 1)) & 1;
                    const float wa = (va ? wy * q.ux : 0.0f) * q.wt;
                    const float wb = (vb ? wy * q.fx : 0.0f) * q.wt;
                    const int oa = half ? q.o10 : q.o00, ob = half ? q.o11 : q.o01;
                    for (int c = cl; c < p.Cg; c += 32) {
                        const float G = sg[c];
                        if (wa != 0.0f) unsafeAtomicAdd(ab + oa + c, wa * G);
                        if (wb != 0.0f) unsafeAtomicAdd(ab + ob + c, wb * G);
                    }
                }
            }
        }
        // ---- per-sample and per-(point, camera) results (a wavefront's own LDS
        // writes are visible to its later reads: LDS keeps a wave's accesses in order)
        if (own) {
            const float gt = res[lane][0];
            dot = fmaf(wt, gt, dot);
            if (p.want_w) gw[((size_t)ba * T + t_nat) * p.G + g] = gt;
            if (wn) wn[((size_t)ba * T + t_nat) * p.G + g] = wt;
        }
        if (p.want_loc && lane < p.npc && pc0 + lane < NPC) {
            float su = 0.0f, sv = 0.0f;
            for (int k = 0; k < p.scales; ++k) {
                su += res[lane * p.scales + k][1];
                sv += res[lane * p.scales + k][2];
            }
            float *dst = gloc_part + (((size_t)g * p.BA + ba) * NPC + pc0 + lane) * 2;
            dst[0] = su;
            dst[1] = sv;
        }
    }
    // ---- softmax: grad_logit_t = wt (g_t - sum_j wj g_j); each lane rewrites the
    // samples it stored above (its own earlier writes)
    if (p.softmax && p.want_w) {
        const float tot = wsum(dot);
        for (int pc0 = 0; pc0 < NPC; pc0 += p.npc) {
            const int lpc = lane / p.scales, lsc = lane - lpc * p.scales;
            const int pc = pc0 + lpc;
            if (lane < per_round && pc < NPC) {
                const int t_nat = pc * p.scales + lsc;
                const float wt = expf(wrow[(size_t)t_nat * p.G] - mx) * inv;
                float *q = gw + ((size_t)ba * T + t_nat) * p.G + g;
                *q = wt * (*q - tot);
            }
        }
    }
}

// Sum over each aligned S-lane slice (S <= 16, a power of two), complete in the
// slice's last lane: row_shr DPP steps, so no LDS permutes and no waits.
template <int N>
__device__ __forceinline__ float row_shr(float v) {  // lane i gets lane i - N of its row, or 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xf, 0xf, true));
}
template <int S>
__device__ __forceinline__ float slice_sum_to_last(float v) {
    static_assert(S >= 1 && S <= 16 && (S & (S - 1)) == 0, "slice of 1-16 lanes");
    if constexpr (S > 1) v += row_shr<1>(v);
    if constexpr (S > 2) v += row_shr<2>(v);
    if constexpr (S > 4) v += row_shr<4>(v);
    if constexpr (S > 8) v += row_shr<8>(v);
    return v;
}

// The main kernel when a group's channels are S 16-byte vectors (S = 2..16, a power
// of two), no atomic accumulation is asked for and a workspace is given: the same
// records and dot products as agg_bwd_kernel, with the corner loads of each batch of
// Z = 64/S records issued through a buffer resource one batch ahead of the dots
// (record offsets in bytes inside the batch's features, which must be under 2 GiB),
// the unit's logits read once into registers (at most kRegRounds rounds), and per
// unit g_t (unit-major) plus max, 1/sum and sum_t wt g_t into the workspace for
// agg_bwd_finish_kernel.
template <class E, int S>
__global__ __launch_bounds__(kThreads) void agg_bwd_pipe_kernel(
    const typename E::bits *__restrict__ feat, const float *__restrict__ loc,
    const float *__restrict__ weights, const typename E::bits *__restrict__ gout,
    float *__restrict__ gloc_part, float *__restrict__ gts, float *__restrict__ us,
    const AggBwdParams p) {
    using Bt = typename E::bits;
    constexpr int elt = (int)sizeof(Bt);
    constexpr int V = 16 / elt;
    constexpr int Z = 64 / S;
    __shared__ int s_h[kAggMaxMaps], s_w[kAggMaxMaps], s_start[kAggMaxMaps];
    __shared__ AggRec s_rec[kWaves][64];
    __shared__ float s_res[kWaves][64][3];

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
    const int z = lane / S, s = lane - z * S;
    const int g = unit / p.BA, ba = unit - g * p.BA;  // group-major
    const int b = ba / p.A;
    const int T = p.pts * p.cams * p.scales;
    const int NPC = p.pts * p.cams;
    const int GC = p.G * p.Cg;
    const float *wrow = weights + (size_t)ba * T * p.G + g;
    const float *lrow = loc + (size_t)ba * NPC * 2;
    const Bt *fb = feat + (size_t)b * p.P_total * GC;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(fb, (unsigned)((size_t)p.P_total * GC * elt));
    const int lane_off = (g * p.Cg + s * V) * elt;  // this lane's channels, bytes
    AggRec *rec = s_rec[wv];
    float(*res)[3] = s_res[wv];

    // the lane's logits, round k in lgr[k] (sample k * per_round + lane), read once
    const int per_round = p.npc * p.scales;
    const int lpc = lane / p.scales, lsc = lane - lpc * p.scales;
    float lgr[kRegRounds];
#pragma unroll
    for (int k = 0; k < kRegRounds; ++k) {
        const int pc = k * p.npc + lpc;
        lgr[k] = (lane < per_round && pc < NPC) ? wrow[(size_t)(pc * p.scales + lsc) * p.G] : -INFINITY;
    }
    float mx = 0.0f, inv = 1.0f;
    if (p.softmax) {
        float m = lgr[0];
#pragma unroll
        for (int k = 1; k < kRegRounds; ++k) m = fmaxf(m, lgr[k]);
        mx = wmax(m);
        float e = 0.0f;
#pragma unroll
        for (int k = 0; k < kRegRounds; ++k) e += expf(lgr[k] - mx);
        inv = 1.0f / wsum(e);
    }
    float gc[V];  // this lane's channels s*V .. s*V + V - 1 of G
    unpack<E, V>(*reinterpret_cast<const uint4 *>(gout + (size_t)ba * GC + g * p.Cg + s * V), gc);

    // this lane's location for the round at pc0 (read one round ahead)
    auto fetch = [&](int pc0, float2 &uv) __attribute__((always_inline)) {
        const int pc = pc0 + lpc;
        if (lane < per_round && pc < NPC) uv = *reinterpret_cast<const float2 *>(lrow + 2 * pc);
    };
    float2 uv_next = make_float2(0.0f, 0.0f);
    fetch(0, uv_next);
    float dot = 0.0f;
    for (int pc0 = 0; pc0 < NPC; pc0 += p.npc) {
        const int pc = pc0 + lpc;
        const bool own = lane < per_round && pc < NPC;
        const float lg = lgr[0];
#pragma unroll
        for (int k = 0; k + 1 < kRegRounds; ++k) lgr[k] = lgr[k + 1];
        const float2 uv = uv_next;
        fetch(pc0 + p.npc, uv_next);
        int t_nat = 0;
        float wt = 0.0f;
        if (own) {
            const int cam = pc % p.cams;
            const int cs = cam * p.scales + lsc;
            t_nat = pc * p.scales + lsc;
            wt = p.softmax ? expf(lg - mx) * inv : lg;
            const int Hs = s_h[cs], Ws = s_w[cs];
            const float xf = __fsub_rn(mul_rn(uv.x, (float)Ws), 0.5f);
            const float yf = __fsub_rn(mul_rn(uv.y, (float)Hs), 0.5f);
            int x0, y0;
            AggRec r;
            split_fu(yf, y0, r.fy, r.uy);
            split_fu(xf, x0, r.fx, r.ux);
            const bool vy0 = (unsigned)y0 < (unsigned)Hs, vy1 = (unsigned)(y0 + 1) < (unsigned)Hs;
            const bool vx0 = (unsigned)x0 < (unsigned)Ws, vx1 = (unsigned)(x0 + 1) < (unsigned)Ws;
            const int yc0 = min(max(y0, 0), Hs - 1), yc1 = min(max(y0 + 1, 0), Hs - 1);
            const int xc0 = min(max(x0, 0), Ws - 1), xc1 = min(max(x0 + 1, 0), Ws - 1);
            const int base = s_start[cs];
            r.o00 = (base + yc0 * Ws + xc0) * GC * elt;  // bytes
            r.o01 = (base + yc0 * Ws + xc1) * GC * elt;
            r.o10 = (base + yc1 * Ws + xc0) * GC * elt;
            r.o11 = (base + yc1 * Ws + xc1) * GC * elt;
            r.valid = (vy0 && vx0 ? 1 : 0) | (vy0 && vx1 ? 2 : 0) | (vy1 && vx0 ? 4 : 0) |
                      (vy1 && vx1 ? 8 : 0);
            r.wt = wt;
            r.Ws = (float)Ws;
            r.Hs = (float)Hs;
            rec[lane] = r;
        }
        const int nrec = min(per_round, (NPC - pc0) * p.scales);
        const int iters = (nrec + Z - 1) / Z;
        uint4 cb[2][4];
        // batch it: slice z takes record it*Z + z (record 0 again past the end, unused)
        auto issue = [&](int it, int slot) __attribute__((always_inline)) {
            const int j = it * Z + z;
            const int4 o = *reinterpret_cast<const int4 *>(&rec[j < nrec ? j : 0].o00);
            cb[slot][0] = buffer_load<uint4>(rsrc, o.x + lane_off);
            cb[slot][1] = buffer_load<uint4>(rsrc, o.y + lane_off);
            cb[slot][2] = buffer_load<uint4>(rsrc, o.z + lane_off);
            cb[slot][3] = buffer_load<uint4>(rsrc, o.w + lane_off);
        };
        auto compute = [&](int it, int slot) __attribute__((always_inline)) {
            const int j = it * Z + z;
            float va[V], vb[V], vc[V], ve[V];
            unpack<E, V>(cb[slot][0], va);
            unpack<E, V>(cb[slot][1], vb);
            unpack<E, V>(cb[slot][2], vc);
            unpack<E, V>(cb[slot][3], ve);
            float D00 = 0.0f, D01 = 0.0f, D10 = 0.0f, D11 = 0.0f;
#pragma unroll
            for (int u = 0; u < V; ++u) {
                D00 = fmaf(gc[u], va[u], D00);
                D01 = fmaf(gc[u], vb[u], D01);
                D10 = fmaf(gc[u], vc[u], D10);
                D11 = fmaf(gc[u], ve[u], D11);
            }
            D00 = slice_sum_to_last<S>(D00);
            D01 = slice_sum_to_last<S>(D01);
            D10 = slice_sum_to_last<S>(D10);
            D11 = slice_sum_to_last<S>(D11);
            if (j < nrec && s == S - 1) {
                const AggRec r = rec[j];
                const float d00 = (r.valid & 1) ? D00 : 0.0f, d01 = (r.valid & 2) ? D01 : 0.0f;
                const float d10 = (r.valid & 4) ? D10 : 0.0f, d11 = (r.valid & 8) ? D11 : 0.0f;
                res[j][0] = r.uy * (r.ux * d00 + r.fx * d01) + r.fy * (r.ux * d10 + r.fx * d11);
                res[j][1] = r.wt * r.Ws * (r.uy * (d01 - d00) + r.fy * (d11 - d10));
                res[j][2] = r.wt * r.Hs * (r.ux * (d10 - d00) + r.fx * (d11 - d01));
            }
        };
        // issues are unconditional (past the end they reread record 0): a skipped
        // issue would make the compiler's wait for the current batch also cover the
        // next one
        issue(0, 0);
        for (int it = 0; it < iters; it += 2) {
            issue(it + 1, 1);
            compute(it, 0);
            issue(it + 2, 0);
            if (it + 1 < iters) compute(it + 1, 1);
        }
        if (own) {
            const float gt = res[lane][0];
            dot = fmaf(wt, gt, dot);
            if (p.want_w) gts[(size_t)unit * T + t_nat] = gt;  // contiguous per unit
        }
        if (p.want_loc && lane < p.npc && pc0 + lane < NPC) {
            float su = 0.0f, sv = 0.0f;
            for (int k = 0; k < p.scales; ++k) {
                su += res[lane * p.scales + k][1];
                sv += res[lane * p.scales + k][2];
            }
            float *dst = gloc_part + (((size_t)g * p.BA + ba) * NPC + pc0 + lane) * 2;
            dst[0] = su;
            dst[1] = sv;
        }
    }
    // normalisation and sum_t wt g_t of the unit, for the finishing pass
    const float tot = p.softmax ? wsum(dot) : 0.0f;
    if (lane == 0) {
        us[unit] = mx;
        us[p.nunits + unit] = inv;
        us[2 * p.nunits + unit] = tot;
    }
}

// Finishing pass of the pipelined main kernel, one thread per element of the
// [B*A*T, G] weight layout: wt = exp(l - max) / sum (the main kernel's arithmetic, from
// its per-unit max and 1/sum) or the weight itself; grad_weights = g_t, or
// wt (g_t - sum_j wj g_j) with the softmax; wn = wt for the feature gather. Reads and
// writes run along the layout, so no partial lines are left to other XCDs.
__global__ __launch_bounds__(256) void agg_bwd_finish_kernel(const float *__restrict__ weights,
                                                             const float *__restrict__ gts,
                                                             const float *__restrict__ us,
                                                             float *__restrict__ gw, float *__restrict__ wn,
                                                             long long n, int T, int G, int BA, int softmax) {
    const long long nunits = (long long)G * BA;
    const bool narrow = n < (1LL << 31);  // 32-bit index arithmetic
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
        long long smp, ba;
        int g, t;
        if (narrow) {
            const unsigned s32 = (unsigned)e / (unsigned)G, b32 = s32 / (unsigned)T;
            smp = s32;
            ba = b32;
            g = (int)((unsigned)e - s32 * (unsigned)G);
            t = (int)(s32 - b32 * (unsigned)T);
        } else {
            smp = e / G;
            ba = smp / T;
            g = (int)(e - smp * G);
            t = (int)(smp - ba * T);
        }
        const long long u = (long long)g * BA + ba;
        const float w = weights[e];
        const float wt = softmax ? expf(w - us[u]) * us[nunits + u] : w;
        if (wn) wn[e] = wt;
        if (gw) {
            const float gt = gts[u * T + t];
            gw[e] = softmax ? wt * (gt - us[2 * nunits + u]) : gt;
        }
    }
}

// ------------------------------------------------------ feature buckets --

constexpr int kHashSlots = 2048;  // >= 4 corners x 256 samples per block, load <= 1/2
constexpr unsigned kNoKey = 0xffffffffu;

// Sample index i of the bucket passes, map-major: i = (cs * BA + ba) * pts + point
// for map cs = cam * scales + scale; returns (ba, t) with t the natural sample index
// (point * cams + cam) * scales + scale.
__device__ __forceinline__ void bucket_sample(long long i, const AggBwdParams &p, int &ba, int &t) {
    const int pt = (int)(i % p.pts);
    const long long rest = i / p.pts;
    ba = (int)(rest % p.BA);
    const int cs = (int)(rest / p.BA);
    const int cam = cs / p.scales, sc = cs - cam * p.scales;
    t = (pt * p.cams + cam) * p.scales + sc;
}

// The four corner rows (in [B*P_total)) and bilinear weights of sample (ba, t), with
// the main kernel's position arithmetic; a weight is zero for a corner outside its map.
__device__ __forceinline__ void bucket_corners(const float *__restrict__ loc, const AggBwdParams &p,
                                               const int *s_h, const int *s_w, const int *s_start,
                                               int ba, int t, unsigned (&row)[4], float (&w)[4]) {
    const int pc = t / p.scales, sc = t - pc * p.scales;
    const int cam = pc % p.cams;
    const int cs = cam * p.scales + sc;
    const float2 uv = *reinterpret_cast<const float2 *>(loc + ((size_t)ba * p.pts * p.cams + pc) * 2);
    const int Hs = s_h[cs], Ws = s_w[cs];
    const float xf = __fsub_rn(mul_rn(uv.x, (float)Ws), 0.5f);
    const float yf = __fsub_rn(mul_rn(uv.y, (float)Hs), 0.5f);
    int x0, y0;
    float fy, uy, fx, ux;
    split_fu(yf, y0, fy, uy);
    split_fu(xf, x0, fx, ux);
    const bool vy0 = (unsigned)y0 < (unsigned)Hs, vy1 = (unsigned)(y0 + 1) < (unsigned)Hs;
    const bool vx0 = (unsigned)x0 < (unsigned)Ws, vx1 = (unsigned)(x0 + 1) < (unsigned)Ws;
    w[0] = (vy0 && vx0) ? uy * ux : 0.0f;
    w[1] = (vy0 && vx1) ? uy * fx : 0.0f;
    w[2] = (vy1 && vx0) ? fy * ux : 0.0f;
    w[3] = (vy1 && vx1) ? fy * fx : 0.0f;
    const unsigned r00 = (unsigned)((ba / p.A) * p.P_total + s_start[cs]) + (unsigned)(y0 * Ws + x0);
    row[0] = r00;
    row[1] = r00 + 1u;
    row[2] = r00 + (unsigned)Ws;
    row[3] = r00 + (unsigned)Ws + 1u;
}

// Insert one occurrence of key: returns its slot; *rank = occurrences before it in
// this block.
// Insert (or find) key; the thread that inserts a key appends its slot to `used`.
__device__ __forceinline__ int hash_add(unsigned *keys, unsigned *cnts, unsigned *used,
                                       unsigned *nused, unsigned key, unsigned &rank) {
    int h = (int)((key * 2654435761u) >> 21);  // 11 bits
    for (;;) {
        const unsigned k = keys[h];
        if (k == key) break;
        if (k == kNoKey) {
            const unsigned prev = atomicCAS(&keys[h], kNoKey, key);
            if (prev == kNoKey) {
                used[atomicAdd(nused, 1u)] = (unsigned)h;
                break;
            }
            if (prev == key) break;
        }
        h = (h + 1) & (kHashSlots - 1);
    }
    rank = atomicAdd(&cnts[h], 1u);
    return h;
}

// Count (FILL = false) or file (FILL = true) every corner with a non-zero weight in its
// row's bucket. Per block: merge the corners per row in LDS, then one global atomic
// per row (the count, or the reservation of the block's range in the bucket).
template <bool FILL>
__global__ __launch_bounds__(256) void agg_bucket_kernel(const float *__restrict__ loc,
                                                         unsigned *__restrict__ cnt,
                                                         const unsigned *__restrict__ starts,
                                                         uint2 *__restrict__ entries, AggBwdParams p) {
    __shared__ int s_h[kAggMaxMaps], s_w[kAggMaxMaps], s_start[kAggMaxMaps];
    __shared__ unsigned s_key[kHashSlots], s_cnt[kHashSlots], s_base[kHashSlots];
    __shared__ unsigned s_used[4 * 256], s_nused;  // slots in use (<= 4 corners x 256 samples)
    const int nmaps = p.cams * p.scales;
    for (int i = threadIdx.x; i < nmaps; i += 256) {
        s_h[i] = p.maps.H[i];
        s_w[i] = p.maps.W[i];
        s_start[i] = p.maps.start[i];
    }
    for (int i = threadIdx.x; i < kHashSlots; i += 256) {
        s_key[i] = kNoKey;
        s_cnt[i] = 0;
    }
    if (threadIdx.x == 0) s_nused = 0;
    __syncthreads();
    const int T = p.pts * p.cams * p.scales;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const bool on = i < (long long)p.BA * T;
    int ba = 0, t = 0;
    unsigned row[4];
    float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int slot[4];
    unsigned rank[4];
    if (on) {
        bucket_sample(i, p, ba, t);
        bucket_corners(loc, p, s_h, s_w, s_start, ba, t, row, w);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (w[q] != 0.0f) slot[q] = hash_add(s_key, s_cnt, s_used, &s_nused, row[q], rank[q]);
    }
    __syncthreads();
    unsigned *fill = cnt + (size_t)p.B * p.P_total;  // fill cursors follow the counts
    // one global atomic per slot in use; the four per thread are issued together
    const int nused = (int)s_nused;
    unsigned hs[4], key[4], n[4], res[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int j = threadIdx.x + 256 * r;
        hs[r] = j < nused ? s_used[j] : 0u;
        key[r] = s_key[hs[r]];
        n[r] = j < nused ? s_cnt[hs[r]] : 0u;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (n[r] == 0) continue;
        if constexpr (FILL) res[r] = atomicAdd(&fill[key[r]], n[r]);
        else atomicAdd(&cnt[key[r]], n[r]);
    }
    if constexpr (FILL) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (n[r] != 0) s_base[hs[r]] = starts[key[r]] + res[r];
    }
    if constexpr (FILL) {
        __syncthreads();
        if (on) {
            const unsigned smp = (unsigned)ba * (unsigned)T + (unsigned)t;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (w[q] != 0.0f) entries[s_base[slot[q]] + rank[q]] = make_uint2(smp, __float_as_uint(w[q]));
        }
    }
}

__global__ __launch_bounds__(256) void agg_u32_zero_kernel(unsigned *__restrict__ p, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        p[i] = 0u;
}

// Exclusive prefix sum of cnt[0..D) into starts in three launches: per-block sums of
// 4096-value chunks (1024 threads, 4 consecutive values each), one block scanning
// those sums, and a second pass over the chunks adding each block's offset.
__device__ __forceinline__ void load4(const unsigned *__restrict__ src, long long b, long long D,
                                      unsigned (&v)[4]) {
    if (b + 3 < D) {
        const uint4 q = *reinterpret_cast<const uint4 *>(src + b);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (b + i < D) ? src[b + i] : 0u;
    }
}

// Block-wide exclusive scan of one value per thread (1024 threads); returns the
// thread's exclusive prefix and the block total in *total.
__device__ __forceinline__ unsigned block_scan(unsigned x, unsigned *s_wave, unsigned &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    unsigned incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const unsigned u = __shfl_up(incl, off, 64);
        if (lane >= off) incl += u;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    unsigned before = 0;
    total = 0;
    for (int w = 0; w < 16; ++w) {
        const unsigned sw = s_wave[w];
        if (w < wave) before += sw;
        total += sw;
    }
    __syncthreads();  // s_wave is reused by the next call
    return before + incl - x;
}

__global__ __launch_bounds__(1024) void agg_scan_sums_kernel(const unsigned *__restrict__ cnt,
                                                             unsigned *__restrict__ bsum, long long D) {
    __shared__ unsigned s_wave[16];
    unsigned v[4];
    load4(cnt, (long long)blockIdx.x * 4096 + 4LL * threadIdx.x, D, v);
    unsigned total;
    block_scan(v[0] + v[1] + v[2] + v[3], s_wave, total);
    if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

__global__ __launch_bounds__(1024) void agg_scan_top_kernel(unsigned *__restrict__ bsum, int nb) {
    __shared__ unsigned s_wave[16];
    unsigned carry = 0;
    for (int c0 = 0; c0 < nb; c0 += 1024) {
        const int i = c0 + (int)threadIdx.x;
        const unsigned x = i < nb ? bsum[i] : 0u;
        unsigned total;
        const unsigned ex = block_scan(x, s_wave, total);
        if (i < nb) bsum[i] = carry + ex;
        carry += total;
    }
}

__global__ __launch_bounds__(1024) void agg_scan_final_kernel(const unsigned *__restrict__ cnt,
                                                              const unsigned *__restrict__ bsum,
                                                              unsigned *__restrict__ starts, long long D) {
    __shared__ unsigned s_wave[16];
    const long long b = (long long)blockIdx.x * 4096 + 4LL * threadIdx.x;
    unsigned v[4];
    load4(cnt, b, D, v);
    unsigned total;
    unsigned run = bsum[blockIdx.x] + block_scan(v[0] + v[1] + v[2] + v[3], s_wave, total);
    if (b + 3 < D) {
        uint4 q;
        q.x = run; run += v[0];
        q.y = run; run += v[1];
        q.z = run; run += v[2];
        q.w = run;
        *reinterpret_cast<uint4 *>(starts + b) = q;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (b + i < D) starts[b + i] = run;
            run += v[i];
        }
    }
}

struct AggGatherParams {
    int GC, Cg, G, T;  // channels per row and per group; groups; samples per anchor
    int CT;            // tiles of 16*V channels per row (<= 4*NB per item)
    int NB;            // tile blocks per row: an item takes 4 tiles
    long long nitems;
    int nblocks;
};

// One wavefront per (feature row, block of up to 4 tiles of 16*V channels): four
// 16-lane groups take every fourth entry of the row's bucket, two entries at a time;
// each lane holds V channels of each tile (within one group since Cg % V == 0) and
// sums wt[g] * w_ab * grad_out[anchor]; two shuffles combine the groups and the tile
// is stored once in the dtype (rows outside every map get zeros).
template <class E, int V>
__global__ __launch_bounds__(256) void agg_feat_gather_kernel(
    const typename E::bits *__restrict__ gout, const float *__restrict__ wn,
    const unsigned *__restrict__ starts, const unsigned *__restrict__ cnt,
    const uint2 *__restrict__ entries, typename E::bits *__restrict__ gfeat, AggGatherParams q) {
    const int blk = xcd_remap((int)blockIdx.x, q.nblocks);
    const long long item = (long long)blk * 4 + (threadIdx.x >> 6);
    if (item >= q.nitems) return;  // whole wavefronts; no barrier in this kernel
    const int lane = threadIdx.x & 63, grp = lane >> 4, l = lane & 15;
    const long long row = item / q.NB;
    const int tb = (int)(item - row * q.NB);
    int cc[4], gg[4];
    bool has[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = ((tb * 4 + k) * 16 + l) * V;
        has[k] = (tb * 4 + k) < q.CT && c < q.GC;
        cc[k] = has[k] ? c : 0;
        gg[k] = cc[k] / q.Cg;
    }
    const unsigned b0 = starts[row], e = b0 + cnt[row];
    float acc[4][V];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int u = 0; u < V; ++u) acc[k][u] = 0.0f;
    auto add = [&](const uint2 en) {
        const unsigned smp = en.x;
        const float w = __uint_as_float(en.y);
        const unsigned ba = smp / (unsigned)q.T;
        const typename E::bits *gr = gout + (size_t)ba * q.GC;
        const float *wr = wn + (size_t)smp * q.G;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (!has[k]) continue;
            const float coef = w * wr[gg[k]];
            float gv[V];
            load_f32<E, V>(gr + cc[k], gv);
#pragma unroll
            for (int u = 0; u < V; ++u) acc[k][u] = fmaf(coef, gv[u], acc[k][u]);
        }
    };
    unsigned i = b0 + grp;
    for (; i + 4 < e; i += 8) {
        const uint2 e0 = entries[i], e1 = entries[i + 4];
        add(e0);
        add(e1);
    }
    if (i < e) add(entries[i]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int u = 0; u < V; ++u) {
            acc[k][u] += __shfl_xor(acc[k][u], 16, 64);
            acc[k][u] += __shfl_xor(acc[k][u], 32, 64);
        }
    if (grp == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (has[k]) store_f32<E, V>(gfeat + (size_t)row * q.GC + cc[k], acc[k]);
    }
}

// grad_loc = sum over groups (in group order) of the per-group partials.
__global__ __launch_bounds__(256) void agg_loc_reduce_kernel(const float *__restrict__ part,
                                                             float *__restrict__ gloc, long long n,
                                                             int G) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float s = 0.0f;
    for (int g = 0; g < G; ++g) s += part[(size_t)g * n + i];
    gloc[i] = s;
}

__global__ __launch_bounds__(256) void agg_zero_kernel(float *__restrict__ dst, long long n) {
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = 0.0f;
}

template <class E>
__global__ __launch_bounds__(256) void agg_round_kernel(const float *__restrict__ src,
                                                        typename E::bits *__restrict__ dst,
                                                        long long n) {
    const long long stride = (long long)gridDim.x * 256;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        dst[i] = from_f32(E{}, src[i]);
}

int grid_for(long long n) {
    const long long b = (n + 255) / 256;
    return (int)(b < 1 ? 1 : (b > 16384 ? 16384 : b));
}

template <class E>
hipError_t launch_e(const AggBwdLaunch &a, const AggBwdPlan &pl, hipStream_t stream) {
    AggBwdParams p;
    p.B = a.B; p.P_total = a.P_total; p.A = a.A; p.pts = a.pts; p.cams = a.cams;
    p.scales = a.scales; p.G = a.G; p.Cg = a.Cg; p.softmax = a.softmax ? 1 : 0;
    p.maps = a.maps;
    constexpr int elt = (int)sizeof(typename E::bits);
    int V = 4;  // channel vector of the corner loads: V | Cg, feat 4*V-byte aligned
    while (V > 1 && (a.Cg % V != 0 || ((uintptr_t)a.feat % (V * elt)) != 0)) V >>= 1;
    const int lanes = (a.Cg + V - 1) / V;
    int S = 1;
    while (S < lanes && S < 64) S <<= 1;
    p.S = S;
    p.Z = 64 / S;
    p.crounds = (lanes + S - 1) / S;
    p.npc = 64 / a.scales;
    p.BA = a.B * a.A;
    p.nunits = p.BA * a.G;
    p.nblocks = (p.nunits + kWaves - 1) / kWaves;
    p.want_feat = a.grad_feat != nullptr;
    p.want_loc = a.grad_loc != nullptr;
    p.want_w = a.grad_weights != nullptr;

    char *ws = static_cast<char *>(a.workspace);
    float *part = a.grad_loc ? reinterpret_cast<float *>(ws + pl.off_loc) : nullptr;
    const long long nfeat = (long long)a.B * a.P_total * a.G * a.Cg;
    const bool bins = a.grad_feat && pl.binned;
    float *gacc = nullptr;
    float *wn = nullptr;
    unsigned *cnt = nullptr, *starts = nullptr;
    uint2 *entries = nullptr;
    const long long nsamp = (long long)p.BA * a.pts * a.cams * a.scales;
    if (bins) {
        wn = reinterpret_cast<float *>(ws + pl.off_wn);
        cnt = reinterpret_cast<unsigned *>(ws + pl.off_cnt);
        starts = reinterpret_cast<unsigned *>(ws + pl.off_starts);
        entries = reinterpret_cast<uint2 *>(ws + pl.off_ent);
        hipLaunchKernelGGL(agg_u32_zero_kernel, dim3(grid_for(2 * pl.D / 4)), dim3(256), 0, stream, cnt,
                           2 * pl.D);
        if (nsamp > 0)
            hipLaunchKernelGGL((agg_bucket_kernel<false>), dim3((unsigned)((nsamp + 255) / 256)), dim3(256),
                               0, stream, a.loc, cnt, (const unsigned *)nullptr, (uint2 *)nullptr, p);
        const int nsb = (int)((pl.D + 4095) / 4096);
        unsigned *bsum = reinterpret_cast<unsigned *>(ws + pl.off_bsum);
        hipLaunchKernelGGL(agg_scan_sums_kernel, dim3(nsb), dim3(1024), 0, stream, cnt, bsum, pl.D);
        hipLaunchKernelGGL(agg_scan_top_kernel, dim3(1), dim3(1024), 0, stream, bsum, nsb);
        hipLaunchKernelGGL(agg_scan_final_kernel, dim3(nsb), dim3(1024), 0, stream, cnt, bsum, starts,
                           pl.D);
        if (nsamp > 0)
            hipLaunchKernelGGL((agg_bucket_kernel<true>), dim3((unsigned)((nsamp + 255) / 256)), dim3(256),
                               0, stream, a.loc, cnt, starts, entries, p);
    } else if (a.grad_feat) {
        gacc = (E::id == DCN_F32) ? static_cast<float *>(a.grad_feat)
                                  : reinterpret_cast<float *>(ws + pl.off_acc);
        hipLaunchKernelGGL(agg_zero_kernel, dim3(grid_for(nfeat / 4)), dim3(256), 0, stream, gacc, nfeat);
    }
    hipError_t err0 = hipGetLastError();
    if (err0 != hipSuccess) return err0;
    using B = typename E::bits;
    if (p.nunits > 0) {  // no anchors: only the (zero) feature gradient is written
        const B *ft = static_cast<const B *>(a.feat);
        const B *go = static_cast<const B *>(a.grad_out);
        const dim3 grid(p.nblocks), block(kThreads);
        // 2-16 channel vectors of 16 bytes per group, no atomics, a workspace and at
        // most kRegRounds rounds of samples: the pipelined kernel, one lane per vector
        constexpr int V16 = 16 / elt;
        const int nv16 = a.Cg % V16 == 0 ? a.Cg / V16 : 0;
        const int rounds = (a.pts * a.cams + p.npc - 1) / p.npc;
        const bool pipe = !gacc && a.workspace && !(a.path & DCN_BWD_GENERAL_MAIN) && rounds <= kRegRounds &&
                          nv16 >= 2 && nv16 <= 16 &&
                          (nv16 & (nv16 - 1)) == 0 && (uintptr_t)a.feat % 16 == 0 &&
                          (uintptr_t)a.grad_out % 16 == 0 &&
                          (long long)a.P_total * a.G * a.Cg * elt < (1LL << 31);
        float *gts = pipe ? reinterpret_cast<float *>(ws + pl.off_gt) : nullptr;
        float *us = pipe ? reinterpret_cast<float *>(ws + pl.off_us) : nullptr;
        if (pipe) {
            switch (nv16) {  // S = nv16 lanes of one 16-byte vector each
                case 2: hipLaunchKernelGGL((agg_bwd_pipe_kernel<E, 2>), grid, block, 0, stream, ft, a.loc, a.weights, go, part, gts, us, p); break;
                case 4: hipLaunchKernelGGL((agg_bwd_pipe_kernel<E, 4>), grid, block, 0, stream, ft, a.loc, a.weights, go, part, gts, us, p); break;
                case 8: hipLaunchKernelGGL((agg_bwd_pipe_kernel<E, 8>), grid, block, 0, stream, ft, a.loc, a.weights, go, part, gts, us, p); break;
                default: hipLaunchKernelGGL((agg_bwd_pipe_kernel<E, 16>), grid, block, 0, stream, ft, a.loc, a.weights, go, part, gts, us, p); break;
            }
            if (a.grad_weights || wn) {
                const long long n = nsamp * a.G;
                hipLaunchKernelGGL(agg_bwd_finish_kernel, dim3(grid_for(n)), dim3(256), 0, stream, a.weights,
                                   gts, us, a.grad_weights, wn, n, a.pts * a.cams * a.scales, a.G, p.BA,
                                   p.softmax);
            }
        } else switch (V) {
            case 4: hipLaunchKernelGGL((agg_bwd_kernel<E, 4>), grid, block, 0, stream, ft, a.loc, a.weights, go, gacc, part, a.grad_weights, wn, p); break;
            case 2: hipLaunchKernelGGL((agg_bwd_kernel<E, 2>), grid, block, 0, stream, ft, a.loc, a.weights, go, gacc, part, a.grad_weights, wn, p); break;
            default: hipLaunchKernelGGL((agg_bwd_kernel<E, 1>), grid, block, 0, stream, ft, a.loc, a.weights, go, gacc, part, a.grad_weights, wn, p); break;
        }
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.grad_loc && p.nunits > 0) {
        const long long nl = (long long)p.BA * a.pts * a.cams * 2;
        hipLaunchKernelGGL(agg_loc_reduce_kernel, dim3((unsigned)((nl + 255) / 256)), dim3(256), 0,
                           stream, part, a.grad_loc, nl, a.G);
    }
    if (bins) {
        AggGatherParams q;
        q.GC = a.G * a.Cg;
        q.Cg = a.Cg;
        q.G = a.G;
        q.T = a.pts * a.cams * a.scales;
        int VG = 4;  // channels per lane: VG | Cg, grad_out and grad_feat VG*elt-byte aligned
        while (VG > 1 && (a.Cg % VG != 0 || ((uintptr_t)a.grad_out % (VG * elt)) != 0 ||
                          ((uintptr_t)a.grad_feat % (VG * elt)) != 0))
            VG >>= 1;
        q.CT = (q.GC + 16 * VG - 1) / (16 * VG);
        q.NB = (q.CT + 3) / 4;
        q.nitems = (long long)a.B * a.P_total * q.NB;
        q.nblocks = (int)((q.nitems + 3) / 4);
        const B *gop = static_cast<const B *>(a.grad_out);
        B *gf = static_cast<B *>(a.grad_feat);
        switch (VG) {
            case 4: hipLaunchKernelGGL((agg_feat_gather_kernel<E, 4>), dim3(q.nblocks), dim3(256), 0, stream, gop, wn, starts, cnt, entries, gf, q); break;
            case 2: hipLaunchKernelGGL((agg_feat_gather_kernel<E, 2>), dim3(q.nblocks), dim3(256), 0, stream, gop, wn, starts, cnt, entries, gf, q); break;
            default: hipLaunchKernelGGL((agg_feat_gather_kernel<E, 1>), dim3(q.nblocks), dim3(256), 0, stream, gop, wn, starts, cnt, entries, gf, q); break;
        }
    } else if constexpr (E::id != DCN_F32) {
        if (a.grad_feat)
            hipLaunchKernelGGL((agg_round_kernel<E>), dim3(grid_for(nfeat / 4)), dim3(256), 0,
                               stream, gacc, static_cast<B *>(a.grad_feat), nfeat);
    }
    return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

void plan_agg_bwd(int B, int P_total, int A, int pts, int cams, int scales, int G, int Cg,
                  dcn_dtype dtype, bool force_atomic, AggBwdPlan &pl) {
    pl = AggBwdPlan();
    const long long T = (long long)pts * cams * scales;
    pl.D = (long long)B * P_total;
    pl.nent = (long long)B * A * T * 4;
    pl.binned = !force_atomic && pl.nent < (1LL << 31) && 2 * pl.D < (1LL << 31) &&
                (long long)B * A * T < (1LL << 31);
    size_t off = 0;
    pl.off_loc = off;
    off = align256(off + (size_t)G * B * A * pts * cams * 2 * sizeof(float));
    pl.off_gt = off;  // g_t per sample, unit-major (pipelined kernel)
    off = align256(off + (size_t)B * A * T * G * sizeof(float));
    pl.off_us = off;  // max, 1/sum and sum_t wt g_t per unit
    off = align256(off + (size_t)3 * G * B * A * sizeof(float));
    if (pl.binned) {
        pl.off_wn = off;
        off = align256(off + (size_t)B * A * T * G * sizeof(float));
        pl.off_cnt = off;
        off = align256(off + (size_t)pl.D * 2 * sizeof(unsigned));
        pl.off_starts = off;
        off = align256(off + (size_t)pl.D * sizeof(unsigned));
        pl.off_bsum = off;
        off = align256(off + (size_t)((pl.D + 4095) / 4096) * sizeof(unsigned));
        pl.off_ent = off;
        off = align256(off + (size_t)pl.nent * 8);
    } else {
        pl.off_acc = off;
        if (dtype != DCN_F32) off = align256(off + (size_t)B * P_total * G * Cg * sizeof(float));
    }
    pl.total = off;
}

hipError_t launch_deform_agg_bwd(const AggBwdLaunch &a, const AggBwdPlan &plan, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_e<EF32>(a, plan, stream);
        case DCN_F16: return launch_e<EF16>(a, plan, stream);
        case DCN_BF16: return launch_e<EBF16>(a, plan, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
