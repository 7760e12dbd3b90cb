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
// grad_offset and grad_mask: one pass over (pixel, group) pairs, as the forward
// (S lanes of V channels per pair, 16-byte vectors where alignment allows): the
// four corner dots are summed over the pair's lanes and kept in LDS; the pair's
// gradients are formed there and stored with contiguous writes.
//
// grad_x is a scatter: every tap adds to four input pixels. fp32 atomic adds are
// slow on this GPU (in global memory and in LDS alike, about 40-340 G adds/s
// depending on coalescing), so the scatter is turned into a gather by sorting the
// samples by destination, and grad_x is written once, without atomics:
//   1. count: each sample (pair, tap) whose bilinear cell has a corner inside the
//      image belongs to the 16x16 destination tile holding the cell's corner
//      (y0+1, x0+1) (its "home"); each block counts its samples per home bin in an
//      LDS hash table and adds one count per distinct bin to the global counters
//      (one atomic per bin and block). A bin is (image, group, tile, sub-bin),
//      the sub-bin telling whether the cell lies on the tile's first row and/or
//      column, i.e. whether it also touches the tile above / to the left.
//   2. scan: exclusive prefix sum over the bins.
//   3. the pair pass above also writes one 16-byte record per sample into its bin
//      (source pixel, cell within the tile, the two scaled offsets, m_k), ranges
//      being reserved the same way, per block and bin.
//   4. gather: one block per destination tile reads its own bin and the first-row /
//      first-column sub-bins of the tiles below and to the right, sorts the
//      records by cell in LDS (a counting sort with integer LDS atomics, which are
//      fast), and every destination pixel sums, in registers, m_k * w * G over the
//      records of the four cells it is a corner of. grad_x is stored once, in the
//      output dtype.
// Sizes beyond the record packing (Ho*Wo >= 2^24 pixels, or 2^31 samples) use a
// fallback: fp32 atomic adds into an accumulator that is then rounded to dtype.
#include "dcn_common.hpp"
#include "internal.hpp"

#include <stdlib.h>

namespace dcn {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;           // destination tile edge (pixels)
constexpr int kCells = kTile + 1;   // cells touching a tile, per axis
constexpr int kGatherCap = 3072;    // records per LDS chunk in the gather

struct BwdParams {
    int N, H, W, G, C, kh, kw, sh, sw, ph, pw, dh, dw, Ho, Wo;
    float offset_scale;
    int softmax, has_mask, vec_io;
    int want_x, want_off, want_mask;
    int dots;  // 0: the pair pass only files the grad_x records (gradients come from the tile kernel)
    int npairs, S, Q, nchunk, PB, nblocks;
    int TY, TX;  // bin grid: tiles per image column / row (floor(H/16)+1, floor(W/16)+1)
    int TXo, otiles;  // tiled pair order: output tiles per row, per image and group
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

__device__ __forceinline__ TapGeo tap_geo(int by, int bx, float2 d, float s, int H, int W) {
    TapGeo t;
    split_coord_fu(by, mul_rn(s, d.y), t.y0, t.fy, t.uy);
    split_coord_fu(bx, mul_rn(s, d.x), t.x0, t.fx, t.ux);
    t.vy0 = (unsigned)t.y0 < (unsigned)H;
    t.vy1 = (unsigned)(t.y0 + 1) < (unsigned)H;
    t.vx0 = (unsigned)t.x0 < (unsigned)W;
    t.vx1 = (unsigned)(t.x0 + 1) < (unsigned)W;
    return t;
}

// Pair index e -> (image n, group g, output pixel pix in [0, Ho*Wo)); false for
// the padding pairs of the tiled order.
// Pixel-major: e = (n*Ho*Wo + pix)*G + g (the memory order of offsets and masks).
// Tiled: e = ((n*TYo*TXo + tile)*G + g)*256 + 16*ly + lx: output pixels in 16x16
// tiles (ragged tiles padded), one group per 256 pairs. A wavefront then takes one
// tap of 4 rows of 16 neighbouring pixels of one group, whose samples fall into
// few destination bins, while the G groups of a tile stay adjacent (with the XCD
// remap of the blocks, in one L2: the groups share the cache lines of offsets,
// x and grad_out).
template <bool TILED>
__device__ __forceinline__ bool decode_pair(int e, const BwdParams &p, int &n, int &g, int &pix) {
    if constexpr (TILED) {
        const int per = (p.otiles * p.G) << 8;
        n = e / per;
        const int rem = e - n * per;
        const int tg = rem >> 8, l = rem & 255;
        const int tile = tg / p.G;
        g = tg - tile * p.G;
        const int oty = tile / p.TXo, otx = tile - oty * p.TXo;
        const int ho = oty * kTile + (l >> 4), wo = otx * kTile + (l & 15);
        pix = ho * p.Wo + wo;
        return ho < p.Ho && wo < p.Wo;
    } else {
        const int P = p.Ho * p.Wo;
        const int pg = e / p.G;
        g = e - pg * p.G;
        n = pg / P;
        pix = pg - n * P;
        return true;
    }
}

// samples per block of the pair pass: PB * K <= 4 * (65536 / (28 * K)) * K < 2344
constexpr int kBinMaxSamples = 2344;

#include "core_bwd_bins.hpp"
static_assert(kBinTile == kTile, "bins and destination tiles share their edge");

// Inclusive prefix sum over a full wavefront (every lane active) without LDS permutes:
// row_shr DPP steps within 16-lane rows, then row_bcast steps carry each row's total
// into the rows above it.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned v) {
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// 1. Samples per home bin. A block takes the 256 pairs of one output tile of one
// group (tiled order) and its samples tap-fastest; it counts them per bin in LDS
// and adds one count per distinct bin to the global counters.
template <int KH, int KW>
__global__ __launch_bounds__(kThreads) void bwd_count_kernel(const float *__restrict__ offset,
                                                             unsigned *__restrict__ counts,
                                                             BwdParams p) {
    __shared__ unsigned s_key[kHash], s_cnt[kHash], s_win[kWinSlots];
    for (int i = threadIdx.x; i < kHash; i += kThreads) {
        s_key[i] = kEmpty;
        s_cnt[i] = 0;
    }
    for (int i = threadIdx.x; i < kWinSlots; i += kThreads) s_win[i] = 0;
    __syncthreads();
    const int kh = KH > 0 ? KH : p.kh, kw = KW > 0 ? KW : p.kw, K = kh * kw;
    const int blk = xcd_remap((int)blockIdx.x, (int)gridDim.x);  // (image, tile, group)
    int n, g, pix0;
    decode_pair<true>(blk * kThreads, p, n, g, pix0);  // local pixel 0 of the tile
    const int tile = (blk / p.G) % p.otiles;
    const int oy = (tile / p.TXo) * kTile, ox = (tile % p.TXo) * kTile;
    const BinWin win = bin_window(oy, ox, p);
    const float2 *od = reinterpret_cast<const float2 *>(offset);
    if constexpr (KH > 0 && KW > 0) {
        // window compiled in: thread = pixel of the tile, its K taps in turn; taps of one
        // pixel mostly share a few bins, so window counts are merged in registers (up to
        // four distinct slots) before the LDS atomics
        const int lq = (int)threadIdx.x;
        const int ho = oy + (lq >> 4), wo = ox + (lq & 15);
        int ms[4] = {-1, -1, -1, -1};
        unsigned mc[4] = {0u, 0u, 0u, 0u};
        if (ho < p.Ho && wo < p.Wo) {
            const float2 *pd = od + (((size_t)n * p.Ho * p.Wo + (size_t)ho * p.Wo + wo) * p.G + g) * K;
            float2 dd[KH * KW];
#pragma unroll
            for (int k = 0; k < KH * KW; ++k) dd[k] = pd[k];
#pragma unroll
            for (int k = 0; k < KH * KW; ++k) {
                const int i = k / KW, j = k - i * KW;
                int y0, x0;
                float f, u;
                split_coord_fu(ho * p.sh - p.ph + i * p.dh, mul_rn(p.offset_scale, dd[k].y), y0, f, u);
                split_coord_fu(wo * p.sw - p.pw + j * p.dw, mul_rn(p.offset_scale, dd[k].x), x0, f, u);
                unsigned bin = 0, local, rank = 0;
                if (!home_bin(y0, x0, n, g, p, bin, local)) continue;
                const int ws = win_slot(y0, x0, win);
                if (ws < 0) {
                    if (block_bin_slot(s_key, s_cnt, bin, rank) == kHash)
                        atomicAdd(&counts[bin], 1u);  // table full: direct
                    continue;
                }
                bool done = false;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (!done && ms[e] == ws) { ++mc[e]; done = true; }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (!done && ms[e] < 0) { ms[e] = ws; mc[e] = 1u; done = true; }
                }
                if (!done) atomicAdd(&s_win[ws], 1u);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (ms[e] >= 0) atomicAdd(&s_win[ms[e]], mc[e]);
    } else
    for (int r = 0; r < K; ++r) {
        const int idx = r * kThreads + (int)threadIdx.x;  // sample: local pair idx/K, tap idx%K
        const int lq = idx / K, k = idx - lq * K;
        const int ho = oy + (lq >> 4), wo = ox + (lq & 15);
        bool want = false;
        unsigned bin = 0, local, rank = 0;
        if (ho < p.Ho && wo < p.Wo) {
            const int i = k / kw, j = k - i * kw;
            const float2 d = od[(((size_t)n * p.Ho * p.Wo + (size_t)ho * p.Wo + wo) * p.G + g) * K + k];
            int y0, x0;
            float f, u;
            split_coord_fu(ho * p.sh - p.ph + i * p.dh, mul_rn(p.offset_scale, d.y), y0, f, u);
            split_coord_fu(wo * p.sw - p.pw + j * p.dw, mul_rn(p.offset_scale, d.x), x0, f, u);
            want = home_bin(y0, x0, n, g, p, bin, local);
            if (want) {
                const int ws = win_slot(y0, x0, win);
                if (ws >= 0) {
                    atomicAdd(&s_win[ws], 1u);
                    want = false;
                }
            }
        }
        if (want && block_bin_slot(s_key, s_cnt, bin, rank) == kHash)
            atomicAdd(&counts[bin], 1u);  // table full: direct
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kHash; i += kThreads)
        if (s_cnt[i]) atomicAdd(&counts[s_key[i]], s_cnt[i]);
    for (int i = threadIdx.x; i < kWinSlots; i += kThreads)
        if (s_win[i]) atomicAdd(&counts[win_bin(i, n, g, win, p)], s_win[i]);
}

// 2. Exclusive prefix sum of nb counts, one block of 1024 threads; starts[nb] =
// total. Chunks of 16384 counts: every 16-byte load of a chunk is issued at once
// into LDS (one memory latency per chunk, where 4096-count steps of dependent loads
// had cost one each), each thread scans its 16 consecutive counts, and the starts
// leave from LDS in 16-byte stores. One 16-byte pad after every four chunk entries
// keeps a thread's run of four entries off its neighbours' LDS banks. counts and
// starts are 16-byte aligned.
constexpr int kScanChunk = 16384;
constexpr int kScanPer = kScanChunk / 1024;  // counts per thread
__global__ __launch_bounds__(1024) void bwd_scan_kernel(const unsigned *__restrict__ counts,
                                                        unsigned *__restrict__ starts, int nb) {
    __shared__ uint4 s_c[kScanChunk / 4 + kScanChunk / 16];
    auto at = [](int q) { return q + (q >> 2); };  // padded index of entry q
    __shared__ unsigned s_wave[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    unsigned carry = 0;
    for (int c0 = 0; c0 < nb; c0 += kScanChunk) {
#pragma unroll
        for (int j = 0; j < kScanPer / 4; ++j) {
            const int q = t + 1024 * j, e = c0 + 4 * q;
            uint4 v;
            if (e + 3 < nb) {
                v = *reinterpret_cast<const uint4 *>(counts + e);
            } else {
                v.x = e < nb ? counts[e] : 0u;
                v.y = e + 1 < nb ? counts[e + 1] : 0u;
                v.z = e + 2 < nb ? counts[e + 2] : 0u;
                v.w = 0u;
            }
            s_c[at(q)] = v;
        }
        __syncthreads();
        uint4 a[kScanPer / 4];
        unsigned sum = 0;
#pragma unroll
        for (int k = 0; k < kScanPer / 4; ++k) {
            a[k] = s_c[at(kScanPer / 4 * t + k)];
            sum += a[k].x + a[k].y + a[k].z + a[k].w;
        }
        unsigned incl = sum;
        incl = wave_incl_scan(incl);
        if (lane == 63) s_wave[wave] = incl;
        __syncthreads();
        unsigned run = carry + incl - sum;
        for (int w = 0; w < wave; ++w) run += s_wave[w];
        unsigned total = carry;
        for (int w = 0; w < 16; ++w) total += s_wave[w];
#pragma unroll
        for (int k = 0; k < kScanPer / 4; ++k) {
            uint4 o;
            o.x = run; run += a[k].x;
            o.y = run; run += a[k].y;
            o.z = run; run += a[k].z;
            o.w = run; run += a[k].w;
            s_c[at(kScanPer / 4 * t + k)] = o;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kScanPer / 4; ++j) {
            const int q = t + 1024 * j, e = c0 + 4 * q;
            const uint4 o = s_c[at(q)];
            if (e + 3 < nb) {
                *reinterpret_cast<uint4 *>(starts + e) = o;
            } else {
                if (e < nb) starts[e] = o.x;
                if (e + 1 < nb) starts[e + 1] = o.y;
                if (e + 2 < nb) starts[e + 2] = o.z;
            }
        }
        carry = total;
        __syncthreads();  // s_c and s_wave are rewritten by the next chunk
    }
    if (t == 0) starts[nb] = carry;
}

// 3. The pair pass: corner dots -> grad_offset, grad_mask; grad_x either as sample
// records (BIN) or as fp32 atomic adds into gacc (fallback).
template <class E, int V, int KH, int KW, bool BIN>
__global__ __launch_bounds__(kThreads) void bwd_pair_kernel(
    const typename E::bits *__restrict__ x, const float *__restrict__ offset,
    const float *__restrict__ mask, const typename E::bits *__restrict__ gout,
    float *__restrict__ gacc, float *__restrict__ goff, float *__restrict__ gmask,
    uint4 *__restrict__ rec, const unsigned *__restrict__ starts, unsigned *__restrict__ fill,
    BwdParams p) {
    extern __shared__ float smem[];
    const int kh = KH > 0 ? KH : p.kh;
    const int kw = KW > 0 ? KW : p.kw;
    const int K = kh * kw;
    const int P = p.Ho * p.Wo;
    float *s_off = smem;               // [PB][K][2] offsets, later grad_offset
    float *s_m = s_off + p.PB * K * 2; // [PB][K] modulation m_k, later grad_mask
    float *s_d = s_m + p.PB * K;       // [PB][K][4] corner dots D_ab

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int pair0 = blk * p.PB;
    const int npb = min(p.PB, p.npairs - pair0);

    // 1. offsets and modulation of the block's pairs -> LDS
    __shared__ int s_pn[BIN ? 256 : 1], s_pg[BIN ? 256 : 1], s_phw[BIN ? 256 : 1];
    if constexpr (BIN) {  // tiled pairs: one 2K-float run per pair
        for (int lq = threadIdx.x; lq < npb; lq += kThreads) {
            int n, g, pix;
            const bool ok = decode_pair<true>(pair0 + lq, p, n, g, pix);
            s_pn[lq] = ok ? n : -1;
            s_pg[lq] = g;
            s_phw[lq] = pix;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < npb * K; idx += kThreads) {
            const int lq = idx / K, k = idx - lq * K;
            const int n = s_pn[lq];
            if (n >= 0) {
                const size_t src = (((size_t)n * P + s_phw[lq]) * p.G + s_pg[lq]) * K + k;
                reinterpret_cast<float2 *>(s_off)[idx] = reinterpret_cast<const float2 *>(offset)[src];
                s_m[idx] = p.has_mask ? mask[src] : (p.softmax ? 0.0f : 1.0f);
            } else {
                reinterpret_cast<float2 *>(s_off)[idx] = make_float2(0.0f, 0.0f);
                s_m[idx] = 0.0f;
            }
        }
    } else {
        block_copy(s_off, offset + (size_t)pair0 * K * 2, npb * K * 2, p.vec_io);
        if (p.has_mask) {
            block_copy(s_m, mask + (size_t)pair0 * K, npb * K, p.vec_io);
        } else {
            for (int i = threadIdx.x; i < npb * K; i += kThreads) s_m[i] = p.softmax ? 0.0f : 1.0f;
        }
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane / p.S, s = lane - q * p.S;
    const int lp = wave * p.Q + q;
    int n = 0, g = 0, pix = 0;
    const bool active = (q < p.Q) && (lp < npb) && decode_pair<BIN>(pair0 + lp, p, n, g, pix);

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

    const int ho = pix / p.Wo, wo = pix - ho * p.Wo;
    const int GC = p.G * p.C;
    float *so = s_off + lp * K * 2;
    float *sm = s_m + lp * K;
    float *sd = s_d + lp * K * 4;
    const int by0 = ho * p.sh - p.ph, bx0 = wo * p.sw - p.pw;

    // 2. corner dots (and, in the fallback, the grad_x atomics). Every lane of a pair
    // runs the same number of channel rounds, so the segment sums see all S lanes.
    if (active && p.dots) {
        const size_t img_base = (size_t)n * p.H * p.W * GC + (size_t)g * p.C;
        const typename E::bits *img = x + img_base;
        float *acc = (!BIN && p.want_x) ? gacc + img_base : nullptr;
        const typename E::bits *gp = gout + ((size_t)n * P + pix) * GC + g * p.C;
        int round = 0;
        for (int ch0 = 0; ch0 < p.nchunk; ch0 += p.S, ++round) {
            const int ch = ch0 + s;
            const bool has = ch < p.nchunk;
            const int chc = has ? ch : 0;
            float gv[V];
            load_f32<E, V>(gp + chc * V, gv);
            if (!has) {
#pragma unroll
                for (int u = 0; u < V; ++u) gv[u] = 0.0f;
            }
            const typename E::bits *imgc = img + chc * V;
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
                if (!BIN && acc && has) {
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
    // grad_x records: one per sample with a corner inside the image, in its home
    // bin. The block first counts its samples per bin in LDS (samples spread over
    // the threads tap-fastest: a table slot, the cell and a rank per sample),
    // reserves one range per bin with a single global atomic, then writes the
    // records; slots are checked against the count pass (same arithmetic).
    if constexpr (BIN) {
        if (p.want_x) {
            __shared__ unsigned s_key[kHash], s_cnt[kHash], s_base[kHash], s_lim[kHash];
            __shared__ unsigned s_wcnt[kWinSlots], s_wbase[kWinSlots], s_wlim[kWinSlots];
            __shared__ unsigned s_sr[kBinMaxSamples];  // slot << 20 | cell << 12 | rank
            for (int i = threadIdx.x; i < kHash; i += kThreads) {
                s_key[i] = kEmpty;
                s_cnt[i] = 0;
            }
            for (int i = threadIdx.x; i < kWinSlots; i += kThreads) s_wcnt[i] = 0;
            __syncthreads();
            // the bin window applies when the block's pairs are one (image, tile, group)
            const int unit = pair0 >> 8;
            const bool use_win = (unit == ((pair0 + npb - 1) >> 8));
            const int ug = unit % p.G, un = (unit / p.G) / p.otiles, utile = (unit / p.G) % p.otiles;
            const BinWin win = bin_window((utile / p.TXo) * kTile, (utile % p.TXo) * kTile, p);
            const int ns = npb * K;  // <= kBinMaxSamples (the host caps PB * K)
            for (int idx = threadIdx.x; idx < ns; idx += kThreads) {
                const int lq = idx / K, k = idx - lq * K;
                const int nn = s_pn[lq];
                unsigned code = 0xffffffffu;
                if (nn >= 0) {
                    const int gg = s_pg[lq], pp = s_phw[lq];
                    const int ho2 = pp / p.Wo, wo2 = pp - ho2 * p.Wo;
                    const int i = k / kw, j = k - i * kw;
                    const float2 d = reinterpret_cast<const float2 *>(s_off)[idx];
                    int y0, x0;
                    float f, u;
                    split_coord_fu(ho2 * p.sh - p.ph + i * p.dh, mul_rn(p.offset_scale, d.y), y0, f, u);
                    split_coord_fu(wo2 * p.sw - p.pw + j * p.dw, mul_rn(p.offset_scale, d.x), x0, f, u);
                    unsigned bin, local, rank = 0;
                    if (home_bin(y0, x0, nn, gg, p, bin, local)) {
                        const int ws = use_win ? win_slot(y0, x0, win) : -1;
                        if (ws >= 0) {
                            rank = atomicAdd(&s_wcnt[ws], 1u);
                            code = ((unsigned)(kHash + ws) << 20) | (local << 12) | rank;
                        } else {
                            const int slot = block_bin_slot(s_key, s_cnt, bin, rank);
                            if (slot < kHash) {
                                code = ((unsigned)slot << 20) | (local << 12) | rank;
                            } else {  // table full: reserve directly
                                const unsigned at = starts[bin] + atomicAdd(&fill[bin], 1u);
                                if (at < starts[bin + 1])
                                    rec[at] = make_uint4(((unsigned)pp << 8) | local,
                                                         __float_as_uint(mul_rn(p.offset_scale, d.y)),
                                                         __float_as_uint(mul_rn(p.offset_scale, d.x)),
                                                         __float_as_uint(s_m[idx]));
                            }
                        }
                    }
                }
                s_sr[idx] = code;
            }
            __syncthreads();
            for (int i = threadIdx.x; i < kHash; i += kThreads) {
                if (s_cnt[i]) {
                    const unsigned key = s_key[i];
                    s_base[i] = starts[key] + atomicAdd(&fill[key], s_cnt[i]);
                    s_lim[i] = starts[key + 1];
                }
            }
            for (int i = threadIdx.x; i < kWinSlots; i += kThreads) {
                if (s_wcnt[i]) {
                    const unsigned key = win_bin(i, un, ug, win, p);
                    s_wbase[i] = starts[key] + atomicAdd(&fill[key], s_wcnt[i]);
                    s_wlim[i] = starts[key + 1];
                }
            }
            __syncthreads();
            for (int idx = threadIdx.x; idx < ns; idx += kThreads) {
                const unsigned code = s_sr[idx];
                if (code == 0xffffffffu) continue;
                const int slot = (int)(code >> 20);
                const float2 d = reinterpret_cast<const float2 *>(s_off)[idx];
                const unsigned base = slot < kHash ? s_base[slot] : s_wbase[slot - kHash];
                const unsigned lim = slot < kHash ? s_lim[slot] : s_wlim[slot - kHash];
                const unsigned at = base + (code & 0xfffu);
                if (at < lim)
                    rec[at] = make_uint4(((unsigned)s_phw[idx / K] << 8) | ((code >> 12) & 0xffu),
                                         __float_as_uint(mul_rn(p.offset_scale, d.y)),
                                         __float_as_uint(mul_rn(p.offset_scale, d.x)),
                                         __float_as_uint(s_m[idx]));
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
    if constexpr (BIN) {
        for (int idx = threadIdx.x; idx < npb * K; idx += kThreads) {
            const int lq = idx / K, k = idx - lq * K;
            const int nn = s_pn[lq];
            if (nn < 0) continue;
            const size_t dst = (((size_t)nn * P + s_phw[lq]) * p.G + s_pg[lq]) * K + k;
            if (p.want_off)
                reinterpret_cast<float2 *>(goff)[dst] = reinterpret_cast<const float2 *>(s_off)[idx];
            if (p.want_mask) gmask[dst] = s_m[idx];
        }
    } else {
        if (p.want_off) block_copy(goff + (size_t)pair0 * K * 2, s_off, npb * K * 2, p.vec_io);
        if (p.want_mask) block_copy(gmask + (size_t)pair0 * K, s_m, npb * K, p.vec_io);
    }
}

struct GatherParams {
    int N, G, C, H, W, Ho, Wo;
    int TY, TX;    // bin grid
    int TYr, TXr;  // destination tiles (ceil(H/16), ceil(W/16))
    int S, nchunk, nblocks;
};

// 4. grad_x of one destination tile (image n, group g, 16x16 pixels) from the
// records of the cells touching it. Threads: 256 pixels x S channel lanes. Per LDS
// chunk of records: load them, counting-sort them by cell, then every destination
// pixel walks the records of the four cells it is a corner of.
template <class E, int V>
__global__ __launch_bounds__(1024) void bwd_gather_kernel(const uint4 *__restrict__ rec,
                                                          const unsigned *__restrict__ starts,
                                                          const typename E::bits *__restrict__ gout,
                                                          typename E::bits *__restrict__ gx,
                                                          GatherParams q) {
    __shared__ float4 s_w[kGatherCap];      // cell-sorted: the four corner weights m*w_ab
    __shared__ unsigned s_src[kGatherCap];  // cell-sorted: source pixel of the record
    __shared__ unsigned short s_cell[kGatherCap];
    __shared__ unsigned s_cnt[kCells * kCells];
    __shared__ unsigned s_pos[kCells * kCells];
    __shared__ unsigned s_fill[kCells * kCells];

    const int nthreads = kTile * kTile * q.S;
    const int tid = threadIdx.x;
    const int blk = xcd_remap((int)blockIdx.x, q.nblocks);
    // block order (image, tile, group): the groups of a tile share an L2
    const int g = blk % q.G;
    const int t1 = blk / q.G;
    const int ntile = q.TYr * q.TXr;
    const int n = t1 / ntile;
    const int tile = t1 - n * ntile;
    const int tyi = tile / q.TXr, txi = tile - tyi * q.TXr;
    const int ng = n * q.G + g;

    // record ranges: own bin (4 sub-bins), first-row sub-bins of the tile below,
    // first-column sub-bins of the tile to the right, the corner sub-bin of the tile
    // below-right; each with the shift of its cells into this tile's cell grid
    int rb[5], re[5], sy[5], sx[5];
    {
        auto base = [&](int yy, int xx) { return ((ng * q.TY + yy) * q.TX + xx) << 2; };
        const int own = base(tyi, txi);
        rb[0] = (int)starts[own]; re[0] = (int)starts[own + 4]; sy[0] = 0; sx[0] = 0;
        for (int r = 1; r < 5; ++r) { rb[r] = re[r] = 0; sy[r] = sx[r] = 0; }
        if (tyi + 1 < q.TY) {
            const int d = base(tyi + 1, txi);
            rb[1] = (int)starts[d + 1]; re[1] = (int)starts[d + 2]; sy[1] = kTile;
            rb[2] = (int)starts[d + 3]; re[2] = (int)starts[d + 4]; sy[2] = kTile;
        }
        if (txi + 1 < q.TX) {
            const int r = base(tyi, txi + 1);
            rb[3] = (int)starts[r + 2]; re[3] = (int)starts[r + 4]; sx[3] = kTile;
        }
        if (tyi + 1 < q.TY && txi + 1 < q.TX) {
            const int dr = base(tyi + 1, txi + 1);
            rb[4] = (int)starts[dr + 3]; re[4] = (int)starts[dr + 4]; sy[4] = kTile; sx[4] = kTile;
        }
    }
    int total = 0;
    for (int r = 0; r < 5; ++r) total += re[r] - rb[r];

    const int dp = tid / q.S, s = tid - dp * q.S;
    const int qy = dp / kTile, qx = dp - qy * kTile;
    const int Y = tyi * kTile + qy, X = txi * kTile + qx;
    const bool inside = Y < q.H && X < q.W;
    const int GC = q.G * q.C;
    const size_t gbase = (size_t)n * q.Ho * q.Wo * GC + (size_t)g * q.C;

    for (int ch0 = 0; ch0 < q.nchunk; ch0 += q.S) {
        const int ch = ch0 + s;
        const bool has = ch < q.nchunk;
        float acc[V];
#pragma unroll
        for (int u = 0; u < V; ++u) acc[u] = 0.0f;
        for (int c0 = 0; c0 < total; c0 += kGatherCap) {
            const int nrec = min(kGatherCap, total - c0);
            __syncthreads();  // the previous chunk's readers are done
            for (int i = tid; i < kCells * kCells; i += nthreads) {
                s_cnt[i] = 0;
                s_fill[i] = 0;
            }
            __syncthreads();
            // record r of this chunk -> its place in the five ranges
            auto locate = [&](int r, int &k, int &gi) {
                gi = c0 + r;
                k = 0;
                while (k < 4 && gi >= re[k] - rb[k]) {
                    gi -= re[k] - rb[k];
                    ++k;
                }
            };
            for (int r = tid; r < nrec; r += nthreads) {
                int k, gi;
                locate(r, k, gi);
                const unsigned vx = rec[rb[k] + gi].x;
                const int cy = (int)((vx >> 4) & 15u) + sy[k];
                const int cx = (int)(vx & 15u) + sx[k];
                const int cell = cy * kCells + cx;
                s_cell[r] = (unsigned short)cell;
                atomicAdd(&s_cnt[cell], 1u);
            }
            __syncthreads();
            if (tid < 64) {  // exclusive scan of the 289 cell counts by one wavefront
                constexpr int kPer = (kCells * kCells + 63) / 64;
                unsigned v[kPer], sum = 0;
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const int c = tid * kPer + i;
                    v[i] = c < kCells * kCells ? s_cnt[c] : 0u;
                    sum += v[i];
                }
                unsigned incl = sum;
                incl = wave_incl_scan(incl);
                unsigned run = incl - sum;
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const int c = tid * kPer + i;
                    if (c < kCells * kCells) s_pos[c] = run;
                    run += v[i];
                }
            }
            __syncthreads();
            // counting sort by cell; each record's four corner weights are formed once
            for (int r = tid; r < nrec; r += nthreads) {
                int k, gi;
                locate(r, k, gi);
                const uint4 v = rec[rb[k] + gi];
                const int cell = s_cell[r];
                const unsigned at = s_pos[cell] + atomicAdd(&s_fill[cell], 1u);
                int cyy, cxx;
                float fy, uy, fx, ux;
                split_coord_fu(0, __uint_as_float(v.y), cyy, fy, uy);
                split_coord_fu(0, __uint_as_float(v.z), cxx, fx, ux);
                const float m = __uint_as_float(v.w);
                const float my0 = m * uy, my1 = m * fy;
                s_w[at] = make_float4(my0 * ux, my0 * fx, my1 * ux, my1 * fx);
                s_src[at] = v.x >> 8;
            }
            __syncthreads();
            if (inside && has) {
                const float *sw = reinterpret_cast<const float *>(s_w);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        // the cell whose corner (a, b) is this pixel
                        const int cell = (qy + 1 - a) * kCells + (qx + 1 - b);
                        const int i0 = (int)s_pos[cell], i1 = i0 + (int)s_cnt[cell];
                        for (int i = i0; i < i1; ++i) {
                            const float w = sw[4 * i + 2 * a + b];
                            float gv[V];
                            load_f32<E, V>(gout + gbase + (size_t)s_src[i] * GC + ch * V, gv);
#pragma unroll
                            for (int u = 0; u < V; ++u) acc[u] = fmaf(w, gv[u], acc[u]);
                        }
                    }
                }
            }
        }
        if (inside && has)
            store_f32<E, V>(gx + ((size_t)(n * q.H + Y) * q.W + X) * GC + g * q.C + ch * V, acc);
    }
}

// Clear n 32-bit words (vectorised when dst is 16-byte aligned).
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

// Round the fp32 accumulator into the fp16/bf16 gradient (fallback path), 8
// elements per step where both ends allow it.
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

// Widest vector (16, 8, 4, 2 bytes) dividing C that both pointers are aligned to.
template <class E>
int pick_vec(int C, const void *p0, const void *p1) {
    constexpr int elt = (int)sizeof(typename E::bits);
    int V = 16 / elt;
    while (V > 1 && (C % V != 0 || ((uintptr_t)p0 % (V * elt)) != 0 ||
                     (p1 && ((uintptr_t)p1 % (V * elt)) != 0)))
        V >>= 1;
    return V;
}

template <class E, int V, bool BIN>
hipError_t launch_pair(const CoreBwdLaunch &a, const BwdParams &p, float *gacc, uint4 *rec,
                       const unsigned *starts, unsigned *fill, hipStream_t stream) {
    const int K = a.kh * a.kw;
    const size_t lds = (size_t)p.PB * K * 7 * sizeof(float);
    const dim3 grid(p.nblocks), block(kThreads);
    using B = typename E::bits;
    const B *x = static_cast<const B *>(a.x);
    const B *go = static_cast<const B *>(a.grad_out);
    if (a.kh == 3 && a.kw == 3)
        hipLaunchKernelGGL((bwd_pair_kernel<E, V, 3, 3, BIN>), grid, block, lds, stream, x,
                           a.offset, a.mask, go, gacc, a.grad_offset, a.grad_mask, rec, starts,
                           fill, p);
    else
        hipLaunchKernelGGL((bwd_pair_kernel<E, V, 0, 0, BIN>), grid, block, lds, stream, x,
                           a.offset, a.mask, go, gacc, a.grad_offset, a.grad_mask, rec, starts,
                           fill, p);
    return hipGetLastError();
}

template <class E, bool BIN>
hipError_t launch_pair_v(int V, const CoreBwdLaunch &a, const BwdParams &p, float *gacc,
                         uint4 *rec, const unsigned *starts, unsigned *fill, hipStream_t stream) {
    constexpr int elt = (int)sizeof(typename E::bits);
    switch (V) {
        case 8:
            if constexpr (elt == 2) return launch_pair<E, 8, BIN>(a, p, gacc, rec, starts, fill, stream);
            break;
        case 4: return launch_pair<E, 4, BIN>(a, p, gacc, rec, starts, fill, stream);
        case 2: return launch_pair<E, 2, BIN>(a, p, gacc, rec, starts, fill, stream);
        default: return launch_pair<E, 1, BIN>(a, p, gacc, rec, starts, fill, stream);
    }
    return hipErrorInvalidValue;
}

// The gather for a group slice of one or two 16-byte chunks (C * elt = 16 or 32: the
// lane of a pixel owns one chunk). The cell sort also copies each record's grad_out
// slice into LDS, so the four destination pixels of a record read it from LDS instead
// of each fetching it from memory; records pass in chunks of kStageCap (three blocks
// fit a CU).
constexpr int kStageCap = 992;

template <class E, int NCH>
__global__ __launch_bounds__(256 * NCH) void bwd_gather_staged_kernel(
    const uint4 *__restrict__ rec, const unsigned *__restrict__ starts,
    const typename E::bits *__restrict__ gout, typename E::bits *__restrict__ gx, GatherParams q) {
    constexpr int V = 16 / (int)sizeof(typename E::bits);
    __shared__ uint4 s_g[kStageCap][NCH];   // cell-sorted: the record's grad_out slice
    __shared__ float4 s_w[kStageCap];       // cell-sorted: the four corner weights m*w_ab
    __shared__ unsigned s_cnt[kCells * kCells];
    __shared__ unsigned s_pos[kCells * kCells];
    __shared__ unsigned s_fill[kCells * kCells];

    constexpr int nthreads = kTile * kTile * NCH;
    constexpr int kRecPer = (kStageCap + nthreads - 1) / nthreads;  // records per thread and chunk
    const int tid = threadIdx.x;
    const int blk = xcd_remap((int)blockIdx.x, q.nblocks);
    const int g = blk % q.G;
    const int t1 = blk / q.G;
    const int ntile = q.TYr * q.TXr;
    const int n = t1 / ntile;
    const int tile = t1 - n * ntile;
    const int tyi = tile / q.TXr, txi = tile - tyi * q.TXr;
    const int ng = n * q.G + g;

    int rb[5], re[5], sy[5], sx[5];
    {
        auto base = [&](int yy, int xx) { return ((ng * q.TY + yy) * q.TX + xx) << 2; };
        const int own = base(tyi, txi);
        rb[0] = (int)starts[own]; re[0] = (int)starts[own + 4]; sy[0] = 0; sx[0] = 0;
        for (int r = 1; r < 5; ++r) { rb[r] = re[r] = 0; sy[r] = sx[r] = 0; }
        if (tyi + 1 < q.TY) {
            const int d = base(tyi + 1, txi);
            rb[1] = (int)starts[d + 1]; re[1] = (int)starts[d + 2]; sy[1] = kTile;
            rb[2] = (int)starts[d + 3]; re[2] = (int)starts[d + 4]; sy[2] = kTile;
        }
        if (txi + 1 < q.TX) {
            const int r = base(tyi, txi + 1);
            rb[3] = (int)starts[r + 2]; re[3] = (int)starts[r + 4]; sx[3] = kTile;
        }
        if (tyi + 1 < q.TY && txi + 1 < q.TX) {
            const int dr = base(tyi + 1, txi + 1);
            rb[4] = (int)starts[dr + 3]; re[4] = (int)starts[dr + 4]; sy[4] = kTile; sx[4] = kTile;
        }
    }
    int total = 0;
    for (int r = 0; r < 5; ++r) total += re[r] - rb[r];

    const int dp = tid / NCH, s = tid - dp * NCH;
    const int qy = dp / kTile, qx = dp - qy * kTile;
    const int Y = tyi * kTile + qy, X = txi * kTile + qx;
    const bool inside = Y < q.H && X < q.W;
    const int GC = q.G * q.C;
    const size_t gbase = (size_t)n * q.Ho * q.Wo * GC + (size_t)g * q.C;
    float acc[V];
#pragma unroll
    for (int u = 0; u < V; ++u) acc[u] = 0.0f;

    // record r of the chunk at c0: its run k (own bin or a neighbour's sub-bin) and
    // index gi in that run
    auto locate = [&](int c0, int r, int &k, int &gi) {
        gi = c0 + r;
        k = 0;
        while (k < 4 && gi >= re[k] - rb[k]) {
            gi -= re[k] - rb[k];
            ++k;
        }
    };
    // a chunk's records, loaded one chunk ahead (during the previous chunk's sums) and
    // held in registers through its counting and sorting passes
    uint4 rv[kRecPer];
    int rk[kRecPer];
    auto fetch = [&](int c0) __attribute__((always_inline)) {
        const int nrec = min(kStageCap, total - c0);
#pragma unroll
        for (int j = 0; j < kRecPer; ++j) {
            const int r = tid + j * nthreads;
            rk[j] = 0;
            if (r < nrec) {
                int k, gi;
                locate(c0, r, k, gi);
                rk[j] = k;
                rv[j] = rec[rb[k] + gi];
            }
        }
    };
    if (total > 0) fetch(0);
    for (int c0 = 0; c0 < total; c0 += kStageCap) {
        const int nrec = min(kStageCap, total - c0);
        __syncthreads();  // the previous chunk's readers are done
        for (int i = tid; i < kCells * kCells; i += nthreads) {
            s_cnt[i] = 0;
            s_fill[i] = 0;
        }
        __syncthreads();
        int rcell[kRecPer];
#pragma unroll
        for (int j = 0; j < kRecPer; ++j) {
            const int r = tid + j * nthreads;
            rcell[j] = 0;
            if (r < nrec) {
                const int k = rk[j];
                const unsigned vx = rv[j].x;
                rcell[j] = ((int)((vx >> 4) & 15u) + sy[k]) * kCells + (int)(vx & 15u) + sx[k];
                atomicAdd(&s_cnt[rcell[j]], 1u);
            }
        }
        __syncthreads();
        if (tid < 64) {  // exclusive scan of the 289 cell counts by one wavefront
            constexpr int kPer = (kCells * kCells + 63) / 64;
            unsigned v[kPer], sum = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = tid * kPer + i;
                v[i] = c < kCells * kCells ? s_cnt[c] : 0u;
                sum += v[i];
            }
            unsigned incl = sum;
            incl = wave_incl_scan(incl);
            unsigned run = incl - sum;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int c = tid * kPer + i;
                if (c < kCells * kCells) s_pos[c] = run;
                run += v[i];
            }
        }
        __syncthreads();
        // counting sort by cell: weights, and the grad_out slice fetched once per record
#pragma unroll
        for (int j = 0; j < kRecPer; ++j) {
            const int r = tid + j * nthreads;
            if (r >= nrec) continue;
            const uint4 v = rv[j];
            const int cell = rcell[j];
            const unsigned at = s_pos[cell] + atomicAdd(&s_fill[cell], 1u);
            int cyy, cxx;
            float fy, uy, fx, ux;
            split_coord_fu(0, __uint_as_float(v.y), cyy, fy, uy);
            split_coord_fu(0, __uint_as_float(v.z), cxx, fx, ux);
            const float m = __uint_as_float(v.w);
            const float my0 = m * uy, my1 = m * fy;
            s_w[at] = make_float4(my0 * ux, my0 * fx, my1 * ux, my1 * fx);
            const uint4 *src = reinterpret_cast<const uint4 *>(gout + gbase + (size_t)(v.x >> 8) * GC);
#pragma unroll
            for (int u = 0; u < NCH; ++u) s_g[at][u] = src[u];
        }
        __syncthreads();
        if (c0 + kStageCap < total) fetch(c0 + kStageCap);
        if (inside) {
            const float *sw = reinterpret_cast<const float *>(s_w);
#pragma unroll
            for (int a = 0; a < 2; ++a) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int cell = (qy + 1 - a) * kCells + (qx + 1 - b);
                    const int i0 = (int)s_pos[cell], i1 = i0 + (int)s_cnt[cell];
                    for (int i = i0; i < i1; ++i) {
                        const float w = sw[4 * i + 2 * a + b];
                        float gv[V];
                        unpack<E, V>(s_g[i][s], gv);
#pragma unroll
                        for (int u = 0; u < V; ++u) acc[u] = fmaf(w, gv[u], acc[u]);
                    }
                }
            }
        }
    }
    if (inside)
        store_f32<E, V>(gx + ((size_t)(n * q.H + Y) * q.W + X) * GC + g * q.C + s * V, acc);
}

template <class E>
hipError_t launch_gather(int V, const CoreBwdLaunch &a, const GatherParams &q, const uint4 *rec,
                         const unsigned *starts, hipStream_t stream) {
    constexpr int elt = (int)sizeof(typename E::bits);
    using B = typename E::bits;
    const B *go = static_cast<const B *>(a.grad_out);
    B *gx = static_cast<B *>(a.grad_x);
    const int cbytes = a.C * elt;
    if ((cbytes == 16 || cbytes == 32) && (uintptr_t)go % 16 == 0 && (uintptr_t)gx % 16 == 0 &&
        !(a.path & DCN_BWD_UNSTAGED_GATHER)) {
        const int nch = cbytes / 16;
        const dim3 grid(q.nblocks), block(kTile * kTile * nch);
        if (nch == 2)
            hipLaunchKernelGGL((bwd_gather_staged_kernel<E, 2>), grid, block, 0, stream, rec, starts, go, gx, q);
        else
            hipLaunchKernelGGL((bwd_gather_staged_kernel<E, 1>), grid, block, 0, stream, rec, starts, go, gx, q);
        return hipGetLastError();
    }
    const dim3 grid(q.nblocks), block(kTile * kTile * q.S);
    switch (V) {
        case 8:
            if constexpr (elt == 2)
                hipLaunchKernelGGL((bwd_gather_kernel<E, 8>), grid, block, 0, stream, rec, starts, go, gx, q);
            break;
        case 4: hipLaunchKernelGGL((bwd_gather_kernel<E, 4>), grid, block, 0, stream, rec, starts, go, gx, q); break;
        case 2: hipLaunchKernelGGL((bwd_gather_kernel<E, 2>), grid, block, 0, stream, rec, starts, go, gx, q); break;
        default: hipLaunchKernelGGL((bwd_gather_kernel<E, 1>), grid, block, 0, stream, rec, starts, go, gx, q); break;
    }
    return hipGetLastError();
}

template <class E>
hipError_t launch_e(const CoreBwdLaunch &a, const CoreBwdPlan &pl, hipStream_t stream) {
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
    p.TY = pl.TY;
    p.TX = pl.TX;
    p.TXo = (a.Wo + kTile - 1) / kTile;
    p.otiles = ((a.Ho + kTile - 1) / kTile) * p.TXo;
    const bool bin = a.grad_x && pl.binned;
    p.npairs = bin ? a.N * a.G * p.otiles * 256 : a.N * a.Ho * a.Wo * a.G;
    const int V = pick_vec<E>(a.C, a.x, a.grad_out);
    p.nchunk = a.C / V;
    p.S = p.nchunk < 64 ? p.nchunk : 64;
    const int K = a.kh * a.kw;
    p.Q = 64 / p.S;
    // the block's LDS (7 floats per pair and tap) stays <= 64 KB
    const int qcap = 65536 / (4 * K * 7 * (int)sizeof(float));
    if (p.Q > qcap) p.Q = qcap > 0 ? qcap : 1;
    p.PB = 4 * p.Q;
    p.nblocks = (p.npairs + p.PB - 1) / p.PB;

    // the corner dots feed grad_offset / grad_mask, and in the fallback the grad_x adds
    p.dots = (a.grad_offset || a.grad_mask || !bin) ? 1 : 0;
    char *ws = static_cast<char *>(a.workspace);
    hipError_t err;
    // grad_offset / grad_mask on the forward's LDS halo tiles where a tile plan with one
    // lane per pair applies; that kernel then also files the grad_x records where its
    // variant can, else the pair pass files them (without dots). The atomic fallback
    // keeps the pair pass's dots, which carry its grad_x adds.
    CoreLaunch c;
    c.x = a.x; c.offset = a.offset; c.mask = a.mask; c.out = const_cast<void *>(a.grad_out);
    c.N = a.N; c.H = a.H; c.W = a.W; c.G = a.G; c.C = a.C; c.kh = a.kh; c.kw = a.kw;
    c.sh = a.sh; c.sw = a.sw; c.ph = a.ph; c.pw = a.pw; c.dh = a.dh; c.dw = a.dw;
    c.Ho = a.Ho; c.Wo = a.Wo;
    c.offset_scale = a.offset_scale;
    c.softmax = a.softmax;
    c.dtype = a.dtype;
    c.om_dtype = DCN_F32;
    c.om_plain = true;
    c.off_grp = 2 * K; c.off_pix = a.G * 2 * K; c.mask_grp = K; c.mask_pix = a.G * K;
    CoreTilePlan tp;
    const bool tile = (a.grad_offset || a.grad_mask) && (bin || !a.grad_x) && !(a.path & DCN_BWD_PAIR_PASS) &&
                      a.kh == 3 && a.kw == 3 && plan_core_tile(c, tp) && tp.S == 1;
    if (tile) {
        p.dots = 0;
        p.want_off = 0;
        p.want_mask = 0;
        if (!a.grad_x)
            return launch_dcn_core_bwd_tile(c, tp, a.grad_offset, a.grad_mask, nullptr, nullptr, stream);
    }
    if (bin) {
        unsigned *counts = reinterpret_cast<unsigned *>(ws + pl.off_counts);
        unsigned *starts = reinterpret_cast<unsigned *>(ws + pl.off_starts);
        unsigned *fill = reinterpret_cast<unsigned *>(ws + pl.off_fill);
        uint4 *rec = reinterpret_cast<uint4 *>(ws + pl.off_rec);
        const long long nb = pl.nbins;
        // the counts and the fill cursors lie in [0, off_starts): one clear
        const long long nclr = (long long)(pl.off_starts / 4);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(elementwise_blocks(nclr)), dim3(256), 0, stream,
                           reinterpret_cast<float *>(ws), nclr, 1);
        const dim3 cgrid((unsigned)((p.npairs + kThreads - 1) / kThreads));
        if (a.kh == 3 && a.kw == 3)
            hipLaunchKernelGGL((bwd_count_kernel<3, 3>), cgrid, dim3(kThreads), 0, stream, a.offset, counts, p);
        else
            hipLaunchKernelGGL((bwd_count_kernel<0, 0>), cgrid, dim3(kThreads), 0, stream, a.offset, counts, p);
        hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, stream, counts, starts, (int)nb);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        bool rec_done = false;
        if (tile) {
            const CoreRecArgs ra = {rec, starts, fill, pl.TY, pl.TX};
            if ((err = launch_dcn_core_bwd_tile(c, tp, a.grad_offset, a.grad_mask,
                                                (a.path & DCN_BWD_PAIR_PASS_RECORDS) ? nullptr : &ra, &rec_done,
                                                stream)) != hipSuccess)
                return err;
        }
        if (!rec_done &&
            (err = launch_pair_v<E, true>(V, a, p, nullptr, rec, starts, fill, stream)) != hipSuccess)
            return err;
        GatherParams q;
        q.N = a.N; q.G = a.G; q.C = a.C; q.H = a.H; q.W = a.W; q.Ho = a.Ho; q.Wo = a.Wo;
        q.TY = pl.TY; q.TX = pl.TX; q.TYr = pl.TYr; q.TXr = pl.TXr;
        const int Vg = pick_vec<E>(a.C, a.grad_out, a.grad_x);
        q.nchunk = a.C / Vg;
        q.S = q.nchunk < 4 ? q.nchunk : 4;
        q.nblocks = a.N * a.G * pl.TYr * pl.TXr;
        return launch_gather<E>(Vg, a, q, rec, starts, stream);
    }
    float *gacc = nullptr;
    const long long nx = (long long)a.N * a.H * a.W * a.G * a.C;
    if (a.grad_x) {
        gacc = (E::id == DCN_F32) ? static_cast<float *>(a.grad_x)
                                  : reinterpret_cast<float *>(ws + pl.off_acc);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(elementwise_blocks(nx)), dim3(256), 0, stream,
                           gacc, nx, (int)((uintptr_t)gacc % 16 == 0));
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = launch_pair_v<E, false>(V, a, p, gacc, nullptr, nullptr, nullptr, stream)) != hipSuccess)
        return err;
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

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

void plan_core_bwd(int N, int H, int W, int G, int C, int Ho, int Wo, int K, dcn_dtype dtype,
                   bool force_fallback, CoreBwdPlan &pl) {
    pl = CoreBwdPlan();
    pl.TY = H / kTile + 1;
    pl.TX = W / kTile + 1;
    pl.TYr = (H + kTile - 1) / kTile;
    pl.TXr = (W + kTile - 1) / kTile;
    pl.nbins = (long long)N * G * pl.TY * pl.TX * 4;
    pl.nsamples = (long long)N * Ho * Wo * G * K;
    const long long tiled_pairs = (long long)N * G * ((Ho + kTile - 1) / kTile) *
                                  ((Wo + kTile - 1) / kTile) * kTile * kTile;
    pl.binned = !force_fallback && (long long)Ho * Wo < (1LL << 24) &&
                pl.nsamples < (1LL << 31) && pl.nbins < (1LL << 30) && tiled_pairs < (1LL << 31);
    if (pl.binned) {
        size_t off = 0;
        pl.off_counts = off;
        off += (size_t)pl.nbins * 4 + 4;  // counts, then one spare word
        off = (off + 15) / 16 * 16;
        pl.off_fill = off;
        off += (size_t)pl.nbins * 4;
        off = align256(off);              // [0, off_starts) is cleared at once
        pl.off_starts = off;
        off += (size_t)pl.nbins * 4 + 4;
        off = align256(off);
        pl.off_rec = off;
        off += (size_t)pl.nsamples * 16;
        pl.total = align256(off);
    } else {
        pl.off_acc = 0;
        pl.total = dtype == DCN_F32 ? 0 : align256((size_t)N * H * W * G * C * 4);
    }
}

hipError_t launch_dcn_core_bwd(const CoreBwdLaunch &a, const CoreBwdPlan &plan, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_F32: return launch_e<EF32>(a, plan, stream);
        case DCN_F16: return launch_e<EF16>(a, plan, stream);
        case DCN_BF16: return launch_e<EBF16>(a, plan, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace dcn
