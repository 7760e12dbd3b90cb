// DCNv2 backward (NCHW) for gfx950: gradients w.r.t. x, offsets, masks and weight.
//
// The derivative of the modulated deformable convolution ("DCNv2 in YOLOv5",
// cyqw.cn, section 1; bilinear kernel from "Hands-on DCNv1 in PyTorch",
// agent.csdn.net, section 2; the pages print no backward pass). With the forward's
// columns col[p][r] = m_k(p) * bilinear(x[n,ci], pos_k(p)), r = k*Cin_pad + ci:
//   grad_weight[co][r] = sum_p grad_out[p][co] * col[p][r]      MFMA GEMM, split over p
//   gcol[p][r]         = sum_co grad_out[p][co] * weight[co][r]  MFMA GEMM
// and the sampling derivative of every column entry with upstream value gcol:
//   grad_mask, grad_offset: per (pixel, group, tap) the dots of gcol with the four
//     corner vectors, reduced over the group's channels;
//   grad_x: every (pixel, tap) adds m * w_ab * gcol[p][k, :] to its four corners.
//     This scatter runs as a gather: the (sample, coefficient) entries are bucketed
//     by destination (image pixel, group) with a count, a scan and a fill, then each
//     destination sums its bucket's gcol rows into registers and stores once.
// Launches (caller's stream, no host synchronisation):
//   1. x -> xt [N,H,W,Cin_pad] and grad_out -> gcl [Pp][CoK] (the shared transpose),
//      goT [CoM][Pp] (grad_out with the batch folded into the pixel axis), wT [Rr][CoK]
//   2. colT [Rr][Pp]: the forward's columns, rounded to the dtype, transposed
//   3. gcol = gcl x wT^T (fp32)   4. grad_weight partials = goT x colT^T   5. their sum
//   6. clear the bucket counters  7. count  8. scan
//   9. sample pass: grad_offset, grad_mask and the bucket entries
//  10. destination gather into gx_cl [N,H,W,Cin_pad] fp32  11. transpose to grad_x.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

#include "v2_shared.hpp"

constexpr int kB = 256;

struct V2bGeo {
    int N, H, W, Ho, Wo, kh, kw, sh, sw, ph, pw, dh, dw, dg, K;
    long long P;
    int has_mask, softmax;
};

// Corner geometry of tap k of output pixel r (image n) in deformable group g: the
// corner (y0, x0), fractions f and exact complements u (split_coord_fu), and the
// four corner weights, zero outside the image.
struct V2bTap {
    int y0, x0;
    float fy, fx, uy, ux;
    bool v00, v01, v10, v11;
    float w00, w01, w10, w11;
};

__device__ __forceinline__ V2bTap v2b_tap(const float *__restrict__ offset, const V2bGeo &q, int n,
                                          int r, int g, int k) {
    const int HWo = q.Ho * q.Wo;
    const int ho = r / q.Wo, wo = r - ho * q.Wo;
    const int i = k / q.kw, j = k - i * q.kw;
    const float *o = offset + ((size_t)(n * q.dg + g) * q.K + k) * 2 * HWo + r;
    V2bTap t;
    split_coord_fu(ho * q.sh - q.ph + i * q.dh, o[HWo], t.y0, t.fy, t.uy);
    split_coord_fu(wo * q.sw - q.pw + j * q.dw, o[0], t.x0, t.fx, t.ux);
    const bool vy0 = (unsigned)t.y0 < (unsigned)q.H, vy1 = (unsigned)(t.y0 + 1) < (unsigned)q.H;
    const bool vx0 = (unsigned)t.x0 < (unsigned)q.W, vx1 = (unsigned)(t.x0 + 1) < (unsigned)q.W;
    t.v00 = vy0 && vx0;
    t.v01 = vy0 && vx1;
    t.v10 = vy1 && vx0;
    t.v11 = vy1 && vx1;
    t.w00 = t.v00 ? t.uy * t.ux : 0.0f;
    t.w01 = t.v01 ? t.uy * t.fx : 0.0f;
    t.w10 = t.v10 ? t.fy * t.ux : 0.0f;
    t.w11 = t.v11 ? t.fy * t.fx : 0.0f;
    return t;
}

// Modulation of tap k of (n, g, r): the mask value, its softmax over the K taps, or
// 1 (1/K with softmax) without a mask. mx and inv are the softmax's maximum and
// reciprocal sum (unused otherwise).
__device__ __forceinline__ float v2b_mod(const float *__restrict__ mask, const V2bGeo &q, int n,
                                         int r, int g, int k, float mx, float inv) {
    const int HWo = q.Ho * q.Wo;
    if (!q.has_mask) return q.softmax ? 1.0f / (float)q.K : 1.0f;
    const float v = mask[((size_t)(n * q.dg + g) * q.K + k) * HWo + r];
    return q.softmax ? expf(v - mx) * inv : v;
}

__device__ __forceinline__ void v2b_softmax_stats(const float *__restrict__ mask, const V2bGeo &q,
                                                  int n, int r, int g, float &mx, float &inv) {
    mx = 0.0f;
    inv = 1.0f;
    if (!(q.softmax && q.has_mask)) return;
    const int HWo = q.Ho * q.Wo;
    const float *ml = mask + (size_t)(n * q.dg + g) * q.K * HWo + r;
    mx = -INFINITY;
    for (int k = 0; k < q.K; ++k) mx = fmaxf(mx, ml[(size_t)k * HWo]);
    float sum = 0.0f;
    for (int k = 0; k < q.K; ++k) sum += expf(ml[(size_t)k * HWo] - mx);
    inv = 1.0f / sum;
}

// ------------------------------------------------------------ layout prep --

// goT[co][p] = grad_out[n][co][hw] for p = n*HWo + hw; zero for co >= Cout or p >= P.
// VEC: 8 consecutive pixels per thread (HWo and P multiples of 8, 16-byte aligned rows).
template <bool VEC>
__global__ __launch_bounds__(kB) void v2b_rows_kernel(const uint16_t *__restrict__ gout,
                                                      uint16_t *__restrict__ goT, int Cout, int HWo,
                                                      long long P, long long Pp, long long total) {
    const long long t = (long long)blockIdx.x * kB + threadIdx.x;
    if constexpr (VEC) {
        if (t * 8 >= total) return;
        const long long e = t * 8;
        const long long co = e / Pp, pp = e - co * Pp;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (co < Cout && pp < P) {
            const long long n = pp / HWo, hw = pp - n * HWo;
            v = *reinterpret_cast<const uint4 *>(gout + ((size_t)n * Cout + co) * HWo + hw);
        }
        *reinterpret_cast<uint4 *>(goT + e) = v;
    } else {
        if (t >= total) return;
        const long long co = t / Pp, pp = t - co * Pp;
        uint16_t v = 0;
        if (co < Cout && pp < P) {
            const long long n = pp / HWo, hw = pp - n * HWo;
            v = gout[((size_t)n * Cout + co) * HWo + hw];
        }
        goT[t] = v;
    }
}

// wT[r][co] = weight[co][ci][k] for r = k*Cin_pad + ci; zero for padding entries.
__global__ __launch_bounds__(kB) void v2b_wt_kernel(const uint16_t *__restrict__ w,
                                                    uint16_t *__restrict__ wT, int Cout, int Cin,
                                                    int K, int Cin_pad, int CoK, long long total) {
    const long long t = (long long)blockIdx.x * kB + threadIdx.x;
    if (t >= total) return;
    const int r = (int)(t / CoK), co = (int)(t - (long long)r * CoK);
    const int k = r / Cin_pad, ci = r - k * Cin_pad;
    wT[t] = (co < Cout && k < K && ci < Cin) ? w[((size_t)co * Cin + ci) * K + k] : (uint16_t)0;
}

// ---------------------------------------------------------------- columns --

struct V2bColParams {
    V2bGeo q;
    int Cin_pad, cpg;
    long long Pp;
    int ptiles, nblocks;
};

// colT[k*Cin_pad + c][p] = m_k(p) * bilinear(xt[n,:,:,c], pos_k(p)) rounded to the
// dtype, the forward's column arithmetic (make_tap + accumulate_tap). A block takes 64
// pixels x one tap x 64 channels: 512 (pixel, 8-channel) items into an LDS tile, then
// 64 rows of 64 pixels (128 bytes) out. Pixels p >= P get zero columns.
template <class E>
__global__ __launch_bounds__(kB) void v2b_colT_kernel(const uint16_t *__restrict__ xt,
                                                      const float *__restrict__ offset,
                                                      const float *__restrict__ mask,
                                                      uint16_t *__restrict__ colT, V2bColParams c) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
    const V2bGeo &q = c.q;
    const int blk = xcd_remap((int)blockIdx.x, c.nblocks);
    const int pt = blk % c.ptiles, rest = blk / c.ptiles;
    const int k = rest % q.K, ct = rest / q.K;
    const long long p0 = (long long)pt * 64;
    const int HWo = q.Ho * q.Wo;
    for (int it = threadIdx.x; it < 512; it += kB) {
        const int pl = it >> 3, qc = it & 7;
        const long long p = p0 + pl;
        const int c0 = ct * 64 + qc * kVec;
        float acc[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
        if (p < q.P && c0 < c.Cin_pad) {
            const int n = (int)(p / HWo), r = (int)(p - (long long)n * HWo);
            const int g = min(c0 / c.cpg, q.dg - 1);
            float mx, inv;
            v2b_softmax_stats(mask, q, n, r, g, mx, inv);
            const float m = v2b_mod(mask, q, n, r, g, k, mx, inv);
            const int ho = r / q.Wo, wo = r - ho * q.Wo;
            const int i = k / q.kw, j = k - i * q.kw;
            const float *o = offset + ((size_t)(n * q.dg + g) * q.K + k) * 2 * HWo + r;
            int y0, x0;
            float fy, fx;
            split_coord(ho * q.sh - q.ph + i * q.dh, o[HWo], y0, fy);
            split_coord(wo * q.sw - q.pw + j * q.dw, o[0], x0, fx);
            const Tap t = make_tap(y0, x0, fy, fx, m, q.H, q.W, c.Cin_pad);
            accumulate_tap<E, kVec>(xt + (size_t)n * q.H * q.W * c.Cin_pad + c0, t, acc);
        }
#pragma unroll
        for (int e = 0; e < kVec; ++e) tile[qc * kVec + e][pl] = (uint16_t)from_f32(E{}, acc[e]);
    }
    __syncthreads();
    for (int it = threadIdx.x; it < 512; it += kB) {
        const int cr = it >> 3, part = it & 7;
        const int cc = ct * 64 + cr;
        if (cc >= c.Cin_pad) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(&tile[cr][part * kVec]);
        *reinterpret_cast<uint4 *>(colT + (size_t)(k * c.Cin_pad + cc) * c.Pp + p0 + part * kVec) = v;
    }
}

// grad_weight[co][ci][k] = sum over splits of part[s][co][k*Cin_pad + ci]: threads run
// over (co, r) so the partial rows are read contiguously; the writes are strided by K.
__global__ __launch_bounds__(kB) void v2b_wsum_kernel(const float *__restrict__ part,
                                                      float *__restrict__ gw, int Cout, int Cin,
                                                      int K, int Cin_pad, int R, int splits) {
    const long long t = (long long)blockIdx.x * kB + threadIdx.x;
    if (t >= (long long)Cout * R) return;
    const int co = (int)(t / R), r = (int)(t - (long long)co * R);
    const int k = r / Cin_pad, ci = r - k * Cin_pad;
    if (ci >= Cin) return;
    const size_t stride = (size_t)Cout * R;
    float s = 0.0f;
    for (int i = 0; i < splits; ++i) s += part[i * stride + t];
    gw[((size_t)co * Cin + ci) * K + k] = s;
}

// ---------------------------------------------------------------- buckets --

__global__ __launch_bounds__(kB) void v2b_zero_kernel(int *__restrict__ p, long long n) {
    for (long long i = (long long)blockIdx.x * kB + threadIdx.x; i < n; i += (long long)gridDim.x * kB)
        p[i] = 0;
}

// One thread per sample (p, g, k): count the corners that receive a grad_x entry
// (inside the image, weight non-zero) in their destination's bucket.
__global__ __launch_bounds__(kB) void v2b_count_kernel(const float *__restrict__ offset,
                                                       int *__restrict__ cnt, V2bGeo q) {
    const long long t = (long long)blockIdx.x * kB + threadIdx.x;
    if (t >= q.P * q.dg * q.K) return;
    const int k = (int)(t % q.K);
    const long long pg = t / q.K;
    const int g = (int)(pg % q.dg);
    const long long p = pg / q.dg;
    const int HWo = q.Ho * q.Wo;
    const int n = (int)(p / HWo), r = (int)(p - (long long)n * HWo);
    const V2bTap tp = v2b_tap(offset, q, n, r, g, k);
    const size_t base = ((size_t)n * q.H + tp.y0) * q.W + tp.x0;
    if (tp.w00 != 0.0f) atomicAdd(&cnt[base * q.dg + g], 1);
    if (tp.w01 != 0.0f) atomicAdd(&cnt[(base + 1) * q.dg + g], 1);
    if (tp.w10 != 0.0f) atomicAdd(&cnt[(base + q.W) * q.dg + g], 1);
    if (tp.w11 != 0.0f) atomicAdd(&cnt[(base + q.W + 1) * q.dg + g], 1);
}

// Exclusive prefix sum of cnt[0..D) into starts, one block of 1024 threads walking
// chunks of 4096 (4 consecutive values per thread) with a running carry.
__global__ __launch_bounds__(1024) void v2b_scan_kernel(const int *__restrict__ cnt,
                                                        int *__restrict__ starts, long long D) {
    __shared__ int s_wave[16];
    __shared__ int s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (long long c0 = 0; c0 < D; c0 += 4096) {
        const long long b = c0 + 4LL * tid;
        int v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (b + i < D) ? cnt[b + i] : 0;
        const int mine = v[0] + v[1] + v[2] + v[3];
        int incl = mine;  // inclusive scan over the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int u = __shfl_up(incl, off, 64);
            if (lane >= off) incl += u;
        }
        if (lane == 63) s_wave[wave] = incl;
        __syncthreads();
        int wbase = 0;
        for (int w = 0; w < wave; ++w) wbase += s_wave[w];
        const int carry = s_carry;
        int run = carry + wbase + incl - mine;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (b + i < D) starts[b + i] = run;
            run += v[i];
        }
        __syncthreads();  // every thread has read s_wave and s_carry
        if (tid == 1023) s_carry = carry + wbase + incl;
        __syncthreads();
    }
}

// ------------------------------------------------------------ sample pass --

struct V2bSampleParams {
    V2bGeo q;
    int Cin_pad, gbase_mul;  // xt / gcol channel of group g's first channel = g * gbase_mul
    int R;                   // gcol row length
    int L, Z, nchunk;        // lanes per (pixel, group) pair, pairs per wave, 8-channel chunks
    long long npairs;
    int nblocks;
    int want_off, want_mask, want_x;
};

// One (pixel, group) pair per L lanes (Z pairs per wavefront); lanes split the
// group's channels in 8-channel chunks. Per tap: the four corner dots
// D_ab = sum_c gcol[p][k, c] * x[corner_ab, c], reduced over the pair's lanes; then
// grad of the modulation sum_ab w_ab D_ab, the position derivatives with the weights
// applied outside the differences, and the four bucket entries (lanes 0..3, one
// corner each). The taps' modulation gradients wait in LDS for the softmax (lane 0).
template <class E>
__global__ __launch_bounds__(kB) void v2b_sample_kernel(
    const uint16_t *__restrict__ xt, const float *__restrict__ offset, const float *__restrict__ mask,
    const float *__restrict__ gcol, const int *__restrict__ starts, int *__restrict__ fill,
    uint2 *__restrict__ entries, float *__restrict__ goff, float *__restrict__ gmask,
    V2bSampleParams s) {
    __shared__ float s_gm[kB / 4][64];  // L >= 4: at most 64 pairs per block, K <= 64
    const V2bGeo &q = s.q;
    const int blk = xcd_remap((int)blockIdx.x, s.nblocks);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int z = lane / s.L, l = lane - z * s.L;
    const int slot = wave * s.Z + z;
    const long long pr = ((long long)blk * 4 + wave) * s.Z + z;
    const bool active = pr < s.npairs;
    const long long p = active ? pr / q.dg : 0;
    const int g = active ? (int)(pr - p * q.dg) : 0;
    const int HWo = q.Ho * q.Wo;
    const int n = (int)(p / HWo), r = (int)(p - (long long)n * HWo);
    float mx, inv;
    v2b_softmax_stats(mask, q, n, r, g, mx, inv);
    const uint16_t *img = xt + (size_t)n * q.H * q.W * s.Cin_pad + g * s.gbase_mul;
    const float *gc_row = gcol + (size_t)p * s.R + g * s.gbase_mul;
    float dot = 0.0f;
    for (int k = 0; k < q.K; ++k) {
        const V2bTap tp = v2b_tap(offset, q, n, r, g, k);
        const float m = v2b_mod(mask, q, n, r, g, k, mx, inv);
        const int yc0 = min(max(tp.y0, 0), q.H - 1), yc1 = min(max(tp.y0 + 1, 0), q.H - 1);
        const int xc0 = min(max(tp.x0, 0), q.W - 1), xc1 = min(max(tp.x0 + 1, 0), q.W - 1);
        const size_t o00 = ((size_t)yc0 * q.W + xc0) * s.Cin_pad, o01 = ((size_t)yc0 * q.W + xc1) * s.Cin_pad;
        const size_t o10 = ((size_t)yc1 * q.W + xc0) * s.Cin_pad, o11 = ((size_t)yc1 * q.W + xc1) * s.Cin_pad;
        float d00 = 0.0f, d01 = 0.0f, d10 = 0.0f, d11 = 0.0f;
        if (active) {
            const float *gck = gc_row + (size_t)k * s.Cin_pad;
            for (int ch = l; ch < s.nchunk; ch += s.L) {
                const int c = ch * kVec;
                const float4 ga = *reinterpret_cast<const float4 *>(gck + c);
                const float4 gb = *reinterpret_cast<const float4 *>(gck + c + 4);
                const float gv[kVec] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
                float a[kVec], b[kVec], cc[kVec], d[kVec];
                load_f32<E, kVec>(img + o00 + c, a);
                load_f32<E, kVec>(img + o01 + c, b);
                load_f32<E, kVec>(img + o10 + c, cc);
                load_f32<E, kVec>(img + o11 + c, d);
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    d00 = fmaf(gv[e], a[e], d00);
                    d01 = fmaf(gv[e], b[e], d01);
                    d10 = fmaf(gv[e], cc[e], d10);
                    d11 = fmaf(gv[e], d[e], d11);
                }
            }
        }
        for (int off = s.L >> 1; off > 0; off >>= 1) {
            d00 += __shfl_xor(d00, off, 64);
            d01 += __shfl_xor(d01, off, 64);
            d10 += __shfl_xor(d10, off, 64);
            d11 += __shfl_xor(d11, off, 64);
        }
        if (!tp.v00) d00 = 0.0f;
        if (!tp.v01) d01 = 0.0f;
        if (!tp.v10) d10 = 0.0f;
        if (!tp.v11) d11 = 0.0f;
        if (!active) continue;
        const float gm = tp.w00 * d00 + tp.w01 * d01 + tp.w10 * d10 + tp.w11 * d11;
        if (l == 0) {
            s_gm[slot][k] = gm;
            dot += m * gm;
            if (s.want_off) {
                const float gy = tp.ux * (d10 - d00) + tp.fx * (d11 - d01);
                const float gx = tp.uy * (d01 - d00) + tp.fy * (d11 - d10);
                float *go = goff + ((size_t)(n * q.dg + g) * q.K + k) * 2 * HWo + r;
                go[0] = m * gx;
                go[HWo] = m * gy;
            }
        }
        if (s.want_x && l < 4) {
            const float w = l == 0 ? tp.w00 : l == 1 ? tp.w01 : l == 2 ? tp.w10 : tp.w11;
            if (w != 0.0f) {
                const size_t dst = (((size_t)n * q.H + tp.y0 + (l >> 1)) * q.W + tp.x0 + (l & 1)) * q.dg + g;
                const int pos = starts[dst] + atomicAdd(&fill[dst], 1);
                entries[pos] = make_uint2((unsigned)(p * q.K + k), __float_as_uint(m * w));
            }
        }
    }
    if (active && l == 0 && s.want_mask) {
        for (int k = 0; k < q.K; ++k) {
            const float gm = s_gm[slot][k];
            const float v = q.softmax ? v2b_mod(mask, q, n, r, g, k, mx, inv) * (gm - dot) : gm;
            gmask[((size_t)(n * q.dg + g) * q.K + k) * HWo + r] = v;
        }
    }
}

// ----------------------------------------------------- destination gather --

struct V2bGatherParams {
    int dg, cpg, Cin_pad, K, R, CT;
    long long nitems;
    int nblocks;
};

// One wavefront per (image pixel, 256-channel tile), 4 channels per lane: sum the
// bucket's entries coef * gcol[sample's pixel][tap, c..c+3] and store the fp32 sums
// once (channels-last). With several deformable groups each lane walks the bucket of
// its channels' group.
__global__ __launch_bounds__(kB) void v2b_gather_kernel(const float *__restrict__ gcol,
                                                        const int *__restrict__ starts,
                                                        const int *__restrict__ cnt,
                                                        const uint2 *__restrict__ entries,
                                                        float *__restrict__ gx_cl, V2bGatherParams q) {
    const int blk = xcd_remap((int)blockIdx.x, q.nblocks);
    const long long item = (long long)blk * 4 + (threadIdx.x >> 6);
    if (item >= q.nitems) return;  // no barrier in this kernel
    const int lane = threadIdx.x & 63;
    const long long pix = item / q.CT;
    const int ct = (int)(item - pix * q.CT);
    const int c = ct * 256 + lane * 4;
    if (c >= q.Cin_pad) return;
    const int g = q.dg == 1 ? 0 : c / q.cpg;
    const long long d = pix * q.dg + g;
    const int b = starts[d], e = b + cnt[d];
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
    for (int i = b; i < e; ++i) {
        const uint2 en = entries[i];
        const unsigned smp = en.x;
        const float w = __uint_as_float(en.y);
        const unsigned pp = smp / (unsigned)q.K, k = smp - pp * (unsigned)q.K;
        const float4 v = *reinterpret_cast<const float4 *>(gcol + (size_t)pp * q.R + k * q.Cin_pad + c);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
    }
    *reinterpret_cast<float4 *>(gx_cl + (size_t)pix * q.Cin_pad + c) = acc;
}

// grad_x[n][c][hw] = gx_cl[n][hw][c] in the dtype, through a 64 x 64 LDS tile.
template <class E>
__global__ __launch_bounds__(kB) void v2b_out_kernel(const float *__restrict__ gx_cl,
                                                     typename E::bits *__restrict__ gx, int Cin,
                                                     int Cin_pad, int HW, int ctiles, int htiles) {
    __shared__ float tile[64][65];
    const int b = blockIdx.x;
    const int ct = b % ctiles, ht = (b / ctiles) % htiles, n = b / (ctiles * htiles);
    const int c0 = ct * 64, h0 = ht * 64;
    for (int it = threadIdx.x; it < 4096; it += kB) {
        const int px = it >> 6, c = it & 63;
        float v = 0.0f;
        if (h0 + px < HW && c0 + c < Cin_pad) v = gx_cl[((size_t)n * HW + h0 + px) * Cin_pad + c0 + c];
        tile[c][px] = v;
    }
    __syncthreads();
    for (int it = threadIdx.x; it < 4096; it += kB) {
        const int c = it >> 6, px = it & 63;
        if (h0 + px < HW && c0 + c < Cin) gx[((size_t)n * Cin + c0 + c) * HW + h0 + px] = from_f32(E{}, tile[c][px]);
    }
}

// ----------------------------------------------------------------- launch --

template <class E>
hipError_t launch_e(const V2BwdLaunch &a, hipStream_t stream) {
    const V2BwdPlan &pl = a.plan;
    char *ws = static_cast<char *>(a.workspace);
    uint16_t *xt = reinterpret_cast<uint16_t *>(ws + pl.off_xt);
    uint16_t *wT = reinterpret_cast<uint16_t *>(ws + pl.off_wt);
    uint16_t *gcl = reinterpret_cast<uint16_t *>(ws + pl.off_gcl);
    uint16_t *goT = reinterpret_cast<uint16_t *>(ws + pl.off_got);
    uint16_t *colT = reinterpret_cast<uint16_t *>(ws + pl.off_colt);
    float *gcol = reinterpret_cast<float *>(ws + pl.off_gcol);
    float *wpart = reinterpret_cast<float *>(ws + pl.off_wpart);
    int *cnt = reinterpret_cast<int *>(ws + pl.off_cnt);
    int *fill = cnt + pl.D;
    int *starts = reinterpret_cast<int *>(ws + pl.off_starts);
    uint2 *entries = reinterpret_cast<uint2 *>(ws + pl.off_entries);
    float *gx_cl = reinterpret_cast<float *>(ws + pl.off_gxcl);
    const int HW = a.H * a.W, HWo = pl.Ho * pl.Wo;
    const bool want_w = a.grad_weight != nullptr;
    const bool want_x = a.grad_x != nullptr;
    const bool want_s = want_x || a.grad_offset || a.grad_mask;
    hipError_t err;
    auto transpose = [&](const void *src, uint16_t *dst, int C, int Cpad, int hw) {
        PrepParams pp = {};
        pp.N = a.N; pp.Cin = C; pp.HW = hw; pp.Cin_pad = Cpad;
        pp.vec = (hw % kVec == 0) && ((uintptr_t)src % 16 == 0);
        pp.Mp = 0; pp.Rp = kVec;  // no weight blocks
        pp.tiles_c = (Cpad + 63) / 64;
        pp.tiles_hw = (hw + 63) / 64;
        pp.n_tr_blocks = a.N * pp.tiles_c * pp.tiles_hw;
        hipLaunchKernelGGL(v2_prep_kernel, dim3(pp.n_tr_blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t *>(src), (const uint16_t *)nullptr, dst,
                           (uint16_t *)nullptr, pp);
        return hipGetLastError();
    };
    V2bGeo q;
    q.N = a.N; q.H = a.H; q.W = a.W; q.Ho = pl.Ho; q.Wo = pl.Wo; q.kh = a.kh; q.kw = a.kw;
    q.sh = a.sh; q.sw = a.sw; q.ph = a.ph; q.pw = a.pw; q.dh = a.dh; q.dw = a.dw; q.dg = a.dg;
    q.K = pl.K; q.P = pl.P; q.has_mask = a.mask != nullptr; q.softmax = a.softmax ? 1 : 0;

    // 1. layouts
    if ((err = transpose(a.x, xt, a.Cin, pl.Cin_pad, HW)) != hipSuccess) return err;
    if (want_s) {
        if ((err = transpose(a.grad_out, gcl, a.Cout, pl.CoK, HWo)) != hipSuccess) return err;
        const long long nwt = (long long)pl.Rr * pl.CoK;
        hipLaunchKernelGGL(v2b_wt_kernel, dim3((unsigned)((nwt + kB - 1) / kB)), dim3(kB), 0, stream,
                           static_cast<const uint16_t *>(a.weight), wT, a.Cout, a.Cin, pl.K,
                           pl.Cin_pad, pl.CoK, nwt);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (want_w) {
        const long long nrows = (long long)pl.CoM * pl.Pp;
        const uint16_t *gsrc = static_cast<const uint16_t *>(a.grad_out);
        if (HWo % 8 == 0 && (uintptr_t)gsrc % 16 == 0)  // then P % 8 == 0 too
            hipLaunchKernelGGL((v2b_rows_kernel<true>), dim3((unsigned)((nrows / 8 + kB - 1) / kB)), dim3(kB),
                               0, stream, gsrc, goT, a.Cout, HWo, pl.P, pl.Pp, nrows);
        else
            hipLaunchKernelGGL((v2b_rows_kernel<false>), dim3((unsigned)((nrows + kB - 1) / kB)), dim3(kB),
                               0, stream, gsrc, goT, a.Cout, HWo, pl.P, pl.Pp, nrows);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        // 2. transposed columns
        V2bColParams cp;
        cp.q = q;
        cp.Cin_pad = pl.Cin_pad;
        cp.cpg = a.Cin / a.dg;
        cp.Pp = pl.Pp;
        cp.ptiles = (int)(pl.Pp / 64);
        cp.nblocks = cp.ptiles * pl.K * ((pl.Cin_pad + 63) / 64);
        hipLaunchKernelGGL(v2b_colT_kernel<E>, dim3(cp.nblocks), dim3(kB), 0, stream, xt, a.offset,
                           a.mask, colT, cp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        // 4. weight-gradient partials, 5. their sum
        GemmParams gp = {};
        gp.lda = gp.ldb = (int)pl.Pp;
        gp.nk_total = (int)(pl.Pp / kBK);
        gp.nk = (gp.nk_total + pl.splits - 1) / pl.splits;
        gp.Mtiles = pl.CoM / kBM;
        gp.Ntiles = pl.Rr / kBN;
        gp.nblocks = gp.Mtiles * gp.Ntiles * pl.splits;
        gp.ldc = pl.R; gp.Mstore = a.Cout; gp.Nstore = pl.R;
        gp.split_stride = (long long)a.Cout * pl.R;
        hipLaunchKernelGGL((v2_gemm_kernel<E, 1>), dim3(gp.nblocks), dim3(kGemmThreads), 0, stream,
                           goT, colT, wpart, gp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const long long nw = (long long)a.Cout * pl.R;
        hipLaunchKernelGGL(v2b_wsum_kernel, dim3((unsigned)((nw + kB - 1) / kB)), dim3(kB), 0, stream,
                           wpart, a.grad_weight, a.Cout, a.Cin, pl.K, pl.Cin_pad, pl.R, pl.splits);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (!want_s) return hipSuccess;

    // 3. column gradient
    {
        GemmParams gp = {};
        gp.lda = gp.ldb = pl.CoK;
        gp.nk = gp.nk_total = pl.CoK / kBK;
        gp.Mtiles = (int)(pl.Pp / kBM);
        gp.Ntiles = pl.Rr / kBN;
        gp.nblocks = gp.Mtiles * gp.Ntiles;
        gp.ldc = pl.R; gp.Mstore = (int)pl.P; gp.Nstore = pl.R;
        hipLaunchKernelGGL((v2_gemm_kernel<E, 1>), dim3(gp.nblocks), dim3(kGemmThreads), 0, stream,
                           gcl, wT, gcol, gp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // 6-8. buckets
    const long long nsamp = pl.P * a.dg * pl.K;
    if (want_x) {
        hipLaunchKernelGGL(v2b_zero_kernel, dim3(1024), dim3(kB), 0, stream, cnt, 2 * pl.D);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(v2b_count_kernel, dim3((unsigned)((nsamp + kB - 1) / kB)), dim3(kB), 0,
                           stream, a.offset, cnt, q);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(v2b_scan_kernel, dim3(1), dim3(1024), 0, stream, cnt, starts, pl.D);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // 9. sample pass
    {
        V2bSampleParams sp;
        sp.q = q;
        sp.Cin_pad = pl.Cin_pad;
        sp.gbase_mul = a.dg == 1 ? 0 : a.Cin / a.dg;
        sp.R = pl.R;
        sp.nchunk = (a.dg == 1 ? pl.Cin_pad : a.Cin / a.dg) / kVec;
        int L = 4;
        while (L < sp.nchunk && L < 64) L *= 2;
        sp.L = L;
        sp.Z = 64 / L;
        sp.npairs = pl.P * a.dg;
        const long long waves = (sp.npairs + sp.Z - 1) / sp.Z;
        sp.nblocks = (int)((waves + 3) / 4);
        sp.want_off = a.grad_offset != nullptr;
        sp.want_mask = a.grad_mask != nullptr;
        sp.want_x = want_x;
        hipLaunchKernelGGL(v2b_sample_kernel<E>, dim3(sp.nblocks), dim3(kB), 0, stream, xt, a.offset,
                           a.mask, gcol, starts, fill, entries, a.grad_offset, a.grad_mask, sp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (!want_x) return hipSuccess;
    // 10. destination gather, 11. NCHW grad_x
    {
        V2bGatherParams gq;
        gq.dg = a.dg; gq.cpg = a.Cin / a.dg; gq.Cin_pad = pl.Cin_pad; gq.K = pl.K; gq.R = pl.R;
        gq.CT = (pl.Cin_pad + 255) / 256;
        gq.nitems = (long long)a.N * HW * gq.CT;
        gq.nblocks = (int)((gq.nitems + 3) / 4);
        hipLaunchKernelGGL(v2b_gather_kernel, dim3(gq.nblocks), dim3(kB), 0, stream, gcol, starts, cnt,
                           entries, gx_cl, gq);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const int ctiles = (a.Cin + 63) / 64, htiles = (HW + 63) / 64;
        hipLaunchKernelGGL(v2b_out_kernel<E>, dim3(a.N * ctiles * htiles), dim3(kB), 0, stream, gx_cl,
                           static_cast<typename E::bits *>(a.grad_x), a.Cin, pl.Cin_pad, HW, ctiles,
                           htiles);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace

bool plan_dcn_v2_bwd(int N, int Cin, int H, int W, int Cout, int kh, int kw, int sh, int sw, int ph,
                     int pw, int dh, int dw, int dg, dcn_dtype dtype, V2BwdPlan &pl) {
    if (dtype != DCN_F16 && dtype != DCN_BF16) return false;
    if (N < 0 || Cin <= 0 || H <= 0 || W <= 0 || Cout <= 0 || kh <= 0 || kw <= 0 || dg <= 0) return false;
    if (sh <= 0 || sw <= 0 || dh <= 0 || dw <= 0 || ph < 0 || pw < 0) return false;
    const long long Ho = ((long long)H + 2LL * ph - (long long)dh * (kh - 1) - 1) / sh + 1;
    const long long Wo = ((long long)W + 2LL * pw - (long long)dw * (kw - 1) - 1) / sw + 1;
    if (Ho <= 0 || Wo <= 0) return false;
    pl.Ho = (int)Ho;
    pl.Wo = (int)Wo;
    pl.K = kh * kw;
    pl.P = (long long)N * Ho * Wo;
    pl.Cin_pad = (int)round_up(Cin, kVec);
    pl.R = pl.K * pl.Cin_pad;
    pl.Rr = (int)round_up(pl.R, kBN);
    pl.CoK = (int)round_up(Cout, kBK);
    pl.CoM = (int)round_up(Cout, kBM);
    pl.Pp = round_up(pl.P > 0 ? pl.P : 1, kBM);
    pl.D = (long long)N * H * W * dg;
    // split the pixel reduction of the weight gradient so that about 256 blocks run
    const long long tiles = (long long)(pl.CoM / kBM) * (pl.Rr / kBN);
    const long long nk = pl.Pp / kBK;
    long long splits = tiles >= 256 ? 1 : 256 / tiles;
    if (splits > nk) splits = nk;
    if (splits < 1) splits = 1;
    const long long per = (nk + splits - 1) / splits;
    pl.splits = (int)((nk + per - 1) / per);  // every split non-empty
    const long long nent = pl.P * dg * pl.K * 4;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    pl.off_xt = take((size_t)N * H * W * pl.Cin_pad * 2);
    pl.off_wt = take((size_t)pl.Rr * pl.CoK * 2);
    pl.off_gcl = take((size_t)pl.Pp * pl.CoK * 2);
    pl.off_got = take((size_t)pl.CoM * pl.Pp * 2);
    pl.off_colt = take((size_t)pl.Rr * pl.Pp * 2);
    pl.off_gcol = take((size_t)pl.P * pl.R * 4);
    pl.off_wpart = take((size_t)pl.splits * Cout * pl.R * 4);
    pl.off_cnt = take((size_t)pl.D * 2 * 4);  // counts, then fill cursors
    pl.off_starts = take((size_t)pl.D * 4);
    pl.off_entries = take((size_t)nent * 8);
    pl.off_gxcl = take((size_t)N * H * W * pl.Cin_pad * 4);
    pl.total = off;
    pl.entries = nent;
    return true;
}

hipError_t launch_dcn_v2_bwd(const V2BwdLaunch &a, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_BF16: return launch_e<EBF16>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcn
