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
//      then one launch for goT [CoM][Pp] (grad_out with the batch folded into the pixel
//      axis), wT [Rr][CoK] and clearing the bucket counters
//   2. colT [Rr][Pp]: the forward's columns, rounded to the dtype, transposed
//   3. gcol = gcl x wT^T (fp32)   4. grad_weight partials = goT x colT^T   5. their sum
//   6. count  7. scan
//   8. sample pass: grad_offset, grad_mask and the bucket entries
//   9. destination gather, summed in fp32 and written to NCHW grad_x in the dtype.
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
// FRAG: in MFMA fragment order instead of rows, value (co, p) at element
// (((co/32 * Pp/16 + p/16) * 2 + (p/8) % 2) * 32 + co % 32) * 8 + p % 8 (the fused
// weight-gradient kernel's operand). Block bi of the job.
__device__ __forceinline__ long long got_index(long long co, long long pp, long long Pp, bool frag) {
    if (!frag) return co * Pp + pp;
    return ((((co >> 5) * (Pp >> 4) + (pp >> 4)) * 2 + ((pp >> 3) & 1)) * 32 + (co & 31)) * 8 + (pp & 7);
}
template <bool VEC>
__device__ __forceinline__ void v2b_rows_block(int bi, const uint16_t *__restrict__ gout,
                                               uint16_t *__restrict__ goT, int Cout, int HWo, long long P,
                                               long long Pp, long long total, bool frag) {
    const long long t = (long long)bi * kB + threadIdx.x;
    if constexpr (VEC) {
        if (t * 8 >= total) return;
        const long long e = t * 8;
        long long co = e / Pp, pp = e - co * Pp;
        if (frag) {  // thread t fills 16-byte slot t: consecutive threads write consecutive bytes
            const long long blk = t >> 6;  // (32-row block, 16-pixel group)
            co = (blk / (Pp >> 4)) * 32 + (t & 31);
            pp = (blk % (Pp >> 4)) * 16 + ((t >> 5) & 1) * 8;
        }
        uint4 v = make_uint4(0, 0, 0, 0);
        if (co < Cout && pp < P) {
            const long long n = pp / HWo, hw = pp - n * HWo;
            v = *reinterpret_cast<const uint4 *>(gout + ((size_t)n * Cout + co) * HWo + hw);
        }
        *reinterpret_cast<uint4 *>(goT + got_index(co, pp, Pp, frag)) = v;
    } else {
        if (t >= total) return;
        const long long co = t / Pp, pp = t - co * Pp;
        uint16_t v = 0;
        if (co < Cout && pp < P) {
            const long long n = pp / HWo, hw = pp - n * HWo;
            v = gout[((size_t)n * Cout + co) * HWo + hw];
        }
        goT[got_index(co, pp, Pp, frag)] = v;
    }
}

// wT[r][co] = weight[co][ci][k] for r = k*Cin_pad + ci; zero for padding entries.
__device__ __forceinline__ void v2b_wt_block(int bi, const uint16_t *__restrict__ w, uint16_t *__restrict__ wT,
                                             int Cout, int Cin, int K, int Cin_pad, int CoK, long long total) {
    const long long t = (long long)bi * kB + threadIdx.x;
    if (t >= total) return;
    const int r = (int)(t / CoK), co = (int)(t - (long long)r * CoK);
    const int k = r / Cin_pad, ci = r - k * Cin_pad;
    wT[t] = (co < Cout && k < K && ci < Cin) ? w[((size_t)co * Cin + ci) * K + k] : (uint16_t)0;
}

// The backward's small layout jobs in one launch (a launch costs a few microseconds even
// when it does little): blocks [0, e_wt) transpose the weight, [e_wt, e_rows) lay
// grad_out out pixel-major, [e_rows, e_zero) clear the bucket counters.
struct V2bLayout {
    const uint16_t *gout, *w;
    uint16_t *wT, *goT;
    int Cout, Cin, K, Cin_pad, CoK, HWo, rows_vec, rows_frag;
    long long P, Pp, nwt, nrows;
    int *cnt;
    long long nzero;
    int e_wt, e_rows, e_zero;
};

__global__ __launch_bounds__(kB) void v2b_layout_kernel(const V2bLayout L) {
    const int b = (int)blockIdx.x;
    if (b < L.e_wt) {
        v2b_wt_block(b, L.w, L.wT, L.Cout, L.Cin, L.K, L.Cin_pad, L.CoK, L.nwt);
    } else if (b < L.e_rows) {
        if (L.rows_vec)
            v2b_rows_block<true>(b - L.e_wt, L.gout, L.goT, L.Cout, L.HWo, L.P, L.Pp, L.nrows, L.rows_frag);
        else
            v2b_rows_block<false>(b - L.e_wt, L.gout, L.goT, L.Cout, L.HWo, L.P, L.Pp, L.nrows, L.rows_frag);
    } else {
        const int nb = L.e_zero - L.e_rows;
        for (long long i = (long long)(b - L.e_rows) * kB + threadIdx.x; i < L.nzero; i += (long long)nb * kB)
            L.cnt[i] = 0;
    }
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

// grad_weight[co][ci][k] = sum over splits of part[s][co][k*Cin_pad + ci], the splits
// added in order from zero. One block per output channel: thread t reads the 16-byte
// vectors r = 4t..4t+3 of every split (up to eight splits' loads in flight before the
// adds), the row meets in LDS in [k][ci] order (rows padded by one word) and leaves
// as one contiguous [ci][k] run. Needs (Cin_pad + 1) * K floats of LDS (kWsumLds).
constexpr int kWsumThreads = 1024;
constexpr int kWsumLds = 16384;  // floats
__global__ __launch_bounds__(kWsumThreads) void v2b_wsum_kernel(const float *__restrict__ part,
                                                                float *__restrict__ gw, int Cout, int Cin,
                                                                int K, int Cin_pad, int R, int splits) {
    __shared__ float s_row[kWsumLds];
    const int co = (int)blockIdx.x;
    const size_t stride = (size_t)Cout * R;
    const float *src = part + (size_t)co * R;
    const int CP = Cin_pad + 1;
    for (int q = threadIdx.x; q * 4 < R; q += kWsumThreads) {
        float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int i0 = 0; i0 < splits; i0 += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u < splits) v[u] = *reinterpret_cast<const float4 *>(src + (i0 + u) * stride + 4 * q);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u < splits) {
                    s.x += v[u].x;
                    s.y += v[u].y;
                    s.z += v[u].z;
                    s.w += v[u].w;
                }
        }
        const int r = 4 * q, k = r / Cin_pad, ci = r - k * Cin_pad;  // Cin_pad % 8 == 0: one tap
        float *d = s_row + k * CP + ci;
        d[0] = s.x;
        d[1] = s.y;
        d[2] = s.z;
        d[3] = s.w;
    }
    __syncthreads();
    float *dst = gw + (size_t)co * Cin * K;
    for (int o = threadIdx.x; o < Cin * K; o += kWsumThreads) {
        const int ci = o / K, k = o - ci * K;
        dst[o] = s_row[k * CP + ci];
    }
}

// The same sum for rows too long for that LDS row: one thread per (co, r), writes
// strided by K.
__global__ __launch_bounds__(kB) void v2b_wsum_long_kernel(const float *__restrict__ part,
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

hipError_t launch_wsum(const float *wpart, float *gw, int Cout, int Cin, int K, int Cin_pad, int R,
                       int splits, hipStream_t stream) {
    if ((long long)(Cin_pad + 1) * K <= kWsumLds) {
        hipLaunchKernelGGL(v2b_wsum_kernel, dim3((unsigned)Cout), dim3(kWsumThreads), 0, stream, wpart, gw,
                           Cout, Cin, K, Cin_pad, R, splits);
    } else {
        const long long nw = (long long)Cout * R;
        hipLaunchKernelGGL(v2b_wsum_long_kernel, dim3((unsigned)((nw + kB - 1) / kB)), dim3(kB), 0, stream,
                           wpart, gw, Cout, Cin, K, Cin_pad, R, splits);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- buckets --

// One thread per sample, samples in the offsets' own order (n, g, k, output pixel), so
// a wavefront reads 64 consecutive offsets of one tap. A corner that receives a grad_x
// entry (inside the image, weight non-zero) counts in its destination's bucket; the
// block first counts in an LDS window of kCntWin consecutive counters around its first
// sample's rows (one global atomic per touched counter afterwards), destinations outside
// it go straight to global atomics.
constexpr int kCntWin = 4096;
__global__ __launch_bounds__(kB) void v2b_count_kernel(const float *__restrict__ offset,
                                                       int *__restrict__ cnt, V2bGeo q) {
    __shared__ int s_win[kCntWin];
    const int HWo = q.Ho * q.Wo;
    const long long total = q.P * q.dg * q.K;
    const long long t0 = (long long)blockIdx.x * kB;
    const long long rowc = (long long)q.W * q.dg;  // counters per image row
    long long lo;
    {
        const int r = (int)(t0 % HWo);
        const long long nk = t0 / HWo;
        const int k = (int)(nk % q.K);
        const int n = (int)(nk / q.K / q.dg);
        const int ho = r / q.Wo, wo = r - ho * q.Wo;
        const int y = ho * q.sh - q.ph + (k / q.kw) * q.dh;
        const long long rows = kCntWin / rowc;
        if (rows >= 2) {
            const long long span = (kB + q.Wo - 1) / q.Wo * q.sh + 1;  // base rows the block covers
            const long long margin = rows > span ? (rows - span) / 2 : 0;
            lo = ((long long)n * q.H + y - margin) * rowc;
        } else {
            const int x = wo * q.sw - q.pw + (k % q.kw) * q.dw;
            lo = (((long long)n * q.H + y) * q.W + x) * q.dg - kCntWin / 4;
        }
    }
    for (int i = threadIdx.x; i < kCntWin; i += kB) s_win[i] = 0;
    __syncthreads();
    const long long t = t0 + threadIdx.x;
    if (t < total) {
        const int r = (int)(t % HWo);
        const long long nk = t / HWo;
        const int k = (int)(nk % q.K);
        const long long ng = nk / q.K;
        const int g = (int)(ng % q.dg), n = (int)(ng / q.dg);
        const V2bTap tp = v2b_tap(offset, q, n, r, g, k);
        const long long d00 = (((long long)n * q.H + tp.y0) * q.W + tp.x0) * q.dg + g;
        auto add = [&](long long d) {
            const long long w = d - lo;
            if ((unsigned long long)w < (unsigned long long)kCntWin) atomicAdd(&s_win[w], 1);
            else atomicAdd(&cnt[d], 1);
        };
        if (tp.w00 != 0.0f) add(d00);
        if (tp.w01 != 0.0f) add(d00 + q.dg);
        if (tp.w10 != 0.0f) add(d00 + rowc);
        if (tp.w11 != 0.0f) add(d00 + rowc + q.dg);
    }
    __syncthreads();
    // only counters of real destinations (0 <= lo + i < D) can be non-zero
    for (int i = threadIdx.x; i < kCntWin; i += kB) {
        const int c = s_win[i];
        if (c) atomicAdd(&cnt[lo + i], c);
    }
}

// Exclusive prefix sum of cnt[0..D) into starts, one block of 1024 threads walking
// chunks of 16384 (16 consecutive values per thread, loaded as four 16-byte vectors
// where the chunk is whole; cnt and starts 16-byte aligned) with a running carry.
__global__ __launch_bounds__(1024) void v2b_scan_kernel(const int *__restrict__ cnt,
                                                        int *__restrict__ starts, long long D) {
    __shared__ int s_wave[16];
    __shared__ int s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (long long c0 = 0; c0 < D; c0 += 16384) {
        const long long b = c0 + 16LL * tid;
        int v[16];
        if (b + 16 <= D) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int4 u = *reinterpret_cast<const int4 *>(cnt + b + 4 * i);
                v[4 * i] = u.x;
                v[4 * i + 1] = u.y;
                v[4 * i + 2] = u.z;
                v[4 * i + 3] = u.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = (b + i < D) ? cnt[b + i] : 0;
        }
        int mine = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) mine += v[i];
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
        int o[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            o[i] = run;
            run += v[i];
        }
        if (b + 16 <= D) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<int4 *>(starts + b + 4 * i) =
                    make_int4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (b + i < D) starts[b + i] = o[i];
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
    int dg, cpg, Cin, Cin_pad, K, R, CT, HW, htiles;
    int nblocks;
};

// grad_x in the dtype, NCHW, straight from the buckets. A block takes 16 consecutive
// pixels of one image and one 256-channel tile: wavefront w sums pixel w's bucket,
// 4 channels per lane (entries coef * gcol[sample's pixel][tap, c..c+3]; with several
// deformable groups each lane walks the bucket of its channels' group), the sums meet
// transposed in LDS, and each channel's 16 pixels leave as one 32-byte run.
constexpr int kGxPix = 16;
__global__ __launch_bounds__(64 * kGxPix) void v2b_gather_kernel(const float *__restrict__ gcol,
                                                                 const int *__restrict__ starts,
                                                                 const int *__restrict__ cnt,
                                                                 const uint2 *__restrict__ entries,
                                                                 uint16_t *__restrict__ gx, int dtype_bf16,
                                                                 V2bGatherParams q) {
    __shared__ float tile[256][kGxPix + 1];
    const int blk = xcd_remap((int)blockIdx.x, q.nblocks);
    const int ct = blk % q.CT, rest = blk / q.CT;
    const int ht = rest % q.htiles, n = rest / q.htiles;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int hw = ht * kGxPix + w;
    const int c = ct * 256 + lane * 4;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (hw < q.HW && c < q.Cin_pad) {
        const int g = q.dg == 1 ? 0 : c / q.cpg;
        const long long d = ((long long)n * q.HW + hw) * q.dg + g;
        const int b = starts[d], e = b + cnt[d];
#pragma unroll 4
        for (int i = b; i < e; ++i) {
            const uint2 en = entries[i];
            const unsigned smp = en.x;
            const float wt = __uint_as_float(en.y);
            const unsigned pp = smp / (unsigned)q.K, k = smp - pp * (unsigned)q.K;
            const float4 v = *reinterpret_cast<const float4 *>(gcol + (size_t)pp * q.R + k * q.Cin_pad + c);
            acc.x = fmaf(wt, v.x, acc.x);
            acc.y = fmaf(wt, v.y, acc.y);
            acc.z = fmaf(wt, v.z, acc.z);
            acc.w = fmaf(wt, v.w, acc.w);
        }
    }
    tile[lane * 4 + 0][w] = acc.x;
    tile[lane * 4 + 1][w] = acc.y;
    tile[lane * 4 + 2][w] = acc.z;
    tile[lane * 4 + 3][w] = acc.w;
    __syncthreads();
    for (int it = threadIdx.x; it < 256 * kGxPix; it += 64 * kGxPix) {
        const int cl = it / kGxPix, px = it % kGxPix;
        const int cc = ct * 256 + cl, h = ht * kGxPix + px;
        if (cc < q.Cin && h < q.HW) {
            const float v = tile[cl][px];
            gx[((size_t)n * q.Cin + cc) * q.HW + h] = dtype_bf16 ? from_f32(EBF16{}, v) : from_f32(EF16{}, v);
        }
    }
}

// ----------------------------------------------------------------- launch --

// ------------------------------------------------------ fused weight gradient --
//
// grad_weight partials without the transposed columns in memory (Cin % 64 == 0): the
// GEMM grad_weight[co][r] = sum_p grad_out[p][co] * col[p][r] with the column tile
// formed on chip, in the two-role structure of the forward's fused kernel. A block
// takes 256 output channels x 64 columns r (one tap k, channel block cb) over the
// pixel range of its split, in steps of 64 pixels. Producer waves form the step's
// column tile (m * bilinear in fp32 as the forward forms it, rounded to the dtype)
// and write it transposed into LDS, pixels contiguous per column r: row rr holds 64
// pixels, 16-byte chunk cc at position cc ^ ((rr >> 3) + rr) & 7, so that both the
// producers' 2-byte writes (8 rows rr = 8 bc + e at once) and the MMA waves' 16-byte
// fragment reads (16 consecutive rows at once) fall on distinct banks. MMA waves read
// grad_out (goT in MFMA fragment order: the 8 values (co, 16q + 8h .. +7) at 16-byte
// slot ((co/32 * Pp/16 + q) * 2 + h) * 32 + co % 32) straight from memory one step
// ahead, like the forward's weight. Partials go to wpart[split][co][r] for the fixed-
// order sum of v2b_wsum_kernel. The block's pixels' tap data (the two offsets and the
// modulation of tap k in the block's group, the grid base of the tap and the image)
// are staged in LDS before the K loop, so a producer's step starts from LDS instead of
// two dependent global loads; a block takes at most kWgMaxSteps steps (the plan raises
// the number of splits accordingly), and one deformable group per 64-channel block.
constexpr int kWgMaxSteps = 32;
constexpr int kWgMma = 4;                          // MMA waves: 64 grad_out channels each
constexpr int kWgProd = 8;                         // producer waves: 64 pixels x 8 chunks
constexpr int kWgThreads = 64 * (kWgMma + kWgProd);

struct V2bWgParams {
    V2bGeo q;
    int Cin_pad, cpg, CBn, R, Cout;
    int steps, nsteps;  // 64-pixel steps per split and in all (Pp / 64)
    int Mt, nblocks;    // 256-channel blocks of grad_out; blocks
    long long Pp;
    unsigned xt_bytes, got_bytes;
};

__device__ __forceinline__ int wg_swz(int rr) { return ((rr >> 3) + rr) & 7; }

// whether the weight gradient of a layer takes v2b_wgrad_kernel
__host__ __device__ inline bool v2b_wgrad_fused(int N, int H, int W, int Cin, int Cin_pad, int dg, int CoM,
                                                long long Pp) {
    const int Mt = (CoM + 255) / 256;
    return Cin_pad % kBK == 0 && (dg == 1 || (Cin / dg) % kBK == 0) &&
           (size_t)N * H * W * Cin_pad * 2 < (1ull << 31) && (size_t)Mt * 256 * Pp * 2 < (1ull << 31);
}

template <class E>
__global__ __launch_bounds__(kWgThreads) void v2b_wgrad_kernel(const uint16_t *__restrict__ xt,
                                                               const float *__restrict__ offset,
                                                               const float *__restrict__ mask,
                                                               const uint16_t *__restrict__ gotf,
                                                               float *__restrict__ wpart,
                                                               const V2bWgParams p) {
    __shared__ uint4 sB[2][512];  // [64 columns r][8 chunks of 8 pixels], swizzled
    // per pixel of the block: offsets (y, x) and modulation of tap k; grid base (y, x)
    // of the tap and the image's first element in xt
    __shared__ float4 s_tf[kWgMaxSteps * 64];
    __shared__ int4 s_ti[kWgMaxSteps * 64];
    const V2bGeo &q = p.q;
    const int nrb = q.K * p.CBn;
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    // the blocks of one split are consecutive: one XCD shares the split's grad_out in L2
    const int sp = blk / (nrb * p.Mt), rest = blk - sp * (nrb * p.Mt);
    const int mt = rest / nrb, rb = rest - mt * nrb;
    const int k = rb / p.CBn, cb = rb - k * p.CBn;
    const int s0 = sp * p.steps;
    const int NS = min(p.steps, p.nsteps - s0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HWo = q.Ho * q.Wo;
    const int g = min(cb * kBK / p.cpg, q.dg - 1);  // the block's deformable group
    {
        const int i = k / q.kw, j = k - i * q.kw;
        for (int t = tid; t < NS * 64; t += kWgThreads) {
            const long long pg = (long long)s0 * 64 + t;
            float4 f = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            int4 iv = make_int4(0, 0, 0, 0);
            if (pg < q.P) {
                const int n = (int)(pg / HWo), r = (int)(pg - (long long)n * HWo);
                float mx, inv;
                v2b_softmax_stats(mask, q, n, r, g, mx, inv);
                const float *op = offset + ((size_t)(n * q.dg + g) * q.K + k) * 2 * HWo + r;
                const int ho = r / q.Wo, wo = r - ho * q.Wo;
                f = make_float4(op[HWo], op[0], v2b_mod(mask, q, n, r, g, k, mx, inv), 0.0f);
                iv = make_int4(ho * q.sh - q.ph + i * q.dh, wo * q.sw - q.pw + j * q.dw, n * q.H * q.W * p.Cin_pad, 0);
            }
            s_tf[t] = f;
            s_ti[t] = iv;
        }
        __syncthreads();
    }

    if (wave >= kWgMma) {
        // ------------------------------------------------------------ producers --
        if (NS <= 0) return;  // an empty split: the MMA waves store zeros, no barriers
        const int ptid = tid - 64 * kWgMma;
        const int br = ptid >> 3, bc = ptid & 7;
        const int c0 = cb * kBK + bc * kVec;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xt, p.xt_bytes);
        struct Stage {
            uint4 v[4];
            float w[4];
        };
        // corners of step s (pixel (s0 + s) * 64 + br), loaded unconditionally (pixels
        // past P read offset 0 with weight 0) so the count of loads in flight is exact
        auto load = [&](Stage &st, int s) __attribute__((always_inline)) {
            // pixels past P were staged with modulation 0: weight 0, corners in the image
            const float4 f = s_tf[s * 64 + br];
            const int4 iv = s_ti[s * 64 + br];
            int y0, x0;
            float fy, fx;
            split_coord(iv.x, f.x, y0, fy);
            split_coord(iv.y, f.y, x0, fx);
            const Tap t = make_tap(y0, x0, fy, fx, f.z, q.H, q.W, p.Cin_pad);
            const int base = iv.z + c0;
            st.v[0] = buffer_load<uint4>(rx, (base + t.o00) * 2, 0);
            st.v[1] = buffer_load<uint4>(rx, (base + t.o01) * 2, 0);
            st.v[2] = buffer_load<uint4>(rx, (base + t.o10) * 2, 0);
            st.v[3] = buffer_load<uint4>(rx, (base + t.o11) * 2, 0);
            st.w[0] = t.w00; st.w[1] = t.w01; st.w[2] = t.w10; st.w[3] = t.w11;
        };
        auto fill = [&](const Stage &st, int buf) __attribute__((always_inline)) {
            float acc[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                float f[kVec];
                load_f32<E, kVec>(reinterpret_cast<const typename E::bits *>(&st.v[cn]), f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] = fmaf(st.w[cn], f[e], acc[e]);
            }
            uint16_t *t16 = reinterpret_cast<uint16_t *>(sB[buf]);
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int rr = bc * kVec + e;
                t16[rr * 64 + (((br >> 3) ^ wg_swz(rr)) << 3) + (br & 7)] = (uint16_t)from_f32(E{}, acc[e]);
            }
        };
        Stage st[2];
        load(st[0], 0);
        load(st[1], NS > 1 ? 1 : 0);
        fill(st[0], 0);
        lds_barrier();  // step 0's column tile is in buffer 0
        for (int s = 0; s < NS; s += 2) {
            // buffer s & 1 is read by the MMA waves; fill the other
            load(st[0], s + 2 < NS ? s + 2 : NS - 1);
            if (s + 1 < NS) fill(st[1], 1);
            lds_barrier();
            if (s + 1 < NS) {
                load(st[1], s + 3 < NS ? s + 3 : NS - 1);
                if (s + 2 < NS) fill(st[0], 0);
                lds_barrier();
            }
        }
        return;
    }

    // ---------------------------------------------------------------- MMA waves --
    const int frow = lane & 31, fhalf = lane >> 5;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(gotf, p.got_bytes);
    int aoff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        aoff[t] = (int)((long long)(mt * 8 + wave * 2 + t) * p.Pp * 64) + lane * 16;  // 1 KB per (32 rows, 16 pixels)
    uint4 fa[2][2][4];  // [set][tile][ks]
    auto load_a = [&](uint4 (&f)[2][4], int s) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) f[t][ks] = buffer_load<uint4>(ra, aoff[t], ((s0 + s) * 4 + ks) * 1024);
    };
    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    auto mma = [&](const uint4 (&f)[2][4], int s) __attribute__((always_inline)) {
        const uint4 *sb = sB[s & 1];
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int cc = 2 * ks + fhalf;
            uint4 fb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int rr = u * 32 + frow;
                fb[u] = sb[rr * 8 + (cc ^ wg_swz(rr))];
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma32<E>(f[a][ks], fb[b], acc[a][b]);
        }
    };
    if (NS > 0) {
        load_a(fa[0], 0);
        lds_barrier();  // step 0's column tile
        int s = 0;
        for (; s + 1 < NS; s += 2) {
            load_a(fa[1], s + 1);
            asm volatile("" ::: "memory");
            mma(fa[0], s);
            lds_barrier();
            load_a(fa[0], s + 2 < NS ? s + 2 : s + 1);
            asm volatile("" ::: "memory");
            mma(fa[1], s + 1);
            lds_barrier();
        }
        if (s < NS) {  // odd step count: the last step's fragments are in set 0
            mma(fa[0], s);
            lds_barrier();
        }
    }
    // D[i][j] of a 32x32 tile: lane j + 32*((i/4)%2), register 4*(i/8) + i%4; row i a
    // grad_out channel co, column j a column r
    float *o = wpart + (size_t)sp * p.Cout * p.R;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int rcol = k * p.Cin_pad + cb * kBK + b * 32 + (lane & 31);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = mt * 256 + wave * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (co < p.Cout) o[(size_t)co * p.R + rcol] = acc[a][b][r];
            }
        }
    }
}

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
    const int HW = a.H * a.W, HWo = pl.Ho * pl.Wo;
    const bool want_w = a.grad_weight != nullptr;
    const bool want_x = a.grad_x != nullptr;
    const bool want_s = want_x || a.grad_offset || a.grad_mask;
    hipError_t err;
    // parameters of one channels-last transpose (register transposes where the pixel rows
    // are whole 16-byte vectors, else through the LDS tile); its block count in n_tr_blocks
    auto transpose_params = [&](const void *src, int C, int Cpad, int hw) {
        PrepParams pp = {};
        pp.N = a.N; pp.Cin = C; pp.HW = hw; pp.Cin_pad = Cpad;
        pp.vec = (hw % kVec == 0) && ((uintptr_t)src % 16 == 0);
        pp.Mp = 0; pp.Rp = kVec;  // no weight blocks
        pp.tiles_c = (Cpad + 63) / 64;
        pp.tiles_hw = (hw + 63) / 64;
        pp.cgroups = pp.tiles_c;
        pp.hgroups = pp.tiles_hw;
        pp.reg = pp.vec;
        pp.n_tr_blocks = pp.reg ? (a.N * pp.cgroups * pp.hgroups + 3) / 4 : a.N * pp.tiles_c * pp.tiles_hw;
        return pp;
    };
    // the weight gradient with the columns formed on chip: 64-channel column blocks within
    // a tap, and 32-bit byte offsets into xt and the fragment-order goT
    const int Mt = (pl.CoM + 255) / 256;
    const bool wg_fused = v2b_wgrad_fused(a.N, a.H, a.W, a.Cin, pl.Cin_pad, a.dg, pl.CoM, pl.Pp) &&
                          (pl.Pp / kBK + pl.splits - 1) / pl.splits <= kWgMaxSteps;  // as the plan arranges
    V2bGeo q;
    q.N = a.N; q.H = a.H; q.W = a.W; q.Ho = pl.Ho; q.Wo = pl.Wo; q.kh = a.kh; q.kw = a.kw;
    q.sh = a.sh; q.sw = a.sw; q.ph = a.ph; q.pw = a.pw; q.dh = a.dh; q.dw = a.dw; q.dg = a.dg;
    q.K = pl.K; q.P = pl.P; q.has_mask = a.mask != nullptr; q.softmax = a.softmax ? 1 : 0;

    // 1. layouts: x and grad_out to channels-last (the forward's prep kernel), then the
    // weight transposed, grad_out pixel-major and the bucket counters cleared in one launch
    {
        const PrepParams tx = transpose_params(a.x, a.Cin, pl.Cin_pad, HW);
        hipLaunchKernelGGL(v2_prep_kernel, dim3(tx.n_tr_blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t *>(a.x), (const uint16_t *)nullptr, xt,
                           (uint16_t *)nullptr, tx);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if (want_s) {
            const PrepParams tg = transpose_params(a.grad_out, a.Cout, pl.CoK, HWo);
            hipLaunchKernelGGL(v2_prep_kernel, dim3(tg.n_tr_blocks), dim3(256), 0, stream,
                               static_cast<const uint16_t *>(a.grad_out), (const uint16_t *)nullptr, gcl,
                               (uint16_t *)nullptr, tg);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        V2bLayout L = {};
        L.gout = static_cast<const uint16_t *>(a.grad_out);
        L.w = static_cast<const uint16_t *>(a.weight);
        L.wT = wT; L.goT = goT;
        L.Cout = a.Cout; L.Cin = a.Cin; L.K = pl.K; L.Cin_pad = pl.Cin_pad; L.CoK = pl.CoK; L.HWo = HWo;
        L.P = pl.P; L.Pp = pl.Pp;
        L.cnt = cnt;
        int nb = 0;
        if (want_s) {
            L.nwt = (long long)pl.Rr * pl.CoK;
            nb += (int)((L.nwt + kB - 1) / kB);
        }
        L.e_wt = nb;
        if (want_w) {
            L.nrows = (long long)pl.CoM * pl.Pp;
            L.rows_vec = HWo % 8 == 0 && (uintptr_t)a.grad_out % 16 == 0;  // then P % 8 == 0 too
            L.rows_frag = wg_fused ? 1 : 0;
            nb += (int)(((L.rows_vec ? L.nrows / 8 : L.nrows) + kB - 1) / kB);
        }
        L.e_rows = nb;
        if (want_x) {
            L.nzero = 2LL * pl.D;
            const long long nz = (L.nzero + kB - 1) / kB;
            nb += (int)(nz < 1024 ? nz : 1024);
        }
        L.e_zero = nb;
        if (nb > 0) {
            hipLaunchKernelGGL(v2b_layout_kernel, dim3(nb), dim3(kB), 0, stream, L);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    if (want_w && wg_fused) {
        // 2-4. weight-gradient partials with the columns formed on chip, 5. their sum
        V2bWgParams wg;
        wg.q = q;
        wg.Cin_pad = pl.Cin_pad;
        wg.cpg = a.Cin / a.dg;
        wg.CBn = pl.Cin_pad / kBK;
        wg.R = pl.R;
        wg.Cout = a.Cout;
        wg.nsteps = (int)(pl.Pp / kBK);
        wg.steps = (wg.nsteps + pl.splits - 1) / pl.splits;  // the plan's splits, all non-empty
        wg.Mt = Mt;
        wg.nblocks = pl.splits * Mt * pl.K * wg.CBn;
        wg.Pp = pl.Pp;
        wg.xt_bytes = (unsigned)((size_t)a.N * a.H * a.W * pl.Cin_pad * 2);
        wg.got_bytes = (unsigned)((size_t)pl.CoM * pl.Pp * 2);
        hipLaunchKernelGGL(v2b_wgrad_kernel<E>, dim3(wg.nblocks), dim3(kWgThreads), 0, stream, xt, a.offset,
                           a.mask, goT, wpart, wg);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if ((err = launch_wsum(wpart, a.grad_weight, a.Cout, a.Cin, pl.K, pl.Cin_pad, pl.R, pl.splits,
                               stream)) != hipSuccess)
            return err;
    } else if (want_w) {
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
        if ((err = launch_wsum(wpart, a.grad_weight, a.Cout, a.Cin, pl.K, pl.Cin_pad, pl.R, pl.splits,
                               stream)) != hipSuccess)
            return err;
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
        // a reduction over Cout only: with a few K tiles per block, the two-slot ring
        // lets two blocks share a CU, so one block's fp32 stores overlap the other's MFMAs
        if (gp.nk <= 8)
            hipLaunchKernelGGL((v2_gemm_kernel<E, 1, 2>), dim3(gp.nblocks), dim3(kGemmThreads), 0, stream,
                               gcl, wT, gcol, gp);
        else
            hipLaunchKernelGGL((v2_gemm_kernel<E, 1>), dim3(gp.nblocks), dim3(kGemmThreads), 0, stream,
                               gcl, wT, gcol, gp);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // 6-7. buckets
    const long long nsamp = pl.P * a.dg * pl.K;
    if (want_x) {  // (the counters were cleared with the layouts)
        hipLaunchKernelGGL(v2b_count_kernel, dim3((unsigned)((nsamp + kB - 1) / kB)), dim3(kB), 0,
                           stream, a.offset, cnt, q);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        hipLaunchKernelGGL(v2b_scan_kernel, dim3(1), dim3(1024), 0, stream, cnt, starts, pl.D);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    // 8. sample pass
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
    // 9. destination gather into NCHW grad_x
    {
        V2bGatherParams gq;
        gq.dg = a.dg; gq.cpg = a.Cin / a.dg; gq.Cin = a.Cin; gq.Cin_pad = pl.Cin_pad; gq.K = pl.K;
        gq.R = pl.R;
        gq.CT = (pl.Cin_pad + 255) / 256;
        gq.HW = HW;
        gq.htiles = (HW + kGxPix - 1) / kGxPix;
        gq.nblocks = a.N * gq.htiles * gq.CT;
        hipLaunchKernelGGL(v2b_gather_kernel, dim3(gq.nblocks), dim3(64 * kGxPix), 0, stream, gcol, starts, cnt,
                           entries, static_cast<uint16_t *>(a.grad_x), E::id == DCN_BF16 ? 1 : 0, gq);
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
    // the fused weight-gradient kernel takes at most kWgMaxSteps 64-pixel steps per split
    if (v2b_wgrad_fused(N, H, W, Cin, pl.Cin_pad, dg, pl.CoM, pl.Pp)) {
        const long long need = (nk + kWgMaxSteps - 1) / kWgMaxSteps;
        if (splits < need) splits = need;
    }
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
