// DCNv2 modulated deformable convolution (NCHW) for gfx950: deform-im2col + MFMA GEMM.
//
// Operation ("DCNv2 in YOLOv5", cyqw.cn, section 1; bilinear kernel from "Hands-on
// DCNv1 in PyTorch", agent.csdn.net, section 2):
//   out[n,co,ho,wo] = sum_{ci,k} weight[co,ci,k] * m_k * bilinear(x[n,ci], pos_k)
// Three launches on the caller's stream, no host synchronisation:
//   1. prep:   x [N,Cin,H,W] -> xt [N,H,W,Cin_pad] (channels-last, so one tap's
//              channel vector is contiguous) and weight [Cout,Cin,K] ->
//              wp [Mp][Rp] with wp[co][k*Cin_pad + ci] (tap-major), zero padded.
//   2. im2col: col[p][k*Cin_pad + ci] = m_k(p) * bilinear(xt[n,:,:,ci], pos_k(p)),
//              one K-contiguous row per output pixel p = (n*Ho + ho)*Wo + wo.
//   3. gemm:   out[n][co][hw] = sum_r wp[co][r] * col[p][r]; both operands are
//              K-contiguous, so every MFMA fragment is one 16-byte read. 128x128
//              block tiles, 64-deep K steps through a 4-slot LDS ring filled by
//              direct global->LDS copies, v_mfma_f32_32x32x16 (bf16/fp16 in, fp32
//              accumulate).
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

#include "v2_shared.hpp"

// ----------------------------------------------------------------- im2col --

struct ColParams {
    int N, H, W, Ho, Wo, kh, kw, sh, sw, ph, pw, dh, dw, dg, Cin, Cin_pad, cpg;
    int K, R, Rp;
    long long P, Pp;
    int has_mask, softmax;
    int S, Q, nchunk;  // lanes per (pixel, tap) item, items per wave, chunks per item
    int TP;            // pixels per block
    int nblocks;
    unsigned magic_k, magic_kw;  // ceil(2^20 / K), ceil(2^20 / kw): exact quotients below 2^12
};

// floor(a / d) for 0 <= a < 2^12 and 1 <= d < 2^6 from m = ceil(2^20 / d): a * m / 2^20
// exceeds a / d by less than a / 2^20 < 2^-8 < 1 / d, so the floor is exact, and
// a * m < 2^12 * 2^20 fits 32 bits.
__device__ __forceinline__ int div_small(int a, unsigned m) { return (int)(((unsigned)a * m) >> 20); }

constexpr int kColMaxTP = 64;  // pixels per im2col block, at most

template <class E>
__global__ __launch_bounds__(256) void v2_im2col_kernel(const uint16_t *__restrict__ xt,
                                                        const float *__restrict__ offset,
                                                        const float *__restrict__ mask,
                                                        uint16_t *__restrict__ col, ColParams p) {
    extern __shared__ float smem[];
    const int K = p.K;
    float *s_off = smem;                          // [TP][dg][K][2]
    float *s_m = smem + p.TP * p.dg * K * 2;      // [TP][dg][K]
    __shared__ int s_pix[3][kColMaxTP];  // image, output row, output column of the block's pixels
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const long long p0 = (long long)blk * p.TP;
    const long long HWo = (long long)p.Ho * p.Wo;

    // 0. the block's pixels split into (image, row, column) once (64-bit divisions)
    if ((int)threadIdx.x < p.TP) {
        const long long pg = p0 + threadIdx.x;
        int n = 0, ho = 0, wo = 0;
        if (pg < p.P) {
            const long long r = pg % HWo;
            n = (int)(pg / HWo);
            ho = (int)(r / p.Wo);
            wo = (int)(r - (long long)ho * p.Wo);
        }
        s_pix[0][threadIdx.x] = n;
        s_pix[1][threadIdx.x] = ho;
        s_pix[2][threadIdx.x] = wo;
    }
    __syncthreads();

    // 1. stage offsets / masks of this block's pixels (pixel-fastest: coalesced NCHW rows)
    const int per_pix = p.dg * K;
    for (int i = threadIdx.x; i < p.TP * per_pix * 2; i += 256) {
        const int pl = i % p.TP, c = i / p.TP;  // c = offset channel (g*K + k)*2 + xy
        const long long pg = p0 + pl;
        float v = 0.0f;
        if (pg < p.P) {
            const size_t r = (size_t)s_pix[1][pl] * p.Wo + s_pix[2][pl];
            v = offset[((size_t)s_pix[0][pl] * per_pix * 2 + c) * HWo + r];
        }
        s_off[pl * per_pix * 2 + c] = v;
    }
    for (int i = threadIdx.x; i < p.TP * per_pix; i += 256) {
        const int pl = i % p.TP, c = i / p.TP;
        const long long pg = p0 + pl;
        float v = 1.0f;
        if (p.has_mask && pg < p.P) {
            const size_t r = (size_t)s_pix[1][pl] * p.Wo + s_pix[2][pl];
            v = mask[((size_t)s_pix[0][pl] * per_pix + c) * HWo + r];
        }
        s_m[pl * per_pix + c] = v;
    }
    __syncthreads();
    if (p.softmax) {  // softmax over K per (pixel, deformable group)
        for (int i = threadIdx.x; i < p.TP * p.dg; i += 256) {
            float *ml = s_m + i * K;
            float mx = -INFINITY;
            for (int k = 0; k < K; ++k) mx = fmaxf(mx, ml[k]);
            float sum = 0.0f;
            for (int k = 0; k < K; ++k) sum += expf(ml[k] - mx);
            const float inv = 1.0f / sum;
            for (int k = 0; k < K; ++k) ml[k] = expf(ml[k] - mx) * inv;
        }
        __syncthreads();
    }

    // 2. items (pixel, tap): S lanes x 8 channels cover the Cin_pad channels
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int q = lane / p.S, s = lane - q * p.S;
    const int nitems = p.TP * K;
    const int per_pass = 4 * p.Q;
    if (q < p.Q && p.nchunk <= p.S && nitems < 4096 && K < 64) {
        // one 16-byte chunk per lane and item: items are taken kB passes at a time, the
        // corners of all kB loaded before any is summed, so that a wave has kB items'
        // gathers in flight instead of one
        constexpr int kB = 3;
        const int ch = s, ci0 = ch * kVec;
        const bool lane_on = ch < p.nchunk;
        const int g = min(ci0 / p.cpg, p.dg - 1);
        for (int it0 = wave * p.Q + q; it0 < nitems; it0 += per_pass * kB) {
            uint4 cr[kB][4];
            Tap tb[kB];
            uint16_t *crow[kB];
            bool live[kB];
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                const int it = it0 + b * per_pass;
                live[b] = it < nitems;
                const int pl = live[b] ? div_small(it, p.magic_k) : 0, k = live[b] ? it - pl * K : 0;
                const long long pg = p0 + pl;
                crow[b] = col + (size_t)pg * p.Rp + (size_t)k * p.Cin_pad + ci0;
                const bool real = live[b] && pg < p.P && lane_on;
                const int n = s_pix[0][pl], ho = s_pix[1][pl], wo = s_pix[2][pl];
                const int i = div_small(k, p.magic_kw), j = k - i * p.kw;
                const float *so = s_off + ((pl * p.dg + g) * K + k) * 2;
                int y0, x0;
                float fy, fx;
                split_coord(ho * p.sh - p.ph + i * p.dh, so[1], y0, fy);
                split_coord(wo * p.sw - p.pw + j * p.dw, so[0], x0, fx);
                tb[b] = make_tap(y0, x0, fy, fx, real ? s_m[(pl * p.dg + g) * K + k] : 0.0f, p.H, p.W,
                                 p.Cin_pad);
                const uint16_t *img = xt + (size_t)n * p.H * p.W * p.Cin_pad + ci0;
                cr[b][0] = *reinterpret_cast<const uint4 *>(img + tb[b].o00);
                cr[b][1] = *reinterpret_cast<const uint4 *>(img + tb[b].o01);
                cr[b][2] = *reinterpret_cast<const uint4 *>(img + tb[b].o10);
                cr[b][3] = *reinterpret_cast<const uint4 *>(img + tb[b].o11);
            }
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                if (!live[b] || !lane_on) continue;
                float va[kVec], vb[kVec], vc[kVec], ve[kVec];
                unpack<E, kVec>(cr[b][0], va);
                unpack<E, kVec>(cr[b][1], vb);
                unpack<E, kVec>(cr[b][2], vc);
                unpack<E, kVec>(cr[b][3], ve);
                float acc[kVec];
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    acc[e] = 0.0f;
                    acc[e] = fmaf(tb[b].w00, va[e], acc[e]);
                    acc[e] = fmaf(tb[b].w01, vb[e], acc[e]);
                    acc[e] = fmaf(tb[b].w10, vc[e], acc[e]);
                    acc[e] = fmaf(tb[b].w11, ve[e], acc[e]);
                }
                store_f32<E, kVec>(crow[b], acc);  // rows past P get zeros (weight 0)
            }
        }
    } else if (q < p.Q) {
        for (int it = wave * p.Q + q; it < nitems; it += per_pass) {
            const int pl = it / K, k = it - pl * K;
            const long long pg = p0 + pl;
            uint16_t *crow = col + (size_t)pg * p.Rp + (size_t)k * p.Cin_pad;
            if (pg >= p.P) {
                for (int ch = s; ch < p.nchunk; ch += p.S)
                    *reinterpret_cast<uint4 *>(crow + ch * kVec) = make_uint4(0, 0, 0, 0);
                continue;
            }
            const int n = s_pix[0][pl], ho = s_pix[1][pl], wo = s_pix[2][pl];
            const int i = k / p.kw, j = k - i * p.kw;
            const uint16_t *img = xt + (size_t)n * p.H * p.W * p.Cin_pad;
            for (int ch = s; ch < p.nchunk; ch += p.S) {
                const int ci0 = ch * kVec;
                const int g = min(ci0 / p.cpg, p.dg - 1);
                const float *so = s_off + ((pl * p.dg + g) * K + k) * 2;
                int y0, x0;
                float fy, fx;
                split_coord(ho * p.sh - p.ph + i * p.dh, so[1], y0, fy);
                split_coord(wo * p.sw - p.pw + j * p.dw, so[0], x0, fx);
                const Tap t = make_tap(y0, x0, fy, fx, s_m[(pl * p.dg + g) * K + k], p.H, p.W,
                                       p.Cin_pad);
                float acc[kVec];
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
                accumulate_tap<E, kVec>(img + ci0, t, acc);
                store_f32<E, kVec>(crow + ci0, acc);
            }
        }
    }
    // zero the reduction padding [R, Rp) of this block's rows
    const int padn = p.Rp - p.R;
    if (padn > 0) {
        for (int i = threadIdx.x; i < p.TP * padn; i += 256) {
            const int pl = i / padn, c = i % padn;
            const long long pg = p0 + pl;
            if (pg < p.Pp) col[(size_t)pg * p.Rp + p.R + c] = 0;
        }
    }
}

// ------------------------------------------------------------------ fused --
//
// Deform-im2col fused into the GEMM (implicit GEMM): the columns never reach memory.
// A block computes all kFBM output channels of kFBN output pixels. The K loop runs
// tap-major in steps of 64 channels of one tap (Cin_pad % 64 == 0); per step the
// column tile B ([kFBN pixels][64 channels], formed as m * bilinear in fp32 exactly as
// the deform-im2col stage forms it, rounded to the input type) sits in one of two LDS
// buffers as [pixel][8 chunks], chunk cc stored at cc ^ ((pixel >> 1) & 7) (the 16
// lanes of a fragment read hit 16 different 16-byte bank groups).

#ifndef DCN_V2_FUSED
#define DCN_V2_FUSED 1
#endif
constexpr int kFBM = 256;                    // output channels per block
constexpr int kFBN = 64;                     // output pixels per block
constexpr int kFBChunks = kFBN * kBK / 8;    // 512 of B

struct FusedParams {
    int N, H, W, Ho, Wo, kw, sh, sw, ph, pw, dh, dw;
    int dg, cpg, Cin_pad, K, CB, Rp, Mp;
    int Cout, HWo;
    long long P;
    int has_mask, softmax;
    int Mtiles, nblocks;
    unsigned xt_bytes;  // all of xt
    int tiles_x, tiles_y;  // 8x8 pixel tiles per image row / column (staged-region kernel)
};

// --------------------------------------------------- fused, specialised waves --
//
// The same implicit GEMM with the waves of a block split by role, so that the column
// arithmetic of one step runs on the VALUs while the MFMAs of the previous step run on
// the matrix cores of the same SIMDs. A block (kFBM output channels x kFBN pixels) has
// four MMA waves, one per SIMD, each owning 64 channels x 64 pixels (2 x 2 tiles of
// 32 x 32, 16 MFMAs per K step), and eight producer waves, two per SIMD.
//   - The MMA waves read their weight fragments straight from memory (L2: every block
//     reads the same permuted weight) into registers, one K step ahead, in the
//     operand layout of the MFMA: the weight never passes through LDS.
//   - Per K step the producers gather the column tile's corners DCN_V2_WS_STAGES steps
//     ahead, form m * bilinear in fp32 as the deform-im2col stage does, round it to
//     the input type and write it into one of two LDS buffers.
// One barrier per step hands the column buffers over. The barrier carries no memory
// fence: LDS writes are complete (lgkmcnt(0)) before it, and the weight loads still in
// flight are waited for only where their registers are used.
constexpr int kWSConsumers = 4;                           // MMA waves
constexpr int kWSProducers = 8;                           // producer waves
constexpr int kWSThreads = 64 * (kWSConsumers + kWSProducers);
constexpr int kWSPThreads = 64 * kWSProducers;            // 512: one B chunk each per step
static_assert(kWSPThreads == kFBChunks, "one column chunk per producer thread and step");
#ifndef DCN_V2_WS_STAGES
#define DCN_V2_WS_STAGES 2
#endif

template <class E>
__global__ __launch_bounds__(kWSThreads) void v2_ws_kernel(const uint16_t *__restrict__ xt,
                                                           const float *__restrict__ offset,
                                                           const float *__restrict__ mask,
                                                           const uint16_t *__restrict__ wp,
                                                           uint16_t *__restrict__ out,
                                                           const FusedParams p) {
    __shared__ uint4 sB[2][kFBChunks];
    extern __shared__ float smem[];  // offsets [kFBN][dg][K][2], then masks [kFBN][dg][K]
    const int K = p.K;
    const int per_pix = p.dg * K;
    float *s_off = smem;
    float *s_m = smem + kFBN * per_pix * 2;

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int mt = blk % p.Mtiles, nt = blk / p.Mtiles;
    const int m0 = mt * kFBM;
    const long long n0 = (long long)nt * kFBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long long HWo = p.HWo;

    for (int i = tid; i < kFBN * per_pix * 2; i += kWSThreads) {
        const int pl = i % kFBN, c = i / kFBN;
        const long long pg = n0 + pl;
        float v = 0.0f;
        if (pg < p.P) {
            const long long n = pg / HWo, r = pg % HWo;
            v = offset[((size_t)n * per_pix * 2 + c) * HWo + r];
        }
        s_off[pl * per_pix * 2 + c] = v;
    }
    for (int i = tid; i < kFBN * per_pix; i += kWSThreads) {
        const int pl = i % kFBN, c = i / kFBN;
        const long long pg = n0 + pl;
        float v = 1.0f;
        if (p.has_mask && pg < p.P) {
            const long long n = pg / HWo, r = pg % HWo;
            v = mask[((size_t)n * per_pix + c) * HWo + r];
        }
        s_m[pl * per_pix + c] = v;
    }
    __syncthreads();
    if (p.softmax) {
        for (int i = tid; i < kFBN * p.dg; i += kWSThreads) {
            float *ml = s_m + i * K;
            float mx = -INFINITY;
            for (int k = 0; k < K; ++k) mx = fmaxf(mx, ml[k]);
            float sum = 0.0f;
            for (int k = 0; k < K; ++k) sum += expf(ml[k] - mx);
            const float inv = 1.0f / sum;
            for (int k = 0; k < K; ++k) ml[k] = expf(ml[k] - mx) * inv;
        }
    }
    __syncthreads();
    const int NS = K * p.CB;

    if (wave >= kWSConsumers) {
        // ------------------------------------------------------------ producers --
        const int ptid = tid - 64 * kWSConsumers;
        const int br = ptid >> 3, bc = ptid & 7;
        const long long pg = n0 + br;
        const bool pvalid = pg < p.P;
        const long long pgc = pvalid ? pg : 0;
        const int n = (int)(pgc / HWo);
        const int rr = (int)(pgc - (long long)n * HWo);
        const int ho = rr / p.Wo, wo = rr - (rr / p.Wo) * p.Wo;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xt, p.xt_bytes);
        const int img_off = n * p.H * p.W * p.Cin_pad;
        const int bdst = br * 8 + (bc ^ ((br >> 1) & 7));
        struct Stage {
            uint4 g[4];
            float w[4];
        };
        int ld_n = 0, ld_k = 0, ld_i = 0, ld_j = 0, ld_cb = 0;
        int to[4];
        float tw[4];
        auto load = [&](Stage &st) __attribute__((always_inline)) {
            if (p.dg > 1 || ld_cb == 0) {
                const int grp = p.dg == 1 ? 0 : min((ld_cb * 64 + bc * 8) / p.cpg, p.dg - 1);
                const float *so = s_off + ((br * p.dg + grp) * K + ld_k) * 2;
                int y0, x0;
                float fy, fx;
                split_coord(ho * p.sh - p.ph + ld_i * p.dh, so[1], y0, fy);
                split_coord(wo * p.sw - p.pw + ld_j * p.dw, so[0], x0, fx);
                const float mk = pvalid ? s_m[(br * p.dg + grp) * K + ld_k] : 0.0f;
                const Tap tp = make_tap(y0, x0, fy, fx, mk, p.H, p.W, p.Cin_pad);
                const int cl = img_off + bc * 8;
                to[0] = (cl + tp.o00) * 2; to[1] = (cl + tp.o01) * 2;
                to[2] = (cl + tp.o10) * 2; to[3] = (cl + tp.o11) * 2;
                tw[0] = tp.w00; tw[1] = tp.w01; tw[2] = tp.w10; tw[3] = tp.w11;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                st.g[c] = buffer_load<uint4>(rx, to[c], ld_cb * kBK * 2);
                st.w[c] = tw[c];
            }
            if (ld_n < NS - 1) {
                ++ld_n;
                if (++ld_cb == p.CB) {
                    ld_cb = 0;
                    ++ld_k;
                    if (++ld_j == p.kw) {
                        ld_j = 0;
                        ++ld_i;
                    }
                }
            }
        };
        auto fill = [&](const Stage &st, int buf) __attribute__((always_inline)) {
            float acc[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float f[kVec];
                load_f32<E, kVec>(reinterpret_cast<const typename E::bits *>(&st.g[c]), f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] = fmaf(st.w[c], f[e], acc[e]);
            }
            typename E::bits b[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) b[e] = from_f32(E{}, acc[e]);
            uint4 v;
            __builtin_memcpy(&v, b, 16);
            sB[buf][bdst] = v;
        };
        constexpr int NST = DCN_V2_WS_STAGES;
        Stage st[NST];
#pragma unroll
        for (int i = 0; i < NST; ++i) load(st[i]);
        fill(st[0], 0);
        lds_barrier();  // step 0's column tile is in buffer 0
        for (int s = 0; s < NS; s += NST) {
#pragma unroll
            for (int u = 0; u < NST; ++u) {
                if (s + u >= NS) break;
                // buffer (s+u)&1 is being read by the MMA waves; fill the other
                load(st[u]);  // step min(s + u + NST, NS - 1)
                if (s + u + 1 < NS) fill(st[(u + 1) % NST], (s + u + 1) & 1);
                lds_barrier();
            }
        }
        return;
    }

    // ---------------------------------------------------------------- MMA waves --
    // Weight fragment of tile t, K sub-step ks of step s: lane l holds row
    // m0 + wave*64 + t*32 + (l & 31), elements [s*64 + ks*16 + (l >> 5)*8, +8), which the
    // prep stored (fragment order) as 1 KB per (32-row block, s, ks) with lane l's 16
    // bytes at 16 l: each load is one contiguous 1 KB. Rows past Mp read zeros.
    const int frow = lane & 31, fhalf = lane >> 5;
    const unsigned wp_bytes = (unsigned)((size_t)(p.Mp - m0) * p.Rp * 2);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(wp + (size_t)m0 * p.Rp, wp_bytes);
    int aoff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) aoff[t] = (wave * 2 + t) * p.Rp * 64 + lane * 16;
    // two register sets of fragments, used in turn: the loads of step s+1 are issued
    // as step s begins (past the last step a set reloads the last step's fragments:
    // unconditional loads keep the compiler's count of loads in flight exact)
    uint4 fa[2][2][4];  // [set][tile][ks]
    auto load_a = [&](uint4 (&f)[2][4], int s) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) f[t][ks] = buffer_load<uint4>(ra, aoff[t], (s * 4 + ks) * 1024);
    };
    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    auto mma = [&](const uint4 (&f)[2][4], int s) __attribute__((always_inline)) {
        const v4u *sb = reinterpret_cast<const v4u *>(sB[s & 1]);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int cc = 2 * ks + fhalf;
            v4u fb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rb = t * 32 + frow;
                fb[t] = sb[rb * 8 + (cc ^ ((rb >> 1) & 7))];
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = mfma32<E>(f[a][ks], __builtin_bit_cast(uint4, fb[b]), acc[a][b]);
        }
    };
    load_a(fa[0], 0);
    lds_barrier();  // step 0's column tile
    int s = 0;
    // (the empty asm statements keep the loads ahead of the step's LDS reads, so the
    // two sets stay distinct)
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
    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register
    // 4*(i/8) + i%4; row i is an output channel, column j an output pixel
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const long long po = n0 + b * 32 + (lane & 31);
        if (po >= p.P) continue;
        const long long nimg = po / HWo;
        const int hw = (int)(po - nimg * HWo);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = m0 + wave * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (co < p.Cout)
                    out[((size_t)nimg * p.Cout + co) * HWo + hw] = from_f32(E{}, acc[a][b][r]);
            }
        }
    }
}

// ------------------------------------------------- fused, staged region --
//
// The two-role kernel for 3x3 windows at stride 1 and dilation 1 with one deformable
// group. A block takes an 8 x 8 tile of output pixels and all kFBM output channels;
// the K loop runs channel-block-major: for 64-channel block c the nine taps in turn,
// step t = 9c + k reading weight rows k*Cin_pad + 64c .. +63 (the two-stage GEMM
// visits its K tiles in the same order for these layers, so both paths sum alike).
// Per channel block the producers copy the tile's receptive region of xt into LDS
// (kRW x kRW pixels x 64 channels: the tile's 3x3 bases +-kRHalo px and one more
// for the bilinear corner) with direct global->LDS copies, one channel block ahead
// in a second region buffer; a step's column corners are then four 16-byte LDS
// reads instead of four loads through the vector memory path. Taps whose corners
// leave the region (offsets beyond about +-6 px) read xt directly. A producer lane
// keeps its pixel's nine tap records (region cell, four weights) in registers for
// the whole K loop.
constexpr int kRT = 8;                                  // tile edge: kRT * kRT = kFBN pixels
constexpr int kRHalo = 6;
constexpr int kRW = kRT + 2 + 2 * kRHalo;               // 22: region edge in pixels
constexpr int kRChunks = kRW * kRW * 8;                 // 16-byte chunks per region
constexpr int kRCopies = (kRChunks + kWSPThreads - 1) / kWSPThreads;
static_assert(kRT * kRT == kFBN, "one pixel tile per block");
constexpr int kRK = 9;                                  // taps of the 3x3 window

template <class E>
__global__ __launch_bounds__(kWSThreads) void v2_wsr_kernel(const uint16_t *__restrict__ xt,
                                                            const float *__restrict__ offset,
                                                            const float *__restrict__ mask,
                                                            const uint16_t *__restrict__ wp,
                                                            uint16_t *__restrict__ out,
                                                            const FusedParams p) {
    __shared__ uint4 sR[2][kRChunks];    // region buffers, [pixel row][pixel][8 chunks]
    __shared__ uint4 sB[4][kFBChunks];   // column tiles (layout as in v2_ws_kernel), step t in t % 4
    __shared__ float s_off[kFBN * kRK * 2];
    __shared__ float s_m[kFBN * kRK];

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int mt = blk % p.Mtiles, tile = blk / p.Mtiles;
    const int tpi = p.tiles_x * p.tiles_y;
    const int n = tile / tpi, trest = tile - n * tpi;
    const int ty0 = (trest / p.tiles_x) * kRT, tx0 = (trest - (trest / p.tiles_x) * p.tiles_x) * kRT;
    const int m0 = mt * kFBM;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int HWo = p.HWo;
    const int ry0 = ty0 - p.ph - kRHalo, rx0 = tx0 - p.pw - kRHalo;
    const int CBn = p.CB;
    const int NS = kRK * CBn;

    // Region chunk i = 8 * (region pixel) + (16-byte chunk): its byte offset in xt, or an
    // offset past the end of the resource over xt (reads as zeros) outside the image
    auto region_voff = [&](int i) __attribute__((always_inline)) {
        const int q = i >> 3, cc = i & 7;
        const int ry = q / kRW, rx = q - ry * kRW;
        const int yy = ry0 + ry, xx = rx0 + rx;
        const bool ok = (unsigned)yy < (unsigned)p.H && (unsigned)xx < (unsigned)p.W;
        return ok ? ((n * p.H + yy) * p.W + xx) * p.Cin_pad * 2 + cc * 16 : (int)p.xt_bytes;
    };
    // Copy j (< kRCopies) of a producer lane moves region chunk j * 512 + (producer
    // thread) of channel block c into buffer b.
    const rsrc_words_t rxw = rsrc_words(xt, p.xt_bytes);
    auto region_copy = [&](int j, int c, int b) __attribute__((always_inline)) {
        const int i0 = j * kWSPThreads + (wave - kWSConsumers) * 64;
        if (i0 < kRChunks && i0 + lane < kRChunks)
            lds_copy16_buf(lds_addr(&sR[b][i0]), rxw, region_voff(i0 + lane), c * kBK * 2);
    };
    if (wave >= kWSConsumers) {  // region 0, waited for below
#pragma unroll
        for (int j = 0; j < kRCopies; ++j) region_copy(j, 0, 0);
    }
    // offsets and masks of the tile's pixels: pixel pl = 8 py + px
    for (int i = tid; i < kFBN * kRK * 2; i += kWSThreads) {
        const int pl = i % kFBN, c = i / kFBN;
        const int ho = ty0 + (pl >> 3), wo = tx0 + (pl & 7);
        float v = 0.0f;
        if (ho < p.Ho && wo < p.Wo) v = offset[((size_t)n * kRK * 2 + c) * HWo + ho * p.Wo + wo];
        s_off[pl * kRK * 2 + c] = v;
    }
    for (int i = tid; i < kFBN * kRK; i += kWSThreads) {
        const int pl = i % kFBN, c = i / kFBN;
        const int ho = ty0 + (pl >> 3), wo = tx0 + (pl & 7);
        float v = 1.0f;
        if (p.has_mask && ho < p.Ho && wo < p.Wo) v = mask[((size_t)n * kRK + c) * HWo + ho * p.Wo + wo];
        s_m[pl * kRK + c] = v;
    }
    V2_WAIT_VMCNT(0);  // region 0 has landed (this wave's copies)
    __syncthreads();
    if (p.softmax) {
        for (int i = tid; i < kFBN; i += kWSThreads) {
            float *ml = s_m + i * kRK;
            float mx = -INFINITY;
            for (int k = 0; k < kRK; ++k) mx = fmaxf(mx, ml[k]);
            float sum = 0.0f;
            for (int k = 0; k < kRK; ++k) sum += expf(ml[k] - mx);
            const float inv = 1.0f / sum;
            for (int k = 0; k < kRK; ++k) ml[k] = expf(ml[k] - mx) * inv;
        }
    }
    __syncthreads();

    if (wave >= kWSConsumers) {
        // ------------------------------------------------------------ producers --
        const int ptid = tid - 64 * kWSConsumers;
        const int br = ptid >> 3, bc = ptid & 7;
        const int ho = ty0 + (br >> 3), wo = tx0 + (br & 7);
        const bool pvalid = ho < p.Ho && wo < p.Wo;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(xt, p.xt_bytes);
        const int img_off = n * p.H * p.W * p.Cin_pad + bc * kVec;
        const int bdst = br * 8 + (bc ^ ((br >> 1) & 7));
        // tap records: region chunk of the (y0, x0) corner (this lane's 16 bytes), the
        // four weights as the deform-im2col stage forms them; `far` marks taps that
        // touch the image but leave the region
        int cell[kRK];
        float tw[kRK][4];
        unsigned far = 0;
#pragma unroll
        for (int k = 0; k < kRK; ++k) {
            const float *so = s_off + (br * kRK + k) * 2;
            int y0, x0;
            float fy, fx;
            split_coord(ho - p.ph + k / 3, so[1], y0, fy);
            split_coord(wo - p.pw + k % 3, so[0], x0, fx);
            const float mk = pvalid ? s_m[br * kRK + k] : 0.0f;
            const Tap tp = make_tap(y0, x0, fy, fx, mk, p.H, p.W, p.Cin_pad);
            const int ly = y0 - ry0, lx = x0 - rx0;
            const bool inreg = (unsigned)ly <= (unsigned)(kRW - 2) && (unsigned)lx <= (unsigned)(kRW - 2);
            const bool touch = (unsigned)(y0 + 1) <= (unsigned)p.H && (unsigned)(x0 + 1) <= (unsigned)p.W;
            far |= (pvalid && !inreg && touch) ? (1u << k) : 0u;
            cell[k] = inreg ? (ly * kRW + lx) * 8 + bc : bc;
            tw[k][0] = tp.w00; tw[k][1] = tp.w01; tw[k][2] = tp.w10; tw[k][3] = tp.w11;
        }
        // corners of step (c, k): LDS, or xt for a far tap
        auto load = [&](uint4 (&g)[4], int k, int c) __attribute__((always_inline)) {
            if (far & (1u << k)) {
                const float *so = s_off + (br * kRK + k) * 2;
                int y0, x0;
                float fy, fx;
                split_coord(ho - p.ph + k / 3, so[1], y0, fy);
                split_coord(wo - p.pw + k % 3, so[0], x0, fx);
                const Tap tp = make_tap(y0, x0, fy, fx, 1.0f, p.H, p.W, p.Cin_pad);
                g[0] = buffer_load<uint4>(rx, (img_off + tp.o00) * 2, c * kBK * 2);
                g[1] = buffer_load<uint4>(rx, (img_off + tp.o01) * 2, c * kBK * 2);
                g[2] = buffer_load<uint4>(rx, (img_off + tp.o10) * 2, c * kBK * 2);
                g[3] = buffer_load<uint4>(rx, (img_off + tp.o11) * 2, c * kBK * 2);
            } else {
                const uint4 *q = &sR[c & 1][cell[k]];
                g[0] = q[0];
                g[1] = q[8];
                g[2] = q[kRW * 8];
                g[3] = q[kRW * 8 + 8];
            }
        };
        auto fill = [&](const uint4 (&g)[4], int k, int buf) __attribute__((always_inline)) {
            float acc[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int cn = 0; cn < 4; ++cn) {
                float f[kVec];
                load_f32<E, kVec>(reinterpret_cast<const typename E::bits *>(&g[cn]), f);
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] = fmaf(tw[k][cn], f[e], acc[e]);
            }
            typename E::bits b[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) b[e] = from_f32(E{}, acc[e]);
            uint4 v;
            __builtin_memcpy(&v, b, 16);
            sB[buf][bdst] = v;
        };
        // Step t's corners sit in stage registers st[t % 3], loaded two steps ahead (9
        // steps per channel block keep t % 3 = k % 3); its column tile goes to sB[t & 1].
        // Region r sits in sR[r & 1]. Region c + 1 is copied during steps 0..5 of block c,
        // into the buffer that region c - 1 left (last read in step 6 of block c - 1),
        // one or two copies per step so that a wait for a far tap's corners finds the
        // copies of earlier steps landed; all are waited for in step 6 (the loads from
        // step 7 on read it).
        // One barrier per two steps: between barriers j and j + 1 the MMA waves take
        // tiles 2j and 2j + 1 and the producers fill tiles 2j + 2 and 2j + 3 (four
        // column-tile buffers, tile t in sB[t % 4]); barrier j follows step 2j + 1's
        // fill, so the K loop of NS steps has 1 + ceil(NS / 2) barriers in each role.
        uint4 st[3][4];
        load(st[0], 0, 0);
        load(st[1], 1, 0);
        for (int c = 0; c < CBn; ++c) {
#pragma unroll
            for (int k = 0; k < kRK; ++k) {
                const int u = c * kRK + k;
                if (u + 2 < NS) load(st[(k + 2) % 3], (k + 2) % kRK, c + (k + 2) / kRK);
                fill(st[k % 3], k, u & 3);
                if (c + 1 < CBn) {
                    static_assert(kRCopies <= 12, "two copies per step at most");
                    if (k < 6) region_copy(k, c + 1, (c + 1) & 1);
                    if (k < kRCopies - 6) region_copy(k + 6, c + 1, (c + 1) & 1);
                    // region c + 1 is first read by step 7's loads: wait before the last
                    // barrier ahead of them (after step 5 or 6, whichever is odd)
                    if ((k == 5 || k == 6) && (u & 1)) V2_WAIT_VMCNT(0);
                }
                if (u & 1) lds_barrier();
            }
        }
        lds_barrier();  // the MMA waves' last pair
        if (NS & 1) lds_barrier();
        return;
    }

    // ---------------------------------------------------------------- MMA waves --
    // As in v2_ws_kernel; step t = 9c + k takes the weight fragments of K block
    // k * CB + c.
    const int frow = lane & 31, fhalf = lane >> 5;
    const unsigned wp_bytes = (unsigned)((size_t)(p.Mp - m0) * p.Rp * 2);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(wp + (size_t)m0 * p.Rp, wp_bytes);
    int aoff[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) aoff[t] = (wave * 2 + t) * p.Rp * 64 + lane * 16;
    uint4 fa[2][2][4];  // [set][tile][ks]
    auto load_a = [&](uint4 (&f)[2][4], int t) __attribute__((always_inline)) {
        const int sw = (t % kRK) * CBn + t / kRK;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) f[u][ks] = buffer_load<uint4>(ra, aoff[u], (sw * 4 + ks) * 1024);
    };
    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    // The column fragments of K slice ks + 1 are read before the MFMAs of slice ks (the
    // scheduling barrier keeps the compiler from sinking the reads behind them), so an
    // LDS read's latency overlaps four MFMAs instead of stalling the next one.
    auto mma = [&](const uint4 (&f)[2][4], int t) __attribute__((always_inline)) {
        const v4u *sb = reinterpret_cast<const v4u *>(sB[t & 3]);
        v4u fb[2][2];
        auto rd = [&](v4u (&d)[2], int ks) __attribute__((always_inline)) {
            const int cc = 2 * ks + fhalf;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int rb = u * 32 + frow;
                d[u] = sb[rb * 8 + (cc ^ ((rb >> 1) & 7))];
            }
        };
        rd(fb[0], 0);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            if (ks + 1 < kBK / 16) rd(fb[(ks + 1) & 1], ks + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = mfma32<E>(f[a][ks], __builtin_bit_cast(uint4, fb[ks & 1][b]), acc[a][b]);
        }
    };
    load_a(fa[0], 0);
    lds_barrier();  // tiles 0 and 1
    int t = 0;
    for (; t + 1 < NS; t += 2) {
        load_a(fa[1], t + 1);
        asm volatile("" ::: "memory");
        mma(fa[0], t);
        load_a(fa[0], t + 2 < NS ? t + 2 : t + 1);
        asm volatile("" ::: "memory");
        mma(fa[1], t + 1);
        lds_barrier();
    }
    if (t < NS) {  // odd step count: the last step's fragments are in set 0
        mma(fa[0], t);
        lds_barrier();
    }
    // epilogue: column j of a 32x32 tile is tile pixel b*32 + j = 8 py + px
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int pl = b * 32 + (lane & 31);
        const int ho = ty0 + (pl >> 3), wo = tx0 + (pl & 7);
        if (ho >= p.Ho || wo >= p.Wo) continue;
        const int hw = ho * p.Wo + wo;
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = m0 + wave * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (co < p.Cout)
                    out[((size_t)n * p.Cout + co) * HWo + hw] = from_f32(E{}, acc[a][b][r]);
            }
        }
    }
}

// Layers taken by v2_wsr_kernel when fused; their two-stage GEMM visits the K tiles in
// the same channel-block-major order.
bool v2_region_order(const V2Launch &a) {
    return a.kh == 3 && a.kw == 3 && a.sh == 1 && a.sw == 1 && a.dh == 1 && a.dw == 1 && a.dg == 1 &&
           a.plan.Cin_pad % kBK == 0;
}

template <class E>
hipError_t launch_e(const V2Launch &a, hipStream_t stream) {
    const V2Plan &pl = a.plan;
    char *ws = static_cast<char *>(a.workspace);
    uint16_t *xt = reinterpret_cast<uint16_t *>(ws + pl.off_xt);
    // the fused kernel reads a pre-packed weight where the caller passes one
    const uint16_t *wp_in = static_cast<const uint16_t *>(a.packed_weight);
    uint16_t *wp = reinterpret_cast<uint16_t *>(ws + pl.off_wp);
    uint16_t *col = reinterpret_cast<uint16_t *>(ws + pl.off_col);

    // 1. prep
    PrepParams pp = {};
    pp.N = a.N; pp.Cin = a.Cin; pp.HW = a.H * a.W; pp.Cin_pad = pl.Cin_pad;
    pp.vec = (pp.HW % kVec == 0) && ((uintptr_t)a.x % 16 == 0);
    pp.Cout = a.Cout; pp.K = pl.K; pp.Mp = pl.Mp; pp.Rp = pl.Rp;
    pp.tiles_c = (pl.Cin_pad + 63) / 64;
    pp.tiles_hw = (pp.HW + 63) / 64;
    pp.n_tr_blocks = a.N * pp.tiles_c * pp.tiles_hw;
    // register transposes where the pixel rows are whole 16-byte vectors: one wave per
    // 64 channels x 64 pixels, four waves per block
    pp.reg = pp.vec;
    pp.cgroups = (pl.Cin_pad + 63) / 64;
    pp.hgroups = (pp.HW + 63) / 64;
    if (pp.reg) pp.n_tr_blocks = (a.N * pp.cgroups * pp.hgroups + 3) / 4;
    const bool fused = v2_fused_applies(pl, a.dg, a.weight != nullptr);
    pp.frag = fused ? 1 : 0;  // the fused kernel reads the weight in MFMA fragment order
    // one block per weight row; no weight (columns only) or a packed one: none
    const int nwb = (a.weight && !wp_in) ? pl.Mp : 0;
    pp.w_first = nwb > 0 ? 1 : 0;
    hipLaunchKernelGGL(v2_prep_kernel, dim3(pp.n_tr_blocks + nwb), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.weight),
                       xt, wp, pp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const size_t fused_lds = (size_t)kFBN * a.dg * pl.K * 3 * sizeof(float);
    if (fused) {  // 2+3. deform-im2col fused into the GEMM
        FusedParams fp;
        fp.N = a.N; fp.H = a.H; fp.W = a.W; fp.Ho = pl.Ho; fp.Wo = pl.Wo; fp.kw = a.kw;
        fp.sh = a.sh; fp.sw = a.sw; fp.ph = a.ph; fp.pw = a.pw; fp.dh = a.dh; fp.dw = a.dw;
        fp.dg = a.dg; fp.cpg = a.Cin / a.dg; fp.Cin_pad = pl.Cin_pad; fp.K = pl.K;
        fp.CB = pl.Cin_pad / kBK; fp.Rp = pl.Rp; fp.Mp = pl.Mp;
        fp.Cout = a.Cout; fp.HWo = pl.Ho * pl.Wo; fp.P = pl.P;
        fp.has_mask = a.mask != nullptr;
        fp.softmax = a.softmax ? 1 : 0;
        fp.Mtiles = (pl.Mp + kFBM - 1) / kFBM;
        fp.nblocks = (int)(fp.Mtiles * ((pl.P + kFBN - 1) / kFBN));
        fp.xt_bytes = (unsigned)((size_t)a.N * a.H * a.W * pl.Cin_pad * 2);
        const uint16_t *wf = wp_in ? wp_in : wp;
        if (v2_region_order(a)) {
            fp.tiles_x = (pl.Wo + kRT - 1) / kRT;
            fp.tiles_y = (pl.Ho + kRT - 1) / kRT;
            fp.nblocks = fp.Mtiles * a.N * fp.tiles_x * fp.tiles_y;
            hipLaunchKernelGGL(v2_wsr_kernel<E>, dim3(fp.nblocks), dim3(kWSThreads), 0, stream, xt, a.offset,
                               a.mask, wf, static_cast<uint16_t *>(a.out), fp);
        } else {
            hipLaunchKernelGGL(v2_ws_kernel<E>, dim3(fp.nblocks), dim3(kWSThreads), fused_lds, stream, xt,
                               a.offset, a.mask, wf, static_cast<uint16_t *>(a.out), fp);
        }
        return hipGetLastError();
    }

    // 2. im2col
    ColParams cp;
    cp.N = a.N; cp.H = a.H; cp.W = a.W; cp.Ho = pl.Ho; cp.Wo = pl.Wo;
    cp.kh = a.kh; cp.kw = a.kw; cp.sh = a.sh; cp.sw = a.sw; cp.ph = a.ph; cp.pw = a.pw;
    cp.dh = a.dh; cp.dw = a.dw; cp.dg = a.dg; cp.Cin = a.Cin; cp.Cin_pad = pl.Cin_pad;
    cp.cpg = a.Cin / a.dg;
    cp.K = pl.K; cp.R = pl.R; cp.Rp = pl.Rp; cp.P = pl.P; cp.Pp = pl.Pp;
    cp.has_mask = a.mask != nullptr;
    cp.softmax = a.softmax ? 1 : 0;
    cp.nchunk = pl.Cin_pad / kVec;
    cp.S = cp.nchunk < 64 ? cp.nchunk : 64;
    cp.Q = 64 / cp.S;
    cp.TP = 8;  // 4 waves x 2 items x 9 passes: many small blocks hide gather latency
    static_assert(8 <= kColMaxTP, "im2col block pixels");
    cp.nblocks = (int)((pl.Pp + cp.TP - 1) / cp.TP);
    cp.magic_k = (unsigned)(((1u << 20) + pl.K - 1) / pl.K);
    cp.magic_kw = (unsigned)(((1u << 20) + a.kw - 1) / a.kw);
    const size_t lds = (size_t)cp.TP * a.dg * pl.K * 3 * sizeof(float);
    hipLaunchKernelGGL(v2_im2col_kernel<E>, dim3(cp.nblocks), dim3(256), lds, stream, xt,
                       a.offset, a.mask, col, cp);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    if (!a.weight) return hipSuccess;  // columns only

    // 3. gemm
    GemmParams gp = {};
    gp.lda = pl.Rp; gp.ldb = pl.Rp;
    gp.nk = gp.nk_total = pl.Rp / kBK;
    gp.Cout = a.Cout; gp.HWo = pl.Ho * pl.Wo; gp.P = pl.P;
    gp.Mtiles = pl.Mp / kBM;
    gp.Ntiles = (int)(pl.Pp / kBN);
    gp.nblocks = gp.Mtiles * gp.Ntiles;
    if (v2_region_order(a)) {
        gp.perm_taps = pl.K;
        gp.perm_cb = pl.Cin_pad / kBK;
    }
    // short reductions (few K tiles): the two-slot ring, two blocks per CU
    if (gp.nk <= 8)
        hipLaunchKernelGGL((v2_gemm_kernel<E, 0, 2>), dim3(gp.nblocks), dim3(kGemmThreads), 0, stream, wp, col,
                           a.out, gp);
    else
        hipLaunchKernelGGL((v2_gemm_kernel<E, 0>), dim3(gp.nblocks), dim3(kGemmThreads), 0, stream, wp, col,
                           a.out, gp);
    return hipGetLastError();
}

}  // namespace

bool plan_dcn_v2(int N, int Cin, int H, int W, int Cout, int kh, int kw, int sh, int sw, int ph,
                 int pw, int dh, int dw, dcn_dtype dtype, V2Plan &pl) {
    if (dtype != DCN_F16 && dtype != DCN_BF16) return false;
    if (N < 0 || Cin <= 0 || H < 0 || W < 0 || Cout <= 0 || kh <= 0 || kw <= 0) return false;
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
    pl.Rp = (int)round_up(pl.R, kBK);
    pl.Pp = round_up(pl.P > 0 ? pl.P : 1, kBN);
    pl.Mp = (int)round_up(Cout, kBM);
    const size_t elt = 2;
    size_t off = 0;
    pl.off_xt = off;
    off = align256(off + (size_t)N * H * W * pl.Cin_pad * elt);
    pl.off_wp = off;
    off = align256(off + (size_t)pl.Mp * pl.Rp * elt);
    pl.off_col = off;
    off = align256(off + (size_t)pl.Pp * pl.Rp * elt);
    pl.total = off;
    // fused deform-im2col + GEMM: 64-channel steps within one tap, and byte offsets of
    // one image of xt and of the weight fit the 32-bit buffer range
    pl.fused = DCN_V2_FUSED && pl.Cin_pad % kBK == 0 &&
               (size_t)N * H * W * pl.Cin_pad * elt < (1ull << 31) &&
               (size_t)pl.Mp * pl.Rp * elt < (1ull << 31);
    return true;
}

bool v2_fused_applies(const V2Plan &pl, int dg, bool has_weight) {
    // the block's offsets and masks ([kFBN][dg][K] x 3 floats) fit its 64 KB of dynamic LDS
    return has_weight && pl.fused && (size_t)kFBN * dg * pl.K * 3 * sizeof(float) <= 64 * 1024;
}

hipError_t launch_dcn_v2_pack_weight(const void *weight, void *packed, int Cout, int Cin, const V2Plan &pl,
                                     hipStream_t stream) {
    PrepParams pp = {};
    pp.Cin = Cin; pp.Cin_pad = pl.Cin_pad;
    pp.Cout = Cout; pp.K = pl.K; pp.Mp = pl.Mp; pp.Rp = pl.Rp;
    pp.frag = 1;
    pp.n_tr_blocks = 0;  // weight rows only
    hipLaunchKernelGGL(v2_prep_kernel, dim3(pl.Mp), dim3(256), 0, stream, (const uint16_t *)nullptr,
                       static_cast<const uint16_t *>(weight), (uint16_t *)nullptr, static_cast<uint16_t *>(packed),
                       pp);
    return hipGetLastError();
}

hipError_t launch_dcn_v2(const V2Launch &a, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_BF16: return launch_e<EBF16>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcn
