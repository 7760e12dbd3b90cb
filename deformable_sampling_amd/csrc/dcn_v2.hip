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
};

template <class E>
__global__ __launch_bounds__(256) void v2_im2col_kernel(const uint16_t *__restrict__ xt,
                                                        const float *__restrict__ offset,
                                                        const float *__restrict__ mask,
                                                        uint16_t *__restrict__ col, ColParams p) {
    extern __shared__ float smem[];
    const int K = p.K;
    float *s_off = smem;                          // [TP][dg][K][2]
    float *s_m = smem + p.TP * p.dg * K * 2;      // [TP][dg][K]
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const long long p0 = (long long)blk * p.TP;
    const long long HWo = (long long)p.Ho * p.Wo;

    // 1. stage offsets / masks of this block's pixels (pixel-fastest: coalesced NCHW rows)
    const int per_pix = p.dg * K;
    for (int i = threadIdx.x; i < p.TP * per_pix * 2; i += 256) {
        const int pl = i % p.TP, c = i / p.TP;  // c = offset channel (g*K + k)*2 + xy
        const long long pg = p0 + pl;
        float v = 0.0f;
        if (pg < p.P) {
            const long long n = pg / HWo, r = pg % HWo;
            v = offset[((size_t)n * per_pix * 2 + c) * HWo + r];
        }
        s_off[pl * per_pix * 2 + c] = v;
    }
    for (int i = threadIdx.x; i < p.TP * per_pix; i += 256) {
        const int pl = i % p.TP, c = i / p.TP;
        const long long pg = p0 + pl;
        float v = 1.0f;
        if (p.has_mask && pg < p.P) {
            const long long n = pg / HWo, r = pg % HWo;
            v = mask[((size_t)n * per_pix + c) * HWo + r];
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
    if (q < p.Q) {
        for (int it = wave * p.Q + q; it < nitems; it += per_pass) {
            const int pl = it / K, k = it - pl * K;
            const long long pg = p0 + pl;
            uint16_t *crow = col + (size_t)pg * p.Rp + (size_t)k * p.Cin_pad;
            if (pg >= p.P) {
                for (int ch = s; ch < p.nchunk; ch += p.S)
                    *reinterpret_cast<uint4 *>(crow + ch * kVec) = make_uint4(0, 0, 0, 0);
                continue;
            }
            const int n = (int)(pg / HWo);
            const int r = (int)(pg % HWo);
            const int ho = r / p.Wo, wo = r % p.Wo;
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
// tap-major in steps of 64 channels of one tap (Cin_pad % 64 == 0). Per step:
//  - A (weight rows, [kFBM][64]) comes from wp in memory, loaded two steps ahead into
//    registers and written to one of two LDS buffers;
//  - B ([kFBN pixels][64 channels]) is computed: each thread owns one (pixel, 8-channel
//    chunk), gathers its four corners two steps ahead, and in the step before use forms
//    m * bilinear in fp32 exactly as the deform-im2col stage does, rounds it to the
//    input dtype and writes one 16-byte chunk of the B buffer;
//  - 8 waves (4 along channels x 2 along pixels, 64 x 32 each) run the MFMAs.
// Both operands sit in LDS as [row][8 chunks] with chunk cc stored at cc ^ ((row >> 1) & 7).

#ifndef DCN_V2_FUSED
#define DCN_V2_FUSED 1
#endif
constexpr int kFBM = 256;                    // output channels per block
constexpr int kFBN = 64;                     // output pixels per block
constexpr int kFThreads = 512;               // one B chunk per thread per step
constexpr int kFAChunks = kFBM * kBK / 8;    // 2048 16-byte chunks of A per step
constexpr int kFBChunks = kFBN * kBK / 8;    // 512 of B
constexpr int kFAPer = kFAChunks / kFThreads;  // A chunks per thread (4)
#ifndef DCN_V2_FUSED_STAGES
#define DCN_V2_FUSED_STAGES 2
#endif
constexpr int kFStages = DCN_V2_FUSED_STAGES;  // register stages of loads in flight

struct FusedParams {
    int N, H, W, Ho, Wo, kw, sh, sw, ph, pw, dh, dw;
    int dg, cpg, Cin_pad, K, CB, Rp, Mp;
    int Cout, HWo;
    long long P;
    int has_mask, softmax;
    int Mtiles, nblocks;
    unsigned xt_bytes;  // all of xt
};

template <class E>
__global__ __launch_bounds__(kFThreads) void v2_fused_kernel(const uint16_t *__restrict__ xt,
                                                             const float *__restrict__ offset,
                                                             const float *__restrict__ mask,
                                                             const uint16_t *__restrict__ wp,
                                                             uint16_t *__restrict__ out,
                                                             const FusedParams p) {
    __shared__ uint4 sA[2][kFAChunks];
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
    const int lane = tid & 63, wave = tid >> 6;
    const long long HWo = p.HWo;

    // offsets and masks of this block's pixels (pixel-fastest: coalesced NCHW rows)
    for (int i = tid; i < kFBN * per_pix * 2; i += kFThreads) {
        const int pl = i % kFBN, c = i / kFBN;
        const long long pg = n0 + pl;
        float v = 0.0f;
        if (pg < p.P) {
            const long long n = pg / HWo, r = pg % HWo;
            v = offset[((size_t)n * per_pix * 2 + c) * HWo + r];
        }
        s_off[pl * per_pix * 2 + c] = v;
    }
    for (int i = tid; i < kFBN * per_pix; i += kFThreads) {
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
    if (p.softmax) {  // softmax over K per (pixel, deformable group)
        for (int i = tid; i < kFBN * p.dg; i += kFThreads) {
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

    // this thread's B item: pixel row br, chunk bc (channels cb*64 + bc*8 .. +8)
    const int br = tid >> 3, bc = tid & 7;
    const long long pg = n0 + br;
    const bool pvalid = pg < p.P;
    const long long pgc = pvalid ? pg : 0;
    const int n = (int)(pgc / HWo);
    const int rr = (int)(pgc - (long long)n * HWo);
    const int ho = rr / p.Wo, wo = rr - (rr / p.Wo) * p.Wo;
    // one resource over all of xt (wave-uniform); the image is part of the lane offset
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xt, p.xt_bytes);
    const int img_off = n * p.H * p.W * p.Cin_pad;  // elements
    const unsigned wp_bytes = (unsigned)((size_t)(p.Mp - m0) * p.Rp * 2);  // rows m0 .. Mp-1
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(wp + (size_t)m0 * p.Rp, wp_bytes);
    const int bdst = br * 8 + (bc ^ ((br >> 1) & 7));

    // A chunk i of this thread: LDS position c = i*512 + tid, row c >> 3, logical
    // chunk (c & 7) ^ ((row >> 1) & 7); rows past Mp read past the buffer's end (zeros)
    int aoff[kFAPer];
#pragma unroll
    for (int i = 0; i < kFAPer; ++i) {
        const int c = i * kFThreads + tid;
        const int row = c >> 3, cc = (c & 7) ^ ((row >> 1) & 7);
        aoff[i] = (m0 + row < p.Mp) ? (row * p.Rp + cc * 8) * 2 : (int)wp_bytes;
    }

    // corner byte offsets (this thread's channels folded in) and weights of one tap
    struct TapB {
        int o[4];
        float w[4];
    };
    // Corners and weights of tap (i, j) for this thread's channels in 64-channel block cb
    // (the block's byte offset cb*128 is added by the loads' scalar offset).
    auto tap_of = [&](int k, int i, int j, int cb, TapB &t) __attribute__((always_inline)) {
        const int grp = p.dg == 1 ? 0 : min((cb * 64 + bc * 8) / p.cpg, p.dg - 1);
        const float *so = s_off + ((br * p.dg + grp) * K + k) * 2;
        int y0, x0;
        float fy, fx;
        split_coord(ho * p.sh - p.ph + i * p.dh, so[1], y0, fy);
        split_coord(wo * p.sw - p.pw + j * p.dw, so[0], x0, fx);
        const float mk = pvalid ? s_m[(br * p.dg + grp) * K + k] : 0.0f;
        const Tap tp = make_tap(y0, x0, fy, fx, mk, p.H, p.W, p.Cin_pad);
        const int cl = img_off + bc * 8;
        t.o[0] = (cl + tp.o00) * 2; t.o[1] = (cl + tp.o01) * 2;
        t.o[2] = (cl + tp.o10) * 2; t.o[3] = (cl + tp.o11) * 2;
        t.w[0] = tp.w00; t.w[1] = tp.w01; t.w[2] = tp.w10; t.w[3] = tp.w11;
    };
    struct Stage {
        uint4 a[kFAPer];
        uint4 g[4];
        float w[4];
    };
    const int NS = K * p.CB;
    // Loads run in step order 0, 1, ..., NS-1 (then NS-1 again): counters track the next
    // step's tap (k = i*kw + j) and 64-channel block cb, and the tap's corners and
    // weights are recomputed only when the tap changes (every step when dg > 1, where a
    // lane's group can change with the block).
    int ld_n = 0, ld_s = 0, ld_k = 0, ld_i = 0, ld_j = 0, ld_cb = 0;
    TapB tb;
    auto load = [&](Stage &st) __attribute__((always_inline)) {
        const int soff = ld_s * kBK * 2;  // this step's 64 columns of wp
#pragma unroll
        for (int i = 0; i < kFAPer; ++i) st.a[i] = buffer_load<uint4>(ra, aoff[i], soff);
        if (p.dg > 1 || ld_cb == 0) tap_of(ld_k, ld_i, ld_j, ld_cb, tb);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            st.g[c] = buffer_load<uint4>(rx, tb.o[c], ld_cb * kBK * 2);
            st.w[c] = tb.w[c];
        }
        if (ld_n < NS - 1) {  // after the last step, further loads repeat it (unused)
            ++ld_n;
            ++ld_s;
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
#pragma unroll
        for (int i = 0; i < kFAPer; ++i) sA[buf][i * kFThreads + tid] = st.a[i];
        // m * bilinear of 8 channels in fp32, in the deform-im2col stage's order
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

    f32x16_t acc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][r] = 0.0f;
    const int wm = wave & 3, wn = wave >> 2;  // 4 x 2 waves, 64 channels x 32 pixels each
    const int frow = lane & 31, fhalf = lane >> 5;
    // All 12 fragments of the step are read first; the empty asm takes them as in/out
    // operands, so the MFMAs (which use its outputs) start after a single wait instead of
    // each waiting for its own reads.
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    auto mma = [&](int buf) __attribute__((always_inline)) {
        const v4u *sa = reinterpret_cast<const v4u *>(sA[buf]);
        const v4u *sb = reinterpret_cast<const v4u *>(sB[buf]);
        v4u fa[4][2], fb[4];
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int cc = 2 * ks + fhalf;
            const int rb = wn * 32 + frow;
            fb[ks] = sb[rb * 8 + (cc ^ ((rb >> 1) & 7))];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ra_ = wm * 64 + t * 32 + frow;
                fa[ks][t] = sa[ra_ * 8 + (cc ^ ((ra_ >> 1) & 7))];
            }
        }
        asm volatile("" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[1][0]), "+v"(fa[1][1]),
                          "+v"(fa[2][0]), "+v"(fa[2][1]), "+v"(fa[3][0]), "+v"(fa[3][1]),
                          "+v"(fb[0]), "+v"(fb[1]), "+v"(fb[2]), "+v"(fb[3]));
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[t] = mfma32<E>(__builtin_bit_cast(uint4, fa[ks][t]),
                                   __builtin_bit_cast(uint4, fb[ks]), acc[t]);
    };

    // Step s: LDS buffers s & 1 hold step s; the NST register stages hold the next NST
    // steps. Load step s + NST into the stage step s used, run step s's MFMAs, then fill
    // the other buffers with step s + 1. Loads past the last step repeat it: no branches
    // around loads, so the compiler's wait counts stay exact.
    constexpr int NST = kFStages;
    Stage st[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) load(st[i]);
    fill(st[0], 0);
    auto step = [&](int s, Stage &mine, Stage &next) __attribute__((always_inline)) {
        __syncthreads();
        load(mine);  // step min(s + NST, NS - 1)
        mma(s & 1);
        if (s + 1 < NS) fill(next, (s + 1) & 1);
    };
    for (int s = 0; s < NS; s += NST) {
        step(s, st[0], st[1 % NST]);
        if (s + 1 >= NS) break;
        step(s + 1, st[1 % NST], st[2 % NST]);
        if constexpr (NST == 3) {
            if (s + 2 >= NS) break;
            step(s + 2, st[2], st[0]);
        }
    }

    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register
    // 4*(i/8) + i%4; row i is an output channel, column j an output pixel
    const long long po = n0 + wn * 32 + (lane & 31);
    if (po < p.P) {
        const long long nimg = po / HWo;
        const int hw = (int)(po - nimg * HWo);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = m0 + wm * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (co < p.Cout)
                    out[((size_t)nimg * p.Cout + co) * HWo + hw] = from_f32(E{}, acc[a][r]);
            }
        }
    }
}

template <class E>
hipError_t launch_e(const V2Launch &a, hipStream_t stream) {
    const V2Plan &pl = a.plan;
    char *ws = static_cast<char *>(a.workspace);
    uint16_t *xt = reinterpret_cast<uint16_t *>(ws + pl.off_xt);
    uint16_t *wp = reinterpret_cast<uint16_t *>(ws + pl.off_wp);
    uint16_t *col = reinterpret_cast<uint16_t *>(ws + pl.off_col);

    // 1. prep
    PrepParams pp;
    pp.N = a.N; pp.Cin = a.Cin; pp.HW = a.H * a.W; pp.Cin_pad = pl.Cin_pad;
    pp.vec = (pp.HW % kVec == 0) && ((uintptr_t)a.x % 16 == 0);
    pp.Cout = a.Cout; pp.K = pl.K; pp.Mp = pl.Mp; pp.Rp = pl.Rp;
    pp.tiles_c = (pl.Cin_pad + 63) / 64;
    pp.tiles_hw = (pp.HW + 63) / 64;
    pp.n_tr_blocks = a.N * pp.tiles_c * pp.tiles_hw;
    const long long wchunks = (long long)pl.Mp * (pl.Rp / kVec);
    const int nwb = a.weight ? (int)((wchunks + 255) / 256) : 0;  // no weight: columns only
    hipLaunchKernelGGL(v2_prep_kernel, dim3(pp.n_tr_blocks + nwb), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.weight),
                       xt, wp, pp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const size_t fused_lds = (size_t)kFBN * a.dg * pl.K * 3 * sizeof(float);
    if (a.weight && pl.fused && fused_lds <= 64 * 1024) {  // 2+3. deform-im2col fused into the GEMM
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
        hipLaunchKernelGGL(v2_fused_kernel<E>, dim3(fp.nblocks), dim3(kFThreads), fused_lds, stream, xt,
                           a.offset, a.mask, wp, static_cast<uint16_t *>(a.out), fp);
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
    cp.nblocks = (int)((pl.Pp + cp.TP - 1) / cp.TP);
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

hipError_t launch_dcn_v2(const V2Launch &a, hipStream_t stream) {
    switch (a.dtype) {
        case DCN_BF16: return launch_e<EBF16>(a, stream);
        case DCN_F16: return launch_e<EF16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcn
