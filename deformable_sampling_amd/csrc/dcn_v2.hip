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
//              block tiles, 64-deep K steps double-buffered through LDS,
//              v_mfma_f32_32x32x16 (bf16/fp16 in, fp32 accumulate).
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

constexpr int kVec = 8;    // channel vector (16 bytes of bf16/fp16)
constexpr int kBM = 128;   // GEMM tile: output channels
constexpr int kBN = 128;   // GEMM tile: output pixels
constexpr int kBK = 64;    // GEMM tile: reduction
constexpr int kLdsPad = 8; // elements of padding per LDS row (bank spreading)

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
long long round_up(long long v, long long m) { return (v + m - 1) / m * m; }

// ------------------------------------------------------------------- prep --

struct PrepParams {
    int N, Cin, HW, Cin_pad;
    int Cout, K, Mp, Rp;
    int n_tr_blocks;  // blocks doing the transpose; the rest permute the weight
    int tiles_c, tiles_hw;
};

// Transpose of 64 channels x 64 pixels through LDS, or 8 weight elements per thread.
__global__ __launch_bounds__(256) void v2_prep_kernel(const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ w,
                                                      uint16_t *__restrict__ xt,
                                                      uint16_t *__restrict__ wp, PrepParams p) {
    __shared__ uint16_t tile[64][66];
    const int b = blockIdx.x;
    if (b < p.n_tr_blocks) {
        const int tc = b % p.tiles_c;
        const int th = (b / p.tiles_c) % p.tiles_hw;
        const int n = b / (p.tiles_c * p.tiles_hw);
        const int c0 = tc * 64, hw0 = th * 64;
        const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
        const uint16_t *xn = x + (size_t)n * p.Cin * p.HW;
        for (int cy = ty; cy < 64; cy += 4) {
            const int c = c0 + cy, hw = hw0 + tx;
            tile[cy][tx] = (c < p.Cin && hw < p.HW) ? xn[(size_t)c * p.HW + hw] : (uint16_t)0;
        }
        __syncthreads();
        uint16_t *xtn = xt + (size_t)n * p.HW * p.Cin_pad;
        for (int py = ty; py < 64; py += 4) {
            const int hw = hw0 + py, c = c0 + tx;
            if (hw < p.HW && c < p.Cin_pad) xtn[(size_t)hw * p.Cin_pad + c] = tile[tx][py];
        }
        return;
    }
    // weight: wp[co][k*Cin_pad + ci] = w[co][ci][k]; 8 consecutive r per thread
    const long long t = (long long)(b - p.n_tr_blocks) * 256 + threadIdx.x;
    const int rv = p.Rp / kVec;
    if (t >= (long long)p.Mp * rv) return;
    const int co = (int)(t / rv);
    const int r0 = (int)(t % rv) * kVec;
    uint16_t v[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
        const int r = r0 + i;
        const int k = r / p.Cin_pad, ci = r % p.Cin_pad;
        v[i] = (co < p.Cout && k < p.K && ci < p.Cin) ? w[((size_t)co * p.Cin + ci) * p.K + k]
                                                      : (uint16_t)0;
    }
    uint4 o;
    __builtin_memcpy(&o, v, 16);
    *reinterpret_cast<uint4 *>(wp + (size_t)co * p.Rp + r0) = o;
}

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

// ------------------------------------------------------------------- gemm --

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <class E>
__device__ __forceinline__ f32x16_t mfma32(const uint4 &a, const uint4 &b, f32x16_t c) {
    if constexpr (E::id == DCN_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

struct GemmParams {
    int Cout, Rp, HWo, Mtiles;
    long long P;
    int nblocks;
};

constexpr int kLdsRow = kBK + kLdsPad;  // elements per LDS row

template <class E>
__global__ __launch_bounds__(256) void v2_gemm_kernel(const uint16_t *__restrict__ wp,
                                                      const uint16_t *__restrict__ col,
                                                      uint16_t *__restrict__ out, GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kBN * kLdsRow];

    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int mt = blk % p.Mtiles, nt = blk / p.Mtiles;
    const int m0 = mt * kBM;
    const long long n0 = (long long)nt * kBN;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave & 1, wn = wave >> 1;  // 2 x 2 waves, 64 x 64 each

    // global -> register staging: 128 rows x 64 elements = 1024 chunks of 16 B per
    // operand; thread t moves chunks t, t+256, t+512, t+768 (row = c/8, col = c%8).
    const uint16_t *ga = wp + (size_t)m0 * p.Rp;
    const uint16_t *gb = col + (size_t)n0 * p.Rp;
    uint4 ra[4], rb[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + i * 256, row = c >> 3, cc = (c & 7) * 8;
            ra[i] = *reinterpret_cast<const uint4 *>(ga + (size_t)row * p.Rp + k0 + cc);
            rb[i] = *reinterpret_cast<const uint4 *>(gb + (size_t)row * p.Rp + k0 + cc);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + i * 256, row = c >> 3, cc = (c & 7) * 8;
            *reinterpret_cast<uint4 *>(&sA[buf][row * kLdsRow + cc]) = ra[i];
            *reinterpret_cast<uint4 *>(&sB[buf][row * kLdsRow + cc]) = rb[i];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int nk = p.Rp / kBK;
    gload(0);
    sstore(0);
    __syncthreads();
    // fragment addressing: lane l reads row (l % 32), elements 8*(l/32) .. +8 of a
    // 16-deep k step.
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kBK);
        const uint16_t *a_base = &sA[buf][(wm * 64 + frow) * kLdsRow + fk];
        const uint16_t *b_base = &sB[buf][(wn * 64 + frow) * kLdsRow + fk];
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            uint4 fa[2], fb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                fa[t] = *reinterpret_cast<const uint4 *>(a_base + t * 32 * kLdsRow + ks);
                fb[t] = *reinterpret_cast<const uint4 *>(b_base + t * 32 * kLdsRow + ks);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma32<E>(fa[a], fb[b], acc[a][b]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register
    // 4*(i/8) + i%4. Row i is an output channel, column j an output pixel.
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const long long pg = n0 + wn * 64 + b * 32 + (lane & 31);
            if (pg >= p.P) continue;
            const long long nimg = pg / p.HWo;
            const int hw = (int)(pg - nimg * p.HWo);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int co = m0 + wm * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (co < p.Cout)
                    out[((size_t)nimg * p.Cout + co) * p.HWo + hw] = from_f32(E{}, acc[a][b][r]);
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
    pp.Cout = a.Cout; pp.K = pl.K; pp.Mp = pl.Mp; pp.Rp = pl.Rp;
    pp.tiles_c = (pl.Cin_pad + 63) / 64;
    pp.tiles_hw = (pp.HW + 63) / 64;
    pp.n_tr_blocks = a.N * pp.tiles_c * pp.tiles_hw;
    const long long wchunks = (long long)pl.Mp * (pl.Rp / kVec);
    const int nwb = (int)((wchunks + 255) / 256);
    hipLaunchKernelGGL(v2_prep_kernel, dim3(pp.n_tr_blocks + nwb), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(a.x), static_cast<const uint16_t *>(a.weight),
                       xt, wp, pp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

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
    cp.TP = 32;
    cp.nblocks = (int)((pl.Pp + cp.TP - 1) / cp.TP);
    const size_t lds = (size_t)cp.TP * a.dg * pl.K * 3 * sizeof(float);
    hipLaunchKernelGGL(v2_im2col_kernel<E>, dim3(cp.nblocks), dim3(256), lds, stream, xt,
                       a.offset, a.mask, col, cp);
    err = hipGetLastError();
    if (err != hipSuccess) return err;

    // 3. gemm
    GemmParams gp;
    gp.Cout = a.Cout; gp.Rp = pl.Rp; gp.HWo = pl.Ho * pl.Wo; gp.P = pl.P;
    gp.Mtiles = pl.Mp / kBM;
    gp.nblocks = (int)(gp.Mtiles * (pl.Pp / kBN));
    hipLaunchKernelGGL(v2_gemm_kernel<E>, dim3(gp.nblocks), dim3(256), 0, stream, wp, col,
                       static_cast<uint16_t *>(a.out), gp);
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
