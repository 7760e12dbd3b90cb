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

constexpr int kVec = 8;    // channel vector (16 bytes of bf16/fp16)
constexpr int kBM = 128;   // GEMM tile: output channels
constexpr int kBN = 128;   // GEMM tile: output pixels
constexpr int kBK = 64;    // GEMM tile: reduction

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

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt with only the vector-memory counter constrained to <= n (gfx9 encoding).
#define V2_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 0x3) << 14))

constexpr int kStages = 4;                          // K tiles in flight (LDS ring)
constexpr int kTileChunks = kBM * kBK / 8;          // 16-byte chunks per operand tile (1024)
constexpr int kDmaPerWave = kTileChunks / 256;      // direct-to-LDS copies per wave per operand (4)

// Operand tiles live in LDS as [128 rows][8 chunks of 8 elements], chunk cc of row r
// stored at position cc ^ (r & 7): the 8 lanes an LDS cycle serves (8 consecutive
// rows, same logical chunk) then hit 8 different 16-byte bank groups.
__shared__ uint4 s_gA0[kTileChunks], s_gA1[kTileChunks], s_gA2[kTileChunks], s_gA3[kTileChunks];
__shared__ uint4 s_gB0[kTileChunks], s_gB1[kTileChunks], s_gB2[kTileChunks], s_gB3[kTileChunks];
template <int S> __device__ __forceinline__ uint4 *ring_a() {
    if constexpr (S == 0) return s_gA0;
    else if constexpr (S == 1) return s_gA1;
    else if constexpr (S == 2) return s_gA2;
    else return s_gA3;
}
template <int S> __device__ __forceinline__ uint4 *ring_b() {
    if constexpr (S == 0) return s_gB0;
    else if constexpr (S == 1) return s_gB1;
    else if constexpr (S == 2) return s_gB2;
    else return s_gB3;
}
static_assert(kStages == 4, "the ring has four named slots");

// Copy a 128 x 64 operand tile (rows row0.., reduction k0..k0+63) into an LDS ring slot:
// wave w, copy i moves LDS chunks (i*4 + w)*64 + lane, i.e. row c >> 3, position c & 7.
__device__ __forceinline__ void gemm_dma(uint4 *slot, const uint16_t *g, int Rp, int k0) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int c = (i * 4 + w) * 64 + lane;
        const int row = c >> 3, pos = c & 7;
        const int cc = pos ^ (row & 7);
        const uint16_t *src = g + (size_t)row * Rp + k0 + cc * 8;
        lds_copy16(lds_addr(slot + (i * 4 + w) * 64), src);
    }
}

// One K step from ring slot S: wait until its tile has landed, barrier, refill the slot
// the previous step used with tile kt + kStages - 1, then 4 x (2 x 2) MFMAs.
template <class E, int S>
__device__ __forceinline__ void gemm_step(int kt, int nk, const uint16_t *ga, const uint16_t *gb, int Rp,
                                          f32x16_t (&acc)[2][2], int wm, int wn, int frow, int fhalf) {
    if (kt >= nk) return;
    // this wave's copies issued after tile kt: min(nk-1-kt, kStages-2) tiles x 2 operands
    const int after = (nk - 1 - kt) < (kStages - 2) ? (nk - 1 - kt) : (kStages - 2);
    if (after >= 2) V2_WAIT_VMCNT(2 * 2 * kDmaPerWave);
    else if (after == 1) V2_WAIT_VMCNT(1 * 2 * kDmaPerWave);
    else V2_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();  // all waves: tile kt in LDS, tile kt-1 consumed
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const int nx = kt + kStages - 1;
    if (nx < nk) {
        constexpr int R = (S + kStages - 1) % kStages;
        gemm_dma(ring_a<R>(), ga, Rp, nx * kBK);
        gemm_dma(ring_b<R>(), gb, Rp, nx * kBK);
    }
    const uint4 *sa = ring_a<S>();
    const uint4 *sb = ring_b<S>();
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
        const int cc = 2 * ks + fhalf;
        uint4 fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ra = wm * 64 + t * 32 + frow;
            const int rb = wn * 64 + t * 32 + frow;
            fa[t] = sa[ra * 8 + (cc ^ (ra & 7))];
            fb[t] = sb[rb * 8 + (cc ^ (rb & 7))];
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = mfma32<E>(fa[a], fb[b], acc[a][b]);
    }
}

// out[n][co][hw] = sum_r wp[co][r] * col[p][r] for a 128 (co) x 128 (p) tile; 4 waves in
// a 2 x 2 grid, each 64 x 64 = 2 x 2 v_mfma_f32_32x32x16 tiles with fp32 accumulators.
// The K loop runs over a kStages-deep ring of LDS tiles filled by direct global->LDS
// copies, so HBM/L2 latency overlaps the MFMA work of the previous stages.
template <class E>
__global__ __launch_bounds__(256) void v2_gemm_kernel(const uint16_t *__restrict__ wp,
                                                      const uint16_t *__restrict__ col,
                                                      uint16_t *__restrict__ out, GemmParams p) {
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int mt = blk % p.Mtiles, nt = blk / p.Mtiles;
    const int m0 = mt * kBM;
    const long long n0 = (long long)nt * kBN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;  // 2 x 2 waves, 64 x 64 each
    const uint16_t *ga = wp + (size_t)m0 * p.Rp;
    const uint16_t *gb = col + (size_t)n0 * p.Rp;

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int nk = p.Rp / kBK;
    // prologue: tiles 0 .. kStages-2 in flight
    if (0 < nk) { gemm_dma(ring_a<0>(), ga, p.Rp, 0); gemm_dma(ring_b<0>(), gb, p.Rp, 0); }
    if (1 < nk) { gemm_dma(ring_a<1>(), ga, p.Rp, kBK); gemm_dma(ring_b<1>(), gb, p.Rp, kBK); }
    if (2 < nk) { gemm_dma(ring_a<2>(), ga, p.Rp, 2 * kBK); gemm_dma(ring_b<2>(), gb, p.Rp, 2 * kBK); }
    // fragment of lane l in a 16-deep k step ks: row (l % 32), logical chunk 2*ks + l/32
    const int frow = lane & 31, fhalf = lane >> 5;
    for (int kt = 0; kt < nk; kt += kStages) {
        gemm_step<E, 0>(kt + 0, nk, ga, gb, p.Rp, acc, wm, wn, frow, fhalf);
        gemm_step<E, 1>(kt + 1, nk, ga, gb, p.Rp, acc, wm, wn, frow, fhalf);
        gemm_step<E, 2>(kt + 2, nk, ga, gb, p.Rp, acc, wm, wn, frow, fhalf);
        gemm_step<E, 3>(kt + 3, nk, ga, gb, p.Rp, acc, wm, wn, frow, fhalf);
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
    cp.TP = 8;  // 4 waves x 2 items x 9 passes: many small blocks hide gather latency
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
