// Pieces shared by the DCNv2 forward and backward, included inside namespace dcn's
// anonymous namespace by each, after dcn_common.hpp: tile constants, the NCHW ->
// channels-last transpose with the weight permutation, and the MFMA GEMM over
// K-contiguous operands.
#pragma once

constexpr int kVec = 8;    // channel vector (16 bytes of bf16/fp16)
constexpr int kBM = 128;   // GEMM tile: output channels
constexpr int kBN = 128;   // GEMM tile: output pixels
constexpr int kBK = 64;    // GEMM tile: reduction

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
long long round_up(long long v, long long m) { return (v + m - 1) / m * m; }

// ------------------------------------------------------------------- prep --

struct PrepParams {
    int N, Cin, HW, Cin_pad;
    int vec;  // 16-byte transpose path: HW % 8 == 0 and x 16-byte aligned
    int reg;  // register transpose (implies vec): blocks of 4 waves, each wave 64 x 64
    int cgroups, hgroups;  // register transpose: 64-channel and 64-pixel groups per image
    int Cout, K, Mp, Rp;
    int frag;         // weight in MFMA fragment order (see below) instead of rows [Mp][Rp]
    int n_tr_blocks;  // blocks doing the transpose; the rest (Mp of them) permute the weight
    int w_first;      // launch order: the weight rows' blocks first (their load -> LDS ->
                      // permute chain is the longer one), then the transpose blocks
    int tiles_c, tiles_hw;
};

// Transpose of 64 channels x 64 pixels through LDS, or 8 weight elements per thread.
__global__ __launch_bounds__(256) void v2_prep_kernel(const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ w,
                                                      uint16_t *__restrict__ xt,
                                                      uint16_t *__restrict__ wp, PrepParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // [channel][pixel], 144-byte rows
    int b = blockIdx.x;
    if (p.w_first) b = b < p.Mp ? p.n_tr_blocks + b : b - p.Mp;
    if (b < p.n_tr_blocks && p.reg) {
        // 8 x 8 transposes in registers: lane (cl, hl) of a wave loads the 8 channel rows
        // cb*8..+7 over the 8 pixels hb*8..+7 (16 bytes each; the wave's 8 lanes of one
        // row read 128 contiguous bytes), swaps 16-bit halves with byte permutes, and
        // stores 8 pixels of 8 channels (8 lanes write 128 contiguous bytes of a pixel).
        const int wave = b * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
        const int hg = wave % p.hgroups, cg = (wave / p.hgroups) % p.cgroups;
        const int n = wave / (p.hgroups * p.cgroups);
        if (n >= p.N) return;  // no barrier in this path
        const int cb = cg * 8 + (lane & 7), hb = hg * 8 + (lane >> 3);
        if (cb * 8 >= p.Cin_pad || hb * 8 >= p.HW) return;
        const uint16_t *xn = x + (size_t)n * p.Cin * p.HW + (size_t)hb * 8;
        uint4 r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = cb * 8 + i;
            r[i] = c < p.Cin ? *reinterpret_cast<const uint4 *>(xn + (size_t)c * p.HW) : make_uint4(0, 0, 0, 0);
        }
        uint16_t *dst = xt + ((size_t)n * p.HW + (size_t)hb * 8) * p.Cin_pad + cb * 8;
        auto dw = [](const uint4 &v, int d) { return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w; };
#pragma unroll
        for (int px = 0; px < 8; ++px) {
            // pixel px sits in dword px/2 of every row, low half for even px
            const unsigned sel = (px & 1) ? 0x07060302u : 0x05040100u;
            unsigned o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = __builtin_amdgcn_perm(dw(r[2 * q + 1], px >> 1), dw(r[2 * q], px >> 1), sel);
            *reinterpret_cast<uint4 *>(dst + (size_t)px * p.Cin_pad) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        return;
    }
    if (b < p.n_tr_blocks) {
        const int tc = b % p.tiles_c;
        const int th = (b / p.tiles_c) % p.tiles_hw;
        const int n = b / (p.tiles_c * p.tiles_hw);
        const int c0 = tc * 64, hw0 = th * 64;
        const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
        const uint16_t *xn = x + (size_t)n * p.Cin * p.HW;
        if (p.vec) {
            // 16-byte accesses: a thread loads 8 pixels of one channel, then stores 8
            // channels of one pixel
            const int q = threadIdx.x & 7, r = threadIdx.x >> 3;  // 8 chunks x 32 rows
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = c0 + r + 32 * j, hw = hw0 + q * kVec;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c < p.Cin && hw < p.HW)
                    v = *reinterpret_cast<const uint4 *>(xn + (size_t)c * p.HW + hw);
                *reinterpret_cast<uint4 *>(&tile[r + 32 * j][q * kVec]) = v;
            }
            __syncthreads();
            uint16_t *xtn = xt + (size_t)n * p.HW * p.Cin_pad;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int hw = hw0 + r + 32 * j, c = c0 + q * kVec;
                uint16_t e[kVec];
#pragma unroll
                for (int i = 0; i < kVec; ++i) e[i] = tile[q * kVec + i][r + 32 * j];
                uint4 v;
                __builtin_memcpy(&v, e, 16);
                if (hw < p.HW && c < p.Cin_pad)
                    *reinterpret_cast<uint4 *>(xtn + (size_t)hw * p.Cin_pad + c) = v;
            }
            return;
        }
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
    // weight: wp[co][k*Cin_pad + ci] = w[co][ci][k], one row co per block. Rows of up
    // to 4608 elements are first copied into LDS with coalesced 16-byte loads (the
    // permutation then reads LDS at stride K), longer ones are read from memory directly;
    // each thread writes 8 consecutive r as one 16-byte store. With frag set, the eight
    // values (co, r0..r0+7), r0 = 64 s + 16 ks + 8 h, go to 16-byte slot
    // (((co/32 * Rp/64 + s) * 4 + ks) * 2 + h) * 32 + co%32: the operand of one
    // 32x32x16 MFMA (32 rows x 16 K values) is then 1 KB of consecutive memory, lane
    // l's 16 bytes at 16 l.
    const int co = b - p.n_tr_blocks;
    if (co >= p.Mp) return;
    const int rowlen = p.Cin * p.K;
    const bool real = co < p.Cout;
    const uint16_t *wr = w + (size_t)(real ? co : 0) * rowlen;
    uint16_t *row = &tile[0][0];
    const bool staged = real && rowlen <= 64 * 72;
    if (staged) {
        const bool v16 = rowlen % kVec == 0 && ((uintptr_t)wr % 16) == 0;
        if (v16) {
            for (int i = threadIdx.x; i < rowlen / kVec; i += 256)
                reinterpret_cast<uint4 *>(row)[i] = reinterpret_cast<const uint4 *>(wr)[i];
        } else {
            for (int i = threadIdx.x; i < rowlen; i += 256) row[i] = wr[i];
        }
    }
    __syncthreads();
    for (int r0 = threadIdx.x * kVec; r0 < p.Rp; r0 += 256 * kVec) {
        // Cin_pad is a multiple of kVec: the 8 values share their tap k
        const int k = r0 / p.Cin_pad, ci0 = r0 - k * p.Cin_pad;
        uint16_t v[kVec];
#pragma unroll
        for (int i = 0; i < kVec; ++i) {
            const int ci = ci0 + i;
            const bool in = real && k < p.K && ci < p.Cin;
            const int e = in ? ci * p.K + k : 0;
            v[i] = in ? (staged ? row[e] : wr[e]) : (uint16_t)0;
        }
        uint4 o;
        __builtin_memcpy(&o, v, 16);
        size_t dst = (size_t)co * p.Rp + r0;
        if (p.frag) {
            const int c8 = r0 / kVec;  // s = c8 / 8, ks = (c8 / 2) % 4, h = c8 % 2
            dst = (((((size_t)(co / 32) * (p.Rp / 64) + c8 / 8) * 4 + (c8 / 2) % 4) * 2 + c8 % 2) * 32 + co % 32) *
                  kVec;
        }
        *reinterpret_cast<uint4 *>(wp + dst) = o;
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

// C[m][n] = sum_k A[m][k] * B[n][k] over 128 x 128 tiles; A and B hold K contiguous
// (row strides lda, ldb, rows padded to whole tiles, K to whole 64-deep steps).
// Split-K: block (mt, nt, split) takes K steps [split*nk, min((split+1)*nk, nk_total)).
// MODE 0 stores out[img][m][hw] in the input dtype (n = img*HWo + hw, m < Cout,
// n < P: the DCNv2 forward's NCHW output); MODE 1 stores fp32 out[split*split_stride +
// m*ldc + n] for m < Mstore, n < Nstore.
struct GemmParams {
    int lda, ldb, nk, nk_total;
    int Mtiles, Ntiles, nblocks;
    int Cout, HWo;
    long long P;
    int ldc, Mstore, Nstore;
    long long split_stride;
    // K tile order: natural (perm_taps 0), or channel-block-major over taps: step kt
    // takes tile (kt % perm_taps) * perm_cb + kt / perm_taps (perm_taps * perm_cb tiles)
    int perm_taps, perm_cb;
};

__device__ __forceinline__ int gemm_ktile(const GemmParams &p, int kt) {
    return p.perm_taps ? (kt % p.perm_taps) * p.perm_cb + kt / p.perm_taps : kt;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// s_waitcnt with only the vector-memory counter constrained to <= n (gfx9 encoding).
#define V2_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (0x7 << 4) | (0xF << 8) | ((((n) >> 4) & 0x3) << 14))

// Barrier after this wave's LDS accesses have completed; global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

constexpr int kStages = 4;                          // K tiles in flight (LDS ring), at most
constexpr int kTileChunks = kBM * kBK / 8;          // 16-byte chunks per operand tile (1024)
// Waves per GEMM block: 8 (2 x 4, 64 x 32 each: two per SIMD, so one wave's LDS
// waits overlap the other's MFMAs) or 4 (2 x 2, 64 x 64 each).
#ifndef DCN_V2_GEMM_WAVES
#define DCN_V2_GEMM_WAVES 8
#endif
constexpr int kGemmWaves = DCN_V2_GEMM_WAVES;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kDmaPerWave = kTileChunks / kGemmThreads;  // direct-to-LDS copies per wave per operand
constexpr int kWaveN = kBN / (kGemmWaves / 2);           // pixels per wave (64 or 32)
constexpr int kTB = kWaveN / 32;                         // 32-wide MFMA tiles per wave along N

// Operand tiles live in LDS as [128 rows][8 chunks of 8 elements], chunk cc of row r
// stored at position cc ^ ((r >> 1) & 7). A 16-byte read by 64 lanes is served 16 lanes
// (256 bytes, all 64 banks) at a time; the 16 lanes of a fragment read take 16
// consecutive rows of one logical chunk, and the swizzle puts them on 16 different
// 16-byte bank groups (two rows share a 256-byte bank period).
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
// A kernel instance with NS = 2 uses slots 0 and 1 only, so it holds 64 KB of LDS and
// two blocks share a CU: for short reductions (a few K tiles), where a block's loads
// and stores then overlap the other block's MFMAs.

// Copy a 128 x 64 operand tile (rows row0.., reduction k0..k0+63) into an LDS ring slot:
// wave w, copy i moves LDS chunks (i*W + w)*64 + lane, i.e. row c >> 3, position c & 7.
__device__ __forceinline__ void gemm_dma(uint4 *slot, const uint16_t *g, int ld, int k0) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
        const int c = (i * kGemmWaves + w) * 64 + lane;
        const int row = c >> 3, pos = c & 7;
        const int cc = pos ^ ((row >> 1) & 7);
        const uint16_t *src = g + (size_t)row * ld + k0 + cc * 8;
        lds_copy16(lds_addr(slot + (i * kGemmWaves + w) * 64), src);
    }
}

// One K step from ring slot S of an NS-slot ring: wait until its tile has landed,
// barrier, refill the slot the previous step used with tile kt + NS - 1, then
// 4 x (2 x kTB) MFMAs.
template <class E, int S, int NS>
__device__ __forceinline__ void gemm_step(int kt, int nk, const uint16_t *ga, const uint16_t *gb,
                                          const GemmParams &p, f32x16_t (&acc)[2][kTB], int wm, int wn,
                                          int frow, int fhalf) {
    if (kt >= nk) return;
    // this wave's copies issued after tile kt: min(nk-1-kt, NS-2) tiles x 2 operands
    const int after = (nk - 1 - kt) < (NS - 2) ? (nk - 1 - kt) : (NS - 2);
    if (after >= 2) V2_WAIT_VMCNT(2 * 2 * kDmaPerWave);
    else if (after == 1) V2_WAIT_VMCNT(1 * 2 * kDmaPerWave);
    else V2_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();  // all waves: tile kt in LDS, tile kt-1 consumed
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const int nx = kt + NS - 1;
    if (nx < nk) {
        constexpr int R = (S + NS - 1) % NS;
        const int k0 = gemm_ktile(p, nx) * kBK;
        gemm_dma(ring_a<R>(), ga, p.lda, k0);
        gemm_dma(ring_b<R>(), gb, p.ldb, k0);
    }
    const uint4 *sa = ring_a<S>();
    const uint4 *sb = ring_b<S>();
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
        const int cc = 2 * ks + fhalf;
        uint4 fa[2], fb[kTB];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int ra = wm * 64 + t * 32 + frow;
            fa[t] = sa[ra * 8 + (cc ^ ((ra >> 1) & 7))];
        }
#pragma unroll
        for (int t = 0; t < kTB; ++t) {
            const int rb = wn * kWaveN + t * 32 + frow;
            fb[t] = sb[rb * 8 + (cc ^ ((rb >> 1) & 7))];
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < kTB; ++b) acc[a][b] = mfma32<E>(fa[a], fb[b], acc[a][b]);
    }
}

// One 128 x 128 tile of C (see GemmParams); the waves form a 2 x (W/2) grid, each
// 64 x kWaveN = 2 x kTB v_mfma_f32_32x32x16 tiles with fp32 accumulators. The K loop
// runs over a kStages-deep ring of LDS tiles filled by direct global->LDS copies, so
// HBM/L2 latency overlaps the MFMA work of the previous stages.
template <class E, int MODE, int NS = kStages>
__global__ __launch_bounds__(kGemmThreads) void v2_gemm_kernel(const uint16_t *__restrict__ A,
                                                      const uint16_t *__restrict__ B,
                                                      void *__restrict__ out, GemmParams p) {
    const int blk = xcd_remap((int)blockIdx.x, p.nblocks);
    const int mt = blk % p.Mtiles, rest = blk / p.Mtiles;
    const int nt = rest % p.Ntiles, split = rest / p.Ntiles;
    const int m0 = mt * kBM;
    const long long n0 = (long long)nt * kBN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;  // 2 x (W/2) waves, 64 x kWaveN each
    const int kt0 = split * p.nk;
    const int nk = min(p.nk, p.nk_total - kt0);
    const uint16_t *ga = A + (size_t)m0 * p.lda + (size_t)kt0 * kBK;
    const uint16_t *gb = B + (size_t)n0 * p.ldb + (size_t)kt0 * kBK;

    f32x16_t acc[2][kTB];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < kTB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    static_assert(NS == 2 || NS == 4, "ring of two or four slots");
    // prologue: tiles 0 .. NS-2 in flight
    if (0 < nk) {
        const int k0 = gemm_ktile(p, 0) * kBK;
        gemm_dma(ring_a<0>(), ga, p.lda, k0);
        gemm_dma(ring_b<0>(), gb, p.ldb, k0);
    }
    if constexpr (NS == 4) {
        if (1 < nk) {
            const int k0 = gemm_ktile(p, 1) * kBK;
            gemm_dma(ring_a<1>(), ga, p.lda, k0);
            gemm_dma(ring_b<1>(), gb, p.ldb, k0);
        }
        if (2 < nk) {
            const int k0 = gemm_ktile(p, 2) * kBK;
            gemm_dma(ring_a<2>(), ga, p.lda, k0);
            gemm_dma(ring_b<2>(), gb, p.ldb, k0);
        }
    }
    // fragment of lane l in a 16-deep k step ks: row (l % 32), logical chunk 2*ks + l/32
    const int frow = lane & 31, fhalf = lane >> 5;
    for (int kt = 0; kt < nk; kt += NS) {
        gemm_step<E, 0, NS>(kt + 0, nk, ga, gb, p, acc, wm, wn, frow, fhalf);
        gemm_step<E, 1, NS>(kt + 1, nk, ga, gb, p, acc, wm, wn, frow, fhalf);
        if constexpr (NS == 4) {
            gemm_step<E, 2, NS>(kt + 2, nk, ga, gb, p, acc, wm, wn, frow, fhalf);
            gemm_step<E, 3, NS>(kt + 3, nk, ga, gb, p, acc, wm, wn, frow, fhalf);
        }
    }

    // epilogue: D[i][j] of a 32x32 tile sits in lane j + 32*((i/4)%2), register
    // 4*(i/8) + i%4. Row i indexes m, column j indexes n.
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < kTB; ++b) {
            const long long n = n0 + wn * kWaveN + b * 32 + (lane & 31);
            if constexpr (MODE == 0) {
                if (n >= p.P) continue;
                const long long nimg = n / p.HWo;
                const int hw = (int)(n - nimg * p.HWo);
                typename E::bits *o = static_cast<typename E::bits *>(out);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int co = m0 + wm * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (co < p.Cout) o[((size_t)nimg * p.Cout + co) * p.HWo + hw] = from_f32(E{}, acc[a][b][r]);
                }
            } else {
                if (n >= p.Nstore) continue;
                float *o = static_cast<float *>(out) + (size_t)split * p.split_stride;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * 64 + a * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (m < p.Mstore) o[(size_t)m * p.ldc + n] = acc[a][b][r];
                }
            }
        }
    }
}

