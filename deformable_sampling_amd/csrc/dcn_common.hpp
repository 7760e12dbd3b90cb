// Device helpers shared by the deformable-sampling kernels (gfx950 / CDNA4).
//
// Element types are handled as raw bits: fp32, fp16 (IEEE binary16) and bf16.
// Loads and stores move 2/4/8/16 bytes per lane; arithmetic is always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn.h"

namespace dcn {

// ---------------------------------------------------------------- elements --

struct EF32 { using bits = uint32_t; static constexpr dcn_dtype id = DCN_F32; };
struct EF16 { using bits = uint16_t; static constexpr dcn_dtype id = DCN_F16; };
struct EBF16 { using bits = uint16_t; static constexpr dcn_dtype id = DCN_BF16; };

__device__ __forceinline__ float to_f32(EF32, uint32_t b) { return __uint_as_float(b); }
__device__ __forceinline__ float to_f32(EF16, uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float to_f32(EBF16, uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint32_t from_f32(EF32, float f) { return __float_as_uint(f); }
__device__ __forceinline__ uint16_t from_f32(EF16, float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}
__device__ __forceinline__ uint16_t from_f32(EBF16, float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
}

// Raw vector of BYTES bytes.
template <int BYTES> struct Raw;
template <> struct Raw<16> { using t = uint4; };
template <> struct Raw<8> { using t = uint2; };
template <> struct Raw<4> { using t = uint32_t; };
template <> struct Raw<2> { using t = uint16_t; };

// Load V consecutive elements starting at p (aligned to V*sizeof) as fp32.
template <class E, int V>
__device__ __forceinline__ void load_f32(const typename E::bits *p, float (&f)[V]) {
    using B = typename E::bits;
    constexpr int BYTES = V * (int)sizeof(B);
    using R = typename Raw<BYTES>::t;
    R r = *reinterpret_cast<const R *>(p);
    B b[V];
    __builtin_memcpy(b, &r, BYTES);
#pragma unroll
    for (int i = 0; i < V; ++i) f[i] = to_f32(E{}, b[i]);
}

// The V = 16/sizeof elements of one 16-byte chunk as fp32.
template <class E, int V>
__device__ __forceinline__ void unpack(const uint4 &r, float (&f)[V]) {
    using B = typename E::bits;
    B b[V];
    __builtin_memcpy(b, &r, 16);
#pragma unroll
    for (int i = 0; i < V; ++i) f[i] = to_f32(E{}, b[i]);
}

// Store V fp32 values as V consecutive elements at p (aligned to V*sizeof).
template <class E, int V>
__device__ __forceinline__ void store_f32(typename E::bits *p, const float (&f)[V]) {
    using B = typename E::bits;
    constexpr int BYTES = V * (int)sizeof(B);
    using R = typename Raw<BYTES>::t;
    B b[V];
#pragma unroll
    for (int i = 0; i < V; ++i) b[i] = from_f32(E{}, f[i]);
    R r;
    __builtin_memcpy(&r, b, BYTES);
    *reinterpret_cast<R *>(p) = r;
}

// ---------------------------------------------------------------- bilinear --

// a * b rounded to fp32 by itself. hipcc contracts a*b +- c into one FMA by default
// and __fmul_rn is a plain multiply here, so a position such as fl32(u*W) - 0.5 or
// fl32(s*d) - floor(...) could otherwise be formed with a single rounding. An
// explicit fma with a zero addend is the correctly rounded product (a*b + 0 rounded
// once), and an fma is never fused into a following add.
__device__ __forceinline__ float mul_rn(float a, float b) { return __builtin_fmaf(a, b, 0.0f); }

// Split a sampling coordinate base + t (base integer, t fp32) into the integer
// corner c0 = base + floor(t) and the fraction f = t - floor(t). The fraction is
// exact in fp32 except for t in (-1/2, 0), where f = 1 + t is rounded (by at most
// 2^-25), so the position is never rounded to the grid's precision. |t| is clamped
// at 2^24 px: such taps are outside any image this library accepts, so clamping
// changes nothing.
__device__ __forceinline__ void split_coord(int base, float t, int &c0, float &f) {
    t = fminf(fmaxf(t, -16777216.0f), 16777216.0f);
    float fl = floorf(t);
    f = t - fl;
    c0 = base + (int)fl;
}

// base + t -> corner c0 = base + floor(t), f = t - floor(t), u = (floor(t) + 1) - t.
// Each of f and u is exact whenever it is below 1/2 (f = 1 + t rounds only for t in
// (-1/2, 0), where u = -t is exact; u = 1 - t rounds only for t in (0, 1/2), where f
// = t is exact), so both bilinear weight factors carry a relative error of at most
// one rounding. Deriving u as 1 - f instead would give a small u an absolute error
// of up to 2^-25, and a large relative one. |t| is clamped at 2^24 px as in the
// forward.
__device__ __forceinline__ void split_coord_fu(int base, float t, int &c0, float &f, float &u) {
    t = fminf(fmaxf(t, -16777216.0f), 16777216.0f);
    const float fl = floorf(t);
    f = t - fl;
    u = (fl + 1.0f) - t;
    c0 = base + (int)fl;
}

// The four corners of one tap as element offsets (pixel index * pstride) and
// weights pre-multiplied by the modulation m. A corner outside [0,H) x [0,W) gets
// weight exactly 0 and its read is redirected to the nearest pixel inside the
// image, so every corner load is in bounds and the loads of a whole window can be
// issued back to back without branches (it then adds 0 * finite = 0).
struct Tap {
    int o00, o01, o10, o11;
    float w00, w01, w10, w11;
};

__device__ __forceinline__ Tap make_tap(int y0, int x0, float fy, float fx, float m, int H, int W,
                                        int pstride) {
    const bool vy0 = (unsigned)y0 < (unsigned)H, vy1 = (unsigned)(y0 + 1) < (unsigned)H;
    const bool vx0 = (unsigned)x0 < (unsigned)W, vx1 = (unsigned)(x0 + 1) < (unsigned)W;
    const int yc0 = min(max(y0, 0), H - 1), yc1 = min(max(y0 + 1, 0), H - 1);
    const int xc0 = min(max(x0, 0), W - 1), xc1 = min(max(x0 + 1, 0), W - 1);
    const float gy0 = vy0 ? (1.0f - fy) * m : 0.0f, gy1 = vy1 ? fy * m : 0.0f;
    const float gx0 = vx0 ? 1.0f - fx : 0.0f, gx1 = vx1 ? fx : 0.0f;
    Tap t;
    t.w00 = gy0 * gx0;
    t.w01 = gy0 * gx1;
    t.w10 = gy1 * gx0;
    t.w11 = gy1 * gx1;
    const int r0 = yc0 * W, r1 = yc1 * W;
    t.o00 = (r0 + xc0) * pstride;
    t.o01 = (r0 + xc1) * pstride;
    t.o10 = (r1 + xc0) * pstride;
    t.o11 = (r1 + xc1) * pstride;
    return t;
}

// acc += sum over the four corners of w * X[corner]; `img` points at pixel (0, 0)
// of the image, already advanced to this lane's channels.
template <class E, int V>
__device__ __forceinline__ void accumulate_tap(const typename E::bits *img, const Tap &t,
                                               float (&acc)[V]) {
    float a[V], b[V], c[V], d[V];
    load_f32<E, V>(img + t.o00, a);
    load_f32<E, V>(img + t.o01, b);
    load_f32<E, V>(img + t.o10, c);
    load_f32<E, V>(img + t.o11, d);
#pragma unroll
    for (int i = 0; i < V; ++i) {
        acc[i] = fmaf(t.w00, a[i], acc[i]);
        acc[i] = fmaf(t.w01, b[i], acc[i]);
        acc[i] = fmaf(t.w10, c[i], acc[i]);
        acc[i] = fmaf(t.w11, d[i], acc[i]);
    }
}

// ------------------------------------------------------------ buffer loads --

// A buffer resource over `bytes` bytes from `base` (gfx9 descriptor word 3); reads
// past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 2/4/8/16-byte loads through a buffer resource: per-lane byte offset `off` plus a
// wave-uniform byte offset `soff`.
template <class R>
__device__ __forceinline__ R buffer_load(__amdgpu_buffer_rsrc_t r, int off, int soff = 0);
template <>
__device__ __forceinline__ uint4 buffer_load<uint4>(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <>
__device__ __forceinline__ uint2 buffer_load<uint2>(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
    return make_uint2(v.x, v.y);
}
template <>
__device__ __forceinline__ uint32_t buffer_load<uint32_t>(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
template <>
__device__ __forceinline__ uint16_t buffer_load<uint16_t>(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}

// ------------------------------------------------------- global -> LDS copy --

// One direct global->LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l
// of the wave writes LDS bytes [lds_wave_base + 16*l, +16). lds_wave_base must be the
// same for the whole wave. The copy is issued from inline assembly so that the
// compiler's wait insertion does not drain copies still in flight before unrelated
// LDS reads; the caller orders it with s_waitcnt vmcnt and a barrier. It writes no
// register, so nothing of the copy is left in flight in a register.
__device__ __forceinline__ void lds_copy16(unsigned lds_wave_base, const void *src) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(src)
        : "memory", "m0");
}

// The same copy through a buffer resource (buffer_load_dwordx4 ... lds): lane l reads
// bytes [voff + soff, +16) of the resource, which reads as zeros where that range
// passes the resource's end (a chunk outside the image costs no memory traffic). The
// resource is given as its four descriptor words (gfx9 layout, as make_rsrc builds).
typedef int rsrc_words_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_words_t rsrc_words(const void *base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)(size_t)base;
    rsrc_words_t r;
    r.x = (int)(unsigned)a;
    r.y = (int)((unsigned)(a >> 32) & 0xffffu);
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}
__device__ __forceinline__ void lds_copy16_buf(unsigned lds_wave_base, rsrc_words_t rsrc, int voff, int soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_wave_base)), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory", "m0");
}

// LDS byte address of a pointer into __shared__ memory.
template <class T>
__device__ __forceinline__ unsigned lds_addr(const T *p) {
    return (unsigned)(size_t)(const __attribute__((address_space(3))) T *)p;
}

// --------------------------------------------------------------- launching --

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD b % 8).
// Remap so that each XCD works on one contiguous range of logical blocks: tiles
// that share input rows then share that XCD's L2 instead of being spread over all
// eight. Bijective for any block count.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
    constexpr int NX = 8;
    const int q = nb / NX, r = nb % NX;
    const int x = b % NX, j = b / NX;
    return x * q + (x < r ? x : r) + j;
}

// Sum over the `width` lanes of an aligned segment (width a power of two <= 64).
__device__ __forceinline__ float seg_sum_pow2(float v, int width) {
    for (int o = 1; o < width; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float seg_max_pow2(float v, int width) {
    for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace dcn
