// Measurement probe: the chip's sustained dense bf16 MFMA rate, with no memory
// traffic, for judging the DCNv2 contraction against a measured ceiling beside the
// published one. Every wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 (32*32*16*2 flops each) on register operands and writes
// one float per lane at the end so that the work is kept.
#include "dcn_common.hpp"
#include "internal.hpp"

namespace dcn {
namespace {

typedef float p_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 p_bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(float *__restrict__ sink, int iters) {
    const int lane = threadIdx.x & 63;
    p_bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    p_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float *sink, int blocks, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
    return hipGetLastError();
}

}  // namespace dcn
