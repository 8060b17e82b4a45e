// kernels_loop.hip -- non-GEMM glue of the looped block: the parameter-free
// LayerNorm that feeds each projection pair from the FP32 residual stream
// ("Model" page: buf.main is the FP32 residual, the norm scratch is FP16).
//
// One 256-thread workgroup per row.  Two passes over the row held in
// registers (mean, then population variance of the centred values), each
// reduced by a fixed xor-butterfly inside waves and then in wave order, so the
// result is deterministic.
#include "device.h"
#include "internal.h"

namespace qg {
namespace {

constexpr int kLnThreads = 256;
constexpr int kLnMaxPerThread = 32;  // D <= 8192

__device__ __forceinline__ float block_sum(float v, float* sh) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[wave] = v;
    __syncthreads();
    float t = sh[0];
#pragma unroll
    for (int w = 1; w < kLnThreads / 64; ++w) t += sh[w];
    return t;
}

__global__ __launch_bounds__(kLnThreads) void k_layernorm(const float* __restrict__ h, int D,
                                                          uint16_t* __restrict__ out) {
    __shared__ float sh[kLnThreads / 64];
    const float* row = h + (int64_t)blockIdx.x * D;
    uint16_t* orow = out + (int64_t)blockIdx.x * D;
    float v[kLnMaxPerThread];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kLnMaxPerThread; ++i) {
        const int k = threadIdx.x + i * kLnThreads;
        v[i] = k < D ? row[k] : 0.0f;
        s += v[i];
    }
    const float mean = block_sum(s, sh) / (float)D;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < kLnMaxPerThread; ++i) {
        const int k = threadIdx.x + i * kLnThreads;
        const float d = k < D ? v[i] - mean : 0.0f;
        v[i] = d;
        q += d * d;
    }
    const float var = block_sum(q, sh) / (float)D;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
#pragma unroll
    for (int i = 0; i < kLnMaxPerThread; ++i) {
        const int k = threadIdx.x + i * kLnThreads;
        if (k < D) orow[k] = f32_to_f16_bits(v[i] * rstd);
    }
}

}  // namespace

hipError_t launch_layernorm(const float* h, int M, int D, qg_half* norm, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    k_layernorm<<<M, kLnThreads, 0, s>>>(h, D, norm);
    return hipGetLastError();
}

}  // namespace qg
