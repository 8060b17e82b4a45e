// kernels_loop.hip -- non-GEMM glue of the looped block: the parameter-free
// LayerNorm that feeds each projection pair from the FP32 residual stream
// ("Model" page: buf.main is the FP32 residual, the norm scratch is FP16).
//
// One 256-thread workgroup per row.  Two passes over the row held in
// registers (mean, then population variance of the centred values), each
// reduced in a fixed order inside waves and then in wave order, so the result
// is deterministic.  Rows of a multiple of 1024 values take the vectorised
// variant (contiguous runs per thread, 16-byte accesses); others the
// element-strided one.
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

// D a multiple of 1024: thread t normalises the contiguous run of VPT = D/256
// values starting at t * VPT (float4 loads, 16-byte FP16 stores; 8 bytes
// when VPT = 4), reducing by DPP inside each wave and then in wave order -- the
// same arithmetic, in the same order, as the LayerNorm the M == 1 GEMV fuses.
template <int VPT>
__global__ __launch_bounds__(kLnThreads) void k_layernorm_vec(const float* __restrict__ h,
                                                              uint16_t* __restrict__ out) {
    static_assert(VPT % 4 == 0 && VPT <= kLnMaxPerThread, "D = 256 VPT, a multiple of 1024");
    constexpr int D = 256 * VPT;
    __shared__ float part[2][kLnThreads / 64];
    const int t = threadIdx.x, w = t >> 6;
    const float4* hp = (const float4*)(h + (int64_t)blockIdx.x * D + t * VPT);
    float v[VPT];
#pragma unroll
    for (int i = 0; i < VPT / 4; ++i) {
        const float4 q = hp[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) sum += v[i];
    sum = segment_sum<64>(sum);
    if ((t & 63) == 0) part[0][w] = sum;
    __syncthreads();
    const float mean = ((part[0][0] + part[0][1]) + (part[0][2] + part[0][3])) / (float)D;
    float sq = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        v[i] -= mean;
        sq += v[i] * v[i];
    }
    sq = segment_sum<64>(sq);
    if ((t & 63) == 0) part[1][w] = sq;
    __syncthreads();
    const float var = ((part[1][0] + part[1][1]) + (part[1][2] + part[1][3])) / (float)D;
    const float rstd = 1.0f / sqrtf(var + 1e-5f);
    uint16_t* orow = out + (int64_t)blockIdx.x * D + t * VPT;
    auto pair = [&](int i) {
        return (uint32_t)f32_to_f16_bits(v[i] * rstd) |
               ((uint32_t)f32_to_f16_bits(v[i + 1] * rstd) << 16);
    };
    if constexpr (VPT % 8 == 0) {
#pragma unroll
        for (int i = 0; i < VPT / 8; ++i)
            ((u32x4*)orow)[i] = u32x4{pair(8 * i), pair(8 * i + 2), pair(8 * i + 4), pair(8 * i + 6)};
    } else {  // VPT == 4
        *(u32x2*)orow = u32x2{pair(0), pair(2)};
    }
}

}  // namespace

hipError_t launch_layernorm(const float* h, int M, int D, qg_half* norm, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    switch (D) {
        case 1024: k_layernorm_vec<4><<<M, kLnThreads, 0, s>>>(h, norm); break;
        case 2048: k_layernorm_vec<8><<<M, kLnThreads, 0, s>>>(h, norm); break;
        case 4096: k_layernorm_vec<16><<<M, kLnThreads, 0, s>>>(h, norm); break;
        case 8192: k_layernorm_vec<32><<<M, kLnThreads, 0, s>>>(h, norm); break;
        default: k_layernorm<<<M, kLnThreads, 0, s>>>(h, D, norm); break;
    }
    return hipGetLastError();
}

}  // namespace qg
