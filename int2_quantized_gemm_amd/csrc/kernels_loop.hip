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

// LayerNorm of one row of D = 256 VPT values, thread t holding values
// t VPT .. t VPT + VPT - 1 in v (FP32): the mean, then the population variance
// of the centred values, each summed in order over the thread's run, by DPP
// inside each wave and then in wave order -- the arithmetic and order of the
// LayerNorm the M == 1 GEMV fuses.  Writes fp16((v - mean) rstd) to orow_t,
// the thread's run of the output row (16-byte stores; 8 bytes when VPT = 4).
// Every thread of the workgroup must call it (two barriers).
template <int VPT>
__device__ __forceinline__ void ln_row_vec(float (&v)[VPT], float (*part)[kLnThreads / 64],
                                           uint16_t* orow_t) {
    static_assert(VPT % 4 == 0 && VPT <= kLnMaxPerThread, "D = 256 VPT, a multiple of 1024");
    constexpr int D = 256 * VPT;
    const int t = threadIdx.x, w = t >> 6;
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
    auto pair = [&](int i) {
        return (uint32_t)f32_to_f16_bits(v[i] * rstd) |
               ((uint32_t)f32_to_f16_bits(v[i + 1] * rstd) << 16);
    };
    if constexpr (VPT % 8 == 0) {
#pragma unroll
        for (int i = 0; i < VPT / 8; ++i)
            ((u32x4*)orow_t)[i] = u32x4{pair(8 * i), pair(8 * i + 2), pair(8 * i + 4), pair(8 * i + 6)};
    } else {  // VPT == 4
        *(u32x2*)orow_t = u32x2{pair(0), pair(2)};
    }
}

// D a multiple of 1024: one workgroup per row, thread t normalises the
// contiguous run of VPT = D/256 values starting at t VPT (float4 loads).
template <int VPT>
__global__ __launch_bounds__(kLnThreads) void k_layernorm_vec(const float* __restrict__ h,
                                                              uint16_t* __restrict__ out) {
    constexpr int D = 256 * VPT;
    __shared__ float part[2][kLnThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * D + threadIdx.x * VPT;
    const float4* hp = (const float4*)(h + base);
    float v[VPT];
#pragma unroll
    for (int i = 0; i < VPT / 4; ++i) {
        const float4 q = hp[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
    ln_row_vec<VPT>(v, part, out + base);
}

// The end of a residual projection and the LayerNorm that follows it, one
// workgroup per row of D = 256 VPT: the projection's FP32 K-part partials
// part[0..S)[M][D] are summed in part order ((p0 + p1) + p2 ...), rounded
// y = fp16(sum) is stored to Y, h += y, and when norm is set the row's
// LayerNorm goes to norm.  The arithmetic and order are those of
// k_splitk_reduce with the residual epilogue followed by k_layernorm_vec, so
// the results are bit-identical to those two launches.  Each thread keeps at
// most 64 partial values in flight (VPT values of up to 64 / VPT parts).
template <int VPT>
__global__ __launch_bounds__(kLnThreads) void k_reduce_residual_ln(
    const float* __restrict__ part, int S, int M, uint16_t* __restrict__ Y, float* __restrict__ h,
    uint16_t* __restrict__ norm) {
    constexpr int D = 256 * VPT;
    constexpr int V4 = VPT / 4;
    constexpr int ZB = VPT <= 8 ? 8 : 64 / VPT;  // parts loaded together
    __shared__ float lnpart[2][kLnThreads / 64];
    const int64_t base = (int64_t)blockIdx.x * D + threadIdx.x * VPT;
    const int64_t plane = (int64_t)M * D;
    f32x4 acc[V4], hv[V4];
#pragma unroll
    for (int i = 0; i < V4; ++i) {
        acc[i] = ((const f32x4*)(part + base))[i];
        hv[i] = ((const f32x4*)(h + base))[i];
    }
    for (int z0 = 1; z0 < S; z0 += ZB) {
        f32x4 pv[ZB][V4];
#pragma unroll
        for (int j = 0; j < ZB; ++j)
            if (z0 + j < S) {
#pragma unroll
                for (int i = 0; i < V4; ++i) pv[j][i] = ((const f32x4*)(part + (z0 + j) * plane + base))[i];
            }
#pragma unroll
        for (int j = 0; j < ZB; ++j)
            if (z0 + j < S) {
#pragma unroll
                for (int i = 0; i < V4; ++i) acc[i] += pv[j][i];
            }
    }
    float v[VPT];
    uint32_t yw[VPT / 2];
#pragma unroll
    for (int i = 0; i < V4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            const uint16_t y0 = f32_to_f16_bits(acc[i][e]), y1 = f32_to_f16_bits(acc[i][e + 1]);
            yw[2 * i + e / 2] = (uint32_t)y0 | ((uint32_t)y1 << 16);
            v[4 * i + e] = hv[i][e] + (float)as_f16(y0);
            v[4 * i + e + 1] = hv[i][e + 1] + (float)as_f16(y1);
        }
        ((float4*)(h + base))[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    }
    if constexpr (VPT % 8 == 0) {
#pragma unroll
        for (int i = 0; i < VPT / 8; ++i)
            ((u32x4*)(Y + base))[i] = u32x4{yw[4 * i], yw[4 * i + 1], yw[4 * i + 2], yw[4 * i + 3]};
    } else {  // VPT == 4
        *(u32x2*)(Y + base) = u32x2{yw[0], yw[1]};
    }
    if (norm == nullptr) return;  // (uniform: no barrier is skipped by part of the group)
    ln_row_vec<VPT>(v, lnpart, norm + base);
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

bool reduce_ln_supported(int D) { return D == 1024 || D == 2048 || D == 4096 || D == 8192; }

hipError_t launch_reduce_residual_ln(const float* part, int S, int M, int D, qg_half* Y, float* h,
                                     qg_half* norm, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    switch (D) {
        case 1024: k_reduce_residual_ln<4><<<M, kLnThreads, 0, s>>>(part, S, M, Y, h, norm); break;
        case 2048: k_reduce_residual_ln<8><<<M, kLnThreads, 0, s>>>(part, S, M, Y, h, norm); break;
        case 4096: k_reduce_residual_ln<16><<<M, kLnThreads, 0, s>>>(part, S, M, Y, h, norm); break;
        case 8192: k_reduce_residual_ln<32><<<M, kLnThreads, 0, s>>>(part, S, M, Y, h, norm); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qg
