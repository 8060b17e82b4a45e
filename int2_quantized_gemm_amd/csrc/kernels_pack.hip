// kernels_pack.hip -- quantise FP32 weights into layout v1 (qg_pack) and the
// unpack / dequant test exports.
//
// Quantiser ("β-Informed Deployment Features" page, CTX-TIER "Details of the
// shipped kernel": per-group asymmetric quantisation, scale = range / 3 for
// INT2, i.e. range / (2^b - 1)): one thread per (output channel n, group g),
// groups of gl = 128 values along K, or gl = K for per-row groups (Phase 2b
// of the same section meets weights quantised per row).  Threads of a wave
// take consecutive n, so each of the gl reads of a group (W[k][n], row-major
// [K][ldw]) is a coalesced 256-byte wave access.  All
// arithmetic is FP64 with correctly rounded division and round-half-even, so
// the result is bit-identical to the definition.
#include "device.h"
#include "internal.h"

namespace qg {
namespace {

// PER_ROW: gl = K (runtime); otherwise gl = 128, a compile-time loop bound.
// CHECK: the validation pass -- the same range and scale, then the call's tag
// stored to *status when W holds a non-finite value or the scale overflows
// FP16, and nothing else written; the packing pass (CHECK false) runs only
// after a clean validation pass and writes codes, scales and zeros.
template <int BITS, bool PER_ROW, bool CHECK>
__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ W, int64_t ldw, int K,
                                              int N, uint32_t* __restrict__ codes,
                                              uint16_t* __restrict__ scales,
                                              uint16_t* __restrict__ zeros, int* status,
                                              int tag) {
    using F = Fmt<BITS>;
    const int gl = PER_ROW ? K : kGroup;
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    const int g = blockIdx.y;
    if (n >= N) return;
    const int groups = K / gl;
    const float* col = W + (int64_t)g * gl * ldw + n;

    double lo = 0.0, hi = 0.0;
    bool bad = false;
    for (int k = 0; k < gl; ++k) {
        const double w = (double)col[(int64_t)k * ldw];
        bad |= !isfinite(w);
        lo = w < lo ? w : lo;
        hi = w > hi ? w : hi;
    }
    const uint16_t s_bits = f64_to_f16_bits((hi - lo) / (double)F::kQMax);
    double s = f16_bits_to_f64(s_bits);
    bad |= !isfinite(s);
    if constexpr (CHECK) {
        if (bad) *status = tag;  // every failing thread stores the same call tag
        return;
    }
    uint16_t s_store = s_bits;
    if (s == 0.0) {
        s = 1.0;
        s_store = 0x3c00;  // 1.0
    }
    double z = rint(-lo / s);
    z = z < 0.0 ? 0.0 : (z > (double)F::kQMax ? (double)F::kQMax : z);
    scales[(int64_t)n * groups + g] = s_store;
    zeros[(int64_t)n * groups + g] = f64_to_f16_bits(z);

    const int words = gl / F::kCodesPerWord;
    uint32_t* out = codes + (int64_t)n * (K / F::kCodesPerWord) + (int64_t)g * words;
    for (int wi = 0; wi < words; ++wi) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < F::kCodesPerWord; ++j) {
            const int k = wi * F::kCodesPerWord + j;
            double q = rint((double)col[(int64_t)k * ldw] / s) + z;
            q = q >= 0.0 ? q : 0.0;
            q = q > (double)F::kQMax ? (double)F::kQMax : q;
            word |= (uint32_t)q << (16 * (j & 1) + BITS * (j >> 1));
        }
        out[wi] = word;
    }
}

// One thread per packed word (i = n * wpr + word of row n, wpr = K*b/32,
// rows ldc words apart in memory): writes the word's codes q[n][k] as bytes.
template <int BITS>
__global__ __launch_bounds__(256) void k_unpack(const uint32_t* __restrict__ codes, int64_t wpr,
                                                int64_t ldc, int64_t words,
                                                uint8_t* __restrict__ q) {
    using F = Fmt<BITS>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const uint32_t w = codes[(i / wpr) * ldc + i % wpr];
    uint8_t* o = q + i * F::kCodesPerWord;
#pragma unroll
    for (int p = 0; p < F::kPairsPerWord; ++p) {
        uint32_t a, b;
        code_pair<BITS>(w, p, a, b);
        o[2 * p] = (uint8_t)a;
        o[2 * p + 1] = (uint8_t)b;
    }
}

// One thread per packed word: writes w^[n][k] for the word's codes, FP32
// (exact) or FP16 (one rounding), with the GEMM kernels' dequant helpers.
template <int BITS, bool F16OUT>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ codes, int64_t ldc,
                                                 const uint16_t* __restrict__ scales,
                                                 const uint16_t* __restrict__ zeros, SzIdx sz,
                                                 int K, int64_t words, void* __restrict__ out) {
    using F = Fmt<BITS>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words) return;
    const int64_t wpr = K / F::kCodesPerWord;
    const int64_t n = i / wpr;
    const int64_t g = (i % wpr) / F::kWordsPerGroup;
    const int64_t sg = sz.at(n, g);
    const GroupConst c = group_const(scales[sg], zeros[sg]);
    const uint32_t w = codes[n * ldc + i % wpr];
    const int64_t k0 = i * F::kCodesPerWord;  // == n*K + (i % wpr) * codes/word
#pragma unroll
    for (int p = 0; p < F::kPairsPerWord; ++p) {
        if (F16OUT) {
            const f16x2 v = dequant_pair_f16<BITS>(w, p, c);
            ((uint32_t*)out)[(k0 >> 1) + p] = as_u32(v);
        } else {
            float a, b;
            dequant_pair_f32<BITS>(w, p, c, a, b);
            ((float*)out)[k0 + 2 * p] = a;
            ((float*)out)[k0 + 2 * p + 1] = b;
        }
    }
}

}  // namespace

template <bool CHECK>
hipError_t launch_pack_pass(const float* W, int64_t ldw, int K, int N, int bits, int group,
                            uint32_t* codes, qg_half* scales, qg_half* zeros, int* status,
                            int tag, hipStream_t s) {
    dim3 grid((N + 255) / 256, K / group);
    const bool row = group != kGroup;
    if (bits == 4 && row)
        k_pack<4, true, CHECK><<<grid, 256, 0, s>>>(W, ldw, K, N, codes, scales, zeros, status, tag);
    else if (bits == 4)
        k_pack<4, false, CHECK><<<grid, 256, 0, s>>>(W, ldw, K, N, codes, scales, zeros, status, tag);
    else if (row)
        k_pack<2, true, CHECK><<<grid, 256, 0, s>>>(W, ldw, K, N, codes, scales, zeros, status, tag);
    else
        k_pack<2, false, CHECK><<<grid, 256, 0, s>>>(W, ldw, K, N, codes, scales, zeros, status, tag);
    return hipGetLastError();
}

hipError_t launch_pack_check(const float* W, int64_t ldw, int K, int N, int bits, int group,
                             int* status, int tag, hipStream_t s) {
    return launch_pack_pass<true>(W, ldw, K, N, bits, group, nullptr, nullptr, nullptr, status,
                                  tag, s);
}

hipError_t launch_pack(const float* W, int64_t ldw, int K, int N, int bits, int group,
                       uint32_t* codes, qg_half* scales, qg_half* zeros, hipStream_t s) {
    return launch_pack_pass<false>(W, ldw, K, N, bits, group, codes, scales, zeros, nullptr, 0, s);
}

hipError_t launch_unpack(const qg_weight& w, uint8_t* q, hipStream_t s) {
    const int64_t words = (int64_t)w.N * (w.K * w.bits / 32);
    const int64_t blocks = (words + 255) / 256;
    const int64_t wpr = w.K * w.bits / 32;
    if (w.bits == 4)
        k_unpack<4><<<(unsigned)blocks, 256, 0, s>>>(w.codes, wpr, code_ld(w), words, q);
    else
        k_unpack<2><<<(unsigned)blocks, 256, 0, s>>>(w.codes, wpr, code_ld(w), words, q);
    return hipGetLastError();
}

hipError_t launch_dequant(const qg_weight& w, bool fp16, void* out, hipStream_t s) {
    const int64_t words = (int64_t)w.N * (w.K * w.bits / 32);
    const SzIdx sz = sz_idx(w);
    const unsigned blocks = (unsigned)((words + 255) / 256);
    if (w.bits == 4) {
        if (fp16)
            k_dequant<4, true><<<blocks, 256, 0, s>>>(w.codes, code_ld(w), w.scales, w.zeros, sz, w.K, words, out);
        else
            k_dequant<4, false><<<blocks, 256, 0, s>>>(w.codes, code_ld(w), w.scales, w.zeros, sz, w.K, words, out);
    } else {
        if (fp16)
            k_dequant<2, true><<<blocks, 256, 0, s>>>(w.codes, code_ld(w), w.scales, w.zeros, sz, w.K, words, out);
        else
            k_dequant<2, false><<<blocks, 256, 0, s>>>(w.codes, code_ld(w), w.scales, w.zeros, sz, w.K, words, out);
    }
    return hipGetLastError();
}

}  // namespace qg
