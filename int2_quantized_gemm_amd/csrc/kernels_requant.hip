// kernels_requant.hip -- INT4 -> INT2 re-quantisation on the device
// (qg_requant_4to2).
//
// "β-Informed Deployment Features" page, CTX-TIER, details of the shipped
// kernel: each quantisation group is dequantised, given a new asymmetric INT2
// scale from its range and packed four codes per byte, in place or into a
// separate buffer.  Here each group's exact INT4 dequant w^ = (q - z) s (FP64)
// goes through the same quantiser as qg_pack with bits = 2: range with 0
// included, s2 = fp16((hi - lo) / 3) (1 when it rounds to 0), integer zero
// z2 = rne(-lo / s2), codes rne(w^ / s2) + z2, all clamped to [0, 3], FP64
// with correctly rounded division -- bit-identical to the definition.
//
// Four lanes per group: lane r takes INT4 words 4r .. 4r+3 of the group (32
// codes).  The group's range needs only its smallest and largest INT4 code
// (w^ is monotone in q): lo = min(0, (qmin - z) s, (qmax - z) s), likewise hi.
// The INT2 code of a weight depends only on its INT4 code (0..15), so lane r
// computes the INT2 codes of INT4 values 4r .. 4r+3 with the definition's
// FP64 steps, the four lanes OR them into one 32-bit table of sixteen 2-bit
// codes, and every weight's code is a shift and mask of that table.  Lane r
// then writes INT2 words 2r, 2r+1 of the group.  A wave covers 16 groups; its
// reads and writes are contiguous.
// In place the INT2 codes are written compactly (K/16 words per row) over the
// front of the INT4 buffer: INT2 group (n, g) lands inside INT4 group
// (n/2, ...) of the same buffer, so it may be written only once that INT4
// data has been read.  Row 0 runs group ranges [0, 1), [1, 2), [2, 4), ...
// (group g writes into INT4 group g/2 of row 0, consumed by an earlier launch;
// group 0 writes into itself, which is safe within its one wave because every
// lane's load feeds the shuffled OR before any lane stores), then rows
// [1, 2), [2, 4), [4, 8), ... (INT2 row n lies in INT4 row n/2, consumed by
// an earlier launch; none of the rows a launch reads has been written).  The
// pages' in-place mode keeps the INT4 row stride instead; the weight
// descriptor here has no row stride, so the compact form is the one the INT2
// GEMM can read.  Scales and zeros are overwritten element for element by
// the lane that read them.
//
// Per-row groups (group size K; the same section's Phase 2b meets them) take
// k_requant_4to2_row: one workgroup per row holds the row's INT4 words in
// registers, reduces the row's smallest and largest code through LDS, builds
// the same 16-entry table from the row's scale and zero (threads 0..15, one
// entry each), and after that barrier writes the INT2 row: every read of the
// row precedes every write, so in place row n may overwrite INT4 row n / 2,
// and rows run in the same launch order [0, 1), [1, 2), [2, 4), ...
#include "device.h"
#include "internal.h"

namespace qg {
namespace {

// CHECK: the validation pass -- each group's INT4 scale and zero and new INT2
// scale, then the call's tag stored to *status when one is non-finite (or
// the INT2 scale overflows FP16), and nothing else written; the writing pass
// (CHECK false) runs only after a clean validation pass.
// One group's re-quantisation on its four lanes (r = lane quarter, the four
// lanes of a group consecutive in the wave and all active): from the lane's
// four INT4 words w4 and the group's INT4 scale and zero, the lane's two INT2
// words, the group's INT2 scale and zero (bits), and whether the group is bad
// (a non-finite INT4 scale or zero, or an INT2 scale overflowing FP16).
struct GroupOut {
    uint32_t out[2];
    uint16_t s_store, z_store;
    bool bad;
};

__device__ __forceinline__ GroupOut requant_group(const u32x4& w4, double s4, double z4, bool live,
                                                  int r) {
    GroupOut o;
    // smallest and largest INT4 code of the group
    int qmin = 15, qmax = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int q = (int)((w4[i] >> (16 * (j & 1) + 4 * (j >> 1))) & 0xFu);
            qmin = q < qmin ? q : qmin;
            qmax = q > qmax ? q : qmax;
        }
#pragma unroll
    for (int m = 2; m >= 1; m >>= 1) {
        const int a = __shfl_xor(qmin, m, 4), b = __shfl_xor(qmax, m, 4);
        qmin = a < qmin ? a : qmin;
        qmax = b > qmax ? b : qmax;
    }
    const double wa = ((double)qmin - z4) * s4, wb = ((double)qmax - z4) * s4;
    const double lo = fmin(0.0, fmin(wa, wb)), hi = fmax(0.0, fmax(wa, wb));
    o.s_store = f64_to_f16_bits((hi - lo) / 3.0);
    double s2 = f16_bits_to_f64(o.s_store);
    o.bad = live && (!isfinite(s4) || !isfinite(z4) || !isfinite(s2));
    if (s2 == 0.0) {
        s2 = 1.0;
        o.s_store = 0x3c00;  // 1.0
    }
    double z2 = rint(-lo / s2);
    z2 = z2 < 0.0 ? 0.0 : (z2 > 3.0 ? 3.0 : z2);
    o.z_store = f64_to_f16_bits(z2);
    // INT2 codes of INT4 values 4r .. 4r+3, then the whole 16-entry table
    uint32_t table = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        double q = rint((((double)(4 * r + v) - z4) * s4) / s2) + z2;
        q = q >= 0.0 ? q : 0.0;
        q = q > 3.0 ? 3.0 : q;
        table |= (uint32_t)q << (2 * (4 * r + v));
    }
    table |= (uint32_t)__shfl_xor((int)table, 1, 4);
    table |= (uint32_t)__shfl_xor((int)table, 2, 4);
    // INT4 words 4r + 2i, 4r + 2i + 1 hold the 16 codes of INT2 word 2r + i
    o.out[0] = o.out[1] = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t q4 = (w4[i] >> (16 * (j & 1) + 4 * (j >> 1))) & 0xFu;
            const uint32_t q2 = (table >> (2 * q4)) & 3u;
            const int jj = 8 * (i & 1) + j;  // code index inside the INT2 word
            o.out[i >> 1] |= q2 << (16 * (jj & 1) + 2 * (jj >> 1));
        }
    return o;
}

template <bool CHECK>
__global__ __launch_bounds__(256) void k_requant_4to2(
    const uint32_t* codes4, int64_t ldc4, const uint16_t* scales4, const uint16_t* zeros4, int K,
    int row0, int g0, int gcount, uint32_t* codes2, int64_t ldc2, uint16_t* scales2,
    uint16_t* zeros2, int* status, int tag) {
    const int groups = K / kGroup;
    // grid: x over the groups of a row (4 lanes each), y over the rows
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int r = t & 3;
    const bool live = (t >> 2) < gcount;  // all 4 lanes of a group alike
    const int64_t n = row0 + blockIdx.y;
    const int g = g0 + (live ? (t >> 2) : 0);
    const int64_t sg = n * groups + g;

    u32x4 w4 = {0u, 0u, 0u, 0u};
    double s4 = 0.0, z4 = 0.0;
    if (live) {
        w4 = *(const u32x4*)(codes4 + n * ldc4 + g * 16 + 4 * r);
        s4 = f16_bits_to_f64(scales4[sg]);
        z4 = f16_bits_to_f64(zeros4[sg]);
    }
    const GroupOut o = requant_group(w4, s4, z4, live, r);
    if constexpr (CHECK) {
        if (o.bad) *status = tag;  // every failing thread stores the same call tag
        return;
    }
    if (!live) return;
    *(u32x2*)(codes2 + n * ldc2 + g * 8 + 2 * r) = u32x2{o.out[0], o.out[1]};
    if (r == 0) {
        scales2[sg] = o.s_store;
        zeros2[sg] = o.z_store;
    }
}

// In place at the INT4 row stride (the pages' in-place mode, groups of 128):
// one workgroup of T threads per row, lane t + T c (c < CH) on quarter t % 4 of
// group (t + T c) / 4.  Every lane reads its part of the row, computes its
// INT2 words and, after one barrier, writes them: INT2 group g lands in the
// row's first half, inside INT4 group g / 2 of the same row, which by then
// the whole workgroup has read.  Scales and zeros (in place or not) are
// written element for element by the lane that read them.
template <int CH>
__global__ __launch_bounds__(256) void k_requant_4to2_inrow(uint32_t* codes, int64_t ldc,
                                                            const uint16_t* scales4,
                                                            const uint16_t* zeros4,
                                                            uint16_t* scales2, uint16_t* zeros2,
                                                            int K) {
    const int groups = K / kGroup;
    const int64_t n = blockIdx.x;
    const int r = threadIdx.x & 3;
    GroupOut o[CH];
    int g[CH];
    bool live[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int gg = (threadIdx.x + blockDim.x * c) >> 2;
        live[c] = gg < groups;  // all 4 lanes of a group alike
        g[c] = live[c] ? gg : 0;
        u32x4 w4 = {0u, 0u, 0u, 0u};
        double s4 = 0.0, z4 = 0.0;
        if (live[c]) {
            w4 = *(const u32x4*)(codes + n * ldc + g[c] * 16 + 4 * r);
            s4 = f16_bits_to_f64(scales4[n * groups + g[c]]);
            z4 = f16_bits_to_f64(zeros4[n * groups + g[c]]);
        }
        o[c] = requant_group(w4, s4, z4, live[c], r);
    }
    __syncthreads();  // every read of the row precedes every write
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        if (!live[c]) continue;
        *(u32x2*)(codes + n * ldc + g[c] * 8 + 2 * r) = u32x2{o[c].out[0], o[c].out[1]};
        if (r == 0) {
            scales2[n * groups + g[c]] = o[c].s_store;
            zeros2[n * groups + g[c]] = o[c].z_store;
        }
    }
}

// Per-row groups: workgroup x covers row row0 + x; thread t takes
// INT2 words t, t + 256, ... of the row (INT4 words 2j, 2j + 1 for INT2 word j).
constexpr int kRowPairs = kRequantRowMaxK / 16 / 256;  // INT2 words per thread, at most

template <bool CHECK>
__global__ __launch_bounds__(256) void k_requant_4to2_row(
    const uint32_t* codes4, int64_t ldc4, const uint16_t* scales4, const uint16_t* zeros4, int K,
    int row0, uint32_t* codes2, int64_t ldc2, uint16_t* scales2, uint16_t* zeros2, int* status,
    int tag) {
    __shared__ int red[2][4];
    __shared__ uint32_t tab[16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t n = row0 + blockIdx.x;
    const int words2 = K / 16;
    const double s4 = f16_bits_to_f64(scales4[n]), z4 = f16_bits_to_f64(zeros4[n]);
    u32x2 w[kRowPairs];
    int qmin = 15, qmax = 0;
#pragma unroll
    for (int i = 0; i < kRowPairs; ++i) {
        const int j = t + 256 * i;
        w[i] = j < words2 ? *(const u32x2*)(codes4 + n * ldc4 + 2 * j) : u32x2{0u, 0u};
        if (j < words2) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int q = (int)((w[i][h] >> (16 * (c & 1) + 4 * (c >> 1))) & 0xFu);
                    qmin = q < qmin ? q : qmin;
                    qmax = q > qmax ? q : qmax;
                }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const int a = __shfl_xor(qmin, m), b = __shfl_xor(qmax, m);
        qmin = a < qmin ? a : qmin;
        qmax = b > qmax ? b : qmax;
    }
    if (lane == 0) {
        red[0][wave] = qmin;
        red[1][wave] = qmax;
    }
    __syncthreads();
    qmin = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
    qmax = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    const double wa = ((double)qmin - z4) * s4, wb = ((double)qmax - z4) * s4;
    const double lo = fmin(0.0, fmin(wa, wb)), hi = fmax(0.0, fmax(wa, wb));
    uint16_t s_store = f64_to_f16_bits((hi - lo) / 3.0);
    double s2 = f16_bits_to_f64(s_store);
    const bool bad = !isfinite(s4) || !isfinite(z4) || !isfinite(s2);
    if constexpr (CHECK) {
        if (t == 0 && bad) *status = tag;
        return;
    }
    if (s2 == 0.0) {
        s2 = 1.0;
        s_store = 0x3c00;  // 1.0
    }
    double z2 = rint(-lo / s2);
    z2 = z2 < 0.0 ? 0.0 : (z2 > 3.0 ? 3.0 : z2);
    if (t < 16) {
        double q = rint((((double)t - z4) * s4) / s2) + z2;
        q = q >= 0.0 ? q : 0.0;
        q = q > 3.0 ? 3.0 : q;
        tab[t] = (uint32_t)q;
    }
    __syncthreads();
    uint32_t table = 0;
#pragma unroll
    for (int v = 0; v < 16; ++v) table |= tab[v] << (2 * v);
#pragma unroll
    for (int i = 0; i < kRowPairs; ++i) {
        const int j = t + 256 * i;
        if (j >= words2) continue;
        uint32_t out = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t q4 = (w[i][h] >> (16 * (c & 1) + 4 * (c >> 1))) & 0xFu;
                const int jj = 8 * h + c;  // code index inside the INT2 word
                out |= ((table >> (2 * q4)) & 3u) << (16 * (jj & 1) + 2 * (jj >> 1));
            }
        codes2[n * ldc2 + j] = out;
    }
    if (t == 0) {
        scales2[n] = s_store;
        zeros2[n] = f64_to_f16_bits(z2);
    }
}

}  // namespace

hipError_t launch_requant_4to2_check(const qg_weight& w4, int* status, int tag, hipStream_t s) {
    const int K = w4.K, N = w4.N, groups = K / kGroup;
    const int64_t l4 = code_ld(w4);
    if (per_row(w4)) {
        k_requant_4to2_row<true><<<(unsigned)N, 256, 0, s>>>(w4.codes, l4, w4.scales, w4.zeros, K, 0,
                                                             nullptr, 0, nullptr, nullptr, status,
                                                             tag);
        return hipGetLastError();
    }
    const int lanes = groups * 4;
    const int threads = lanes >= 256 ? 256 : (lanes + 63) / 64 * 64;
    const dim3 grid((unsigned)((lanes + threads - 1) / threads), (unsigned)N);
    k_requant_4to2<true><<<grid, threads, 0, s>>>(w4.codes, l4, w4.scales, w4.zeros, K, 0, 0, groups,
                                                  nullptr, 0, nullptr, nullptr, status, tag);
    return hipGetLastError();
}

hipError_t launch_requant_4to2(const qg_weight& w4, const qg_weight& w2, bool in_place,
                               hipStream_t s) {
    const int K = w4.K, N = w4.N, groups = K / kGroup;
    const int64_t l4 = code_ld(w4), l2 = code_ld(w2);
    uint32_t* c2 = const_cast<uint32_t*>(w2.codes);
    uint16_t* s2 = const_cast<uint16_t*>(w2.scales);
    uint16_t* z2 = const_cast<uint16_t*>(w2.zeros);
    // in place at the INT4 row stride: each INT2 row stays inside its INT4 row
    const bool same_stride = in_place && l2 == l4;
    auto run = [&](int row0, int rows, int g0, int gcount) {
        // workgroups of one to four waves, as many as a row's groups fill
        const int lanes = gcount * 4;
        const int threads = lanes >= 256 ? 256 : (lanes + 63) / 64 * 64;
        const dim3 grid((unsigned)((lanes + threads - 1) / threads), (unsigned)rows);
        k_requant_4to2<false><<<grid, threads, 0, s>>>(w4.codes, l4, w4.scales, w4.zeros, K, row0,
                                                       g0, gcount, c2, l2, s2, z2, nullptr, 0);
        return hipGetLastError();
    };
    if (per_row(w4)) {
        // a workgroup reads its whole row before writing it
        auto rows = [&](int64_t row0, int64_t count) {
            k_requant_4to2_row<false><<<(unsigned)count, 256, 0, s>>>(
                w4.codes, l4, w4.scales, w4.zeros, K, (int)row0, c2, l2, s2, z2, nullptr, 0);
            return hipGetLastError();
        };
        if (!in_place || same_stride) return rows(0, N);
        hipError_t e = rows(0, 1);
        for (int64_t lo = 1; e == hipSuccess && lo < N; lo *= 2)
            e = rows(lo, (2 * lo < N ? 2 * lo : N) - lo);
        return e;
    }
    if (!in_place) return run(0, N, 0, groups);
    if (same_stride) {
        const int lanes = groups * 4;
        if (lanes <= 4 * 256) {  // K <= 32768: one workgroup per row, one launch
            const int threads = lanes >= 256 ? 256 : (lanes + 63) / 64 * 64;
            const int ch = (lanes + threads - 1) / threads;
            uint32_t* c = c2;
            switch (ch) {
                case 1: k_requant_4to2_inrow<1><<<(unsigned)N, threads, 0, s>>>(
                    c, l4, w4.scales, w4.zeros, s2, z2, K);
                    break;
                case 2: k_requant_4to2_inrow<2><<<(unsigned)N, threads, 0, s>>>(
                    c, l4, w4.scales, w4.zeros, s2, z2, K);
                    break;
                case 3: k_requant_4to2_inrow<3><<<(unsigned)N, threads, 0, s>>>(
                    c, l4, w4.scales, w4.zeros, s2, z2, K);
                    break;
                default: k_requant_4to2_inrow<4><<<(unsigned)N, threads, 0, s>>>(
                    c, l4, w4.scales, w4.zeros, s2, z2, K);
                    break;
            }
            return hipGetLastError();
        }
        // longer rows: every row's groups in ranges [0, 1), [1, 2), [2, 4), ...
        // (INT2 group g lands in INT4 group g / 2, read by an earlier launch)
        hipError_t e = run(0, N, 0, 1);
        for (int lo = 1; e == hipSuccess && lo < groups; lo *= 2)
            e = run(0, N, lo, (2 * lo < groups ? 2 * lo : groups) - lo);
        return e;
    }
    // compact INT2 rows over the front of the INT4 buffer: launches ordered by
    // row (INT2 row n lands in INT4 row n / 2) and, in row 0, by group
    hipError_t e = run(0, 1, 0, 1);
    for (int lo = 1; e == hipSuccess && lo < groups; lo *= 2)
        e = run(0, 1, lo, (2 * lo < groups ? 2 * lo : groups) - lo);
    for (int64_t lo = 1; e == hipSuccess && lo < N; lo *= 2)
        e = run((int)lo, (int)((2 * lo < N ? 2 * lo : N) - lo), 0, groups);
    return e;
}

}  // namespace qg
