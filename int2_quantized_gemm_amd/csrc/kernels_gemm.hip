// kernels_gemm.hip -- Y[M][N] = X[M][K] . dequant(W)[K][N] for layout-v1 INT4/INT2
// weights (quant_gemm / int2_gemm, "β-Informed Deployment Features" page,
// CTX-TIER section), FP16 activations, FP32 accumulation, FP16 output.
//
// Three kernel families, chosen by M:
//   * k_gemv (M == 1): bandwidth-bound GEMV.  Lanes split K: each lane loads
//     16 contiguous bytes of packed codes per chunk (a wave reads a contiguous
//     1 KiB run of a row), converts codes with the exponent-bias trick, forms
//     exact (q - z) FP16 pairs and accumulates x*(q - z) with v_dot2_f32_f16;
//     the per-group scale multiplies the lane's partial once.  Lane partials of
//     a row are combined by a fixed xor-butterfly (deterministic).
//   * k_gemm_skinny (2 <= M <= 16): one 16-row MFMA tile of output channels per
//     workgroup, K split over the workgroup's waves and reduced through LDS in
//     wave order.  v_mfma_f32_16x16x32_f16 takes X rows as A (M padded to 16)
//     and dequantised weights as B.
//   * k_gemm_tiled (M > 16): 128x128 output tiles, 2x2 waves of 64x64, the
//     same MFMA; weights dequantised to FP16 (one rounding of (q - z) * s).
//
// MFMA operand mapping used everywhere (16x16x32 f16): lane l supplies row
// (A) or column (B) l % 16 and eight k values selected by l / 16; A and B use
// the same selection, so the product sums over all 32 k of the step.  Within
// a 128-k group, lane quarter c = l / 16 owns k in [32c, 32c + 32) and MFMA j
// (j = 0..3) consumes its k in [32c + 8j, 32c + 8j + 8).  The accumulator
// holds D[4*(l/16) + r][l % 16] in register r.
#include "device.h"
#include "internal.h"

namespace qg {
namespace {

// ------------------------------------------------------------------ GEMV ----

// LPR lanes cover one row per chunk of 4*LPR words; CPR chunks per row;
// 64/LPR rows per wave step; U row steps per wave.
template <int BITS, int LPR, int CPR, int U>
__global__ __launch_bounds__(256) void k_gemv(const uint16_t* __restrict__ X,
                                              const uint32_t* __restrict__ codes,
                                              const uint16_t* __restrict__ scales,
                                              const uint16_t* __restrict__ zeros, int K, int N,
                                              uint16_t* __restrict__ Y, float* __restrict__ h,
                                              int epi) {
    using F = Fmt<BITS>;
    constexpr int RPW = 64 / LPR;
    constexpr int PAIRS = 4 * F::kPairsPerWord;  // FP16 pairs of X per lane and chunk
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int sub = lane % LPR;
    const int rsub = lane / LPR;
    const int wpr = K / F::kCodesPerWord;
    const int groups = K / kGroup;
    const int row0 = wave * U * RPW;
    if (row0 >= N) return;

    // Activations for this lane's k positions, reused for every row.
    f16x2 xr[CPR][PAIRS];
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
        const int k0 = (c * LPR * 4 + sub * 4) * F::kCodesPerWord;
        const u32x4* xp = (const u32x4*)(X + k0);
#pragma unroll
        for (int v = 0; v < PAIRS / 4; ++v) {
            const u32x4 t = xp[v];
            xr[c][4 * v + 0] = as_f16x2(t.x);
            xr[c][4 * v + 1] = as_f16x2(t.y);
            xr[c][4 * v + 2] = as_f16x2(t.z);
            xr[c][4 * v + 3] = as_f16x2(t.w);
        }
    }

    // Issue every load of this wave before any arithmetic.
    u32x4 wv[U][CPR];
    uint16_t sv[U][CPR], zv[U][CPR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = row0 + u * RPW + rsub;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const int wi = c * LPR * 4 + sub * 4;
            if (row < N) {
                wv[u][c] = *(const u32x4*)(codes + (int64_t)row * wpr + wi);
                const int64_t sg = (int64_t)row * groups + wi / F::kWordsPerGroup;
                sv[u][c] = scales[sg];
                zv[u][c] = zeros[sg];
            } else {
                wv[u][c] = u32x4{0, 0, 0, 0};
                sv[u][c] = 0;
                zv[u][c] = 0;
            }
        }
    }

    float part[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const GroupConst gc = group_const(sv[u][c], zv[u][c]);
            float a = 0.0f;
            const uint32_t w4[4] = {wv[u][c].x, wv[u][c].y, wv[u][c].z, wv[u][c].w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int p = 0; p < F::kPairsPerWord; ++p)
                    a = __builtin_amdgcn_fdot2(centered_pair<BITS>(w4[q], p, gc.nbz),
                                               xr[c][q * F::kPairsPerWord + p], a, false);
            acc += a * (float)gc.s2.x;
        }
        part[u] = acc;
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) part[u] += __shfl_xor(part[u], off);
        const int row = row0 + u * RPW + rsub;
        if (sub == 0 && row < N) {
            const uint16_t y = f32_to_f16_bits(part[u]);
            Y[row] = y;
            if (epi == kResidual) h[row] += (float)as_f16(y);
        }
    }
}

// ------------------------------------------------------ MFMA B fragments ----

// Codes of one 128-k group for one lane (k in [32c, 32c + 32) of row n).
template <int BITS>
struct LaneCodes;
template <>
struct LaneCodes<4> {
    u32x4 w;
    __device__ __forceinline__ void load(const uint32_t* row, int g, int c) {
        w = *(const u32x4*)(row + g * 16 + c * 4);
    }
    __device__ __forceinline__ void zero() { w = u32x4{0, 0, 0, 0}; }
    // FP16 B fragment of MFMA step j: codes 8j..8j+7 of the lane = word j.
    __device__ __forceinline__ f16x8 frag(int j, const GroupConst& gc) const {
        const uint32_t x = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
        const f16x2 p0 = dequant_pair_f16<4>(x, 0, gc), p1 = dequant_pair_f16<4>(x, 1, gc);
        const f16x2 p2 = dequant_pair_f16<4>(x, 2, gc), p3 = dequant_pair_f16<4>(x, 3, gc);
        return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
};
template <>
struct LaneCodes<2> {
    u32x2 w;
    __device__ __forceinline__ void load(const uint32_t* row, int g, int c) {
        w = *(const u32x2*)(row + g * 8 + c * 2);
    }
    __device__ __forceinline__ void zero() { w = u32x2{0, 0}; }
    // Step j: codes 8j..8j+7 = pairs 4(j&1)..4(j&1)+3 of word j>>1.
    __device__ __forceinline__ f16x8 frag(int j, const GroupConst& gc) const {
        const uint32_t x = (j >> 1) ? w.y : w.x;
        const int p = (j & 1) * 4;
        const f16x2 p0 = dequant_pair_f16<2>(x, p + 0, gc), p1 = dequant_pair_f16<2>(x, p + 1, gc);
        const f16x2 p2 = dequant_pair_f16<2>(x, p + 2, gc), p3 = dequant_pair_f16<2>(x, p + 3, gc);
        return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
};

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// A fragments of one 128-k group for one lane: X[m][g*128 + 32c + 8j .. +8].
__device__ __forceinline__ void load_a(const uint16_t* xrow, bool valid, int g, int c, f16x8 a[4]) {
    if (valid) {
        const f16x8* p = (const f16x8*)(xrow + g * kGroup + c * 32);
        a[0] = p[0];
        a[1] = p[1];
        a[2] = p[2];
        a[3] = p[3];
    } else {
        a[0] = a[1] = a[2] = a[3] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
}

__device__ __forceinline__ void store_out(uint16_t* Y, int64_t ldy, float* h, int64_t ldh, int epi,
                                          int m, int n, float v) {
    const uint16_t y = f32_to_f16_bits(v);
    Y[(int64_t)m * ldy + n] = y;
    if (epi == kResidual) h[(int64_t)m * ldh + n] += (float)as_f16(y);
}

// ---------------------------------------------------------------- skinny ----

template <int BITS, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void k_gemm_skinny(
    const uint16_t* __restrict__ X, int64_t ldx, int M, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int K, int N,
    uint16_t* __restrict__ Y, int64_t ldy, float* __restrict__ h, int64_t ldh, int epi) {
    using F = Fmt<BITS>;
    __shared__ f32x4 red[KSPLIT][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nl = lane & 15, c = lane >> 4;
    const int n = blockIdx.x * 16 + nl;
    const bool nvalid = n < N;
    const bool mvalid = nl < M;  // A row of this lane
    const int groups = K / kGroup;
    const int g0 = (int)((int64_t)groups * wave / KSPLIT);
    const int g1 = (int)((int64_t)groups * (wave + 1) / KSPLIT);
    const uint32_t* crow = codes + (int64_t)(nvalid ? n : 0) * (K / F::kCodesPerWord);
    const uint16_t* xrow = X + (int64_t)(mvalid ? nl : 0) * ldx;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int g = g0; g < g1; ++g) {
        LaneCodes<BITS> lc;
        uint16_t sb = 0, zb = 0;
        if (nvalid) {
            lc.load(crow, g, c);
            sb = scales[(int64_t)n * groups + g];
            zb = zeros[(int64_t)n * groups + g];
        } else {
            lc.zero();
        }
        f16x8 a[4];
        load_a(xrow, mvalid, g, c, a);
        const GroupConst gc = group_const(sb, zb);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16(a[j], lc.frag(j, gc), acc);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < KSPLIT; ++w) sum += red[w][lane];
    if (!nvalid) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * c + r;
        if (m < M) store_out(Y, ldy, h, ldh, epi, m, n, sum[r]);
    }
}

// ----------------------------------------------------------------- tiled ----

template <int BITS>
__global__ __launch_bounds__(256) void k_gemm_tiled(
    const uint16_t* __restrict__ X, int64_t ldx, int M, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int K, int N,
    uint16_t* __restrict__ Y, int64_t ldy, float* __restrict__ h, int64_t ldh, int epi) {
    using F = Fmt<BITS>;
    constexpr int WM = 4, WN = 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nl = lane & 15, c = lane >> 4;
    const int m_base = blockIdx.y * 128 + (wave >> 1) * 64;
    const int n_base = blockIdx.x * 128 + (wave & 1) * 64;
    const int groups = K / kGroup;
    const int wpr = K / F::kCodesPerWord;

    const uint32_t* crow[WN];
    bool nvalid[WN];
    int nrow[WN];
#pragma unroll
    for (int jn = 0; jn < WN; ++jn) {
        nrow[jn] = n_base + 16 * jn + nl;
        nvalid[jn] = nrow[jn] < N;
        crow[jn] = codes + (int64_t)(nvalid[jn] ? nrow[jn] : 0) * wpr;
    }
    const uint16_t* xrow[WM];
    bool mvalid[WM];
#pragma unroll
    for (int im = 0; im < WM; ++im) {
        const int m = m_base + 16 * im + nl;
        mvalid[im] = m < M;
        xrow[im] = X + (int64_t)(mvalid[im] ? m : 0) * ldx;
    }

    f32x4 acc[WM][WN];
#pragma unroll
    for (int im = 0; im < WM; ++im)
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) acc[im][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int g = 0; g < groups; ++g) {
        LaneCodes<BITS> lc[WN];
        GroupConst gc[WN];
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) {
            uint16_t sb = 0, zb = 0;
            if (nvalid[jn]) {
                lc[jn].load(crow[jn], g, c);
                sb = scales[(int64_t)nrow[jn] * groups + g];
                zb = zeros[(int64_t)nrow[jn] * groups + g];
            } else {
                lc[jn].zero();
            }
            gc[jn] = group_const(sb, zb);
        }
        f16x8 a[WM][4];
#pragma unroll
        for (int im = 0; im < WM; ++im) load_a(xrow[im], mvalid[im], g, c, a[im]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x8 b[WN];
#pragma unroll
            for (int jn = 0; jn < WN; ++jn) b[jn] = lc[jn].frag(j, gc[jn]);
#pragma unroll
            for (int im = 0; im < WM; ++im)
#pragma unroll
                for (int jn = 0; jn < WN; ++jn) acc[im][jn] = mfma16(a[im][j], b[jn], acc[im][jn]);
        }
    }

#pragma unroll
    for (int im = 0; im < WM; ++im)
#pragma unroll
        for (int jn = 0; jn < WN; ++jn) {
            if (!nvalid[jn]) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m_base + 16 * im + 4 * c + r;
                if (m < M) store_out(Y, ldy, h, ldh, epi, m, nrow[jn], acc[im][jn][r]);
            }
        }
}

// ------------------------------------------------------------ dispatch ----

struct GemvShape {
    int lpr, cpr;
    bool ok;
};

GemvShape gemv_shape(int bits, int K) {
    const int quads = K * bits / 128;  // 16-byte lane chunks per row
    GemvShape s{0, 0, false};
    if (quads >= 64) {
        if (quads % 64) return s;
        s.lpr = 64;
        s.cpr = quads / 64;
        s.ok = s.cpr == 1 || s.cpr == 2 || s.cpr == 4 || s.cpr == 8;
    } else {
        s.lpr = quads;
        s.cpr = 1;
        s.ok = quads == 16 || quads == 32;
    }
    return s;
}

template <int BITS, int LPR, int CPR>
hipError_t launch_gemv_t(const GemmArgs& a, hipStream_t s) {
    constexpr int RPW = 64 / LPR;
    const int N = a.w->N;
    const int steps = (N + RPW - 1) / RPW;
    // Several rows per wave reuse the activations held in registers; keep at
    // least ~4 waves per CU for latency hiding.
    int U = 1;
    if (CPR <= 2 && steps >= 4 * 1024) U = 4;
    else if (CPR <= 4 && steps >= 2 * 1024) U = 2;
    const int waves_per_block = 4;
#define QG_GEMV_LAUNCH(UU)                                                                     \
    {                                                                                          \
        const int waves = (steps + UU - 1) / UU;                                               \
        const int blocks = (waves + waves_per_block - 1) / waves_per_block;                    \
        k_gemv<BITS, LPR, CPR, UU><<<blocks, 64 * waves_per_block, 0, s>>>(                    \
            a.X, a.w->codes, a.w->scales, a.w->zeros, a.w->K, N, a.Y, a.h, (int)a.epi);        \
    }
    if (U == 4) QG_GEMV_LAUNCH(4) else if (U == 2) QG_GEMV_LAUNCH(2) else QG_GEMV_LAUNCH(1)
#undef QG_GEMV_LAUNCH
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_gemv(const GemmArgs& a, hipStream_t s) {
    const GemvShape g = gemv_shape(BITS, a.w->K);
    if (g.lpr == 64) {
        switch (g.cpr) {
            case 1: return launch_gemv_t<BITS, 64, 1>(a, s);
            case 2: return launch_gemv_t<BITS, 64, 2>(a, s);
            case 4: return launch_gemv_t<BITS, 64, 4>(a, s);
            default: return launch_gemv_t<BITS, 64, 8>(a, s);
        }
    }
    if (g.lpr == 32) return launch_gemv_t<BITS, 32, 1>(a, s);
    return launch_gemv_t<BITS, 16, 1>(a, s);
}

template <int BITS>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
    constexpr int KSPLIT = 4;
    const int blocks = (a.w->N + 15) / 16;
    k_gemm_skinny<BITS, KSPLIT><<<blocks, 64 * KSPLIT, 0, s>>>(
        a.X, a.ldx, a.M, a.w->codes, a.w->scales, a.w->zeros, a.w->K, a.w->N, a.Y, a.ldy, a.h,
        a.ldh, (int)a.epi);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t s) {
    dim3 grid((a.w->N + 127) / 128, (a.M + 127) / 128);
    k_gemm_tiled<BITS><<<grid, 256, 0, s>>>(a.X, a.ldx, a.M, a.w->codes, a.w->scales,
                                             a.w->zeros, a.w->K, a.w->N, a.Y, a.ldy, a.h, a.ldh,
                                             (int)a.epi);
    return hipGetLastError();
}

}  // namespace

GemmPath gemm_path(int bits, int M, int K, int N) {
    (void)N;
    if (M == 1 && gemv_shape(bits, K).ok) return kPathGemv;
    if (M <= 16) return kPathSkinny;
    return kPathTiled;
}

size_t gemm_ws_bytes(int bits, int M, int K, int N) {
    (void)bits;
    (void)M;
    (void)K;
    (void)N;
    return 0;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    const int bits = a.w->bits;
    switch (gemm_path(bits, a.M, a.w->K, a.w->N)) {
        case kPathGemv: return bits == 4 ? launch_gemv<4>(a, s) : launch_gemv<2>(a, s);
        case kPathSkinny: return bits == 4 ? launch_skinny<4>(a, s) : launch_skinny<2>(a, s);
        default: return bits == 4 ? launch_tiled<4>(a, s) : launch_tiled<2>(a, s);
    }
}

}  // namespace qg
