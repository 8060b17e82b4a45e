// kernels_gemm.hip -- Y[M][N] = X[M][K] . dequant(W)[K][N] for layout-v1 INT4/INT2
// weights (quant_gemm / int2_gemm, "β-Informed Deployment Features" page,
// CTX-TIER section), FP16 activations, FP32 accumulation, FP16 output.
//
// Three kernel families, chosen by M:
//   * M == 1: the bandwidth-bound GEMV of kernels_gemv.hip.
//   * k_gemm_skinny (2 <= M <= 16): one or two 16-row MFMA tiles of output
//     channels per workgroup, K split over the workgroup's waves and reduced
//     through LDS in wave order.  v_mfma_f32_16x16x32_f16 takes X rows as A
//     (M padded to 16) and dequantised weights as B.
//   * M > 16: the LDS-staged MFMA GEMM of kernels_prefill.hip.
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

// ------------------------------------------------------ MFMA B fragments ----

// fp16_rne((q - z) s) of codes 2i, 2i+1 of word w: (1024 + q) pairs by one
// fused mask-and-or (mask in an SGPR, bias in a VGPR), then the exact
// subtraction of 1024 + z and one rounding of the product.
template <int BITS>
__device__ __forceinline__ f16x2 dequant_pair_fused(uint32_t w, int i, const GroupConst& gc,
                                                    uint32_t mask, uint32_t bias) {
    return (as_f16x2(((w >> (BITS * i)) & mask) | bias) + gc.nbz) * gc.s2;
}

// Codes of one 128-k group for one lane (k in [32c, 32c + 32) of row n).
template <int BITS>
struct LaneCodes;
template <>
struct LaneCodes<4> {
    u32x4 w;
    __device__ __forceinline__ void load(const uint32_t* row, int g, int c) {
        w = *(const u32x4*)(row + g * 16 + c * 4);
    }
    // FP16 B fragment of MFMA step j: codes 8j..8j+7 of the lane = word j.
    __device__ __forceinline__ f16x8 frag(int j, const GroupConst& gc, uint32_t mask,
                                          uint32_t bias) const {
        const uint32_t x = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
        const f16x2 p0 = dequant_pair_fused<4>(x, 0, gc, mask, bias);
        const f16x2 p1 = dequant_pair_fused<4>(x, 1, gc, mask, bias);
        const f16x2 p2 = dequant_pair_fused<4>(x, 2, gc, mask, bias);
        const f16x2 p3 = dequant_pair_fused<4>(x, 3, gc, mask, bias);
        return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
};
template <>
struct LaneCodes<2> {
    u32x2 w;
    __device__ __forceinline__ void load(const uint32_t* row, int g, int c) {
        w = *(const u32x2*)(row + g * 8 + c * 2);
    }
    // Step j: codes 8j..8j+7 = pairs 4(j&1)..4(j&1)+3 of word j>>1.
    __device__ __forceinline__ f16x8 frag(int j, const GroupConst& gc, uint32_t mask,
                                          uint32_t bias) const {
        const uint32_t x = (j >> 1) ? w.y : w.x;
        const int p = (j & 1) * 4;
        const f16x2 p0 = dequant_pair_fused<2>(x, p + 0, gc, mask, bias);
        const f16x2 p1 = dequant_pair_fused<2>(x, p + 1, gc, mask, bias);
        const f16x2 p2 = dequant_pair_fused<2>(x, p + 2, gc, mask, bias);
        const f16x2 p3 = dequant_pair_fused<2>(x, p + 3, gc, mask, bias);
        return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
};

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- skinny ----

// 2 <= M <= 16.  A workgroup of W = 8 waves computes NT tiles of 16 output
// channels over one K part (at most kSkinnyMaxK values; K is cut into S
// parts, summed by k_splitk_reduce when S > 1).  The activation rows of the part are staged
// once in LDS -- the M rows of R values (LDS rows M..15 hold stale data that
// only reaches accumulator rows that are never stored),
// 16-byte chunk ci of row m at chunk slot ci ^ (m % 16), so the fragment
// reads of the 16 rows hit distinct banks -- by LDS DMA of contiguous row
// pieces; the MFMA A fragments then come from LDS instead of 16-byte pieces of
// 16 rows 2K bytes apart in global memory, which had kept the skinny shapes
// far from the GEMV's bandwidth (measured: 15 us -> 8 us plus the reduction
// for M = 16, K = 8192, N = 2048).  Wave w takes the part's groups w, w+W, ...;
// the W partial tiles are summed through LDS in wave order.  (Normalising
// h inside this kernel, as the GEMV does, costs more than the LayerNorm
// kernel: every workgroup must read all M rows of h.)  NT = 2 feeds each A
// fragment read to two MFMAs and halves the activation staging per weight
// byte; it is used while the launch keeps at least kSkinnyPairMinWgs
// workgroups (measured on MI355X, M = 2..16: 9-14 % faster for the loop
// block's QKV, FFN-up and K-split down projections, 14 % slower for the
// 2048-channel out projection, whose 64 workgroups leave most CUs idle;
// NT = 4 was slower everywhere).  Each output's MFMA chain is the same for
// every NT, so the results are too.
constexpr int kSkinnyMaxK = 2048;
// Eight waves rather than four: each wave has half the groups of a part, so
// two waves share every SIMD and one's dequantisation overlaps the other's
// loads (measured on MI355X: every skinny shape 1-5 % faster, C5a 31.1 ->
// 30.7 us per iteration).
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyPairMinWgs = 192;

template <int BITS, int NT, int W>
__global__ __launch_bounds__(64 * W) void k_gemm_skinny(
    const uint16_t* __restrict__ X, int64_t ldx, int M, const uint32_t* __restrict__ codes,
    int64_t ldc, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, SzIdx sz,
    int K, int N, int S, OutEpi out, float* __restrict__ part) {
    static_assert(NT == 1 || NT == 2, "one or two column tiles (wave t stores tile t)");
    static_assert(W == 4 || W == 8, "four or eight waves");
    constexpr int kMaxGpw = kSkinnyMaxK / kGroup / W;  // groups per wave
    __shared__ __attribute__((aligned(1024))) uint8_t xs[16 * kSkinnyMaxK * 2];
    __shared__ f32x4 red[W][NT][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, c = lane >> 4;
    const int groups = K / kGroup;
    const int p = blockIdx.y;
    const int gbeg = (int)((int64_t)groups * p / S);
    const int gcnt = (int)((int64_t)groups * (p + 1) / S) - gbeg;  // <= kSkinnyMaxK / 128
    const int cpr = gcnt * 16;  // 16-byte chunks per staged row

    // weights of this wave's groups first, for each column tile (rows past N
    // clamped, zeroed by scale)
    LaneCodes<BITS> lc[NT][kMaxGpw];
    uint16_t sb[NT][kMaxGpw], zb[NT][kMaxGpw];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = (blockIdx.x * NT + t) * 16 + nl;
        const bool nvalid = n < N;
        const int nr = nvalid ? n : N - 1;
        const uint32_t* crow = codes + (int64_t)nr * ldc;
#pragma unroll
        for (int i = 0; i < kMaxGpw; ++i) {
            const int gi = wave + W * i;
            if (gi < gcnt) {
                const int g = gbeg + gi;
                lc[t][i].load(crow, g, c);
                sb[t][i] = nvalid ? scales[sz.at(nr, g)] : (uint16_t)0;
                zb[t][i] = zeros[sz.at(nr, g)];
            }
        }
    }

    // the part's M activation rows, 1 KiB per DMA instruction.  LDS rows
    // M..15 are left as they are: MFMA rows do not mix, so they only reach
    // accumulator rows >= M, which are never stored.
    const i32x4 rx = make_rsrc_sgpr(X, ((int64_t)(M - 1) * ldx + K) * 2);
    const int units = M * cpr;
    if (cpr % 64 == 0) {
        // each instruction's 64 units lie in one row: the row and the run's
        // first chunk advance by scalar steps (no per-lane division)
        int row = (wave * 64) / cpr, slot0 = (wave * 64) % cpr;
        for (int u0 = wave * 64; u0 < units; u0 += 64 * W) {
            const int ci = (slot0 + lane) ^ (row & 15);
            dma16(rx, xs + u0 * 16,
                  (uint32_t)(((int64_t)row * ldx + (int64_t)gbeg * kGroup + ci * 8) * 2));
            slot0 += 64 * W;
            while (slot0 >= cpr) {
                slot0 -= cpr;
                ++row;
            }
        }
    } else {
        for (int u0 = wave * 64; u0 < units; u0 += 64 * W) {
            const int u = u0 + lane;
            const int row = u / cpr, slot = u % cpr;
            const int ci = slot ^ (row & 15);
            dma16(rx, xs + u0 * 16, (uint32_t)((row * ldx + (int64_t)gbeg * kGroup + ci * 8) * 2));
        }
    }
    wait_vmcnt<0>();
    lds_barrier();

    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const uint32_t pair_mask = sgpr_const(Fmt<BITS>::kPairMask);
    const uint32_t bias = vgpr_const(kBias2);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = zero4;
#pragma unroll
    for (int i = 0; i < kMaxGpw; ++i) {
        const int gi = wave + W * i;
        if (gi < gcnt) {
            GroupConst gc[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) gc[t] = group_const(sb[t][i], zb[t][i]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ci = gi * 16 + 4 * c + j;  // row nl, k = 128 gi + 32 c + 8 j
                const f16x8 a = *(const f16x8*)(xs + (nl * cpr + (ci ^ nl)) * 16);
                f16x8 bf[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) bf[t] = lc[t][i].frag(j, gc[t], pair_mask, bias);
                // MFMAs at raised wave priority (two workgroups share a CU:
                // measured 2-4 % faster, bit-identical)
                __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] = mfma16(a, bf[t], acc[t]);
                __builtin_amdgcn_s_setprio(0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    // wave t sums column tile t in wave order and stores it
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (wave != t) continue;
        const int n = (blockIdx.x * NT + t) * 16 + nl;
        if (n >= N) continue;
        f32x4 sum = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[w][t][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * c + r;
            if (m >= M) continue;
            if (part != nullptr)
                part[(int64_t)p * M * N + (int64_t)m * N + n] = sum[r];
            else
                epi_store(out, m, n, sum[r]);
        }
    }
}

// ------------------------------------------------------------ dispatch ----

// K parts of the skinny kernel: enough that each spans at most kSkinnyMaxK.
// In parts mode the partials are summed by the launch that follows anyway,
// so more parts cost little and give more workgroups with shorter activation
// staging: at least 4 parts of at least 4 groups where K allows (measured on
// MI355X, the D = 2048 block's out projection at M = 4..16: 4 parts 5-7 %
// faster per loop iteration than 1 or 2, 8 parts slower).
int skinny_parts(int K, bool parts_mode = false) {
    int S = (K + kSkinnyMaxK - 1) / kSkinnyMaxK;
    if (parts_mode) {
        const int groups = K / kGroup;
        while (S < 4 && groups % (2 * S) == 0 && groups / (2 * S) >= 4) S *= 2;
    }
    return S;
}

template <int BITS>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
    const int S = skinny_parts(a.w->K, a.parts != nullptr);
    float* part = S > 1 || a.parts ? (float*)a.ws : nullptr;
    const int pairs = (a.w->N + 31) / 32;
    if ((int64_t)pairs * S >= kSkinnyPairMinWgs)
        k_gemm_skinny<BITS, 2, kSkinnyWaves><<<dim3(pairs, S), 64 * kSkinnyWaves, 0, s>>>(
            a.X, a.ldx, a.M, a.w->codes, code_ld(*a.w), a.w->scales, a.w->zeros, sz_idx(*a.w),
            a.w->K, a.w->N, S,
            a.out(), part);
    else
        k_gemm_skinny<BITS, 1, kSkinnyWaves><<<dim3((a.w->N + 15) / 16, S), 64 * kSkinnyWaves, 0, s>>>(
            a.X, a.ldx, a.M, a.w->codes, code_ld(*a.w), a.w->scales, a.w->zeros, sz_idx(*a.w),
            a.w->K, a.w->N, S,
            a.out(), part);
    hipError_t e = hipGetLastError();
    if (a.parts) *a.parts = S;
    if (e != hipSuccess || S == 1 || a.parts) return e;
    return launch_splitk_reduce(part, S, a, s);
}

}  // namespace

GemmPath gemm_path(int bits, int M, int K, int N) {
    (void)N;
    if (M == 1 && gemv_supported(bits, K)) return kPathGemv;
    if (M <= 16 && K <= 4 * kSkinnyMaxK) return kPathSkinny;
    return kPathTiled;
}

bool gemm_fuses_layernorm(int bits, int M, int K, int N) {
    return gemm_path(bits, M, K, N) == kPathGemv && K % 1024 == 0 && K <= 8192;
}

bool gemm_fuses_swiglu(int bits, int M, int K, int N) {
    return gemm_path(bits, M, K, N) == kPathGemv && gemv_pairs_supported(bits, K);
}

size_t gemm_parts_ws_bytes(int bits, int M, int K, int N) {
    switch (gemm_path(bits, M, K, N)) {
        case kPathSkinny: return (size_t)skinny_parts(K, true) * M * N * sizeof(float);
        case kPathTiled: {
            const size_t split = prefill_ws_bytes(M, N, K);
            return split > 0 ? split : (size_t)M * N * sizeof(float);
        }
        default: return 0;
    }
}

size_t gemm_ws_bytes(int bits, int M, int K, int N) {
    switch (gemm_path(bits, M, K, N)) {
        case kPathSkinny: {
            const int S = skinny_parts(K);
            return S > 1 ? (size_t)S * M * N * sizeof(float) : 0;
        }
        case kPathTiled: return prefill_ws_bytes(M, N, K);
        default: return 0;
    }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
    const int bits = a.w->bits;
    if (a.w2 != nullptr && !(gemm_fuses_swiglu(bits, a.M, a.w->K, a.w->N) && a.epi == kStore &&
                             a.w2->bits == bits && a.w2->K == a.w->K && a.w2->N == a.w->N &&
                             a.w2->group == a.w->group))
        return hipErrorInvalidValue;
    const GemmPath path = gemm_path(bits, a.M, a.w->K, a.w->N);
    if (a.parts != nullptr && (path == kPathGemv || a.w2 != nullptr))
        return hipErrorInvalidValue;  // parts mode is for the MFMA kernels
    switch (path) {
        case kPathGemv: return launch_gemv(a, s);
        case kPathSkinny: return bits == 4 ? launch_skinny<4>(a, s) : launch_skinny<2>(a, s);
        default: return launch_prefill(a, s);
    }
}

}  // namespace qg
