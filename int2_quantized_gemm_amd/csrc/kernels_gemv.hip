// kernels_gemv.hip -- Y[1][N] = x[K] . dequant(W)[K][N] for layout-v1 INT4/INT2
// weights: the M == 1 path of quant_gemm / int2_gemm ("β-Informed Deployment
// Features" page, CTX-TIER section), FP16 activations, FP32 accumulation, FP16
// output, optionally with the activations as the LayerNorm of an FP32 row and
// as the SwiGLU pair of a gated FFN (the loop block of the "Model" page).
//
// k_gemv is bandwidth-bound: lanes split K, each lane loads the 32 contiguous
// codes of a chunk (16 bytes INT4, 8 bytes INT2; a wave reads a contiguous run
// of a row), converts codes with the exponent-bias trick and accumulates
// x . (1024 + 2^j q) with v_dot2_f32_f16; bias, zero point and the per-group
// scale are applied once per lane chunk.  Lane partials of a row are combined
// by a fixed xor-butterfly (deterministic).
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace qg {
namespace {

// ------------------------------------------------------------------ GEMV ----

// Dot products of one lane chunk (32 codes: WPL = b packed words) with its
// activations.  The chunk holds 32 codes for both widths, so an INT2 lane does
// the same decode and activation work per chunk as an INT4 lane and moves half
// the bytes (16-byte chunks would double the activation loads and the
// arithmetic per byte of INT2 codes).
//
// Codes 2i and 2i+1 of a word sit at bits b*i and 16 + b*i.  Rather than
// shifting every pair down, a word and its copy shifted right by 8 are each
// masked at the NC = 8/b code positions of a byte: mask class j keeps the
// codes at bits b*j and 16 + b*j, and OR-ing 0x6400 into both halves gives
// the FP16 pair 1024 + 2^(b*j) * q exactly (all values stay below 2048, where
// the FP16 spacing is 1).  Class j accumulates x . (1024 + 2^(b*j) q) in FP32
// with v_dot2_f32_f16; the bias 1024 * sum(x) and the factor 2^(b*j) come
// out once per chunk from precomputed activation sums.
template <int BITS>
struct GemvMath {
    using F = Fmt<BITS>;
    static constexpr int NC = 8 / BITS;   // mask classes
    static constexpr int PPW = 16 / BITS;  // FP16 pairs per word (= 2 * NC)
    static constexpr int WPL = BITS;       // words per lane chunk (32 codes)
    static constexpr int PAIRS = 16;       // FP16 activation pairs per chunk
    using Chunk = std::conditional_t<BITS == 4, u32x4, u32x2>;

    // Pair index (relative to the chunk) of class j, half h (h = 1: word >> 8).
    static __device__ __forceinline__ int pair(int q, int h, int j) { return q * PPW + j + NC * h; }

    // The class masks (in SGPRs) and the bias (in a VGPR), so that each
    // mask-and-or is one instruction.
    struct Consts {
        uint32_t mask[NC];
        uint32_t bias;
        __device__ __forceinline__ Consts() {
#pragma unroll
            for (int j = 0; j < NC; ++j) mask[j] = sgpr_const(F::kPairMask << (BITS * j));
            bias = vgpr_const(kBias2);
        }
    };

    static __device__ __forceinline__ void accumulate(const Chunk& w, const f16x2* xp,
                                                      const Consts& k, float acc[NC]) {
#pragma unroll
        for (int q = 0; q < WPL; ++q) {
            const uint32_t v[2] = {w[q], w[q] >> 8};
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < NC; ++j)
                    acc[j] = __builtin_amdgcn_fdot2(as_f16x2((v[h] & k.mask[j]) | k.bias),
                                                    xp[pair(q, h, j)], acc[j], false);
        }
    }

    // Per-class sums of the activations of a chunk.
    static __device__ __forceinline__ void xsums(const f16x2* xp, float xs[NC]) {
        const f16x2 one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
        for (int j = 0; j < NC; ++j) xs[j] = 0.0f;
#pragma unroll
        for (int q = 0; q < WPL; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < NC; ++j)
                    xs[j] = __builtin_amdgcn_fdot2(xp[pair(q, h, j)], one, xs[j], false);
    }

    // sum_k x_k * (q_k - z) of the chunk, from the class accumulators.
    static __device__ __forceinline__ float centred(const float acc[NC], const float xs[NC],
                                                    float xs_all, float z) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < NC; ++j)
            t += (acc[j] - 1024.0f * xs[j]) * (1.0f / (float)(1 << (BITS * j)));
        return t - z * xs_all;
    }
};

// LPR lanes cover one row per chunk of 32*LPR codes; CPR chunks per row;
// 64/LPR rows per wave step; U row steps per wave; K = 32*LPR*CPR is a
// compile-time constant of each variant.  KW > 1 (rows of several chunks
// per lane, LPR = 64) splits K over KW waves of the workgroup: wave w takes
// chunks [w' CPR/KW, (w'+1) CPR/KW) (w' = w mod KW) of the same U rows, so
// each wave loads only its part of the activations (a wave holding whole
// rows re-reads all K activations per U rows, which for K = 8192 moved more
// bytes than the codes); the KW wave sums of a row are added in wave order
// through LDS.  With LN, the activations are
// fp16(LayerNorm(hln)): the workgroup's 256 threads normalise the row once
// (mean, then population variance of the centred values, eps 1e-5, reduced
// by DPP in each wave and then in wave order through LDS), stage it in LDS
// for the lanes to pick up, and workgroup 0 also writes it to norm_out.
//
// NW = 2 is the SwiGLU pair of a gated FFN: weight 0 is the gate and weight 1
// the up projection, both of the same shape and bits.  Each row step loads
// the same rows of both, and the lane that finishes row n stores
// g = fp16(x . Wgate[n]) to gout[n] and fp16(silu(g) * fp16(x . Wup[n])) to
// out.Y[n] (plain store epilogue), so one launch and one activation pass serve
// both projections.
struct GemvWeights {
    const uint32_t* codes[2];
    const uint16_t* scales[2];
    const uint16_t* zeros[2];
    int64_t ldc[2];  // code row strides (words)
    SzIdx sz;        // scale addressing, the same for both weights
};

template <int BITS, int LPR, int CPR, int KW, int U, bool LN, int NW>
__global__ __launch_bounds__(256) void k_gemv(const uint16_t* __restrict__ X,
                                              const float* __restrict__ hln,
                                              uint16_t* __restrict__ norm_out,
                                              GemvWeights W, int N, OutEpi out,
                                              uint16_t* __restrict__ gout) {
    using F = Fmt<BITS>;
    using G = GemvMath<BITS>;
    constexpr int RPW = 64 / LPR;
    constexpr int WPL = G::WPL;
    constexpr int PAIRS = G::PAIRS;  // FP16 pairs of x per lane and chunk
    constexpr int K = 32 * LPR * CPR;
    constexpr int CW = CPR / KW;  // chunks per lane (this wave's part of K)
    static_assert(KW == 1 || (LPR == 64 && CPR % KW == 0 && KW <= 4 && U <= 64),
                  "K parts of whole waves");
    const int lane = threadIdx.x & 63;
    const int wib = threadIdx.x >> 6;  // wave in the workgroup
    const int kp = wib % KW;           // this wave's K part
    // Workgroup i runs on XCD i mod 8 and each XCD has its own L2: the
    // launch's first 8 floor(nb / 8) workgroups are renumbered so that each
    // XCD takes a contiguous eighth of the row blocks (the rest keep their
    // index).  The loop re-reads the same weights every iteration, and each
    // XCD then keeps a contiguous share of them in its L2 (measured: the
    // K = 8192 down projection 3.38 -> 3.25 us, the loop block at M = 1
    // 1.5-2.6 % faster per iteration, bit-identical).
    const int nb8 = (int)gridDim.x & ~7;
    const int blk = (int)blockIdx.x < nb8
                        ? ((int)blockIdx.x & 7) * (nb8 >> 3) + ((int)blockIdx.x >> 3)
                        : (int)blockIdx.x;
    const int set = blk * (4 / KW) + wib / KW;
    const int sub = lane % LPR;
    const int rsub = lane / LPR;
    const int row0 = set * U * RPW;
    const int c0 = kp * CW;  // first chunk of the lane
    const bool active = row0 < N;
    // (LN variants and K parts keep every wave for the barriers)
    if (!LN && KW == 1 && !active) return;

    // Load order.  Vector-memory loads of a wave complete in issue order, so
    // the activations (or the LayerNorm input) go first: the arithmetic that
    // needs only them (the LayerNorm, the per-chunk activation sums) then
    // waits for them alone and runs while the weight loads are in flight, and
    // each chunk's dot products wait only for that chunk's codes.  Every load
    // is unconditional (rows past N read row N - 1 and are never stored), so
    // no branch splits the loads into dependent round trips.
    constexpr int VPT = LN ? K / 256 : 4;  // LayerNorm values per thread
    float4 hv[VPT / 4];
    u32x4 xv[CW][PAIRS / 4];
    if constexpr (LN) {
        static_assert(K % 1024 == 0, "K must be a multiple of 1024 for the fused LayerNorm");
        const float4* hp = (const float4*)(hln + threadIdx.x * VPT);
#pragma unroll
        for (int i = 0; i < VPT / 4; ++i) hv[i] = hp[i];
    } else {
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const u32x4* xp = (const u32x4*)(X + ((c0 + c) * LPR + sub) * 32);
#pragma unroll
            for (int v = 0; v < PAIRS / 4; ++v) xv[c][v] = xp[v];
        }
    }

    typename G::Chunk wv[NW][U][CW];
    uint16_t sv[NW][U][CW], zv[NW][U][CW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = min(row0 + u * RPW + rsub, N - 1);
#pragma unroll
        for (int b = 0; b < NW; ++b)
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                const int wi = ((c0 + c) * LPR + sub) * WPL;
                wv[b][u][c] = *(const typename G::Chunk*)(W.codes[b] + (int64_t)row * W.ldc[b] + wi);
                const int64_t sg = W.sz.at(row, wi / F::kWordsPerGroup);
                sv[b][u][c] = W.scales[b][sg];
                zv[b][u][c] = W.zeros[b][sg];
            }
    }
    // The epilogue's own input (the residual element, or the gate output),
    // loaded with the rest so that the store does not wait for a round trip.
    // With K parts lane u < U of the part-0 wave stores row u of the set.
    constexpr int NE = KW == 1 ? U : 1;
    uint32_t ein[NE];
#pragma unroll
    for (int u = 0; u < NE; ++u) {
        const int row = KW == 1 ? min(row0 + u * RPW + rsub, N - 1)
                                : min(row0 + min(lane, U - 1), N - 1);
        ein[u] = NW == 1 ? epi_input(out, 0, row, W.codes[0]) : 0u;
    }
    // Keep the compiler's scheduler from sinking loads into the arithmetic
    // below (it would, to save registers, and each sunk load then costs a
    // memory round trip of its own).
    __builtin_amdgcn_sched_barrier(0);

    // Activations for this lane's k positions, reused for every row.
    f16x2 xr[CW][PAIRS];
    if constexpr (LN) {
        // The workgroup's 256 threads normalise the row once: mean, then the
        // population variance of the centred values (eps 1e-5), each reduced
        // by DPP in every wave and then in wave order through LDS; the FP16
        // result is staged in LDS for the lanes to pick up.  The barriers
        // wait for LDS traffic only, never for the weight loads in flight.
        __shared__ uint32_t xl[K / 2];
        __shared__ float part[2][4];
        const int t = threadIdx.x;
        const int w = t >> 6;
        float v[VPT];
#pragma unroll
        for (int i = 0; i < VPT / 4; ++i) {
            v[4 * i] = hv[i].x;
            v[4 * i + 1] = hv[i].y;
            v[4 * i + 2] = hv[i].z;
            v[4 * i + 3] = hv[i].w;
        }
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) sum += v[i];
        sum = segment_sum<64>(sum);
        if (lane == 0) part[0][w] = sum;
        lds_barrier();
        const float mean = ((part[0][0] + part[0][1]) + (part[0][2] + part[0][3])) / (float)K;
        float sq = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            v[i] -= mean;
            sq += v[i] * v[i];
        }
        sq = segment_sum<64>(sq);
        if (lane == 0) part[1][w] = sq;
        lds_barrier();
        const float var = ((part[1][0] + part[1][1]) + (part[1][2] + part[1][3])) / (float)K;
        const float rstd = 1.0f / sqrtf(var + 1e-5f);
#pragma unroll
        for (int i = 0; i < VPT / 2; ++i)
            xl[t * (VPT / 2) + i] =
                as_u32(f16x2{(f16)(v[2 * i] * rstd), (f16)(v[2 * i + 1] * rstd)});
        if (norm_out != nullptr && blockIdx.x == 0) {
            uint32_t* op = (uint32_t*)norm_out + t * (VPT / 2);
#pragma unroll
            for (int i = 0; i < VPT / 2; ++i) op[i] = xl[t * (VPT / 2) + i];
        }
        lds_barrier();
        if (KW == 1 && !active) return;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const int p0 = ((c0 + c) * LPR + sub) * 16;
#pragma unroll
            for (int i = 0; i < PAIRS; ++i) xr[c][i] = as_f16x2(xl[p0 + i]);
        }
    } else {
#pragma unroll
        for (int c = 0; c < CW; ++c)
#pragma unroll
            for (int v = 0; v < PAIRS / 4; ++v) {
                xr[c][4 * v + 0] = as_f16x2(xv[c][v].x);
                xr[c][4 * v + 1] = as_f16x2(xv[c][v].y);
                xr[c][4 * v + 2] = as_f16x2(xv[c][v].z);
                xr[c][4 * v + 3] = as_f16x2(xv[c][v].w);
            }
    }
    float xs[CW][G::NC], xs_all[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
        G::xsums(xr[c], xs[c]);
        xs_all[c] = 0.0f;
#pragma unroll
        for (int j = 0; j < G::NC; ++j) xs_all[c] += xs[c][j];
    }

    const typename G::Consts kc;
    __shared__ float red[KW > 1 ? 4 : 1][KW > 1 ? U : 1][NW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float acc[NW];
#pragma unroll
        for (int b = 0; b < NW; ++b) {
            acc[b] = 0.0f;
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                float a[G::NC];
#pragma unroll
                for (int j = 0; j < G::NC; ++j) a[j] = 0.0f;
                G::accumulate(wv[b][u][c], xr[c], kc, a);
                const float t = G::centred(a, xs[c], xs_all[c], (float)as_f16(zv[b][u][c]));
                acc[b] += t * (float)as_f16(sv[b][u][c]);
            }
            acc[b] = segment_sum<LPR>(acc[b]);
            if constexpr (KW > 1) {
                if (lane == 0) red[wib][u][b] = acc[b];
            }
        }
        const int row = row0 + u * RPW + rsub;
        if (KW == 1 && sub == 0 && row < N) {
            if constexpr (NW == 1) {
                epi_store_pre(out, 0, row, acc[0], ein[KW == 1 ? u : 0]);
            } else {
                const uint16_t g16 = f32_to_f16_bits(acc[0]);
                gout[row] = g16;
                out.Y[row] = swiglu_f16(g16, f32_to_f16_bits(acc[1]));
            }
        }
    }
    if constexpr (KW > 1) {
        // the K parts of row row0 + lane, summed in part order
        lds_barrier();
        const int row = row0 + lane;
        if (kp == 0 && lane < U && row < N) {
            float acc[NW];
#pragma unroll
            for (int b = 0; b < NW; ++b) {
                acc[b] = red[wib][lane][b];
#pragma unroll
                for (int q = 1; q < KW; ++q) acc[b] += red[wib + q][lane][b];
            }
            if constexpr (NW == 1) {
                epi_store_pre(out, 0, row, acc[0], ein[0]);
            } else {
                const uint16_t g16 = f32_to_f16_bits(acc[0]);
                gout[row] = g16;
                out.Y[row] = swiglu_f16(g16, f32_to_f16_bits(acc[1]));
            }
        }
    }
}

// ------------------------------------------------------------ dispatch ----

struct GemvShape {
    int lpr, cpr;
    bool ok;
};

GemvShape gemv_shape(int bits, int K) {
    (void)bits;  // a lane chunk is 32 codes for both widths
    const int chunks = K / 32;  // lane chunks per row
    GemvShape s{0, 0, false};
    if (chunks >= 64) {
        if (chunks % 64) return s;
        s.lpr = 64;
        s.cpr = chunks / 64;
        s.ok = s.cpr == 1 || s.cpr == 2 || s.cpr == 4 || s.cpr == 8;
    } else {
        s.lpr = chunks;
        s.cpr = 1;
        s.ok = chunks == 16 || chunks == 32;
    }
    return s;
}

// Rows per wave U: several rows per wave amortise the activations held in
// registers (and the fused LayerNorm) but cut the number of waves in flight.
// Measured on MI355X inside the looped block with its weights cache-resident
// (D = 2048, F = 8192, M = 1), rows of one chunk per lane: U = 2 from 2048
// row steps (QKV, out, up, the SwiGLU pair), else U = 1.  U = 4 on the
// 8192-step FFN projections was even for INT4 and 2-6 % slower per iteration
// for INT2 and the SwiGLU pair; U = 1 and U = 4 on the 2048-step ones were
// slower.  At most 8 outstanding code loads per lane (U * CPR/KW * NW <= 8,
// NW = 2 for the SwiGLU pair).
template <int BITS, int LPR, int CPR, int KW, int U, bool LN, int NW>
hipError_t launch_gemv_u(const GemmArgs& a, hipStream_t s) {
    static_assert(U * (CPR / KW) * NW <= 8, "at most 8 code loads per lane");
    constexpr int RPW = 64 / LPR;
    constexpr int kSetsPerBlock = 4 / KW;  // row sets of U * RPW rows
    const int N = a.w->N;
    const int steps = (N + RPW - 1) / RPW;
    const int sets = (steps + U - 1) / U;
    const int blocks = (sets + kSetsPerBlock - 1) / kSetsPerBlock;
    const qg_weight* w1 = NW == 2 ? a.w2 : a.w;
    const GemvWeights W{{a.w->codes, w1->codes}, {a.w->scales, w1->scales}, {a.w->zeros, w1->zeros},
                        {code_ld(*a.w), code_ld(*w1)}, sz_idx(*a.w)};
    k_gemv<BITS, LPR, CPR, KW, U, LN, NW><<<blocks, 256, 0, s>>>(
        a.X, a.ln_h, a.norm_out, W, N, a.out(), a.g_out);
    return hipGetLastError();
}

// The fused LayerNorm needs K = 32*LPR*CPR to be a multiple of 1024 and
// at most 8192 (the LN input is a residual row of D <= 8192 values).
template <int BITS, int LPR, int CPR>
constexpr bool ln_variant_ok() {
    constexpr int K = 32 * LPR * CPR;
    return K % 1024 == 0 && K <= 8192;
}

// Rows of several chunks per lane (K >= 4096) split K over KW = min(CPR, 4)
// waves, with U = 8 / (CPR/KW * NW) rows per set (the same code loads per
// lane as whole rows at U = 2), halved while that leaves fewer than 256
// workgroups.
template <int BITS, int LPR, int CPR, bool LN, int NW>
hipError_t launch_gemv_kparts(const GemmArgs& a, hipStream_t s) {
    constexpr int KW = CPR < 4 ? CPR : 4;
    constexpr int UMAX = 8 / (CPR / KW * NW);
    const int N = a.w->N;
    auto blocks = [&](int u) { return (N + u * (4 / KW) - 1) / (u * (4 / KW)); };
    if (blocks(UMAX) >= 256 || UMAX == 1) return launch_gemv_u<BITS, LPR, CPR, KW, UMAX, LN, NW>(a, s);
    if constexpr (UMAX >= 2) {
        if (blocks(UMAX / 2) >= 256 || UMAX == 2)
            return launch_gemv_u<BITS, LPR, CPR, KW, UMAX / 2, LN, NW>(a, s);
    }
    if constexpr (UMAX >= 4) {
        return launch_gemv_u<BITS, LPR, CPR, KW, UMAX / 4, LN, NW>(a, s);
    }
    return hipErrorInvalidValue;  // not reached
}

template <int BITS, int LPR, int CPR, bool LN>
hipError_t launch_gemv_t(const GemmArgs& a, hipStream_t s) {
    if constexpr (LN && !ln_variant_ok<BITS, LPR, CPR>()) {
        return hipErrorInvalidValue;  // never dispatched: see gemm_fuses_layernorm
    } else if constexpr (CPR > 1) {
        if (a.w2 != nullptr) {  // SwiGLU pair: two weights per row
            if constexpr (CPR <= 4) return launch_gemv_kparts<BITS, LPR, CPR, LN, 2>(a, s);
            return hipErrorInvalidValue;  // never dispatched: see gemm_fuses_swiglu
        }
        return launch_gemv_kparts<BITS, LPR, CPR, LN, 1>(a, s);
    } else {
    constexpr int RPW = 64 / LPR;
    const int steps = (a.w->N + RPW - 1) / RPW;
    if (a.w2 != nullptr) {  // SwiGLU pair: two weights per row step
        if (steps >= 2 * 1024) return launch_gemv_u<BITS, LPR, CPR, 1, 2, LN, 2>(a, s);
        return launch_gemv_u<BITS, LPR, CPR, 1, 1, LN, 2>(a, s);
    }
    if (steps >= 2 * 1024) return launch_gemv_u<BITS, LPR, CPR, 1, 2, LN, 1>(a, s);
    return launch_gemv_u<BITS, LPR, CPR, 1, 1, LN, 1>(a, s);
    }
}

template <int BITS, bool LN>
hipError_t launch_gemv_ln(const GemmArgs& a, hipStream_t s) {
    const GemvShape g = gemv_shape(BITS, a.w->K);
    if (g.lpr == 64) {
        switch (g.cpr) {
            case 1: return launch_gemv_t<BITS, 64, 1, LN>(a, s);
            case 2: return launch_gemv_t<BITS, 64, 2, LN>(a, s);
            case 4: return launch_gemv_t<BITS, 64, 4, LN>(a, s);
            default: return launch_gemv_t<BITS, 64, 8, LN>(a, s);
        }
    }
    if (g.lpr == 32) return launch_gemv_t<BITS, 32, 1, LN>(a, s);
    return launch_gemv_t<BITS, 16, 1, LN>(a, s);
}

template <int BITS>
hipError_t launch_gemv_bits(const GemmArgs& a, hipStream_t s) {
    return a.ln_h ? launch_gemv_ln<BITS, true>(a, s) : launch_gemv_ln<BITS, false>(a, s);
}

}  // namespace

bool gemv_supported(int bits, int K) { return gemv_shape(bits, K).ok; }

bool gemv_pairs_supported(int bits, int K) {
    const GemvShape g = gemv_shape(bits, K);
    return g.ok && g.cpr <= 4;
}

hipError_t launch_gemv(const GemmArgs& a, hipStream_t s) {
    return a.w->bits == 4 ? launch_gemv_bits<4>(a, s) : launch_gemv_bits<2>(a, s);
}

}  // namespace qg
