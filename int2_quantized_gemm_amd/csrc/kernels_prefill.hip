// kernels_prefill.hip -- prefill GEMM (M > 16): Y[M][N] = X[M][K] . dequant(W)[K][N]
// on FP16 MFMA, for the chunked-prefill row counts of the "Model" page
// (prefill_chunk = 512 rows) and single-shot prefill.
//
// One K step is one quantisation group (128 values along K).  Per step the
// workgroup
//   * stages the A tile (BM x 128 FP16 activations) in LDS, and
//   * dequantises the B tile once -- BN output channels x 128 codes, each
//     converted to fp16_rne((q - z) * s) with the exponent-bias trick -- into
//     LDS, so every weight is decoded once per workgroup, not once per wave;
// the next group's global loads (raw buffer loads: rows past M or N read 0)
// are issued before the current group's MFMAs, and with two LDS stages the
// next group's LDS stores are interleaved with the current MFMAs (one
// barrier per step).  Both operands are K-contiguous per row, matching the
// MFMA lane layout, so no transpose is needed; rows are padded by 16 bytes in
// LDS against bank conflicts of the 16-byte fragment reads.
//
// Instruction: v_mfma_f32_32x32x16_f16 (measured on MI355X at about twice the
// FP16 rate of the 16x16x32 form).  Lane l supplies row (A) / column (B)
// l % 32 and the eight k values 16j + 8(l / 32) .. +8 of k-slice j; the
// accumulator holds D[8*(r/4) + 4*(l/32) + r%4][l % 32] in register r.  The
// eight k-slices of a step are split over KSPLIT waves that share a wave
// tile; their partial tiles are summed through LDS in k-part order at the end.
// Accumulation is FP32 in a fixed order (deterministic); the epilogue rounds
// to FP16 and optionally adds the rounded value into the FP32 residual.
#include "device.h"
#include "internal.h"

namespace qg {
namespace {

constexpr int kBK = 128;              // K values per step (one group)
constexpr int kPitch = kBK + 8;       // FP16 per LDS row (16-byte pad)

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BITS, int BM, int BN, int WAVES_M, int WAVES_N, int KSPLIT, int STAGES>
struct Cfg {
    static constexpr int WAVES = WAVES_M * WAVES_N * KSPLIT;
    static constexpr int THREADS = 64 * WAVES;
    static_assert(WAVES == 4 || WAVES == 8, "four or eight waves per workgroup");
    static_assert(KSPLIT == 1 || KSPLIT == 2 || KSPLIT == 4, "k slices split 1, 2 or 4 ways");
    static_assert(STAGES == 1 || STAGES == 2, "one or two LDS stages");
    using F = Fmt<BITS>;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
    static constexpr int WM = WTM / 32, WN = WTN / 32;           // 32x32 MFMA tiles per wave
    static_assert(WM >= 1 && WN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "32x32 tiles");
    static constexpr int A_CHUNKS = BM * kBK / 8;                // 16-byte chunks of A
    static constexpr int A_PER_T = A_CHUNKS / THREADS;
    static constexpr int WPG = F::kWordsPerGroup;                // code words per row and step
    static constexpr int CHUNKS_PER_ROW = WPG / 4;               // 16-byte code chunks per row
    static constexpr int B_CHUNKS = BN * CHUNKS_PER_ROW;
    static constexpr int B_PER_T = (B_CHUNKS + THREADS - 1) / THREADS;
    static constexpr int CODES_PER_CHUNK = 4 * F::kCodesPerWord; // 32 or 64 k values
    static constexpr int STAGE = (BM + BN) * kPitch;             // FP16 per LDS stage
    static constexpr int RED_HALVES = KSPLIT > 1 ? WAVES * WM * WN * 64 * 32 : 0;  // f32x16 partials
    static constexpr int LDS_HALVES = STAGES * STAGE > RED_HALVES ? STAGES * STAGE : RED_HALVES;
    static constexpr int LDS_BYTES = LDS_HALVES * 2;
    static_assert(A_CHUNKS % THREADS == 0, "A tile splits evenly over the workgroup");
    static_assert((WM * WN) % KSPLIT == 0, "k-split waves share the epilogue tiles evenly");
};

// Buffer resource over [base, base + bytes): loads at offsets past the end
// return 0, which zero-fills the rows beyond M or N without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)(bytes < 0 ? 0 : bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n, 0x00020000);
}

// STAGES == 2: double-buffered LDS; the next step's A copies and B dequant are
// interleaved with the MFMA k-slices from slice STORE_FROM on.  STAGES == 1:
// one LDS stage (two workgroups fit per CU), stored between two barriers.
template <int BITS, int BM, int BN, int WAVES_M, int WAVES_N, int KSPLIT, int STAGES,
          int STORE_FROM>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N * KSPLIT) void k_gemm_prefill(
    const uint16_t* __restrict__ X, int64_t ldx, int M, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int K, int N,
    uint16_t* __restrict__ Y, int64_t ldy, float* __restrict__ h, int64_t ldh, int epi,
    int groups_per_part, float* __restrict__ part) {
    using C = Cfg<BITS, BM, BN, WAVES_M, WAVES_N, KSPLIT, STAGES>;
    __shared__ __attribute__((aligned(16))) f16 lds[C::LDS_HALVES];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int ks = wave % KSPLIT;
    const int wn = (wave / KSPLIT) % WAVES_N;
    const int wm = wave / (KSPLIT * WAVES_N);
    const int l32 = lane & 31, hh = lane >> 5;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int groups = K / kBK;
    const int wpr = K / Fmt<BITS>::kCodesPerWord;
    // K split: workgroup z covers groups [g_lo, g_lo + groups_per_part) and,
    // when `part` is set, writes its FP32 partial tile to part[z][M][N].
    const int g_lo = blockIdx.z * groups_per_part;
    const int g_n = groups_per_part;

    // Block-relative buffer resources (offsets stay far below 2^31).
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(X + (int64_t)m0 * ldx, ((int64_t)(M - m0 - 1) * ldx + K) * 2);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(codes + (int64_t)n0 * wpr, (int64_t)(N - n0) * wpr * 4);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(scales + (int64_t)n0 * groups, (int64_t)(N - n0) * groups * 2);
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(zeros + (int64_t)n0 * groups, (int64_t)(N - n0) * groups * 2);

    // ---- global -> registers for step g
    u32x4 a_reg[C::A_PER_T];
    u32x4 b_reg[C::B_PER_T];
    uint16_t s_reg[C::B_PER_T], z_reg[C::B_PER_T];
    auto load = [&](int g) {
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) {
            const int ch = t + C::THREADS * i;
            const int row = ch >> 4, col = ch & 15;
            a_reg[i] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, (uint32_t)((row * ldx + g * kBK + col * 8) * 2), 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i) {
            const int ch = t + C::THREADS * i;
            const int row = ch / C::CHUNKS_PER_ROW, kc = ch % C::CHUNKS_PER_ROW;
            // Chunks past the tile (INT2, BN = 64) use an offset past the end of
            // every resource, so they read 0 (and are not stored).
            const bool in = ch < C::B_CHUNKS;
            const uint32_t ob = in ? (uint32_t)((row * wpr + g * C::WPG + kc * 4) * 4) : 0xFFFFFF00u;
            const uint32_t os = in ? (uint32_t)((row * groups + g) * 2) : 0xFFFFFF00u;
            b_reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, ob, 0, 0);
            s_reg[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0);
            z_reg[i] = __builtin_amdgcn_raw_buffer_load_b16(rz, os, 0, 0);
        }
    };

    // ---- registers -> LDS stage, in four pieces (A chunks i with i % 4 ==
    // piece, and word `piece` of every B chunk, dequantised)
    auto store_piece = [&](int stage, int piece) {
        f16* As = lds + stage * C::STAGE;
        f16* Bs = As + BM * kPitch;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) {
            if (i % 4 != piece) continue;
            const int ch = t + C::THREADS * i;
            const int row = ch >> 4, col = ch & 15;
            *(u32x4*)(As + row * kPitch + col * 8) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i) {
            const int ch = t + C::THREADS * i;
            if (ch >= C::B_CHUNKS) continue;
            const int row = ch / C::CHUNKS_PER_ROW, kc = ch % C::CHUNKS_PER_ROW;
            const GroupConst gc = group_const(s_reg[i], z_reg[i]);
            f16* dst = Bs + row * kPitch + kc * C::CODES_PER_CHUNK;
            const uint32_t wd = piece == 0 ? b_reg[i].x : piece == 1 ? b_reg[i].y
                              : piece == 2 ? b_reg[i].z : b_reg[i].w;
#pragma unroll
            for (int half = 0; half < Fmt<BITS>::kPairsPerWord / 4; ++half) {
                const int p = half * 4;
                const f16x2 p0 = dequant_pair_f16<BITS>(wd, p + 0, gc);
                const f16x2 p1 = dequant_pair_f16<BITS>(wd, p + 1, gc);
                const f16x2 p2 = dequant_pair_f16<BITS>(wd, p + 2, gc);
                const f16x2 p3 = dequant_pair_f16<BITS>(wd, p + 3, gc);
                *(u32x4*)(dst + piece * Fmt<BITS>::kCodesPerWord + half * 8) =
                    u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
            }
        }
    };

    f32x16 acc[C::WM][C::WN];
#pragma unroll
    for (int im = 0; im < C::WM; ++im)
#pragma unroll
        for (int jn = 0; jn < C::WN; ++jn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[im][jn][r] = 0.0f;

    // MFMAs of k-slices j (16 values each) of a stage with j % KSPLIT == ks.
    auto compute_slices = [&](int stage, int j0, int j1) {
        const f16* As = lds + stage * C::STAGE + (wm * C::WTM + l32) * kPitch + 8 * hh;
        const f16* Bs = lds + stage * C::STAGE + BM * kPitch + (wn * C::WTN + l32) * kPitch + 8 * hh;
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            if (j % KSPLIT != ks) continue;
            f16x8 a[C::WM], b[C::WN];
#pragma unroll
            for (int im = 0; im < C::WM; ++im) a[im] = *(const f16x8*)(As + 32 * im * kPitch + 16 * j);
#pragma unroll
            for (int jn = 0; jn < C::WN; ++jn) b[jn] = *(const f16x8*)(Bs + 32 * jn * kPitch + 16 * j);
#pragma unroll
            for (int im = 0; im < C::WM; ++im)
#pragma unroll
                for (int jn = 0; jn < C::WN; ++jn)
                    acc[im][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[im], b[jn], acc[im][jn],
                                                                         0, 0, 0);
        }
    };

    load(g_lo);
#pragma unroll
    for (int p = 0; p < 4; ++p) store_piece(0, p);
    __syncthreads();
    for (int g = 0; g < g_n; ++g) {
        const bool more = g + 1 < g_n;
        if (more) load(g_lo + g + 1);
        if constexpr (STAGES == 2) {
            const int cur = g & 1;
            // four quarters of the step's eight k-slices; the next stage's
            // store pieces follow the quarters from STORE_FROM on
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                compute_slices(cur, 2 * q, 2 * q + 2);
                if (more && q >= STORE_FROM) {
                    constexpr int quarters = 4 - STORE_FROM;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        if (p * quarters / 4 == q - STORE_FROM) store_piece(cur ^ 1, p);
                }
            }
        } else {
            compute_slices(0, 0, 8);
            __syncthreads();
            if (more) {
#pragma unroll
                for (int p = 0; p < 4; ++p) store_piece(0, p);
            }
        }
        __syncthreads();
    }

    auto emit = [&](int im, int jn, const f32x16& v) {
        const int n = n0 + wn * C::WTN + 32 * jn + l32;
        if (n >= N) return;
        if (part != nullptr) {
            float* pz = part + (int64_t)blockIdx.z * M * N;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * C::WTM + 32 * im + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (m < M) pz[(int64_t)m * N + n] = v[r];
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm * C::WTM + 32 * im + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (m < M) {
                const uint16_t y = f32_to_f16_bits(v[r]);
                Y[(int64_t)m * ldy + n] = y;
                if (epi == kResidual) h[(int64_t)m * ldh + n] += (float)as_f16(y);
            }
        }
    };

    if constexpr (KSPLIT == 1) {
#pragma unroll
        for (int im = 0; im < C::WM; ++im)
#pragma unroll
            for (int jn = 0; jn < C::WN; ++jn) emit(im, jn, acc[im][jn]);
    } else {
        // Partial tiles of the KSPLIT waves that share a wave tile, summed in
        // k-part order; wave ks finishes tiles ks, ks + KSPLIT, ...
        f32x16* red = (f32x16*)lds;
        const int tile = wm * WAVES_N + wn;
#pragma unroll
        for (int im = 0; im < C::WM; ++im)
#pragma unroll
            for (int jn = 0; jn < C::WN; ++jn)
                red[(((tile * KSPLIT + ks) * C::WM + im) * C::WN + jn) * 64 + lane] = acc[im][jn];
        __syncthreads();
#pragma unroll
        for (int q = 0; q < C::WM * C::WN / KSPLIT; ++q) {
            const int idx = ks + q * KSPLIT;
            const int im = idx / C::WN, jn = idx % C::WN;
            f32x16 sum = red[(((tile * KSPLIT + 0) * C::WM + im) * C::WN + jn) * 64 + lane];
#pragma unroll
            for (int w = 1; w < KSPLIT; ++w)
                sum += red[(((tile * KSPLIT + w) * C::WM + im) * C::WN + jn) * 64 + lane];
            emit(im, jn, sum);
        }
    }
}

// Sum of the K-split partial tiles part[0..S)[M][N] in split order, rounded to
// FP16, with the optional residual epilogue.  Four elements per thread.
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int S,
                                                       int M, int N, uint16_t* __restrict__ Y,
                                                       int64_t ldy, float* __restrict__ h,
                                                       int64_t ldh, int epi) {
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t total = (int64_t)M * N;
    if (i4 >= total) return;
    const int64_t plane = total;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i4 + e;
        if (i >= total) break;
        float v = part[i];
        for (int z = 1; z < S; ++z) v += part[z * plane + i];
        const int64_t m = i / N, n = i % N;
        const uint16_t y = f32_to_f16_bits(v);
        Y[m * ldy + n] = y;
        if (epi == kResidual) h[m * ldh + n] += (float)as_f16(y);
    }
}

struct Plan {
    int cfg;    // 0: 128x128 single stage, 1: 128x128 eight waves, 2: 64x64
    int split;  // K parts
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Tile choice, from a sweep on MI355X: with at least two 128x128 tiles per CU,
// single-stage 128x128 workgroups (two resident per CU overlap each other's
// barriers); with about one per CU, 128x128 on eight waves splitting each
// step's k-slices in two; with fewer tiles, 64x64 workgroups of four 32x32
// waves, several resident per CU.  When even that leaves CUs idle, K is split
// over up to 8 parts of at least 4 groups (512 values) each.
Plan plan_for(int M, int N, int K) {
    const int groups = K / kBK;
    const int t128 = ceil_div(M, 128) * ceil_div(N, 128);
    const int t64 = ceil_div(M, 64) * ceil_div(N, 64);
    if (t128 >= 512) return {0, 1};
    if (t128 >= 240) return {1, 1};
    auto best_split = [&](int tiles) {
        int sp = 1;
        while (sp < 8 && tiles * sp < 240 && groups % (2 * sp) == 0 && groups / (2 * sp) >= 4) sp *= 2;
        return sp;
    };
    const int s128 = best_split(t128);
    if (t128 * s128 >= 240 && groups / s128 >= 16) return {1, s128};
    if (t64 >= 240) return {2, 1};
    return {2, best_split(t64)};
}

template <int BITS, int BM, int BN, int WAVES_M, int WAVES_N, int KSPLIT, int STAGES,
          int STORE_FROM>
hipError_t launch_cfg(const GemmArgs& a, int split, hipStream_t s) {
    dim3 grid((a.w->N + BN - 1) / BN, (a.M + BM - 1) / BM, split);
    constexpr int threads = 64 * WAVES_M * WAVES_N * KSPLIT;
    float* part = split > 1 ? (float*)a.ws : nullptr;
    k_gemm_prefill<BITS, BM, BN, WAVES_M, WAVES_N, KSPLIT, STAGES, STORE_FROM><<<grid, threads, 0, s>>>(
        a.X, a.ldx, a.M, a.w->codes, a.w->scales, a.w->zeros, a.w->K, a.w->N, a.Y, a.ldy, a.h,
        a.ldh, (int)a.epi, a.w->K / kBK / split, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || split == 1) return e;
    const int64_t total = (int64_t)a.M * a.w->N;
    const unsigned blocks = (unsigned)((total + 4 * 256 - 1) / (4 * 256));
    k_splitk_reduce<<<blocks, 256, 0, s>>>(part, split, a.M, a.w->N, a.Y, a.ldy, a.h, a.ldh,
                                           (int)a.epi);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const GemmArgs& a, hipStream_t s) {
    const Plan p = plan_for(a.M, a.w->N, a.w->K);
    switch (p.cfg) {
        case 0: return launch_cfg<BITS, 128, 128, 2, 2, 1, 1, 0>(a, p.split, s);
        case 1: return launch_cfg<BITS, 128, 128, 2, 2, 2, 2, 2>(a, p.split, s);
        default: return launch_cfg<BITS, 64, 64, 2, 2, 1, 1, 0>(a, p.split, s);
    }
}

}  // namespace

hipError_t launch_prefill(const GemmArgs& a, hipStream_t s) {
    return a.w->bits == 4 ? launch_bits<4>(a, s) : launch_bits<2>(a, s);
}

size_t prefill_ws_bytes(int M, int N, int K) {
    const Plan p = plan_for(M, N, K);
    return p.split > 1 ? (size_t)p.split * M * N * sizeof(float) : 0;
}

}  // namespace qg
