// kernels_prefill.hip -- tiled GEMM (M > 16): Y[M][N] = X[M][K] . dequant(W)[K][N]
// on FP16 MFMA, for batched decode, the chunked-prefill row counts of the
// "Model" page (prefill_chunk = 512 rows) and single-shot prefill.
//
// Two kernels, picked per shape by plan_for (measured tile plan, below):
//   * k_gemm_ring (the usual one): every operand streamed into LDS by LDS DMA
//     through rings of stages, 32-, 64- or 128-row tiles of 128 columns,
//     described with the kernel;
//   * k_gemm_prefill (staged): for operands the ring's DMA cannot take and
//     shapes it does not suit, described next.
// Both can split K into parts whose FP32 partial tiles k_splitk_reduce sums
// in part order.
//
// Staged kernel: one K step is one quantisation group (128 values along K).
// Per step the workgroup
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

#include <utility>

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
    int64_t ldc, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, SzIdx sz,
    int K, int N, OutEpi out, int groups_per_part, float* __restrict__ part) {
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
    const int wpr = (int)ldc;  // code row stride in words (<= 2^20)
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
        make_rsrc(scales + (int64_t)n0 * sz.srow, (int64_t)(N - n0) * sz.srow * 2);
    const __amdgpu_buffer_rsrc_t rz =
        make_rsrc(zeros + (int64_t)n0 * sz.srow, (int64_t)(N - n0) * sz.srow * 2);

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
            const uint32_t os = in ? (uint32_t)(sz.at(row, g) * 2) : 0xFFFFFF00u;
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
            if (m < M) epi_store(out, m, n, v[r]);
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

// ---- Deep-prefetch variant ("ring").  Every operand of a step reaches LDS by
// LDS DMA (buffer_load_dwordx4 ... lds), issued ahead into rings of stages,
// so global latency is hidden without holding data in registers and without
// the compiler's conservative waits on register loads.  The A tile (reused by
// many workgroups, mostly an L2 hit) is issued RA-1 steps ahead; the packed
// codes, scales and zeros (read by few workgroups, mostly from HBM with its
// longer latency) RB-1 steps ahead.  Each step a wave waits for its own DMAs
// of that step (s_waitcnt vmcnt with the exact count of later DMAs left
// outstanding), then one barrier publishes all waves' data and frees the
// stages read in the previous step.
//
// Stage layout, in 16-byte units:
//   A: BM rows x 16 chunks; chunk c of row r at unit 16 r + (c ^ (r % 16)), so
//      the fragment reads of 16 consecutive rows hit distinct banks;
//   B: 128 columns x CH chunks (CH = 4 for INT4, 2 for INT2) of the packed
//      codes of one group; chunk q of column n at unit CH n + (q ^ swz(n)),
//      again so that 16 consecutive columns read distinct banks.
// Scales and zeros (mode SZ) come 8 groups at a time (16 contiguous bytes per
// column) into a double buffer (kSzDma); a K part of at most 8 groups instead
// holds its column's scales and zeros in registers, loaded once before the
// first step (kSzRegs); per-row groups have one scale and zero per column,
// loaded once (kSzRow).
//
// Four strips of 32 columns of the 128-wide tile (TM = BM/32 MFMA tiles of
// 32 x 32 down each), so a strip's B fragments are dequantised once and feed
// TM MFMAs each; that keeps the dequantisation at under 4 VALU instructions
// per MFMA, which a wave's VALU work still overlaps with its own MFMAs
// (measured; a 2 x 2 wave grid, which halves the LDS reads but doubles the
// dequantisation, was slower).  KS = 1: one wave per strip.  KS = 2: two
// waves per strip (8 per workgroup), wave 4 s + k taking k-slices 4 k ..
// 4 k + 3 of every step, so that two waves share each SIMD and one's
// dequantisation and waits overlap the other's MFMAs; at the end the k = 1
// wave hands its partial tiles to the k = 0 wave through LDS, which adds them
// (k = 0 + k = 1) and stores the strip (a different FP32 summation order
// from KS = 1, within the same tolerance of the oracle).  Measured on MI355X:
// 64- and 128-row tiles 2-6 % faster on every
// shape (C5b 80.6 -> 76.5 us, the M = 512 down projection 33.6 -> 31.6 us,
// C3 -1.4 %, M = 256 block -5 %); 32-row tiles at M <= 128 about 1 % slower,
// but they too run KS = 2, so that every tile height sums each output in the
// same order and K split (a GEMM over some of a weight's columns then equals
// those columns of the whole GEMM bit for bit across tile heights, as the
// FP16-h cache's K/V rebuild relies on).  Lane l takes column l % 32 of the strip and
// the k run [64 h, 64 h + 64) of a step (h = l / 32), slice j the j-th 8 of
// that run, and reads A fragments with the same assignment, one slice ahead
// of the MFMAs.
template <int BITS>
struct RingB {
    static constexpr int CH = BITS == 4 ? 4 : 2;  // 16-byte chunks per column and group
    static constexpr int BYTES = 128 * CH * 16;
    __device__ static int swz(int n) { return BITS == 4 ? (n >> 2) & 3 : (n >> 3) & 1; }
};

enum SzMode { kSzDma = 0, kSzRegs = 1, kSzRow = 2 };

// Scale mode of a ring launch over K parts of `per` groups.
int ring_sz_mode(const GemmArgs& a, int per) {
    return per_row(*a.w) ? kSzRow : per % 8 == 0 ? kSzDma : kSzRegs;
}

// The ring kernel needs 16-byte aligned DMA sources, and (groups of 128) K
// parts of whole runs of 8 groups of scales (DMA) or of at most 8 groups
// (registers).
bool ring_ok(const GemmArgs& a, int split) {
    const int groups = a.w->K / kBK;
    const int per = groups / split;
    if (groups % split != 0 || (a.ldx % 8) != 0 || ((uintptr_t)a.X % 16) != 0 ||
        ((uintptr_t)a.w->codes % 16) != 0)
        return false;
    switch (ring_sz_mode(a, per)) {
        case kSzRow: return true;
        case kSzRegs: return per <= 8;
        default: return ((uintptr_t)a.w->scales % 16) == 0 && ((uintptr_t)a.w->zeros % 16) == 0;
    }
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// XCD-aware order of output tiles.  Workgroup i of a launch runs on XCD
// i mod 8, and each XCD has its own L2, so the tiles of one XCD should share
// operands: the gx x gy tile grid is cut into rx x ry sub-grids of sx x sy
// tiles (rx ry = 8), sub-grid c for XCD c.  Each A row-block is then fetched
// into rx L2s and each B column-block into ry, instead of up to 8 each; the
// host picks (rx, ry) for the least total.  The launch has 8 sx sy
// workgroups; those past the grid's edge exit at once.
struct Raster {
    int gx, gy, rx, sx, sy;
    __device__ bool tile(int i, int& tx, int& ty) const {
        const int xcd = i & 7, slot = i >> 3;
        tx = (xcd % rx) * sx + slot % sx;
        ty = (xcd / rx) * sy + slot / sx;
        return tx < gx && ty < gy;
    }
};

// Choose the raster for a gx x gy grid whose A row-blocks are a_bytes each
// and B column-blocks b_bytes each.
Raster make_raster(int gx, int gy, double a_bytes, double b_bytes) {
    Raster best{gx, gy, 8, 1, 1};
    double best_cost = -1.0;
    for (int rx = 1; rx <= 8; rx *= 2) {
        const int ry = 8 / rx;
        const int sx = (gx + rx - 1) / rx, sy = (gy + ry - 1) / ry;
        const double idle = 8.0 * sx * sy - (double)gx * gy;
        // fetches: each of gy row-blocks into min(rx, gx) L2s, each of gx
        // column-blocks into min(ry, gy); idle slots cost a wave of tiles
        const double cost = gy * a_bytes * (rx < gx ? rx : gx) + gx * b_bytes * (ry < gy ? ry : gy) +
                            idle * (a_bytes + b_bytes);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = Raster{gx, gy, rx, sx, sy};
        }
    }
    return best;
}

// f(integral_constant<int, i>) for i = 0 .. n-1, in order (compile-time i).
template <class Fn, int... Is>
__device__ __forceinline__ void for_each_index(Fn&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}

template <int BITS, int BM, int RA, int RBS, int SZ, int KS>
__global__ __launch_bounds__(256 * KS) void k_gemm_ring(
    const uint16_t* __restrict__ X, int64_t ldx, int M, const uint32_t* __restrict__ codes,
    int64_t ldc, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int K,
    int N, OutEpi out, int groups_per_part, float* __restrict__ part, Raster rs) {
    using F = Fmt<BITS>;
    using RB = RingB<BITS>;
    constexpr int TM = BM / 32;
    constexpr int NWV = 4 * KS;                  // waves
    constexpr int A_BYTES = BM * kBK * 2;
    constexpr int A_INSTR = A_BYTES / 1024;      // A DMA instructions per step
    constexpr int B_INSTR = RB::BYTES / 1024;    // B DMA instructions per step
    // per issuing wave and step; the first A_INSTR / A_DMA (B_INSTR / B_DMA)
    // waves issue them
    constexpr int A_DMA = A_INSTR >= NWV ? A_INSTR / NWV : 1;
    constexpr int B_DMA = B_INSTR >= NWV ? B_INSTR / NWV : 1;
    static_assert(KS == 1 || KS == 2, "k slices of a step split over 1 or 2 waves per strip");
    static_assert(A_INSTR % NWV == 0 || NWV % A_INSTR == 0, "A DMA over whole waves");
    static_assert(B_INSTR % NWV == 0 || NWV % B_INSTR == 0, "B DMA over whole waves");
    constexpr int JB = 8 / KS;                   // k-slices of a step per wave
    constexpr int CH = RB::CH;
    constexpr int LANE_WORDS = 64 / F::kCodesPerWord;  // packed words of a lane's k run
    constexpr int U = RA * RBS / gcd_c(RA, RBS);       // steps per unrolled round
    static_assert(RA >= 2 && RBS > RA && RBS <= 9, "stage counts");
    static_assert(A_DMA >= 1 && B_DMA >= 1, "whole DMA instructions per wave");
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[RA][A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b[RBS][RB::BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_sz[2][2][128 * 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int strip = wave & 3;  // 32-column strip of the tile
    const int ks = wave >> 2;    // which k-slices of a step (KS = 2: slices 4 ks .. 4 ks + 3)
    const bool a_issuer = wave < A_INSTR / A_DMA;
    const bool b_issuer = wave < B_INSTR / B_DMA;
    const int a_n = a_issuer ? A_DMA : 0, b_n = b_issuer ? B_DMA : 0;  // this wave's DMAs per step
    const int l32 = lane & 31, hh = lane >> 5;
    int tx, ty;
    if (!rs.tile(blockIdx.x, tx, ty)) return;  // padding workgroup of the raster
    const int m0 = ty * BM;
    const int n0 = tx * 128;
    const int groups = K / kBK;
    const int wpr = (int)ldc;  // code row stride in words (<= 2^20)
    const int g_lo = blockIdx.z * groups_per_part;
    const int G = groups_per_part;

    const i32x4 ra =
        make_rsrc_sgpr(X + (int64_t)m0 * ldx, ((int64_t)(M - m0 - 1) * ldx + K) * 2);
    const i32x4 rb = make_rsrc_sgpr(codes + (int64_t)n0 * wpr, (int64_t)(N - n0) * wpr * 4);
    // Waves 0, 1 load scales and waves 2, 3 zeros, of columns 64 (w % 2) + lane.
    const i32x4 rsz = make_rsrc_sgpr((strip < 2 ? scales : zeros) + (int64_t)n0 * groups,
                                     (int64_t)(N - n0) * groups * 2);

    // Source offsets of this lane's DMA slots at step 0 of the part.
    uint32_t a_off[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int unit = (wave * A_DMA + i) * 64 + lane;
        const int row = unit >> 4;
        const int c = (unit & 15) ^ (row & 15);
        a_off[i] = (uint32_t)((row * ldx + (int64_t)g_lo * kBK + c * 8) * 2);
    }
    uint32_t b_off[B_DMA];
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const int unit = (wave * B_DMA + i) * 64 + lane;
        const int n = unit / CH;
        const int q = (unit % CH) ^ RB::swz(n);
        b_off[i] = (uint32_t)(n * wpr * 4 + g_lo * F::kWordsPerGroup * 4 + q * 16);
    }
    const uint32_t sz_off = (uint32_t)((((strip & 1) * 64 + lane) * groups + g_lo) * 2);
    // kSzRegs: this lane's column's scales and zeros of the part (G <= 8
    // groups); kSzRow: its column's one scale and zero (groups of K).
    uint16_t sreg[8], zreg[8];
    if constexpr (SZ == kSzRegs) {
        const int n = n0 + strip * 32 + l32;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool ok = i < G && n < N;
            sreg[i] = ok ? scales[(int64_t)n * groups + g_lo + i] : (uint16_t)0;
            zreg[i] = ok ? zeros[(int64_t)n * groups + g_lo + i] : (uint16_t)0;
        }
    }
    GroupConst gc_row{};
    if constexpr (SZ == kSzRow) {
        const int n = n0 + strip * 32 + l32;
        gc_row = group_const(n < N ? scales[n] : (uint16_t)0, n < N ? zeros[n] : (uint16_t)0);
    }

    // Iteration t issues A of step t + RA - 1, then B (and, every 8 steps,
    // the scales and zeros of the next 8) of step t + RB - 1.
    // (With 8 waves the A and B instructions are spread over the waves that
    // issue them, and the 4 waves of k-half 0 load the scales and zeros.)
    auto issue = [&](int t) {
        const int sa = t + RA - 1;
        if (a_issuer && sa >= 0 && sa < G) {
            uint8_t* dst = lds_a[sa % RA] + wave * A_DMA * 1024;
#pragma unroll
            for (int i = 0; i < A_DMA; ++i) dma16(ra, dst + i * 1024, a_off[i] + sa * kBK * 2);
        }
        const int sb = t + RBS - 1;
        if (sb >= 0 && sb < G) {
            if (b_issuer) {
                uint8_t* dst = lds_b[sb % RBS] + wave * B_DMA * 1024;
#pragma unroll
                for (int i = 0; i < B_DMA; ++i)
                    dma16(rb, dst + i * 1024, b_off[i] + sb * F::kWordsPerGroup * 4);
            }
            if (SZ == kSzDma && ks == 0 && (sb & 7) == 0)
                dma16(rsz, &lds_sz[(sb >> 3) & 1][strip >> 1][(strip & 1) * 1024],
                      sz_off + sb * 2);
        }
    };

    f32x16 acc[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tm][r] = 0.0f;

    // Per-lane LDS byte offsets within a stage: the A fragment of slice j for
    // tile row 0 (tile row tm adds 32 rows, 8 KiB), the B codes of this
    // lane's k run, its column's scale and zero.
    const int col = strip * 32 + l32;  // output channel within the block
    const int j0 = ks * JB;             // first k-slice of this wave
    uint32_t a_lds[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj)
        a_lds[jj] = (uint32_t)((l32 * 16 + ((8 * hh + j0 + jj) ^ (l32 & 15))) * 16);
    uint32_t b_lds[LANE_WORDS / 4];
#pragma unroll
    for (int v = 0; v < LANE_WORDS / 4; ++v)
        b_lds[v] = (uint32_t)((col * CH + ((hh * (LANE_WORDS / 4) + v) ^ RB::swz(col))) * 16);
    const uint32_t sz_lds = (uint32_t)(col * 16);
    const uint32_t pair_mask = sgpr_const(F::kPairMask);
    const uint32_t bias = vgpr_const(kBias2);

    auto compute = [&](int step, auto sa_c, auto sb_c) {
        constexpr int SA = decltype(sa_c)::value;
        constexpr int SB = decltype(sb_c)::value;
        const uint8_t* As = lds_a[SA];
        const uint8_t* Bs = lds_b[SB];
        GroupConst gc;
        if constexpr (SZ == kSzRegs) {
            gc = group_const(sreg[step & 7], zreg[step & 7]);
        } else if constexpr (SZ == kSzRow) {
            gc = gc_row;
        } else {
            const uint8_t* Sz = &lds_sz[(step >> 3) & 1][0][(step & 7) * 2];
            gc = group_const(*(const uint16_t*)(Sz + sz_lds),
                             *(const uint16_t*)(Sz + 128 * 16 + sz_lds));
        }
        // the packed words of this wave's slices (all of the lane's k run
        // with one wave per strip; its half with two)
        constexpr int WW = JB * 8 / F::kCodesPerWord;
        uint32_t wd[WW];
        if constexpr (KS == 1) {
#pragma unroll
            for (int v = 0; v < LANE_WORDS / 4; ++v) {
                const u32x4 t = *(const u32x4*)(Bs + b_lds[v]);
                wd[4 * v + 0] = t[0];
                wd[4 * v + 1] = t[1];
                wd[4 * v + 2] = t[2];
                wd[4 * v + 3] = t[3];
            }
        } else if constexpr (LANE_WORDS == 8) {  // INT4: words 4 ks .. 4 ks + 3
            const u32x4 t = *(const u32x4*)(Bs + (ks ? b_lds[1] : b_lds[0]));
            wd[0] = t[0];
            wd[1] = t[1];
            wd[2] = t[2];
            wd[3] = t[3];
        } else {  // INT2: words 2 ks, 2 ks + 1
            const u32x4 t = *(const u32x4*)(Bs + b_lds[0]);
            wd[0] = ks ? t[2] : t[0];
            wd[1] = ks ? t[3] : t[1];
        }
        f16x8 a_cur[TM], a_nxt[TM];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) a_cur[tm] = *(const f16x8*)(As + a_lds[0] + tm * 8192);
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            // the next slice's A reads are issued before this slice's MFMAs
            // (the scheduler would otherwise sink each read next to its use)
            if (j < JB - 1) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    a_nxt[tm] = *(const f16x8*)(As + a_lds[j + 1] + tm * 8192);
            }
            __builtin_amdgcn_sched_barrier(0);
            // dequantise this slice's 8 codes: (1024 + q) pairs by one fused
            // mask-and-or, then (q - z) exactly and one rounding of (q - z) s
            const uint32_t w = wd[(8 * j) / F::kCodesPerWord];
            const int p0 = ((8 * j) % F::kCodesPerWord) / 2;
            f16x2 d[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t biased = ((w >> (BITS * (p0 + p))) & pair_mask) | bias;
                d[p] = (as_f16x2(biased) + gc.nbz) * gc.s2;
            }
            const f16x8 b = f16x8{d[0].x, d[0].y, d[1].x, d[1].y, d[2].x, d[2].y, d[3].x, d[3].y};
            // The slice's MFMAs at raised wave priority: where two waves share
            // a SIMD (64- and 32-row tiles, two workgroups per CU) the issuer
            // of MFMAs goes first and the other's dequantisation and LDS
            // reads fill in behind (measured 2.5-10 % faster on the block's
            // prefill shapes, bit-identical).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                acc[tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_cur[tm], b, acc[tm], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
            if (j < JB - 1) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) a_cur[tm] = a_nxt[tm];
            }
        }
    };

    // DMA instructions this wave issued after its A DMAs of step g, by the end
    // of iteration g - 1 (scale/zero DMAs not counted: waiting for fewer
    // outstanding than exist is only stricter).
    constexpr int C_STEADY = (RA - 2) * A_DMA + (RA - 1) * B_DMA;
    static_assert(C_STEADY <= 63, "vmcnt field");
    auto later_ops = [&](int g) {
        const int na = min(g - 1, G - RA) - (g - RA + 2) + 1;
        const int nb = min(g - 1, G - RBS) - (g - RA + 1) + 1;
        return (na > 0 ? na : 0) * a_n + (nb > 0 ? nb : 0) * b_n;
    };

    for (int t = -(RBS - 1); t < 0; ++t) issue(t);
    // (kSzRegs: a fixed, fully unrolled trip count, so that the register
    // arrays are indexed by constants)
    constexpr bool REGS = SZ == kSzRegs;
    constexpr int G_UNROLL = REGS ? (8 + U - 1) / U * U : 0;
#pragma unroll
    for (int g0 = 0; g0 < (REGS ? G_UNROLL : G); g0 += U) {
        // steps g0 .. g0 + U - 1 with compile-time stage indices (g0 % U == 0)
        for_each_index([&](auto u_c) {
            constexpr int u = decltype(u_c)::value;
            const int g = g0 + u;
            if (g < G) {
                wait_vmcnt_le<C_STEADY>(later_ops(g));
                lds_barrier();
                issue(g);
                compute(g, std::integral_constant<int, u % RA>{},
                        std::integral_constant<int, u % RBS>{});
            }
        }, std::make_integer_sequence<int, U>{});
    }

    // Epilogue.  The accumulator layout gives each lane one column and 16
    // rows; transposed through LDS, each lane holds runs of 8 consecutive
    // columns of one row instead, so the outputs (and the residual or gate
    // operands) move in 16-byte accesses rather than 2- and 4-byte ones.
    // Each wave stages its 32 x 32 FP32 tile in its own 4 KiB of the (then
    // idle) A ring: element (row, c) at row * 32 + (c ^ 4 (row mod 8)), so
    // the column-wise writes and the row-wise 16-byte reads spread over the
    // banks.
    static_assert(RA * A_BYTES >= 4 * TM * 4096, "epilogue staging fits the A ring");
    lds_barrier();  // every wave is done reading the ring stages
    if constexpr (KS > 1) {
        // the k = 1 wave of each strip hands its partial tiles to the k = 0
        // wave through the A ring, which adds them (k0 + k1) and stores the
        // strip (written for KS waves per strip, added in k order)
        float* pr = (float*)&lds_a[0][0] + strip * (TM * 1024);
#pragma unroll
        for (int kk = 1; kk < KS; ++kk) {
            if (ks == kk) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int r = 0; r < 16; ++r) pr[(tm * 16 + r) * 64 + lane] = acc[tm][r];
            }
            lds_barrier();
            if (ks == 0) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[tm][r] += pr[(tm * 16 + r) * 64 + lane];
            }
            lds_barrier();  // read before the next hand-over (or the staging) reuses the ring
        }
        if (ks != 0) return;
    }
    float* st = (float*)&lds_a[0][0] + strip * 1024;
    const bool vec = part != nullptr ? N % 8 == 0 : epi_vec8_ok(out, N);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hh + (r & 3);
            st[row * 32 + (l32 ^ ((row & 7) << 2))] = acc[tm][r];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = lane + 64 * k;  // run q: row q / 4, columns 8 (q mod 4) + 0..7
            const int row = q >> 2, c8 = (q & 3) * 8;
            const int sw = (row & 7) << 2;
            const f32x4 a = *(const f32x4*)(st + row * 32 + (c8 ^ sw));
            const f32x4 b = *(const f32x4*)(st + row * 32 + ((c8 + 4) ^ sw));
            const int m = m0 + 32 * tm + row;
            const int nn = n0 + strip * 32 + c8;
            if (m >= M || nn >= N) continue;
            const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            if (part != nullptr) {
                float* pp = part + (int64_t)blockIdx.z * M * N + (int64_t)m * N + nn;
                if (vec) {
                    ((f32x4*)pp)[0] = a;
                    ((f32x4*)pp)[1] = b;
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (nn + i < N) pp[i] = v[i];
                }
            } else {
                epi_store8(out, m, nn, N, v, vec);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

// Sum of the K-split partial tiles part[0..S)[M][N] in split order
// (((p0 + p1) + p2) + ...), then the output epilogue.  Four consecutive
// elements per thread.  With N % 4 == 0 they share a row: one 16-byte load
// per part, the loads of up to 8 parts issued before the first add, and one
// row/column split per thread (these launches are latency-bound, so the
// per-element scalar loads and 64-bit divisions of the general path cost
// several microseconds at the loop block's shapes).
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int S,
                                                       int M, int N, OutEpi out) {
    const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t total = (int64_t)M * N;
    if (i4 >= total) return;
    const int64_t plane = total;
    if ((N & 3) == 0) {
        const int m = total <= 0x7FFFFFFF ? (int)((uint32_t)i4 / (uint32_t)N) : (int)(i4 / N);
        const int n = (int)(i4 - (int64_t)m * N);
        const f32x4* p = (const f32x4*)(part + i4);
        const int64_t pl4 = plane / 4;
        f32x4 acc = p[0];
        for (int z0 = 1; z0 < S; z0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (z0 + j < S) v[j] = p[(z0 + j) * pl4];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (z0 + j < S) acc += v[j];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) epi_store(out, m, n + e, acc[e]);
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t i = i4 + e;
        if (i >= total) break;
        float v = part[i];
        for (int z = 1; z < S; ++z) v += part[z * plane + i];
        epi_store(out, i / N, i % N, v);
    }
}

struct Plan {
    int cfg;    // 0: 128x128 single stage, 1: 128x128 eight waves, 2: 64x64, 3: ring 128x128,
                // 4: ring 32x128, 5: ring 64x128
    int split;  // K parts
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Up to this M the ring kernel always runs 32-row tiles.
constexpr int kSmallM = 128;

// Ring kernel with 32-row tiles: K split into the most parts (at most 8) that
// keep at most 256 workgroups and at least 8 groups per part (also in parts
// mode: parts of 4 groups there were 1-2 % slower per loop iteration at
// M = 64..128); {-1, 0} where the parts would not suit the ring.
Plan plan_ring32(int M, int N, int groups) {
    const int t32 = ceil_div(M, 32) * ceil_div(N, 128);
    int sp = 1;
    while (2 * sp <= 8 && t32 * 2 * sp <= 256 && groups % (2 * sp) == 0 && groups / (2 * sp) >= 8)
        sp *= 2;
    const int per = groups / sp;
    if (groups % sp == 0 && (per % 8 == 0 || per <= 8)) return {4, sp};
    return {-1, 0};
}

// Ring kernel with 64-row tiles: no split from 144 tiles on; below that, for
// K of at least 32 groups, K split (parts of >= 8 groups) towards 192
// workgroups; {-1, 0} otherwise.
Plan plan_ring64(int M, int N, int groups) {
    const int t64 = ceil_div(M, 64) * ceil_div(N, 128);
    const bool whole = groups % 8 == 0 || groups <= 8;
    if (t64 >= 144) return whole ? Plan{5, 1} : Plan{-1, 0};
    if (groups < 32 || groups % 8 != 0) return {-1, 0};
    int sp = 1;
    while (sp < 8 && t64 * sp < 192 && groups % (2 * sp) == 0 && groups / (2 * sp) >= 8) sp *= 2;
    return (groups / sp) % 8 == 0 ? Plan{5, sp} : Plan{-1, 0};
}


// Tile choice, from graph-timed sweeps on MI355X over the block's four
// shapes, INT4 and INT2, M = 17..2048.  The ring kernels (operands prefetched
// by LDS DMA) need aligned operands (ring = false otherwise):
//   * M <= kSmallM (batched decode): 32-row ring tiles (plan_ring32).  More,
//     smaller tiles beat fewer larger ones although each 32-row tile
//     dequantises its B tile again: these launches are bound by per-step
//     latency and by how many CUs have work, not by the dequantisation;
//   * K of >= 64 groups with >= 256 128-row tiles: 128-row ring tiles (the
//     long prefill projection, where the 128-row tile's A reuse pays);
//   * otherwise 64-row ring tiles (plan_ring64): two workgroups fit per CU,
//     so one wave's dequantisation overlaps another's MFMAs on the same SIMD
//     (5-17 % faster than 128-row tiles at M = 192..2048; a 2 x 2 wave grid
//     that halves the A reads but doubles the dequantisation was slower);
//   * where they would have too few tiles, 32-row ring tiles again.
// The staged kernels remain for operands the ring cannot take: past 512
// 128-row tiles single-stage 128x128 workgroups (two resident per CU overlap
// each other's barriers); with about one tile per CU, 128x128 on eight waves
// splitting each step's k-slices in two; with fewer tiles, 64x64 workgroups of
// four 32x32 waves, several resident per CU, K split over up to 8 parts of at
// least 4 groups.
Plan plan_for(int M, int N, int K, bool ring) {
    const int groups = K / kBK;
    const int t128 = ceil_div(M, 128) * ceil_div(N, 128);
    const int t64 = ceil_div(M, 64) * ceil_div(N, 64);
    if (ring) {
        if (M <= kSmallM) {
            const Plan p = plan_ring32(M, N, groups);
            if (p.cfg >= 0) return p;
        }
        if (groups % 8 == 0 && groups >= 64 && t128 >= 256) return {3, 1};
        Plan p = plan_ring64(M, N, groups);
        if (p.cfg >= 0) return p;
        p = plan_ring32(M, N, groups);
        if (p.cfg >= 0) return p;
    }
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

hipError_t reduce_parts(const GemmArgs& a, int split, const float* part, hipStream_t s) {
    return launch_splitk_reduce(part, split, a, s);
}

template <int BITS, int BM, int BN, int WAVES_M, int WAVES_N, int KSPLIT, int STAGES,
          int STORE_FROM>
hipError_t launch_cfg(const GemmArgs& a, int split, hipStream_t s) {
    dim3 grid((a.w->N + BN - 1) / BN, (a.M + BM - 1) / BM, split);
    constexpr int threads = 64 * WAVES_M * WAVES_N * KSPLIT;
    float* part = split > 1 || a.parts ? (float*)a.ws : nullptr;
    k_gemm_prefill<BITS, BM, BN, WAVES_M, WAVES_N, KSPLIT, STAGES, STORE_FROM><<<grid, threads, 0, s>>>(
        a.X, a.ldx, a.M, a.w->codes, code_ld(*a.w), a.w->scales, a.w->zeros, sz_idx(*a.w),
        a.w->K, a.w->N, a.out(), a.w->K / kBK / split, part);
    hipError_t e = hipGetLastError();
    if (a.parts) *a.parts = split;
    if (e != hipSuccess || split == 1 || a.parts) return e;
    return reduce_parts(a, split, part, s);
}

template <int BITS, int BM, int RA, int RBS, int SZ, int KS = 1>
hipError_t launch_ring(const GemmArgs& a, int split, hipStream_t s) {
    const int gx = (a.w->N + 127) / 128, gy = (a.M + BM - 1) / BM;
    const double a_bytes = (double)BM * a.w->K * 2 / split;
    const double b_bytes = 128.0 * a.w->K * BITS / 8 / split;
    const Raster rs = make_raster(gx, gy, a_bytes, b_bytes);
    dim3 grid(8 * rs.sx * rs.sy, 1, split);
    float* part = split > 1 || a.parts ? (float*)a.ws : nullptr;
    k_gemm_ring<BITS, BM, RA, RBS, SZ, KS><<<grid, 256 * KS, 0, s>>>(
        a.X, a.ldx, a.M, a.w->codes, code_ld(*a.w), a.w->scales, a.w->zeros, a.w->K, a.w->N,
        a.out(), a.w->K / kBK / split, part, rs);
    hipError_t e = hipGetLastError();
    if (a.parts) *a.parts = split;
    if (e != hipSuccess || split == 1 || a.parts) return e;
    return reduce_parts(a, split, part, s);
}

template <int BITS, int BM, int KS>
hipError_t launch_ring_sz(const GemmArgs& a, int split, hipStream_t s) {
    const int sz = ring_sz_mode(a, a.w->K / kBK / split);
    return sz == kSzRow    ? launch_ring<BITS, BM, 2, 4, kSzRow, KS>(a, split, s)
           : sz == kSzRegs ? launch_ring<BITS, BM, 2, 4, kSzRegs, KS>(a, split, s)
                           : launch_ring<BITS, BM, 2, 4, kSzDma, KS>(a, split, s);
}

template <int BITS>
hipError_t launch_bits(const GemmArgs& a, hipStream_t s) {
    Plan p = plan_for(a.M, a.w->N, a.w->K, true);
    if (p.cfg >= 3 && !ring_ok(a, p.split)) p = plan_for(a.M, a.w->N, a.w->K, false);
    switch (p.cfg) {
        case 0: return launch_cfg<BITS, 128, 128, 2, 2, 1, 1, 0>(a, p.split, s);
        case 1: return launch_cfg<BITS, 128, 128, 2, 2, 2, 2, 2>(a, p.split, s);
        case 2: return launch_cfg<BITS, 64, 64, 2, 2, 1, 1, 0>(a, p.split, s);
        default: break;
    }
    // every tile height on eight waves (two per strip, each half of a
    // step's k-slices): see k_gemm_ring
    if (p.cfg == 3) return launch_ring_sz<BITS, 128, 2>(a, p.split, s);
    if (p.cfg == 5) return launch_ring_sz<BITS, 64, 2>(a, p.split, s);
    return launch_ring_sz<BITS, 32, 2>(a, p.split, s);
}

}  // namespace

// Second kernel of a K-split launch: the in-order reduction of the partials
// part[0..S)[M][N] into Y (and h for the residual epilogue).
hipError_t launch_splitk_reduce(const float* part, int S, const GemmArgs& a, hipStream_t s) {
    const int64_t total = (int64_t)a.M * a.w->N;
    const unsigned blocks = (unsigned)((total + 4 * 256 - 1) / (4 * 256));
    k_splitk_reduce<<<blocks, 256, 0, s>>>(part, S, a.M, a.w->N, a.out());
    return hipGetLastError();
}

hipError_t launch_prefill(const GemmArgs& a, hipStream_t s) {
    return a.w->bits == 4 ? launch_bits<4>(a, s) : launch_bits<2>(a, s);
}

// Workspace for the K-split partials: enough for either plan, since whether
// the ring kernel's alignment holds is known only at launch.
size_t prefill_ws_bytes(int M, int N, int K) {
    const Plan p = plan_for(M, N, K, true), q = plan_for(M, N, K, false);
    const int split = p.split > q.split ? p.split : q.split;
    return split > 1 ? (size_t)split * M * N * sizeof(float) : 0;
}

}  // namespace qg
