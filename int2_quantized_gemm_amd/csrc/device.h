// device.h -- device-side building blocks shared by every kernel of the library:
// the packed-code extraction and dequantisation of layout v1, FP16 helpers and
// MFMA vector types.  One definition here, so the GEMM kernels and the
// qg_unpack / qg_dequant test exports run exactly the same code.
//
// Layout v1 (see include/qgemm.h): code j of a uint32 word sits at bit
// 16*(j mod 2) + b*floor(j/2).  Codes 2i and 2i+1 therefore sit at bits b*i
// and 16 + b*i, and one AND with (2^b - 1) * 0x00010001 followed by an OR with
// 0x64006400 (FP16 1024.0 in both halves) yields the FP16 pair
// (1024 + q[2i], 1024 + q[2i+1]) exactly: at 1024 the FP16 spacing is 1.0, so
// the low mantissa bits are the code itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;
constexpr uint32_t kBias2 = 0x64006400u;  // FP16 1024.0 in both halves

// Where the scale and zero of (output channel n, 128-k group g) sit in a
// weight's scales and zeros: element n * srow + g * sgrp.  Groups of 128
// have (K / 128, 1); per-row groups (group size K, one scale and zero per
// output channel) have (1, 0).  Kernels walk K in 128-k groups either way.
struct SzIdx {
    int srow, sgrp;
    __host__ __device__ int64_t at(int64_t n, int64_t g) const { return n * srow + g * sgrp; }
};

template <int BITS>
struct Fmt {
    static_assert(BITS == 4 || BITS == 2, "layout v1 has 4- and 2-bit codes");
    static constexpr int kCodesPerWord = 32 / BITS;
    static constexpr int kPairsPerWord = kCodesPerWord / 2;
    static constexpr int kWordsPerGroup = kGroup / kCodesPerWord;   // 16 or 8
    static constexpr uint32_t kPairMask = ((1u << BITS) - 1u) * 0x00010001u;
    static constexpr int kQMax = (1 << BITS) - 1;
};

// 32-bit constants in registers the compiler cannot fold (an SGPR and a
// VGPR), so that a mask and an OR constant meet in one fused VOP3 instruction
// (v_and_or / v_bitop3), which can take neither a literal nor two SGPRs;
// left as literals, each mask-and-or costs a v_and and a v_or.
__device__ __forceinline__ uint32_t sgpr_const(uint32_t v) {
    uint32_t r;
    asm volatile("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
    return r;
}
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
    return r;
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16 as_f16(uint16_t v) { return __builtin_bit_cast(f16, v); }
__device__ __forceinline__ uint16_t as_u16(f16 v) { return __builtin_bit_cast(uint16_t, v); }

// FP16 pair (1024 + q[2i], 1024 + q[2i+1]) of codes 2i, 2i+1 of word w.
template <int BITS>
__device__ __forceinline__ f16x2 biased_pair(uint32_t w, int i) {
    return as_f16x2(((w >> (BITS * i)) & Fmt<BITS>::kPairMask) | kBias2);
}

// Integer codes q[2i], q[2i+1] of word w (used by the unpack export).
template <int BITS>
__device__ __forceinline__ void code_pair(uint32_t w, int i, uint32_t& q0, uint32_t& q1) {
    const uint32_t v = (w >> (BITS * i)) & Fmt<BITS>::kPairMask;
    q0 = v & 0xFFFFu;
    q1 = v >> 16;
}

// Per-group constants of the dequantisation w^ = (q - z) * s, as FP16 pairs:
// nbz = -(1024 + z) (exact: z is an integer <= 15), s2 = (s, s).
struct GroupConst {
    f16x2 nbz;
    f16x2 s2;
};

__device__ __forceinline__ GroupConst group_const(uint16_t s_bits, uint16_t z_bits) {
    const f16 z = as_f16(z_bits);
    const f16 nb = (f16)(-1024.0f) - z;
    GroupConst c;
    c.nbz = f16x2{nb, nb};
    c.s2 = f16x2{as_f16(s_bits), as_f16(s_bits)};
    return c;
}

// (q - z) as an exact FP16 pair.
template <int BITS>
__device__ __forceinline__ f16x2 centered_pair(uint32_t w, int i, f16x2 nbz) {
    return biased_pair<BITS>(w, i) + nbz;
}

// fp16_rne((q - z) * s) as an FP16 pair: exact subtraction, one rounding.
template <int BITS>
__device__ __forceinline__ f16x2 dequant_pair_f16(uint32_t w, int i, const GroupConst& c) {
    return centered_pair<BITS>(w, i, c.nbz) * c.s2;
}

// Exact FP32 dequant of a pair: (q - z) is exact in FP16, the product with an
// FP16 scale is exact in FP32 (at most 4 + 11 significant bits).
template <int BITS>
__device__ __forceinline__ void dequant_pair_f32(uint32_t w, int i, const GroupConst& c, float& a,
                                                 float& b) {
    const f16x2 d = centered_pair<BITS>(w, i, c.nbz);
    const float s = (float)c.s2.x;
    a = (float)d.x * s;
    b = (float)d.y * s;
}

// Nearest FP16 (ties to even) of an FP64 value, as bits; overflow -> +-inf.
// Works on the bit pattern: the result counts quanta of 2^qe, where
// qe = max(E, -14) - 10 for the unbiased exponent E of x, and the FP16 bit
// pattern is ((qe + 24) << 10) + that count for normals and subnormals alike.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    const int e = (int)((b >> 52) & 0x7ff);
    const uint64_t m = b & 0xFFFFFFFFFFFFFull;
    if (e == 0x7ff) return sign | (m ? 0x7e00 : 0x7c00);
    if (e == 0) return sign;  // |x| < 2^-1022
    const uint64_t sig = m | (1ull << 52);
    const int E = e - 1023;
    const int qe = (E < -14 ? -14 : E) - 10;
    const int shift = 52 + qe - E;  // >= 42
    if (shift > 63) return sign;
    uint64_t r = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1ull);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (r & 1ull))) ++r;
    const int64_t bits = ((int64_t)(qe + 24) << 10) + (int64_t)r;
    if (bits >= 0x7c00) return sign | 0x7c00;
    return sign | (uint16_t)bits;
}

__device__ __forceinline__ double f16_bits_to_f64(uint16_t h) { return (double)(float)as_f16(h); }

// Round an FP32 accumulator to FP16 (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) { return as_u16((f16)v); }

// ---- output epilogue shared by every GEMM kernel.  The FP32 accumulator is
// rounded to FP16 (y16), then
//   kStore:    Y[m][n] = y16
//   kResidual: Y[m][n] = y16 and h[m][n] += float(y16)          (h FP32 [.][ldh])
//   kGateMul:  Y[m][n] = fp16(silu(g[m][n]) * y16), silu(z) = z / (1 + e^-z)
//              in FP32 (g FP16 [.][ldg]: the gate projection of a SwiGLU FFN)
enum Epilogue { kStore = 0, kResidual = 1, kGateMul = 2 };

struct OutEpi {
    uint16_t* Y;
    int64_t ldy;
    float* h;
    int64_t ldh;
    const uint16_t* g;
    int64_t ldg;
    int kind;
};

// fp16(silu(g) * u) for FP16 bit patterns g and u, in FP32 (the SwiGLU
// activation; the gate-multiply epilogue and the fused gate-and-up GEMV both
// use it, so their results agree bit for bit).
__device__ __forceinline__ uint16_t swiglu_f16(uint16_t g16, uint16_t u16) {
    const float gv = (float)as_f16(g16);
    return f32_to_f16_bits(gv / (1.0f + expf(-gv)) * (float)as_f16(u16));
}

__device__ __forceinline__ void epi_store(const OutEpi& e, int64_t m, int64_t n, float acc) {
    uint16_t y = f32_to_f16_bits(acc);
    if (e.kind == kGateMul) y = swiglu_f16(e.g[m * e.ldg + n], y);
    e.Y[m * e.ldy + n] = y;
    if (e.kind == kResidual) e.h[m * e.ldh + n] += (float)as_f16(y);
}

// Whether the 8-wide epilogue below may use 16-byte accesses for runs of 8
// outputs n0 .. n0+7 with n0 a multiple of 8: every run lies inside the row
// (N % 8 == 0) and every operand row starts 16-byte aligned.
__device__ __forceinline__ bool epi_vec8_ok(const OutEpi& e, int N) {
    bool ok = N % 8 == 0 && e.ldy % 8 == 0 && ((uintptr_t)e.Y & 15) == 0;
    if (e.kind == kResidual) ok = ok && e.ldh % 4 == 0 && ((uintptr_t)e.h & 15) == 0;
    if (e.kind == kGateMul) ok = ok && e.ldg % 8 == 0 && ((uintptr_t)e.g & 15) == 0;
    return ok;
}

// The epilogue of outputs (m, n0 .. n0+7) with FP32 accumulators v: the same
// arithmetic per element as epi_store, with 16-byte loads and stores when vec
// (epi_vec8_ok); otherwise element by element, skipping columns >= N.
__device__ __forceinline__ void epi_store8(const OutEpi& e, int64_t m, int n0, int N,
                                           const float v[8], bool vec) {
    if (!vec) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (n0 + i < N) epi_store(e, m, n0 + i, v[i]);
        return;
    }
    uint16_t y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = f32_to_f16_bits(v[i]);
    if (e.kind == kGateMul) {
        const u32x4 g = *(const u32x4*)(e.g + m * e.ldg + n0);
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = swiglu_f16((uint16_t)(g[i / 2] >> (16 * (i & 1))), y[i]);
    }
    u32x4 yw;
#pragma unroll
    for (int i = 0; i < 4; ++i) yw[i] = (uint32_t)y[2 * i] | ((uint32_t)y[2 * i + 1] << 16);
    *(u32x4*)(e.Y + m * e.ldy + n0) = yw;
    if (e.kind == kResidual) {
        f32x4* hp = (f32x4*)(e.h + m * e.ldh + n0);
        f32x4 h0 = hp[0], h1 = hp[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h0[i] += (float)as_f16(y[i]);
            h1[i] += (float)as_f16(y[4 + i]);
        }
        hp[0] = h0;
        hp[1] = h1;
    }
}

// The epilogue's input element (h[m][n] as FP32 bits for kResidual, g[m][n]
// for kGateMul, 0 for kStore), for kernels that load it ahead of their
// arithmetic; epi_store_pre then finishes exactly like epi_store.  The load is
// one unconditional aligned dword (a control-flow split would make the
// compiler wait for every load in flight at the join): h[m][n] itself, or the
// dword of g holding g[m][n] (g 4-byte aligned, ldg even), or for kStore any
// valid dword (`any`).
__device__ __forceinline__ uint32_t epi_input(const OutEpi& e, int64_t m, int64_t n,
                                              const uint32_t* any) {
    const bool res = e.kind == kResidual, gm = e.kind == kGateMul;
    const uint32_t* p = res ? (const uint32_t*)(e.h + m * e.ldh + n)
                            : gm ? (const uint32_t*)(e.g + m * e.ldg + (n & ~int64_t(1))) : any;
    const uint32_t v = *p;
    return gm ? (v >> (16 * (int)(n & 1))) & 0xFFFFu : v;
}

__device__ __forceinline__ void epi_store_pre(const OutEpi& e, int64_t m, int64_t n, float acc,
                                              uint32_t in) {
    uint16_t y = f32_to_f16_bits(acc);
    if (e.kind == kGateMul) y = swiglu_f16((uint16_t)in, y);
    e.Y[m * e.ldy + n] = y;
    if (e.kind == kResidual) e.h[m * e.ldh + n] = __builtin_bit_cast(float, in) + (float)as_f16(y);
}

}  // namespace qg

namespace qg {

// ---- cross-lane sums without LDS traffic: DPP within rows of 16 lanes, then
// v_readlane across the four rows of a wave64.  The order of additions is
// fixed, so every lane of a segment gets bit-identical sums.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over each row of 16 lanes (quad_perm xor 1, xor 2, then row rotations
// by 4 and 8), present in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_mov<0x124>(v);  // row_ror:4
    v += dpp_mov<0x128>(v);  // row_ror:8
    return v;
}

// Sum over aligned segments of S lanes (S = 16, 32 or 64), in every lane.
template <int S>
__device__ __forceinline__ float segment_sum(float v) {
    static_assert(S == 16 || S == 32 || S == 64, "segments of 16, 32 or 64 lanes");
    v = row16_sum(v);
    if constexpr (S == 16) {
        return v;
    } else if constexpr (S == 32) {
        const float lo = readlane_f(v, 0) + readlane_f(v, 16);
        const float hi = readlane_f(v, 32) + readlane_f(v, 48);
        return (threadIdx.x & 63) < 32 ? lo : hi;
    } else {
        return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
    }
}

}  // namespace qg

namespace qg {

// ---- LDS DMA: global -> LDS copies that bypass registers (gfx950
// buffer_load ... lds), with explicit completion waits.

// Buffer descriptor as four SGPRs (base, no stride, num_records bytes, raw
// buffer flags as for make_rsrc), for the inline-asm LDS DMA below.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc_sgpr(const void* base, int64_t bytes) {
    const uint64_t b = (uint64_t)base;
    const int32_t n = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)(bytes < 0 ? 0 : bytes);
    return i32x4{__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b),
                 __builtin_amdgcn_readfirstlane((int32_t)((b >> 32) & 0xFFFF)),
                 __builtin_amdgcn_readfirstlane(n), 0x00020000};
}

// One 16-byte-per-lane buffer load written straight to LDS (lane l's bytes
// land at lds + 16 l; the wave's LDS base goes through M0, which an LDS DMA
// may read only one wait state after the SALU write).  Issued as inline
// asm so that the compiler does not wait for it before unrelated LDS reads:
// completion is the caller's business (wait_vmcnt, then a barrier).  Out of
// range offsets read as zero.
__device__ __forceinline__ void dma16(i32x4 rsrc, const void* lds, uint32_t voffset) {
    const int32_t m0 = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are pending
// (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Workgroup barrier for LDS producers/consumers whose vector-memory waits are
// explicit: finishes this wave's LDS accesses, then s_barrier.  The asm
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most c (runtime, 0 <= c) vector-memory operations are
// pending; c >= N is treated as N.
template <int N>
__device__ __forceinline__ void wait_vmcnt_le(int c) {
    if constexpr (N == 0) {
        wait_vmcnt<0>();
    } else {
        if (c >= N)
            wait_vmcnt<N>();
        else
            wait_vmcnt_le<N - 1>(c);
    }
}

}  // namespace qg
