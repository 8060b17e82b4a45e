// internal.h -- host-side interfaces between the C-ABI layer (qgemm.hip) and the
// kernel translation units.  Every launcher assumes its arguments were already
// validated by the C-ABI layer and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qgemm.h"
#include "device.h"

namespace qg {

// Scale addressing of a validated weight (group 128, or K for per-row groups).
inline SzIdx sz_idx(const qg_weight& w) {
    return w.group == kGroup ? SzIdx{w.K / kGroup, 1} : SzIdx{1, 0};
}
inline bool per_row(const qg_weight& w) { return w.group != kGroup; }
// Row stride of a validated weight's codes, in uint32 words.
inline int64_t code_ld(const qg_weight& w) {
    return w.ldc ? w.ldc : (int64_t)w.K * w.bits / 32;
}

// ---- pack / unpack / dequant (kernels_pack.hip)
// Pack and re-quantisation run in two passes.  The validation pass writes
// nothing but, when the input holds a non-finite value or a scale overflows
// FP16, `tag` (the caller's nonzero call tag) into *status; the word is never
// cleared, so the caller compares it with its own tag.  The writing pass is
// launched only after a clean validation pass.
hipError_t launch_pack_check(const float* W, int64_t ldw, int K, int N, int bits, int group,
                             int* status, int tag, hipStream_t s);
hipError_t launch_pack(const float* W, int64_t ldw, int K, int N, int bits, int group,
                       uint32_t* codes, qg_half* scales, qg_half* zeros, hipStream_t s);
hipError_t launch_unpack(const qg_weight& w, uint8_t* q, hipStream_t s);
hipError_t launch_requant_4to2_check(const qg_weight& w4, int* status, int tag, hipStream_t s);
// in_place: w2 aliases w4 (codes, scales, zeros); the INT2 rows keep w2's
// row stride (w4's for the pages' in-place form, compact otherwise).
hipError_t launch_requant_4to2(const qg_weight& w4, const qg_weight& w2, bool in_place,
                               hipStream_t s);
// Largest K the per-row re-quantisation holds in one workgroup's registers.
constexpr int kRequantRowMaxK = 32768;
hipError_t launch_dequant(const qg_weight& w, bool fp16, void* out, hipStream_t s);

// ---- GEMM (kernels_gemm.hip); the epilogue kinds are in device.h.

struct GemmArgs {
    const qg_half* X;
    int64_t ldx;
    const qg_weight* w;
    qg_half* Y;
    int64_t ldy;
    int M;
    Epilogue epi;
    float* h;
    int64_t ldh;
    void* ws;
    size_t ws_bytes;
    // M == 1 GEMV only (where gemm_fuses_layernorm holds): when ln_h is set,
    // the activations are fp16(LN(ln_h)) (ln_h FP32 [K]) and X is ignored;
    // norm_out, if set, receives them.
    const float* ln_h = nullptr;
    qg_half* norm_out = nullptr;
    // kGateMul: the gate projection g [M][ldg] (FP16) the output multiplies.
    const qg_half* gm = nullptr;
    int64_t ldg = 0;
    // SwiGLU pair (M == 1 GEMV only, where gemm_fuses_swiglu holds): w is the
    // gate and w2 the up projection of the same shape and bits; g_out [N]
    // receives fp16(X . w) and Y fp16(silu(g) * fp16(X . w2)); epi must be
    // kStore.
    const qg_weight* w2 = nullptr;
    qg_half* g_out = nullptr;
    // Parts mode (M > 1 only): the GEMM writes its FP32 K-part partials
    // ws[0..S)[M][N] (S >= 1, also when it would not split) and no output;
    // *parts receives S.  The caller finishes with launch_reduce_residual_ln.
    int* parts = nullptr;

    OutEpi out() const { return OutEpi{Y, ldy, h, ldh, gm, ldg, (int)epi}; }
};

// ---- M == 1 GEMV (kernels_gemv.hip)
// True when the GEMV has a lane arrangement for this K (K / 32 lane chunks of
// 32 codes: 16 or 32 lanes per row, or 64 lanes and 1, 2, 4 or 8 chunks).
bool gemv_supported(int bits, int K);
// True when it also has the SwiGLU pair variant (at most 4 chunks per lane).
bool gemv_pairs_supported(int bits, int K);
// The GEMV of a.w (bits 4 or 2; M == 1, gemv_supported), with a.ln_h's fused
// LayerNorm and a.w2's SwiGLU pair when set.
hipError_t launch_gemv(const GemmArgs& a, hipStream_t s);

// True when a GEMM of this shape can take its activations as the fused
// LayerNorm of an FP32 row (the M == 1 GEMV path).
bool gemm_fuses_layernorm(int bits, int M, int K, int N);
// True when the gate and up projections of this shape can run as one SwiGLU
// pair launch (GemmArgs::w2).
bool gemm_fuses_swiglu(int bits, int M, int K, int N);

// Which kernel family and tile a (bits, M, K, N) problem goes to.
enum GemmPath { kPathGemv = 0, kPathSkinny = 1, kPathTiled = 2 };
GemmPath gemm_path(int bits, int M, int K, int N);
size_t gemm_ws_bytes(int bits, int M, int K, int N);
// Workspace a parts-mode launch of this shape needs (its partials).
size_t gemm_parts_ws_bytes(int bits, int M, int K, int N);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// M > 16 (and M <= 16 with K > 8192): the tiled MFMA GEMMs of
// kernels_prefill.hip (ring kernel with 32-, 64- or 128-row tiles, or the
// staged kernel), picked by the tile plan; when the plan splits K, a.ws must
// hold prefill_ws_bytes(M, N, K) bytes of FP32 partials.
hipError_t launch_prefill(const GemmArgs& a, hipStream_t s);
// Deterministic sum of K-split partials part[0..S)[M][N] (FP32, in split
// order) into a.Y with a's epilogue.
hipError_t launch_splitk_reduce(const float* part, int S, const GemmArgs& a, hipStream_t s);
size_t prefill_ws_bytes(int M, int N, int K);

// ---- loop glue (kernels_loop.hip)
// norm[m][:] = fp16(LN(h[m][:])), parameter-free, eps 1e-5, FP32.
hipError_t launch_layernorm(const float* h, int M, int D, qg_half* norm, hipStream_t s);
// A residual projection's end and the following LayerNorm in one launch:
// y = fp16(sum of part[0..S)[M][D] in part order) to Y [M][D], h += y, and
// norm = fp16(LN(h)) unless norm is NULL.  Bit-identical to the split-K
// reduction with the residual epilogue followed by launch_layernorm.  For
// the D that reduce_ln_supported accepts.
bool reduce_ln_supported(int D);
hipError_t launch_reduce_residual_ln(const float* part, int S, int M, int D, qg_half* Y, float* h,
                                     qg_half* norm, hipStream_t s);

}  // namespace qg
