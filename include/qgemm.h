/*
 * qgemm.h -- C ABI of the MI355X (gfx950) weight-only INT4/INT2 quantised GEMM
 * library (libqgemm.so) and of the looped, weight-shared block that calls it.
 *
 * The operation is the quantised linear layer of the TinyLoop runtime
 * (quant_gemm for INT4 weights, int2_gemm after the CTX-TIER switch to INT2;
 * "β-Informed Deployment Features" page, CTX-TIER section): FP16 activations
 * times INT4- or INT2-packed weights that carry one FP16 scale and one FP16
 * zero per group of 128 weights along K ("Model" page, VRAM cost; CTX-TIER
 * "Details of the shipped kernel"), or per row: one group spanning all of K
 * (CTX-TIER Phase 2b meets such per-row weights, group size = K).
 *
 * Packed format, layout version 1 (b = bits in {4, 2}, G = group = 128 or K,
 * g = k / G):
 *   - codes:  uint32 rows, row n = output channel n, contiguous along K
 *             (INT4 rows hold K/2 bytes, INT2 rows K/4 bytes), row n starting
 *             at word n * ldc (ldc = K*b/32 for compact rows; a larger ldc
 *             leaves the words past K*b/32 of each row unused, e.g. INT2 rows
 *             kept at the INT4 row stride after an in-place re-quantisation,
 *             CTX-TIER "Details of the shipped kernel").  Inside a word,
 *             code j (j = k mod 32/b) sits at bit 16*(j mod 2) + b*floor(j/2):
 *             even codes in the low half-word, odd codes in the high half-word.
 *   - scales: FP16 [N][K/G];  zeros: FP16 [N][K/G], integer values in
 *             [0, 2^b - 1].
 *   - dequant: w^[k][n] = (q[n][k] - zeros[n][g]) * scales[n][g].
 *   - pack of FP32 W [K][N], per (n, g): lo = min(0, min W), hi = max(0, max W),
 *     s = fp16_rne((hi - lo) / (2^b - 1)) (quotient in FP64; s := 1 if it
 *     rounds to 0), z = clamp(rne(-lo / s), 0, 2^b - 1),
 *     q = clamp(rne(W / s) + z, 0, 2^b - 1); rne = round half to even.
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     never frees or retains them beyond the call (cached launch plans keep
 *     only their values, see qg_release_cache).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     in stream order and the call returns without synchronising unless the
 *     entry says otherwise.  Kernel faults surface at the caller's next sync.
 *   - Every argument is validated before any output is written; on a non-zero
 *     return no output was touched (and, apart from the validation pass of
 *     qg_pack / qg_requant_4to2, which writes nothing, nothing was
 *     enqueued).  qg_last_error() (thread-local) then names the failed check.
 *   - Calls on the same outputs/scratch from two streams race; calls on
 *     distinct buffers may run concurrently.
 *   - Results are deterministic: the same call on the same inputs gives the
 *     same bits (no floating-point atomics).
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 3
#define QG_LAYOUT_VERSION 1

/* Status codes.  EINVAL: bad argument (the pages' ValueError); EUNSUPPORTED:
 * bits/group outside layout v1; ENOMEM / EHIP: runtime failure (the pages'
 * RuntimeError, "Model" page, Raises). */
#define QG_OK 0
#define QG_EINVAL (-1)
#define QG_EUNSUPPORTED (-2)
#define QG_ENOMEM (-3)
#define QG_EHIP (-4)

typedef uint16_t qg_half; /* IEEE binary16 bit pattern */

/* One packed weight (the pages' QuantWeight: packed data, FP16 scales and
 * zeros, bits; CTX-TIER Phase 2).  bits in {4, 2}; group == 128 or group == K
 * (per-row: scales and zeros are [N][1]); K % 128 == 0 and K <= 2^22; N >= 1;
 * codes 16-byte aligned; scales/zeros 2-byte aligned.  ldc: uint32 words
 * from one code row to the next; 0 means compact rows (K*bits/32), otherwise
 * at least K*bits/32, a multiple of 4 (16-byte rows) and at most 2^20. */
typedef struct qg_weight {
    int32_t bits;
    int32_t K;
    int32_t N;
    int32_t group;
    const uint32_t* codes;
    const qg_half* scales;
    const qg_half* zeros;
    int64_t ldc;
} qg_weight;

/* The looped block's weights: qkv K=D, N=3D; out K=D, N=D; up K=D, N=F;
 * down K=F, N=D.  gate.codes == NULL (all of gate zero): four
 * projections and the identity FFN activation.  Otherwise gate is the fifth
 * weight of the pages' block (mlp_gate; "β-Informed Deployment Features"
 * page, CTX-TIER Phase 2 lists attn_qkv, attn_out, mlp_gate, mlp_up,
 * mlp_down) with the shape of up (K = D, N = F), and the FFN is SwiGLU
 * ("Model" page, Parameters: ffn_dim is the width of the gate and up
 * projections): a = fp16(silu(g) * u), g = fp16(x . Wgate),
 * u = fp16(x . Wup), silu(z) = z / (1 + e^-z) evaluated in FP32.  Each weight
 * carries its own bits and group. */
typedef struct qg_block {
    int32_t D;
    int32_t F;
    qg_weight qkv;
    qg_weight out;
    qg_weight up;
    qg_weight down;
    qg_weight gate;
} qg_block;

int qg_abi_version(void);
int qg_layout_version(void);
/* Message of the last failed call on this thread ("" if none). */
const char* qg_last_error(void);

/* Quantise FP32 W [K][ldw] (ldw >= N) into layout v1 (see the format above;
 * CTX-TIER kernel details: per-group asymmetric scale = range / (levels - 1)).
 * group: 128, or K for per-row groups (QG_EUNSUPPORTED otherwise).
 * codes [N][K*bits/32] (compact rows), scales and zeros [N][K/group] are
 * written in full.
 * Bit-identical to the definition (FP64 arithmetic on the device).
 * Runs in two passes on `stream`: a validation pass that computes every
 * group's range and scale and writes nothing (no output at all), then, after
 * synchronising `stream` to read its verdict, the packing pass.  Non-finite W
 * or a scale that overflows FP16 returns QG_EINVAL with codes, scales and
 * zeros untouched; otherwise the packing pass is enqueued and the call
 * returns without waiting for it (stream order, like every other call). */
int qg_pack(const float* W, int64_t ldw, int32_t K, int32_t N, int32_t bits, int32_t group,
            uint32_t* codes, qg_half* scales, qg_half* zeros, void* stream);

/* INT4 -> INT2 re-quantisation ("β-Informed Deployment Features" page,
 * CTX-TIER, details of the shipped kernel: each group is dequantised and
 * quantised again to INT2 with a new scale and zero).  Every group's exact
 * INT4 dequant (q - z) s goes through qg_pack's quantiser with bits = 2; the
 * result is bit-identical to that definition.
 * w4: bits 4; w2: bits 2, same K, N and group; both described like any
 * qg_weight, each with its own row stride.  Per-row groups (group == K)
 * need K <= 32768 (QG_EUNSUPPORTED otherwise).  Out of place, w2's buffers
 * must not overlap w4's or each other.  In place (w2->codes == w4->codes,
 * w2->scales == w4->scales, w2->zeros == w4->zeros; any other overlap is
 * QG_EINVAL), two forms: with w2's row stride equal to w4's -- the pages'
 * in-place mode, INT2 rows kept at the INT4 stride (K/2 bytes), each INT2 row
 * over the front half of its own INT4 row -- one launch for groups of 128 up
 * to K = 32768 (beyond that one launch per doubling of the group index), and
 * with compact w2 rows (K/4 bytes), written over the first half of the INT4
 * buffer, which takes launches ordered by row (about log2 of the rows and of
 * the groups); the bytes past the INT2 data are left as they were.  Runs in two
 * passes on `stream`, like qg_pack: a validation pass that writes nothing,
 * then, after synchronising `stream` to read its verdict, the re-quantisation.
 * A non-finite INT4 scale or zero, or an INT2 scale that overflows FP16,
 * returns QG_EINVAL with w2 (and, in place, w4) untouched; otherwise the
 * re-quantisation is enqueued and the call returns without waiting for it:
 * free or reuse the INT4 buffers only after that work (stream order, as the
 * pages' tier switch frees them after a stream sync). */
int qg_requant_4to2(const qg_weight* w4, const qg_weight* w2, void* stream);

/* Y[M][N] = X[M][K] . dequant(w)[K][N] (quant_gemm, "β-Informed Deployment
 * Features" page).  X FP16 [M][ldx], Y FP16 [M][ldy], K <= ldx <= 2^22, ldy >= N, both
 * multiples of 8 and 16-byte aligned pointers; FP32 accumulation, one
 * round-to-nearest-even to FP16 at the end.  M == 0 is a no-op.
 * w->bits must be 4 (qg_gemm_int4) or 2 (qg_gemm_int2), like the pages'
 * dispatch on QuantWeight::bits.  ws/ws_bytes: device workspace of at least
 * qg_gemm_ws_bytes(w, M) bytes (may be NULL when that is 0). */
int qg_gemm_int4(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y, int64_t ldy,
                 int32_t M, void* ws, size_t ws_bytes, void* stream);
int qg_gemm_int2(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y, int64_t ldy,
                 int32_t M, void* ws, size_t ws_bytes, void* stream);
size_t qg_gemm_ws_bytes(const qg_weight* w, int32_t M);

/* The GEMM of qg_gemm_int4 / qg_gemm_int2 (dispatching on w->bits, which
 * must be 4 or 2) for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Instead of a caller's workspace it uses a library-owned static device
 * workspace of 16 MiB (each GPU the library runs on holds its own copy until
 * the process ends); it calls no allocator.  Same arguments, validation,
 * kernels and results (bit for bit) as qg_gemm_int4 / qg_gemm_int2 with a
 * workspace.  A shape whose qg_gemm_ws_bytes(w, M) exceeds 16 MiB is
 * rejected with QG_EINVAL before anything is enqueued.  The workspace holds
 * K-split partials only, every one written before it is read, so no call
 * depends on what an earlier call left there; but every call on one GPU
 * shares that GPU's copy, so two calls whose execution may overlap on one GPU
 * (different streams without ordering between them) race. */
int qg_gemm_static_ws(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y,
                      int64_t ldy, int32_t M, void* stream);

/* Iterations [L0, L1) of the shared block, in place on the FP32 residual
 * h [M][D] (run_loop_iters_range, "Warm-start mid-loop" page, internal flow:
 * the same weights are applied on every iteration).  Per iteration:
 *   x = fp16(LN(h)); qkv = fp16(x . Wqkv); o = fp16(qkv[:, 2D:3D] . Wout);
 *   h += o; x = fp16(LN(h)); u = fp16(x . Wup); d = fp16(u . Wdown); h += d;
 * and with a gate weight u = fp16(silu(fp16(x . Wgate)) * fp16(x . Wup)).
 * LN is parameter-free, eps 1e-5, population variance, computed in FP32.
 * Requires 0 <= L0 <= L1; L0 == L1 (or M == 0) is a no-op.  [L0, L1) followed
 * by [L1, L2) gives the same bits as [L0, L2).
 * scratch: device buffer of at least qg_loop_scratch_bytes(blk, M) bytes; after
 * the call it holds the last iteration's FP16 intermediates at the offsets
 * given by qg_loop_scratch_offsets (norm = second LN output [M][D],
 * qkv [M][3D], u [M][F] = the down projection's input, y = last
 * down-projection output [M][D], and with a gate g = gate output [M][F]).
 * Outside stream capture the iterations replay from a library-cached graph
 * (keyed by every pointer and size above; see qg_release_cache).  Inside a
 * caller's capture on `stream` the kernels are enqueued one by one, so the
 * call can be part of the caller's graph; qg_gemm_int4 / qg_gemm_int2 only
 * enqueue kernels and may be captured too, while qg_pack and
 * qg_requant_4to2 synchronise: on a stream under capture they return
 * QG_EINVAL before enqueuing anything. */
int qg_loop_range(const qg_block* blk, float* h, int32_t M, int32_t L0, int32_t L1,
                  void* scratch, size_t scratch_bytes, void* stream);
size_t qg_loop_scratch_bytes(const qg_block* blk, int32_t M);

/* Chunked prefill ("Model" page, Chunked prefill; Parameters: prefill_chunk):
 * the chunk-first driver.  Rows [0, M) of h are split into chunks of `chunk`
 * rows (the last one may be shorter) and each chunk runs through all
 * iterations [L0, L1) of the block (as qg_loop_range on those rows) before
 * the next chunk starts, so the FP16 scratch is sized for `chunk` rows, not
 * M: scratch_bytes >= qg_loop_chunked_scratch_bytes(blk, M, chunk); after the
 * call it holds the last chunk's intermediates.  chunk >= M is qg_loop_range.
 * Rows do not interact in this block (its attention stand-in attends each row
 * to itself), so each row's result is that of qg_loop_range on the chunk that
 * holds it; it equals the single-shot result within the GEMM tolerance, and
 * bit for bit where the chunk's tile plans match the single-shot M's.
 * hcache: NULL, or the FP16-h cache (the pages' FP16-h KV mode keeps h and
 * rebuilds K = W_k h and V = W_v h instead of storing K and V): FP16
 * [L1 - L0][M][D], 16-byte aligned; iteration L0 + i of row r writes its
 * attention input x = fp16(LN(h)), the QKV projection's input, at
 * hcache[i][r][:].  qg_gemm_int4 / qg_gemm_int2 of cached x with the K (or
 * V) rows of the QKV weight -- output channels [D, 2D) (or [2D, 3D)) of the
 * N-major codes, scales and zeros, a contiguous row range -- rebuilds that
 * iteration's K (V) columns of qkv, bit for bit where the GEMM's tile plan
 * matches the QKV projection's.  Validation, stream order and the cached
 * graphs (one per chunk) as in qg_loop_range. */
int qg_loop_range_chunked(const qg_block* blk, float* h, int32_t M, int32_t L0, int32_t L1,
                          int32_t chunk, void* scratch, size_t scratch_bytes, qg_half* hcache,
                          void* stream);
size_t qg_loop_chunked_scratch_bytes(const qg_block* blk, int32_t M, int32_t chunk);
/* Byte offsets of norm, qkv, u, y and g inside the loop scratch (any pointer
 * may be NULL; g is 0 for a block without a gate).  Returns QG_EINVAL for a
 * bad block. */
int qg_loop_scratch_offsets(const qg_block* blk, int32_t M, size_t* norm, size_t* qkv,
                            size_t* u, size_t* y, size_t* g);

/* Test exports running the same device unpack/dequant code the GEMM kernels
 * use.  qg_unpack writes codes q [N][K] as uint8.  qg_dequant writes
 * w^ [N][K] (N-major) as FP32 when out_fp16 == 0 (exact) or as FP16
 * (round-to-nearest-even of the exact value) when out_fp16 != 0. */
int qg_unpack(const qg_weight* w, uint8_t* q, void* stream);
int qg_dequant(const qg_weight* w, int32_t out_fp16, void* out, void* stream);

/* Frees library-owned state (cached loop graphs and their capture streams;
 * the device and pinned host status words of qg_pack and qg_requant_4to2)
 * after synchronising every device that holds some of it.  Safe to call at
 * any time when no library call is in flight on another thread. */
void qg_release_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
