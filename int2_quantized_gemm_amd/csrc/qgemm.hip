// qgemm.hip -- the C ABI of include/qgemm.h: argument validation, dispatch to
// the kernel families, and the loop driver (run_loop_iters_range of the
// "Warm-start mid-loop" page: iterations [L0, L1) applied in place on the
// residual with the same weights every iteration).
//
// Every entry point validates all arguments on the host before enqueuing
// anything; a failed check returns a negative status, leaves every output
// untouched and records a message for qg_last_error() (thread-local), the way
// the pages' errors name the failure point ("Model" page, Raises).
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdlib.h>
#include <string.h>
#include <vector>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return QG_OK;
}

int hip_fail(const char* where, hipError_t e) {
    return fail(QG_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Largest K and activation leading dimension (elements): the tiled kernels
// address a tile's operands through buffer descriptors of at most 2 GiB
// from the tile's first row (128 rows of up to 2^22 FP16 values = 1 GiB).
constexpr int64_t kMaxK = int64_t(1) << 22;

// Layout-v1 checks shared by every entry point taking a weight.
int check_weight(const qg_weight* w, const char* fn, const char* name) {
    if (!w) return fail(QG_EINVAL, "%s: %s is NULL", fn, name);
    if (w->bits != 4 && w->bits != 2)
        return fail(QG_EUNSUPPORTED, "%s: %s.bits = %d, layout v1 supports 4 and 2", fn, name,
                    w->bits);
    if (w->K <= 0 || w->K % 128 != 0 || w->K > kMaxK)
        return fail(QG_EINVAL, "%s: %s.K = %d must be a positive multiple of 128, at most %lld",
                    fn, name, w->K, (long long)kMaxK);
    if (w->group != 128 && w->group != w->K)
        return fail(QG_EUNSUPPORTED, "%s: %s.group = %d, layout v1 has groups of 128 or per-row "
                                     "groups (group = K = %d)", fn, name, w->group, w->K);
    if (w->N <= 0) return fail(QG_EINVAL, "%s: %s.N = %d must be positive", fn, name, w->N);
    if (!w->codes || !w->scales || !w->zeros)
        return fail(QG_EINVAL, "%s: %s has a NULL codes/scales/zeros pointer", fn, name);
    if (!aligned(w->codes, 16))
        return fail(QG_EINVAL, "%s: %s.codes must be 16-byte aligned", fn, name);
    if (!aligned(w->scales, 2) || !aligned(w->zeros, 2))
        return fail(QG_EINVAL, "%s: %s.scales/zeros must be 2-byte aligned", fn, name);
    const int64_t compact = (int64_t)w->K * w->bits / 32;
    if (w->ldc != 0 && (w->ldc < compact || w->ldc % 4 != 0 || w->ldc > (int64_t(1) << 20)))
        return fail(QG_EINVAL, "%s: %s.ldc = %lld must be 0 (compact) or a multiple of 4 in "
                               "[K*bits/32 = %lld, 2^20]", fn, name, (long long)w->ldc,
                    (long long)compact);
    return QG_OK;
}

// Everything but the workspace.
int check_gemm_io(const qg_half* X, int64_t ldx, const qg_weight* w, const qg_half* Y,
                  int64_t ldy, int32_t M, int bits, const char* fn) {
    int st = check_weight(w, fn, "w");
    if (st) return st;
    if (w->bits != bits)
        return fail(QG_EINVAL, "%s: w->bits = %d but this entry point computes %d-bit weights", fn,
                    w->bits, bits);
    if (M < 0) return fail(QG_EINVAL, "%s: M = %d must be >= 0", fn, M);
    if (M == 0) return QG_OK;
    if (!X || !Y) return fail(QG_EINVAL, "%s: X or Y is NULL", fn);
    if (ldx < w->K || ldx % 8 != 0 || ldx > kMaxK)
        return fail(QG_EINVAL, "%s: ldx = %lld must be >= K = %d, a multiple of 8 and at most %lld",
                    fn, (long long)ldx, w->K, (long long)kMaxK);
    if (ldy < w->N || ldy % 8 != 0)
        return fail(QG_EINVAL, "%s: ldy = %lld must be >= N = %d and a multiple of 8", fn,
                    (long long)ldy, w->N);
    if (!aligned(X, 16) || !aligned(Y, 16))
        return fail(QG_EINVAL, "%s: X and Y must be 16-byte aligned", fn);
    return QG_OK;
}

int check_gemm(const qg_half* X, int64_t ldx, const qg_weight* w, const qg_half* Y, int64_t ldy,
               int32_t M, const void* ws, size_t ws_bytes, int bits, const char* fn) {
    const int st = check_gemm_io(X, ldx, w, Y, ldy, M, bits, fn);
    if (st || M == 0) return st;
    const size_t need = qg::gemm_ws_bytes(w->bits, M, w->K, w->N);
    if (ws_bytes < need)
        return fail(QG_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu required", fn,
                    ws_bytes, need);
    if (need > 0 && !aligned(ws, 16))
        return fail(QG_EINVAL, "%s: workspace must be a 16-byte aligned pointer", fn);
    return QG_OK;
}

// ---- loop scratch layout: norm [M][D], qkv [M][3D], u [M][F], y [M][D] (FP16),
// then the GEMM workspace; every region 256-byte aligned.
struct LoopLayout {
    size_t norm, qkv, u, y, g, ws, ws_bytes, total;
};

bool gated(const qg_block* b) { return b->gate.codes != nullptr; }

LoopLayout loop_layout(const qg_block* b, int32_t M) {
    LoopLayout L{};
    const size_t m = (size_t)M;
    L.norm = 0;
    L.qkv = align_up(L.norm + m * b->D * 2, 256);
    L.u = align_up(L.qkv + m * 3 * b->D * 2, 256);
    L.y = align_up(L.u + m * b->F * 2, 256);
    L.g = gated(b) ? align_up(L.y + m * b->D * 2, 256) : 0;
    L.ws = align_up((gated(b) ? L.g + m * b->F * 2 : L.y + m * b->D * 2), 256);
    size_t ws = 0;
    const qg_weight* ws_list[5] = {&b->qkv, &b->out, &b->up, &b->down, &b->gate};
    for (const qg_weight* w : ws_list) {
        if (w == &b->gate && !gated(b)) continue;
        size_t n = qg::gemm_ws_bytes(w->bits, M, w->K, w->N);
        // the residual projections' partials when their end is fused with
        // the next LayerNorm (M > 1)
        if (M > 1 && (w == &b->out || w == &b->down) && qg::reduce_ln_supported(b->D)) {
            const size_t p = qg::gemm_parts_ws_bytes(w->bits, M, w->K, w->N);
            n = p > n ? p : n;
        }
        ws = n > ws ? n : ws;
    }
    L.ws_bytes = ws;
    L.total = align_up(L.ws + ws, 256);
    return L;
}

int check_block(const qg_block* b, const char* fn) {
    if (!b) return fail(QG_EINVAL, "%s: blk is NULL", fn);
    if (b->D <= 0 || b->D % 128 != 0 || b->D > 8192)
        return fail(QG_EINVAL, "%s: D = %d must be a positive multiple of 128, at most 8192", fn,
                    b->D);
    if (b->F <= 0 || b->F % 128 != 0)
        return fail(QG_EINVAL, "%s: F = %d must be a positive multiple of 128", fn, b->F);
    struct {
        const qg_weight* w;
        const char* name;
        int K, N;
    } ws[5] = {{&b->qkv, "qkv", b->D, 3 * b->D},
               {&b->out, "out", b->D, b->D},
               {&b->up, "up", b->D, b->F},
               {&b->down, "down", b->F, b->D},
               {&b->gate, "gate", b->D, b->F}};
    for (auto& e : ws) {
        if (e.w == &b->gate && !gated(b)) continue;  // no gate: identity FFN activation
        int st = check_weight(e.w, fn, e.name);
        if (st) return st;
        if (e.w->K != e.K || e.w->N != e.N)
            return fail(QG_EINVAL, "%s: %s is %dx%d (KxN) but the block needs %dx%d", fn, e.name,
                        e.w->K, e.w->N, e.K, e.N);
    }
    return QG_OK;
}

// QG_FUSE_SWIGLU=0 keeps the gate and up projections of a gated block as two
// launches even where one SwiGLU pair launch could run them (the fused-versus-
// separate parity test); read on every call.
bool swiglu_fusion_enabled() {
    const char* v = getenv("QG_FUSE_SWIGLU");
    return !(v && v[0] == '0');
}

// QG_FUSE_REDUCE_LN=0 ends the residual projections at M > 1 with the split-K
// reduction and the LayerNorm kernel as two launches over the same partials,
// instead of one fused launch (the fused-versus-separate parity test); read on
// every call.
bool reduce_ln_fusion_enabled() {
    const char* v = getenv("QG_FUSE_REDUCE_LN");
    return !(v && v[0] == '0');
}

// Enqueue `iters` iterations of the loop block on stream s (no validation).
// hcache (optional): FP16 rows receiving each iteration's attention input
// x = fp16(LN(h)), iteration l at hcache + l * hstride (the FP16-h cache:
// the QKV GEMM then reads x from there instead of the norm scratch).
hipError_t enqueue_loop(const qg_block* blk, float* h, int32_t M, int32_t iters, void* scratch,
                        const LoopLayout& L, bool fuse_swiglu, bool fuse_rln, qg_half* hcache,
                        int64_t hstride, hipStream_t s) {
    char* base = (char*)scratch;
    qg_half* norm = (qg_half*)(base + L.norm);
    qg_half* qkv = (qg_half*)(base + L.qkv);
    qg_half* u = (qg_half*)(base + L.u);
    qg_half* y = (qg_half*)(base + L.y);
    void* ws = base + L.ws;
    const int D = blk->D, F = blk->F;
    hipError_t e = hipSuccess;
    // At M == 1 the QKV GEMV computes the LayerNorm of h in its prologue;
    // at M > 1 a LayerNorm kernel writes norm before the first iteration and
    // the previous iteration's down-projection launch before the others.
    const bool gate = gated(blk);
    qg_half* g = gate ? (qg_half*)(base + L.g) : nullptr;
    const bool fuse_qkv = qg::gemm_fuses_layernorm(blk->qkv.bits, M, D, 3 * D);
    const bool fuse_first = qg::gemm_fuses_layernorm(gate ? blk->gate.bits : blk->up.bits, M, D, F);
    // At M == 1 a gated block runs gate and up as one SwiGLU pair launch.
    const bool pair = gate && fuse_swiglu && blk->gate.bits == blk->up.bits &&
                      blk->gate.group == blk->up.group &&
                      qg::gemm_fuses_swiglu(blk->up.bits, M, D, F);
    // At M > 1 each residual projection (out, down) writes its K-part
    // partials and one launch sums them, adds the result into h and computes
    // the LayerNorm that follows (of the FFN input after out, of the next
    // iteration's QKV input after down; not after the last down, so that norm
    // keeps the last FFN input).  With fuse_rln off the same partials go
    // through the split-K reduction and the LayerNorm kernel instead, with
    // bit-identical results.
    const bool rln = M > 1 && qg::reduce_ln_supported(D);
    // where iteration l's QKV input x is written and read
    auto xbuf = [&](int32_t l) { return hcache ? hcache + (int64_t)l * hstride : norm; };
    auto residual_ln = [&](const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* ln_out) {
        int parts = 0;
        qg::GemmArgs ra{X, ldx, w, y, D, M, qg::kResidual, h, D, ws, L.ws_bytes};
        ra.parts = &parts;
        hipError_t r = qg::launch_gemm(ra, s);
        if (r != hipSuccess) return r;
        if (fuse_rln)
            return qg::launch_reduce_residual_ln((const float*)ws, parts, M, D, y, h, ln_out, s);
        ra.parts = nullptr;
        r = qg::launch_splitk_reduce((const float*)ws, parts, ra, s);
        if (r == hipSuccess && ln_out) r = qg::launch_layernorm(h, M, D, ln_out, s);
        return r;
    };
    for (int32_t l = 0; l < iters && e == hipSuccess; ++l) {
        qg::GemmArgs qa{xbuf(l), D, &blk->qkv, qkv, 3 * D, M, qg::kStore, nullptr, 0, ws,
                        L.ws_bytes};
        if (fuse_qkv) {
            qa.ln_h = h;
            qa.norm_out = hcache ? xbuf(l) : nullptr;
        } else if (!(rln && l > 0)) {  // (else the previous down's launch wrote x)
            e = qg::launch_layernorm(h, M, D, xbuf(l), s);
        }
        if (e == hipSuccess) e = qg::launch_gemm(qa, s);
        if (e == hipSuccess && rln)
            e = residual_ln(qkv + 2 * D, 3 * D, &blk->out, norm);
        else if (e == hipSuccess)
            e = qg::launch_gemm({qkv + 2 * D, 3 * D, &blk->out, y, D, M, qg::kResidual, h, D, ws,
                                 L.ws_bytes},
                                s);
        // FFN input: the first FFN projection (gate, else up) normalises h
        // itself at M == 1 and stores norm; at M > 1 the out projection's
        // launch wrote it (a LayerNorm kernel where D has no fused form).
        // With a gate, up multiplies silu(g) in.
        const qg_weight* first = gate ? &blk->gate : &blk->up;
        qg::GemmArgs fa{norm, D, first, gate ? g : u, F, M, qg::kStore, nullptr, 0, ws,
                        L.ws_bytes};
        if (fuse_first) {
            fa.ln_h = h;
            fa.norm_out = norm;
        } else if (e == hipSuccess && !rln) {
            e = qg::launch_layernorm(h, M, D, norm, s);
        }
        if (pair) {
            fa.w2 = &blk->up;
            fa.g_out = g;
            fa.Y = u;
        }
        if (e == hipSuccess) e = qg::launch_gemm(fa, s);
        if (gate && !pair && e == hipSuccess) {
            qg::GemmArgs ua{norm, D, &blk->up, u, F, M, qg::kGateMul, nullptr, 0, ws, L.ws_bytes};
            ua.gm = g;
            ua.ldg = F;
            e = qg::launch_gemm(ua, s);
        }
        if (e == hipSuccess && rln)
            e = residual_ln(u, F, &blk->down, l + 1 < iters ? xbuf(l + 1) : nullptr);
        else if (e == hipSuccess)
            e = qg::launch_gemm({u, F, &blk->down, y, D, M, qg::kResidual, h, D, ws, L.ws_bytes},
                                s);
    }
    return e;
}

// QG_LOOP_GRAPHS=0 makes qg_loop_range enqueue kernels one by one (debugging
// and the graph-versus-direct parity test); read on every call.
bool loop_graphs_enabled() {
    const char* v = getenv("QG_LOOP_GRAPHS");
    return !(v && v[0] == '0');
}

// Cached, instantiated graphs of the loop's kernel sequence.  A graph bakes in
// every pointer and shape it was built with, so the key holds all of them.
struct LoopKey {
    qg_block blk;
    const float* h;
    void* scratch;
    qg_half* hcache;
    int64_t hstride;
    int32_t M, iters, device;
    bool fuse_swiglu, fuse_rln;
    bool operator==(const LoopKey& o) const { return memcmp(this, &o, sizeof *this) == 0; }
};

struct LoopGraph {
    LoopKey key;
    hipGraphExec_t exec;
    uint64_t last_use;
};

std::mutex g_graph_mu;
std::vector<LoopGraph> g_graphs;
uint64_t g_graph_clock = 0;
hipStream_t g_capture_stream[64] = {nullptr};
constexpr size_t kMaxGraphs = 32;

// Waits for all work on `device` (a launch of a cached graph may still be
// running there) and restores the caller's current device.
void sync_device(int device) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    if (cur != device) (void)hipSetDevice(device);
    (void)hipDeviceSynchronize();
    if (cur != device) (void)hipSetDevice(cur);
}

// Launches the cached graph for these arguments on stream s, capturing and
// instantiating it first if needed.  The launch happens under the cache lock,
// so no other thread can evict (destroy) the graph between lookup and launch.
hipError_t launch_loop_graph(const qg_block* blk, float* h, int32_t M, int32_t iters,
                             void* scratch, const LoopLayout& L, bool fuse_swiglu, bool fuse_rln,
                             qg_half* hcache, int64_t hstride, hipStream_t s) {
    LoopKey key;
    memset(&key, 0, sizeof key);  // padding takes part in the comparison
    key.blk = *blk;
    key.h = h;
    key.scratch = scratch;
    key.M = M;
    key.iters = iters;
    key.fuse_swiglu = fuse_swiglu;
    key.fuse_rln = fuse_rln;
    key.hcache = hcache;
    key.hstride = hcache ? hstride : 0;
    hipError_t e = hipGetDevice(&key.device);
    if (e != hipSuccess) return e;
    if (key.device < 0 || key.device >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_graph_mu);
    for (LoopGraph& g : g_graphs) {
        if (g.key == key) {
            g.last_use = ++g_graph_clock;
            return hipGraphLaunch(g.exec, s);
        }
    }
    hipStream_t& cs = g_capture_stream[key.device];
    if (!cs && (e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking)) != hipSuccess) {
        cs = nullptr;
        return e;
    }
    if ((e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal)) != hipSuccess) return e;
    hipError_t le =
        enqueue_loop(blk, h, M, iters, scratch, L, fuse_swiglu, fuse_rln, hcache, hstride, cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    if (le != hipSuccess || e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return le != hipSuccess ? le : e;
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return e;
    if (g_graphs.size() >= kMaxGraphs) {
        // Evict the least recently used graph; a launch of it may still be
        // running on its device, so wait for that device first.
        size_t lru = 0;
        for (size_t i = 1; i < g_graphs.size(); ++i)
            if (g_graphs[i].last_use < g_graphs[lru].last_use) lru = i;
        sync_device(g_graphs[lru].key.device);
        (void)hipGraphExecDestroy(g_graphs[lru].exec);
        g_graphs.erase(g_graphs.begin() + lru);
    }
    g_graphs.push_back({key, exec, ++g_graph_clock});
    return hipGraphLaunch(exec, s);
}

// Per-device status word for qg_pack and qg_requant_4to2: a device int into
// which a failing kernel stores the call's tag, and a pinned host int it is
// copied back to (a copy into pageable memory goes through a staging buffer
// and costs several times the copy).  Each call takes the next nonzero tag, so
// the word needs no clearing launch: it reports a failure of this call only
// when it holds this call's tag.  Library-owned, freed by qg_release_cache.
struct StatusWord {
    int* dev = nullptr;
    int* host = nullptr;
    int tag = 0;
};
std::mutex g_pack_mu;
StatusWord g_pack_status[64];

// Enqueues the validation pass check(status, tag) on s with the current
// device's status word and a fresh tag, copies the word back and
// synchronises s; *bad is set when the pass reported a failure (the pass
// writes nothing else, so on failure no output has been touched).  Caller
// holds g_pack_mu.  Refused, before anything is enqueued or allocated, on a
// stream that is being captured: the read-back and the synchronisation cannot
// be part of a graph.
template <class Launch>
int run_with_status(const char* fn, hipStream_t s, Launch&& launch, int* bad) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (cap != hipStreamCaptureStatusNone)
        return fail(QG_EINVAL, "%s: the stream is being captured; this call synchronises its "
                               "stream and cannot be part of a graph", fn);
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (dev < 0 || dev >= 64) return fail(QG_EHIP, "%s: device index %d out of range", fn, dev);
    StatusWord& w = g_pack_status[dev];
    if (!w.dev) {
        // a fresh word starts at 0, which is never a tag
        if ((e = hipMalloc((void**)&w.dev, sizeof(int))) != hipSuccess) {
            w.dev = nullptr;
            return fail(QG_ENOMEM, "%s: cannot allocate the 4-byte status word (%s)", fn,
                        hipGetErrorString(e));
        }
        if ((e = hipMemset(w.dev, 0, sizeof(int))) != hipSuccess) {
            (void)hipFree(w.dev);
            w.dev = nullptr;
            return hip_fail(fn, e);
        }
        w.tag = 0;
    }
    if (!w.host && (e = hipHostMalloc((void**)&w.host, sizeof(int), hipHostMallocDefault)) !=
                       hipSuccess) {
        w.host = nullptr;
        return fail(QG_ENOMEM, "%s: cannot allocate the pinned status word (%s)", fn,
                    hipGetErrorString(e));
    }
    w.tag = w.tag == 0x7FFFFFFF ? 1 : w.tag + 1;
    if ((e = launch(w.dev, w.tag)) != hipSuccess) return hip_fail(fn, e);
    if ((e = hipMemcpyAsync(w.host, w.dev, sizeof(int), hipMemcpyDeviceToHost, s)) != hipSuccess)
        return hip_fail(fn, e);
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(fn, e);
    *bad = *w.host == w.tag;
    return QG_OK;
}

// ---- static workspace of qg_gemm_static_ws (callers that cannot allocate).
// A file-scope device array: each GPU the library runs on holds its own copy
// from module load until the process ends.  In host code `static_ws` is only
// a host-side stand-in for the symbol; the device address of each GPU's copy
// comes from hipGetSymbolAddress with that GPU current, once, and only that
// address is ever handed to kernels.
constexpr size_t kStaticWsBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t static_ws[kStaticWsBytes];

std::mutex g_static_ws_mu;
void* g_static_ws_ptr[64] = {nullptr};

// Device address of the current device's static workspace (looked up on the
// first call on that device); QG_OK or a failure status with its message.
int static_ws_address(const char* fn, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(fn, e);
    if (dev < 0 || dev >= 64) return fail(QG_EHIP, "%s: device index %d out of range", fn, dev);
    std::lock_guard<std::mutex> lock(g_static_ws_mu);
    if (!g_static_ws_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(static_ws));
        if (e != hipSuccess || p == nullptr)
            return hip_fail(fn, e != hipSuccess ? e : hipErrorInvalidSymbol);
        g_static_ws_ptr[dev] = p;
    }
    *out = g_static_ws_ptr[dev];
    return QG_OK;
}

}  // namespace

extern "C" {

int qg_abi_version(void) { return QG_ABI_VERSION; }
int qg_layout_version(void) { return QG_LAYOUT_VERSION; }
const char* qg_last_error(void) { return g_last_error.c_str(); }

int qg_pack(const float* W, int64_t ldw, int32_t K, int32_t N, int32_t bits, int32_t group,
            uint32_t* codes, qg_half* scales, qg_half* zeros, void* stream) {
    const char* fn = "qg_pack";
    if (bits != 4 && bits != 2)
        return fail(QG_EUNSUPPORTED, "%s: bits = %d, layout v1 supports 4 and 2", fn, bits);
    if (group != 128 && group != K)
        return fail(QG_EUNSUPPORTED, "%s: group = %d, layout v1 has groups of 128 or per-row "
                                     "groups (group = K = %d)", fn, group, K);
    if (K <= 0 || K % 128 != 0 || K > kMaxK)
        return fail(QG_EINVAL, "%s: K = %d must be a positive multiple of 128, at most %lld", fn,
                    K, (long long)kMaxK);
    if (N <= 0) return fail(QG_EINVAL, "%s: N = %d must be positive", fn, N);
    if (ldw < N) return fail(QG_EINVAL, "%s: ldw = %lld must be >= N = %d", fn, (long long)ldw, N);
    if (!W || !codes || !scales || !zeros)
        return fail(QG_EINVAL, "%s: W, codes, scales and zeros must be non-NULL", fn);
    if (!aligned(W, 4) || !aligned(codes, 4) || !aligned(scales, 2) || !aligned(zeros, 2))
        return fail(QG_EINVAL, "%s: misaligned pointer", fn);
    hipStream_t s = (hipStream_t)stream;
    std::lock_guard<std::mutex> lock(g_pack_mu);
    int bad = 0;
    const int st = run_with_status(fn, s, [&](int* status, int tag) {
        return qg::launch_pack_check(W, ldw, K, N, bits, group, status, tag, s);
    }, &bad);
    if (st) return st;
    if (bad)
        return fail(QG_EINVAL, "%s: W holds a non-finite value or a group whose scale overflows "
                               "FP16", fn);
    const hipError_t e = qg::launch_pack(W, ldw, K, N, bits, group, codes, scales, zeros, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

// [p, p + bytes) and [q, q + bytes2) share a byte.
static bool overlaps(const void* p, size_t bytes, const void* q, size_t bytes2) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + bytes2 && b < a + bytes;
}

int qg_requant_4to2(const qg_weight* w4, const qg_weight* w2, void* stream) {
    const char* fn = "qg_requant_4to2";
    if (!w4 || !w2) return fail(QG_EINVAL, "%s: w4 and w2 must be non-NULL", fn);
    int st = check_weight(w4, fn, "w4");
    if (st) return st;
    st = check_weight(w2, fn, "w2");
    if (st) return st;
    if (w4->bits != 4 || w2->bits != 2)
        return fail(QG_EINVAL, "%s: w4.bits = %d and w2.bits = %d must be 4 and 2", fn, w4->bits,
                    w2->bits);
    if (w2->K != w4->K || w2->N != w4->N)
        return fail(QG_EINVAL, "%s: w2 is %d x %d but w4 is %d x %d (K x N)", fn, w2->K, w2->N,
                    w4->K, w4->N);
    if (w2->group != w4->group)
        return fail(QG_EINVAL, "%s: w2.group = %d must equal w4.group = %d", fn, w2->group,
                    w4->group);
    if (w4->group != 128 && w4->K > qg::kRequantRowMaxK)
        return fail(QG_EUNSUPPORTED, "%s: per-row groups need K <= %d (K = %d)", fn,
                    qg::kRequantRowMaxK, w4->K);
    const int groups = w4->K / w4->group;
    const int64_t l4 = qg::code_ld(*w4), l2 = qg::code_ld(*w2);
    // bytes each code array spans: N - 1 strides and one row
    const size_t c4 = ((size_t)(w4->N - 1) * l4 + w4->K / 8) * 4;
    const size_t c2 = ((size_t)(w4->N - 1) * l2 + w4->K / 16) * 4;
    const size_t sz = (size_t)w4->N * groups * 2;
    const void* in[3] = {w4->codes, w4->scales, w4->zeros};
    const size_t in_bytes[3] = {c4, sz, sz};
    const void* out[3] = {w2->codes, w2->scales, w2->zeros};
    const size_t out_bytes[3] = {c2, sz, sz};
    // each output is either its own input (in place) or apart from every
    // input, and the outputs are apart from each other
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j) {
            if (i == j && out[i] == in[j]) continue;
            if (overlaps(out[i], out_bytes[i], in[j], in_bytes[j]))
                return fail(QG_EINVAL, "%s: output %s overlaps input %s (only exact in-place "
                                       "aliasing of codes, scales or zeros is allowed)", fn,
                            i == 0 ? "codes" : i == 1 ? "scales" : "zeros",
                            j == 0 ? "codes" : j == 1 ? "scales" : "zeros");
        }
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(out[i], out_bytes[i], out[j], out_bytes[j]))
                return fail(QG_EINVAL, "%s: the outputs overlap each other", fn);
    }
    const bool in_place = w2->codes == w4->codes;
    if (in_place && l2 != l4 && l2 != w4->K / 16)
        return fail(QG_EINVAL, "%s: in place, w2.ldc must give w4's row stride (%lld words) or "
                               "compact rows (%d words), got %lld", fn, (long long)l4, w4->K / 16,
                    (long long)l2);
    hipStream_t s = (hipStream_t)stream;
    std::lock_guard<std::mutex> lock(g_pack_mu);
    int bad = 0;
    const int rc = run_with_status(fn, s, [&](int* status, int tag) {
        return qg::launch_requant_4to2_check(*w4, status, tag, s);
    }, &bad);
    if (rc) return rc;
    if (bad)
        return fail(QG_EINVAL, "%s: w4 holds a non-finite scale or zero, or a group whose INT2 "
                               "scale overflows FP16", fn);
    const hipError_t e = qg::launch_requant_4to2(*w4, *w2, in_place, s);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

size_t qg_gemm_ws_bytes(const qg_weight* w, int32_t M) {
    if (!w || (w->bits != 4 && w->bits != 2) || M < 0) return 0;
    return qg::gemm_ws_bytes(w->bits, M, w->K, w->N);
}

static int gemm_entry(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y, int64_t ldy,
                      int32_t M, void* ws, size_t ws_bytes, void* stream, int bits,
                      const char* fn) {
    int st = check_gemm(X, ldx, w, Y, ldy, M, ws, ws_bytes, bits, fn);
    if (st) return st;
    if (M == 0) return ok();
    qg::GemmArgs a{X, ldx, w, Y, ldy, M, qg::kStore, nullptr, 0, ws, ws_bytes};
    hipError_t e = qg::launch_gemm(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

int qg_gemm_int4(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y, int64_t ldy,
                 int32_t M, void* ws, size_t ws_bytes, void* stream) {
    return gemm_entry(X, ldx, w, Y, ldy, M, ws, ws_bytes, stream, 4, "qg_gemm_int4");
}

int qg_gemm_int2(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y, int64_t ldy,
                 int32_t M, void* ws, size_t ws_bytes, void* stream) {
    return gemm_entry(X, ldx, w, Y, ldy, M, ws, ws_bytes, stream, 2, "qg_gemm_int2");
}

int qg_gemm_static_ws(const qg_half* X, int64_t ldx, const qg_weight* w, qg_half* Y,
                      int64_t ldy, int32_t M, void* stream) {
    const char* fn = "qg_gemm_static_ws";
    int st = check_weight(w, fn, "w");
    if (st) return st;
    // validate as qg_gemm_int4 / qg_gemm_int2 (dispatching on w->bits), with
    // the static workspace standing in for the caller's
    const size_t need = qg::gemm_ws_bytes(w->bits, M < 0 ? 0 : M, w->K, w->N);
    if (need > kStaticWsBytes)
        return fail(QG_EINVAL, "%s: this shape needs %zu bytes of workspace, more than the %zu "
                               "of the static workspace (use qg_gemm_int%d with a workspace)",
                    fn, need, kStaticWsBytes, w->bits);
    st = check_gemm_io(X, ldx, w, Y, ldy, M, w->bits, fn);
    if (st) return st;
    if (M == 0) return ok();
    void* ws = nullptr;
    if (need > 0 && (st = static_ws_address(fn, &ws)) != QG_OK) return st;
    qg::GemmArgs a{X, ldx, w, Y, ldy, M, qg::kStore, nullptr, 0, ws, need};
    hipError_t e = qg::launch_gemm(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

size_t qg_loop_scratch_bytes(const qg_block* blk, int32_t M) {
    if (!blk || M < 0 || blk->D <= 0 || blk->F <= 0) return 0;
    return loop_layout(blk, M).total;
}

size_t qg_loop_chunked_scratch_bytes(const qg_block* blk, int32_t M, int32_t chunk) {
    if (!blk || M < 0 || chunk < 1 || blk->D <= 0 || blk->F <= 0) return 0;
    if (M == 0) return 0;
    const int32_t rows = chunk < M ? chunk : M, tail = M % rows;
    const size_t a = loop_layout(blk, rows).total, b = tail ? loop_layout(blk, tail).total : 0;
    return a > b ? a : b;
}

int qg_loop_scratch_offsets(const qg_block* blk, int32_t M, size_t* norm, size_t* qkv, size_t* u,
                            size_t* y, size_t* g) {
    int st = check_block(blk, "qg_loop_scratch_offsets");
    if (st) return st;
    if (M < 0) return fail(QG_EINVAL, "qg_loop_scratch_offsets: M = %d must be >= 0", M);
    const LoopLayout L = loop_layout(blk, M);
    if (norm) *norm = L.norm;
    if (qkv) *qkv = L.qkv;
    if (u) *u = L.u;
    if (y) *y = L.y;
    if (g) *g = L.g;
    return ok();
}

// Iterations [L0, L1) on rows h [M][D] (validated), by the cached graph or,
// under a caller's capture or with graphs off, kernel by kernel.
static hipError_t run_loop(const qg_block* blk, float* h, int32_t M, int32_t iters, void* scratch,
                           const LoopLayout& L, qg_half* hcache, int64_t hstride, hipStream_t s) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return e;
    // Inside a caller's graph capture, or with graphs switched off, the
    // kernels are enqueued one by one; otherwise the iteration sequence is
    // replayed from a cached graph (one launch instead of 4-6 per iteration).
    const bool fuse_swiglu = swiglu_fusion_enabled();
    const bool fuse_rln = reduce_ln_fusion_enabled();
    if (cap != hipStreamCaptureStatusNone || !loop_graphs_enabled())
        return enqueue_loop(blk, h, M, iters, scratch, L, fuse_swiglu, fuse_rln, hcache, hstride,
                            s);
    return launch_loop_graph(blk, h, M, iters, scratch, L, fuse_swiglu, fuse_rln, hcache, hstride,
                             s);
}

int qg_loop_range(const qg_block* blk, float* h, int32_t M, int32_t L0, int32_t L1, void* scratch,
                  size_t scratch_bytes, void* stream) {
    const char* fn = "qg_loop_range";
    int st = check_block(blk, fn);
    if (st) return st;
    if (M < 0) return fail(QG_EINVAL, "%s: M = %d must be >= 0", fn, M);
    if (L0 < 0 || L1 < L0)
        return fail(QG_EINVAL, "%s: need 0 <= L0 <= L1, got L0 = %d, L1 = %d", fn, L0, L1);
    if (M == 0 || L0 == L1) return ok();
    if (!h || !aligned(h, 16)) return fail(QG_EINVAL, "%s: h must be a 16-byte aligned pointer", fn);
    const LoopLayout L = loop_layout(blk, M);
    if (!scratch || !aligned(scratch, 256))
        return fail(QG_EINVAL, "%s: scratch must be a 256-byte aligned pointer", fn);
    if (scratch_bytes < L.total)
        return fail(QG_EINVAL, "%s: scratch of %zu bytes is smaller than the %zu required", fn,
                    scratch_bytes, L.total);
    const hipError_t e = run_loop(blk, h, M, L1 - L0, scratch, L, nullptr, 0, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
}

int qg_loop_range_chunked(const qg_block* blk, float* h, int32_t M, int32_t L0, int32_t L1,
                          int32_t chunk, void* scratch, size_t scratch_bytes, qg_half* hcache,
                          void* stream) {
    const char* fn = "qg_loop_range_chunked";
    int st = check_block(blk, fn);
    if (st) return st;
    if (M < 0) return fail(QG_EINVAL, "%s: M = %d must be >= 0", fn, M);
    if (chunk < 1) return fail(QG_EINVAL, "%s: chunk = %d must be >= 1", fn, chunk);
    if (L0 < 0 || L1 < L0)
        return fail(QG_EINVAL, "%s: need 0 <= L0 <= L1, got L0 = %d, L1 = %d", fn, L0, L1);
    if (M == 0 || L0 == L1) return ok();
    if (!h || !aligned(h, 16)) return fail(QG_EINVAL, "%s: h must be a 16-byte aligned pointer", fn);
    if (hcache && !aligned(hcache, 16))
        return fail(QG_EINVAL, "%s: hcache must be NULL or a 16-byte aligned pointer", fn);
    const int32_t rows = chunk < M ? chunk : M;
    const LoopLayout L = loop_layout(blk, rows);
    const int32_t tail = M % rows;
    const LoopLayout Lt = loop_layout(blk, tail ? tail : rows);
    const size_t need = L.total > Lt.total ? L.total : Lt.total;
    if (!scratch || !aligned(scratch, 256))
        return fail(QG_EINVAL, "%s: scratch must be a 256-byte aligned pointer", fn);
    if (scratch_bytes < need)
        return fail(QG_EINVAL, "%s: scratch of %zu bytes is smaller than the %zu required for "
                               "chunks of %d rows (qg_loop_chunked_scratch_bytes)", fn,
                    scratch_bytes, need, rows);
    // chunk first: rows [r0, r0 + m) run through all iterations before the
    // next chunk starts; a ragged last chunk has a layout of its own
    const int64_t D = blk->D;
    for (int32_t r0 = 0; r0 < M; r0 += rows) {
        const int32_t m = M - r0 < rows ? M - r0 : rows;
        const LoopLayout& Lc = m == rows ? L : Lt;
        const hipError_t e = run_loop(blk, h + (int64_t)r0 * D, m, L1 - L0, scratch, Lc,
                                      hcache ? hcache + (int64_t)r0 * D : nullptr,
                                      (int64_t)M * D, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(fn, e);
    }
    return ok();
}

int qg_unpack(const qg_weight* w, uint8_t* q, void* stream) {
    int st = check_weight(w, "qg_unpack", "w");
    if (st) return st;
    if (!q) return fail(QG_EINVAL, "qg_unpack: q is NULL");
    hipError_t e = qg::launch_unpack(*w, q, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("qg_unpack", e);
    return ok();
}

int qg_dequant(const qg_weight* w, int32_t out_fp16, void* out, void* stream) {
    int st = check_weight(w, "qg_dequant", "w");
    if (st) return st;
    if (!out || !aligned(out, 4)) return fail(QG_EINVAL, "qg_dequant: out must be 4-byte aligned");
    hipError_t e = qg::launch_dequant(*w, out_fp16 != 0, out, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail("qg_dequant", e);
    return ok();
}

void qg_release_cache(void) {
    {
        std::lock_guard<std::mutex> glock(g_graph_mu);
        bool synced[64] = {false};
        for (LoopGraph& g : g_graphs) {
            if (!synced[g.key.device]) {
                sync_device(g.key.device);
                synced[g.key.device] = true;
            }
            (void)hipGraphExecDestroy(g.exec);
        }
        g_graphs.clear();
        // the per-device capture streams (they only ever record, never run)
        int cur = 0;
        (void)hipGetDevice(&cur);
        for (int d = 0; d < 64; ++d) {
            if (!g_capture_stream[d]) continue;
            (void)hipSetDevice(d);
            (void)hipStreamDestroy(g_capture_stream[d]);
            g_capture_stream[d] = nullptr;
        }
        (void)hipSetDevice(cur);
    }
    std::lock_guard<std::mutex> lock(g_pack_mu);
    bool any = false;
    for (const StatusWord& w : g_pack_status) any |= w.dev != nullptr || w.host != nullptr;
    if (!any) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (int d = 0; d < 64; ++d) {
        StatusWord& w = g_pack_status[d];
        if (w.dev || w.host) {
            (void)hipSetDevice(d);
            (void)hipDeviceSynchronize();
            if (w.dev) (void)hipFree(w.dev);
            if (w.host) (void)hipHostFree(w.host);
            w = StatusWord{};
        }
    }
    (void)hipSetDevice(cur);
}

}  // extern "C"
