"""GPU parity of qg_loop_range against the oracle's loop driver.

Every row is checked against the oracle, the measured D=2048/F=8192
workloads at their real M and L included (the FP64 oracle takes seconds to
tens of seconds for them on the host's cores).  The residual h must
meet rel-L2 <= 2e-3 and max-abs <= 1e-2*max(1, rms(h_ref)); the last
iteration's FP16 intermediates in the scratch meet the GEMM tolerance.
Invariants: an empty range leaves h untouched, [L0,L1) then [L1,L2) equals
[L0,L2) bit for bit, and repeated runs are bit-identical.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu


def _blocks(orc, M, bits, D, F, seed, gated=False):
    inp = workloads.block(M, seed=seed, D=D, F=F, gated=gated)
    blk = qg.pack_block(inp.W, bits, D, F)
    oblk = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, bits, D, F)
    return inp, blk, oblk


def _check_h(h, href, what):
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h, href, what, max_abs=1e-2 * max(1.0, rms))


def _fp16_ulps(x: np.ndarray) -> np.ndarray:
    """FP16 spacing at each |x| (subnormal spacing below 2^-14)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _swiglu_bound(orc, oblk, last):
    """Element-wise bound on |a_gpu - a_ref| for the SwiGLU activation
    a = fp16(silu(g) u), g and u FP16 projection outputs: the GEMM contract
    lets each of g and u be off by up to E = 1e-2 (max-abs; the MFMA paths
    round every dequantised weight to FP16 once, and over K terms that error
    reaches a few FP16 steps of the output), which moves a by up to
    |silu'(g)| E |u| + |silu(g)| E, plus a's own rounding.  u (the up
    projection before the product) is recomputed from the oracle's last FFN
    input, rounded to FP16 like the oracle's."""
    E = 1e-2
    g = last["g"]
    u = orc.gemm(last["norm"].astype(np.float16), oblk.up).astype(np.float16).astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(-g))
    silu, dsilu = g * sig, sig * (1.0 + g * (1.0 - sig))
    return E * (np.abs(dsilu) * np.abs(u) + np.abs(silu)) + _fp16_ulps(last["u"])


def _check_scratch(views, last, rows, what, swiglu_bound=None):
    for k in ("norm", "qkv", "u", "y", "g"):
        if k not in last:
            continue
        got = views[k].float().cpu().numpy()[rows]
        if k == "u" and "g" in last:
            # The SwiGLU activation: rel-L2 as for the GEMMs, and each element
            # within max(1e-2, swiglu_bound) (the GEMM tolerance of its two
            # inputs carried through silu(g) u, plus its own rounding).
            assert swiglu_bound is not None, "gated scratch needs its SwiGLU bound"
            assert_close(got, last[k], f"{what} scratch {k}", max_abs=np.inf)
            err = np.abs(got - last[k])
            lim = np.maximum(1e-2, swiglu_bound[rows] if not isinstance(rows, slice)
                             else swiglu_bound)
            bad = np.argwhere(err > lim)
            assert bad.size == 0, (f"{what} scratch u: {len(bad)} elements beyond the SwiGLU bound, "
                                   f"first {tuple(bad[0])}: err {err[tuple(bad[0])]:.3e} "
                                   f"> {lim[tuple(bad[0])]:.3e}")
            continue
        assert_close(got, last[k], f"{what} scratch {k}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [1, 3, 16, 33])
def test_loop_small_block_full(orc, bits, M):
    D, F, L = 256, 640, 3
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=M)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, f"h bits={bits} M={M}")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, slice(None), f"bits={bits} M={M}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M", [2, 9, 16])
def test_loop_skinny_k_parts(orc, bits, M):
    """2 <= M <= 16 through the whole block with F = 4608: the down projection
    runs as three K parts and the split reduction with the residual epilogue."""
    D, F, L = 512, 4608, 2
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=40 + M)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, f"h bits={bits} M={M}")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, slice(None), f"bits={bits} M={M}")
    # one iteration per call gives the same bits
    split = inp.X.float().cuda()
    for l in range(L):
        qg.qg_loop_range(blk, split, l, l + 1, scratch)
    assert torch.equal(split, h)


@pytest.mark.parametrize("M,D", [(1, 256), (16, 256), (40, 256), (16, 1024), (40, 2048)])
def test_loop_empty_range_split_and_repeat(orc, M, D):
    """(D = 1024 and 2048 at M > 1: a call's first LayerNorm is a kernel of
    its own, the others come from the fused residual launches; the split
    must still give the same bits.)"""
    F = 512
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=11)
    h0 = inp.X.float().cuda()
    h = h0.clone()
    qg.qg_loop_range(blk, h, 5, 5)
    assert torch.equal(h, h0)
    full = h0.clone()
    qg.qg_loop_range(blk, full, 0, 4)
    split = h0.clone()
    qg.qg_loop_range(blk, split, 0, 1)
    qg.qg_loop_range(blk, split, 1, 3)
    qg.qg_loop_range(blk, split, 3, 4)
    assert torch.equal(full, split)
    again = h0.clone()
    qg.qg_loop_range(blk, again, 0, 4)
    assert torch.equal(full, again)
    assert not torch.equal(full, h0)


MEASURED = [
    # (name, bits, M, L): every row checked
    ("c2_int4_m1_l8", 4, 1, 8),
    ("c3_int4_m512_l8", 4, 512, 8),
    ("c4a_int2_m1_l16", 2, 1, 16),
    ("c4b_int2_m128_l8", 2, 128, 8),
    ("c5a_int4_m16_l32", 4, 16, 32),
    ("medium_int4_m64_l8", 4, 64, 8),
]


@pytest.mark.parametrize("name,bits,M,L", MEASURED, ids=[m[0] for m in MEASURED])
def test_loop_measured_workloads_all_rows(orc, name, bits, M, L):
    D, F = workloads.D_MODEL, workloads.D_FFN
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=0)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    h = h.cpu().numpy()
    assert np.all(np.isfinite(h))
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h, href, name)
    _check_scratch(qg.scratch_views(blk, M, scratch), last, slice(None), name)


@pytest.mark.parametrize("M", [1, 16, 40])
def test_loop_graph_replays_match_direct_enqueue(orc, M, monkeypatch):
    """The cached-graph path and the kernel-by-kernel path give the same bits;
    every replay is checked, with eager library work and syncs in between
    (D = 1024 at M > 1 takes the fused end-and-LayerNorm launches)."""
    D, F = (256, 512) if M == 1 else (1024, 1536)
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=21)
    h0 = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    monkeypatch.setenv("QG_LOOP_GRAPHS", "0")
    ref = h0.clone()
    qg.qg_loop_range(blk, ref, 0, 3, scratch)
    torch.cuda.synchronize()
    h = torch.empty_like(h0)
    for r in range(4):
        monkeypatch.setenv("QG_LOOP_GRAPHS", "1")
        h.copy_(h0)
        qg.qg_loop_range(blk, h, 0, 3, scratch)
        torch.cuda.synchronize()
        assert torch.equal(h, ref), f"graph replay {r} differs from direct enqueue"
        monkeypatch.setenv("QG_LOOP_GRAPHS", "0")
        other = h0.clone()
        qg.qg_loop_range(blk, other, 0, 1, scratch)   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,D,F", [(1, 256, 512), (16, 1024, 2048), (64, 1024, 1024)])
def test_loop_inside_caller_graph_capture(orc, M, D, F):
    """Under a caller's stream capture the kernels are recorded into the
    caller's graph; each replay must equal the eager result (D = 1024 at
    M > 1: the residual projections' fused end-and-LayerNorm launches)."""
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=22)
    h0 = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    ref = h0.clone()
    qg.qg_loop_range(blk, ref, 0, 2, scratch)
    h = h0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qg_loop_range(blk, h, 0, 2, scratch)
    for r in range(3):
        h.copy_(h0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, ref), f"captured replay {r}"
        tmp = h0.clone()
        qg.qg_loop_range(blk, tmp, 0, 1, scratch)
        torch.cuda.synchronize()


# SwiGLU blocks (a gate weight): every kernel family takes the gate-multiply
# epilogue -- GEMV (M=1), skinny (M=3, 16), staged tiled (M=33), ring (M=300),
# and the split reduction (D=4096: skinny K parts at M=5, tiled K split at
# M=20).
# M = 1 at D = 512 (no fused LayerNorm), 4096 and 8192 runs the
# gate and up projections as one SwiGLU pair launch (1, 2 and 4 lane chunks
# per row for INT4).
GATED = [(1, 256, 640), (3, 256, 640), (16, 256, 640), (33, 256, 640), (300, 2048, 8192),
         (5, 4096, 256), (20, 4096, 256), (1, 512, 1152), (1, 4096, 384), (1, 8192, 128)]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,D,F", GATED)
def test_loop_gated_block(orc, bits, M, D, F):
    L = 2
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=M + D, gated=True)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    rows = slice(None)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    h = h.cpu().numpy()
    assert np.all(np.isfinite(h))
    _check_h(h[rows], href, f"gated h bits={bits} M={M} D={D}")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, rows, f"gated bits={bits} M={M}",
                   _swiglu_bound(orc, oblk, last))


@pytest.mark.parametrize("M,L", [(1, 8), (16, 4), (512, 8)])
def test_loop_gated_measured_block_all_rows(orc, M, L):
    """The pages' five-weight block at D=2048, F=8192 (INT4), every row."""
    D, F = workloads.D_MODEL, workloads.D_FFN
    inp, blk, oblk = _blocks(orc, M, 4, D, F, seed=0, gated=True)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, f"gated measured M={M}")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, slice(None), f"gated measured M={M}",
                   _swiglu_bound(orc, oblk, last))


def test_loop_gated_graph_replays_match_direct_enqueue(orc, monkeypatch):
    D, F, M = 256, 512, 1
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=23, gated=True)
    h0 = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    monkeypatch.setenv("QG_LOOP_GRAPHS", "0")
    ref = h0.clone()
    qg.qg_loop_range(blk, ref, 0, 3, scratch)
    torch.cuda.synchronize()
    h = torch.empty_like(h0)
    for r in range(3):
        monkeypatch.setenv("QG_LOOP_GRAPHS", "1")
        h.copy_(h0)
        qg.qg_loop_range(blk, h, 0, 3, scratch)
        torch.cuda.synchronize()
        assert torch.equal(h, ref), f"graph replay {r}"
        monkeypatch.setenv("QG_LOOP_GRAPHS", "0")
        qg.qg_loop_range(blk, h0.clone(), 0, 1, scratch)
        torch.cuda.synchronize()


# The SwiGLU pair launch (gate and up in one M = 1 GEMV) computes exactly what
# the separate gate GEMV and gate-multiply up GEMV compute: same lanes, same
# reduction order, same FP32 silu.  INT2 at D = 512 has no GEMV shape, so it
# stays on the separate path on both sides.
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("D,F", [(512, 1152), (1024, 2944), (2048, 8192), (4096, 384),
                                 (8192, 128)])
def test_loop_swiglu_pair_matches_separate_launches(orc, monkeypatch, bits, D, F):
    M, L = 1, 3
    inp, blk, _ = _blocks(orc, M, bits, D, F, seed=D + F, gated=True)
    h0 = inp.X.float().cuda()
    out = {}
    for fuse in ("1", "0"):
        monkeypatch.setenv("QG_FUSE_SWIGLU", fuse)
        h = h0.clone()
        scratch = qg.alloc_loop_scratch(blk, M)
        qg.qg_loop_range(blk, h, 0, L, scratch)
        torch.cuda.synchronize()
        v = qg.scratch_views(blk, M, scratch)
        out[fuse] = (h.cpu(), v["g"].cpu(), v["u"].cpu(), v["norm"].cpu())
    for name, a, b in zip(("h", "g", "u", "norm"), out["1"], out["0"]):
        assert torch.equal(a, b), f"bits={bits} D={D} F={F}: {name} differs between the pair " \
                                  f"launch and the separate launches"


def test_loop_gated_mixed_bits_block(orc):
    """A gate in INT4 with the rest in INT2 (not a SwiGLU pair: the bits
    differ) at M = 1, against the oracle."""
    D, F, M, L = 2048, 1024, 1, 2
    inp = workloads.block(M, seed=5, D=D, F=F, gated=True)
    ws = {k: qg.qg_pack(v.cuda(), 4 if k == "gate" else 2) for k, v in inp.W.items()}
    blk = qg.Block(D, F, ws["qkv"], ws["out"], ws["up"], ws["down"], ws["gate"])
    ow = {k: orc.pack(v.numpy(), 4 if k == "gate" else 2) for k, v in inp.W.items()}
    oblk = orc.Block(D, F, ow["qkv"], ow["out"], ow["up"], ow["down"], ow["gate"])
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, "mixed-bits gated h")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, slice(None), "mixed-bits gated",
                   _swiglu_bound(orc, oblk, last))


def test_loop_graph_cache_from_threads(orc, monkeypatch):
    """Four threads run the loop on 48 distinct residual/scratch pairs (48
    cached graphs, more than the cache holds, so evictions interleave with
    other threads' lookups and launches); every result equals the direct
    enqueue of the same call."""
    import threading
    D, F, M, L = 256, 512, 1, 2
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=77)
    h0 = inp.X.float().cuda()
    monkeypatch.setenv("QG_LOOP_GRAPHS", "0")
    ref_s = qg.alloc_loop_scratch(blk, M)
    ref = h0.clone()
    qg.qg_loop_range(blk, ref, 0, L, ref_s)
    torch.cuda.synchronize()
    monkeypatch.setenv("QG_LOOP_GRAPHS", "1")
    hs = [h0.clone() for _ in range(48)]
    scratches = [qg.alloc_loop_scratch(blk, M) for _ in range(48)]
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            for i in range(t, 48, 4):
                qg.qg_loop_range(blk, hs[i], 0, L, scratches[i])
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, h in enumerate(hs):
        assert torch.equal(h, ref), f"call {i}"


@pytest.mark.parametrize("M", [1, 16])
def test_loop_after_release_cache(orc, M):
    """qg_release_cache frees the cached graphs and their capture streams; the
    next call captures again and gives the same bits (twice in a row, so a
    release with nothing cached is harmless too)."""
    D, F = 256, 640
    inp, blk, _ = _blocks(orc, M, 4, D, F, seed=31)
    h0 = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    first = h0.clone()
    qg.qg_loop_range(blk, first, 0, 3, scratch)
    for _ in range(2):
        qg.qg_release_cache()
        again = h0.clone()
        qg.qg_loop_range(blk, again, 0, 3, scratch)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


@pytest.mark.parametrize("D,F", [(1024, 256), (2048, 256), (4096, 384), (8192, 256), (384, 256)])
def test_loop_layernorm_widths(orc, D, F):
    """The LayerNorm kernel of M > 1 at every row width it has a vectorised
    variant for (D = 1024 .. 8192) and at an element-strided one (D = 384):
    the block at M = 3 against the oracle, h and the last iteration's scratch
    (its norm is the LayerNorm kernel's output)."""
    M, L = 3, 2
    inp, blk, oblk = _blocks(orc, M, 4, D, F, seed=D + F)
    h = inp.X.float().cuda()
    scratch = qg.alloc_loop_scratch(blk, M)
    qg.qg_loop_range(blk, h, 0, L, scratch)
    href, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, f"LN width D={D}")
    _check_scratch(qg.scratch_views(blk, M, scratch), last, list(range(M)), f"LN width D={D}")


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("M,D,F,gated", [(2, 1024, 2304, False), (16, 2048, 8192, False),
                                         (16, 1024, 4096, True), (33, 1024, 1152, False),
                                         (64, 2048, 8192, False), (128, 1024, 2048, True),
                                         (300, 2048, 1024, False), (5, 4096, 512, False),
                                         (3, 8192, 256, False)])
def test_loop_fused_residual_layernorm_matches_separate_launches(orc, monkeypatch, bits, M, D, F,
                                                                 gated):
    """At M > 1 the residual projections write K-part partials and one launch
    sums them, adds into h and computes the next LayerNorm.  It must give the
    same bits as the split-K reduction of the same partials followed by the
    LayerNorm kernel (QG_FUSE_REDUCE_LN=0): h and every scratch region, over
    several iterations (skinny with one and several K parts, ring tiles with
    and without a K split, INT4 and INT2, plain and gated)."""
    inp, blk, _ = _blocks(orc, M, bits, D, F, seed=M + D + F + bits, gated=gated)
    scratch = qg.alloc_loop_scratch(blk, M)
    out = {}
    for fuse in ("0", "1"):
        monkeypatch.setenv("QG_FUSE_REDUCE_LN", fuse)
        h = inp.X.float().cuda()
        qg.qg_loop_range(blk, h, 0, 3, scratch)
        torch.cuda.synchronize()
        out[fuse] = (h.clone(), {k: v.clone() for k, v in qg.scratch_views(blk, M, scratch).items()})
    assert torch.equal(out["0"][0], out["1"][0])
    for k in out["0"][1]:
        assert torch.equal(out["0"][1][k], out["1"][1][k]), k
