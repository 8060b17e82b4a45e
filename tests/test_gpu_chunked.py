"""Chunked prefill and the FP16-h cache ("Model" page, Chunked prefill;
Parameters: prefill_chunk).

qg_loop_range_chunked runs the rows of h chunk by chunk, each chunk through
all iterations before the next, with a scratch sized for one chunk.  Checked:
every row against the FP64 oracle (M = 2048 in chunks of 512, and a ragged
M = 1100); bit for bit against qg_loop_range on each chunk's rows; against the
single-shot M = 2048 loop within the loop tolerance (their tile plans differ:
at M = 512 the down projection splits K in two, at M = 2048 it does not, so
the FP32 sums are ordered differently), and bit for bit where the chunk's
plans equal the single shot's (2 <= M <= 16, the skinny kernel, whose
per-row arithmetic does not depend on M).

The FP16-h cache holds each iteration's attention input x; the pages' h-mode
rebuilds K = W_k x (and V = W_v x) from it.  Here qg_gemm on the K and V rows
of the QKV weight (a view of output channels [D, 2D) and [2D, 3D)) rebuilds
the last iteration's K and V columns of qkv bit for bit (the pages: the
reconstruction is exact), and matches the oracle's qkv within the GEMM
tolerance."""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_close

qg = pytest.importorskip("int2_quantized_gemm_amd")
pytestmark = pytest.mark.gpu


def _blocks(orc, M, bits, D, F, seed):
    inp = workloads.block(M, seed=seed, D=D, F=F)
    blk = qg.pack_block(inp.W, bits, D, F)
    oblk = orc.pack_block({k: v.numpy() for k, v in inp.W.items()}, bits, D, F)
    return inp, blk, oblk


def _check_h(h, href, what):
    rms = float(np.sqrt(np.mean(href ** 2)))
    assert_close(h, href, what, max_abs=1e-2 * max(1.0, rms))


@pytest.mark.parametrize("M,chunk,L", [(2048, 512, 2), (1100, 512, 3)])
def test_chunked_prefill_all_rows(orc, M, chunk, L):
    D, F = workloads.D_MODEL, workloads.D_FFN
    inp, blk, oblk = _blocks(orc, M, 4, D, F, seed=0)
    h0 = inp.X.float().cuda()
    h = h0.clone()
    need = qg.qg_loop_chunked_scratch_bytes(blk, M, chunk)
    assert need < qg.qg_loop_scratch_bytes(blk, M)  # the point of the chunked path
    scratch = torch.empty(need, dtype=torch.uint8, device="cuda")
    qg.qg_loop_range_chunked(blk, h, 0, L, chunk, scratch)
    # bit for bit: qg_loop_range on each chunk's rows, in the same scratch
    manual = h0.clone()
    for r0 in range(0, M, chunk):
        part = manual[r0:r0 + chunk]
        qg.qg_loop_range(blk, part, 0, L, scratch)
    assert torch.equal(h, manual)
    href, _ = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    hc = h.cpu().numpy()
    _check_h(hc, href, f"chunked M={M} chunk={chunk}")
    # single shot: the same rows within the loop tolerance of each other and
    # of the oracle
    single = h0.clone()
    qg.qg_loop_range(blk, single, 0, L)
    _check_h(single.cpu().numpy(), href, f"single shot M={M}")
    _check_h(hc, single.cpu().numpy().astype(np.float64), f"chunked vs single shot M={M}")


@pytest.mark.parametrize("M,chunk", [(16, 8), (12, 5), (9, 3)])
@pytest.mark.parametrize("bits", [4, 2])
def test_chunked_bit_exact_where_plans_match(orc, M, chunk, bits):
    """2 <= M <= 16 runs the skinny kernels, whose per-row results do not
    depend on M: chunked and single shot agree bit for bit."""
    D, F, L = 1024, 4096, 3
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=M + chunk)
    h0 = inp.X.float().cuda()
    single = h0.clone()
    qg.qg_loop_range(blk, single, 0, L)
    h = h0.clone()
    qg.qg_loop_range_chunked(blk, h, 0, L, chunk)
    assert torch.equal(h, single)
    href, _ = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    _check_h(h.cpu().numpy(), href, f"chunked skinny M={M}")


# (M, chunk, exact): the rebuild of a chunk's K and V runs qg_gemm on that
# chunk's cached rows.  It reproduces the loop's QKV columns bit for bit where
# the GEMM on the K (or V) rows alone takes the same K split as the QKV GEMM:
# M = 1 (the GEMV: per-row arithmetic independent of N), M = 16 (the skinny
# kernel, one K part for K = 2048 either way) and M = 512 (no split for
# either); at M = 256 and 188 the 2048-channel GEMM splits K in two parts
# where the 6144-channel one does not, so its FP32 sums are ordered
# differently and only the tolerance holds.
HCACHE = [(1, 1, True), (16, 16, True), (512, 512, True), (700, 256, False)]


@pytest.mark.parametrize("M,chunk,exact", HCACHE)
@pytest.mark.parametrize("bits", [4, 2])
def test_hcache_rebuilds_k_and_v(orc, M, chunk, exact, bits):
    D, F, L = workloads.D_MODEL, workloads.D_FFN, 2
    inp, blk, oblk = _blocks(orc, M, bits, D, F, seed=M + 3)
    h = inp.X.float().cuda()
    hcache = torch.full((L, M, D), float("nan"), dtype=torch.float16, device="cuda")
    scratch = torch.empty(qg.qg_loop_chunked_scratch_bytes(blk, M, chunk), dtype=torch.uint8,
                          device="cuda")
    qg.qg_loop_range_chunked(blk, h, 0, L, chunk, scratch, hcache=hcache)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(hcache).all()), "every row of every iteration written"
    gemm = qg.qg_gemm_int4 if bits == 4 else qg.qg_gemm_int2
    Wk, Wv = blk.qkv.rows(D, 2 * D), blk.qkv.rows(2 * D, 3 * D)
    # rebuild chunk by chunk, as the cache would be read
    K = torch.cat([gemm(hcache[L - 1, r0:r0 + chunk].contiguous(), Wk) for r0 in range(0, M, chunk)])
    V = torch.cat([gemm(hcache[L - 1, r0:r0 + chunk].contiguous(), Wv) for r0 in range(0, M, chunk)])
    # the scratch holds the last chunk's qkv
    r0 = (M - 1) // chunk * chunk
    qkv = qg.scratch_views(blk, M - r0, scratch)["qkv"]
    if exact:
        assert torch.equal(K[r0:], qkv[:, D:2 * D]), "K = W_k x rebuilt bit for bit"
        assert torch.equal(V[r0:], qkv[:, 2 * D:]), "V = W_v x rebuilt bit for bit"
    else:
        assert_close(K[r0:].float().cpu().numpy(), qkv[:, D:2 * D].float().cpu().numpy(), "K vs qkv")
        assert_close(V[r0:].float().cpu().numpy(), qkv[:, 2 * D:].float().cpu().numpy(), "V vs qkv")
    # and against the oracle's last iteration, every row
    _, last = orc.loop_range(oblk, inp.X.numpy().astype(np.float64), 0, L)
    assert_close(K.float().cpu().numpy(), last["qkv"][:, D:2 * D], f"K rebuilt M={M}")
    assert_close(V.float().cpu().numpy(), last["qkv"][:, 2 * D:], f"V rebuilt M={M}")
