"""Guard bands around the loop's buffers: the residual h, the loop scratch
and the chunked driver's FP16-h cache each sit inside a larger buffer whose
margins hold a canary pattern, and after the loop every margin must still
hold it (no launch of the loop writes outside the buffers it was given).
The loop's results on the guarded views must equal, bit for bit, those on
plainly allocated buffers."""
from __future__ import annotations

import pytest
import torch

import int2_quantized_gemm_amd as qg
import workloads

pytestmark = pytest.mark.gpu

PAD = 64 * 1024           # bytes of margin on each side (a multiple of 256)
H_CANARY = 0x7FC0DEAD     # a quiet-NaN FP32 pattern, never a loop result
S_CANARY = 0xA5           # scratch margin bytes
C_CANARY = 0x7BAD         # FP16 cache margin (finite, no result here by accident)


class _Band:
    """A `nbytes` view inside a byte buffer with PAD canary bytes on each side."""

    def __init__(self, nbytes: int, fill_word: int, word_bytes: int):
        n_words = (2 * PAD + nbytes + word_bytes - 1) // word_bytes
        dt = {4: torch.int32, 2: torch.int16, 1: torch.uint8}[word_bytes]
        w = fill_word - (1 << (8 * word_bytes)) if word_bytes > 1 and fill_word >= 1 << (8 * word_bytes - 1) \
            else fill_word
        self.buf = torch.full((n_words,), w, dtype=dt, device="cuda").view(torch.uint8)
        self.nbytes = nbytes
        self.ref = self.buf[:PAD].clone()

    def inner(self) -> torch.Tensor:
        return self.buf[PAD:PAD + self.nbytes]

    def check(self, what: str):
        b = self.buf
        assert torch.equal(b[:PAD], self.ref), f"{what}: write before the buffer"
        tail = b[PAD + self.nbytes:PAD + self.nbytes + PAD]
        assert torch.equal(tail, self.ref[:tail.numel()]), f"{what}: write after the buffer"


def _run(blk, M, L, h0, chunk=None, hcache_rows=False):
    """The loop on guarded h / scratch (/ hcache) and on plain buffers; checks
    the margins and returns both results."""
    D = blk.D
    hb = _Band(M * D * 4, H_CANARY, 4)
    h = hb.inner().view(torch.float32).view(M, D)
    h.copy_(h0)
    if chunk is None:
        nbytes = max(qg.qg_loop_scratch_bytes(blk, M), 256)
    else:
        nbytes = max(qg.qg_loop_chunked_scratch_bytes(blk, M, chunk), 256)
    sb = _Band(nbytes, S_CANARY, 1)
    cb = _Band(L * M * D * 2, C_CANARY, 2) if hcache_rows else None
    hc = cb.inner().view(torch.float16).view(L, M, D) if cb else None
    if chunk is None:
        qg.qg_loop_range(blk, h, 0, L, sb.inner())
    else:
        qg.qg_loop_range_chunked(blk, h, 0, L, chunk, sb.inner(), hcache=hc)
    torch.cuda.synchronize()
    hb.check("h")
    sb.check("scratch")
    if cb:
        cb.check("hcache")
    # the same call on plainly allocated buffers
    h2 = h0.clone()
    if chunk is None:
        qg.qg_loop_range(blk, h2, 0, L, qg.alloc_loop_scratch(blk, M))
    else:
        hc2 = torch.empty((L, M, D), dtype=torch.float16, device="cuda") if cb else None
        qg.qg_loop_range_chunked(blk, h2, 0, L, chunk,
                                 torch.empty(nbytes, dtype=torch.uint8, device="cuda"), hcache=hc2)
        if cb:
            assert torch.equal(hc.view(torch.int16), hc2.view(torch.int16)), "hcache differs"
    torch.cuda.synchronize()
    assert torch.equal(h, h2), "guarded and plain buffers give different h"


# (M, bits, D, F, L, gated): the measured block at every kernel family's M
# (GEMV, skinny with K parts, 32-, 64- and 128-row ring tiles), ragged M, a
# small block (LayerNorm kernel widths, staged GEMM), and gated blocks.
CASES = [(1, 4, 2048, 8192, 2, False), (1, 2, 2048, 8192, 2, False), (5, 4, 2048, 8192, 2, False),
         (16, 4, 2048, 8192, 2, False), (40, 2, 2048, 8192, 2, False), (128, 2, 2048, 8192, 1, False),
         (300, 4, 2048, 8192, 1, False), (512, 4, 2048, 8192, 1, False), (1024, 4, 2048, 8192, 1, False),
         (3, 4, 640, 1280, 3, False), (77, 2, 640, 1280, 3, False),
         (1, 4, 2048, 8192, 2, True), (33, 4, 1024, 2048, 2, True)]


@pytest.mark.parametrize("M,bits,D,F,L,gated", CASES)
def test_loop_writes_stay_inside_h_and_scratch(M, bits, D, F, L, gated):
    print(f"guards: M={M} bits={bits} D={D} F={F} L={L} gated={gated}", flush=True)
    inp = workloads.block(M, seed=M + D + bits, D=D, F=F, gated=gated)
    blk = qg.pack_block(inp.W, bits, D, F)
    _run(blk, M, L, inp.X.float().cuda())


@pytest.mark.parametrize("M,chunk,bits", [(700, 256, 4), (20, 16, 2), (1, 1, 4)])
def test_chunked_loop_writes_stay_inside_h_scratch_and_cache(M, chunk, bits):
    print(f"guards chunked: M={M} chunk={chunk} bits={bits}", flush=True)
    inp = workloads.block(M, seed=M + chunk)
    blk = qg.pack_block(inp.W, bits, workloads.D_MODEL, workloads.D_FFN)
    _run(blk, M, 2, inp.X.float().cuda(), chunk=chunk, hcache_rows=True)
