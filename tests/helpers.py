"""Shared helpers of the GPU parity tests: conversions between the binding's
torch tensors and the oracle's numpy arrays, and the tolerance checks.

Tolerances (from the GEMM contract): relative L2 error <= 2e-3 and max
absolute error <= 1e-2 against the FP64 oracle.  For the FP32 residual of the
loop block the max-abs bound scales with max(1, rms(h_ref)), since h grows
with every iteration.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 2e-3
MAX_ABS = 1e-2


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    return float(np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-30))


def assert_close(a, ref, what: str, max_abs: float = MAX_ABS, rel: float = REL_L2):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert a.shape == ref.shape, (what, a.shape, ref.shape)
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    e = rel_l2(a, ref)
    m = float(np.abs(a - ref).max()) if a.size else 0.0
    assert e <= rel and m <= max_abs, f"{what}: rel-L2 {e:.3e} (<= {rel}), max-abs {m:.3e} (<= {max_abs})"
    return e, m


def compact_codes(p) -> np.ndarray:
    """The codes of a PackedWeight as compact uint32 rows [N][K*bits/32]
    (rows kept at a larger stride give their first K*bits/32 words)."""
    return np.ascontiguousarray(p.codes[:, :p.K * p.bits // 32].cpu().numpy().view(np.uint32))


def to_oracle(p, orc):
    """PackedWeight (GPU) -> oracle.Packed, for comparisons of outputs only."""
    return orc.Packed(p.bits, p.K, p.N, compact_codes(p),
                      p.scales.cpu().numpy().view(np.uint16).copy(),
                      p.zeros.cpu().numpy().view(np.uint16).copy())


def to_gpu(op, qg, device="cuda"):
    """oracle.Packed -> PackedWeight on the GPU (hand-built test weights)."""
    return qg.PackedWeight(op.bits, op.K, op.N,
                           torch.from_numpy(op.codes.view(np.int32).copy()).to(device),
                           torch.from_numpy(op.scales.view(np.float16).copy()).to(device),
                           torch.from_numpy(op.zeros.view(np.float16).copy()).to(device))


def f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint16)


class Guarded:
    """A 2-D FP16 output view [rows][cols] with leading dimension ld inside a
    larger buffer filled with a canary pattern, to catch out-of-bounds writes."""
    CANARY = 0x7BAD  # a finite FP16 value no kernel produces here by accident

    def __init__(self, rows: int, cols: int, ld: int, device="cuda", pad: int = 4096):
        self.rows, self.cols, self.ld, self.pad = rows, cols, ld, pad
        n = pad + max(rows, 1) * ld + pad
        self.buf = torch.full((n,), self.CANARY, dtype=torch.int16, device=device)
        self.view = self.buf[pad:pad + rows * ld].view(torch.float16).view(rows, ld)[:, :cols] \
            if rows else self.buf[pad:pad].view(torch.float16).view(0, cols)

    def check(self):
        b = self.buf.cpu().numpy().view(np.uint16)
        assert np.all(b[:self.pad] == self.CANARY), "write before the output"
        assert np.all(b[self.pad + self.rows * self.ld:] == self.CANARY), "write after the output"
        if self.ld > self.cols and self.rows:
            body = b[self.pad:self.pad + self.rows * self.ld].reshape(self.rows, self.ld)
            assert np.all(body[:, self.cols:] == self.CANARY), "write into the row padding"
