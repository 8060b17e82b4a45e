"""Python binding of libqgemm.so, the MI355X (gfx950) weight-only INT4/INT2
quantised GEMM library (C ABI in include/qgemm.h).

Argument marshalling only: every function here takes torch tensors that live
on the GPU, passes their device pointers and the current HIP stream to the
C entry point of the same name, and raises on a non-zero status.  No step of
the computation runs in Python, and there is no CPU fallback: importing the
package fails loudly when the compiled library is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QG_LIBRARY names another build of the same library to load instead of the
# in-tree one (the host AddressSanitizer build of the CPU test suite); like
# the in-tree library, it must exist: there is no fallback.
LIB_PATH = os.environ.get("QG_LIBRARY") or os.path.join(_HERE, "libqgemm.so")

QG_OK, QG_EINVAL, QG_EUNSUPPORTED, QG_ENOMEM, QG_EHIP = 0, -1, -2, -3, -4
GROUP = 128


class QGError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class QGValueError(QGError, ValueError):
    pass


class _Weight(C.Structure):
    _fields_ = [("bits", C.c_int32), ("K", C.c_int32), ("N", C.c_int32), ("group", C.c_int32),
                ("codes", C.c_void_p), ("scales", C.c_void_p), ("zeros", C.c_void_p),
                ("ldc", C.c_int64)]


class _Block(C.Structure):
    _fields_ = [("D", C.c_int32), ("F", C.c_int32),
                ("qkv", _Weight), ("out", _Weight), ("up", _Weight), ("down", _Weight),
                ("gate", _Weight)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
            f"g.build()'` (hipcc, gfx950).  There is no fallback implementation.")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    W, B = C.POINTER(_Weight), C.POINTER(_Block)
    sig = {
        "qg_abi_version": (C.c_int, []),
        "qg_layout_version": (C.c_int, []),
        "qg_last_error": (C.c_char_p, []),
        "qg_pack": (C.c_int, [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp]),
        "qg_gemm_int4": (C.c_int, [vp, i64, W, vp, i64, i32, vp, sz, vp]),
        "qg_gemm_int2": (C.c_int, [vp, i64, W, vp, i64, i32, vp, sz, vp]),
        "qg_gemm_ws_bytes": (sz, [W, i32]),
        "qg_gemm_static_ws": (C.c_int, [vp, i64, W, vp, i64, i32, vp]),
        "qg_loop_range": (C.c_int, [B, vp, i32, i32, i32, vp, sz, vp]),
        "qg_loop_scratch_bytes": (sz, [B, i32]),
        "qg_loop_range_chunked": (C.c_int, [B, vp, i32, i32, i32, i32, vp, sz, vp, vp]),
        "qg_loop_chunked_scratch_bytes": (sz, [B, i32, i32]),
        "qg_loop_scratch_offsets": (C.c_int, [B, i32, C.POINTER(sz), C.POINTER(sz),
                                              C.POINTER(sz),
                                              C.POINTER(sz), C.POINTER(sz)]),
        "qg_unpack": (C.c_int, [W, vp, vp]),
        "qg_dequant": (C.c_int, [W, i32, vp, vp]),
        "qg_requant_4to2": (C.c_int, [W, W, vp]),
        "qg_release_cache": (None, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(fn: str, status: int):
    if status != QG_OK:
        msg = lib.qg_last_error().decode()
        cls = QGValueError if status in (QG_EINVAL, QG_EUNSUPPORTED) else QGError
        raise cls(fn, status, msg)


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.data_ptr()


def qg_abi_version() -> int:
    return lib.qg_abi_version()


def qg_layout_version() -> int:
    return lib.qg_layout_version()


def qg_last_error() -> str:
    return lib.qg_last_error().decode()


@dataclass
class PackedWeight:
    """Layout-v1 packed weight: codes int32 [N][>= K*bits/32] (uint32 bit
    patterns; each row's first K*bits/32 words hold its codes, rows
    codes.stride(0) words apart -- more than K*bits/32 for INT2 rows kept at
    the INT4 stride), scales/zeros float16 [N][K/group]; group 128, or K for
    per-row groups (one scale and zero per output channel)."""
    bits: int
    K: int
    N: int
    codes: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor
    group: int = GROUP

    def cstruct(self) -> _Weight:
        # the C side sees only pointers: the tensors must hold what bits, K,
        # N and group say
        words = self.K * self.bits // 32
        if (self.codes.dim() != 2 or self.codes.shape[0] != self.N or self.codes.shape[1] < words
                or self.codes.element_size() != 4 or self.codes.stride(1) != 1
                or self.codes.stride(0) < words):
            raise ValueError(f"codes must be a 32-bit [{self.N}][>= {words}] tensor with unit column "
                             f"stride, got {tuple(self.codes.shape)} {self.codes.dtype} strides "
                             f"{self.codes.stride()}")
        groups = self.K // self.group if self.group else 0
        for name, t in (("scales", self.scales), ("zeros", self.zeros)):
            if (tuple(t.shape) != (self.N, groups) or t.dtype != torch.float16
                    or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous FP16 [{self.N}][{groups}] tensor, "
                                 f"got {tuple(t.shape)} {t.dtype}")
        ldc = self.codes.stride(0) if self.N > 1 else words
        return _Weight(self.bits, self.K, self.N, self.group, self.codes.data_ptr(),
                       self.scales.data_ptr(), self.zeros.data_ptr(), 0 if ldc == words else ldc)

    @staticmethod
    def empty(K: int, N: int, bits: int, device="cuda", group: int = GROUP) -> "PackedWeight":
        if group not in (GROUP, K) or K % GROUP:
            raise ValueError(f"group = {group}: layout v1 has groups of {GROUP} or per-row "
                             f"groups (group = K = {K}), K a multiple of {GROUP}")
        return PackedWeight(bits, K, N,
                            torch.empty((N, K * bits // 32), dtype=torch.int32, device=device),
                            torch.empty((N, K // group), dtype=torch.float16, device=device),
                            torch.empty((N, K // group), dtype=torch.float16, device=device),
                            group)

    def nbytes(self) -> int:
        """Bytes the weight holds: its codes (K*bits/8 a row, row padding not
        counted), scales and zeros."""
        return (self.N * self.K * self.bits // 8
                + sum(t.numel() * t.element_size() for t in (self.scales, self.zeros)))

    def rows(self, n0: int, n1: int) -> "PackedWeight":
        """Output channels [n0, n1) as a weight of their own: the N-major codes,
        scales and zeros of a channel range are contiguous row ranges, so this
        is a view (no copy); e.g. the K rows [D, 2D) of a QKV weight."""
        if not 0 <= n0 < n1 <= self.N:
            raise ValueError(f"rows [{n0}, {n1}) outside [0, {self.N})")
        return PackedWeight(self.bits, self.K, n1 - n0, self.codes[n0:n1], self.scales[n0:n1],
                            self.zeros[n0:n1], self.group)


def qg_pack(W: torch.Tensor, bits: int, group: int = GROUP, out: PackedWeight | None = None,
            stream=None) -> PackedWeight:
    """Quantise FP32 W [K][N] (GPU) into layout v1: a validation pass (which
    synchronises the stream and raises, with nothing written, on non-finite W
    or an overflowing scale), then the packing, enqueued on the stream."""
    if W.dtype != torch.float32 or W.dim() != 2 or W.stride(1) != 1:
        raise ValueError("W must be a row-major FP32 [K][N] tensor")
    K, N = W.shape
    if out is not None and out.group != group:
        raise ValueError(f"out.group = {out.group} but group = {group}")
    p = out if out is not None else PackedWeight.empty(K, N, bits, W.device, group)
    _check("qg_pack", lib.qg_pack(_dev(W, "W"), W.stride(0), K, N, bits, group, p.codes.data_ptr(),
                                  p.scales.data_ptr(), p.zeros.data_ptr(), _stream(stream)))
    return p


def qg_gemm_ws_bytes(w: PackedWeight, M: int) -> int:
    ws = w.cstruct()
    return lib.qg_gemm_ws_bytes(C.byref(ws), M)


def _gemm(fn, name, X, w, Y, ws, stream):
    if X.dim() != 2 or X.shape[1] != w.K:
        raise ValueError(f"X must be [M][{w.K}], got {tuple(X.shape)}")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.float16, device=X.device)
    if Y.dim() != 2 or tuple(Y.shape) != (M, w.N):
        raise ValueError(f"Y must be [{M}][{w.N}], got {tuple(Y.shape)}")
    if X.dtype != torch.float16 or Y.dtype != torch.float16 or X.stride(1) != 1 or Y.stride(1) != 1:
        raise ValueError("X and Y must be row-major FP16 tensors")
    need = qg_gemm_ws_bytes(w, M)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_ptr, ws_bytes = (ws.data_ptr(), ws.numel() * ws.element_size()) if ws is not None else (None, 0)
    cw = w.cstruct()
    _check(name, fn(_dev(X, "X"), X.stride(0), C.byref(cw), _dev(Y, "Y"), Y.stride(0), M, ws_ptr,
                    ws_bytes, _stream(stream)))
    return Y


def qg_gemm_int4(X: torch.Tensor, w: PackedWeight, Y: torch.Tensor | None = None, ws=None,
                 stream=None) -> torch.Tensor:
    """Y[M][N] = X[M][K] . dequant(w), FP16 in/out, FP32 accumulation."""
    return _gemm(lib.qg_gemm_int4, "qg_gemm_int4", X, w, Y, ws, stream)


def qg_gemm_int2(X: torch.Tensor, w: PackedWeight, Y: torch.Tensor | None = None, ws=None,
                 stream=None) -> torch.Tensor:
    """Y[M][N] = X[M][K] . dequant(w) for 2-bit w, FP16 in/out, FP32 accumulation."""
    return _gemm(lib.qg_gemm_int2, "qg_gemm_int2", X, w, Y, ws, stream)


def qg_gemm_static_ws(X: torch.Tensor, w: PackedWeight, Y: torch.Tensor | None = None,
                      stream=None) -> torch.Tensor:
    """qg_gemm_int4 / qg_gemm_int2 (by w.bits) on the library's static device
    workspace: allocates nothing when Y is given."""
    if X.dim() != 2 or X.shape[1] != w.K:
        raise ValueError(f"X must be [M][{w.K}], got {tuple(X.shape)}")
    M = X.shape[0]
    if Y is None:
        Y = torch.empty((M, w.N), dtype=torch.float16, device=X.device)
    if Y.dim() != 2 or tuple(Y.shape) != (M, w.N):
        raise ValueError(f"Y must be [{M}][{w.N}], got {tuple(Y.shape)}")
    if X.dtype != torch.float16 or Y.dtype != torch.float16 or X.stride(1) != 1 or Y.stride(1) != 1:
        raise ValueError("X and Y must be row-major FP16 tensors")
    cw = w.cstruct()
    _check("qg_gemm_static_ws", lib.qg_gemm_static_ws(_dev(X, "X"), X.stride(0), C.byref(cw),
                                                      _dev(Y, "Y"), Y.stride(0), M,
                                                      _stream(stream)))
    return Y


@dataclass
class Block:
    """The loop block's packed projections; gate None means four projections
    and the identity FFN activation, otherwise the FFN is SwiGLU."""
    D: int
    F: int
    qkv: PackedWeight
    out: PackedWeight
    up: PackedWeight
    down: PackedWeight
    gate: PackedWeight | None = None

    def weights(self) -> dict:
        ws = {"qkv": self.qkv, "out": self.out, "up": self.up, "down": self.down}
        if self.gate is not None:
            ws["gate"] = self.gate
        return ws

    def cstruct(self) -> _Block:
        gate = self.gate.cstruct() if self.gate is not None else _Weight(0, 0, 0, 0, None, None,
                                                                           None)
        return _Block(self.D, self.F, self.qkv.cstruct(), self.out.cstruct(), self.up.cstruct(),
                      self.down.cstruct(), gate)

    def nbytes(self) -> int:
        return sum(w.nbytes() for w in self.weights().values())


def qg_loop_scratch_bytes(blk: Block, M: int) -> int:
    b = blk.cstruct()
    return lib.qg_loop_scratch_bytes(C.byref(b), M)


def qg_loop_scratch_offsets(blk: Block, M: int) -> dict:
    b = blk.cstruct()
    vals = [C.c_size_t() for _ in range(5)]
    _check("qg_loop_scratch_offsets",
           lib.qg_loop_scratch_offsets(C.byref(b), M, *(C.byref(v) for v in vals)))
    return dict(zip(("norm", "qkv", "u", "y", "g"), (v.value for v in vals)))


def alloc_loop_scratch(blk: Block, M: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(qg_loop_scratch_bytes(blk, M), 256), dtype=torch.uint8, device=device)


def scratch_views(blk: Block, M: int, scratch: torch.Tensor) -> dict:
    """FP16 views of the last iteration's intermediates inside a loop scratch."""
    off = qg_loop_scratch_offsets(blk, M)
    shapes = {"norm": (M, blk.D), "qkv": (M, 3 * blk.D), "u": (M, blk.F), "y": (M, blk.D)}
    if blk.gate is not None:
        shapes["g"] = (M, blk.F)
    out = {}
    for k, shp in shapes.items():
        n = shp[0] * shp[1]
        out[k] = scratch[off[k]:off[k] + 2 * n].view(torch.float16).view(shp)
    return out


def qg_loop_range(blk: Block, h: torch.Tensor, L0: int, L1: int,
                  scratch: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Apply iterations [L0, L1) of the block in place on FP32 h [M][D]."""
    if h.dtype != torch.float32 or not h.is_contiguous() or h.dim() != 2 or h.shape[1] != blk.D:
        raise ValueError(f"h must be a contiguous FP32 [M][{blk.D}] tensor, got "
                         f"{tuple(h.shape)} {h.dtype}")
    M = h.shape[0]
    if scratch is None:
        scratch = alloc_loop_scratch(blk, M, h.device)
    b = blk.cstruct()
    _check("qg_loop_range", lib.qg_loop_range(C.byref(b), _dev(h, "h"), M, L0, L1,
                                              scratch.data_ptr(),
                                              scratch.numel() * scratch.element_size(),
                                              _stream(stream)))
    return h


def qg_loop_chunked_scratch_bytes(blk: Block, M: int, chunk: int) -> int:
    b = blk.cstruct()
    return lib.qg_loop_chunked_scratch_bytes(C.byref(b), M, chunk)


def qg_loop_range_chunked(blk: Block, h: torch.Tensor, L0: int, L1: int, chunk: int,
                          scratch: torch.Tensor | None = None, hcache: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """Chunk-first driver: rows of FP32 h [M][D] in chunks of `chunk`, each
    through iterations [L0, L1) before the next (scratch sized for a chunk).
    hcache: optional FP16 [L1 - L0][M][D] receiving each iteration's
    attention input x (the FP16-h cache)."""
    if h.dtype != torch.float32 or not h.is_contiguous() or h.dim() != 2 or h.shape[1] != blk.D:
        raise ValueError(f"h must be a contiguous FP32 [M][{blk.D}] tensor, got "
                         f"{tuple(h.shape)} {h.dtype}")
    M = h.shape[0]
    if hcache is not None and (hcache.dtype != torch.float16 or not hcache.is_contiguous()
                               or tuple(hcache.shape) != (L1 - L0, M, blk.D)):
        raise ValueError(f"hcache must be a contiguous FP16 [{L1 - L0}][{M}][{blk.D}] tensor")
    if scratch is None:
        scratch = torch.empty(max(qg_loop_chunked_scratch_bytes(blk, M, chunk), 256),
                              dtype=torch.uint8, device=h.device)
    b = blk.cstruct()
    _check("qg_loop_range_chunked",
           lib.qg_loop_range_chunked(C.byref(b), _dev(h, "h"), M, L0, L1, chunk,
                                     scratch.data_ptr(), scratch.numel() * scratch.element_size(),
                                     None if hcache is None else _dev(hcache, "hcache"),
                                     _stream(stream)))
    return h


def qg_unpack(w: PackedWeight, stream=None) -> torch.Tensor:
    q = torch.empty((w.N, w.K), dtype=torch.uint8, device=w.codes.device)
    cw = w.cstruct()
    _check("qg_unpack", lib.qg_unpack(C.byref(cw), q.data_ptr(), _stream(stream)))
    return q


def qg_dequant(w: PackedWeight, fp16: bool = False, stream=None) -> torch.Tensor:
    out = torch.empty((w.N, w.K), dtype=torch.float16 if fp16 else torch.float32,
                      device=w.codes.device)
    cw = w.cstruct()
    _check("qg_dequant", lib.qg_dequant(C.byref(cw), 1 if fp16 else 0, out.data_ptr(),
                                        _stream(stream)))
    return out


def qg_release_cache() -> None:
    lib.qg_release_cache()


def qg_requant_4to2(w4: PackedWeight, out: PackedWeight | None = None, in_place: bool = False,
                    compact: bool = False, stream=None) -> PackedWeight:
    """INT4 -> INT2 re-quantisation on the GPU: a validation pass (which
    synchronises the stream and raises, with nothing written, on a non-finite
    INT4 scale or zero or an overflowing INT2 scale), then the re-quantisation,
    enqueued on the stream.

    Out of place the result goes to `out` (or new compact tensors).  With
    in_place=True the INT2 weight takes over w4's memory (codes, scales and
    zeros): its rows keep the INT4 row stride (K/2 bytes, each INT2 row over
    the front half of its INT4 row; one launch), or with compact=True they are
    packed K/4 bytes apart over the front of the INT4 buffer.  The returned
    weight views w4's memory, and w4 no longer holds INT4 data."""
    if w4.bits != 4:
        raise ValueError("w4 must be an INT4 weight")
    K, N = w4.K, w4.N
    if in_place:
        if out is not None:
            raise ValueError("in_place and out are exclusive")
        if compact:
            if not w4.codes.is_contiguous():
                raise ValueError("compact in place needs contiguous INT4 codes")
            codes = w4.codes.view(-1)[:N * (K // 16)].view(N, K // 16)
        else:
            codes = w4.codes
        out = PackedWeight(2, K, N, codes, w4.scales, w4.zeros, w4.group)
    elif out is None:
        out = PackedWeight.empty(K, N, 2, w4.codes.device, w4.group)
    c4, c2 = w4.cstruct(), out.cstruct()
    _check("qg_requant_4to2", lib.qg_requant_4to2(C.byref(c4), C.byref(c2), _stream(stream)))
    return out


def requant_block(blk: Block, in_place: bool = False, compact: bool = False, stream=None) -> Block:
    """The INT4 -> INT2 tier switch of a loop block ("β-Informed Deployment
    Features" page, CTX-TIER apply step): re-quantise each INT4 projection
    (INT2 ones are kept).  The re-quantisations are enqueued on the stream;
    torch's allocator is stream-ordered, so the INT4 tensors may be dropped
    (out of place) as soon as the caller releases `blk`."""
    ws = {k: qg_requant_4to2(w, in_place=in_place, compact=compact, stream=stream) if w.bits == 4 else w
          for k, w in blk.weights().items()}
    return Block(blk.D, blk.F, ws["qkv"], ws["out"], ws["up"], ws["down"], ws.get("gate"))


def pack_block(W: dict, bits: int, D: int, F: int, device="cuda", per_row: bool = False) -> Block:
    """qg_pack each FP32 [K][N] projection weight of a block (qkv, out, up,
    down, and gate when W has one); per_row: one group per output channel
    (group = K) instead of groups of 128."""
    ws = {k: qg_pack(W[k].to(device=device, dtype=torch.float32).contiguous(), bits,
                     W[k].shape[0] if per_row else GROUP)
          for k in ("qkv", "out", "up", "down", "gate") if k in W}
    return Block(D, F, ws["qkv"], ws["out"], ws["up"], ws["down"], ws.get("gate"))
