"""FP64 CPU oracle for the INT4/INT2 weight-only quantised GEMM and loop block.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg use it; the product library never does.  It shares no code
with the HIP path (it is plain C built with gcc, wrapped here with ctypes and
numpy) and imports nothing from the product package.

Each function follows a passage of the TinyLoop documentation pages; see the
header of oracle.c for the passages and for the readings taken where the pages
are silent.  `brute.py` beside this file re-derives pack and GEMM with exact
rational arithmetic for tiny shapes.  Parity unpinned against the pages: the
loop's glue readings (LayerNorm, self-only attention, identity FFN activation)
and the integer zero-point convention, pinned only to closed forms of those
readings.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, EINVAL, EUNSUPPORTED, ENOMEM = 0, -1, -2, -3
GROUP = 128


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, FP64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Weight(C.Structure):
    _fields_ = [("bits", C.c_int32), ("K", C.c_int32), ("N", C.c_int32), ("group", C.c_int32),
                ("codes", C.c_void_p), ("scales", C.c_void_p), ("zeros", C.c_void_p)]


class _Block(C.Structure):
    _fields_ = [("D", C.c_int32), ("F", C.c_int32),
                ("qkv", _Weight), ("out", _Weight), ("up", _Weight), ("down", _Weight),
                ("gate", _Weight)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.or_half_to_double.restype = C.c_double
        L.or_half_to_double.argtypes = [C.c_uint16]
        L.or_round_half.restype = C.c_double
        L.or_round_half.argtypes = [C.c_double]
        L.or_double_to_half_bits.restype = C.c_uint16
        L.or_double_to_half_bits.argtypes = [C.c_double]
        L.or_pack.restype = C.c_int
        L.or_pack.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp]
        L.or_unpack.restype = C.c_int
        L.or_unpack.argtypes = [vp, i32, i32, i32, vp]
        L.or_dequant.restype = C.c_int
        L.or_dequant.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
        L.or_gemm.restype = C.c_int
        L.or_gemm.argtypes = [vp, i64, i32, C.POINTER(_Weight), vp, i64]
        L.or_layernorm.restype = C.c_int
        L.or_layernorm.argtypes = [vp, i32, i32, vp]
        L.or_loop_range.restype = C.c_int
        L.or_loop_range.argtypes = [C.POINTER(_Block), vp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.or_silu.restype = C.c_double
        L.or_silu.argtypes = [C.c_double]
        for name in ("or_round_half_array", "or_half_to_double_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [vp, i64, vp]
        L.or_num_threads.restype = C.c_int
        L.or_num_threads.argtypes = []
        L.or_set_num_threads.restype = None
        L.or_set_num_threads.argtypes = [C.c_int]
        L.or_half_bits_array.restype = None
        L.or_half_bits_array.argtypes = [vp, i64, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


class OracleError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"oracle {fn} returned status {status}")
        self.status = status


def _check(fn: str, st: int):
    if st != OK:
        raise OracleError(fn, st)


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all cores)."""
    return lib().or_num_threads()


def set_num_threads(n: int) -> None:
    """Threads for later oracle calls (timing only; results do not depend on it)."""
    lib().or_set_num_threads(int(n))


# ------------------------------------------------------------------ FP16 ----

def half_to_double(bits: int) -> float:
    return lib().or_half_to_double(int(bits) & 0xFFFF)


def round_half(x) -> np.ndarray:
    """Nearest FP16 value (ties to even) of each FP64 element, as FP64."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(a)
    lib().or_round_half_array(_ptr(a), a.size, _ptr(out))
    return out


def half_bits(x) -> np.ndarray:
    """FP16 bit patterns (uint16) of the nearest FP16 value of each element."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().or_half_bits_array(_ptr(a), a.size, _ptr(out))
    return out


def halves_to_double(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits).view(np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().or_half_to_double_array(_ptr(b), b.size, _ptr(out))
    return out


# --------------------------------------------------------------- format ----

@dataclass
class Packed:
    """One packed weight: codes [N][K*bits/32] uint32, scales/zeros [N][K/group]
    FP16 bit patterns (uint16); group 128, or K for per-row groups."""
    bits: int
    K: int
    N: int
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    group: int = GROUP

    def cstruct(self) -> _Weight:
        return _Weight(self.bits, self.K, self.N, self.group, _ptr(self.codes),
                       _ptr(self.scales), _ptr(self.zeros))


def pack(W, bits: int, group: int = GROUP) -> Packed:
    """Quantise FP32 W [K][N] (see or_pack in oracle.c)."""
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float32))
    K, N = W.shape
    if K % group or bits not in (2, 4):
        raise OracleError("pack", EINVAL if bits in (2, 4) else EUNSUPPORTED)
    codes = np.zeros((N, K * bits // 32), dtype=np.uint32)
    scales = np.zeros((N, K // group), dtype=np.uint16)
    zeros = np.zeros((N, K // group), dtype=np.uint16)
    _check("pack", lib().or_pack(_ptr(W), N, K, N, bits, group, _ptr(codes), _ptr(scales),
                                 _ptr(zeros)))
    return Packed(bits, K, N, codes, scales, zeros, group)


def unpack(p: Packed) -> np.ndarray:
    """Codes q [N][K] as uint8."""
    q = np.empty((p.N, p.K), dtype=np.uint8)
    _check("unpack", lib().or_unpack(_ptr(p.codes), p.K, p.N, p.bits, _ptr(q)))
    return q


def dequant(p: Packed) -> np.ndarray:
    """w^ [N][K] = (q - z) * s in FP64 (N-major, like the packed rows)."""
    out = np.empty((p.N, p.K), dtype=np.float64)
    _check("dequant", lib().or_dequant(_ptr(p.codes), _ptr(p.scales), _ptr(p.zeros), p.K, p.N,
                                       p.bits, p.group, _ptr(out)))
    return out


def requant_4to2(p: Packed) -> Packed:
    """INT4 -> INT2 re-quantisation ("β-Informed Deployment Features" page,
    CTX-TIER, details of the shipped kernel: every group is dequantised, given
    a new INT2 scale from its range, and packed four codes per byte).  Here:
    the exact INT4 dequant w^ = (q - z) s, quantised again by `pack` with
    bits = 2 under the same readings (range with 0 included, integer zero
    point, round-half-even).  w^ has at most 15 significant bits, so its FP32
    copy handed to `pack` is exact."""
    if p.bits != 4:
        raise OracleError("requant_4to2", EINVAL)
    w = dequant(p)                                   # [N][K], FP64
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w), "INT4 dequant must be exact in FP32"
    return pack(np.ascontiguousarray(w32.T), 2, p.group)


def gemm(X, p: Packed) -> np.ndarray:
    """Y [M][N] = X [M][K] (FP16) @ w^ [K][N], FP64, unrounded."""
    X16 = np.ascontiguousarray(np.asarray(X, dtype=np.float16)).view(np.uint16)
    M = X16.shape[0]
    Y = np.empty((M, p.N), dtype=np.float64)
    w = p.cstruct()
    _check("gemm", lib().or_gemm(_ptr(X16), p.K, M, C.byref(w), _ptr(Y), p.N))
    return Y


def layernorm(h) -> np.ndarray:
    """FP16-rounded parameter-free LayerNorm of each row of FP64 h [M][D]."""
    h = np.ascontiguousarray(h, dtype=np.float64)
    out = np.empty_like(h)
    _check("layernorm", lib().or_layernorm(_ptr(h), h.shape[0], h.shape[1], _ptr(out)))
    return out


@dataclass
class Block:
    """The block's projections; gate None = four projections with the
    identity FFN activation, else the SwiGLU FFN (see or_block in oracle.c)."""
    D: int
    F: int
    qkv: Packed
    out: Packed
    up: Packed
    down: Packed
    gate: Packed | None = None

    def cstruct(self) -> _Block:
        gate = self.gate.cstruct() if self.gate is not None else _Weight(0, 0, 0, 0, None, None,
                                                                           None)
        return _Block(self.D, self.F, self.qkv.cstruct(), self.out.cstruct(), self.up.cstruct(),
                      self.down.cstruct(), gate)


def pack_block(W: dict, bits: int, D: int, F: int, per_row: bool = False) -> Block:
    """Pack qkv, out, up, down (and gate, when W has one); per_row: one group
    per output channel (group = K) instead of groups of 128."""
    def p(k):
        a = np.asarray(W[k])
        return pack(a, bits, a.shape[0] if per_row else GROUP)
    ws = {k: p(k) for k in ("qkv", "out", "up", "down")}
    gate = p("gate") if "gate" in W else None
    return Block(D, F, ws["qkv"], ws["out"], ws["up"], ws["down"], gate)


def silu(z: float) -> float:
    """silu(z) = z / (1 + e^-z) in FP64 (or_silu)."""
    return lib().or_silu(float(z))


def loop_range(blk: Block, h, L0: int, L1: int):
    """Apply iterations [L0, L1) to a copy of FP64 h [M][D].  Returns (h, last)
    where last holds the final iteration's FP16-valued norm, qkv, u (the FFN
    hidden: the up output, or fp16(silu(g) * u) when gated), y and, when
    gated, g."""
    h = np.array(h, dtype=np.float64, order="C", copy=True)
    M = h.shape[0]
    last = {"norm": np.zeros((M, blk.D)), "qkv": np.zeros((M, 3 * blk.D)),
            "u": np.zeros((M, blk.F)), "y": np.zeros((M, blk.D)), "g": np.zeros((M, blk.F))}
    b = blk.cstruct()
    _check("loop_range", lib().or_loop_range(C.byref(b), _ptr(h), M, L0, L1, _ptr(last["norm"]),
                                             _ptr(last["qkv"]), _ptr(last["u"]),
                                             _ptr(last["y"]), _ptr(last["g"])))
    if blk.gate is None:
        del last["g"]
    return h, last
