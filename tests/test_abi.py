"""CPU-side checks of the C ABI: the library loads, exports every function
include/qgemm.h declares, and rejects bad arguments on the host before
touching the device (no kernel is launched by any call in this file)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT

qg = pytest.importorskip("int2_quantized_gemm_amd")

HEADER = os.path.join(ROOT, "include", "qgemm.h")
FAKE = 1 << 20  # a 256-byte aligned, never dereferenced address


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qg_[a-z0-9_]+)\s*\(", text)))


def test_header_functions_are_exported():
    names = _declared()
    assert "qg_pack" in names and "qg_loop_range" in names and len(names) >= 13
    for n in names:
        assert hasattr(qg.lib, n), f"libqgemm.so does not export {n}"


def test_versions():
    assert qg.qg_abi_version() == 3
    assert qg.qg_layout_version() == 1
    text = open(HEADER).read()
    assert "#define QG_ABI_VERSION 3" in text and "#define QG_LAYOUT_VERSION 1" in text


def _w(bits=4, K=2048, N=2048, group=128, codes=FAKE, scales=FAKE, zeros=FAKE):
    return qg._Weight(bits, K, N, group, codes, scales, zeros)


def _gemm(fn, w, X=FAKE, ldx=2048, Y=FAKE, ldy=2048, M=1, ws=None, ws_bytes=0):
    return fn(X, ldx, C.byref(w), Y, ldy, M, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(bits=3), qg.QG_EUNSUPPORTED, "bits"),
    (dict(group=64), qg.QG_EUNSUPPORTED, "group"),
    (dict(group=1024), qg.QG_EUNSUPPORTED, "group"),       # neither 128 nor K
    (dict(K=100), qg.QG_EINVAL, "K"),
    (dict(K=(1 << 22) + 128), qg.QG_EINVAL, "K"),
    (dict(K=0), qg.QG_EINVAL, "K"),
    (dict(N=0), qg.QG_EINVAL, "N"),
    (dict(codes=0), qg.QG_EINVAL, "NULL"),
    (dict(codes=FAKE + 4), qg.QG_EINVAL, "aligned"),
    (dict(scales=FAKE + 1), qg.QG_EINVAL, "aligned"),
])
def test_gemm_rejects_bad_weight(kw, code, needle):
    st = _gemm(qg.lib.qg_gemm_int4, _w(**kw))
    assert st == code
    assert needle in qg.qg_last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(ldx=2040), "ldx"), (dict(ldx=2052), "ldx"), (dict(ldx=(1 << 22) + 8), "ldx"),
    (dict(ldy=100), "ldy"),
    (dict(M=-1), "M"), (dict(X=0), "NULL"), (dict(Y=FAKE + 2), "aligned"),
])
def test_gemm_rejects_bad_operands(kw, needle):
    assert _gemm(qg.lib.qg_gemm_int4, _w(), **kw) == qg.QG_EINVAL
    assert needle in qg.qg_last_error()


def test_gemm_accepts_per_row_groups():
    """group == K passes the weight check: the call then stops at the next
    operand check (ldy too small), before any launch."""
    assert _gemm(qg.lib.qg_gemm_int4, _w(group=2048), ldy=100) == qg.QG_EINVAL
    assert "ldy" in qg.qg_last_error()


def test_gemm_bits_must_match_entry_point():
    assert _gemm(qg.lib.qg_gemm_int2, _w(bits=4)) == qg.QG_EINVAL
    assert "bits" in qg.qg_last_error()
    assert _gemm(qg.lib.qg_gemm_int4, _w(bits=2)) == qg.QG_EINVAL


def test_gemm_m0_is_a_noop_without_device_work():
    assert _gemm(qg.lib.qg_gemm_int4, _w(), M=0, X=None, Y=None) == qg.QG_OK
    assert qg.qg_last_error() == ""
    assert qg.lib.qg_gemm_ws_bytes(C.byref(_w()), 1) == 0


def _block(D=256, F=512, bits=4, **over):
    ws = dict(qkv=_w(bits, D, 3 * D), out=_w(bits, D, D), up=_w(bits, D, F), down=_w(bits, F, D),
              gate=qg._Weight(0, 0, 0, 0, None, None, None))
    ws.update(over)
    return qg._Block(D, F, ws["qkv"], ws["out"], ws["up"], ws["down"], ws["gate"])


def _loop(b, h=FAKE, M=1, L0=0, L1=1, scratch=FAKE, nbytes=1 << 30):
    return qg.lib.qg_loop_range(C.byref(b), h, M, L0, L1, scratch, nbytes, None)


def test_loop_validation():
    b = _block()
    assert _loop(b, L0=2, L1=1) == qg.QG_EINVAL and "L0" in qg.qg_last_error()
    assert _loop(b, L0=-1, L1=1) == qg.QG_EINVAL
    assert _loop(b, M=-2) == qg.QG_EINVAL
    assert _loop(_block(out=_w(4, 256, 128))) == qg.QG_EINVAL and "out" in qg.qg_last_error()
    assert _loop(_block(D=200)) == qg.QG_EINVAL
    assert _loop(_block(up=_w(3, 256, 512))) == qg.QG_EUNSUPPORTED
    # a gate, when present, must have the shape of up
    assert _loop(_block(gate=_w(4, 256, 256))) == qg.QG_EINVAL and "gate" in qg.qg_last_error()
    assert _loop(_block(gate=_w(2, 256, 512)), L0=3, L1=3) == qg.QG_OK
    need = qg.lib.qg_loop_scratch_bytes(C.byref(b), 4)
    assert need > 0
    assert _loop(b, M=4, nbytes=need - 1) == qg.QG_EINVAL and "scratch" in qg.qg_last_error()
    assert _loop(b, scratch=FAKE + 16) == qg.QG_EINVAL
    assert _loop(b, h=FAKE + 4) == qg.QG_EINVAL
    # empty ranges and M == 0 are no-ops that touch nothing
    assert _loop(b, L0=3, L1=3) == qg.QG_OK
    assert _loop(b, M=0) == qg.QG_OK


@pytest.mark.parametrize("gated", [False, True])
def test_loop_scratch_layout_is_documented_and_aligned(gated):
    D, F, M = 2048, 8192, 512
    b = _block(D, F, gate=_w(4, D, F)) if gated else _block(D, F)
    vals = [C.c_size_t() for _ in range(5)]
    assert qg.lib.qg_loop_scratch_offsets(C.byref(b), M, *(C.byref(v) for v in vals)) == 0
    norm, qkv, u, y, g = (v.value for v in vals)
    assert norm == 0 and qkv >= M * D * 2 and u >= qkv + M * 3 * D * 2 and y >= u + M * F * 2
    assert all(o % 256 == 0 for o in (norm, qkv, u, y, g))
    end = y + M * D * 2
    if gated:
        assert g >= end
        end = g + M * F * 2
    else:
        assert g == 0
    assert qg.lib.qg_loop_scratch_bytes(C.byref(b), M) >= end


def test_pack_validation():
    f = qg.lib.qg_pack
    assert f(FAKE, 64, 128, 64, 3, 128, FAKE, FAKE, FAKE, None) == qg.QG_EUNSUPPORTED
    assert f(FAKE, 64, 128, 64, 4, 32, FAKE, FAKE, FAKE, None) == qg.QG_EUNSUPPORTED
    assert f(FAKE, 64, 100, 64, 4, 128, FAKE, FAKE, FAKE, None) == qg.QG_EINVAL
    assert f(FAKE, 32, 128, 64, 4, 128, FAKE, FAKE, FAKE, None) == qg.QG_EINVAL
    assert "ldw" in qg.qg_last_error()
    assert f(0, 64, 128, 64, 4, 128, FAKE, FAKE, FAKE, None) == qg.QG_EINVAL
    assert f(FAKE + 2, 64, 128, 64, 4, 128, FAKE, FAKE, FAKE, None) == qg.QG_EINVAL


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        qg.qg_pack(torch.zeros(128, 8), 4)


def test_python_binding_checks_shapes():
    """The C side sees pointers and leading dimensions only, so the binding
    checks the tensors' logical shapes before any call (CPU tensors: the
    shape checks come first)."""
    import torch
    w = qg.PackedWeight(4, 256, 16, torch.zeros(16, 32, dtype=torch.int32),
                        torch.zeros(16, 2, dtype=torch.float16),
                        torch.zeros(16, 2, dtype=torch.float16))
    X = torch.zeros(3, 256, dtype=torch.float16)
    with pytest.raises(ValueError, match="X must be"):
        qg.qg_gemm_int4(torch.zeros(3, 128, dtype=torch.float16), w)
    with pytest.raises(ValueError, match="Y must be"):
        qg.qg_gemm_int4(X, w, Y=torch.zeros(3, 8, dtype=torch.float16))
    bad_codes = qg.PackedWeight(4, 256, 16, torch.zeros(16, 16, dtype=torch.int32), w.scales,
                                w.zeros)
    with pytest.raises(ValueError, match="codes must be"):
        qg.qg_gemm_ws_bytes(bad_codes, 3)
    bad_scales = qg.PackedWeight(4, 256, 16, w.codes, torch.zeros(16, 1, dtype=torch.float16),
                                 w.zeros)
    with pytest.raises(ValueError, match="scales must be"):
        qg.qg_gemm_ws_bytes(bad_scales, 3)
    blk = qg.Block(256, 512, *(w,) * 4)
    with pytest.raises(ValueError, match="h must be"):
        qg.qg_loop_range(blk, torch.zeros(2, 128, dtype=torch.float32), 0, 1)


def test_product_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "int2_quantized_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "liboracle" not in text, f
                assert "from oracle" not in text, f


def _rq(w4, w2):
    return qg.lib.qg_requant_4to2(C.byref(w4), C.byref(w2), None)


# INT4 2048 x 2048: codes 2 MiB, scales/zeros 32 KiB each; INT2 codes 1 MiB.
_C4, _S4, _Z4 = FAKE, FAKE + (4 << 20), FAKE + (5 << 20)
_C2, _S2, _Z2 = FAKE + (8 << 20), FAKE + (12 << 20), FAKE + (13 << 20)


@pytest.mark.parametrize("w4kw,w2kw,needle", [
    (dict(bits=2), dict(bits=2), "bits"),
    (dict(), dict(bits=4), "bits"),
    (dict(), dict(K=4096), "K x N"),
    (dict(), dict(N=1024), "K x N"),
    (dict(), dict(codes=_C4 + 64), "overlaps input codes"),      # partial overlap
    (dict(), dict(scales=_C4), "overlaps input codes"),
    (dict(), dict(zeros=_S4 + 2), "overlaps input scales"),
    (dict(), dict(codes=_S2), "outputs overlap"),
    (dict(group=2048), dict(), "group"),                        # per-row in, groups of 128 out
    (dict(), dict(group=2048), "group"),
])
def test_requant_rejects_bad_arguments(w4kw, w2kw, needle):
    w4 = _w(**{**dict(bits=4, codes=_C4, scales=_S4, zeros=_Z4), **w4kw})
    w2 = _w(**{**dict(bits=2, codes=_C2, scales=_S2, zeros=_Z2), **w2kw})
    assert _rq(w4, w2) == qg.QG_EINVAL
    assert needle in qg.qg_last_error()


def test_requant_per_row_k_limit():
    """Per-row re-quantisation holds a row in one workgroup: K <= 32768."""
    K = 65536
    w4 = _w(bits=4, K=K, N=4, group=K, codes=_C4, scales=_S4, zeros=_Z4)
    w2 = _w(bits=2, K=K, N=4, group=K, codes=_C2, scales=_S2, zeros=_Z2)
    assert _rq(w4, w2) == qg.QG_EUNSUPPORTED
    assert "per-row" in qg.qg_last_error()


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback: a copy of the package whose libqgemm.so is absent must
    refuse to import (in a fresh interpreter, so this process's loaded
    library is not reused)."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "int2_quantized_gemm_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "int2_quantized_gemm_amd", "__init__.py"), pkg / "__init__.py")
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "try:\n"
            "    import int2_quantized_gemm_amd\n"
            "except ImportError as e:\n"
            "    print('IMPORT-ERROR', e)\n"
            "else:\n"
            "    print('IMPORTED', int2_quantized_gemm_amd.LIB_PATH)\n")
    r = subprocess.run([sys.executable, "-c", code, str(tmp_path)], capture_output=True, text=True,
                       timeout=300)
    assert "IMPORT-ERROR" in r.stdout and "no fallback" in r.stdout, r.stdout + r.stderr


def _gemm_static(w, X=FAKE, ldx=None, Y=FAKE, ldy=None, M=1):
    ldx = w.K if ldx is None else ldx
    ldy = w.N if ldy is None else ldy
    return qg.lib.qg_gemm_static_ws(X, ldx, C.byref(w), Y, ldy, M, None)


def test_static_ws_rejects_shapes_beyond_its_workspace():
    """A shape whose K-split workspace exceeds the 16 MiB static workspace is
    refused on the host, before anything is enqueued, and names the sizes;
    the loop block's shapes up to M = 512 fit."""
    w = _w(bits=4, K=8192, N=2048)
    need = qg.lib.qg_gemm_ws_bytes(C.byref(w), 768)
    assert need > 16 << 20
    assert _gemm_static(w, M=768) == qg.QG_EINVAL
    msg = qg.qg_last_error()
    assert "static workspace" in msg and str(need) in msg
    for K, N in ((2048, 6144), (2048, 2048), (2048, 8192), (8192, 2048)):
        for M in range(1, 513):
            assert qg.lib.qg_gemm_ws_bytes(C.byref(_w(bits=4, K=K, N=N)), M) <= 16 << 20


@pytest.mark.parametrize("kw,code,needle", [
    (dict(bits=3), qg.QG_EUNSUPPORTED, "bits"),
    (dict(K=100), qg.QG_EINVAL, "K"),
    (dict(codes=FAKE + 4), qg.QG_EINVAL, "aligned"),
])
def test_static_ws_rejects_bad_weight(kw, code, needle):
    assert _gemm_static(_w(**kw)) == code
    assert needle in qg.qg_last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(ldx=2040), "ldx"), (dict(ldy=100), "ldy"), (dict(M=-1), "M"), (dict(X=0), "NULL"),
    (dict(Y=FAKE + 2), "aligned"),
])
def test_static_ws_rejects_bad_operands(kw, needle):
    assert _gemm_static(_w(), **kw) == qg.QG_EINVAL
    assert needle in qg.qg_last_error()


def _block_struct(D=256, F=512):
    w = lambda K, N: _w(bits=4, K=K, N=N)
    g = qg._Weight(0, 0, 0, 0, None, None, None)
    return qg._Block(D, F, w(D, 3 * D), w(D, D), w(D, F), w(F, D), g)


def test_chunked_scratch_bytes():
    """The chunked driver's scratch covers a full chunk and the ragged tail,
    and is no larger than a single shot's once chunks are smaller than M."""
    b = _block_struct(2048, 8192)
    one = lambda M: qg.lib.qg_loop_scratch_bytes(C.byref(b), M)
    ch = lambda M, c: qg.lib.qg_loop_chunked_scratch_bytes(C.byref(b), M, c)
    assert ch(2048, 512) == one(512) < one(2048)
    assert ch(1100, 512) >= max(one(512), one(76))
    assert ch(300, 4096) == one(300)
    assert ch(0, 512) == 0 and ch(10, 0) == 0


@pytest.mark.parametrize("kw,needle", [
    (dict(chunk=0), "chunk"), (dict(scratch_bytes=100), "smaller"), (dict(hcache=FAKE + 2), "hcache"),
    (dict(L0=3, L1=2), "L0"), (dict(h=FAKE + 4), "h must"),
])
def test_chunked_rejects_bad_arguments(kw, needle):
    b = _block_struct()
    a = dict(h=FAKE, M=40, L0=0, L1=2, chunk=16, scratch=FAKE, scratch_bytes=1 << 30, hcache=None)
    a.update(kw)
    st = qg.lib.qg_loop_range_chunked(C.byref(b), a["h"], a["M"], a["L0"], a["L1"], a["chunk"],
                                      a["scratch"], a["scratch_bytes"], a["hcache"], None)
    assert st == qg.QG_EINVAL
    assert needle in qg.qg_last_error()


@pytest.mark.parametrize("ldc,ok", [(0, True), (256, True), (260, True), (1 << 20, True),
                                    (255, False), (258, False), (60, False), (102, False),
                                    ((1 << 20) + 4, False)])
def test_weight_code_row_stride(ldc, ok):
    """ldc: 0 (compact) or a multiple of 4 words in [K*bits/32, 2^20]; a good
    stride passes the weight check and the call stops at the next operand
    check (ldy too small), before any launch."""
    w = _w(bits=4, K=512, N=64)  # compact rows: 64 words
    w.ldc = ldc if ldc != 256 else 64
    st = _gemm(qg.lib.qg_gemm_int4, w, ldx=512, ldy=8)
    assert st == qg.QG_EINVAL
    assert ("ldy" in qg.qg_last_error()) == ok, qg.qg_last_error()
    if not ok:
        assert "ldc" in qg.qg_last_error()
