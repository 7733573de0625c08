"""The C ABI on the CPU: the library loads, exports every declared symbol and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes as C
import os
import re

import pytest

import dequant_matmul_int3_amd as qt
from dequant_matmul_int3_amd import qt as qtmod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qt.h")

QT_OK, QT_ERR_NULL, QT_ERR_SHAPE, QT_ERR_ALIGN, QT_ERR_DTYPE, QT_ERR_ARG, QT_ERR_ALIAS = range(7)
QT_ERR_WORKSPACE = 8

# fake device addresses: validation must reject these calls before any
# dereference or launch
A = 0x7F0000000000
B = 0x7F1000000000
Cc = 0x7F2000000000
D = 0x7F3000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qt_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_named_entry_points():
    names = declared_functions()
    for n in ("qt_quantize_g64", "qt_pack_i3", "qt_matvec_i3", "qt_matmul_i3", "qt_hessian_diag"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = qt.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) <= set(qtmod._SIGS), "binding misses a declared function"


def test_sizes():
    assert qt.qt_groups(0) == 0 and qt.qt_groups(1) == 1 and qt.qt_groups(64) == 1
    assert qt.qt_groups(65) == 2 and qt.qt_groups(7200) == 113
    assert qt.qt_packed_bytes(2048, 7168) == 5505024
    assert qt.qt_packed_bytes(2048, 7200) == 2048 * 113 * 24
    assert qt.qt_packed_bytes(0, 5) == 0 and qt.qt_packed_bytes(3, -1) == 0
    assert qt.qt_packed_bytes(1 << 62, 1 << 20) == 0  # overflow is reported as 0
    assert qt.qt_hessian_workspace_bytes(100, 64) == 0  # a single slab needs none
    assert qt.qt_hessian_workspace_bytes(8192, 17408) >= 8192 // 128 * 17408 * 4
    for s in range(9):
        assert qt.qt_status_str(s)


L = None


def setup_module(_):
    global L
    L = qt.lib()


def test_quantize_signed_rejects():
    f = L.qt_quantize_g64_signed
    assert f(None, 4, 64, None, 64, 32, 0.5, 1.0, B, Cc, None) == QT_ERR_NULL
    assert f(A, 0, 64, None, 64, 32, 0.5, 1.0, B, Cc, None) == QT_ERR_SHAPE
    assert f(A, 4, 64, None, 1, 32, 0.5, 1.0, B, Cc, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 0, 32, 0.5, 1.0, B, Cc, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 257, 32, 0.5, 1.0, B, Cc, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 1, 0.5, 1.0, B, Cc, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 257, 0.5, 1.0, B, Cc, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 32, 0.0, 1.0, B, Cc, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 32, 1.0, 0.5, B, Cc, None) == QT_ERR_ARG
    assert f(A + 2, 4, 64, None, 64, 32, 0.5, 1.0, B, Cc, None) == QT_ERR_ALIGN
    assert f(A, 4, 64, None, 64, 32, 0.5, 1.0, A + 16, Cc, None) == QT_ERR_ALIAS


def test_quantize_rejects():
    f = L.qt_quantize_g64
    assert f(None, 4, 64, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_NULL
    assert f(A, 0, 64, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_SHAPE
    assert f(A, 4, 0, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_SHAPE
    assert f(A, 4, 1 << 31, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_SHAPE
    assert f(A, 4, 64, None, 1, 0.5, 1.0, B, Cc, None, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 257, 0.5, 1.0, B, Cc, None, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 0.0, 1.0, B, Cc, None, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 1.0, 0.5, B, Cc, None, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 0.5, float("inf"), B, Cc, None, None) == QT_ERR_ARG
    assert f(A + 2, 4, 64, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_ALIGN
    assert f(A, 4, 64, D + 1, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_ALIGN
    assert f(A, 4, 64, None, 0, 0.5, 1.0, A + 16, Cc, None, None) == QT_ERR_ALIAS
    assert f(A, 4, 64, None, 0, 0.5, 1.0, B, B + 8, None, None) == QT_ERR_ALIAS
    assert f(A, 4, 64, None, 0, 0.5, 1.0, B, Cc, A + 100, None) == QT_ERR_ALIAS


def test_pack_rejects():
    f = L.qt_pack_i3
    assert f(None, 2, 64, B, None) == QT_ERR_NULL
    assert f(A, -1, 64, B, None) == QT_ERR_SHAPE
    assert f(A, 2, 64, B + 2, None) == QT_ERR_ALIGN
    assert f(A, 2, 64, A + 16, None) == QT_ERR_ALIAS
    # packed at 4 bytes passes the alignment check (the overlap is caught next)
    assert f(A, 2, 64, A + 4, None) == QT_ERR_ALIAS


def test_matvec_rejects():
    f = L.qt_matvec_i3
    assert f(A, B, 4, 64, Cc, None, None) == QT_ERR_NULL
    assert f(A, B, 4, 0, Cc, D, None) == QT_ERR_SHAPE
    assert f(A + 2, B, 4, 64, Cc, D, None) == QT_ERR_ALIGN
    assert f(A, B + 2, 4, 64, Cc, D, None) == QT_ERR_ALIGN
    assert f(A + 4, B, 4, 64, Cc, A + 36, None) == QT_ERR_ALIAS  # packed at 4 bytes is accepted
    assert f(A, B, 4, 64, Cc, A + 32, None) == QT_ERR_ALIAS
    assert f(A, B, 4, 64, Cc, Cc + 4, None) == QT_ERR_ALIAS


def test_hessian_full_limits_and_rejects():
    # rows pad to 256 and the f32 kernel's 128-row tiles fit a 65535-wide grid
    lim = 32767 * 256
    assert qt.qt_hessian_full_workspace_bytes(100, 300, 0) == 512 * 128 * 4
    assert qt.qt_hessian_full_workspace_bytes(64, lim, 1) == lim * 64 * 2
    assert qt.qt_hessian_full_workspace_bytes(64, lim + 1, 1) == 0
    assert qt.qt_hessian_full_workspace_bytes(0, 64, 1) == 0
    f = L.qt_hessian_full
    ws = 1 << 30
    assert f(None, 1, 64, 64, B, 0, Cc, ws, None) == QT_ERR_NULL
    assert f(A, 1, 64, 64, None, 0, Cc, ws, None) == QT_ERR_NULL
    assert f(A, 7, 64, 64, B, 0, Cc, ws, None) == QT_ERR_DTYPE
    assert f(A, 1, 0, 64, B, 0, Cc, ws, None) == QT_ERR_SHAPE
    assert f(A, 1, 64, lim + 1, B, 0, Cc, ws, None) == QT_ERR_SHAPE
    assert f(A, 1, 64, 64, B, 2, Cc, ws, None) == QT_ERR_ARG
    assert f(A, 1, 64, 64, B, 0, Cc, 100, None) == QT_ERR_WORKSPACE
    assert f(A + 2, 1, 64, 64, B, 0, Cc, ws, None) == QT_ERR_ALIGN


def test_matmul_rejects():
    f = L.qt_matmul_i3
    assert f(A, B, 4, 64, None, 0, 2, D, None) == QT_ERR_NULL
    assert f(A, B, 4, 64, Cc, 7, 2, D, None) == QT_ERR_DTYPE
    assert f(A, B, 4, 64, Cc, 0, 0, D, None) == QT_ERR_SHAPE
    assert f(A, B, 4, 64, Cc, 0, 65535 * 128 + 1, D, None) == QT_ERR_SHAPE
    assert f(A, B, 4, 64, Cc + 1, 1, 32, D, None) == QT_ERR_ALIGN  # bf16 needs 2 bytes
    assert f(A, B, 4, 64, Cc + 2, 0, 32, D, None) == QT_ERR_ALIGN  # f32 needs 4 bytes
    assert f(A + 2, B, 4, 64, Cc, 1, 32, D, None) == QT_ERR_ALIGN
    assert f(A, B, 4, 64, Cc, 1, 32, Cc + 64, None) == QT_ERR_ALIAS
    # bf16 X at 2 bytes and packed at 4 bytes pass the alignment check
    assert f(A + 4, B, 4, 64, Cc + 2, 1, 32, Cc + 64, None) == QT_ERR_ALIAS


def test_grouped_rejects():
    f = L.qt_matvec_i3_grouped
    assert f(A, B, 8, 4, 64, Cc, 4, None, None, 4, D, None) == QT_ERR_NULL
    assert f(A, B, 0, 4, 64, Cc, 4, None, A, 4, D, None) == QT_ERR_SHAPE
    assert f(A, B, 8, 4, 64, Cc, 3, None, A + (1 << 30), 4, D, None) == QT_ERR_SHAPE
    assert f(A, B, 8, 4, 64, Cc, 4, D + 2, A + (1 << 30), 4, D + 4096, None) == QT_ERR_ALIGN
    assert f(A, B, 8, 4, 64, Cc, 4, None, A + (1 << 30), 4, B + 64, None) == QT_ERR_ALIAS


def test_hessian_rejects():
    f = L.qt_hessian_diag
    assert f(None, 0, 8, 64, B, 0, None, 0, None) == QT_ERR_NULL
    assert f(A, 3, 8, 64, B, 0, None, 0, None) == QT_ERR_DTYPE
    assert f(A, 0, 0, 64, B, 0, None, 0, None) == QT_ERR_SHAPE
    assert f(A, 0, 8, 64, B, 2, None, 0, None) == QT_ERR_ARG
    assert f(A + 2, 0, 8, 64, B, 0, None, 0, None) == QT_ERR_ALIGN
    assert f(A, 0, 8192, 64, B, 0, None, 0, None) == QT_ERR_WORKSPACE
    assert f(A, 0, 8192, 64, B, 0, Cc, 16, None) == QT_ERR_WORKSPACE
    assert f(A, 0, 8, 64, A + 64, 0, None, 0, None) == QT_ERR_ALIAS


def test_int4_sizes():
    assert qt.qt_packed_bytes_i4(2048, 7168) == 2048 * 112 * 32
    assert qt.qt_packed_bytes_i4(2048, 7200) == 2048 * 113 * 32
    assert qt.qt_packed_bytes_i4(0, 5) == 0 and qt.qt_packed_bytes_i4(3, -1) == 0
    assert qt.qt_packed_bytes_i4(1 << 62, 1 << 20) == 0


def test_int4_rejects():
    f = L.qt_quantize_g64_i4
    assert f(None, 4, 64, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_NULL
    assert f(A, 4, 0, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_SHAPE
    assert f(A, 4, 64, None, 1, 0.5, 1.0, B, Cc, None, None) == QT_ERR_ARG
    assert f(A, 4, 64, None, 64, 1.0, 0.5, B, Cc, None, None) == QT_ERR_ARG
    assert f(A + 2, 4, 64, None, 0, 0.5, 1.0, B, Cc, None, None) == QT_ERR_ALIGN
    assert f(A, 4, 64, None, 0, 0.5, 1.0, B, A + 8, None, None) == QT_ERR_ALIAS
    f = L.qt_pack_i4
    assert f(None, 2, 64, B, None) == QT_ERR_NULL
    assert f(A, 2, 0, B, None) == QT_ERR_SHAPE
    assert f(A, 2, 64, B + 8, None) == QT_ERR_ALIGN
    # 2 x 64 codes end at A + 128; the 64 packed bytes from A + 96 overlap them
    assert f(A, 2, 64, A + 96, None) == QT_ERR_ALIAS
    f = L.qt_matvec_i4
    assert f(A, B, 4, 64, Cc, None, None) == QT_ERR_NULL
    assert f(A + 8, B, 4, 64, Cc, D, None) == QT_ERR_ALIGN
    # 4 rows x 32 bytes: a y at A + 100 lies inside the int4 weights
    assert f(A, B, 4, 64, Cc, A + 100, None) == QT_ERR_ALIAS
    f = L.qt_matmul_i4
    assert f(A, B, 4, 64, Cc, 7, 2, D, None) == QT_ERR_DTYPE
    assert f(A, B, 4, 64, Cc, 0, 0, D, None) == QT_ERR_SHAPE
    assert f(A, B, 4, 64, Cc + 1, 1, 32, D, None) == QT_ERR_ALIGN
    assert f(A, B, 4, 64, Cc, 0, 2, A + 100, None) == QT_ERR_ALIAS


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        qt.qt_pack_i3(torch.zeros((2, 64), dtype=torch.int8))


def test_int4_grouped_rejects():
    f = L.qt_matvec_i4_grouped
    assert f(A, B, 8, 4, 64, Cc, 4, None, None, 4, D, None) == QT_ERR_NULL
    assert f(A, B, 0, 4, 64, Cc, 4, None, A, 4, D, None) == QT_ERR_SHAPE
    assert f(A + 8, B, 8, 4, 64, Cc, 4, None, A + (1 << 30), 4, D, None) == QT_ERR_ALIGN
    # 8 experts x 4 rows x 32 bytes = 1024 packed bytes from A: Y at A + 1000 overlaps
    assert f(A, B, 8, 4, 64, Cc, 4, None, A + (1 << 30), 4, A + 1000, None) == QT_ERR_ALIAS


def test_moe_layer_rejects():
    f = L.qt_moe_layer
    ok = dict(T=4, D=256, F=128, E=8, k=2)

    def call(X=A, T=4, D=256, F=128, lg=B, E=8, k=2, gb=3, ub=3, db=3, out=D_OUT, ws=WS,
             wsb=1 << 30):
        return f(X, T, D, F, lg, E, k, P1, S1, gb, P2, S2, ub, P3, S3, db, out, ws, wsb, None)
    assert call(X=None) == QT_ERR_NULL
    assert call(D=200) == QT_ERR_SHAPE          # not a multiple of 128
    assert call(F=64) == QT_ERR_SHAPE
    assert call(k=0) == QT_ERR_SHAPE and call(k=9, E=8) == QT_ERR_SHAPE and call(k=33, E=64) == QT_ERR_SHAPE
    assert call(gb=5) == QT_ERR_ARG
    assert call(wsb=16) == QT_ERR_WORKSPACE
    assert call(X=A + 4) == QT_ERR_ALIGN
    assert call(out=A + 1024) == QT_ERR_ALIAS    # inside X (4 x 256 f32)
    assert ok


P1, S1, P2, S2, P3, S3 = (0x7F4000000000, 0x7F5000000000, 0x7F6000000000, 0x7F7000000000,
                          0x7F8000000000, 0x7F9000000000)
D_OUT = 0x7FA000000000
WS = 0x7FB000000000


def test_hessian_noalloc_rejects():
    f = L.qt_hessian_diag_noalloc
    QT_ERR_SCRATCH = 9
    assert qt.qt_hessian_scratch_bytes() == 16 << 20
    assert f(None, 0, 100, 64, B, 0, None) == QT_ERR_NULL
    assert f(A, 2, 100, 64, B, 0, None) == QT_ERR_DTYPE
    assert f(A, 0, 0, 64, B, 0, None) == QT_ERR_SHAPE
    assert f(A, 0, 100, 64, B, 2, None) == QT_ERR_ARG
    assert f(A + 2, 0, 100, 64, B, 0, None) == QT_ERR_ALIGN
    assert f(A, 0, 100, 64, A + 4, 0, None) == QT_ERR_ALIAS
    # 128 slabs x 32769 columns x 4 bytes is past the 16 MiB scratch; 32768 fits
    assert qt.qt_hessian_workspace_bytes(128 * 128, 32768) == 16 << 20
    assert f(A, 0, 128 * 128, 32769, B, 0, None) == QT_ERR_SCRATCH
    assert "scratch" in qt.qt_status_str(QT_ERR_SCRATCH)


def test_missing_library_raises(monkeypatch, tmp_path):
    # no fallback: without libqt.so every call raises instead of computing
    monkeypatch.setattr(qtmod, "_SO", str(tmp_path / "libqt.so"))
    monkeypatch.setattr(qtmod, "_lib", None)
    with pytest.raises(ImportError):
        qtmod.qt_groups(64)
