"""ctypes binding of libqt.so with the same names as include/qt.h.

Argument marshalling only: shapes and dtypes of torch tensors are turned into
pointers and sizes, optional outputs are allocated with torch on the tensors'
device, and the call is enqueued on torch's current HIP stream (or the stream
given).  Every step of the computation runs in the library's kernels; there is
no fallback: if libqt.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

QT_F32 = 0
QT_BF16 = 1

_SO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqt.so")
_lib = None

_SIGS = {
    "qt_groups": (C.c_int64, [C.c_int64]),
    "qt_packed_bytes": (C.c_int64, [C.c_int64, C.c_int64]),
    "qt_status_str": (C.c_char_p, [C.c_int]),
    "qt_hessian_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64]),
    "qt_hessian_diag": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_void_p,
                                  C.c_int, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qt_hessian_diag_noalloc": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64,
                                          C.c_void_p, C.c_int, C.c_void_p]),
    "qt_hessian_scratch_bytes": (C.c_size_t, []),
    "qt_quantize_g64": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int32,
                                  C.c_float, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p]),
    "qt_quantize_g64_signed": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                                         C.c_int32, C.c_int32, C.c_float, C.c_float,
                                         C.c_void_p, C.c_void_p, C.c_void_p]),
    "qt_pack_i3": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]),
    "qt_matvec_i3": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                               C.c_void_p, C.c_void_p]),
    "qt_matmul_i3": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                               C.c_int, C.c_int64, C.c_void_p, C.c_void_p]),
    "qt_matvec_i3_grouped": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                       C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32,
                                       C.c_void_p, C.c_void_p]),
    "qt_matvec_i4_grouped": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                       C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32,
                                       C.c_void_p, C.c_void_p]),
    "qt_packed_bytes_i4": (C.c_int64, [C.c_int64, C.c_int64]),
    "qt_moe_layer_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int32, C.c_int32, C.c_int64,
                                                  C.c_int64]),
    "qt_moe_layer": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int32,
                               C.c_int32, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                               C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                               C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qt_hessian_full_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64, C.c_int]),
    "qt_hessian_full": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_void_p, C.c_int,
                                  C.c_void_p, C.c_size_t, C.c_void_p]),
    "qt_gptq_factor_workspace_bytes": (C.c_size_t, [C.c_int64]),
    "qt_gptq_factor": (C.c_int, [C.c_void_p, C.c_int64, C.c_double, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_size_t, C.c_void_p]),
    "qt_gptq_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64]),
    "qt_gptq_i3": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                             C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qt_gptq_proxy_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int64]),
    "qt_gptq_proxy": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qt_quantize_g64_i4": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int32,
                                     C.c_float, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p]),
    "qt_pack_i4": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p]),
    "qt_matvec_i4": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                               C.c_void_p, C.c_void_p]),
    "qt_matmul_i4": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                               C.c_int, C.c_int64, C.c_void_p, C.c_void_p]),
}


class QtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({qt_status_str(status)})")


def lib():
    """Load libqt.so (built in-tree by dequant_matmul_int3_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise ImportError(f"{_SO} is not built; run `python -m dequant_matmul_int3_amd.build`")
        L = C.CDLL(_SO)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is not None:
        return C.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libqt takes device tensors only")
        if not t.is_contiguous():
            raise ValueError("libqt takes contiguous tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _check(status: int, where: str):
    if status != 0:
        raise QtError(status, where)


def qt_status_str(status: int) -> str:
    return lib().qt_status_str(status).decode()


def qt_groups(I: int) -> int:
    return int(lib().qt_groups(I))


def qt_packed_bytes(O: int, I: int) -> int:
    return int(lib().qt_packed_bytes(O, I))


def qt_hessian_workspace_bytes(T: int, I: int) -> int:
    return int(lib().qt_hessian_workspace_bytes(T, I))


def qt_hessian_diag(X, d=None, accumulate: bool = False, workspace=None, stream=None):
    """d[j] (+)= sum_t X[t,j]^2 for X [T, I] f32 or bf16 -> d [I] f32."""
    T, I = X.shape
    if d is None:
        d = torch.zeros(I, dtype=torch.float32, device=X.device)
    ws_need = qt_hessian_workspace_bytes(T, I)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=X.device)
    dev = _dev(X, d, workspace)
    xt = QT_BF16 if X.dtype == torch.bfloat16 else QT_F32 if X.dtype == torch.float32 else -1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qt_hessian_diag(_ptr(X), xt, T, I, _ptr(d), int(accumulate), _ptr(workspace),
                                 ws_bytes, _stream(stream, dev)), "qt_hessian_diag")
    return d


def qt_hessian_scratch_bytes() -> int:
    return int(lib().qt_hessian_scratch_bytes())


def qt_hessian_diag_noalloc(X, d=None, accumulate: bool = False, stream=None):
    """qt_hessian_diag with the library's built-in scratch (no workspace)."""
    T, I = X.shape
    if d is None:
        d = torch.zeros(I, dtype=torch.float32, device=X.device)
    dev = _dev(X, d)
    xt = QT_BF16 if X.dtype == torch.bfloat16 else QT_F32 if X.dtype == torch.float32 else -1
    _check(lib().qt_hessian_diag_noalloc(_ptr(X), xt, T, I, _ptr(d), int(accumulate),
                                         _stream(stream, dev)), "qt_hessian_diag_noalloc")
    return d


def qt_packed_bytes_i4(O: int, I: int) -> int:
    return int(lib().qt_packed_bytes_i4(O, I))


def _quantize(name, W, d, n_grid, lo, hi, scales, codes, grid_idx, want_grid_idx, stream):
    O, I = W.shape
    G = qt_groups(I)
    if scales is None:
        scales = torch.empty((O, G), dtype=torch.float32, device=W.device)
    if codes is None:
        codes = torch.empty((O, I), dtype=torch.int8, device=W.device)
    if grid_idx is None and want_grid_idx:
        grid_idx = torch.empty((O, G), dtype=torch.uint8, device=W.device)
    dev = _dev(W, d, scales, codes, grid_idx)
    if W.dtype != torch.float32 or (d is not None and d.dtype != torch.float32):
        raise ValueError("W and d must be float32")
    _check(getattr(lib(), name)(_ptr(W), O, I, _ptr(d), n_grid, lo, hi, _ptr(scales),
                                _ptr(codes), _ptr(grid_idx), _stream(stream, dev)), name)
    return scales, codes, grid_idx


def qt_quantize_g64(W, d=None, n_grid: int = 0, lo: float = 0.5, hi: float = 1.0,
                    scales=None, codes=None, grid_idx=None, want_grid_idx: bool = True,
                    stream=None):
    """W [O, I] f32 -> (scales [O, G] f32, codes [O, I] int8, grid_idx [O, G] uint8 or None)."""
    return _quantize("qt_quantize_g64", W, d, n_grid, lo, hi, scales, codes, grid_idx,
                     want_grid_idx, stream)


def qt_quantize_g64_i4(W, d=None, n_grid: int = 0, lo: float = 0.5, hi: float = 1.0,
                       scales=None, codes=None, grid_idx=None, want_grid_idx: bool = True,
                       stream=None):
    """Grouped int4: W [O, I] f32 -> (scales [O, G], codes [O, I] in [-8, 7], grid_idx)."""
    return _quantize("qt_quantize_g64_i4", W, d, n_grid, lo, hi, scales, codes, grid_idx,
                     want_grid_idx, stream)


def qt_quantize_g64_signed(W, d=None, n1: int = 64, n2: int = 32, lo: float = 0.5,
                           hi: float = 1.0, scales=None, codes=None, stream=None):
    """Two-stage signed search: W [O, I] f32 -> (scales [O, G] f32, codes [O, I] int8)."""
    O, I = W.shape
    G = qt_groups(I)
    if scales is None:
        scales = torch.empty((O, G), dtype=torch.float32, device=W.device)
    if codes is None:
        codes = torch.empty((O, I), dtype=torch.int8, device=W.device)
    dev = _dev(W, d, scales, codes)
    if W.dtype != torch.float32 or (d is not None and d.dtype != torch.float32):
        raise ValueError("W and d must be float32")
    _check(lib().qt_quantize_g64_signed(_ptr(W), O, I, _ptr(d), n1, n2, lo, hi, _ptr(scales),
                                        _ptr(codes), _stream(stream, dev)),
           "qt_quantize_g64_signed")
    return scales, codes


def _pack(name, nbytes, codes, packed, stream):
    O, I = codes.shape
    if packed is None:
        packed = torch.empty(nbytes(O, I), dtype=torch.uint8, device=codes.device)
    dev = _dev(codes, packed)
    _check(getattr(lib(), name)(_ptr(codes), O, I, _ptr(packed), _stream(stream, dev)), name)
    return packed


def qt_pack_i3(codes, packed=None, stream=None):
    """codes [O, I] int8 -> packed [O*G*24] uint8."""
    return _pack("qt_pack_i3", qt_packed_bytes, codes, packed, stream)


def qt_pack_i4(codes, packed=None, stream=None):
    """codes [O, I] int8 in [-8, 7] -> packed [O*G*32] uint8."""
    return _pack("qt_pack_i4", qt_packed_bytes_i4, codes, packed, stream)


def _matvec(name, packed, scales, O, I, x, y, stream):
    if y is None:
        y = torch.empty(O, dtype=torch.float32, device=x.device)
    dev = _dev(packed, scales, x, y)
    _check(getattr(lib(), name)(_ptr(packed), _ptr(scales), O, I, _ptr(x), _ptr(y),
                                _stream(stream, dev)), name)
    return y


def qt_matvec_i3(packed, scales, O: int, I: int, x, y=None, stream=None):
    """y [O] f32 = W x for x [I] f32."""
    return _matvec("qt_matvec_i3", packed, scales, O, I, x, y, stream)


def qt_matvec_i4(packed, scales, O: int, I: int, x, y=None, stream=None):
    """y [O] f32 = W x for int4 weights and x [I] f32."""
    return _matvec("qt_matvec_i4", packed, scales, O, I, x, y, stream)


def _matmul(name, packed, scales, O, I, X, Y, stream):
    B = X.shape[0]
    if Y is None:
        Y = torch.empty((B, O), dtype=torch.float32, device=X.device)
    dev = _dev(packed, scales, X, Y)
    xt = QT_BF16 if X.dtype == torch.bfloat16 else QT_F32 if X.dtype == torch.float32 else -1
    _check(getattr(lib(), name)(_ptr(packed), _ptr(scales), O, I, _ptr(X), xt, B, _ptr(Y),
                                _stream(stream, dev)), name)
    return Y


def qt_matmul_i3(packed, scales, O: int, I: int, X, Y=None, stream=None):
    """Y [B, O] f32 = X W^T for X [B, I] f32 or bf16."""
    return _matmul("qt_matmul_i3", packed, scales, O, I, X, Y, stream)


def qt_matmul_i4(packed, scales, O: int, I: int, X, Y=None, stream=None):
    """Y [B, O] f32 = X W^T for int4 weights and X [B, I] f32 or bf16."""
    return _matmul("qt_matmul_i4", packed, scales, O, I, X, Y, stream)


def _grouped(name, packed, scales, E, O, I, X, expert_offsets, P, pair_row, Y, stream):
    if Y is None:
        Y = torch.empty((P, O), dtype=torch.float32, device=X.device)
    dev = _dev(packed, scales, X, expert_offsets, pair_row, Y)
    _check(getattr(lib(), name)(_ptr(packed), _ptr(scales), E, O, I, _ptr(X), X.shape[0],
                                _ptr(pair_row), _ptr(expert_offsets), P, _ptr(Y),
                                _stream(stream, dev)), name)
    return Y


def qt_matvec_i3_grouped(packed, scales, E: int, O: int, I: int, X, expert_offsets, P: int,
                         pair_row=None, Y=None, stream=None):
    """Y [P, O] f32: Y[p] = W_{e(p)} X[row(p)] for pairs sorted by expert."""
    return _grouped("qt_matvec_i3_grouped", packed, scales, E, O, I, X, expert_offsets, P,
                    pair_row, Y, stream)


def qt_matvec_i4_grouped(packed, scales, E: int, O: int, I: int, X, expert_offsets, P: int,
                         pair_row=None, Y=None, stream=None):
    """qt_matvec_i3_grouped for grouped int4 experts."""
    return _grouped("qt_matvec_i4_grouped", packed, scales, E, O, I, X, expert_offsets, P,
                    pair_row, Y, stream)


# ---------------------------------------------------------------- GPTQ
def qt_hessian_full_workspace_bytes(T: int, I: int, xt: int) -> int:
    return int(lib().qt_hessian_full_workspace_bytes(T, I, xt))


def qt_gptq_factor_workspace_bytes(I: int) -> int:
    return int(lib().qt_gptq_factor_workspace_bytes(I))


def qt_gptq_workspace_bytes(O: int, I: int) -> int:
    return int(lib().qt_gptq_workspace_bytes(O, I))


def qt_gptq_proxy_workspace_bytes(O: int, I: int) -> int:
    return int(lib().qt_gptq_proxy_workspace_bytes(O, I))


def _ws(nbytes, device, workspace):
    if workspace is None:
        workspace = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def qt_hessian_full(X, H=None, accumulate: bool = False, workspace=None, stream=None):
    """H [I, I] f32 (+)= X^T X for X [T, I] f32 or bf16."""
    T, I = X.shape
    xt = QT_BF16 if X.dtype == torch.bfloat16 else QT_F32 if X.dtype == torch.float32 else -1
    if H is None:
        H = torch.empty((I, I), dtype=torch.float32, device=X.device)
    need = int(lib().qt_hessian_full_workspace_bytes(T, I, xt if xt >= 0 else 0))
    workspace, wsb = _ws(need, X.device, workspace)
    dev = _dev(X, H, workspace)
    _check(lib().qt_hessian_full(_ptr(X), xt, T, I, _ptr(H), int(accumulate), _ptr(workspace),
                                 wsb, _stream(stream, dev)), "qt_hessian_full")
    return H


def qt_gptq_factor(H, damp: float = 0.01, U=None, info=None, workspace=None, stream=None):
    """-> (U [I, I] f32 upper Cholesky factor of the damped H^-1, info int32 [1])."""
    I = H.shape[0]
    if U is None:
        U = torch.empty((I, I), dtype=torch.float32, device=H.device)
    if info is None:
        info = torch.empty(1, dtype=torch.int32, device=H.device)
    workspace, wsb = _ws(lib().qt_gptq_factor_workspace_bytes(I), H.device, workspace)
    dev = _dev(H, U, info, workspace)
    _check(lib().qt_gptq_factor(_ptr(H), I, float(damp), _ptr(U), _ptr(info), _ptr(workspace),
                                wsb, _stream(stream, dev)), "qt_gptq_factor")
    return U, info


def qt_gptq_i3(W, U, scales=None, codes=None, workspace=None, stream=None):
    """GPTQ sweep: W [O, I] f32, U [I, I] -> (scales [O, G] f32, codes [O, I] int8)."""
    O, I = W.shape
    if scales is None:
        scales = torch.empty((O, qt_groups(I)), dtype=torch.float32, device=W.device)
    if codes is None:
        codes = torch.empty((O, I), dtype=torch.int8, device=W.device)
    workspace, wsb = _ws(lib().qt_gptq_workspace_bytes(O, I), W.device, workspace)
    dev = _dev(W, U, scales, codes, workspace)
    _check(lib().qt_gptq_i3(_ptr(W), O, I, _ptr(U), _ptr(scales), _ptr(codes), _ptr(workspace),
                            wsb, _stream(stream, dev)), "qt_gptq_i3")
    return scales, codes


def qt_gptq_proxy(W, packed, scales, H, terms=None, workspace=None, stream=None):
    """-> terms [2] f64 on the device: (tr(E H E^T), tr(W H W^T))."""
    O, I = W.shape
    if terms is None:
        terms = torch.empty(2, dtype=torch.float64, device=W.device)
    workspace, wsb = _ws(lib().qt_gptq_proxy_workspace_bytes(O, I), W.device, workspace)
    dev = _dev(W, packed, scales, H, terms, workspace)
    _check(lib().qt_gptq_proxy(_ptr(W), _ptr(packed), _ptr(scales), O, I, _ptr(H), _ptr(terms),
                               _ptr(workspace), wsb, _stream(stream, dev)), "qt_gptq_proxy")
    return terms


# ---------------------------------------------------------------- MoE layer
def qt_moe_layer_workspace_bytes(T: int, k: int, E: int, D: int, F: int) -> int:
    return int(lib().qt_moe_layer_workspace_bytes(T, k, E, D, F))


def qt_moe_layer(X, logits, k: int, gate, up, down, out=None, workspace=None, stream=None):
    """X [T, D] f32, logits [T, E] f32; gate / up / down = (packed [E, bytes],
    scales [E, O, G], bits) with gate, up [F x D] and down [D x F] per expert
    -> out [T, D] f32."""
    T, D = X.shape
    E = logits.shape[1]
    F = gate[1].shape[1]
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=X.device)
    workspace, wsb = _ws(qt_moe_layer_workspace_bytes(T, k, E, D, F), X.device, workspace)
    dev = _dev(X, logits, gate[0], gate[1], up[0], up[1], down[0], down[1], out, workspace)
    _check(lib().qt_moe_layer(_ptr(X), T, D, F, _ptr(logits), E, k, _ptr(gate[0]),
                              _ptr(gate[1]), int(gate[2]), _ptr(up[0]), _ptr(up[1]), int(up[2]),
                              _ptr(down[0]), _ptr(down[1]), int(down[2]), _ptr(out),
                              _ptr(workspace), wsb, _stream(stream, dev)), "qt_moe_layer")
    return out
