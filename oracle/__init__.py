"""int3-g64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

A thin ctypes binding over liboracle.so (plain scalar C in oracle.c).  Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product library never does.  Every function mirrors one in
oracle.h, which cites the passage of the pages each one follows.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.SO):
            _build.build()
        L = C.CDLL(_build.SO)
        P, I64, I32, F32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
        L.qto_groups.restype = I64
        L.qto_groups.argtypes = [I64]
        L.qto_packed_bytes.restype = I64
        L.qto_packed_bytes.argtypes = [I64, I64]
        L.qto_grid_factor.restype = F32
        L.qto_grid_factor.argtypes = [I32, I32, F32, F32]
        L.qto_quantize_g64.argtypes = [P, I64, I64, P, I32, F32, F32, P, P, P, P]
        L.qto_quantize_g64_signed.argtypes = [P, I64, I64, P, I32, I32, F32, F32, P, P]
        L.qto_packed_bytes_i4.restype = I64
        L.qto_packed_bytes_i4.argtypes = [I64, I64]
        L.qto_quantize_g64_i4.argtypes = [P, I64, I64, P, I32, F32, F32, P, P, P]
        L.qto_pack_i4.argtypes = [P, I64, I64, P]
        L.qto_unpack_i4.argtypes = [P, I64, I64, P]
        L.qto_matvec_i4_f64.argtypes = [P, P, I64, I64, P, P, P]
        L.qto_pack_i3.argtypes = [P, I64, I64, P]
        L.qto_unpack_i3.argtypes = [P, I64, I64, P]
        L.qto_matvec_f64.argtypes = [P, P, I64, I64, P, P, P]
        L.qto_matmul_f64_sampled.argtypes = [P, P, I64, I64, P, I64, I64, P, P, P, P]
        L.qto_matvec_f32.argtypes = [P, P, I64, I64, P, P]
        L.qto_hessian_diag.argtypes = [P, I64, I64, P, P]
        L.qto_rowint_recon.argtypes = [P, I64, I64, I32, P]
        L.qto_dequant_f64.argtypes = [P, P, I64, I64, P]
        L.qto_hessian_full.argtypes = [P, I64, I64, P]
        L.qto_gptq_factor.restype = I32
        L.qto_gptq_factor.argtypes = [P, I64, C.c_double, P]
        L.qto_gptq_i3.argtypes = [P, I64, I64, P, I32, P, P]
        L.qto_gptq_replay.argtypes = [P, I64, I64, P, P, P, P, P]
        L.qto_proxy_terms.argtypes = [P, I64, I64, P, P, P, P, P]
        for f in ("qto_hessian_full", "qto_gptq_i3", "qto_gptq_replay", "qto_proxy_terms"):
            getattr(L, f).restype = None
        for f in ("qto_quantize_g64_i4", "qto_pack_i4", "qto_unpack_i4", "qto_matvec_i4_f64",
                  "qto_quantize_g64", "qto_quantize_g64_signed", "qto_pack_i3", "qto_unpack_i3", "qto_matvec_f64",
                  "qto_matmul_f64_sampled", "qto_matvec_f32", "qto_hessian_diag",
                  "qto_rowint_recon", "qto_dequant_f64"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def groups(I: int) -> int:
    return int(lib().qto_groups(I))


def packed_bytes(O: int, I: int) -> int:
    return int(lib().qto_packed_bytes(O, I))


def grid_factor(k: int, n: int, lo: float, hi: float) -> float:
    return float(lib().qto_grid_factor(k, n, lo, hi))


def quantize_g64(W, d=None, n_grid: int = 0, lo: float = 0.5, hi: float = 1.0,
                 return_errs: bool = False):
    """-> (scales[O,G] f32, codes[O,I] int8, grid_idx[O,G] uint8[, errs[O,G,n]])."""
    W = _c(W, np.float32)
    O, I = W.shape
    G = groups(I)
    d = None if d is None else _c(d, np.float32)
    scales = np.empty((O, G), np.float32)
    codes = np.empty((O, I), np.int8)
    gidx = np.empty((O, G), np.uint8)
    n = max(n_grid, 1)
    errs = np.empty((O, G, n), np.float32) if return_errs else None
    lib().qto_quantize_g64(_p(W), O, I, _p(d), n_grid, lo, hi, _p(scales), _p(codes),
                           _p(gidx), _p(errs))
    if return_errs:
        return scales, codes, gidx, errs
    return scales, codes, gidx


def quantize_g64_signed(W, d=None, n1: int = 64, n2: int = 32, lo: float = 0.5,
                        hi: float = 1.0):
    """Two-stage signed scale search -> (scales[O,G] f32, codes[O,I] int8)."""
    W = _c(W, np.float32)
    O, I = W.shape
    G = groups(I)
    d = None if d is None else _c(d, np.float32)
    scales = np.empty((O, G), np.float32)
    codes = np.empty((O, I), np.int8)
    lib().qto_quantize_g64_signed(_p(W), O, I, _p(d), n1, n2, lo, hi, _p(scales),
                                  _p(codes))
    return scales, codes


def packed_bytes_i4(O: int, I: int) -> int:
    return int(lib().qto_packed_bytes_i4(O, I))


def quantize_g64_i4(W, d=None, n_grid: int = 0, lo: float = 0.5, hi: float = 1.0):
    """Grouped int4 -> (scales[O,G] f32, codes[O,I] int8 in [-8,7], grid_idx[O,G] uint8)."""
    W = _c(W, np.float32)
    O, I = W.shape
    G = groups(I)
    d = None if d is None else _c(d, np.float32)
    scales = np.empty((O, G), np.float32)
    codes = np.empty((O, I), np.int8)
    gidx = np.empty((O, G), np.uint8)
    lib().qto_quantize_g64_i4(_p(W), O, I, _p(d), n_grid, lo, hi, _p(scales), _p(codes),
                              _p(gidx))
    return scales, codes, gidx


def pack_i4(codes):
    codes = _c(codes, np.int8)
    O, I = codes.shape
    out = np.empty(packed_bytes_i4(O, I), np.uint8)
    lib().qto_pack_i4(_p(codes), O, I, _p(out))
    return out


def unpack_i4(packed, O: int, I: int):
    packed = _c(packed, np.uint8)
    assert packed.size == packed_bytes_i4(O, I)
    out = np.empty((O, I), np.int8)
    lib().qto_unpack_i4(_p(packed), O, I, _p(out))
    return out


def matvec_i4_f64(packed, scales, O: int, I: int, x):
    """-> (y[O] f64, sum_i |w_oi x_i| [O] f64) for grouped int4 weights."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.float32)
    x = _c(x, np.float32)
    y = np.empty(O, np.float64)
    a = np.empty(O, np.float64)
    lib().qto_matvec_i4_f64(_p(packed), _p(scales), O, I, _p(x), _p(y), _p(a))
    return y, a


def pack_i3(codes):
    codes = _c(codes, np.int8)
    O, I = codes.shape
    out = np.empty(packed_bytes(O, I), np.uint8)
    lib().qto_pack_i3(_p(codes), O, I, _p(out))
    return out


def unpack_i3(packed, O: int, I: int):
    packed = _c(packed, np.uint8)
    assert packed.size == packed_bytes(O, I)
    out = np.empty((O, I), np.int8)
    lib().qto_unpack_i3(_p(packed), O, I, _p(out))
    return out


def matvec_f64(packed, scales, O: int, I: int, x):
    """-> (y[O] f64, absy[O] f64)."""
    packed, scales, x = _c(packed, np.uint8), _c(scales, np.float32), _c(x, np.float32)
    y = np.empty(O, np.float64)
    a = np.empty(O, np.float64)
    lib().qto_matvec_f64(_p(packed), _p(scales), O, I, _p(x), _p(y), _p(a))
    return y, a


def matmul_f64_sampled(packed, scales, O: int, I: int, X, t_idx, o_idx):
    """Y[t,o] of X[B,I] @ W_hat^T at the sample points -> (y, absy)."""
    packed, scales, X = _c(packed, np.uint8), _c(scales, np.float32), _c(X, np.float32)
    t_idx, o_idx = _c(t_idx, np.int64), _c(o_idx, np.int64)
    n = t_idx.size
    y = np.empty(n, np.float64)
    a = np.empty(n, np.float64)
    lib().qto_matmul_f64_sampled(_p(packed), _p(scales), O, I, _p(X), X.shape[0], n,
                                 _p(t_idx), _p(o_idx), _p(y), _p(a))
    return y, a


def matvec_f32(packed, scales, O: int, I: int, x):
    packed, scales, x = _c(packed, np.uint8), _c(scales, np.float32), _c(x, np.float32)
    y = np.empty(O, np.float32)
    lib().qto_matvec_f32(_p(packed), _p(scales), O, I, _p(x), _p(y))
    return y


def hessian_diag(X, d_in=None):
    X = _c(X, np.float32)
    T, I = X.shape
    d_in = None if d_in is None else _c(d_in, np.float64)
    out = np.empty(I, np.float64)
    lib().qto_hessian_diag(_p(X), T, I, _p(d_in), _p(out))
    return out


def rowint_recon(W, bits: int = 4):
    W = _c(W, np.float32)
    O, I = W.shape
    out = np.empty((O, I), np.float64)
    lib().qto_rowint_recon(_p(W), O, I, bits, _p(out))
    return out


# ---------------------------------------------------------------- GPTQ / LDLQ
def hessian_full(X):
    """H [I, I] f64 = sum_t X[t]^T X[t] for X [T, I] f32."""
    X = _c(X, np.float32)
    T, I = X.shape
    H = np.empty((I, I), np.float64)
    lib().qto_hessian_full(_p(X), T, I, _p(H))
    return H


def gptq_factor(H, damp: float = 0.01):
    """U [n, n] f64: the upper Cholesky factor of (H + damp*mean(diag H)*I)^-1."""
    H = _c(H, np.float64)
    n = H.shape[0]
    U = np.empty((n, n), np.float64)
    if lib().qto_gptq_factor(_p(H), n, float(damp), _p(U)) != 0:
        raise ValueError("matrix is not positive definite")
    return U


def gptq_i3(W, U, block: int = 128):
    """GPTQ sweep with the int3-g64 rounder: -> (scales [O, G] f32, codes [O, I] int8)."""
    W = _c(W, np.float32)
    U = _c(U, np.float32)
    O, I = W.shape
    scales = np.empty((O, groups(I)), np.float32)
    codes = np.empty((O, I), np.int8)
    lib().qto_gptq_i3(_p(W), O, I, _p(U), block, _p(scales), _p(codes))
    return scales, codes


def gptq_replay(W, U, scales, codes):
    """-> (column values [O, I] f64 at decision time, group bases [O, G] f64)."""
    W = _c(W, np.float32)
    U = _c(U, np.float32)
    scales = _c(scales, np.float32)
    codes = _c(codes, np.int8)
    O, I = W.shape
    wt = np.empty((O, I), np.float64)
    base = np.empty((O, groups(I)), np.float64)
    lib().qto_gptq_replay(_p(W), O, I, _p(U), _p(scales), _p(codes), _p(wt), _p(base))
    return wt, base


def proxy_terms(W, codes, scales, H):
    """(tr(E H E^T), tr(W H W^T)) in f64 with E = W - s*v; H [I, I] f32."""
    W = _c(W, np.float32)
    codes = _c(codes, np.int8)
    scales = _c(scales, np.float32)
    H = _c(H, np.float32)
    O, I = W.shape
    num = C.c_double()
    den = C.c_double()
    lib().qto_proxy_terms(_p(W), O, I, _p(codes), _p(scales), _p(H), C.byref(num), C.byref(den))
    return num.value, den.value


# ---------------------------------------------------------------- MoE expert layer
# The pull request page's MoE setting (every routed expert's weights read once
# per decode step; the per-projection ablation names gate_proj, up_proj and
# down_proj of each expert) with the MoE decode configuration's top-8 routing.
# The pages give no expert formula and no combine rule.  Readings:
#   - expert e: y = W_down,e (silu(W_gate,e x) * (W_up,e x)), silu(z) = z / (1 + exp(-z));
#   - routing: the k largest logits of the token (equal logits: the lower
#     expert index first), combine weights a softmax over those k logits;
#   - out_t = sum_j w_tj y_{e_tj}(x_t).
def dequant_f64(packed, scales, O: int, I: int, bits: int = 3):
    """The weights a packed matrix denotes, s * v, in f64 [O, I] (int3-g64 by
    the C routine, grouped int4 from its unpacked codes)."""
    if bits == 3:
        packed, scales = _c(packed, np.uint8), _c(scales, np.float32)
        out = np.empty((O, I), np.float64)
        lib().qto_dequant_f64(_p(packed), _p(scales), O, I, _p(out))
        return out
    codes = unpack_i4(packed, O, I)
    s = np.repeat(np.asarray(scales, np.float64).reshape(O, -1), 64, axis=1)[:, :I]
    return s * codes.astype(np.float64)


def moe_route(logits, k: int):
    """-> (experts [T, k] int32 in descending logit order, weights [T, k] f64)."""
    L = np.asarray(logits, np.float32)
    idx = np.argsort(-L, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(L, idx, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])  # the first is the largest
    return idx.astype(np.int32), z / z.sum(axis=1, keepdims=True)


def silu_f64(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):  # exp(-z) = inf for very negative z gives -0
        return z / (1.0 + np.exp(-z))


def moe_layer_f64(X, logits, k: int, gate, up, down):
    """gate / up / down: (packed [E, bytes], scales [E, O, G], bits) with gate
    and up [F x D] per expert and down [D x F].  -> (out [T, D] f64, bound
    [T, D]): bound is the error budget of an implementation whose gate/up/
    down products each meet 1e-5 of their absolute sums (the grouped
    multiply's tolerance), scaled so that |out - ref| <= 1e-5 * bound."""
    X = np.asarray(X, np.float32)
    T, D = X.shape
    F = gate[1].shape[1]
    experts, w = moe_route(logits, k)
    out = np.zeros((T, D))
    bound = np.zeros((T, D))
    cache = {}

    def mats(e):
        if e not in cache:
            cache[e] = (dequant_f64(gate[0][e], gate[1][e], F, D, gate[2]),
                        dequant_f64(up[0][e], up[1][e], F, D, up[2]),
                        dequant_f64(down[0][e], down[1][e], D, F, down[2]))
        return cache[e]

    for t in range(T):
        x = X[t].astype(np.float64)
        for j in range(k):
            Wg, Wu, Wd = mats(int(experts[t, j]))
            g, u = Wg @ x, Wu @ x
            ag, au = np.abs(Wg) @ np.abs(x), np.abs(Wu) @ np.abs(x)
            h = silu_f64(g) * u
            y = Wd @ h
            dh = 1.1 * ag * np.abs(u) + np.abs(silu_f64(g)) * au  # |silu'| <= 1.1
            out[t] += w[t, j] * y
            bound[t] += w[t, j] * (np.abs(Wd) @ dh + np.abs(Wd) @ np.abs(h) + np.abs(y))
    return out, bound


def moe_layer_f64_tokens(X, logits, k: int, expert, tokens):
    """moe_layer_f64 for the rows `tokens` only, without holding whole
    dequantized matrices: expert(e) -> (gate, up, down), each (packed [bytes],
    scales [O, G], bits) of one expert.  The gate and up products of a token
    are the f64 matvecs (which also give sum |w x|); the down matrix of one
    expert at a time is dequantized in f64.  -> (out [n, D], bound [n, D])."""
    X = np.asarray(X, np.float32)
    tokens = [int(t) for t in tokens]
    experts, w = moe_route(logits, k)
    D = X.shape[1]
    out = np.zeros((len(tokens), D))
    bound = np.zeros((len(tokens), D))

    def mv(m, O, I, x):
        return (matvec_f64 if m[2] == 3 else matvec_i4_f64)(m[0], m[1], O, I, x)

    for i, t in enumerate(tokens):
        x = X[t]
        for j in range(k):
            gate, up, down = expert(int(experts[t, j]))
            F = np.asarray(gate[1]).shape[0]
            g, ag = mv(gate, F, D, x)
            u, au = mv(up, F, D, x)
            h = silu_f64(g) * u
            Wd = dequant_f64(down[0], down[1], D, F, down[2])
            y = Wd @ h
            dh = 1.1 * ag * np.abs(u) + np.abs(silu_f64(g)) * au  # |silu'| <= 1.1
            out[i] += w[t, j] * y
            bound[i] += w[t, j] * (np.abs(Wd) @ dh + np.abs(Wd) @ np.abs(h) + np.abs(y))
    return out, bound
