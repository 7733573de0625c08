"""Comparison helpers shared by the tests (no method arithmetic here)."""
import numpy as np


def componentwise_err(y, y_ref, abs_ref):
    """max_o |y_o - y_ref_o| / A_o with A_o = sum_i |w_hat[o,i] * x_i| (f64).

    Rows with A_o == 0 must match exactly (y_ref is then exactly 0)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    abs_ref = np.asarray(abs_ref, np.float64)
    diff = np.abs(y - y_ref)
    zero = abs_ref == 0
    if np.any(diff[zero] != 0):
        return np.inf
    if np.all(zero):
        return 0.0
    return float(np.max(diff[~zero] / abs_ref[~zero]))


def normwise_err(y, y_ref):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.max(np.abs(y_ref))
    return float(np.max(np.abs(y - y_ref)) / den) if den > 0 else float(np.max(np.abs(y)))


def np_decode_planes(packed, O, I):
    """Independent decoder of the int3-g64 planes built on numpy.unpackbits.

    Low plane: value j of a group at bits 2j, 2j+1 of the 16-byte plane read
    little-endian; high plane: value j at bit j of the 8-byte plane."""
    G = -(-I // 64)
    p = np.asarray(packed, np.uint8).reshape(O, G, 24)
    lo_bits = np.unpackbits(p[:, :, :16], axis=2, bitorder="little").reshape(O, G, 64, 2)
    hi_bits = np.unpackbits(p[:, :, 16:], axis=2, bitorder="little").reshape(O, G, 64)
    u = lo_bits[..., 0].astype(np.int16) + 2 * lo_bits[..., 1] + 4 * hi_bits
    v = (u - 4).reshape(O, G * 64)[:, :I]
    return v.astype(np.int8)
