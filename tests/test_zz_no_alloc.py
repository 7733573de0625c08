"""qt_hessian_diag_noalloc (the entry point that allocates nothing, for
callers that cannot call hipMalloc) against qt_hessian_diag through the C
ABI: bit-identical results on two calls in a row, the second smaller, and
both within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import dequant_matmul_int3_amd as qt
import oracle
import workloads
from tests.gpu_util import bits, dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu


def test_hessian_diag_noalloc_matches_the_workspace_entry_point():
    # two calls in a row on the shared scratch, the second with fewer slabs
    # and columns (stale partials of the first call must not leak into it)
    for T, I, acc in ((8192, 4096, False), (1000, 1500, True), (300, 77, False)):
        X = workloads.generic_matrix(T, I, seed=T + I)
        Xd = dev(X)
        d0 = workloads.generic_vector(I, seed=I).astype(np.float32) ** 2
        say(f"hessian noalloc T={T} I={I} accumulate={acc}")
        ref = host(qt.qt_hessian_diag(Xd, dev(d0) if acc else None, accumulate=acc))
        got = host(qt.qt_hessian_diag_noalloc(Xd, dev(d0) if acc else None, accumulate=acc))
        assert np.array_equal(bits(got), bits(ref)), "differs from qt_hessian_diag"
        want = oracle.hessian_diag(X, d0 if acc else None)
        assert np.max(np.abs(got - want) / want) <= 1e-5


def test_hessian_diag_noalloc_bf16_and_repeat():
    T, I = 4096, 2048
    Xb = workloads.bf16_bits_rne(workloads.generic_matrix(T, I, seed=5))
    Xd = dev_bf16(Xb)
    say(f"hessian noalloc bf16 T={T} I={I}, three calls")
    ref = host(qt.qt_hessian_diag(Xd))
    for _ in range(3):
        assert np.array_equal(bits(host(qt.qt_hessian_diag_noalloc(Xd))), bits(ref))
