"""Seeded synthetic inputs for the int3-g64 hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scales, codes, packing or products).  Both the HIP path
and the CPU oracle are fed the very same arrays produced here, so neither side
contains a random number generator of its own.

Workloads (shapes and distributions follow the int3-g64 pull request page,
"Design" and "Tests" sections, and the NeUQI / tt-stack pages for the search and
Hessian shapes; the real checkpoints those pages use are replaced by these
synthetic stand-ins):

* tiny     : W[256x512] ~ N(0, 0.02), 4 distinct random rows each with 8
             distinct random columns multiplied by 20; x[512] ~ N(0, 1).
* decode   : W[2048x7168] ~ N(0, 0.02) with each entry independently replaced,
             with probability 0.005, by a draw from N(0, 0.5); x[7168] ~ N(0, 1).
             A tail variant uses I = 7200 (113 groups, the last one 32 wide).
* moe      : 128 experts, each an up matrix [2048x7168] and a down matrix
             [7168x2048] drawn like `decode`; X[32x7168] ~ N(0, 1); routing
             logits U(0, 1) of shape [32x128], top-8 experts per token.
* prefill  : X[512x7168] ~ N(0, 1) rounded to bf16 (round-to-nearest-even);
             W[18432x7168] drawn like `decode`.
* search   : W[5120x17408] drawn like `decode`; activations
             X[8192x17408] = Z * c with Z ~ N(0, 1) and one c_j = exp(N(0, 1))
             per column (lognormal(0, 1) column importance).

"N(mu, s)" means standard deviation s.  Every draw is made in float64 by numpy's
default generator (PCG64) and rounded once to float32.
"""
from __future__ import annotations

import concurrent.futures as _cf
import numpy as np

SEED = 0

# (O, I) of each weight matrix
TINY_SHAPE = (256, 512)
DECODE_SHAPE = (2048, 7168)
DECODE_TAIL_SHAPE = (2048, 7200)
MOE_EXPERTS = 128
MOE_TOKENS = 32
MOE_TOPK = 8
MOE_UP_SHAPE = (2048, 7168)
MOE_DOWN_SHAPE = (7168, 2048)
PREFILL_TOKENS = 512
PREFILL_SHAPE = (18432, 7168)
SEARCH_SHAPE = (5120, 17408)
SEARCH_TOKENS = 8192

# stream tags, so that every array has a seed of its own and can be regenerated
# independently of the others (and in parallel)
_TAG = {"decode": 1, "decode_tail": 2, "moe_up": 3, "moe_down": 4, "moe_x": 5,
        "moe_route": 6, "prefill_w": 7, "prefill_x": 8, "search_w": 9,
        "search_z": 10, "search_c": 11, "generic": 12, "moe_gate": 13}


def rng_for(tag: str, *idx: int) -> np.random.Generator:
    """Independent PCG64 stream for (SEED, tag, idx...)."""
    return np.random.default_rng([SEED, _TAG[tag], *idx])


def _normal_f32(rng: np.random.Generator, std: float, shape) -> np.ndarray:
    return rng.normal(0.0, std, size=shape).astype(np.float32)


def outlier_weights(rng: np.random.Generator, O: int, I: int,
                    std: float = 0.02, p_out: float = 0.005,
                    std_out: float = 0.5) -> np.ndarray:
    """N(0, std) weights with each entry replaced by N(0, std_out) w.p. p_out."""
    w = rng.normal(0.0, std, size=(O, I))
    mask = rng.random(size=(O, I)) < p_out
    w[mask] = rng.normal(0.0, std_out, size=int(mask.sum()))
    return w.astype(np.float32)


def tiny():
    """W[256x512] with 4 outlier rows (8 entries x20 each) and x[512]; seed 0."""
    rng = np.random.default_rng(SEED)
    O, I = TINY_SHAPE
    w = rng.normal(0.0, 0.02, size=(O, I))
    rows = rng.choice(O, size=4, replace=False)
    for r in rows:
        cols = rng.choice(I, size=8, replace=False)
        w[r, cols] *= 20.0
    x = rng.normal(0.0, 1.0, size=I)
    return w.astype(np.float32), x.astype(np.float32), np.sort(rows)


def decode(tail: bool = False):
    """Decode GEMV inputs: W[2048x7168] (or [2048x7200]) and x."""
    tag = "decode_tail" if tail else "decode"
    O, I = DECODE_TAIL_SHAPE if tail else DECODE_SHAPE
    rng = rng_for(tag)
    w = outlier_weights(rng, O, I)
    x = _normal_f32(rng, 1.0, I)
    return w, x


def moe_expert(e: int, which: str) -> np.ndarray:
    """Weight matrix of expert e; which is 'gate' or 'up' [2048x7168], or 'down' [7168x2048]."""
    shape = MOE_DOWN_SHAPE if which == "down" else MOE_UP_SHAPE
    return outlier_weights(rng_for("moe_" + which, e), *shape)


def moe_experts_parallel(which: str, experts, workers: int = 8):
    """moe_expert for many experts, drawn on a thread pool (numpy releases the GIL)."""
    with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda e: moe_expert(e, which), experts))


def moe_logits() -> np.ndarray:
    """Routing logits [32x128], uniform in [0, 1) (float64 draws)."""
    return rng_for("moe_route").random(size=(MOE_TOKENS, MOE_EXPERTS))


def moe_tokens():
    """X[32x7168] and the top-8 routing: (X, topk_experts[32x8])."""
    x = _normal_f32(rng_for("moe_x"), 1.0, (MOE_TOKENS, MOE_UP_SHAPE[1]))
    logits = moe_logits()
    # top-8 by value, descending; stable order for equal logits (none occur)
    topk = np.argsort(-logits, axis=1, kind="stable")[:, :MOE_TOPK]
    return x, topk.astype(np.int32)


def route_pairs(topk: np.ndarray, n_experts: int):
    """(token, expert) pairs sorted by expert, then token.

    Returns pair_token[P] (int32), pair_expert[P] (int32) and
    expert_offsets[E+1] (int32): the pairs of expert e are
    pair_token[expert_offsets[e]:expert_offsets[e+1]].
    """
    T, K = topk.shape
    tok = np.repeat(np.arange(T, dtype=np.int32), K)
    exp = topk.reshape(-1).astype(np.int32)
    order = np.lexsort((tok, exp))
    tok, exp = tok[order], exp[order]
    offs = np.zeros(n_experts + 1, dtype=np.int32)
    np.add.at(offs, exp + 1, 1)
    return tok, exp, np.cumsum(offs).astype(np.int32)


def bf16_bits_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they denote (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def prefill_x() -> np.ndarray:
    """X[512x7168] as bf16 bit patterns (uint16)."""
    z = rng_for("prefill_x").normal(0.0, 1.0, size=(PREFILL_TOKENS, PREFILL_SHAPE[1]))
    return bf16_bits_rne(z.astype(np.float32))


def prefill_w(rows=None) -> np.ndarray:
    """W[18432x7168]; drawn in 1024-row slabs so that a subset is cheap.

    rows: optional iterable of slab indices (0..17) to draw; default all.
    """
    O, I = PREFILL_SHAPE
    slabs = range(O // 1024) if rows is None else rows
    return np.concatenate([outlier_weights(rng_for("prefill_w", s), 1024, I)
                           for s in slabs], axis=0)


def search_w(slabs=None) -> np.ndarray:
    """W[5120x17408] in 256-row slabs (slab s = rows 256s .. 256s+255)."""
    O, I = SEARCH_SHAPE
    idx = range(O // 256) if slabs is None else slabs
    return np.concatenate([outlier_weights(rng_for("search_w", s), 256, I)
                           for s in idx], axis=0)


def search_colscale() -> np.ndarray:
    """c_j = exp(N(0,1)) per column of the search activations (float32)."""
    return np.exp(rng_for("search_c").normal(0.0, 1.0, size=SEARCH_SHAPE[1])).astype(np.float32)


def search_x(slabs=None, tokens_per_slab: int = 1024) -> np.ndarray:
    """X[8192x17408] = Z * c, in slabs of 1024 tokens (Z drawn per slab)."""
    c = search_colscale()
    n = SEARCH_TOKENS // tokens_per_slab
    idx = range(n) if slabs is None else slabs
    out = []
    for s in idx:
        z = rng_for("search_z", s).normal(0.0, 1.0, size=(tokens_per_slab, SEARCH_SHAPE[1]))
        out.append((z.astype(np.float32) * c[None, :]).astype(np.float32))
    return np.concatenate(out, axis=0)


def generic_weights(O: int, I: int, seed: int = 0, outliers: bool = True) -> np.ndarray:
    """Weights of any shape for edge-case tests (decode distribution)."""
    rng = rng_for("generic", seed, O, I)
    if outliers:
        return outlier_weights(rng, O, I)
    return _normal_f32(rng, 0.02, (O, I))


def generic_vector(n: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    return _normal_f32(rng_for("generic", 1000 + seed, n), std, n)


def generic_matrix(rows: int, cols: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    return _normal_f32(rng_for("generic", 2000 + seed, rows, cols), std, (rows, cols))
