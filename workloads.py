"""Seeded synthetic inputs for the routing workloads.

This module only draws random numbers and lays them out; it holds none of the
routing arithmetic, and both the CPU oracle's tests and the GPU path's tests
and benchmark take their inputs from it.  bf16 rounding of activations (an
input-recipe step, "bf16 activations widened to fp32") is done by torch's CPU
conversion, not by either implementation under test.

Shapes follow the pages: a 256-output fp32 router feeding top_k(8 of 256) and a
19-token request scanned over total batch sizes ("Batch changed the model's
mind", sections "m-scan: the staircase" and "16% of routing decisions"); 512
experts with top-10 and exact bf16 ties at the boundary (vllm.cpp PR #2556,
summary); a 40-layer prefill stack; a shared-expert dense GEMM plus a one-output
gate dot.  No public dataset is named by the pages; these synthetic draws stand
in for the models' real activations.
"""
from __future__ import annotations

import numpy as np
import torch

W_STD = np.float32(0.02)

SEED_W = 1001
SEED_FIXED_REQUEST = 1002
SEED_COARRIVAL = 2000   # + c
SEED_LENGTHS = 3000
SEED_LAYER_W = 4000     # + layer
SEED_REQUEST = 5000     # + request (layer enters as a second seed word)
SEED_DENSE = 6000
SEED_TIES = 7000


def rng(*seed_words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(seed_words) if len(seed_words) > 1 else seed_words[0]))


def normal_f32(g: np.random.Generator, shape, std: np.float32 | None = None) -> np.ndarray:
    a = g.standard_normal(shape, dtype=np.float32)
    if std is not None:
        a *= std
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of an fp32 array, via torch's CPU conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_valued(a: np.ndarray) -> np.ndarray:
    """fp32 array whose values are all bf16-representable (RNE of a)."""
    return bf16_bits_to_f32(to_bf16_bits(a))


# ---------------------------------------------------------------- router W

def router_weights(K: int = 2048, E: int = 256, seed: int = SEED_W) -> np.ndarray:
    """W [K,E] fp32 ~ N(0, 0.02)."""
    return normal_f32(rng(seed), (K, E), W_STD)


# ---------------------------------------------------------------- m-scan (19..80)

def mscan_fixed_request(K: int = 2048, n: int = 19) -> np.ndarray:
    """The fixed 19-token request, x fp32 ~ N(0,1)."""
    return normal_f32(rng(SEED_FIXED_REQUEST), (n, K))


def mscan_coarrivals(c: int, K: int = 2048) -> np.ndarray:
    """c co-arriving tokens, seeded by their count, x fp32 ~ N(0,1)."""
    return normal_f32(rng(SEED_COARRIVAL + c), (c, K))


def mscan_batch(c: int, K: int = 2048, fixed_first: bool = True):
    """(x [19+c, K], offset of the fixed rows)."""
    fx = mscan_fixed_request(K)
    co = mscan_coarrivals(c, K)
    if fixed_first:
        return np.concatenate([fx, co], axis=0), 0
    return np.concatenate([co, fx], axis=0), c


# ---------------------------------------------------------------- router sweep

SWEEP_MS = (1, 16, 64, 65, 75, 256, 1024, 4096, 8192)


def sweep_x(M: int = 8192, K: int = 2048, seed: int = 1003) -> np.ndarray:
    """bf16-valued activations ~ N(0,1), widened to fp32, [M,K].  A prefix
    x[:m] is the m-token batch of the sweep."""
    return bf16_valued(normal_f32(rng(seed), (M, K)))


# ---------------------------------------------------------------- tie-heavy router

TIE_K, TIE_E, TIE_TOPK = 4096, 512, 10


def tie_pairs(P: int, E: int = TIE_E, seed: int = SEED_TIES):
    """P disjoint column pairs (src, dst); for half of them dst > src and for
    the other half dst < src, so both tie-break directions occur."""
    g = rng(seed)
    perm = g.permutation(E)[: 2 * P]
    pairs = []
    for p in range(P):
        a, b = int(perm[2 * p]), int(perm[2 * p + 1])
        lo, hi = min(a, b), max(a, b)
        pairs.append((lo, hi) if p % 2 == 0 else (hi, lo))
    return pairs


def tie_weights(P: int, K: int = TIE_K, E: int = TIE_E, seed: int = SEED_TIES) -> np.ndarray:
    """W [K,E] ~ N(0,0.02) with P column pairs made near-identical: in even
    pairs W[:,dst] = W[:,src] exactly, in odd pairs W[:,dst] = W[:,src]*(1+2^-12),
    which stays within one bf16 step of the source column's logits."""
    W = normal_f32(rng(seed, 1), (K, E), W_STD)
    bump = np.float32(1.0 + 2.0 ** -12)
    for p, (src, dst) in enumerate(tie_pairs(P, E, seed)):
        W[:, dst] = W[:, src] if p % 2 == 0 else W[:, src] * bump
    return W


def tie_x(M: int = 4096, K: int = TIE_K, seed: int = SEED_TIES) -> np.ndarray:
    return bf16_valued(normal_f32(rng(seed, 2), (M, K)))


# ---------------------------------------------------------------- 40-layer prefill stack

STACK_LAYERS, STACK_TOKENS, STACK_REQUESTS = 40, 16384, 16
STACK_MIN_LEN, STACK_MAX_LEN = 64, 2048


def stack_lengths(total: int = STACK_TOKENS, n: int = STACK_REQUESTS, lo: int = STACK_MIN_LEN,
                  hi: int = STACK_MAX_LEN, seed: int = SEED_LENGTHS):
    """n request lengths in [lo, hi] summing to total: the first n-1 are drawn
    uniformly (rejection-sampled until the remainder is also in [lo, hi])."""
    g = rng(seed)
    while True:
        first = g.integers(lo, hi + 1, size=n - 1)
        last = total - int(first.sum())
        if lo <= last <= hi:
            return [int(v) for v in first] + [last]


def stack_layer_weights(layer: int, K: int = 2048, E: int = 256) -> np.ndarray:
    return normal_f32(rng(SEED_LAYER_W + layer), (K, E), W_STD)


def stack_request_x(request: int, layer: int, length: int, K: int = 2048) -> np.ndarray:
    """A request's activations at one layer: the same rows whether the request
    runs alone or inside the batch.  bf16-valued, ~N(0,1)."""
    return bf16_valued(normal_f32(rng(SEED_REQUEST + request, layer), (length, K)))


def stack_layer_x(layer: int, lengths, K: int = 2048) -> np.ndarray:
    return np.concatenate([stack_request_x(r, layer, L, K) for r, L in enumerate(lengths)], axis=0)


# ---------------------------------------------------------------- dense bf16 GEMM + gate

DENSE_MS = (19, 65, 75, 512, 4096)
DENSE_K = DENSE_N = 4096


def dense_x_bits(M: int = 4096, K: int = DENSE_K) -> np.ndarray:
    return to_bf16_bits(normal_f32(rng(SEED_DENSE), (M, K)))


def dense_w_bits(K: int = DENSE_K, N: int = DENSE_N) -> np.ndarray:
    return to_bf16_bits(normal_f32(rng(SEED_DENSE + 1), (K, N), W_STD))


def gate_w_bits(K: int = DENSE_K) -> np.ndarray:
    return to_bf16_bits(normal_f32(rng(SEED_DENSE + 2), (K,), W_STD))


# ---- after routing: expert outputs for the combine (stand-ins; no trained
# experts exist here).  D is the model width, the router's K.
SEED_MOE = 8000


def moe_expert_out_bits(P: int, D: int = 2048, seed: int = SEED_MOE) -> np.ndarray:
    """Per-slot expert outputs y [P,D] in grouped order, bf16 bits, N(0,1)."""
    return to_bf16_bits(normal_f32(rng(seed), (P, D)))


def moe_shared_out_bits(M: int, D: int = 2048, seed: int = SEED_MOE + 1) -> np.ndarray:
    """Shared-expert outputs [M,D], bf16 bits, N(0,1)."""
    return to_bf16_bits(normal_f32(rng(seed), (M, D)))


def moe_gate_w_bits(D: int = 2048, seed: int = SEED_MOE + 2) -> np.ndarray:
    """Shared-expert gate vector [D], bf16 bits, N(0, 0.02)."""
    return to_bf16_bits(normal_f32(rng(seed), (D,), W_STD))


def random_routes(M: int, k: int, E: int, seed: int) -> np.ndarray:
    """ids [M,k]: k distinct experts per token, uniformly drawn (rank order is
    irrelevant to grouping and combine)."""
    g = rng(seed)
    keys = g.random((M, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def expert_w_bits(E: int, K: int = 2048, N: int = 1024, seed: int = SEED_MOE + 3) -> np.ndarray:
    """Expert weights W [E,K,N] for the grouped GEMM, bf16 bits, N(0, 0.02).
    No expert width is given by the pages; N = 1024 (gate and up projections
    of width 512 side by side) is the stand-in."""
    return to_bf16_bits(normal_f32(rng(seed), (E, K, N), W_STD))
