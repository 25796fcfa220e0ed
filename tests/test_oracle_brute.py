"""The oracle against exact-arithmetic brute force on tiny inputs.

Every fmaf and add of the canonical order is recomputed in exact rationals and
rounded to nearest-even by hand (tests/brute.py); selection is checked against
an exhaustive search over all k-subsets; the margin's ULP count against a count
of representable bf16 steps.  A plausible slip in the oracle -- a dropped block,
a different grouping, a mul+add instead of fmaf, a highest-index tie-break, a
two's-complement ULP count -- changes at least one of these bits.
"""
import math

import numpy as np
import pytest

import brute
import oracle


def _rand_case(rng, M, K, E, kind):
    if kind == "normal":
        x = rng.standard_normal((M, K)).astype(np.float32)
        W = (rng.standard_normal((K, E)) * 0.02).astype(np.float32)
    elif kind == "subnormal":
        # products land in the fp32 subnormal range and some partials round
        x = (rng.standard_normal((M, K)) * 2.0 ** -70).astype(np.float32)
        W = (rng.standard_normal((K, E)) * 2.0 ** -70).astype(np.float32)
    elif kind == "cancel":
        # huge terms that cancel across blocks, small terms that only survive
        # under one grouping
        x = rng.choice(np.array([1e8, -1e8, 1.0, -1.0, 3.0], np.float32), size=(M, K))
        W = rng.choice(np.array([1.0, 0.5, -1.0, 1e-3], np.float32), size=(K, E))
    elif kind == "zeros":
        x = rng.choice(np.array([0.0, -0.0, 1.0, -1.0], np.float32), size=(M, K))
        W = rng.choice(np.array([0.0, -0.0, 2.0, -0.5], np.float32), size=(K, E))
    elif kind == "wide":
        x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-20, 20, (M, K)))).astype(np.float32)
        W = (rng.standard_normal((K, E)) * np.exp2(rng.integers(-20, 20, (K, E)))).astype(np.float32)
    else:
        raise ValueError(kind)
    return x, W


@pytest.mark.parametrize("kind", ["normal", "subnormal", "cancel", "zeros", "wide"])
@pytest.mark.parametrize("kblock", [1, 2, 3, 4, 7, 64])
def test_logits_match_exact_rounding(kind, kblock):
    rng = np.random.default_rng(hash((kind, kblock)) % 2**32)
    for trial in range(3):
        M, K, E = int(rng.integers(1, 4)), int(rng.integers(1, 41)), int(rng.integers(1, 7))
        x, W = _rand_case(rng, M, K, E, kind)
        got = oracle.logits(x, W, kblock=kblock)
        for m in range(M):
            for e in range(E):
                want = brute.canonical_dot(x[m], W[:, e], kblock)
                assert brute.f32_bits(float(got[m, e])) == brute.f32_bits(want), (kind, kblock, m, e, got[m, e], want)


def test_single_block_is_one_sequential_chain():
    rng = np.random.default_rng(5)
    x, W = _rand_case(rng, 2, 37, 3, "normal")
    got = oracle.logits(x, W, kblock=37)
    for m in range(2):
        for e in range(3):
            assert brute.f32_bits(float(got[m, e])) == brute.f32_bits(brute.sequential_dot(x[m], W[:, e]))


def test_tree_grouping_is_distinguished():
    """Block partials 1e8, 1, -1e8, 1 (kblock=1): the pairwise tree gives
    (1e8+1)+(-1e8+1) = 0, a left-to-right sum gives 1, a right fold gives 0 by a
    different route; the oracle must give the tree's value."""
    x = np.array([[1e8, 1.0, -1e8, 1.0]], np.float32)
    W = np.ones((4, 1), np.float32)
    got = float(oracle.logits(x, W, kblock=1)[0, 0])
    assert got == 0.0
    seq = brute.add(brute.add(brute.add(1e8, 1.0), -1e8), 1.0)
    assert seq == 1.0  # the test has teeth: another grouping differs
    # odd count: 5 partials -> ((p0+p1)+(p2+p3)) + p4
    x5 = np.array([[1e8, 1.0, -1e8, 1.0, 0.75]], np.float32)
    got5 = float(oracle.logits(x5, np.ones((5, 1), np.float32), kblock=1)[0, 0])
    assert got5 == 0.75


def test_fma_not_mul_add():
    """(1+2^-12)^2 - 1 = 2^-11 + 2^-24 exactly.  Chain -1*1 then a*a: the
    second step is fmaf(a, a, -1), which keeps the 2^-24 term; a rounded
    product followed by an add would lose it.  In the other order the first
    product is rounded on its own (fmaf(a, a, +0)) and both agree on 2^-11."""
    a = np.float32(1.0 + 2.0 ** -12)
    x2 = np.array([[-1.0, a]], np.float32)
    W2 = np.array([[1.0], [a]], np.float32)
    assert float(oracle.logits(x2, W2, kblock=2)[0, 0]) == 2.0 ** -11 + 2.0 ** -24
    x = np.array([[a, -1.0]], np.float32)
    W = np.array([[a], [1.0]], np.float32)
    assert float(oracle.logits(x, W, kblock=2)[0, 0]) == 2.0 ** -11


@pytest.mark.parametrize("E,k", [(1, 1), (3, 2), (5, 5), (6, 3), (8, 2), (8, 7)])
def test_selection_and_margin_bruteforce(E, k):
    rng = np.random.default_rng(E * 31 + k)
    for trial in range(12):
        M, K = 3, int(rng.integers(1, 9))
        # small integers: logits are exact small integers with many ties
        x = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
        W = rng.integers(-2, 3, size=(K, E)).astype(np.float32)
        if trial % 3 == 0:
            W *= np.float32(1.0 / 3.0)  # inexact values, fewer ties
        ids, w, lg, mg = oracle.route(x, W, k)
        for m in range(M):
            vals = [brute.canonical_dot(x[m], W[:, e], 256) for e in range(E)]
            ranked = brute.select_topk_bruteforce(vals, k)
            assert list(ids[m]) == ranked, (vals, ids[m], ranked)
            sel = vals[ranked[-1]]
            assert brute.f32_bits(float(mg[m]["sel_min"])) == brute.f32_bits(sel)
            assert int(mg[m]["sel_min_bf16"]) == brute.bf16_bits(sel)
            if k < E:
                rest = sorted((e for e in range(E) if e not in ranked), key=lambda e: (-vals[e], e))
                rej = vals[rest[0]]
                assert brute.f32_bits(float(mg[m]["rej_max"])) == brute.f32_bits(rej)
                assert int(mg[m]["rej_max_bf16"]) == brute.bf16_bits(rej)
                assert int(mg[m]["ulps"]) == brute.bf16_steps(brute.bf16_bits(sel), brute.bf16_bits(rej))
            else:
                assert float(mg[m]["rej_max"]) == -math.inf
                assert int(mg[m]["rej_max_bf16"]) == 0xFF80
                assert int(mg[m]["ulps"]) == 2**31 - 1


def test_bf16_logit_mode_selects_on_rounded_values():
    """Two logits that differ in fp32 but round to the same bf16 value tie in
    bf16 mode, so the lower index wins even though it is the smaller fp32."""
    lo_val = np.float32(1.0 + 2.0 ** -10)       # rounds to 1.0 in bf16
    hi_val = np.float32(1.0 + 3 * 2.0 ** -10)   # also rounds to 1.0 in bf16
    x = np.ones((1, 1), np.float32)
    W = np.array([[lo_val, hi_val, 0.5]], np.float32)
    ids32, _, _, mg32 = oracle.route(x, W, 1)
    ids16, _, lg16, mg16 = oracle.route(x, W, 1, logits_bf16=True)
    assert ids32[0, 0] == 1
    assert ids16[0, 0] == 0
    assert lg16[0, 0] == 1.0 and lg16[0, 1] == 1.0
    assert mg16[0]["ulps"] == 0
    assert brute.bf16_bits(float(lo_val)) == brute.bf16_bits(float(hi_val)) == 0x3F80


def test_weights_against_float64_softmax():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    W = (rng.standard_normal((64, 32))).astype(np.float32)
    for renorm in (False, True):
        ids, w, lg, _ = oracle.route(x, W, 5, renormalize=renorm)
        # the exponent's argument is the fp32 difference l - max (one IEEE
        # subtraction, as the method defines it); from there on float64
        t32 = (lg - lg.max(axis=1, keepdims=True)).astype(np.float32)
        p = np.exp(t32.astype(np.float64))
        p /= p.sum(axis=1, keepdims=True)
        want = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        if renorm:
            want = want / want.sum(axis=1, keepdims=True)
        rel = np.abs(w.astype(np.float64) - want) / want
        # exp within 2 ulp, a depth-5 tree of positive terms, one division;
        # renormalising adds a k-term sum and a second division
        bound = (10 if renorm else 8) * 2.0 ** -24
        assert rel.max() < bound, rel.max()


def test_weights_exact_tree_denominator():
    """Weights bit for bit from exact rationals: u_e = expf(l_e - max) with
    the oracle's exp (pinned on its own), the denominator the pairwise tree of
    the u_e in index order with each add rounded to nearest-even, one rounded
    division per weight; renormalisation by the left-to-right sum of the k
    weights.  A sequential denominator or another grouping changes bits."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    E, k = 48, 6
    x = rng.standard_normal((12, 40)).astype(np.float32)
    W = (rng.standard_normal((40, E)) * 0.7).astype(np.float32)
    for renorm in (False, True):
        ids, w, lg, _ = oracle.route(x, W, k, renormalize=renorm)
        for m in range(x.shape[0]):
            l = lg[m]
            mx = np.float32(l[ids[m, 0]])
            u = oracle.expf((l - mx).astype(np.float32))
            s = brute.tree([float(v) for v in u])
            want = [brute.rne_f32(Fraction(float(u[i])) / Fraction(s)) for i in ids[m]]
            if renorm:
                r = want[0]
                for v in want[1:]:
                    r = brute.add(r, v)
                want = [brute.rne_f32(Fraction(v) / Fraction(r)) for v in want]
            got = [float(v) for v in w[m]]
            assert [brute.f32_bits(v) for v in got] == [brute.f32_bits(v) for v in want], (renorm, m)
