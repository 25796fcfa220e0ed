"""The oracle's selection on given logits (dro_select) against exhaustive
search, and against the selection dro_route makes on its own logits.

dro_select is the part of dro_route after the logits; the GPU's
dr_route_select is compared with it.  Pins: the ranking is the unique k-subset
in which every selected expert beats every rejected one (larger value, or the
same value and a lower index) -- "vllm.cpp PR #2556", summary: the
lowest-index tie-break -- and the margin's ULP count is the number of bf16
steps between the two values ("Why a value tap could never have said this").
"""
import math

import numpy as np
import pytest

import brute
import oracle


@pytest.mark.parametrize("E,k", [(1, 1), (4, 2), (6, 6), (7, 3), (9, 8)])
def test_select_matches_exhaustive_search(E, k):
    rng = np.random.default_rng(100 + E * 7 + k)
    # few distinct values: many exact ties, both zeros, infinities
    pool = np.array([0.0, -0.0, 1.0, -1.0, 0.5, 2.0, np.inf, -np.inf, 1.0 + 2.0 ** -20], np.float32)
    lg = rng.choice(pool, size=(40, E)).astype(np.float32)
    ids, w, mg = oracle.select(lg, k)
    for m in range(lg.shape[0]):
        vals = [float(v) for v in lg[m]]
        ranked = brute.select_topk_bruteforce(vals, k)
        assert list(ids[m]) == ranked, (vals, ids[m], ranked)
        sel = vals[ranked[-1]]
        assert int(mg[m]["sel_min_bf16"]) == brute.bf16_bits(sel)
        if k < E:
            rest = sorted((e for e in range(E) if e not in ranked), key=lambda e: (-vals[e], e))
            rej = vals[rest[0]]
            assert int(mg[m]["rej_max_bf16"]) == brute.bf16_bits(rej)
            if math.isfinite(sel) and math.isfinite(rej):
                assert int(mg[m]["ulps"]) == brute.bf16_steps(brute.bf16_bits(sel), brute.bf16_bits(rej))
        else:
            assert float(mg[m]["rej_max"]) == -math.inf and int(mg[m]["ulps"]) == 2**31 - 1


def test_signed_zero_values_are_reported_exactly():
    """-0 and +0 tie (the lower index wins) but the margin keeps each value's
    own sign bit."""
    lg = np.array([[-0.0, 0.0, -1.0]], np.float32)
    ids, _, mg = oracle.select(lg, 1)
    assert ids[0, 0] == 0
    assert brute.f32_bits(float(mg[0]["sel_min"])) == 0x80000000
    assert brute.f32_bits(float(mg[0]["rej_max"])) == 0x00000000
    assert int(mg[0]["ulps"]) == 0


def test_nan_ranks_last():
    lg = np.array([[np.nan, -np.inf, 3.0, np.nan]], np.float32)
    ids, _, _ = oracle.select(lg, 4)
    assert list(ids[0]) == [2, 1, 0, 3]


@pytest.mark.parametrize("logits_bf16", [False, True])
@pytest.mark.parametrize("renorm", [False, True])
def test_select_reproduces_route(logits_bf16, renorm):
    """dro_route = logits, then dro_select on the values the selection saw."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((64, 300)).astype(np.float32)
    W = (rng.standard_normal((300, 64)) * 0.05).astype(np.float32)
    ids, w, lg, mg = oracle.route(x, W, 6, logits_bf16=logits_bf16, renormalize=renorm)
    ids2, w2, mg2 = oracle.select(lg, 6, renormalize=renorm)
    assert np.array_equal(ids, ids2)
    assert np.array_equal(w.view(np.uint32), w2.view(np.uint32))
    assert np.array_equal(mg.view(np.uint8), mg2.view(np.uint8))
