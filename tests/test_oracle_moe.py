"""Pins for the oracle's token permutation and MoE combine.

The permutation is pinned to numpy's stable argsort of the flattened expert
ids (a library routine that states "group by expert, keep token order"
independently of the oracle's per-expert loop) and to special cases whose
answer is known in closed form.  The combine is pinned by exact-rational
recomputation of every fmaf on tiny inputs, by its defining property (the
result does not depend on the order of a token's k slots; vllm.cpp PR #2556,
section "Why a value tap could never have said this"), by integer inputs whose
sums are exact, and by the sign of an all-zero sum.  The grouped expert GEMM
reference is pinned per group to numpy's float64 matmul, to exact integer
products, and to its own pre-gathered form.
"""
import numpy as np
import pytest

import brute
import oracle


def _distinct_ids(rng, M, k, E):
    return np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32).reshape(M, k)


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("M,k,E", [(1, 1, 1), (5, 2, 4), (19, 8, 256), (64, 10, 512), (300, 8, 64),
                                   (33, 32, 64), (7, 4, 1024)])
def test_permute_matches_stable_argsort(M, k, E):
    rng = np.random.default_rng(M * 1000 + k)
    ids = _distinct_ids(rng, M, k, E)
    offsets, rows, pos = oracle.moe_permute(ids, E)
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")  # assignments grouped by expert, token order kept
    assert np.array_equal(rows, order // k)
    want_pos = np.empty(M * k, dtype=np.int64)
    want_pos[order] = np.arange(M * k)
    assert np.array_equal(pos.ravel(), want_pos)
    assert np.array_equal(offsets, np.r_[0, np.cumsum(np.bincount(flat, minlength=E))])
    # consistency: every assignment sits in its expert's range at a row naming its token
    for m in range(M):
        for j in range(k):
            p, e = pos[m, j], ids[m, j]
            assert offsets[e] <= p < offsets[e + 1] and rows[p] == m


def test_permute_closed_forms():
    # no tokens: every expert range is empty
    off, rows, pos = oracle.moe_permute(np.zeros((0, 3), np.int32), 8)
    assert np.array_equal(off, np.zeros(9, np.int32)) and rows.size == 0 and pos.size == 0
    # every token picks every expert (k = E), in any slot order: expert e's rows are 0..M-1
    M, E = 6, 4
    rng = np.random.default_rng(3)
    ids = np.stack([rng.permutation(E) for _ in range(M)]).astype(np.int32)
    off, rows, pos = oracle.moe_permute(ids, E)
    assert np.array_equal(off, np.arange(E + 1) * M)
    assert np.array_equal(rows, np.tile(np.arange(M), E))
    assert np.array_equal(pos, ids * M + np.arange(M)[:, None])
    # one expert, one slot: the identity
    off, rows, pos = oracle.moe_permute(np.zeros((5, 1), np.int32), 1)
    assert np.array_equal(off, [0, 5]) and np.array_equal(rows, np.arange(5)) and np.array_equal(pos[:, 0], np.arange(5))


def test_permute_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.moe_permute(np.array([[0, 4]], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.moe_permute(np.array([[1, -1]], np.int32), 4)
    with pytest.raises(ValueError):
        oracle.moe_permute(np.array([[2, 2]], np.int32), 4)


def test_gather_is_row_indexing():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((9, 13)).astype(np.float32)
    rows = rng.integers(0, 9, 20).astype(np.int32)
    assert np.array_equal(oracle.moe_gather(x, rows).view(np.uint32), x[rows].view(np.uint32))
    xb = rng.integers(0, 1 << 16, (9, 13)).astype(np.uint16)
    assert np.array_equal(oracle.moe_gather(xb, rows), xb[rows])


def _case(rng, M, k, E, D, kind):
    ids = _distinct_ids(rng, M, k, E)
    _, _, pos = oracle.moe_permute(ids, E)
    P = M * k
    if kind == "normal":
        y = rng.standard_normal((P, D)).astype(np.float32)
        w = rng.random((M, k)).astype(np.float32)
    elif kind == "cancel":  # large terms of both signs: the order decides the rounding
        y = (rng.standard_normal((P, D)) * np.float32(2.0) ** rng.integers(-30, 30, (P, D))).astype(np.float32)
        w = (rng.random((M, k)) * 2 - 1).astype(np.float32)
    else:  # tiny values: subnormal products
        y = (rng.standard_normal((P, D)) * np.float32(1e-20)).astype(np.float32)
        w = (rng.random((M, k)) * np.float32(1e-20)).astype(np.float32)
    return ids, w, pos, y


def _exact_combine(ids, w, pos, y, shared=None, gate=None):
    M, k = ids.shape
    D = y.shape[1]
    out = np.empty((M, D), dtype=np.float32)
    for m in range(M):
        order = sorted(range(k), key=lambda s: (int(ids[m, s]), s))
        for d in range(D):
            acc = 0.0
            for s in order:
                acc = brute.fma(float(w[m, s]), float(y[pos[m, s], d]), acc)
            if shared is not None:
                acc = brute.fma(float(gate[m]), float(shared[m, d]), acc)
            out[m, d] = acc
    return out


@pytest.mark.parametrize("kind", ["normal", "cancel", "tiny"])
def test_combine_matches_exact_rounding(kind):
    rng = np.random.default_rng({"normal": 1, "cancel": 2, "tiny": 3}[kind])
    ids, w, pos, y = _case(rng, 4, 5, 9, 6, kind)
    got = oracle.moe_combine(y, w, ids, pos)
    assert np.array_equal(_bits(got), _bits(_exact_combine(ids, w, pos, y)))
    shared = rng.standard_normal((4, 6)).astype(np.float32)
    gate = rng.random(4).astype(np.float32)
    got = oracle.moe_combine(y, w, ids, pos, shared, gate)
    assert np.array_equal(_bits(got), _bits(_exact_combine(ids, w, pos, y, shared, gate)))


def test_combine_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(5)
    ids, w, pos, y = _case(rng, 3, 4, 8, 5, "normal")
    yb = (y.view(np.uint32) >> 16).astype(np.uint16)  # truncation gives some bf16 values
    yw = (yb.astype(np.uint32) << 16).view(np.float32)
    sb = yb[:3]
    gate = rng.random(3).astype(np.float32)
    got = oracle.moe_combine(yb, w, ids, pos, sb, gate)
    want = _exact_combine(ids, w, pos, yw, yw[:3], gate)
    assert np.array_equal(_bits(got), _bits(want))


def test_combine_does_not_depend_on_slot_order():
    rng = np.random.default_rng(6)
    ids, w, pos, y = _case(rng, 40, 8, 64, 16, "cancel")
    base = oracle.moe_combine(y, w, ids, pos)
    for trial in range(5):
        perm = np.stack([rng.permutation(8) for _ in range(40)])
        take = lambda a: np.take_along_axis(a, perm, axis=1)  # noqa: E731
        got = oracle.moe_combine(y, take(w), take(ids), take(pos))
        assert np.array_equal(_bits(got), _bits(base)), f"trial {trial}"


def test_combine_integer_inputs_are_exact():
    rng = np.random.default_rng(7)
    M, k, E, D = 30, 6, 32, 9
    ids = _distinct_ids(rng, M, k, E)
    _, _, pos = oracle.moe_permute(ids, E)
    y = rng.integers(-1000, 1000, (M * k, D)).astype(np.float32)
    w = rng.integers(-50, 50, (M, k)).astype(np.float32)
    shared = rng.integers(-1000, 1000, (M, D)).astype(np.float32)
    gate = rng.integers(-3, 4, M).astype(np.float32)
    want = (np.einsum("mk,mkd->md", w.astype(np.int64), y[pos].astype(np.int64))
            + gate.astype(np.int64)[:, None] * shared.astype(np.int64))
    got = oracle.moe_combine(y, w, ids, pos, shared, gate)
    assert np.array_equal(got.astype(np.int64), want)


def test_combine_zero_sum_is_positive_zero():
    # every product is -0: the chain starts at +0, and -0 + +0 = +0
    M, k, D = 2, 3, 4
    ids = np.array([[2, 0, 1], [1, 2, 0]], np.int32)
    _, _, pos = oracle.moe_permute(ids, 3)
    y = np.zeros((M * k, D), np.float32)
    w = -np.ones((M, k), np.float32)
    got = oracle.moe_combine(y, w, ids, pos)
    assert np.all(_bits(got) == 0)


def test_combine_shared_term_comes_last():
    # two slot terms 2^-24 and the shared term 1.0: summed slots first give
    # 1 + 2^-23 exactly; the shared term first would absorb both small terms
    ids = np.array([[1, 0]], np.int32)
    _, _, pos = oracle.moe_permute(ids, 2)
    y = np.full((2, 1), 2.0 ** -24, np.float32)
    w = np.ones((1, 2), np.float32)
    got = oracle.moe_combine(y, w, ids, pos, np.ones((1, 1), np.float32), np.ones(1, np.float32))
    assert got[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_combine_ascending_expert_order_is_distinguished():
    # slot terms 1.0 (expert 0), 2^-24 and 2^-24 (experts 1, 2): ascending
    # expert order gives 1.0 (each small term is absorbed); the small terms
    # first would give 1 + 2^-23
    ids = np.array([[2, 1, 0]], np.int32)
    _, _, pos = oracle.moe_permute(ids, 3)
    y = np.array([[2.0 ** -24], [2.0 ** -24], [1.0]], np.float32)[::-1].copy()  # rows by expert: 0 -> 1.0
    w = np.ones((1, 3), np.float32)
    got = oracle.moe_combine(y, w, ids, pos)
    assert y[pos[0, 2], 0] == 1.0 and got[0, 0] == np.float32(1.0)


def test_combine_rejects_bad_positions():
    with pytest.raises(ValueError):
        oracle.moe_combine(np.zeros((2, 3), np.float32), np.ones((1, 2), np.float32),
                           np.array([[0, 1]], np.int32), np.array([[0, 2]], np.int32))


# ---- grouped expert GEMM reference

def _bf16_bits(a):
    import workloads as wl
    return wl.to_bf16_bits(np.asarray(a, dtype=np.float32))


def _widen(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_grouped_gemm_ref_matches_numpy_per_group():
    rng = np.random.default_rng(21)
    E, K, N, Mx = 5, 96, 40, 30
    counts = np.array([7, 0, 12, 1, 20])
    offsets = np.r_[0, np.cumsum(counts)].astype(np.int32)
    P = int(offsets[-1])
    x = _bf16_bits(rng.standard_normal((Mx, K)))
    W = _bf16_bits(rng.standard_normal((E, K, N)) * 0.1)
    rows = rng.integers(0, Mx, P).astype(np.int32)
    got = oracle.grouped_gemm_bf16_ref(x, W, offsets, rows)
    for e in range(E):
        seg = slice(offsets[e], offsets[e + 1])
        want = (_widen(x)[rows[seg]].astype(np.float64) @ _widen(W[e]).astype(np.float64)).astype(np.float32)
        assert np.allclose(got[seg], want, rtol=1e-6, atol=1e-6)


def test_grouped_gemm_ref_exact_on_integers_and_rows_equal_pregathered():
    rng = np.random.default_rng(22)
    E, K, N, Mx = 3, 64, 16, 9
    offsets = np.array([0, 4, 4, 11], np.int32)
    x = _bf16_bits(rng.integers(-8, 8, (Mx, K)))
    W = _bf16_bits(rng.integers(-8, 8, (E, K, N)))
    rows = rng.integers(0, Mx, 11).astype(np.int32)
    got = oracle.grouped_gemm_bf16_ref(x, W, offsets, rows)
    xi = _widen(x).astype(np.int64)
    Wi = _widen(W).astype(np.int64)
    for e in range(E):
        for p in range(offsets[e], offsets[e + 1]):
            assert np.array_equal(got[p].astype(np.int64), xi[rows[p]] @ Wi[e])
    pre = oracle.grouped_gemm_bf16_ref(np.ascontiguousarray(x[rows]), W, offsets)
    assert np.array_equal(pre.view(np.uint32), got.view(np.uint32))


def test_grouped_gemm_ref_rejects_inconsistent_offsets():
    x = np.zeros((4, 32), np.uint16)
    W = np.zeros((2, 32, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.grouped_gemm_bf16_ref(x, W, np.array([0, 3, 2], np.int32))
    with pytest.raises(ValueError):
        oracle.grouped_gemm_bf16_ref(x, W, np.array([0, 2, 4], np.int32), rows=np.array([0, 1, 2, 9], np.int32))
