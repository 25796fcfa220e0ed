"""Oracle invariants: selection equals a sort-based selection, ties go to the
lowest index, a row does not depend on its batch-mates, and special inputs
reduce to results fixed by plain mathematics."""
import os

import numpy as np
import pytest

import brute
import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sort_select(l, k):
    """Stable sort on (-value, index) via numpy, for finite values."""
    E = l.shape[-1]
    order = np.lexsort((np.arange(E), -l.astype(np.float64)))
    return order[:k]


def test_topk_equals_sort_selection():
    rng = np.random.default_rng(1)
    x = workloads.bf16_valued(rng.standard_normal((64, 256)).astype(np.float32))
    W = (rng.standard_normal((256, 64)) * 0.05).astype(np.float32)
    for logits_bf16 in (False, True):
        ids, _, lg, _ = oracle.route(x, W, 8, logits_bf16=logits_bf16)
        for m in range(x.shape[0]):
            assert list(ids[m]) == list(_sort_select(lg[m], 8))


def _golden_tiebreak():
    cases = []
    with open(os.path.join(GOLDEN, "tiebreak.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            k, vals, want = (p.strip() for p in line.split("|"))
            cases.append((int(k), [float(v) for v in vals.split()], [int(v) for v in want.split()]))
    return cases


@pytest.mark.parametrize("k,vals,want", _golden_tiebreak())
def test_golden_tiebreak(k, vals, want):
    # logits = x * W with x = [[1]] and W = the row of values: exact
    x = np.ones((1, 1), np.float32)
    W = np.array([vals], np.float32)
    ids, _, lg, _ = oracle.route(x, W, k)
    assert list(ids[0]) == want
    assert brute.select_topk_bruteforce([float(v) for v in lg[0]], k) == want


def _golden_ulps():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_ulps.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b, u = line.split()
                rows.append((int(a, 16), int(b, 16), int(u)))
    return rows


@pytest.mark.parametrize("a,b,want", _golden_ulps())
def test_golden_ulps(a, b, want):
    assert oracle.ulps(a, b) == want
    assert brute.bf16_steps(a, b) == want


def test_ulps_equals_step_count_exhaustively_sampled():
    rng = np.random.default_rng(3)
    finite = [b for b in range(0x10000) if ((b >> 7) & 0xFF) != 0xFF]
    for _ in range(3000):
        a, b = (int(v) for v in rng.choice(finite, 2))
        assert oracle.ulps(a, b) == brute.bf16_steps(a, b), (hex(a), hex(b))


def test_constructed_ties_resolve_to_lowest_index():
    """Duplicate W columns give bit-identical logits; whichever of the pair
    sits at the boundary, the lower index is selected."""
    rng = np.random.default_rng(4)
    K, E, k = 512, 64, 8
    x = rng.standard_normal((200, K)).astype(np.float32)
    W = (rng.standard_normal((K, E)) * 0.02).astype(np.float32)
    W[:, 40] = W[:, 7]
    W[:, 3] = W[:, 50]
    ids, _, lg, mg = oracle.route(x, W, k)
    assert np.array_equal(lg[:, 40], lg[:, 7]) and np.array_equal(lg[:, 3], lg[:, 50])
    n_boundary = 0
    for m in range(x.shape[0]):
        s = set(ids[m].tolist())
        for lo, hi in ((7, 40), (3, 50)):
            assert not (hi in s and lo not in s)  # never the higher without the lower
            if lo in s and hi not in s:
                n_boundary += 1
                assert mg[m]["ulps"] == 0 and mg[m]["sel_min"] == mg[m]["rej_max"]
    assert n_boundary > 0  # the construction did put a pair on the boundary


def test_row_independent_of_batch_mates():
    rng = np.random.default_rng(6)
    K, E = 640, 32
    W = (rng.standard_normal((K, E)) * 0.02).astype(np.float32)
    x = rng.standard_normal((40, K)).astype(np.float32)
    ids, w, lg, mg = oracle.route(x, W, 4, nthreads=3)
    for m in (0, 17, 39):
        ids1, w1, lg1, mg1 = oracle.route(x[m:m + 1], W, 4, nthreads=1)
        assert np.array_equal(lg1[0].view(np.uint32), lg[m].view(np.uint32))
        assert np.array_equal(ids1[0], ids[m])
        assert np.array_equal(w1[0].view(np.uint32), w[m].view(np.uint32))
        assert mg1[0].tobytes() == mg[m].tobytes()
    # inside a shuffled batch with other rows
    perm = rng.permutation(40)
    ids2, w2, lg2, mg2 = oracle.route(x[perm], W, 4, nthreads=5)
    assert np.array_equal(lg2.view(np.uint32), lg[perm].view(np.uint32))
    assert np.array_equal(ids2, ids[perm])


def test_integer_inputs_give_exact_integer_matmul():
    rng = np.random.default_rng(7)
    x = rng.integers(-8, 9, size=(9, 700)).astype(np.float32)
    W = rng.integers(-8, 9, size=(700, 24)).astype(np.float32)
    got = oracle.logits(x, W)
    want = x.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(got.astype(np.int64), want)
    assert np.array_equal(got, want.astype(np.float32))


def test_zero_rows_give_positive_zero():
    """Every chain starts at +0 and fma(+-0, w, +0) = +0 for finite w, so a
    row of zeros (either sign) gives +0.0 logits bit for bit, whatever the
    signs of W."""
    rng = np.random.default_rng(14)
    K, E = 600, 12
    W = rng.standard_normal((K, E)).astype(np.float32)
    # columns of one sign make every product of a -0 or +0 row the same
    # signed zero, so a chain started at -0 would end at -0
    W[:, 0] = np.abs(W[:, 0])
    W[:, 1] = -np.abs(W[:, 1])
    x = np.zeros((3, K), np.float32)
    x[1] = -0.0
    x[2, ::2] = -0.0
    got = oracle.logits(x, W)
    assert np.all(got.view(np.uint32) == 0)


def test_one_hot_row_returns_w_row():
    rng = np.random.default_rng(8)
    K, E = 1000, 48
    W = rng.standard_normal((K, E)).astype(np.float32)
    x = np.zeros((3, K), np.float32)
    for i, kk in enumerate((0, 255, 999)):
        x[i, kk] = 1.0
    got = oracle.logits(x, W)
    for i, kk in enumerate((0, 255, 999)):
        assert np.array_equal(got[i].view(np.uint32), W[kk].view(np.uint32))


def test_bf16_input_storage_equals_widened_fp32():
    rng = np.random.default_rng(9)
    xf = workloads.bf16_valued(rng.standard_normal((5, 300)).astype(np.float32))
    xb = workloads.to_bf16_bits(xf)
    W = (rng.standard_normal((300, 16)) * 0.02).astype(np.float32)
    a = oracle.route(xf, W, 3)
    b = oracle.route(xb, W, 3)
    for u, v in zip(a, b):
        assert u.tobytes() == v.tobytes()


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((33, 512)).astype(np.float32)
    W = (rng.standard_normal((512, 64)) * 0.02).astype(np.float32)
    ref = oracle.route(x, W, 6, nthreads=1)
    for nt in (2, 7, 0):
        got = oracle.route(x, W, 6, nthreads=nt)
        for u, v in zip(ref, got):
            assert u.tobytes() == v.tobytes()


def test_gate_dot_is_canonical_e1_and_sigmoid_is_accurate():
    rng = np.random.default_rng(12)
    K = 700
    x = rng.standard_normal((20, K)).astype(np.float32)
    w = (rng.standard_normal(K) * 0.02).astype(np.float32)
    dot, gate = oracle.gate_dot(x, w)
    lg = oracle.logits(x, w.reshape(K, 1))
    assert np.array_equal(dot.view(np.uint32), lg[:, 0].view(np.uint32))
    for m in range(3):
        assert brute.f32_bits(float(dot[m])) == brute.f32_bits(brute.canonical_dot(x[m], w, 256))
    want = 1.0 / (1.0 + np.exp(-dot.astype(np.float64)))
    rel = np.abs(gate - want) / want
    # exp within 2 ulp, then one add and one division
    assert rel.max() < 6 * 2.0 ** -24
    # bf16 storage of both operands equals the widened values
    xb, wb = workloads.to_bf16_bits(x), workloads.to_bf16_bits(w)
    d2, g2 = oracle.gate_dot(xb, wb)
    d3, g3 = oracle.gate_dot(workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb))
    assert d2.tobytes() == d3.tobytes() and g2.tobytes() == g3.tobytes()
    # saturation and symmetry closed forms
    xs = np.array([[200.0], [-200.0], [0.0]], np.float32)
    d4, g4 = oracle.gate_dot(xs, np.ones(1, np.float32))
    assert list(g4) == [1.0, 0.0, 0.5]


def test_gemm_reference_is_exact_on_integers():
    rng = np.random.default_rng(13)
    xi = rng.integers(-4, 5, size=(7, 300)).astype(np.float32)
    Wi = rng.integers(-4, 5, size=(300, 11)).astype(np.float32)
    out = oracle.gemm_bf16_ref(workloads.to_bf16_bits(xi), workloads.to_bf16_bits(Wi))
    assert np.array_equal(out, (xi.astype(np.int64) @ Wi.astype(np.int64)).astype(np.float32))
    xf = workloads.bf16_valued(rng.standard_normal((5, 64)).astype(np.float32))
    Wf = workloads.bf16_valued(rng.standard_normal((64, 9)).astype(np.float32))
    out2 = oracle.gemm_bf16_ref(workloads.to_bf16_bits(xf), workloads.to_bf16_bits(Wf))
    assert np.array_equal(out2, (xf.astype(np.float64) @ Wf.astype(np.float64)).astype(np.float32))


def test_invalid_arguments_rejected():
    x = np.ones((2, 4), np.float32)
    W = np.ones((4, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.route(x, W, 4)  # k > E
    with pytest.raises(ValueError):
        oracle.route(x, W, 0)
    ids, w, lg, mg = oracle.route(x[:0], W, 2)  # M = 0 is fine
    assert ids.shape == (0, 2)


@pytest.mark.parametrize("nb,G", [(8, 2), (8, 4), (8, 8), (4, 2), (16, 4)])
def test_k_shards_are_aligned_subtrees(nb, G):
    """With nb blocks and G shards of nb/G blocks (powers of two), the logits of
    each K shard are one aligned subtree of the canonical tree, so adding the
    shard logits pairwise, adjacent shards first, rebuilds the full logits
    bit for bit.  The expert shards' logits are the full logits' columns.  (The
    identity sharded routing relies on; a tree that carried odd partials up
    differently, or a chain over blocks, would fail it.)"""
    K, E, M = 256 * nb, 8, 24
    g = np.random.default_rng(nb * 10 + G)
    x = g.standard_normal((M, K)).astype(np.float32)
    W = (g.standard_normal((K, E)) * 0.05).astype(np.float32)
    full = oracle.route(x, W, 2)[2]
    ks = K // G
    parts = [oracle.route(x[:, i * ks:(i + 1) * ks], W[i * ks:(i + 1) * ks], 2)[2] for i in range(G)]
    while len(parts) > 1:
        parts = [(parts[i] + parts[i + 1]).astype(np.float32) for i in range(0, len(parts), 2)]
    assert np.array_equal(parts[0].view(np.uint32), full.view(np.uint32))
    cols = np.concatenate([oracle.route(x, np.ascontiguousarray(W[:, c:c + 4]), 1)[2] for c in (0, 4)], axis=1)
    assert np.array_equal(cols.view(np.uint32), full.view(np.uint32))
