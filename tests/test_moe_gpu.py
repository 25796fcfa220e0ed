"""Token permutation, row gather and MoE combine on the GPU against the oracle.

Permutation and gather are integer/byte work: bit-exact.  The combine is a
defined fp32 fmaf chain per element: bit-exact too.  Cases span the
one-launch permutation (one chunk of 512 tokens, or few assignments per
chunk) and the three-launch one (several chunks) with ragged tails, every expert
count the call accepts, both element types and the shared-expert term, row
widths on and off the 16-byte path, and the full routing workload (M=8192,
K=2048, E=256, k=8) end to end: route -> permute -> gather -> combine.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import dev, dev_bf16_bits, note, require_gpu

pytestmark = pytest.mark.gpu


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("M,k,E", [(1, 1, 64), (19, 8, 256), (1023, 8, 256), (1024, 8, 256), (1025, 8, 256),
                                   (3000, 10, 512), (300, 32, 1024), (2000, 1, 1024), (5000, 3, 7),
                                   (8192, 8, 256), (4097, 1, 1)])
def test_permute_matches_oracle(M, k, E):
    dr = require_gpu()
    if k > E:
        pytest.skip("k > E")
    ids = wl.random_routes(M, k, E, seed=M * 31 + k)
    note(f"moe_permute M={M} k={k} E={E}")
    off, rows, pos = dr.moe_permute(dev(ids), E)
    torch.cuda.synchronize()
    ro, rr, rp = oracle.moe_permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), ro)
    assert np.array_equal(rows.cpu().numpy(), rr)
    assert np.array_equal(pos.cpu().numpy(), rp)


def test_permute_empty_batch_writes_zero_offsets():
    dr = require_gpu()
    note("moe_permute M=0")
    off = torch.full((257,), 7, dtype=torch.int32, device="cuda")
    ids = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    dr.moe_permute(ids, 256, out=(off, torch.empty(0, dtype=torch.int32, device="cuda"),
                                  torch.empty((0, 8), dtype=torch.int32, device="cuda")))
    torch.cuda.synchronize()
    assert torch.all(off == 0)


@pytest.mark.parametrize("M", [40, 3000])  # one launch; three launches (several chunks)
def test_permute_skips_out_of_range_ids(M):
    dr = require_gpu()
    k, E = 4, 16
    ids = wl.random_routes(M, k, E, seed=5)
    ids[3, 1] = E
    ids[7, 0] = -2
    ids[M - 1, 3] = 1 << 20
    note(f"moe_permute with out-of-range ids M={M}")
    off, rows, pos = dr.moe_permute(dev(ids), E)
    torch.cuda.synchronize()
    off, rows, pos = off.cpu().numpy(), rows.cpu().numpy(), pos.cpu().numpy()
    assert pos[3, 1] == -1 and pos[7, 0] == -1 and pos[M - 1, 3] == -1
    valid = (ids >= 0) & (ids < E)
    assert off[-1] == valid.sum()
    # the valid assignments are grouped exactly as the oracle groups them once
    # the invalid ones are removed
    keys = np.where(valid, ids, E + 1).ravel()
    order = np.argsort(keys, kind="stable")[: valid.sum()]
    assert np.array_equal(rows[: valid.sum()], order // k)
    assert np.array_equal(off, np.r_[0, np.cumsum(np.bincount(ids[valid], minlength=E))])
    for m in range(M):
        for j in range(k):
            if valid[m, j]:
                assert rows[pos[m, j]] == m and off[ids[m, j]] <= pos[m, j] < off[ids[m, j] + 1]


@pytest.mark.parametrize("D", [1, 7, 8, 64, 2048, 2050])
def test_gather_matches_oracle(D):
    dr = require_gpu()
    g = np.random.default_rng(D)
    M, P = 300, 1000
    rows = g.integers(0, M, P).astype(np.int32)
    xf = g.standard_normal((M, D)).astype(np.float32)
    xb = wl.to_bf16_bits(xf)
    note(f"moe_gather f32 D={D}")
    out = dr.moe_gather(dev(xf), dev(rows))
    assert np.array_equal(_u32(out), oracle.moe_gather(xf, rows).view(np.uint32))
    note(f"moe_gather bf16 D={D}")
    out = dr.moe_gather(dev_bf16_bits(xb), dev(rows))
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), oracle.moe_gather(xb, rows))


def test_gather_out_of_range_rows_give_zero_rows():
    dr = require_gpu()
    x = np.arange(40, dtype=np.float32).reshape(5, 8) + 1
    rows = np.array([0, 5, -1, 4], np.int32)
    note("moe_gather out-of-range rows")
    out = dr.moe_gather(dev(x), dev(rows)).cpu().numpy()
    assert np.array_equal(out[0], x[0]) and np.array_equal(out[3], x[4])
    assert np.all(out[1] == 0) and np.all(out[2] == 0)


def _combine_case(M, k, E, D, y_bf16, shared_kind, seed):
    g = np.random.default_rng(seed)
    ids = wl.random_routes(M, k, E, seed=seed)
    _, _, pos = oracle.moe_permute(ids, E)
    w = g.random((M, k)).astype(np.float32)
    yf = g.standard_normal((M * k, D)).astype(np.float32)
    y = wl.to_bf16_bits(yf) if y_bf16 else yf
    shared = gate = None
    if shared_kind is not None:
        sf = g.standard_normal((M, D)).astype(np.float32)
        shared = wl.to_bf16_bits(sf) if shared_kind == "bf16" else sf
        gate = g.random(M).astype(np.float32)
    return ids, pos, w, y, shared, gate


def _dev_elem(a):
    return dev_bf16_bits(a) if a.dtype == np.uint16 else dev(a)


@pytest.mark.parametrize("y_bf16", [True, False])
@pytest.mark.parametrize("shared_kind", [None, "bf16", "f32"])
@pytest.mark.parametrize("M,k,D", [(1, 1, 1), (19, 8, 7), (19, 8, 8), (64, 10, 12), (300, 8, 2048),
                                   (33, 32, 260), (5, 8, 4100), (7, 8, 264), (3, 8, 4104)])
def test_combine_matches_oracle(y_bf16, shared_kind, M, k, D):
    dr = require_gpu()
    ids, pos, w, y, shared, gate = _combine_case(M, k, 64, D, y_bf16, shared_kind, seed=M + 7 * k + D)
    note(f"moe_combine M={M} k={k} D={D} y_bf16={y_bf16} shared={shared_kind}")
    out = dr.moe_combine(_dev_elem(y), dev(w), dev(ids), dev(pos),
                         None if shared is None else _dev_elem(shared), None if gate is None else dev(gate))
    want = oracle.moe_combine(y, w, ids, pos, shared, gate)
    assert np.array_equal(_u32(out), want.view(np.uint32))


def test_combine_is_independent_of_slot_order_and_batch():
    dr = require_gpu()
    M, k, E, D = 200, 8, 256, 2048
    ids, pos, w, y, shared, gate = _combine_case(M, k, E, D, True, "bf16", seed=11)
    yd, sd, gd = dev_bf16_bits(y), dev_bf16_bits(shared), dev(gate)
    note("moe_combine slot order")
    base = _u32(dr.moe_combine(yd, dev(w), dev(ids), dev(pos), sd, gd))
    perm = np.stack([np.random.default_rng(m).permutation(k) for m in range(M)])
    take = lambda a: np.ascontiguousarray(np.take_along_axis(a, perm, axis=1))  # noqa: E731
    got = _u32(dr.moe_combine(yd, dev(take(w)), dev(take(ids)), dev(take(pos)), sd, gd))
    assert np.array_equal(got, base)
    note("moe_combine token subset")
    sub = slice(37, 59)
    got = _u32(dr.moe_combine(yd, dev(w[sub]), dev(ids[sub]), dev(pos[sub]),
                              dev_bf16_bits(np.ascontiguousarray(shared[sub])), dev(gate[sub])))
    assert np.array_equal(got, base[sub])


def test_route_permute_gather_combine_full_workload():
    """The routing workload end to end: route M=8192 tokens (K=2048, E=256,
    k=8), group the assignments, gather the bf16 activations into grouped
    order, and combine stand-in bf16 expert outputs with the gated shared
    expert; every stage bit for bit against the oracle."""
    dr = require_gpu()
    M, K, E, k = 8192, 2048, 256, 8
    x = wl.sweep_x(M, K)
    W = wl.router_weights(K, E)
    note("full workload: route")
    ids, wts, _, _ = dr.route(dev(x), dev(W), k)
    ids_h, w_h = ids.cpu().numpy(), wts.cpu().numpy()
    rids, rw, _, _ = oracle.route(x, W, k)
    assert np.array_equal(ids_h, rids) and np.array_equal(w_h.view(np.uint32), rw.view(np.uint32))
    note("full workload: permute")
    off, rows, pos = dr.moe_permute(ids, E)
    ro, rr, rp = oracle.moe_permute(rids, E)
    assert np.array_equal(off.cpu().numpy(), ro) and np.array_equal(rows.cpu().numpy(), rr)
    assert np.array_equal(pos.cpu().numpy(), rp)
    note("full workload: gather")
    xb = wl.to_bf16_bits(x)
    xp = dr.moe_gather(dev_bf16_bits(xb), rows)
    assert np.array_equal(xp.cpu().view(torch.int16).numpy().view(np.uint16), xb[rr])
    note("full workload: combine")
    y = wl.moe_expert_out_bits(M * k, K)
    shared = wl.moe_shared_out_bits(M, K)
    gw = wl.moe_gate_w_bits(K)
    _, gate = dr.gate_dot(dev_bf16_bits(xb), dev_bf16_bits(gw))
    _, rgate = oracle.gate_dot(xb, gw)
    assert np.array_equal(_u32(gate), rgate.view(np.uint32))
    out = dr.moe_combine(dev_bf16_bits(y), wts, ids, pos, dev_bf16_bits(shared), gate)
    want = oracle.moe_combine(y, rw, rids, rp, shared, rgate)
    assert np.array_equal(_u32(out), want.view(np.uint32))
