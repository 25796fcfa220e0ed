"""Batch-invariant grouped expert GEMM on the GPU.

Each output row must (a) be bit-identical to dr_gemm_bf16 of that one row
with its expert's weights -- the same instruction sequence -- whatever the
size and position of its group; (b) be bit-identical between the fused
gather (token-order x through rows) and pre-gathered rows; (c) keep its bits
when the token is routed in a different batch (other group sizes and
offsets); and (d) lie within 1e-2 of the oracle's exact product.  Cases cover
empty experts, one expert, partial K stages, ragged group ends and the
routing workload's 65536 grouped rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import dev, dev_bf16_bits, note, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


def _routes_and_groups(dr, M, k, E, seed):
    ids = wl.random_routes(M, k, E, seed)
    off, rows, pos = dr.moe_permute(dev(ids), E)
    return ids, off, rows, pos


# 128 x 128 tiles below 128 rows per expert on average, 256 x 256 from there
# (the last case: groups of ~300 rows, most in one 320-row tile, some in a
# full and a ragged 256-row tile, and a partial K stage)
@pytest.mark.parametrize("M,k,E,K,N", [(1, 1, 1, 32, 128), (5, 2, 8, 96, 128), (300, 4, 16, 256, 256),
                                       (700, 8, 64, 160, 384), (2048, 8, 256, 2048, 256), (1200, 8, 32, 160, 256)])
def test_grouped_matches_dense_rows_and_oracle(M, k, E, K, N):
    dr = require_gpu()
    g = np.random.default_rng(M + E)
    xb = wl.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    Wb = wl.to_bf16_bits((g.standard_normal((E, K, N)) * 0.02).astype(np.float32))
    ids, off, rows, pos = _routes_and_groups(dr, M, k, E, seed=M * 7 + E)
    xd, Wd = dev_bf16_bits(xb), dev_bf16_bits(Wb)
    note(f"grouped gemm M={M} k={k} E={E} K={K} N={N} (fused gather)")
    out = dr.grouped_gemm_bf16(xd, Wd, off, rows)
    note("grouped gemm pre-gathered")
    xp = dr.moe_gather(xd, rows)
    out2 = dr.grouped_gemm_bf16(xp, Wd, off)
    got = _u32(out)
    assert np.array_equal(got, _u32(out2))
    off_h, rows_h = off.cpu().numpy(), rows.cpu().numpy()
    # every expert with rows: its rows equal the dense GEMM of those rows with W[e]
    experts = [e for e in range(E) if off_h[e + 1] > off_h[e]]
    for e in experts[:: max(1, len(experts) // 12)]:
        seg = slice(off_h[e], off_h[e + 1])
        note(f"dense rows of expert {e}")
        dense = dr.gemm_bf16(dev_bf16_bits(np.ascontiguousarray(xb[rows_h[seg]])), dev_bf16_bits(Wb[e]))
        assert np.array_equal(got[seg], _u32(dense)), f"expert {e}"
    # within the tolerance of the exact product on sampled rows (all rows when small)
    P = M * k
    sample = np.arange(P) if P <= 512 else np.unique(np.r_[0, P - 1, g.integers(0, P, 256)])
    ref = np.empty((sample.size, N), np.float32)
    e_of = np.searchsorted(off_h, sample, side="right") - 1
    for i, (p, e) in enumerate(zip(sample, e_of)):
        ref[i] = oracle.gemm_bf16_ref(xb[rows_h[p]][None, :], Wb[e])[0]
    err = np.abs(out.cpu().numpy()[sample].astype(np.float64) - ref)
    assert err.max() <= TOL, err.max()


def test_grouped_matches_oracle_reference_whole():
    dr = require_gpu()
    g = np.random.default_rng(3)
    M, k, E, K, N = 150, 3, 12, 128, 128
    xb = wl.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    Wb = wl.to_bf16_bits((g.standard_normal((E, K, N)) * 0.05).astype(np.float32))
    ids, off, rows, pos = _routes_and_groups(dr, M, k, E, seed=3)
    note("grouped gemm whole-output oracle comparison")
    out = dr.grouped_gemm_bf16(dev_bf16_bits(xb), dev_bf16_bits(Wb), off, rows).cpu().numpy()
    ref = oracle.grouped_gemm_bf16_ref(xb, Wb, off.cpu().numpy(), rows.cpu().numpy())
    assert np.abs(out.astype(np.float64) - ref).max() <= TOL


def test_grouped_rows_do_not_depend_on_the_batch():
    """A token routed alone-ish (37 tokens) and inside 4096 tokens: its rows
    sit in groups of different sizes at different offsets, with the same bits
    (the two batches also run different tile configurations)."""
    dr = require_gpu()
    M, k, E, K, N = 4096, 8, 64, 512, 256
    g = np.random.default_rng(9)
    xb = wl.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    Wd = dev_bf16_bits(wl.to_bf16_bits((g.standard_normal((E, K, N)) * 0.02).astype(np.float32)))
    ids = wl.random_routes(M, k, E, seed=9)
    outs = {}
    for lo, hi in ((0, M), (100, 137)):
        note(f"grouped gemm batch tokens {lo}..{hi}")
        idd = dev(np.ascontiguousarray(ids[lo:hi]))
        off, rows, pos = dr.moe_permute(idd, E)
        out = dr.grouped_gemm_bf16(dev_bf16_bits(np.ascontiguousarray(xb[lo:hi])), Wd, off, rows)
        outs[(lo, hi)] = (_u32(out), pos.cpu().numpy())
    big, pos_big = outs[(0, M)]
    small, pos_small = outs[(100, 137)]
    for m in range(37):
        for j in range(k):
            assert np.array_equal(small[pos_small[m, j]], big[pos_big[100 + m, j]]), (m, j)


def test_grouped_out_of_range_rows_read_zero_rows():
    dr = require_gpu()
    K, N, E = 64, 128, 2
    x = dev_bf16_bits(wl.to_bf16_bits(np.ones((4, K), np.float32)))
    W = dev_bf16_bits(wl.to_bf16_bits(np.ones((E, K, N), np.float32)))
    off = dev(np.array([0, 3, 5], np.int32))
    rows = dev(np.array([0, 9, 2, -1, 3], np.int32))
    note("grouped gemm out-of-range rows")
    out = dr.grouped_gemm_bf16(x, W, off, rows).cpu().numpy()
    assert np.all(out[[0, 2, 4]] == K) and np.all(out[[1, 3]] == 0)


def test_grouped_tall_tiles_at_their_bounds():
    """From 256 rows per expert on average the 256 x 256 tile runs; an
    expert of 257 to 320 rows takes one 320-row tile instead of a full and a
    ragged one, and one of 321 to 384 rows that tile and a second pass over
    its last rows in the same workgroup: groups of exactly 256, 257, 288,
    300, 320, 321, 352 and 384 rows, 385 (a full and a ragged 256-row tile),
    one row and none, with a partial last K stage.  Every row equals the
    dense GEMM of that row with its expert's weights, bit for bit; sampled
    rows lie within the tolerance of the exact product."""
    dr = require_gpu()
    sizes = [257, 320, 321, 256, 1, 0, 300, 288, 352, 384, 385]
    E, K, N = len(sizes), 160, 512
    off_h = np.r_[0, np.cumsum(sizes)].astype(np.int32)
    P = int(off_h[-1])
    g = np.random.default_rng(12)
    xb = wl.to_bf16_bits(g.standard_normal((P, K)).astype(np.float32))
    Wb = wl.to_bf16_bits((g.standard_normal((E, K, N)) * 0.02).astype(np.float32))
    Wd = dev_bf16_bits(Wb)
    note(f"grouped gemm tall tiles, groups {sizes}")
    out = dr.grouped_gemm_bf16(dev_bf16_bits(xb), Wd, dev(off_h))
    got = _u32(out)
    for e in range(E):
        if sizes[e] == 0:
            continue
        seg = slice(off_h[e], off_h[e + 1])
        note(f"dense rows of expert {e} ({sizes[e]} rows)")
        dense = dr.gemm_bf16(dev_bf16_bits(np.ascontiguousarray(xb[seg])), dev_bf16_bits(Wb[e]))
        assert np.array_equal(got[seg], _u32(dense)), f"expert {e} ({sizes[e]} rows)"
    sample = np.unique(np.r_[off_h[:-1][np.array(sizes) > 0], off_h[1:][np.array(sizes) > 0] - 1, g.integers(0, P, 32)])
    e_of = np.searchsorted(off_h, sample, side="right") - 1
    outh = out.cpu().numpy()
    for p, e in zip(sample, e_of):
        ref = oracle.gemm_bf16_ref(xb[p][None, :], Wb[e])[0]
        assert np.abs(outh[p].astype(np.float64) - ref).max() <= TOL, (p, e)


def test_grouped_full_size_sampled():
    """The routing workload's size: 8192 tokens, k=8 (65536 grouped rows, 193-324
    per expert, so experts take one 256-row tile, or one 320-row tile with a
    second pass over their last rows past 320), K=2048, N=1024,
    E=256.  Sampled experts against the dense GEMM bit for bit, sampled rows
    against the oracle within the tolerance."""
    dr = require_gpu()
    M, k, E, K, N = 8192, 8, 256, 2048, 1024
    g = np.random.default_rng(41)
    xb = wl.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41)
    Wd = (torch.randn((E, K, N), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    ids, off, rows, pos = _routes_and_groups(dr, M, k, E, seed=41)
    note("grouped gemm full size (fused gather)")
    out = dr.grouped_gemm_bf16(dev_bf16_bits(xb), Wd, off, rows)
    got = _u32(out)
    off_h, rows_h = off.cpu().numpy(), rows.cpu().numpy()
    cnt = np.diff(off_h)
    tall = np.nonzero(cnt > 256)[0]
    picks = {int(np.argmax(cnt)), int(np.argmin(cnt)), 0, 77, E - 1}
    if tall.size:
        picks |= {int(tall[0]), int(tall[-1])}
    for e in sorted(picks):
        seg = slice(off_h[e], off_h[e + 1])
        note(f"dense rows of expert {e} ({cnt[e]} rows)")
        dense = dr.gemm_bf16(dev_bf16_bits(np.ascontiguousarray(xb[rows_h[seg]])), Wd[e].contiguous())
        assert np.array_equal(got[seg], _u32(dense)), f"expert {e}"
    sample = np.unique(np.r_[0, M * k - 1, off_h[1:-1], g.integers(0, M * k, 64)])
    e_of = np.searchsorted(off_h, sample, side="right") - 1
    Wh = {}
    for e in np.unique(e_of):
        Wh[e] = Wd[e].view(torch.int16).cpu().numpy().view(np.uint16)
    outh = out.cpu().numpy()
    for p, e in zip(sample, e_of):
        ref = oracle.gemm_bf16_ref(xb[rows_h[p]][None, :], Wh[e])[0]
        assert np.abs(outh[p].astype(np.float64) - ref).max() <= TOL, (p, e)
