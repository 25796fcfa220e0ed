"""Batch-invariant dense bf16 GEMM and the shared-expert gate dot on the GPU.

GEMM: rows bit-identical across M (19 to 4096, every tile configuration) and
across row offsets inside a batch; every sampled output within 1e-2 absolute of the
exact product (the oracle's fp64 evaluation), the tolerance the matrix core's
internal order allows.  Gate dot: the canonical order with one output, bit
for bit against the oracle, across M.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import dev, dev_bf16_bits, f32_equal_bits, note, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-2


@pytest.fixture(scope="module")
def dense():
    return wl.dense_x_bits(4096), wl.dense_w_bits(), wl.gate_w_bits()


def test_gemm_rows_invariant_across_m_and_close_to_exact(dense):
    dr = require_gpu()
    xb, Wb, _ = dense
    xd, Wd = dev_bf16_bits(xb), dev_bf16_bits(Wb)
    note("gemm M=4096")
    full = dr.gemm_bf16(xd, Wd).cpu().numpy()
    # the sweep sizes plus others so that, on a 256-CU device, every tile
    # configuration N = 4096 reaches runs: the 16-column strips with all rows
    # (M <= 16 and 97..128: one to eight row fragments), 32 x 32 (17 <= M <=
    # 96), 64 x 64 (200, 256), 64 x 64 with two stages (300, 512), 128 x 128
    # (1000, 1024), 256 x 128 (2048), 256 x 256 (3000, 4096), several with a
    # ragged last tile (64 x 128 runs where M > N: the bf16 router's logits
    # GEMM)
    for M in sorted(set(wl.DENSE_MS) | {1, 5, 16, 17, 33, 64, 80, 81, 96, 97, 100, 113, 128, 200, 256, 300, 1000,
                                        1024, 2048, 3000}):
        note(f"gemm M={M}")
        out = dr.gemm_bf16(xd[:M].contiguous(), Wd).cpu().numpy()
        assert f32_equal_bits(out, full[:M]), f"M={M} rows differ from the M=4096 run"
    rows = np.r_[0:19, 64:76, 511:513, 4000:4096:16]
    ref = oracle.gemm_bf16_ref(xb[rows], Wb)
    err = np.abs(full[rows].astype(np.float64) - ref.astype(np.float64))
    print(f"gemm max |delta| vs exact: {err.max():.3e}")
    assert err.max() <= TOL


def test_gemm_row_offsets(dense):
    dr = require_gpu()
    xb, Wb, _ = dense
    Wd = dev_bf16_bits(Wb)
    base = dr.gemm_bf16(dev_bf16_bits(xb[:200]), Wd).cpu().numpy()
    for shift in (1, 5, 16, 33, 127):
        filler = wl.to_bf16_bits(np.random.default_rng(shift).standard_normal((shift, wl.DENSE_K)).astype(np.float32))
        xs = np.concatenate([filler, xb[:200]], axis=0)
        note(f"gemm shift={shift}")
        out = dr.gemm_bf16(dev_bf16_bits(xs), Wd).cpu().numpy()
        assert f32_equal_bits(out[shift:shift + 200], base)


def test_gemm_small_shapes_close_to_exact():
    """Within the stated 1e-2 absolute of the exact product.  The inputs are
    bf16, so every product is exact in fp32 and the only error is the fp32
    accumulation's: at most about K * 2^-24 * sum_k |x_k w_k|, which for these
    N(0,1) operands (K <= 224, sum |x w| <= ~200) is below 3e-3 even as a
    worst case, and typically ~1e-5."""
    dr = require_gpu()
    rng = np.random.default_rng(3)
    # partial K stages and ragged M tiles in every tile configuration (on a
    # 256-CU device: 32 x 32 for the first six, then 64 x 64, 64 x 64 with
    # two stages, 128 x 128, 256 x 128, three times 256 x 256 (the last with
    # a single K step), and 64 x 128, which
    # runs only where M > N: a ragged 48-row last tile and a partial K stage;
    # then the 16-column strips (M <= 16 and 97..128) with a partial last K
    # stage, and 32 x 32 tiles at N = 4096)
    shapes = ((1, 32, 128), (3, 64, 256), (130, 96, 128), (300, 224, 384), (1100, 96, 128),
              (1500, 160, 256), (200, 160, 4096), (450, 96, 4096), (900, 224, 4096), (1800, 96, 4096),
              (2100, 96, 4096), (4100, 160, 4096), (2500, 32, 4096), (6000, 96, 256),
              (3, 96, 4096), (16, 288, 2048), (40, 224, 4096), (70, 160, 4096), (1, 32, 4096),
              (100, 544, 4096), (128, 160, 2048))
    worst = 0.0
    for (M, K, N) in shapes:
        xb = wl.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        Wb = wl.to_bf16_bits(rng.standard_normal((K, N)).astype(np.float32))
        note(f"gemm small {M}x{K}x{N}")
        out = dr.gemm_bf16(dev_bf16_bits(xb), dev_bf16_bits(Wb)).cpu().numpy()
        ref = oracle.gemm_bf16_ref(xb, Wb)
        err = float(np.abs(out.astype(np.float64) - ref.astype(np.float64)).max())
        worst = max(worst, err)
        assert err <= TOL, (M, K, N, err)
    print(f"small shapes: max |delta| vs exact {worst:.3e} over {len(shapes)} shapes")


def test_gemm_strip_rows_match_other_tiles():
    """The 16-column strip kernel (M <= 16 and 97..128 at N = 4096 on a
    256-CU device: one to eight row fragments) against the 64 x 64 tiles of
    a 300-row batch, bit for bit, at K with a partial last W stage (K % 512
    != 0), a single K step, and a K that is a whole number of stages."""
    dr = require_gpu()
    rng = np.random.default_rng(11)
    N = 4096
    for K in (32, 96, 544, 1056, 2048, 4128):
        xb = wl.to_bf16_bits(rng.standard_normal((300, K)).astype(np.float32))
        Wb = wl.to_bf16_bits((rng.standard_normal((K, N)) * 0.02).astype(np.float32))
        Wd = dev_bf16_bits(Wb)
        note(f"gemm strip K={K} M=300")
        full = dr.gemm_bf16(dev_bf16_bits(xb), Wd).cpu().numpy()
        for M in (1, 2, 15, 16, 97, 104, 112, 121, 128):
            note(f"gemm strip K={K} M={M}")
            out = dr.gemm_bf16(dev_bf16_bits(xb[:M]), Wd).cpu().numpy()
            assert f32_equal_bits(out, full[:M]), (K, M)
        ref = oracle.gemm_bf16_ref(xb[:16], Wb)
        assert float(np.abs(full[:16].astype(np.float64) - ref.astype(np.float64)).max()) <= TOL


def test_gate_dot_bit_exact_and_m_invariant(dense):
    dr = require_gpu()
    xb, _, wb = dense
    ref_dot, ref_gate = oracle.gate_dot(xb, wb)
    xd, wd = dev_bf16_bits(xb), dev_bf16_bits(wb)
    for M in wl.DENSE_MS:
        note(f"gate dot M={M}")
        d, g = dr.gate_dot(xd[:M].contiguous(), wd)
        assert f32_equal_bits(d.cpu().numpy(), ref_dot[:M])
        assert f32_equal_bits(g.cpu().numpy(), ref_gate[:M])


def test_gate_dot_f32_and_ragged_k():
    """Row groups of 1..64 lanes (K up to 64 blocks), the LDS-staged kernel
    (rows 16-byte aligned, one dtype) and the direct one (rows not aligned,
    mixed dtypes), partial last blocks, M not a multiple of a workgroup's rows."""
    dr = require_gpu()
    rng = np.random.default_rng(8)
    for K in (1, 255, 257, 512, 1000, 2048, 3000, 8192, 16128, 16384):
        x = rng.standard_normal((33, K)).astype(np.float32)
        w = (rng.standard_normal(K) * 0.02).astype(np.float32)
        note(f"gate dot f32 K={K}")
        d, g = dr.gate_dot(dev(x), dev(w))
        rd, rg = oracle.gate_dot(x, w)
        assert f32_equal_bits(d.cpu().numpy(), rd) and f32_equal_bits(g.cpu().numpy(), rg)
    for K in (260, 264, 1000, 2048, 4096, 8000, 16384):
        xb = wl.to_bf16_bits(rng.standard_normal((70, K)).astype(np.float32))
        wb = wl.to_bf16_bits((rng.standard_normal(K) * 0.02).astype(np.float32))
        wf = wl.bf16_bits_to_f32(wb)
        rd, rg = oracle.gate_dot(xb, wb)
        note(f"gate dot bf16 K={K}")
        d, g = dr.gate_dot(dev_bf16_bits(xb), dev_bf16_bits(wb))
        assert f32_equal_bits(d.cpu().numpy(), rd) and f32_equal_bits(g.cpu().numpy(), rg)
        note(f"gate dot bf16 x, f32 w K={K}")
        d, g = dr.gate_dot(dev_bf16_bits(xb), dev(wf))
        assert f32_equal_bits(d.cpu().numpy(), rd) and f32_equal_bits(g.cpu().numpy(), rg)


def test_gemm_operands_of_4gib_and_more_take_the_64bit_path():
    """x of 2^20 rows x 2048 (4 GiB, past a buffer descriptor's 32-bit range)
    runs the transfers with 64-bit addresses; sampled rows, and the grouped
    product reading rows of that x, must equal the same rows computed from a
    small x (the buffer-descriptor path) bit for bit."""
    dr = require_gpu()
    M, K, N = 1 << 20, 2048, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    note("gemm 4 GiB x: allocate")
    x = torch.randn((M, K), device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn((K, N), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    note("gemm 4 GiB x: 64-bit path")
    out = dr.gemm_bf16(x, W)
    rows = torch.tensor([0, 1, 12345, M // 2, M - 2, M - 1], device="cuda")
    note("gemm 4 GiB x: buffer path on the same rows")
    small = dr.gemm_bf16(x[rows].contiguous(), W)
    assert torch.equal(out[rows].view(torch.int32), small.view(torch.int32))
    del out
    E = 4
    Wg = (torch.randn((E, K, N), device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    grows = torch.tensor([M - 1, 7, M // 3, 0, 999999, M - 5, 3, 12], dtype=torch.int32, device="cuda")
    off = torch.tensor([0, 2, 5, 5, 8], dtype=torch.int32, device="cuda")
    note("grouped gemm with 4 GiB x")
    big = dr.grouped_gemm_bf16(x, Wg, off, grows)
    note("grouped gemm with the gathered rows")
    ref = dr.grouped_gemm_bf16(x[grows.long()].contiguous(), Wg, off)
    assert torch.equal(big.view(torch.int32), ref.view(torch.int32))
