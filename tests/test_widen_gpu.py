"""bf16 activations: the exact widening to fp32 (dr_widen_bf16) and the
binding's route through it, which must give the bits of the bf16 families and
of the oracle ("Batch changed the model's mind", section "The fix: m-invariant
twins": a row's result fixed by its own values; a bf16 value widened to fp32
is the same number)."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_route_equal, dev, gpu_route_np, note, oracle_route, require_gpu

pytestmark = pytest.mark.gpu

K, E, TOPK = 2048, 256, 8


def _bits16(n, seed):
    """Every class of bf16 pattern: normals of both signs, +-0, subnormals,
    +-inf and NaNs with payloads."""
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    special = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x7F81, 0x3F80], dtype=np.uint16)
    b[: min(n, len(special))] = special[:n]
    return b


@pytest.mark.parametrize("n", [1, 7, 8, 9, 4096 * 8 + 5, 3_000_001])
def test_widen_is_exact(n):
    dr = require_gpu()
    b = _bits16(n, n)
    note(f"widen n={n}")
    xb = torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    got = dr.widen_bf16(xb).cpu().numpy().view(np.uint32)
    want = b.astype(np.uint32) << 16
    assert np.array_equal(got, want)


def test_widen_leaves_out_past_n_alone():
    dr = require_gpu()
    b = _bits16(13, 5)
    xb = torch.from_numpy(b.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((16,), 7.0, device="cuda")
    st = dr.load_library().dr_widen_bf16(xb.data_ptr(), 13, out.data_ptr(), None)
    assert st == dr.DR_OK
    o = out.cpu().numpy()
    assert np.array_equal(o[:13].view(np.uint32), b.astype(np.uint32) << 16)
    assert np.all(o[13:] == 7.0)


@pytest.fixture(scope="module")
def data():
    W = wl.router_weights(K, E)
    xf = wl.sweep_x(8192, K)  # bf16-valued fp32 rows
    return W, xf


@pytest.mark.parametrize("M", [1, 19, 64, 65, 1024, 8192])
def test_bf16_route_equals_fp32_route_and_bf16_families(data, M):
    dr = require_gpu()
    W, xf = data
    Wd = dev(W)
    xb = dev(xf[:M]).to(torch.bfloat16)
    assert np.array_equal(xb.float().cpu().numpy(), xf[:M])  # the rows are bf16 values
    note(f"bf16 x M={M}: auto widens={dr.widen_bf16_used(M, K, E)}")
    got = gpu_route_np(dr, xb, Wd, TOPK)
    want = gpu_route_np(dr, dev(xf[:M]), Wd, TOPK)
    assert_route_equal(got, want, what=f"bf16 vs fp32 x, M={M}")
    if M <= 1024:
        note(f"bf16 x M={M}: against the register-staged family")
        assert_route_equal(got, gpu_route_np(dr, xb, Wd, TOPK, variant="tiled"), what=f"tiled, M={M}")
    if M <= 65:
        assert_route_equal(got, oracle_route(xf[:M], W, TOPK), what=f"oracle, M={M}")


@pytest.mark.parametrize("Kx", [8, 264, 1000, 2048, 4096])
def test_tiny_reads_bf16_directly(Kx):
    """The vector-ALU family staging bf16 x as it is (widening when read),
    forced at batches that take four and eight wavefronts per workgroup and
    several rounds, against the oracle on the widened rows."""
    dr = require_gpu()
    rng = np.random.default_rng(Kx)
    W = (rng.standard_normal((Kx, 256)) * 0.05).astype(np.float32)
    for M in (1, 37, 200):
        xb = torch.from_numpy(rng.standard_normal((M, Kx)).astype(np.float32)).to(torch.bfloat16)
        x = xb.float().numpy()
        note(f"tiny bf16 x K={Kx} M={M}")
        got = gpu_route_np(dr, xb.cuda(), dev(W), 6, variant="tiny")
        assert_route_equal(got, oracle_route(x, W, 6), what=f"tiny bf16 K={Kx} M={M}")


@pytest.mark.parametrize("Kx,Ex,kx", [(8, 256, 8), (264, 256, 8), (1000, 512, 10), (2048, 256, 8), (2056, 256, 8),
                                      (4096, 512, 10)])
def test_split_reads_bf16_directly(Kx, Ex, kx):
    """The two-kernel family staging bf16 x as it is (8 values per 16-byte
    unit, widened when read), in its one-part and two-part configurations,
    with ragged token tiles and K tails, against the oracle."""
    dr = require_gpu()
    rng = np.random.default_rng(Kx + Ex)
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    for M in (70, 300, 2100):
        xb = torch.from_numpy(rng.standard_normal((M, Kx)).astype(np.float32)).to(torch.bfloat16)
        x = xb.float().numpy()
        note(f"split bf16 x K={Kx} E={Ex} M={M}")
        got = gpu_route_np(dr, xb.cuda(), dev(W), kx, variant="split")
        assert_route_equal(got, oracle_route(x, W, kx), what=f"split bf16 K={Kx} E={Ex} M={M}")
        got_bf = gpu_route_np(dr, xb.cuda(), dev(W), kx, variant="split", logit_dtype="bf16")
        assert_route_equal(got_bf, oracle_route(x, W, kx, logits_bf16=True), what=f"split bf16 logits K={Kx} M={M}")


@pytest.mark.parametrize("Kx,Ex,kx,Ms", [(264, 256, 8, (5, 70)), (1000, 64, 4, (33,)), (2048, 256, 8, (70, 600, 2000)),
                                         (4096, 512, 10, (19, 240)), (5000, 256, 8, (40,))])
def test_narrow_reads_bf16_directly(Kx, Ex, kx, Ms):
    """The narrow tiles staging bf16 x as they are, in every tile and part
    configuration (one to four K-group parts; 16 x 16, 32 x 16 and 32 x 32
    tiles; chunks of 16 and 8 steps), against the oracle."""
    dr = require_gpu()
    rng = np.random.default_rng(Kx * 3 + Ex)
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    for M in Ms:
        xb = torch.from_numpy(rng.standard_normal((M, Kx)).astype(np.float32)).to(torch.bfloat16)
        x = xb.float().numpy()
        note(f"narrow bf16 x K={Kx} E={Ex} M={M}")
        got = gpu_route_np(dr, xb.cuda(), dev(W), kx, variant="narrow")
        assert_route_equal(got, oracle_route(x, W, kx), what=f"narrow bf16 K={Kx} E={Ex} M={M}")
