"""GPU parity of dr_route against the CPU oracle, bit for bit, and its
invariance across M, batch position and kernel family.

Workloads: the m-scan (a fixed 19-token request inside batches of 19..80
tokens, "Batch changed the model's mind", section "m-scan: the staircase"),
the Qwen3-MoE-like sweep (K=2048, E=256, k=8, M up to 8192), and edge cases:
ragged K and M tails, every supported E, signed zeros, subnormals, NaN,
bf16 input storage, renormalised weights, repeated calls.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import (assert_route_equal, dev, f32_equal_bits, gpu_route_np, note, oracle_route,
                      require_gpu)

pytestmark = pytest.mark.gpu

K, E, TOPK = 2048, 256, 8


@pytest.fixture(scope="module")
def dr():
    return require_gpu()


@pytest.fixture(scope="module")
def router_w():
    return wl.router_weights(K, E)


# ---------------------------------------------------------------- m-scan

@pytest.fixture(scope="module")
def mscan_ref(router_w):
    fx = wl.mscan_fixed_request(K)
    return oracle_route(fx, router_w, TOPK)


@pytest.mark.parametrize("variant", ["auto", "rowwise", "tiled", "split", "narrow", "tiny", "fused"])
def test_mscan_fixed_rows_bit_identical(dr, router_w, mscan_ref, variant):
    """Every M in 19..80, the fixed request placed first and last, ascending
    then descending: the fixed rows equal the oracle's solo run bit for bit."""
    Wd = dev(router_w)
    order = list(range(0, 62)) + list(range(61, -1, -1))
    seen_variants = set()
    for c in order:
        for fixed_first in (True, False):
            x, off = wl.mscan_batch(c, K, fixed_first)
            M = x.shape[0]
            note(f"mscan variant={variant} M={M} fixed_first={fixed_first}")
            got = gpu_route_np(dr, dev(x), Wd, TOPK, variant=variant)
            rows = slice(off, off + 19)
            assert_route_equal(tuple(None if g is None else g[rows] for g in got), mscan_ref,
                               what=f"M={M} first={fixed_first}")
            if variant == "auto":
                # without the logits output AUTO picks the fused families; the
                # switch between them lies inside the scanned range (the
                # binding's temporary logits buffer is turned off here)
                seen_variants.add(dr.auto_variant(M, K, E, logits=False))
                got = gpu_route_np(dr, dev(x), Wd, TOPK, logits=False, scratch_logits=False)
                assert_route_equal(tuple(None if g is None else g[rows] for g in got), mscan_ref,
                                   what=f"M={M} first={fixed_first} no logits")
    if variant == "auto":
        assert seen_variants == {"rowwise", "tiled"}


def test_mscan_coarrivals_match_oracle(dr, router_w):
    """All rows, not only the fixed ones, at a few batch sizes."""
    Wd = dev(router_w)
    for c in (0, 29, 45, 46, 61):
        x, _ = wl.mscan_batch(c, K, True)
        note(f"mscan all rows M={x.shape[0]}")
        got = gpu_route_np(dr, dev(x), Wd, TOPK)
        assert_route_equal(got, oracle_route(x, router_w, TOPK), what=f"M={x.shape[0]}")


# ---------------------------------------------------------------- sweep

@pytest.fixture(scope="module")
def sweep(router_w):
    x = wl.sweep_x(8192, K)
    return x, oracle_route(x, router_w, TOPK)


def test_sweep_every_m_matches_oracle(dr, router_w, sweep):
    """M in {1,16,64,65,75,256,1024,4096,8192} on prefixes of one activation
    matrix: each prefix equals the oracle on every row (so rows are also
    bit-identical across M)."""
    x, ref = sweep
    Wd = dev(router_w)
    xd = dev(x)
    for M in wl.SWEEP_MS:
        note(f"sweep M={M} variant={dr.auto_variant(M, K, E)}")
        got = gpu_route_np(dr, xd[:M].contiguous(), Wd, TOPK)
        assert_route_equal(got, tuple(r[:M] for r in ref), what=f"M={M}")


@pytest.mark.parametrize("variant", ["rowwise", "tiled", "split", "narrow", "tiny", "fused"])
def test_sweep_forced_variants(dr, router_w, sweep, variant):
    x, ref = sweep
    Wd = dev(router_w)
    for M in (1, 65, 1024) + ((8192,) if variant in ("split", "fused") else ()):
        note(f"sweep forced {variant} M={M}")
        got = gpu_route_np(dr, dev(x[:M]), Wd, TOPK, variant=variant)
        assert_route_equal(got, tuple(r[:M] for r in ref), what=f"{variant} M={M}")


@pytest.mark.parametrize("Kx,Ex,M", [(2048, 256, 600), (2048, 256, 1500), (2048, 256, 2048), (2048, 512, 300),
                                     (2048, 512, 700), (2048, 128, 2000), (2048, 64, 3000), (4096, 512, 240),
                                     (4096, 512, 500), (4096, 512, 1000), (4096, 256, 1000), (3072, 256, 100),
                                     (3000, 256, 700), (1024, 256, 2000), (768, 256, 1999)])
def test_narrow_tiles_match_oracle(dr, Kx, Ex, M):
    """The narrow family's tiles (16 x 16 with one, two or four parts, 32 x 16
    and 32 x 32 tokens x experts, picked by how many workgroups fit on the
    CUs), each with a ragged last token tile, at one to four K-groups: every
    output equals the oracle's, and the split family's where it exists."""
    rng = np.random.default_rng(Kx + Ex)
    W = wl.router_weights(Kx, Ex) if Ex == E else (rng.standard_normal((Kx, Ex)) * 0.02).astype(np.float32)
    x = wl.sweep_x(M, Kx)
    note(f"narrow tiles K={Kx} E={Ex} M={M}")
    got = gpu_route_np(dr, dev(x), dev(W), TOPK, variant="narrow")
    assert_route_equal(got, oracle_route(x, W, TOPK), what=f"narrow K={Kx} E={Ex} M={M}")
    if Ex in (256, 512):
        note(f"split family K={Kx} E={Ex} M={M}")
        assert_route_equal(gpu_route_np(dr, dev(x), dev(W), TOPK, variant="split"), got,
                           what=f"split K={Kx} E={Ex} M={M}")


def test_bf16_input_storage_is_bit_identical(dr, router_w, sweep):
    x, ref = sweep
    Wd = dev(router_w)
    M = 300
    xb = dev(x[:M]).to(torch.bfloat16)  # exact: x is bf16-valued
    for variant in ("rowwise", "tiled", "fused"):
        note(f"bf16 storage {variant}")
        got = gpu_route_np(dr, xb, Wd, TOPK, variant=variant)
        assert_route_equal(got, tuple(r[:M] for r in ref), what=f"bf16 x {variant}")


def test_repeated_calls_are_identical(dr, router_w, sweep):
    """Level 0: the same call 100 times gives the same bits."""
    x, _ = sweep
    xd, Wd = dev(x[:1024]), dev(router_w)
    note("repeat x100 M=1024")
    first = dr.route(xd, Wd, TOPK)
    for _ in range(100):
        again = dr.route(xd, Wd, TOPK)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b)


# ---------------------------------------------------------------- edge cases

@pytest.mark.parametrize("Kx", [1, 100, 255, 256, 257, 1000, 1023, 1025, 4096, 5000])
def test_ragged_k(dr, Kx):
    """K tails inside a block, single block, partial groups of blocks."""
    rng = np.random.default_rng(Kx)
    W = (rng.standard_normal((Kx, 128)) * 0.05).astype(np.float32)
    x = rng.standard_normal((70, Kx)).astype(np.float32)
    ref = oracle_route(x, W, 6)
    for variant in ("rowwise", "tiled"):
        note(f"ragged K={Kx} {variant}")
        got = gpu_route_np(dr, dev(x), dev(W), 6, variant=variant)
        assert_route_equal(got, ref, what=f"K={Kx} {variant}")


@pytest.mark.parametrize("Kx", [4, 100, 256, 260, 1000, 1024, 4096, 5000])
def test_ragged_k_split(dr, Kx):
    """K tails and partial groups of blocks in the two-kernel family (which
    takes fp32 x in whole 16-byte pieces, so K % 4 == 0), against the oracle
    and the fused kernel; M = 70 leaves a ragged token tile."""
    rng = np.random.default_rng(Kx + 1)
    W = (rng.standard_normal((Kx, 256)) * 0.05).astype(np.float32)
    x = rng.standard_normal((70, Kx)).astype(np.float32)
    ref = oracle_route(x, W, 6)
    for variant in ("split", "narrow", "tiled", "fused") + (("tiny",) if Kx <= 4096 else ()):
        note(f"ragged K={Kx} {variant}")
        got = gpu_route_np(dr, dev(x), dev(W), 6, variant=variant)
        assert_route_equal(got, ref, what=f"K={Kx} {variant}")


@pytest.mark.parametrize("Kx,Ex,M", [(2048, 256, 65), (2048, 256, 200), (2048, 256, 700), (2048, 256, 1500),
                                     (3072, 256, 100), (264, 256, 130), (2048, 512, 60), (4096, 512, 240)])
def test_narrow_tiles_bf16_x(dr, Kx, Ex, M):
    """The narrow family on bf16 x staged as it is (8 values per 16-byte
    unit, widened when read) and on the same values as fp32, across its tile
    shapes -- 8 staged token rows, 16 x 16, 32 x 16 and 32 x 32 -- with one to
    four K-groups and a ragged K, against the oracle."""
    rng = np.random.default_rng(Kx * 3 + Ex + M)
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    xb = torch.from_numpy(rng.standard_normal((M, Kx)).astype(np.float32)).to(torch.bfloat16)
    x = xb.float().numpy()
    ref = oracle_route(x, W, 8)
    for xd, name in ((xb.cuda(), "bf16"), (dev(x), "f32")):
        note(f"narrow K={Kx} E={Ex} M={M} x {name}")
        got = gpu_route_np(dr, xd, dev(W), 8, variant="narrow")
        assert_route_equal(got, ref, what=f"narrow K={Kx} E={Ex} M={M} x {name}")


@pytest.mark.parametrize("Kx", [8, 256, 264, 1000, 2048, 3080, 4096])
@pytest.mark.parametrize("Ex", [64, 256, 512, 1024])
def test_tiny_few_tokens(dr, Kx, Ex):
    """A few tokens in the vector-ALU family, which spreads W over sixteen
    K-block slots (the slots past the last block hold -0) while its
    workgroups fill at most half the CUs, and uses the fewest slots above
    that: 1 to 16 K-blocks, 1 to 8 tokens, fp32 and bf16 x, against the
    oracle."""
    rng = np.random.default_rng(Kx * 7 + Ex)
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    xb = torch.from_numpy(rng.standard_normal((8, Kx)).astype(np.float32)).to(torch.bfloat16)
    x = xb.float().numpy()  # bf16-valued, so both storages hold the same values
    ref = oracle_route(x, W, 8)
    for M in (1, 3, 8):
        for xd, name in ((dev(x[:M]), "f32"), (xb[:M].contiguous().cuda(), "bf16")):
            note(f"tiny K={Kx} E={Ex} M={M} x {name}")
            got = gpu_route_np(dr, xd, dev(W), 8, variant="tiny")
            assert_route_equal(got, tuple(r[:M] for r in ref), what=f"tiny K={Kx} E={Ex} M={M} x {name}")


@pytest.mark.parametrize("Ex,kx", [(64, 1), (64, 32), (128, 5), (256, 32), (512, 10), (1024, 8), (1024, 32)])
def test_every_supported_e(dr, Ex, kx):
    rng = np.random.default_rng(Ex + kx)
    Kx = 768
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    x = rng.standard_normal((77, Kx)).astype(np.float32)
    ref = oracle_route(x, W, kx)
    for variant in ("auto", "rowwise", "tiled", "split", "narrow", "tiny", "fused"):
        if variant in ("tiled", "narrow") and Ex == 1024:
            continue
        if variant == "split" and Ex not in (256, 512, 1024):
            continue
        if variant == "fused" and Ex != 256:
            continue
        note(f"E={Ex} k={kx} {variant}")
        got = gpu_route_np(dr, dev(x), dev(W), kx, variant=variant)
        assert_route_equal(got, ref, what=f"E={Ex} k={kx} {variant}")


@pytest.mark.parametrize("Ex,kx,mode", [(256, 1, "f32"), (256, 32, "f32"), (256, 8, "bf16_logits"),
                                         (512, 10, "renormalize"), (512, 32, "bf16_logits"), (128, 5, "f32")])
def test_large_batch_selection(dr, Ex, kx, mode):
    """Batches above 1024 tokens select with two tokens per wavefront (32
    lanes each; 16 lanes per token below 256 experts): k from 1 to 32, both
    logit modes and renormalisation, against the oracle, at a batch that is
    not a multiple of a workgroup's 8 (or 16) tokens."""
    rng = np.random.default_rng(Ex * 100 + kx)
    Kx, M = 256, 1100
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    x = rng.standard_normal((M, Kx)).astype(np.float32)
    x[5] = 0.0  # every logit +0: all ties, lowest indices win
    kw = {"logit_dtype": "bf16"} if mode == "bf16_logits" else ({"renormalize": True} if mode == "renormalize" else {})
    ref = oracle_route(x, W, kx, logits_bf16=(mode == "bf16_logits"), renormalize=(mode == "renormalize"))
    for variant in ("auto", "split", "narrow"):
        if variant == "split" and Ex not in (256, 512):
            continue
        note(f"large-batch selection E={Ex} k={kx} {mode} {variant}")
        got = gpu_route_np(dr, dev(x), dev(W), kx, variant=variant, **kw)
        assert_route_equal(got, ref, what=f"E={Ex} k={kx} {mode} {variant}")


@pytest.mark.parametrize("mode", ["bf16_logits", "renormalize"])
def test_modes(dr, router_w, sweep, mode):
    x, _ = sweep
    M = 200
    kw = {"logit_dtype": "bf16"} if mode == "bf16_logits" else {"renormalize": True}
    ref = oracle_route(x[:M], router_w, TOPK, logits_bf16=(mode == "bf16_logits"),
                       renormalize=(mode == "renormalize"))
    for variant in ("rowwise", "tiled", "split", "narrow", "tiny", "fused"):
        note(f"mode {mode} {variant}")
        got = gpu_route_np(dr, dev(x[:M]), dev(router_w), TOPK, variant=variant, **kw)
        assert_route_equal(got, ref, what=f"{mode} {variant}")


@pytest.mark.parametrize("Ex", [64, 256])
def test_special_values(dr, Ex):
    """Signed zeros, subnormal products, huge cancelling terms, NaN and inf."""
    rng = np.random.default_rng(99)
    Kx, kx = 600, 4
    x = rng.standard_normal((96, Kx)).astype(np.float32)
    W = (rng.standard_normal((Kx, Ex)) * 0.05).astype(np.float32)
    x[0] = 0.0
    x[1] = -0.0
    x[2] *= np.float32(2.0 ** -70)
    W[:, 5] *= np.float32(2.0 ** -70)          # subnormal products on row 2 / column 5
    x[3, :300] = 1e8
    x[3, 300:] = -1e8                          # cancellation across blocks
    x[4, 17] = np.nan                          # a NaN row
    x[5, 3] = np.inf                           # inf times +-W
    W[:, 9] = -0.0
    W[:, 10] = W[:, 11]                        # exact ties
    ref = oracle_route(x, W, kx)
    for variant in ("rowwise", "tiled", "narrow", "tiny") + (("split", "fused") if Ex == 256 else ()):
        note(f"special values E={Ex} {variant}")
        got = gpu_route_np(dr, dev(x), dev(W), kx, variant=variant)
        assert_route_equal(got, ref, what=f"special {variant}")


def test_empty_batch_is_a_no_op(dr, router_w):
    x = torch.empty((0, K), dtype=torch.float32, device="cuda")
    ids, w, lg, mg = dr.route(x, dev(router_w), TOPK)
    torch.cuda.synchronize()
    assert ids.shape == (0, TOPK)


def test_rows_at_any_offset(dr, router_w, sweep):
    """A row's result does not depend on where it sits in the batch: shift a
    block of rows by 1..40 positions inside otherwise different batches."""
    x, ref = sweep
    Wd = dev(router_w)
    block = x[1000:1050]
    rng = np.random.default_rng(5)
    for shift in (1, 7, 16, 31, 40):
        filler = rng.standard_normal((shift, K)).astype(np.float32)
        xb = np.concatenate([filler, block, filler[: shift // 2]], axis=0)
        for variant in ("auto", "split", "narrow", "tiny"):
            note(f"offset shift={shift} M={xb.shape[0]} {variant}")
            got = gpu_route_np(dr, dev(xb), Wd, TOPK, variant=variant)
            rows = slice(shift, shift + 50)
            assert_route_equal(tuple(g[rows] for g in got), tuple(r[1000:1050] for r in ref),
                               what=f"shift={shift} {variant}")


@pytest.mark.parametrize("Kx,M", [(2048, 2100), (4096, 600), (264, 1500), (8192, 300), (16384, 100)])
def test_split_at_1024_experts(dr, Kx, M):
    """The two-kernel family at E = 1024 (eight 128-expert tiles, or sixteen
    64-expert tiles in two parts), fp32 and bf16 x, against the oracle.  Above
    K = 4096 (fp32 x only) the 8-step-chunk configuration runs, with counter
    stacks of depth 4 (K = 8192) and 5 (K = 16384)."""
    rng = np.random.default_rng(Kx + M)
    W = (rng.standard_normal((Kx, 1024)) * 0.05).astype(np.float32)
    xb = torch.from_numpy(rng.standard_normal((M, Kx)).astype(np.float32)).to(torch.bfloat16)
    x = xb.float().numpy()
    ref = oracle_route(x, W, 8)
    for xd in ((dev(x), xb.cuda()) if Kx <= 4096 else (dev(x),)):
        note(f"split E=1024 K={Kx} M={M} x {xd.dtype}")
        got = gpu_route_np(dr, xd, dev(W), 8, variant="split")
        assert_route_equal(got, ref, what=f"split E=1024 K={Kx} M={M} {xd.dtype}")
