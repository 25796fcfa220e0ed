"""GPU parity of the two halves of the router on their own: dr_route_logits
(the canonical logits) and dr_route_select (top-k, weights, margins from
given logits), each against the CPU oracle bit for bit, and their
composition against dr_route."""
import numpy as np
import pytest
import torch

from gpu_util import assert_route_equal, dev, f32_equal_bits, gpu_route_np, host, note, require_gpu

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dr():
    return require_gpu()


@pytest.mark.parametrize("E,K,M", [(256, 2048, 200), (256, 260, 70), (512, 1024, 130), (256, 4096, 65),
                                   (64, 512, 40), (128, 1000, 33), (256, 2048, 2100)])
def test_route_logits_matches_oracle(dr, E, K, M):
    rng = np.random.default_rng(E + K + M)
    x = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((K, E)) * 0.05).astype(np.float32)
    ref = oracle.logits(x, W)
    note(f"route_logits E={E} K={K} M={M}")
    got = host(dr.route_logits(dev(x), dev(W)))
    assert f32_equal_bits(got, ref)
    note(f"route_logits bf16 E={E} K={K} M={M}")
    got16 = dr.route_logits(dev(x), dev(W), logit_dtype="bf16")
    torch.cuda.synchronize()
    bits = got16.view(torch.int16).cpu().numpy().view(np.uint16)
    want = np.vectorize(oracle.bf16_rne, otypes=[np.uint16])(ref)
    assert np.array_equal(bits, want)


def _special_logits(rng, M, E):
    lg = (rng.standard_normal((M, E)) * 0.9).astype(np.float32)
    lg[0] = 0.0
    lg[1, ::2] = -0.0
    lg[2, 5] = np.nan
    lg[3, 7] = np.inf
    lg[3, 9] = np.inf
    lg[4] = -np.inf
    lg[4, E - 1] = -1.0
    lg[5, 1::3] = lg[5, 0]                 # many exact ties
    lg[6] = np.round(lg[6] * 4) / 4        # coarse values, ties throughout
    # signed zeros on top, tied by index: the margin's exact values keep
    # their signs
    lg[7] = -(np.abs(lg[7]) + 0.5)
    lg[7, 3::9] = -0.0
    lg[7, 7::9] = 0.0
    return lg


@pytest.mark.parametrize("E,k,M", [(64, 1, 90), (64, 32, 90), (128, 8, 90), (256, 8, 90), (256, 32, 90),
                                   (512, 10, 90), (1024, 8, 90), (256, 8, 1100), (64, 32, 1100), (512, 10, 1100),
                                   (512, 1, 90), (512, 32, 90), (1024, 32, 90), (128, 8, 1100), (1024, 10, 1100)])
def test_route_select_matches_oracle(dr, E, k, M):
    """One wavefront per token (M <= 1024, and E = 1024; from 512 experts the
    64-lane rounds, at k = 1, 10 and 32) and several tokens per wavefront
    (larger M: 4 to 16 values per lane, whose lanes sort their values once,
    and 32 at E = 1024, whose rounds scan them) against the oracle."""
    rng = np.random.default_rng(7 * E + k + M)
    lg = _special_logits(rng, M, E)
    for renorm in (False, True):
        ids, w, mg = oracle.select(lg, k, renormalize=renorm)
        note(f"route_select f32 E={E} k={k} M={M} renorm={renorm}")
        gi, gw, gm = dr.route_select(dev(lg), k, renormalize=renorm)
        got = (host(gi), host(gw), None, dr.margins_to_numpy(gm))
        assert_route_equal(got, (ids, w, None, mg), what=f"select E={E} k={k} M={M} renorm={renorm}")


@pytest.mark.parametrize("E,M", [(64, 70), (256, 70), (256, 1100), (1024, 70)])
def test_route_select_bf16_logits(dr, E, M):
    """bf16 logits are widened exactly and used as they are."""
    rng = np.random.default_rng(E + M)
    lg = _special_logits(rng, M, E)
    lg_t = torch.from_numpy(lg).to(torch.bfloat16)
    widened = lg_t.float().numpy()
    ids, w, mg = oracle.select(widened, 8)
    note(f"route_select bf16 E={E}")
    gi, gw, gm = dr.route_select(lg_t.cuda(), 8)
    got = (host(gi), host(gw), None, dr.margins_to_numpy(gm))
    assert_route_equal(got, (ids, w, None, mg), what=f"select bf16 E={E}")


@pytest.mark.parametrize("logit_dtype", ["f32", "bf16"])
def test_halves_compose_to_route(dr, logit_dtype):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 2048)).astype(np.float32)
    W = (rng.standard_normal((2048, 256)) * 0.02).astype(np.float32)
    xd, Wd = dev(x), dev(W)
    note(f"halves {logit_dtype}")
    full = gpu_route_np(dr, xd, Wd, 8, logit_dtype=logit_dtype)
    lg = dr.route_logits(xd, Wd, logit_dtype=logit_dtype)
    gi, gw, gm = dr.route_select(lg, 8)
    got = (host(gi), host(gw), lg.float().cpu().numpy(), dr.margins_to_numpy(gm))
    assert_route_equal(got, full, what=f"halves {logit_dtype}")
