"""The m-scan, on the oracle.

A fixed 19-token request is routed inside batches of 19..80 tokens ("Batch
changed the model's mind", section "m-scan: the staircase": bit-identical for
m in 35..64, a jump at m=65, a larger one and an argmax flip at m=75,
reproduced by a descending sweep).  The canonical order gives maxdiff 0.0 at
every m.  The split-by-M positive control -- K cut into a number of slices
chosen from M -- must reproduce a staircase: flat plateaus with steps at 65 and
75.  If it did not, the scan could not detect an M-dependent order at all.
"""
import numpy as np
import pytest

import oracle
import workloads

K, E, TOPK = 2048, 256, 8
FIXED = 19


@pytest.fixture(scope="module")
def scan():
    W = workloads.router_weights(K, E)
    out = {}
    for split in (False, True):
        rows = {}
        for c in range(0, 62):
            for fixed_first in (True, False):
                x, off = workloads.mscan_batch(c, K, fixed_first)
                ids, w, lg, mg = oracle.route(x, W, TOPK, split_by_m=split)
                sl = slice(off, off + FIXED)
                rows[(FIXED + c, fixed_first)] = (ids[sl], w[sl], lg[sl], mg[sl])
        out[split] = rows
    return out


def _maxdiff(a, b):
    return float(np.abs(a.astype(np.float64) - b.astype(np.float64)).max())


def test_canonical_is_flat_over_m(scan):
    rows = scan[False]
    solo = rows[(FIXED, True)]
    for (m, ff), (ids, w, lg, mg) in rows.items():
        assert lg.tobytes() == solo[2].tobytes(), (m, ff)
        assert ids.tobytes() == solo[0].tobytes()
        assert w.tobytes() == solo[1].tobytes()
        assert mg.tobytes() == solo[3].tobytes()


def test_split_by_m_reproduces_a_staircase(scan):
    rows = scan[True]
    solo = rows[(FIXED, True)][2]
    for ff in (True, False):
        d = {m: _maxdiff(rows[(m, ff)][2], solo) for m in range(FIXED, FIXED + 62)}
        # plateaus: bit-identical inside each regime
        assert all(d[m] == 0.0 for m in range(FIXED, 65))
        for lo, hi in ((65, 75), (75, 81)):
            ref = rows[(lo, ff)][2]
            for m in range(lo, hi):
                assert rows[(m, ff)][2].tobytes() == ref.tobytes()
        # steps at the thresholds
        assert d[65] > 0.0 and d[75] > 0.0
        assert rows[(65, ff)][2].tobytes() != rows[(75, ff)][2].tobytes()


def test_descending_sweep_agrees(scan):
    """The oracle keeps no state between calls, so a descending sweep gives the
    same bits as the ascending one (the page's check against warm-up state)."""
    W = workloads.router_weights(K, E)
    for c in (61, 46, 45, 30, 0):
        x, off = workloads.mscan_batch(c, K, True)
        ids, w, lg, mg = oracle.route(x, W, TOPK)
        assert lg[off:off + FIXED].tobytes() == scan[False][(FIXED + c, True)][2].tobytes()
