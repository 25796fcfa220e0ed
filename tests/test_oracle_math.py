"""The oracle's scalar pieces against mathematics and independent routines:
the exponential against float64 exp, bf16 rounding against torch's CPU
conversion and exact rational rounding, the ULP count's closed forms, and the
FNV-1a digest against its published test vectors."""
import math
import os
import struct

import numpy as np
import pytest
import torch

import brute
import digest
import oracle


def _ulp_err(got32, want64):
    """|got - want| in units of the fp32 ulp at want (normal range)."""
    want64 = np.asarray(want64, np.float64)
    e = np.floor(np.log2(np.abs(want64)))
    e = np.maximum(e, -126)
    return np.abs(got32.astype(np.float64) - want64) / np.exp2(e - 23)


def _expf_ulp_errors(bits: np.ndarray) -> np.ndarray:
    """Errors in fp32 ulps of the oracle's exp against float64 exp at the
    fp32 inputs with these bit patterns.  The ulp is taken at the fp32
    neighbour of the exact value nearer zero, so at a power of two the
    smaller binade's ulp is used: never more lenient than the ulp at the
    exact value.  Every result in [-87, 0] is a normal number."""
    t = bits.view(np.float32)
    got = oracle.expf(t).astype(np.float64)
    want = np.exp(t.astype(np.float64))
    w32 = want.astype(np.float32)
    ulp = np.spacing(np.nextafter(w32, np.float32(0))).astype(np.float64)
    return np.abs(got - want) / ulp


def test_expf_accuracy_strided_sweep():
    """Every 61st fp32 value in [-87, 0] (18.3 million inputs): within 2 ulp
    of float64 exp.  Quick enough for the mutation proofs, which rebuild the
    oracle per planted mistake; the exhaustive sweep below takes every input."""
    lo = struct.unpack("<I", struct.pack("<f", -87.0))[0]
    bits = np.arange(0x80000000, lo + 1, 61, dtype=np.uint64).astype(np.uint32)
    err = _expf_ulp_errors(bits)
    assert err.max() <= 2.0, (err.max(), bits.view(np.float32)[np.argmax(err)])


def test_expf_accuracy_neighbourhoods():
    """Whole neighbourhoods of 40000 values around -1, -0.5, -87 and -10:
    within 2 ulp of float64 exp (a quick check; the exhaustive sweep below
    covers every input)."""
    extra = []
    for v in (-1.0, -0.5, -87.0, -10.0):
        b = struct.unpack("<I", struct.pack("<f", v))[0]
        extra.append(np.arange(b - 20000, b + 20000, dtype=np.uint32))
    bits = np.concatenate(extra)
    t = bits.view(np.float32)
    bits = bits[(t <= 0) & (t >= -87.0)]
    err = _expf_ulp_errors(bits)
    assert err.max() <= 2.0, (err.max(), bits.view(np.float32)[np.argmax(err)])


@pytest.mark.slow
def test_expf_accuracy_exhaustive():
    """Every fp32 value t in [-87, 0] (the bit patterns from -0.0 to -87.0,
    1,118,699,521 inputs): the routing exponential within 2 ulp of float64
    exp.  This pins its accuracy, not its bits (its bits are fixed by the
    written steps, which the device implements the same way)."""
    import concurrent.futures

    lo = 0x80000000  # -0.0
    hi = struct.unpack("<I", struct.pack("<f", -87.0))[0]
    chunk = 1 << 23
    starts = list(range(lo, hi + 1, chunk))

    def run(s):
        bits = np.arange(s, min(s + chunk, hi + 1), dtype=np.uint64).astype(np.uint32)
        err = _expf_ulp_errors(bits)
        i = int(np.argmax(err))
        return float(err[i]), int(bits[i]), bits.size

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(run, starts))
    worst = max(res)
    total = sum(r[2] for r in res)
    print(f"exp sweep: {total} inputs, worst {worst[0]:.3f} ulp at bits {worst[1]:#010x}")
    assert total == hi - lo + 1 == 1118699521
    assert worst[0] <= 2.0, worst


def test_expf_special_values():
    assert oracle.expf([0.0])[0] == 1.0
    assert oracle.expf([-0.0])[0] == 1.0
    assert oracle.expf([-87.0])[0] > 0.0
    assert oracle.expf([-87.01])[0] == 0.0
    assert oracle.expf([-np.inf])[0] == 0.0
    assert np.isnan(oracle.expf([np.nan])[0])
    assert np.isnan(oracle.expf([1e-30])[0])  # outside the t <= 0 domain
    # exp(-ln2 * j) for integers j: within 1 ulp of 2^-j
    for j in range(0, 120, 7):
        t = np.float32(-math.log(2.0) * j)
        g = float(oracle.expf([t])[0])
        assert abs(g - math.exp(float(t))) <= 2 * math.ulp(math.exp(float(t))) * 2**29


def test_expf_monotone_on_a_grid():
    t = np.linspace(-20, 0, 200001, dtype=np.float32)
    g = oracle.expf(t)
    assert np.all(np.diff(g.astype(np.float64)) >= 0)


def _torch_bf16_bits(v):
    return int(torch.tensor([v], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF


def test_bf16_rne_against_torch_and_exact_rounding():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(2000).astype(np.float32))
    vals += [np.float32(v) for v in (0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, 1e-45)]
    # exact halfway cases: lower 16 bits 0x8000 with even and odd upper parts
    for up in (0x3F80, 0x3F81, 0x0001, 0x7F7F, 0xBF80, 0xBF81):
        vals.append(np.uint32((up << 16) | 0x8000).view(np.float32))
        vals.append(np.uint32((up << 16) | 0x7FFF).view(np.float32))
        vals.append(np.uint32((up << 16) | 0x8001).view(np.float32))
    vals += [np.float32(np.inf), np.float32(-np.inf)]
    for v in vals:
        got = oracle.bf16_rne(float(v))
        assert got == _torch_bf16_bits(float(v)), (v, hex(got))
        assert got == brute.bf16_bits(float(v)), (v, hex(got))
    assert oracle.bf16_rne(float("nan")) == 0x7FC0
    assert oracle.bf16_rne(np.uint32(0xFFC12345).view(np.float32).item()) == 0x7FC0


def test_ulps_closed_forms():
    # adjacent values are one step apart; +0/-0 are the same value
    for b in (0x0000, 0x0001, 0x3F80, 0x7F7E):
        assert oracle.ulps(b + 1, b) == 1
    assert oracle.ulps(0x0000, 0x8000) == 0
    # straddling zero: |ord(a)| + |ord(b)|
    for a, b in ((0x3F80, 0xBF80), (0x0005, 0x8003), (0x4000, 0xC100)):
        assert oracle.ulps(a, b) == (a & 0x7FFF) + (b & 0x7FFF)
    # a two's-complement reading of the negative side would give a different
    # count: the sign-magnitude order is what is counted
    assert oracle.ulps(0x0001, 0x8001) == 2
    assert oracle.ulps(0xBF80, 0xBF81) == 1


@pytest.mark.parametrize("data,want", [
    (b"", 0xCBF29CE484222325),
    (b"a", 0xAF63DC4C8601EC8C),
    (b"foobar", 0x85944171F73967E8),
])
def test_fnv1a64_vectors(data, want):
    assert digest.fnv1a64(data) == want
