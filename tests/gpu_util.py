"""Helpers for the GPU parity tests: device transfer, bit comparison and the
oracle reference, with the case printed (and flushed) before each GPU step."""
import sys

import numpy as np
import pytest
import torch

import oracle


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for this test (run with -m 'not gpu' on a CPU host)")
    import deterministic_gemm_amd as dr
    dr.load_library()
    return dr


def note(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def dev_bf16_bits(bits: np.ndarray):
    """bf16 tensor on the GPU from uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def f32_equal_bits(a, b):
    """Bitwise equality of fp32 arrays, any NaN equal to any NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return bool(np.array_equal(na, nb) and np.array_equal(bits32(a)[~na], bits32(b)[~nb]))


def gpu_route_np(dr, x_dev, W_dev, k, **kw):
    """Run dr.route and bring (ids, weights, logits-as-f32, margins) to numpy."""
    ids, w, lg, mg = dr.route(x_dev, W_dev, k, **kw)
    torch.cuda.synchronize()
    ids_n = ids.cpu().numpy()
    w_n = w.cpu().numpy() if w is not None else None
    lg_n = lg.float().cpu().numpy() if lg is not None else None
    mg_n = dr.margins_to_numpy(mg) if mg is not None else None
    return ids_n, w_n, lg_n, mg_n


def assert_route_equal(got, want, rows=None, what=""):
    """got, want: (ids, weights, logits, margins) numpy tuples."""
    gi, gw, gl, gm = got
    wi, ww, wlg, wm = want
    sl = slice(None) if rows is None else rows
    assert np.array_equal(gi[sl], wi[sl]), f"{what}: ids differ at rows {np.nonzero(np.any(gi[sl] != wi[sl], axis=1))[0][:10]}"
    if gl is not None and wlg is not None:
        assert f32_equal_bits(gl[sl], wlg[sl]), f"{what}: logits differ"
    if gw is not None and ww is not None:
        assert f32_equal_bits(gw[sl], ww[sl]), f"{what}: weights differ"
    if gm is not None and wm is not None:
        a, b = gm[sl], wm[sl]
        assert np.array_equal(a["ulps"], b["ulps"]), f"{what}: margin ulps differ"
        assert np.array_equal(a["sel_min_bf16"], b["sel_min_bf16"]) and np.array_equal(a["rej_max_bf16"], b["rej_max_bf16"])
        assert f32_equal_bits(a["sel_min"], b["sel_min"]) and f32_equal_bits(a["rej_max"], b["rej_max"]), f"{what}: margin values differ"


def oracle_route(x, W, k, logits_bf16=False, renormalize=False):
    ids, w, lg, mg = oracle.route(x, W, k, logits_bf16=logits_bf16, renormalize=renormalize)
    return ids, w, lg, mg
