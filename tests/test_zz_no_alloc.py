"""dr_route_noalloc through the C ABI: the entry point that allocates
nothing keeps the two-launch families' logits in the library's static device
buffer when the caller passes no logits buffer.  Its ids, weights and margins
must equal dr_route's (with a logits buffer) bit for bit, on two calls in a
row, the second smaller than the first (the buffer keeps the first call's
contents, which the second must not see), and a batch whose logits exceed
the buffer must be refused with the sizes in the error text."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import dev, note, require_gpu

pytestmark = pytest.mark.gpu

K, E, TOPK = 2048, 256, 8


def _noalloc(dr, L, x, W, k, M):
    ids = torch.full((M, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((M, k), float("nan"), dtype=torch.float32, device="cuda")
    mg = torch.full((M, 4), -1, dtype=torch.int32, device="cuda")
    st = L.dr_route_noalloc(ctypes.c_void_p(x.data_ptr()), dr.DR_F32, ctypes.c_void_p(W.data_ptr()), M, K, E, k,
                            dr.DR_F32, ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(w.data_ptr()), None,
                            ctypes.c_void_p(mg.data_ptr()), 0,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, ids, w, mg


def test_noalloc_equals_dr_route_on_two_calls_second_smaller():
    dr = require_gpu()
    L = dr.load_library()
    x = dev(wl.sweep_x(16384, K))
    W = dev(wl.router_weights(K, E))
    done = []
    # the largest batch the buffer takes (the split family), then smaller
    # ones (the split family again, the narrow tiles, the vector-ALU family)
    for M in (16384, 8000, 300, 19):
        fam = dr.auto_variant(M, K, E, logits=True)
        note(f"noalloc M={M} family={fam}")
        xm = x[:M].contiguous()
        st, ids, w, mg = _noalloc(dr, L, xm, W, TOPK, M)
        assert st == dr.DR_OK, L.dr_last_error().decode()
        rids, rw, _, rmg = dr.route(xm, W, TOPK)
        torch.cuda.synchronize()
        assert torch.equal(ids, rids), f"M={M}: ids differ"
        assert torch.equal(w.view(torch.int32), rw.view(torch.int32)), f"M={M}: weights differ"
        assert torch.equal(mg, rmg), f"M={M}: margins differ"
        done.append((M, fam))
    assert [f for _, f in done] == ["split", "split", "narrow", "tiny"]
    # one token past the buffer: refused before any launch
    M = 16385
    ids = torch.empty((M, TOPK), dtype=torch.int32, device="cuda")
    st = L.dr_route_noalloc(ctypes.c_void_p(x.data_ptr()), dr.DR_F32, ctypes.c_void_p(W.data_ptr()), M, K, E,
                            TOPK, dr.DR_F32, ctypes.c_void_p(ids.data_ptr()), None, None, None, 0, None)
    assert st == dr.DR_ERR_UNSUPPORTED
    assert "16777216" in L.dr_last_error().decode()


@pytest.mark.parametrize("M", [8192, 300])  # the split and the narrow families
def test_noalloc_captured_in_a_graph(M):
    """The caller the entry point is for: code under HIP graph capture.  With
    every output preallocated, the captured call allocates nothing (torch's
    allocated bytes are unchanged across the captured call), and each replay after
    new inputs are copied in gives dr_route's bits on those inputs, with eager
    work and synchronisations between the replays."""
    dr = require_gpu()
    W = dev(wl.router_weights(K, E))
    x_static = dev(wl.sweep_x(M, K))
    out = (torch.empty((M, TOPK), dtype=torch.int32, device="cuda"),
           torch.empty((M, TOPK), dtype=torch.float32, device="cuda"), None,
           torch.empty((M, 4), dtype=torch.int32, device="cuda"))
    dr.route_noalloc(x_static, W, TOPK, out)  # warm
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note(f"noalloc graph capture M={M}")
    with torch.cuda.graph(g):
        # measured inside the capture: torch's own capture state is set up
        # when the context opens
        before = torch.cuda.memory_allocated()
        dr.route_noalloc(x_static, W, TOPK, out)
        after = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    assert after == before
    rng = np.random.default_rng(M + 7)
    replays = 0
    for rep in range(3):
        x_static.copy_(torch.from_numpy(wl.bf16_valued(rng.standard_normal((M, K)).astype(np.float32))))
        torch.cuda.synchronize()
        note(f"noalloc graph replay {rep} M={M}")
        g.replay()
        torch.cuda.synchronize()
        rids, rw, _, rmg = dr.route(x_static, W, TOPK)
        torch.cuda.synchronize()
        assert torch.equal(out[0], rids), f"replay {rep}: ids"
        assert torch.equal(out[1].view(torch.int32), rw.view(torch.int32)), f"replay {rep}: weights"
        assert torch.equal(out[3], rmg), f"replay {rep}: margins"
        replays += 1
    assert replays == 3
