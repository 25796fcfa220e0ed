"""The library on concurrent streams and inside HIP graphs.

dr_route and the calls after it keep no state between calls and allocate
nothing, so (a) calls interleaved on two streams give the bits they give
alone, and (b) a captured graph of them, replayed after the inputs change,
gives the bits of eager calls on the new inputs -- checked on every replay,
with eager work and synchronisations between the replays.  None of these
calls records a memset, so the graphs hold only the library's kernels.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import dev, note, require_gpu

pytestmark = pytest.mark.gpu

K, E, TOPK = 2048, 256, 8


def _bits(t):
    if t is None:
        return None
    return t.view(torch.int32).cpu().numpy() if t.dtype == torch.float32 else t.cpu().numpy()


def _same(a, b):
    return all((x is None and y is None) or np.array_equal(_bits(x), _bits(y)) for x, y in zip(a, b))


def test_two_streams_interleaved():
    dr = require_gpu()
    W = dev(wl.router_weights(K, E))
    xa = dev(wl.sweep_x(4096, K))
    xb = dev(wl.stack_layer_x(3, wl.stack_lengths(), K)[:700])
    note("streams: eager references")
    ref_a = dr.route(xa, W, TOPK)
    ref_b = dr.route(xb, W, TOPK)
    ref_c = dr.route(xb[:9].contiguous(), W, TOPK)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    note("streams: interleaved launches")
    for i in range(8):
        with torch.cuda.stream(s1):
            outs.append(("a", dr.route(xa, W, TOPK)))
        with torch.cuda.stream(s2):
            outs.append(("b", dr.route(xb, W, TOPK)))
            outs.append(("c", dr.route(xb[:9].contiguous(), W, TOPK)))
    torch.cuda.synchronize()
    refs = {"a": ref_a, "b": ref_b, "c": ref_c}
    for name, got in outs:
        assert _same(got, refs[name]), name


@pytest.mark.parametrize("M", [8, 65, 8192])  # tiny, narrow, split families
def test_graph_replays_follow_new_inputs(M):
    dr = require_gpu()
    W = dev(wl.router_weights(K, E))
    x_static = dev(wl.sweep_x(M, K))
    g = torch.cuda.CUDAGraph()
    dr.route(x_static, W, TOPK)  # warm
    torch.cuda.synchronize()
    note(f"graph capture M={M}")
    with torch.cuda.graph(g):
        out = dr.route(x_static, W, TOPK)
        off, rows, pos = dr.moe_permute(out[0], E)
    rng = np.random.default_rng(M)
    for rep in range(3):
        newx = wl.bf16_valued(rng.standard_normal((M, K)).astype(np.float32))
        x_static.copy_(torch.from_numpy(newx))
        torch.cuda.synchronize()
        note(f"graph replay {rep} M={M}")
        g.replay()
        torch.cuda.synchronize()
        eager = dr.route(x_static, W, TOPK)
        e_off, e_rows, e_pos = dr.moe_permute(eager[0], E)
        torch.cuda.synchronize()
        assert _same(out, eager), f"replay {rep}"
        assert torch.equal(off, e_off) and torch.equal(rows, e_rows) and torch.equal(pos, e_pos)
