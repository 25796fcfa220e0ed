"""The 40-layer prefill routing stack: 16 requests of random lengths 64..2048
concatenated into M=16384 tokens per layer, each layer with its own router
weight.  Every request's expert ids must equal its solo run bit for bit
("Batch changed the model's mind": the serve gate byte-compares each stream
alone and batched; section "16% of routing decisions" counts identical,
order-only and set-differing decisions -- here all must be identical)."""
import numpy as np
import pytest
import torch

import digest
import workloads as wl
from gpu_util import dev, note, oracle_route, require_gpu

pytestmark = pytest.mark.gpu

K, E, TOPK = 2048, 256, 8


@pytest.mark.parametrize("layers", [list(range(0, 40, 3))])
def test_batched_equals_solo_per_request(layers):
    dr = require_gpu()
    lengths = wl.stack_lengths()
    assert sum(lengths) == wl.STACK_TOKENS
    offs = np.cumsum([0] + lengths)
    counts = {"identical": 0, "order_only": 0, "set_differs": 0}
    for layer in layers:
        W = dev(wl.stack_layer_weights(layer, K, E))
        xs = [wl.stack_request_x(r, layer, L, K) for r, L in enumerate(lengths)]
        xall = dev(np.concatenate(xs, axis=0))
        note(f"stack layer={layer} batched M={xall.shape[0]}")
        ids_b = dr.route(xall, W, TOPK, weights=False, logits=False, margins=False)[0].cpu().numpy()
        digests = []
        for r, xr in enumerate(xs):
            note(f"stack layer={layer} solo request={r} M={xr.shape[0]}")
            ids_s = dr.route(dev(xr), W, TOPK, weights=False, logits=False, margins=False)[0].cpu().numpy()
            part = ids_b[offs[r]:offs[r + 1]]
            c = digest.categorize(ids_s, part)
            for kk in counts:
                counts[kk] += c[kk]
            assert digest.route_digest(ids_s) == digest.route_digest(part)
            digests.append(digest.route_digest(ids_s))
        # one request per layer against the oracle as an anchor
        r = layer % len(lengths)
        ref = oracle_route(xs[r][:64], wl.stack_layer_weights(layer, K, E), TOPK)
        assert np.array_equal(ids_b[offs[r]:offs[r] + 64], ref[0])
    print("categories:", counts)
    assert counts["order_only"] == 0 and counts["set_differs"] == 0
    assert counts["identical"] == wl.STACK_TOKENS * len(layers)
