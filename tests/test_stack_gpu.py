"""The 40-layer prefill routing stack: 16 requests of random lengths 64..2048
concatenated into M=16384 tokens per layer, each layer with its own router
weight.  Every request's expert ids must equal its solo run bit for bit at
every one of the 40 layers ("Batch changed the model's mind": the serve gate
byte-compares each stream alone and batched; section "16% of routing
decisions" counts identical, order-only and set-differing decisions over 40
layers -- here all 655,360 token-layer decisions must be identical).  Each
layer also anchors one whole request against the oracle."""
import numpy as np
import pytest

import digest
import workloads as wl
from gpu_util import dev, note, oracle_route, require_gpu

pytestmark = pytest.mark.gpu

K, E, TOPK = 2048, 256, 8


def test_batched_equals_solo_per_request_all_layers():
    dr = require_gpu()
    lengths = wl.stack_lengths()
    assert len(lengths) == wl.STACK_REQUESTS and sum(lengths) == wl.STACK_TOKENS
    offs = np.cumsum([0] + lengths)
    counts = {"identical": 0, "order_only": 0, "set_differs": 0}
    anchored = 0
    layers_done = 0
    for layer in range(wl.STACK_LAYERS):
        W_h = wl.stack_layer_weights(layer, K, E)
        W = dev(W_h)
        xs = [wl.stack_request_x(r, layer, L, K) for r, L in enumerate(lengths)]
        xall = dev(np.concatenate(xs, axis=0))
        note(f"stack layer={layer} batched M={xall.shape[0]}")
        ids_b = dr.route(xall, W, TOPK, weights=False, logits=False, margins=False)[0].cpu().numpy()
        for r, xr in enumerate(xs):
            note(f"stack layer={layer} solo request={r} M={xr.shape[0]}")
            ids_s = dr.route(dev(xr), W, TOPK, weights=False, logits=False, margins=False)[0].cpu().numpy()
            c = digest.categorize(ids_s, ids_b[offs[r]:offs[r + 1]])
            for kk in counts:
                counts[kk] += c[kk]
            assert c["identical"] == lengths[r], (layer, r, c)
        # one whole request per layer against the oracle, by ids and by the
        # routing digest the pages' tap compares
        r = layer % len(lengths)
        ref = oracle_route(xs[r], W_h, TOPK)[0]
        part = ids_b[offs[r]:offs[r + 1]]
        assert np.array_equal(part, ref), (layer, r)
        assert digest.route_digest(part) == digest.route_digest(ref)
        anchored += lengths[r]
        layers_done += 1
    print("categories:", counts, "oracle-anchored tokens:", anchored)
    # counted properties: every token-layer decision was compared
    assert layers_done == wl.STACK_LAYERS == 40
    assert counts == {"identical": 655360, "order_only": 0, "set_differs": 0}
    assert anchored == sum(lengths[l % len(lengths)] for l in range(wl.STACK_LAYERS))
