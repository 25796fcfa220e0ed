"""Sharded routing, the part one GPU can show: the shards' results, combined
exactly, give the single-call bits (the exchange itself needs a second GPU).

Expert shards: the logits of W's column slices [K, E/G], concatenated, equal
the full logits bit for bit (no output's order changes), and the selection on
the concatenation gives dr_route's ids, weights and margin records.

K shards: with nb = K/256 blocks and G shards of nb/G blocks (both powers of
two), each shard's canonical tree is an aligned subtree of the full one, so
adding the G shard logits pairwise, adjacent shards first, gives the full
logits bit for bit ("The Illusion of Determinism in Disaggregated Inference",
section "The anatomy of the missing numeric contract": one fixed grouping of
the K reduction, whoever computes its parts).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import dev, note, require_gpu

pytestmark = pytest.mark.gpu

K, E, TOPK, M = 2048, 256, 8, 8192


def _u32(t):
    return t.contiguous().view(torch.int32).cpu().numpy()


@pytest.fixture(scope="module")
def full():
    dr = require_gpu()
    W = wl.router_weights(K, E)
    x = dev(wl.sweep_x(M, K))
    note("sharded: full route")
    return W, x, dr.route(x, dev(W), TOPK)


@pytest.mark.parametrize("G", [2, 4])
def test_expert_shards_concatenate_to_the_full_route(full, G):
    dr = require_gpu()
    W, x, (ids, w, lg, mg) = full
    parts = []
    for g in range(G):
        note(f"expert shard {g} of {G}")
        parts.append(dr.route_logits(x, dev(np.ascontiguousarray(W[:, g * E // G:(g + 1) * E // G]))))
    cat = torch.cat(parts, dim=1).contiguous()
    assert np.array_equal(_u32(cat), _u32(lg))
    note(f"selection on the gathered rows, G={G}")
    ids2, w2, mg2 = dr.route_select(cat, TOPK)
    assert torch.equal(ids2, ids)
    assert np.array_equal(_u32(w2), _u32(w))
    assert torch.equal(mg2, mg)


@pytest.mark.parametrize("G", [2, 4, 8])
def test_k_shards_combine_in_the_tree_to_the_full_logits(full, G):
    dr = require_gpu()
    W, x, (_, _, lg, _) = full
    ks = K // G
    parts = []
    for g in range(G):
        note(f"K shard {g} of {G}")
        parts.append(dr.route_logits(x[:, g * ks:(g + 1) * ks].contiguous(),
                                     dev(np.ascontiguousarray(W[g * ks:(g + 1) * ks]))))
    while len(parts) > 1:  # the upper levels of the tree: adjacent pairs
        parts = [parts[i] + parts[i + 1] for i in range(0, len(parts), 2)]
    assert np.array_equal(_u32(parts[0]), _u32(lg))
