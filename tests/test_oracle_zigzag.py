"""Pins of the zigzag sharding oracle: the pages' own examples, partition and segment-size
properties, and the closed form that makes the layout balanced."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "zigzag_example.json")


def test_pages_examples():
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["cases"]:
        for s, want in enumerate(c["shards"]):
            got = oracle.zigzag_shard(c["n_tokens"], c["n_shards"], s)
            assert got.tolist() == want


@pytest.mark.parametrize("L,G", [(1, 1), (7, 1), (16, 2), (17, 2), (1000, 3), (4099, 8), (5, 4),
                                 (16384, 8)])
def test_shards_partition_the_chunk(L, G):
    seen = np.concatenate([oracle.zigzag_shard(L, G, g) for g in range(G)])
    assert np.array_equal(np.sort(seen), np.arange(L))
    sizes = [e - b for b, e in oracle.zigzag_segments(L, G)]
    assert sum(sizes) == L and max(sizes) - min(sizes) <= 1
    if G == 1:
        assert oracle.zigzag_shard(L, 1, 0).tolist() == list(range(L))


@pytest.mark.parametrize("G,m,P", [(2, 4, 0), (4, 512, 0), (8, 1024, 65536), (3, 7, 11)])
def test_equal_segments_give_equal_causal_cost(G, m, P):
    """With L = 2 G m the shard cost is, in closed form, 2m(P + 1) + m^2 (2G - 1) + m(m - 1)
    for every shard (segment s holds sum over i in [sm, (s+1)m) of P + i + 1 =
    m(P + 1) + s m^2 + m(m - 1)/2, and the two segments of a shard have s + s' = 2G - 1);
    the contiguous split's costs grow shard by shard."""
    L = 2 * G * m
    want = 2 * m * (P + 1) + m * m * (2 * G - 1) + m * (m - 1)
    for g in range(G):
        assert oracle.causal_cost(oracle.zigzag_shard(L, G, g), P) == want
    cont = [oracle.causal_cost(oracle.contiguous_shard(L, G, g), P) for g in range(G)]
    assert all(b > a for a, b in zip(cont, cont[1:]))
    assert sum(cont) == G * want
