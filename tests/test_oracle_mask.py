"""Pins for the oracle's ancestor-or-self mask (O1).

The mask follows the tree-mask loop in the EAGLE-2 deep-dive page's reference
code. Pins that do not reuse that loop: a hand-worked fixture, graph
reachability from scipy's csgraph, closed forms for chains / stars / forests,
and the row(i) = row(parent) | bit(i) and popcount = depth + 1 invariants.
"""
import json
import os

import numpy as np
import pytest
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import shortest_path

import oracle
import tvgen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bits(mask_row, N):
    return np.array([(int(mask_row[j // 64]) >> (j % 64)) & 1 for j in range(N)], np.int64)


def test_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "mask_hand.json")))
    mask, depth = oracle.build_mask(np.array(g["parents"], np.int32))
    assert mask.tolist() == g["mask_words"]
    assert depth.tolist() == g["depth"]


def reach_matrix(parents):
    """anc-or-self by graph reachability along child->parent edges (csgraph)."""
    N = len(parents)
    r = [i for i in range(N) if parents[i] >= 0]
    c = [parents[i] for i in range(N) if parents[i] >= 0]
    A = csr_matrix((np.ones(len(r)), (r, c)), shape=(N, N))
    dist = shortest_path(A, directed=True, unweighted=True)
    return np.isfinite(dist).astype(np.int64), dist


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("N", [1, 2, 15, 37, 64])
def test_matches_graph_reachability(seed, N):
    parents = tvgen.random_tree(77 + seed, N, N, max_depth=min(N, 9))
    if seed % 2:
        parents[N // 2:] = np.where(np.arange(N // 2, N) % 5 == 0, -1, parents[N // 2:])  # add extra roots
    mask, depth = oracle.build_mask(parents[None, :])
    R, dist = reach_matrix(parents)
    for i in range(N):
        assert (bits(mask[0, i], N) == R[i]).all()
        roots = [j for j in range(N) if R[i, j] and parents[j] < 0]
        assert len(roots) == 1
        assert depth[0, i] == dist[i, roots[0]]


def test_invariants_dynamic_trees():
    w = tvgen.make_workload(3, with_kv=False, with_logits=False)
    mask, depth = oracle.build_mask(w.parents)
    for b in range(w.B):
        for i in range(w.N):
            m = int(mask[b, i, 0])
            assert bin(m).count("1") == depth[b, i] + 1
            p = w.parents[b, i]
            expect = (1 << i) | (int(mask[b, p, 0]) if p >= 0 else 0)
            assert m == expect
        assert (depth[b] == tvgen.tree_depths(w.parents[b])).all()
        assert depth[b].max() <= 8


def test_closed_forms():
    N = 64
    mask, depth = oracle.build_mask(tvgen.chain_tree(N)[None])
    tril = np.tril(np.ones((N, N), np.int64))
    assert all((bits(mask[0, i], N) == tril[i]).all() for i in range(N))
    assert (depth[0] == np.arange(N)).all()
    mask, depth = oracle.build_mask(tvgen.forest_tree(N)[None])
    assert [int(x) for x in mask[0, :, 0]] == [1 << i for i in range(N)]
    assert (depth == 0).all()
    mask, depth = oracle.build_mask(tvgen.star_tree(N)[None])
    assert int(mask[0, 0, 0]) == 1
    assert [int(x) for x in mask[0, 1:, 0]] == [(1 << i) | 1 for i in range(1, N)]
    assert depth[0, 0] == 0 and (depth[0, 1:] == 1).all()


def test_status_codes():
    st, _, _ = oracle.status_build_mask(np.array([[-1, 1]], np.int32))  # parent not earlier
    assert st == oracle.INVALID_TREE
    st, _, _ = oracle.status_build_mask(np.array([[-1, -2]], np.int32))
    assert st == oracle.INVALID_TREE
    st, _, _ = oracle.status_build_mask(np.array([[0, 0]], np.int32))  # root with a parent
    assert st == oracle.INVALID_TREE
    st, _, _ = oracle.status_build_mask(np.full((1, 129), -1, np.int32))
    assert st == oracle.UNSUPPORTED
    st, _, _ = oracle.status_build_mask(np.zeros((0, 5), np.int32))
    assert st == oracle.OK
