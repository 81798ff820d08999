"""Pins for the oracle's dynamic draft-tree builder (O7).

The builder is pinned by a hand-worked fixture, by agreement with the
input generator's own implementation of the same best-first expansion (a
heap with insertion counters, written separately), by brute force (the
created nodes are exactly the highest-scoring nodes of the full candidate
tree that the threshold and depth limit allow), and by invariants: scores are
products along root paths, pops never increase in score, masks are ancestor
masks, short trees are padded.
"""
import json
import os

import numpy as np
import pytest

import oracle
import tvgen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_tree_build_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "tree_build_hand.json")))
    r = oracle.build_tree(np.array(g["root_tokens"], np.int32), np.array(g["cand_tokens"], np.int32),
                          np.array(g["cand_probs"], np.float32), k_root=g["k_root"], threshold=g["threshold"],
                          max_depth=g["max_depth"])
    for key, v in g["expect"].items():
        assert r[key].tolist() == v, key
    mask, _ = oracle.build_mask(r["parents"])
    assert np.array_equal(r["mask"], mask)


def generator_tables(seed, B, N, max_depth, topk, V):
    """Trees from the input generator plus the proposal rows it drew, laid
    out by creation order (fp32 probabilities)."""
    trees, toks, probs = [], np.zeros((B, N, topk), np.int32), np.zeros((B, N, topk), np.float32)
    for b in range(B):
        rec = {}
        p, t = tvgen.dynamic_tree(seed, b, N, max_depth, topk, V, record=rec)
        trees.append((p, t))
        for node, (tk, sc) in rec.items():
            if node < N:
                toks[b, node] = tk
                probs[b, node] = sc
    return trees, toks, probs


@pytest.mark.parametrize("seed,N,max_depth,topk", [(1, 64, 6, 10), (2, 60, 8, 10), (3, 40, 4, 4), (4, 64, 8, 3)])
def test_tree_build_matches_generator(seed, N, max_depth, topk):
    B, V = 12, 5000
    trees, toks, probs = generator_tables(seed, B, N, max_depth, topk, V)
    roots = np.array([t[0] for _, t in trees], np.int32)
    r = oracle.build_tree(roots, toks, probs, k_root=topk, threshold=0.0, max_depth=max_depth)
    compared = 0
    for b, (p, t) in enumerate(trees):
        # the generator multiplies fp64 probabilities, the builder their fp32
        # roundings: skip a tree whose best-first order has a near tie
        s = r["scores"][b, 1:]
        if (np.abs(np.diff(np.sort(s))) <= 1e-6 * s.max()).any():
            continue
        compared += 1
        assert np.array_equal(r["parents"][b], p), b
        assert np.array_equal(r["tokens"][b], t), b
        assert r["n_nodes"][b] == N
    assert compared >= B // 2


def full_candidate_tree(seed, k, depth):
    """Every node of the complete k-ary candidate tree to `depth`: id -> (parent
    id, slot, probability); ids in breadth-first order, the root is 0."""
    nodes = {0: (-1, -1, 1.0)}
    probs = tvgen.uniform_f32(seed, 5, (k ** (depth + 1),)).astype(np.float64) * 0.9 + 0.05
    frontier, nid = [0], 1
    for _ in range(depth):
        nxt = []
        for par in frontier:
            for s in range(k):
                nodes[nid] = (par, s, float(np.float32(probs[nid])))
                nxt.append(nid)
                nid += 1
        frontier = nxt
    return nodes


@pytest.mark.parametrize("seed,k,depth,N,threshold", [(7, 3, 3, 20, 0.0), (8, 3, 4, 40, 0.02), (9, 2, 5, 25, 0.05),
                                                      (10, 4, 2, 21, 0.3)])
def test_tree_build_brute_force_top_scores(seed, k, depth, N, threshold):
    nodes = full_candidate_tree(seed, k, depth)
    children = {}
    for nid, (par, s, _) in nodes.items():
        if par >= 0:
            children.setdefault(par, [None] * k)[s] = nid
    score = {0: 1.0}
    for nid in sorted(nodes):
        par, _, pr = nodes[nid]
        if par >= 0:
            score[nid] = score[par] * pr
    depth_of = {0: 0}
    for nid in sorted(nodes):
        if nid:
            depth_of[nid] = depth_of[nodes[nid][0]] + 1
    # eligible: the root's children always; deeper nodes above the threshold
    elig = [n for n in nodes if n and (depth_of[n] == 1 or score[n] > np.float32(threshold))]
    top = sorted(elig, key=lambda n: -score[n])[:N - 1]
    assert len(set(score[n] for n in elig)) == len(elig)  # distinct scores
    # proposal rows by creation order, consistent with the full tree: iterate
    # until the rows of the created nodes are those nodes' children
    rows_nodes = [0] * N
    for _ in range(N + 1):
        toks = np.zeros((1, N, k), np.int32)
        prb = np.zeros((1, N, k), np.float32)
        for i, nid in enumerate(rows_nodes):
            for s, c in enumerate(children.get(nid, [])):
                toks[0, i, s] = c
                prb[0, i, s] = nodes[c][2]
        r = oracle.build_tree(np.array([0], np.int32), toks, prb, k_root=k, threshold=threshold, max_depth=depth)
        created = r["tokens"][0, :r["n_nodes"][0]].tolist()
        if created[1:] == rows_nodes[1:len(created)]:
            break
        rows_nodes = created + [0] * (N - len(created))
    assert sorted(created[1:]) == sorted(top)
    assert r["n_nodes"][0] == min(N, 1 + len(elig))


def test_tree_build_invariants():
    B, N, k, V = 16, 64, 6, 1000
    toks = tvgen.u64(11, 1, B * N * k).reshape(B, N, k) % V
    probs = tvgen.uniform_f32(11, 2, (B, N, k))
    roots = np.arange(B, dtype=np.int32)
    for thr, md in ((0.0, 8), (1e-3, 6), (0.05, 3)):
        r = oracle.build_tree(roots, toks.astype(np.int32), probs, k_root=4, threshold=thr, max_depth=md)
        mask, depth = oracle.build_mask(r["parents"])
        assert np.array_equal(r["mask"], mask)
        for b in range(B):
            n = r["n_nodes"][b]
            s, p, d = r["scores"][b], r["parents"][b], r["depth"][b]
            assert np.array_equal(d[:n], depth[b, :n]) and d.max() <= md
            assert (np.diff(s[1:n]) <= 0).all()  # best-first pops never increase
            for i in range(1, n):
                row = p[i]
                slot = [j for j in range(4 if row == 0 else k) if toks[b, row, j] == r["tokens"][b, i] and
                        s[row] * np.float64(probs[b, row, j]) == s[i]]
                assert slot, (b, i)
                assert d[i] == 1 or s[i] > np.float32(thr)
            assert (p[n:] == -1).all() and (r["tokens"][b, n:] == roots[b]).all() and (s[n:] == 0).all()


def test_tree_build_status():
    toks = np.zeros((2, 4, 3), np.int32)
    probs = np.full((2, 4, 3), 0.5, np.float32)
    roots = np.array([5, 6], np.int32)
    kw = dict(k_root=2, threshold=0.0, max_depth=3)
    st, r = oracle.status_build_tree(roots, toks, probs, **kw)
    assert st == oracle.OK and (r["n_nodes"] == 4).all()
    bad = probs.copy()
    bad[1, 2, 1] = np.nan
    st, r = oracle.status_build_tree(roots, toks, bad, **kw)
    assert st == oracle.INVALID_ARG
    assert r["n_nodes"].tolist() == [4, 0] and (r["parents"][1] == -1).all() and (r["tokens"][1] == 6).all()
    bad[1, 2, 1] = -0.5
    assert oracle.status_build_tree(roots, toks, bad, **kw)[0] == oracle.INVALID_ARG
    assert oracle.status_build_tree(roots, toks, probs, k_root=4, threshold=0.0, max_depth=3)[0] == oracle.INVALID_ARG
    assert oracle.status_build_tree(roots, toks, probs, k_root=2, threshold=0.0, max_depth=0)[0] == oracle.INVALID_ARG
    assert oracle.status_build_tree(roots, toks, probs, B=0, **kw)[0] == oracle.OK
    big = np.zeros((1, 129, 3), np.int32)
    assert oracle.status_build_tree(roots[:1], big, np.zeros((1, 129, 3), np.float32), **kw)[0] == oracle.INVALID_ARG
