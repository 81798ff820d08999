"""Pins for the oracle's accepted-path commit (O6).

The commit is pinned by a hand-worked fixture, by the equivalence it exists
for (after the commit, plain decoding of each accepted node over the grown
prefix gives the same attention as that node's row in tree attention over the
original cache), by greedy losslessness (the emitted tokens are what greedy
decoding with the target alone would emit), by the identity of a fully
accepted chain, and by status codes that leave bad sequences unchanged.
"""
import json
import os

import numpy as np
import pytest

import oracle
import tvgen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tagged_pages(P, Hkv, D, seed):
    """Distinct random bits per row so any misplaced row is visible."""
    k = tvgen.u64(seed, 1, P * Hkv * 16 * D).astype(np.uint16).reshape(P, Hkv, 16, D)
    v = tvgen.u64(seed, 2, P * Hkv * 16 * D).astype(np.uint16).reshape(P, Hkv, 16, D)
    return k, v


def row(pages, table, b, t):
    return pages[table[b, t // 16], :, t % 16, :]


def test_commit_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "commit_hand.json")))
    D, Hkv, P = g["D"], g["Hkv"], g["num_pages"]
    table = np.array(g["page_table"], np.int32)
    lens = np.array(g["prefix_lens"], np.int32)
    B, N = len(lens), len(g["parents"][0])
    k0, v0 = tagged_pages(P, Hkv, D, 5)
    st, k, v, r = oracle.status_commit(k0, v0, table, lens, g["draft_tokens"], g["path"], g["accept_len"],
                                       g["bonus"], B=B, N=N, Hkv=Hkv, D=D)
    assert st == oracle.OK
    e = g["expect"]
    assert r["new_prefix_lens"].tolist() == e["new_prefix_lens"]
    assert r["emitted"].tolist() == e["emitted"]
    assert r["next_root"].tolist() == e["next_root"]
    for b in range(B):
        moved = dict((d, s) for d, s in e["moved_rows"][str(b)])
        for t in range(lens[b] + N):
            src = moved.get(t, t)
            assert np.array_equal(row(k, table, b, t), row(k0, table, b, src)), (b, t)
            assert np.array_equal(row(v, table, b, t), row(v0, table, b, src)), (b, t)
    # pages no sequence touches keep their bits
    used = set(table[table >= 0].tolist())
    for p in range(P):
        if p not in used:
            assert np.array_equal(k[p], k0[p])


def small_tree_workload(seed, B=6, N=12, L=(1, 40), tree="random"):
    ov = dict(B=B, N=N, L=L, V=64, tree=tree, pages="permuted")
    if tree == "random":
        ov["max_depth"] = 6
    return tvgen.make_workload(2, seed, overrides=ov)


@pytest.mark.parametrize("seed", range(4))
def test_commit_then_decode_equals_tree_attention(seed):
    """Row of node v_m in tree attention (original cache) == attention of the
    same query as a single new token at position L+m over the committed cache."""
    w = small_tree_workload(300 + seed)
    tvgen.plant_random(w, 0.8, seed=seed)
    acc = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    mask, _ = oracle.build_mask(w.parents)
    tree_out = oracle.attention(w, mask)
    k, v, r = oracle.commit(w, acc["path"], acc["accept_len"], acc["bonus"])
    assert np.array_equal(r["new_prefix_lens"], w.prefix_lens + acc["accept_len"])
    assert acc["accept_len"].max() >= 3
    one = np.ones((1, 1, 1), np.uint64)
    for b in range(w.B):
        for m in range(acc["accept_len"][b]):
            node = acc["path"][b, m]
            st, out = oracle.status_attention(w.q[b:b + 1, node:node + 1], k, v, w.page_table[b:b + 1],
                                              np.array([w.prefix_lens[b] + m], np.int32), one, B=1, N=1,
                                              Hq=w.Hq, Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale,
                                              num_pages=w.num_pages)
            assert st == oracle.OK
            np.testing.assert_allclose(out.reshape(w.Hq, w.D), tree_out[b, node], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_commit_emits_the_greedy_decode(seed):
    """Greedy speculation is lossless: token m emitted is the target's argmax
    after path node v_m, i.e. what decoding with the target alone gives."""
    w = small_tree_workload(400 + seed, B=8, N=20)
    tvgen.plant_random(w, 0.7, seed=11 + seed)
    acc = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    _, _, r = oracle.commit(w, acc["path"], acc["accept_len"], acc["bonus"])
    for b in range(w.B):
        n = acc["accept_len"][b]
        want = [int(np.argmax(w.target_logits[b, acc["path"][b, m]])) for m in range(n)]
        assert r["emitted"][b, :n].tolist() == want
        assert (r["emitted"][b, n:] == -1).all()
        assert r["next_root"][b] == want[-1]


def test_commit_full_chain_is_identity():
    w = small_tree_workload(500, B=4, N=6, tree="chain")
    path = np.tile(np.arange(w.N, dtype=np.int32), (w.B, 1))
    lens = np.full(w.B, w.N, np.int32)
    bonus = np.arange(w.B, dtype=np.int32) + 100
    k, v, r = oracle.commit(w, path, lens, bonus)
    assert np.array_equal(k, w.k_pages) and np.array_equal(v, w.v_pages)
    assert np.array_equal(r["new_prefix_lens"], w.prefix_lens + w.N)
    assert np.array_equal(r["emitted"], np.concatenate([w.draft_tokens[:, 1:], bonus[:, None]], 1))


def test_commit_root_only_moves_nothing():
    w = small_tree_workload(501, B=3, N=9)
    path = np.full((w.B, w.N), -1, np.int32)
    path[:, 0] = 0
    k, v, r = oracle.commit(w, path, np.ones(w.B, np.int32), np.array([4, 5, 6], np.int32))
    assert np.array_equal(k, w.k_pages) and np.array_equal(v, w.v_pages)
    assert r["emitted"][:, 0].tolist() == [4, 5, 6] and (r["emitted"][:, 1:] == -1).all()


@pytest.mark.parametrize("bad", ["len0", "len_big", "root", "order", "node_big", "bonus", "page", "page_big",
                                 "prefix_big", "prefix_neg"])
def test_commit_bad_sequence_left_unchanged(bad):
    w = small_tree_workload(502, B=3, N=8, tree="chain")
    path = np.full((w.B, w.N), -1, np.int32)
    path[:, :4] = [0, 2, 5, 7]  # a valid increasing path (the commit reads no parents)
    lens = np.full(w.B, 4, np.int32)
    bonus = np.array([1, 2, 3], np.int32)
    table = w.page_table.copy()
    prefix = w.prefix_lens.copy()
    b = 1
    if bad == "len0":
        lens[b] = 0
    elif bad == "len_big":
        lens[b] = w.N + 1
    elif bad == "root":
        path[b, 0] = 1
    elif bad == "order":
        path[b, 1:4] = [5, 2, 7]
    elif bad == "node_big":
        path[b, 3] = w.N
    elif bad == "bonus":
        bonus[b] = -1
    elif bad == "page":
        table[b, (prefix[b] + 7) // 16] = -1
    elif bad == "page_big":
        table[b, (prefix[b] + 7) // 16] = w.num_pages
    elif bad == "prefix_big":
        prefix[b] = table.shape[1] * 16 - w.N + 1
    elif bad == "prefix_neg":
        prefix[b] = -1
    st, k, v, r = oracle.status_commit(w.k_pages, w.v_pages, table, prefix, w.draft_tokens, path, lens, bonus,
                                       B=w.B, N=w.N, Hkv=w.Hkv, D=w.D, num_pages=w.num_pages,
                                       max_prefix_len=max(int(prefix.max()), 0))
    assert st == oracle.INVALID_ARG
    assert r["new_prefix_lens"][b] == prefix[b] and r["next_root"][b] == -1
    assert (r["emitted"][b] == -1).all()
    for pid in w.page_table[b][w.page_table[b] >= 0]:
        assert np.array_equal(k[pid], w.k_pages[pid]) and np.array_equal(v[pid], w.v_pages[pid])
    # the good sequences are still committed
    for g in (0, 2):
        assert r["new_prefix_lens"][g] == prefix[g] + 4 and r["next_root"][g] == bonus[g]
        t_dst, t_src = prefix[g] + 3, prefix[g] + 7
        assert np.array_equal(row(k, table, g, t_dst), row(w.k_pages, table, g, t_src))


def test_commit_argument_errors():
    w = small_tree_workload(503, B=2, N=4, tree="chain")
    path = np.tile(np.arange(w.N, dtype=np.int32), (w.B, 1))
    lens = np.full(w.B, w.N, np.int32)
    bonus = np.zeros(w.B, np.int32)
    args = (w.k_pages, w.v_pages, w.page_table, w.prefix_lens, w.draft_tokens, path, lens, bonus)
    for kw in (dict(D=96), dict(N=0), dict(N=129), dict(Hkv=0), dict(B=-1)):
        base = dict(B=w.B, N=w.N, Hkv=w.Hkv, D=w.D)
        base.update(kw)
        st, *_ = oracle.status_commit(*args, **base, num_pages=w.num_pages)
        assert st == oracle.INVALID_ARG, kw
    st, *_ = oracle.status_commit(*args, B=0, N=w.N, Hkv=w.Hkv, D=w.D, num_pages=w.num_pages)
    assert st == oracle.OK
