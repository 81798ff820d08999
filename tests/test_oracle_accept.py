"""Pins for the oracle's acceptance (O3 greedy, O4 stochastic) and tau (O5).

Greedy is pinned by hand-worked fixtures, planted full matches (a draft that
fully matches accepts depth + 1 tokens), total misses (1 token, the bonus) and
a brute-force enumeration of every root path using numpy's argmax (first
index on ties). Stochastic is pinned by a hand-worked fixture, p == q (always
accept, bonus = numpy searchsorted draw), a chi-square test that the emitted
token follows the target distribution (lossless), the closed-form acceptance
rate sum_x min(p, q), and the temperature -> 0 limit reproducing greedy.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import tvgen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ greedy

def test_greedy_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "greedy_hand.json")))
    r = oracle.accept_greedy(np.array(g["target_logits"], np.float32), np.array(g["draft_tokens"], np.int32),
                             np.array(g["parents"], np.int32))
    for k, v in g["expect"].items():
        assert r[k].tolist() == v, k


def brute_force_greedy(logits, tokens, parents):
    """Enumerate every root->node path; keep the longest all-matching one,
    lexicographically smallest node sequence on ties."""
    N = len(parents)
    y = [int(np.argmax(logits[j])) for j in range(N)]  # first maximal index
    best = None
    for node in range(N):
        path = []
        c = node
        while c >= 0:
            path.append(c)
            c = parents[c]
        path = path[::-1]
        if path[0] != 0:
            continue
        if all(tokens[path[m]] == y[path[m - 1]] for m in range(1, len(path))):
            key = (-len(path), path)
            if best is None or key < best:
                best = key
    path = best[1]
    return len(path), path, y[path[-1]], y


@pytest.mark.parametrize("seed", range(10))
def test_greedy_brute_force_tiny_trees(seed):
    N = 3 + seed
    V = 6  # tiny vocab: many matches, duplicate siblings and exact ties
    w = tvgen.make_workload(1, seed=400 + seed, with_kv=False,
                            overrides=dict(B=16, N=N, V=V, max_depth=3))
    w.target_logits = np.round(w.target_logits * 2) / 2  # force exact ties
    r = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    for b in range(w.B):
        n, path, bonus, y = brute_force_greedy(w.target_logits[b], w.draft_tokens[b], w.parents[b])
        assert r["accept_len"][b] == n
        assert r["path"][b].tolist() == path + [-1] * (N - n)
        assert r["bonus"][b] == bonus
        assert r["target_argmax"][b].tolist() == y


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_planted_full_match_accepts_depth_plus_one(cfg):
    w = tvgen.make_workload(cfg, with_kv=False, overrides=dict(B=4, V=4096))
    depth = np.stack([tvgen.tree_depths(p) for p in w.parents])
    leaves = []
    for b in range(w.B):
        leaf = int(np.argmax(depth[b]))  # a deepest node (lowest id)
        tvgen.plant_full_path(w, b, leaf)
        leaves.append(leaf)
    r = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    for b in range(w.B):
        assert r["accept_len"][b] == depth[b, leaves[b]] + 1
        assert r["bonus"][b] == int(np.argmax(w.target_logits[b, r["path"][b][r["accept_len"][b] - 1]]))


def test_total_miss_accepts_only_bonus():
    w = tvgen.make_workload(2, with_kv=False, overrides=dict(B=3, V=2048))
    y = w.target_logits.argmax(-1)
    # make sure no node matches: move each draft token off its parent's argmax
    for b in range(w.B):
        for c in range(1, w.N):
            if w.draft_tokens[b, c] == y[b, w.parents[b, c]]:
                w.draft_tokens[b, c] = (w.draft_tokens[b, c] + 1) % w.V
    r = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    assert (r["accept_len"] == 1).all()
    assert (r["bonus"] == y[:, 0]).all()
    assert (r["path"][:, 0] == 0).all() and (r["path"][:, 1:] == -1).all()


def test_chain_first_mismatch():
    N, V = 8, 50
    w = tvgen.make_workload(5, with_kv=False, overrides=dict(B=1, N=N, V=V, mode="greedy"))
    y = w.target_logits[0].argmax(-1)
    for c in range(1, N):
        w.draft_tokens[0, c] = y[c - 1] if c != 5 else (y[c - 1] + 1) % V
    r = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    assert r["accept_len"][0] == 5
    assert r["path"][0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert r["bonus"][0] == y[4]


def test_greedy_status_codes():
    w = tvgen.make_workload(1, with_kv=False)
    ok = (w.target_logits, w.draft_tokens, w.parents, w.B, w.N, w.V)
    assert oracle.status_accept_greedy(*ok)[0] == oracle.OK
    p = w.parents.copy()
    p[0, 0] = 0
    assert oracle.status_accept_greedy(w.target_logits, w.draft_tokens, p, w.B, w.N, w.V)[0] == oracle.INVALID_TREE
    t = w.draft_tokens.copy()
    t[0, 3] = w.V
    assert oracle.status_accept_greedy(w.target_logits, t, w.parents, w.B, w.N, w.V)[0] == oracle.INVALID_ARG
    assert oracle.status_accept_greedy(w.target_logits, w.draft_tokens, w.parents, w.B, w.N, 0)[0] == \
        oracle.INVALID_ARG


# ------------------------------------------------------------------ stochastic

def test_stochastic_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "stochastic_hand.json")))
    r = oracle.accept_stochastic(np.array(g["target_logits"], np.float32), np.array(g["draft_logits"], np.float32),
                                 np.array(g["draft_tokens"], np.int32), np.array(g["parents"], np.int32),
                                 np.array(g["uniforms"], np.float32), g["temperature"])
    for k, v in g["expect"].items():
        assert r[k].tolist() == v, k


def softmax64(x, T=1.0):
    z = x.astype(np.float64) / T
    e = np.exp(z - z.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def test_p_equals_q_accepts_everything():
    w = tvgen.make_workload(5, overrides=dict(B=16, V=500), with_kv=False)
    w.draft_logits[:, 1:] = w.target_logits[:, :-1]
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, 1.0)
    assert (r["accept_len"] == w.N).all()
    for b in range(w.B):
        p = softmax64(w.target_logits[b, -1])
        cdf = np.cumsum(p)
        expect = int(np.searchsorted(cdf, w.uniforms[b, -1] * cdf[-1], side="right"))
        assert r["bonus"][b] == expect


def lossless_trial(V=8, M=200000, seed=11, T=1.0):
    """M independent single-draft cycles with fixed rows p0 (target) and q1
    (draft); t1 ~ q1. Returns emitted first tokens and acceptance flags."""
    base = tvgen.normal_f32(seed, 1, (2, V), sigma=1.5)
    tl = np.zeros((M, 2, V), np.float32)
    dl = np.zeros((M, 2, V), np.float32)
    tl[:, 0] = base[0]
    tl[:, 1] = 0.0
    dl[:, 1] = base[1]
    tokens = np.zeros((M, 2), np.int32)
    tokens[:, 1] = tvgen.gumbel_argmax(seed, 2, dl[:, 1], T)
    u = tvgen.uniform_f32(seed, 3, (M, 2))
    parents = np.tile(np.array([-1, 0], np.int32), (M, 1))
    r = oracle.accept_stochastic(tl, dl, tokens, parents, u, T)
    emitted = np.where(r["accept_len"] == 2, tokens[:, 1], r["bonus"])
    return emitted, r["accept_len"] == 2, softmax64(base[0], T), softmax64(base[1], T), tokens[:, 1]


def test_lossless_chi_square():
    emitted, _, p, q, drafts = lossless_trial()
    M = emitted.size
    obs = np.bincount(emitted, minlength=p.size)
    # sanity: the draft tokens really follow q, and q differs from p
    assert stats.chisquare(np.bincount(drafts, minlength=q.size), q * M).pvalue > 1e-4
    assert np.abs(p - q).sum() > 0.3
    assert stats.chisquare(obs, p * M).pvalue > 1e-4


def test_acceptance_rate_closed_form():
    _, acc, p, q, _ = lossless_trial(seed=12)
    rate = np.minimum(p, q).sum()
    M = acc.size
    assert abs(acc.mean() - rate) < 5 * np.sqrt(rate * (1 - rate) / M)


def test_temperature_to_zero_reproduces_greedy():
    V, N = 256, 6
    w = tvgen.make_workload(5, seed=77, with_kv=False, overrides=dict(B=64, N=N, V=V))
    T = 1e-6
    # top-two gaps must dwarf T: runner-up mass <= V * exp(-100), far below
    # the 2^-24 resolution of the uniforms, so the limit holds exactly
    for arr in (w.target_logits, w.draft_logits):
        srt = np.sort(arr.reshape(-1, V), axis=-1)
        assert (srt[:, -1] - srt[:, -2]).min() > 100 * T
    assert w.uniforms.min() > 0
    w.draft_tokens[:, 1:] = w.draft_logits[:, 1:].argmax(-1)  # T -> 0 draft sampling is argmax
    # make about half of the drafts match the target's argmax at the parent
    y = w.target_logits.argmax(-1)
    for b in range(0, w.B, 2):
        for i in range(1, N):
            w.draft_tokens[b, i] = y[b, i - 1]
            w.draft_logits[b, i, y[b, i - 1]] = w.draft_logits[b, i].max() + 1.0
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, T)
    g = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    assert (r["accept_len"] == g["accept_len"]).all()
    assert (r["bonus"] == g["bonus"]).all()
    assert (r["accept_len"][::2] == N).all()


def test_margins_reported():
    w = tvgen.make_workload(5, overrides=dict(B=32, V=1000), with_kv=False)
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, 1.0)
    m = r["margins"]
    for b in range(w.B):
        k = r["accept_len"][b] - 1
        tested = min(k + 1, w.N - 1)
        assert np.isfinite(m[b, :tested]).all()
        assert np.isinf(m[b, tested:w.N - 1]).all()
        assert 0 <= m[b, -1] <= 1


def test_stochastic_status_codes():
    w = tvgen.make_workload(5, overrides=dict(B=2, V=100), with_kv=False)
    args = (w.target_logits, w.draft_logits, w.draft_tokens)
    assert oracle.status_accept_stochastic(*args, w.parents, w.uniforms, w.B, w.N, w.V, 1.0)[0] == oracle.OK
    tree = w.parents.copy()
    tree[:, 2] = 0  # a tree: accepted
    assert oracle.status_accept_stochastic(*args, tree, w.uniforms, w.B, w.N, w.V, 1.0)[0] == oracle.OK
    tree[:, 3] = 3  # a parent not earlier than its child
    assert oracle.status_accept_stochastic(*args, tree, w.uniforms, w.B, w.N, w.V, 1.0)[0] == oracle.INVALID_TREE
    tree = w.parents.copy()
    tree[:, 0] = 0  # the root must have no parent
    assert oracle.status_accept_stochastic(*args, tree, w.uniforms, w.B, w.N, w.V, 1.0)[0] == oracle.INVALID_TREE
    assert oracle.status_accept_stochastic(*args, w.parents, w.uniforms, w.B, w.N, w.V, 0.0)[0] == \
        oracle.INVALID_ARG


# ------------------------------------------------------------------ stochastic on trees

def test_stochastic_tree_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "stochastic_tree_hand.json")))
    B = len(g["parents"])
    tl = np.tile(np.array(g["target_rows"], np.float32)[None], (B, 1, 1))
    dl = np.tile(np.array(g["draft_rows"], np.float32)[None], (B, 1, 1))
    r = oracle.accept_stochastic(tl, dl, np.array(g["draft_tokens"], np.int32), np.array(g["parents"], np.int32),
                                 np.array(g["uniforms"], np.float32), g["temperature"])
    for k, v in g["expect"].items():
        assert r[k].tolist() == v, k
    assert (r["margins"][np.isfinite(r["margins"])] > 0.02).all()


def sample_rows(seed, tid, q):
    """One token per row of the probability matrix q by inverse CDF (seeded)."""
    u = tvgen.uniform_f32(seed, tid, (q.shape[0],)).astype(np.float64)
    c = np.cumsum(q, -1)
    return np.minimum((c < (u * c[:, -1])[:, None]).sum(-1), q.shape[1] - 1).astype(np.int32)


def star_trial(k=3, V=8, M=200000, seed=21, without_replacement=False, with_path=False):
    """M cycles of a root with k children; child c's token drawn from its
    draft row (with or without the earlier siblings' tokens). Target rows of
    the children depend only on their token (table P2), as a real target's
    would. Returns (emitted tokens [M][2], accept_len, p0, q rows, P2)."""
    N = k + 1
    base = tvgen.normal_f32(seed, 1, (1 + k, V), sigma=1.5)
    P2 = tvgen.normal_f32(seed, 2, (V, V), sigma=1.0)
    tl = np.zeros((M, N, V), np.float32)
    dl = np.zeros((M, N, V), np.float32)
    tl[:, 0] = base[0]
    tokens = np.zeros((M, N), np.int32)
    for c in range(1, N):
        row = np.tile(base[c], (M, 1))
        if without_replacement:
            for e in range(1, c):
                row[np.arange(M), tokens[:, e]] = -np.inf
        dl[:, c] = row
        tokens[:, c] = sample_rows(seed, 10 + c, softmax64(row))
        tl[:, c] = P2[tokens[:, c]]
    u = tvgen.uniform_f32(seed, 3, (M, N))
    parents = np.tile(np.array([-1] + [0] * k, np.int32), (M, 1))
    r = oracle.accept_stochastic(tl, dl, tokens, parents, u, 1.0)
    first = np.where(r["accept_len"] >= 2, tokens[np.arange(M), np.maximum(r["path"][:, 1], 0)], r["bonus"])
    second = np.where(r["accept_len"] >= 2, r["bonus"], -1)
    out = (np.stack([first, second], 1), r["accept_len"], softmax64(base[0]), softmax64(base[1:]), P2)
    return out + (r["path"][:, 1],) if with_path else out


@pytest.mark.parametrize("without_replacement", [False, True])
def test_tree_lossless_first_token(without_replacement):
    em, alen, p, q, _ = star_trial(without_replacement=without_replacement, seed=21 + without_replacement)
    M = alen.size
    assert np.abs(p - q[0]).sum() > 0.3 and (alen == 1).mean() > 0.05  # rejections of every sibling happen
    assert stats.chisquare(np.bincount(em[:, 0], minlength=p.size), p * M).pvalue > 1e-4


def test_tree_lossless_second_token():
    """Given the first token x came from an accepted child, the next token
    follows the target's distribution after x (the child's row P2[x])."""
    em, alen, _, _, P2 = star_trial(seed=31)
    for x in range(P2.shape[0]):
        sel = (alen == 2) & (em[:, 0] == x)
        if sel.sum() < 2000:
            continue
        obs = np.bincount(em[sel, 1], minlength=P2.shape[1])
        assert stats.chisquare(obs, softmax64(P2[x]) * sel.sum()).pvalue > 1e-4, x


def test_tree_sibling_acceptance_closed_form():
    # child 1 is accepted w.p. a1 = sum min(p, q1); child 2, tested after a
    # rejection, w.p. (1 - a1) * sum min(pi1, q2) with pi1 = norm(max(0, p - q1))
    _, alen, p, q, _, acc_child = star_trial(k=2, seed=41, with_path=True)
    M = alen.size
    a1 = np.minimum(p, q[0]).sum()
    r1 = np.maximum(p - q[0], 0)
    a2 = (1 - a1) * np.minimum(r1 / r1.sum(), q[1]).sum()
    for child, rate in ((1, a1), (2, a2)):
        got = (acc_child == child).mean()
        assert abs(got - rate) < 5 * np.sqrt(rate * (1 - rate) / M), (child, got, rate)


def test_tree_temperature_to_zero_reproduces_greedy():
    # dynamic trees have distinct sibling tokens, so at most one child of a
    # node matches and the greedy longest path is the first-match walk
    V, N = 200, 24
    w = tvgen.make_workload(2, seed=78, with_kv=False, overrides=dict(B=64, N=N, V=V))
    w.draft_logits = tvgen.normal_f32(78, 90, (w.B, N, V))
    w.uniforms = tvgen.uniform_f32(78, 91, (w.B, N))
    T = 1e-6
    y = w.target_logits.argmax(-1)
    for b in range(w.B):
        for pnode in range(N):
            kids = np.nonzero(w.parents[b] == pnode)[0]
            # plant a match under about a third of the parents, keeping the
            # siblings' tokens distinct
            if len(kids) and (b + pnode) % 3 == 0 and y[b, pnode] not in w.draft_tokens[b, kids]:
                w.draft_tokens[b, kids[(b + pnode) % len(kids)]] = y[b, pnode]
    for b in range(w.B):
        for pnode in range(N):
            kids = np.nonzero(w.parents[b] == pnode)[0]
            assert len(set(w.draft_tokens[b, kids].tolist())) == len(kids)
    for c in range(1, N):
        w.draft_logits[np.arange(w.B), c, w.draft_tokens[:, c]] = w.draft_logits[:, c].max(-1) + 1.0
    for arr in (w.target_logits, w.draft_logits[:, 1:]):
        srt = np.sort(arr.reshape(-1, V), axis=-1)
        assert (srt[:, -1] - srt[:, -2]).min() > 100 * T
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, T)
    g = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
    assert (r["accept_len"] == g["accept_len"]).all()
    assert (r["path"] == g["path"]).all()
    assert (r["bonus"] == g["bonus"]).all()
    assert g["accept_len"].max() >= 3


def test_tree_star_with_p_equal_q_accepts_first_child():
    w = tvgen.make_workload(5, seed=79, with_kv=False, overrides=dict(B=32, V=300, N=6))
    w.parents[:] = [-1, 0, 0, 0, 0, 0]
    w.draft_logits[:, 1:] = w.target_logits[:, :1]
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, 1.0)
    assert (r["accept_len"] == 2).all() and (r["path"][:, 1] == 1).all()


# ------------------------------------------------------------------ tau

def test_tau_is_mean_accepted_tokens():
    assert oracle.tau([]) == 0.0
    assert oracle.tau([1, 2, 3, 4]) == 2.5
    assert oracle.tau(np.array([[5, 1], [1, 1]])) == 2.0
