"""Pins for trees of up to 128 nodes (two mask words per row) and for per-
sequence node counts (tree_sizes) in the oracle.

Two independent references:
  - 128-node chains are causal attention over [prefix | tree] (torch's float64
    scaled_dot_product_attention), and their masks are lower triangles;
  - a sequence with n_b of N slots gives exactly what the same tree truncated
    to n_b nodes gives when computed with N = n_b and no node counts (a
    different size of every loop and mask layout), and its absent rows are
    empty (mask 0, depth -1, attention NaN, argmax -1).
"""
import numpy as np
import pytest
import torch

import oracle
import tvgen
from test_oracle_attention import sdpa, seq_kv, seq_q


def sizes_for(seed, B, N):
    s = tvgen.Stream(seed, 3)
    return np.array([1 + s.randint(N) for _ in range(B)], np.int32)


@pytest.mark.parametrize("N", [65, 100, 128])
def test_long_chain_mask_and_causal_attention(N):
    w = tvgen.make_workload(1, seed=600 + N, with_logits=False,
                            overrides=dict(B=2, Hq=4, Hkv=2, D=64, L=(0, 40), N=N, tree="chain"))
    mask, depth = oracle.build_mask(w.parents)
    assert mask.shape == (2, N, 2)
    dense = np.unpackbits(mask.view(np.uint8), axis=-1, bitorder="little")[..., :N].astype(bool)
    assert np.array_equal(dense[0], np.tril(np.ones((N, N), bool)))
    assert np.array_equal(depth[0], np.arange(N))
    out = oracle.attention(w, mask)
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        k, v = seq_kv(w, b)
        causal = torch.ones(N, L + N, dtype=torch.bool).tril(diagonal=L)
        ref = sdpa(seq_q(w, b), k, v, w.sm_scale, causal)  # [Hq][N][D]
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def truncated(w, b, n):
    """Sequence b of workload w with only its first n nodes, as a workload of N = n."""
    t = tvgen.make_workload(1, seed=w.seed, with_kv=False, with_logits=False,
                            overrides=dict(B=1, N=n, Hq=w.Hq, Hkv=w.Hkv, D=w.D, L=1, tree="chain"))
    t.parents = w.parents[b:b + 1, :n].copy()
    t.draft_tokens = w.draft_tokens[b:b + 1, :n].copy()
    t.prefix_lens = w.prefix_lens[b:b + 1].copy()
    t.max_prefix_len = int(t.prefix_lens[0])
    t.page_table = w.page_table[b:b + 1].copy()
    t.num_pages = w.num_pages
    if w.q is not None:
        t.q = w.q[b:b + 1, :n].copy()
        t.k_pages, t.v_pages = w.k_pages, w.v_pages
    if w.target_logits is not None:
        t.target_logits = w.target_logits[b:b + 1, :n].copy()
    if w.draft_logits is not None:
        t.draft_logits = w.draft_logits[b:b + 1, :n].copy()
        t.uniforms = w.uniforms[b:b + 1, :n].copy()
        t.uniforms[0, n - 1] = w.uniforms[b, w.N - 1]  # the final draw's uniform sits at the last slot
    return t


@pytest.mark.parametrize("N,tree", [(40, "random"), (100, "random"), (128, "dynamic")])
def test_sizes_mask_and_attention_equal_truncated_trees(N, tree):
    over = dict(B=4, Hq=4, Hkv=2, D=64, L=(0, 60), N=N, tree=tree, V=300, max_depth=7)
    if tree == "dynamic":
        over["topk"] = 6
    w = tvgen.make_workload(2, seed=700 + N, overrides=over)
    sizes = sizes_for(N, w.B, N)
    sizes[0] = N
    mask, depth = oracle.build_mask(w.parents, tree_sizes=sizes)
    out = oracle.attention(w, mask, tree_sizes=sizes)
    for b in range(w.B):
        n = int(sizes[b])
        assert (mask[b, n:] == 0).all() and (depth[b, n:] == -1).all()
        assert np.isnan(out[b, n:]).all()
        t = truncated(w, b, n)
        tm, td = oracle.build_mask(t.parents)
        W = tm.shape[-1]
        assert np.array_equal(mask[b, :n, :W], tm[0]) and (mask[b, :n, W:] == 0).all()
        assert np.array_equal(depth[b, :n], td[0])
        np.testing.assert_allclose(out[b, :n], oracle.attention(t, tm)[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("N", [30, 128])
def test_sizes_greedy_equals_truncated_trees(N):
    w = tvgen.make_workload(2, seed=800 + N, with_kv=False,
                            overrides=dict(B=6, N=N, V=200, tree="random", max_depth=9))
    tvgen.plant_random(w, 0.8, seed=N)
    sizes = sizes_for(N + 1, w.B, N)
    # absent nodes may hold anything: bad parents, bad tokens, NaN logits
    for b in range(w.B):
        w.parents[b, sizes[b]:] = 99999
        w.draft_tokens[b, sizes[b]:] = -7
        w.target_logits[b, sizes[b]:] = np.nan
    r = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents, tree_sizes=sizes)
    for b in range(w.B):
        n = int(sizes[b])
        t = truncated(w, b, n)
        ref = oracle.accept_greedy(t.target_logits, t.draft_tokens, t.parents)
        assert r["accept_len"][b] == ref["accept_len"][0] and r["bonus"][b] == ref["bonus"][0]
        assert np.array_equal(r["path"][b, :n], ref["path"][0]) and (r["path"][b, n:] == -1).all()
        assert np.array_equal(r["target_argmax"][b, :n], ref["target_argmax"][0])
        assert (r["target_argmax"][b, n:] == -1).all()
    assert r["accept_len"].max() >= 3


@pytest.mark.parametrize("N,tree", [(12, "random"), (128, "dynamic")])
def test_sizes_stochastic_equals_truncated_trees(N, tree):
    over = dict(B=5, N=N, V=400, tree=tree, max_depth=8, mode="stochastic")
    if tree == "dynamic":
        over["topk"] = 5
    w = tvgen.make_workload(2, seed=900 + N, with_kv=False, overrides=over)
    sizes = sizes_for(N + 2, w.B, N)
    sizes[0] = N
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, 1.0,
                                 tree_sizes=sizes)
    for b in range(w.B):
        n = int(sizes[b])
        t = truncated(w, b, n)
        ref = oracle.accept_stochastic(t.target_logits, t.draft_logits, t.draft_tokens, t.parents, t.uniforms, 1.0)
        assert r["accept_len"][b] == ref["accept_len"][0] and r["bonus"][b] == ref["bonus"][0], b
        assert np.array_equal(r["path"][b, :n], ref["path"][0])


def test_long_chain_stochastic_p_equals_q():
    w = tvgen.make_workload(5, seed=950, with_kv=False, overrides=dict(B=4, N=128, V=300))
    w.draft_logits[:, 1:] = w.target_logits[:, :-1]
    r = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, 1.0)
    assert (r["accept_len"] == 128).all()


def test_sizes_status_codes():
    w = tvgen.make_workload(1, seed=960, with_kv=False, overrides=dict(B=2, N=10, V=50))
    for bad in ([0, 5], [11, 5], [-1, 5]):
        sz = np.array(bad, np.int32)
        assert oracle.status_build_mask(w.parents, tree_sizes=sz)[0] == oracle.INVALID_ARG
        assert oracle.status_accept_greedy(w.target_logits, w.draft_tokens, w.parents, w.B, w.N, w.V,
                                           tree_sizes=sz)[0] == oracle.INVALID_ARG
    # a bad parent inside the present nodes is still caught
    p = w.parents.copy()
    p[1, 3] = 7
    sz = np.array([10, 5], np.int32)
    assert oracle.status_build_mask(p, tree_sizes=sz)[0] == oracle.INVALID_TREE
    assert oracle.status_build_mask(p, tree_sizes=np.array([10, 3], np.int32))[0] == oracle.OK
