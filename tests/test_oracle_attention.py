"""Pins for the oracle's tree-masked paged attention (O2).

None of these re-derive the oracle's loop. They reduce special trees to a
library routine (torch's scaled_dot_product_attention in float64, whose
enable_gqa grouping is the contiguous-group reading), or use closed forms and
invariances:
  chain tree  == causal attention over [prefix | tree]
  forest      == independent single-token decodes over prefix + self
  star        == decodes over prefix + root + self
  tiny trees  == per-row attention over an explicitly walked key list
  constant V, L = 0 / N = 1, all-visible == dense attention,
  page-table permutation, non-ancestor perturbation, topological relabelling.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import tvgen


def small(tree, *, B=2, Hq=4, Hkv=2, D=64, L=(0, 50), N=12, seed=5, pages="permuted", max_depth=4):
    return tvgen.make_workload(1, seed=seed, with_logits=False,
                               overrides=dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, N=N, tree=tree, pages=pages,
                                              max_depth=max_depth))


def seq_kv(w, b):
    """Gather sequence b's K/V as [Hkv][T][D] float64 (T = L_b + N)."""
    T = int(w.prefix_lens[b]) + w.N
    t = np.arange(T)
    pages = w.page_table[b, t // 16]
    k = tvgen.bf16_to_f32(w.k_pages[pages, :, t % 16, :])  # [T][Hkv][D]
    v = tvgen.bf16_to_f32(w.v_pages[pages, :, t % 16, :])
    return (torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2),
            torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2))


def seq_q(w, b):
    return torch.from_numpy(tvgen.bf16_to_f32(w.q[b]).astype(np.float64)).permute(1, 0, 2)  # [Hq][N][D]


def sdpa(q, k, v, scale, mask=None):
    return F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask, scale=float(scale),
                                          enable_gqa=True)[0]


def run_oracle(w, parents=None):
    mask, _ = oracle.build_mask(w.parents if parents is None else parents)
    return oracle.attention(w, mask)  # [B][N][Hq][D]


def test_chain_equals_causal_attention():
    w = small("chain", N=16, L=(0, 70))
    out = run_oracle(w)
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        k, v = seq_kv(w, b)
        causal = torch.ones(w.N, L + w.N, dtype=torch.bool).tril(diagonal=L)
        ref = sdpa(seq_q(w, b), k, v, w.sm_scale, causal)  # [Hq][N][D]
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_forest_equals_independent_decodes():
    w = small("forest", N=10, L=(1, 40))
    out = run_oracle(w)
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        k, v = seq_kv(w, b)
        q = seq_q(w, b)
        for i in range(w.N):
            keys = list(range(L)) + [L + i]
            ref = sdpa(q[:, i:i + 1], k[:, keys], v[:, keys], w.sm_scale)
            np.testing.assert_allclose(out[b, i], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_star_equals_decodes_over_prefix_and_root():
    w = small("star", N=9, L=(0, 33))
    out = run_oracle(w)
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        k, v = seq_kv(w, b)
        q = seq_q(w, b)
        for i in range(w.N):
            keys = list(range(L)) + sorted({L, L + i})
            ref = sdpa(q[:, i:i + 1], k[:, keys], v[:, keys], w.sm_scale)
            np.testing.assert_allclose(out[b, i], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def ancestors(parents, i):
    out = []
    while i >= 0:
        out.append(i)
        i = parents[i]
    return out


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_tiny_trees(seed):
    N = 3 + seed
    w = small("random", N=N, L=(0, 24), seed=100 + seed, Hq=6, Hkv=3, max_depth=3)
    out = run_oracle(w)
    for b in range(w.B):
        L = int(w.prefix_lens[b])
        k, v = seq_kv(w, b)
        q = seq_q(w, b)
        for i in range(N):
            keys = list(range(L)) + sorted(L + j for j in ancestors(w.parents[b], i))
            ref = sdpa(q[:, i:i + 1], k[:, keys], v[:, keys], w.sm_scale)
            np.testing.assert_allclose(out[b, i], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_all_visible_equals_dense_attention():
    w = small("random", N=13, L=(5, 40), D=128, Hq=8, Hkv=2)
    out = oracle.attention(w, None)
    for b in range(w.B):
        k, v = seq_kv(w, b)
        ref = sdpa(seq_q(w, b), k, v, w.sm_scale)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_constant_values_closed_form():
    w = small("random", N=11, L=(0, 60))
    w.v_pages[:] = 0x3EC0  # bf16 0.375
    out = run_oracle(w)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-14)


def test_single_key_returns_v0():
    w = small("chain", N=1, L=0, B=3)
    out = run_oracle(w)
    for b in range(w.B):
        _, v = seq_kv(w, b)
        G = w.Hq // w.Hkv
        for h in range(w.Hq):
            np.testing.assert_array_equal(out[b, 0, h], v[h // G, 0].numpy())


def test_page_permutation_invariance():
    w = small("random", N=14, L=(20, 90), seed=9)
    ref = run_oracle(w)
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.num_pages).astype(np.int32)
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    k2[perm] = w.k_pages
    v2[perm] = w.v_pages
    w.k_pages, w.v_pages = k2, v2
    w.page_table = np.where(w.page_table >= 0, perm[np.maximum(w.page_table, 0)], -1).astype(np.int32)
    np.testing.assert_array_equal(run_oracle(w), ref)


def test_non_ancestor_perturbation_changes_nothing():
    w = small("random", N=12, L=(3, 30), seed=21)
    mask, _ = oracle.build_mask(w.parents)
    ref = oracle.attention(w, mask)
    for b in range(w.B):
        for i in range(w.N):
            w2 = small("random", N=12, L=(3, 30), seed=21)
            anc = set(ancestors(w2.parents[b], i))
            L = int(w2.prefix_lens[b])
            for j in range(w2.N):
                if j in anc:
                    continue
                t = L + j
                p = w2.page_table[b, t // 16]
                w2.k_pages[p, :, t % 16, :] = 0x4120  # bf16 10.0
                w2.v_pages[p, :, t % 16, :] = 0xC120  # bf16 -10.0
            out = oracle.attention(w2, mask, rows=np.array([[b, i, h] for h in range(w2.Hq)], np.int32))
            np.testing.assert_array_equal(out, ref[b, i])


def test_topological_relabelling_permutes_rows():
    w = small("random", N=10, L=(4, 20), seed=31, B=1)
    ref = run_oracle(w)
    par = w.parents[0]
    # new order: visit nodes by (depth, old id) - a different topological order
    depth = tvgen.tree_depths(par)
    order = sorted(range(w.N), key=lambda j: (depth[j], -j if j else -99))
    new_of = {old: new for new, old in enumerate(order)}
    new_par = np.array([-1 if par[o] < 0 else new_of[par[o]] for o in order], np.int32)
    assert all(new_par[i] < i for i in range(w.N))
    w.parents = new_par[None]
    w.q = w.q[:, order].copy()
    L = int(w.prefix_lens[0])
    k_old, v_old = w.k_pages.copy(), w.v_pages.copy()
    for new, old in enumerate(order):
        tn, to = L + new, L + old
        pn, po = w.page_table[0, tn // 16], w.page_table[0, to // 16]
        w.k_pages[pn, :, tn % 16] = k_old[po, :, to % 16]
        w.v_pages[pn, :, tn % 16] = v_old[po, :, to % 16]
    out = run_oracle(w)
    np.testing.assert_allclose(out[0], ref[0, order], rtol=0, atol=1e-13)


def test_status_codes():
    w = small("random", N=8, L=(20, 40))
    mask, _ = oracle.build_mask(w.parents)
    kw = dict(B=w.B, N=w.N, Hq=w.Hq, Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale)
    args = (w.q, w.k_pages, w.v_pages, w.page_table, w.prefix_lens, mask)
    assert oracle.status_attention(*args, **kw)[0] == oracle.OK
    assert oracle.status_attention(*args, **{**kw, "Hkv": 3})[0] == oracle.INVALID_ARG
    assert oracle.status_attention(*args, **{**kw, "D": 96})[0] == oracle.UNSUPPORTED
    assert oracle.status_attention(*args, **{**kw, "N": 129})[0] == oracle.UNSUPPORTED
    assert oracle.status_attention(*args, **kw, maxp=1)[0] == oracle.INVALID_ARG
    bad = w.page_table.copy()
    bad[0, 0] = w.num_pages
    assert oracle.status_attention(w.q, w.k_pages, w.v_pages, bad, w.prefix_lens, mask, **kw)[0] == \
        oracle.INVALID_ARG
    pl = w.prefix_lens.copy()
    pl[0] = -1
    assert oracle.status_attention(w.q, w.k_pages, w.v_pages, w.page_table, pl, mask, **kw,
                                   max_prefix_len=int(w.prefix_lens.max()))[0] == oracle.INVALID_ARG
    assert oracle.status_attention(*args, **{**kw, "B": 0})[0] == oracle.OK
