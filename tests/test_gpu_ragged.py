"""GPU parity for trees of more than 64 nodes (up to 128: two mask words per
row) and for per-sequence node counts (tree_sizes), against the oracle.

Integer outputs bit-exact; attention within the usual tolerance; rows of
absent nodes must be left exactly as they were."""
import numpy as np
import pytest
import torch

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, TIGHT, check_attention, dev, host, mask_np

pytestmark = pytest.mark.gpu


def sizes_for(seed, B, N, full_first=True):
    s = tvgen.Stream(seed, 3)
    sz = np.array([1 + s.randint(N) for _ in range(B)], np.int32)
    if full_first:
        sz[0] = N
    return sz


def workload(N, tree="random", seed=1, **over):
    o = dict(B=4, Hq=8, Hkv=2, D=128, L=(100, 700), N=N, tree=tree, V=500, max_depth=9, topk=6)
    o.update(over)
    return tvgen.make_workload(2, seed=seed, overrides=o)


@pytest.mark.parametrize("N,tree", [(65, "random"), (100, "random"), (128, "dynamic"), (128, "chain")])
@pytest.mark.parametrize("sized", [False, True])
def test_mask_long_trees(N, tree, sized):
    w = tvgen.make_workload(1, seed=N, with_kv=False, with_logits=False,
                            overrides=dict(B=40, N=N, tree=tree, max_depth=9, topk=6, V=500))
    sizes = sizes_for(N, w.B, N) if sized else None
    print(f"[ragged] mask N={N} {tree} sized={sized}", flush=True)
    mask, depth = tv.tv_build_mask(dev(w.parents), tree_sizes=dev(sizes) if sized else None)
    assert tv.tv_device_error(DEV) == 0
    ref_m, ref_d = oracle.build_mask(w.parents, tree_sizes=sizes)
    assert np.array_equal(mask_np(mask), ref_m)
    assert np.array_equal(host(depth), ref_d)


def run_attention(w, mask_np_, sizes, sentinel=12345.0, expect_error=0):
    out = torch.full((w.B, w.N, w.Hq, w.D), sentinel, dtype=torch.float32, device=DEV)
    tv.tv_attention(dev(w.q, torch.bfloat16), dev(w.k_pages, torch.bfloat16), dev(w.v_pages, torch.bfloat16),
                    dev(w.page_table), dev(w.prefix_lens), w.max_prefix_len,
                    dev(mask_np_.view(np.int64)) if mask_np_ is not None else None, float(w.sm_scale), out=out,
                    tree_sizes=dev(sizes) if sizes is not None else None)
    assert tv.tv_device_error(DEV) == expect_error
    return host(out)


@pytest.mark.parametrize("N,tree,D,sized", [(128, "dynamic", 128, False), (128, "dynamic", 128, True),
                                            (100, "random", 64, True), (70, "chain", 128, True),
                                            (128, "dynamic", 128, "nomask")])
def test_attention_long_trees(N, tree, D, sized):
    w = workload(N, tree, seed=200 + N + D, D=D, B=3, L=(30, 400))
    sizes = sizes_for(N + 1, w.B, N) if sized else None
    print(f"[ragged] attention N={N} {tree} D={D} sized={sized}", flush=True)
    mask, _ = oracle.build_mask(w.parents, tree_sizes=sizes)
    got = run_attention(w, None if sized == "nomask" else mask, sizes)
    ref = oracle.attention(w, None if sized == "nomask" else mask, tree_sizes=sizes)
    for b in range(w.B):
        n = N if sizes is None else int(sizes[b])
        check_attention(got[b, :n], ref[b, :n], tight=TIGHT, what=f"b{b}")
        assert (got[b, n:] == 12345.0).all(), f"b{b}: an absent row was written"


def full_compare_present(w, mask, sizes, what):
    # every present row against the fp64 oracle; absent rows keep the sentinel
    got = run_attention(w, mask, sizes)
    ref = oracle.attention(w, mask, tree_sizes=sizes)
    for b in range(w.B):
        n = int(sizes[b])
        check_attention(got[b, :n], ref[b, :n], tight=TIGHT, what=f"{what} b{b}")
        assert (got[b, n:] == 12345.0).all(), f"{what} b{b}: an absent row was written"


def test_attention_128_node_trees_at_layer_shape():
    # the Llama-3-8B layer shape with 128-node EAGLE-2 trees and node counts;
    # every present row
    w = tvgen.make_workload(2, seed=333, with_logits=False, overrides=dict(N=128))
    sizes = sizes_for(334, w.B, 128)
    print(f"[ragged] attention cfg2 shape N=128 sizes={sizes.tolist()}", flush=True)
    mask, _ = oracle.build_mask(w.parents, tree_sizes=sizes)
    full_compare_present(w, mask, sizes, "cfg2-N128")


@pytest.mark.parametrize("cfg", [3, 4])
def test_attention_128_node_trees_at_long_shapes(cfg):
    # the Llama-3.1-70B layer shape and the 32K context with 128-node trees
    # and node counts; every present row
    w = tvgen.make_workload(cfg, seed=340 + cfg, with_logits=False, overrides=dict(N=128))
    sizes = sizes_for(341 + cfg, w.B, 128)
    print(f"[ragged] attention cfg{cfg} shape N=128 sizes={sizes.tolist()}", flush=True)
    mask, _ = oracle.build_mask(w.parents, tree_sizes=sizes)
    full_compare_present(w, mask, sizes, f"cfg{cfg}-N128")


@pytest.mark.parametrize("N,sized", [(128, False), (128, True), (90, True)])
def test_greedy_long_trees(N, sized):
    w = tvgen.make_workload(2, seed=400 + N, with_kv=False,
                            overrides=dict(B=24, N=N, V=3000, tree="random", max_depth=12))
    depths = np.stack([tvgen.tree_depths(p) for p in w.parents])
    sizes = sizes_for(N + 7, w.B, N) if sized else None
    for b in range(w.B):
        n = N if sizes is None else int(sizes[b])
        tvgen.plant_full_path(w, b, int(np.argmax(depths[b, :n])))  # the deepest present node
        if sized:  # absent nodes may hold anything
            w.parents[b, n:] = 9999
            w.draft_tokens[b, n:] = -3
            w.target_logits[b, n:] = np.nan
    print(f"[ragged] greedy N={N} sized={sized}", flush=True)
    got = tv.tv_accept(dev(w.target_logits), dev(w.draft_tokens), dev(w.parents),
                       tree_sizes=dev(sizes) if sized else None)
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents, tree_sizes=sizes)
    for k in ("accept_len", "path", "bonus", "target_argmax"):
        assert (host(got[k]) == ref[k]).all(), k
    assert ref["accept_len"].max() >= 8


@pytest.mark.parametrize("N,sized", [(128, True), (128, False)])
def test_stochastic_long_trees(N, sized):
    w = tvgen.make_workload(2, seed=500 + N + sized, with_kv=False,
                            overrides=dict(B=12, N=N, V=4000, tree="dynamic", max_depth=8, topk=5,
                                           mode="stochastic"))
    near = tvgen.normal_f32(501, 9, w.draft_logits.shape, sigma=0.3)
    for b in range(w.B):  # draft rows near the target rows: long accepted paths
        for c in range(1, N):
            w.draft_logits[b, c] = w.target_logits[b, w.parents[b, c]] + near[b, c]
    sizes = sizes_for(N + 9, w.B, N) if sized else None
    print(f"[ragged] stochastic N={N} sized={sized}", flush=True)
    got = tv.tv_accept(dev(w.target_logits), dev(w.draft_tokens), dev(w.parents), mode=tv.STOCHASTIC,
                       draft_logits=dev(w.draft_logits), uniforms=dev(w.uniforms), temperature=1.0,
                       tree_sizes=dev(sizes) if sized else None)
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, 1.0,
                                   tree_sizes=sizes)
    near_tie = (ref["margins"] <= 1e-9).any(1)
    assert near_tie.mean() < 0.1
    for k in ("accept_len", "path", "bonus"):
        assert (host(got[k])[~near_tie] == ref[k][~near_tie]).all(), k


@pytest.mark.parametrize("D", [64, 128])
def test_commit_127_node_path(D):
    w = tvgen.make_workload(2, seed=600 + D, with_logits=False,
                            overrides=dict(B=3, N=128, D=D, Hkv=2, Hq=4, L=(0, 40), tree="chain"))
    path = np.tile(np.concatenate([[0], np.arange(2, 128)]).astype(np.int32), (w.B, 1))
    path = np.concatenate([path, np.full((w.B, 1), -1, np.int32)], 1)
    lens = np.full(w.B, 127, np.int32)
    bonus = np.arange(w.B, dtype=np.int32)
    k, v = dev(w.k_pages, torch.bfloat16), dev(w.v_pages, torch.bfloat16)
    got = tv.tv_commit(k, v, dev(w.page_table), dev(w.prefix_lens), w.max_prefix_len, dev(w.draft_tokens),
                       dev(path), dev(lens), dev(bonus))
    assert tv.tv_device_error(DEV) == 0
    k_ref, v_ref, ref = oracle.commit(w, path, lens, bonus)
    for key in ("new_prefix_lens", "emitted", "next_root"):
        assert (host(got[key]) == ref[key]).all(), key
    assert torch.equal(k.view(torch.int16), dev(k_ref).view(torch.int16))
    assert torch.equal(v.view(torch.int16), dev(v_ref).view(torch.int16))


@pytest.mark.parametrize("threshold", [0.0, 1e-4])
def test_build_tree_128_nodes(threshold):
    B, N, k, depth = 16, 128, 10, 8
    toks, probs = np.zeros((B, N, k), np.int32), np.zeros((B, N, k), np.float32)
    roots = np.zeros(B, np.int32)
    for b in range(B):
        rec = {}
        _, t = tvgen.dynamic_tree(700, b, N, depth, k, 128256, record=rec)
        roots[b] = t[0]
        for node, (tk, sc) in rec.items():
            if node < N:
                toks[b, node], probs[b, node] = tk, sc
    out = tv.tv_build_tree(dev(roots), dev(toks), dev(probs), k, threshold, depth)
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.build_tree(roots, toks, probs, k_root=k, threshold=threshold, max_depth=depth)
    for key in ("parents", "tokens", "depth", "n_nodes"):
        assert (host(out[key]) == ref[key]).all(), key
    assert (host(out["mask"]).view(np.uint64) == ref["mask"]).all()
    assert (host(out["scores"]).view(np.uint64) == ref["scores"].view(np.uint64)).all()


def test_bad_sizes():
    w = workload(20, seed=800, B=3)
    bad = np.array([20, 0, 21], np.int32)
    mask, depth = tv.tv_build_mask(dev(w.parents), tree_sizes=dev(bad))
    assert tv.tv_device_error(DEV) == tv.INVALID_ARG
    assert (host(depth)[1:] == -1).all() and (mask_np(mask)[1:] == 0).all()
    m, _ = oracle.build_mask(w.parents)
    got = run_attention(w, m, bad, expect_error=tv.INVALID_ARG)
    assert np.isnan(got[1:]).all() and np.isfinite(got[0]).all()
    r = tv.tv_accept(dev(w.target_logits), dev(w.draft_tokens), dev(w.parents), tree_sizes=dev(bad))
    assert tv.tv_device_error(DEV) == tv.INVALID_ARG
    assert host(r["accept_len"]).tolist()[1:] == [-1, -1] and host(r["accept_len"])[0] >= 1
