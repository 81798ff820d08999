"""GPU parity on seeded random shapes: tv_attention compared in full with the
fp64 oracle, over combinations the fixed cases do not pair up (head dim 64 or
128, KV heads 1-4, GQA group 1-8, 1-128 tree nodes, prefix ranges from empty
to about 1,600 keys, random / chain / star / forest trees, batch 1-4), each
with and without per-sequence node counts; greedy acceptance, bit-exact, over
random batch, 1-128 nodes, vocabulary size and planted matches (so both the
one-launch and the two-pass form); and sampled acceptance, bit-exact
against the oracle, over random batch, node count, vocabulary size (and so
the number of workgroups per sequence), tree kind and temperature.

The shapes come from a fixed seed, so every run checks the same cases; a
failure message names the shape.
"""
import numpy as np
import pytest

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, DevWorkload, check_attention, dev, greedy_compare, host, stochastic_compare

pytestmark = pytest.mark.gpu

NCASES = 24


def shape(i):
    r = np.random.default_rng(4200 + i)
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    lo = int(r.integers(0, 1200))
    return dict(B=int(r.integers(1, 5)), Hq=Hkv * G, Hkv=Hkv, D=int(r.choice([64, 128])),
                L=(lo, lo + int(r.integers(0, 400))), N=int(r.integers(1, 129)),
                tree=str(r.choice(["random", "chain", "star", "forest"])), max_depth=int(r.integers(1, 10)),
                pages="permuted")


@pytest.mark.parametrize("sized", [False, True], ids=["all-nodes", "node-counts"])
@pytest.mark.parametrize("i", range(NCASES))
def test_attention_random_shape(i, sized):
    sh = shape(i)
    w = tvgen.make_workload(1, seed=5000 + i, with_logits=False, overrides=sh)
    sizes = None
    if sized:  # each sequence's node count, uniform in [1, N]
        sizes = np.random.default_rng(6000 + i).integers(1, w.N + 1, size=w.B).astype(np.int32)
    what = (f"case {i}: B{w.B} Hq{w.Hq}/Hkv{w.Hkv} D{w.D} N{w.N} tree={sh['tree']} "
            f"prefix lengths {w.prefix_lens.tolist()} node counts {None if sizes is None else sizes.tolist()}")
    print(f"[random shapes] {what}", flush=True)
    dw = DevWorkload(w, logits=False)
    mask, _ = tv.tv_build_mask(dw.parents, tree_sizes=None if sizes is None else dev(sizes))
    out = host(tv.tv_attention(dw.q, dw.k, dw.v, dw.page_table, dw.prefix_lens, w.max_prefix_len, mask,
                               float(w.sm_scale), tree_sizes=None if sizes is None else dev(sizes)))
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.attention(w, oracle.build_mask(w.parents, tree_sizes=sizes)[0], tree_sizes=sizes)
    if sizes is None:
        check_attention(out, ref, what=what)
    else:  # only present nodes have outputs
        for b in range(w.B):
            n = int(sizes[b])
            check_attention(out[b, :n], ref[b, :n], what=f"{what}, sequence {b}")


def stochastic_shape(i):
    r = np.random.default_rng(7300 + i)
    tree = str(r.choice(["random", "dynamic", "star", "chain", "forest"]))
    sh = dict(B=int(r.integers(1, 41)), N=int(r.integers(2, 65)), V=int(r.integers(500, 70001)), tree=tree,
              mode="stochastic", T=float(r.choice([0.6, 1.0, 1.7])))
    if tree in ("random", "dynamic"):
        sh.update(max_depth=int(r.integers(2, 9)), topk=int(r.integers(2, 11)))
    if tree == "dynamic":  # at most the nodes a tree of this depth and top-k holds
        sh["N"] = min(sh["N"], sum(sh["topk"] ** e for e in range(sh["max_depth"] + 1)))
    return sh


@pytest.mark.parametrize("i", range(16))
def test_stochastic_random_shape(i):
    sh = stochastic_shape(i)
    w = tvgen.make_workload(2, seed=8000 + i, with_kv=False, overrides=sh)
    # draft rows near their parent's target row for every other sequence
    # (long accepted paths), the others drawn apart (many rejected siblings)
    near = tvgen.normal_f32(8000 + i, 95, w.draft_logits.shape, sigma=0.3)
    for b in range(0, w.B, 2):
        for c in range(1, w.N):
            pr = w.parents[b, c]
            if pr >= 0:
                w.draft_logits[b, c] = w.target_logits[b, pr] + near[b, c]
    stochastic_compare(w, f"case {i}: {sh}")


@pytest.mark.parametrize("i", range(16))
def test_greedy_random_shape(i):
    r = np.random.default_rng(9100 + i)
    tree = str(r.choice(["random", "star", "chain", "forest"]))
    if i % 2 == 0:  # at most 256 workgroups (B * N <= 128, V <= 32768): the one-launch form
        N = int(r.integers(1, 65))
        B = int(r.integers(1, 128 // N + 1))
        V = int(r.integers(2, 32769))
    else:  # the argmax pass and the path pass, at most 120 MB of logits
        B, N = int(r.integers(1, 65)), int(r.integers(1, 129))
        V = min(int(r.integers(2, 200001)), max(2, 30_000_000 // (B * N)))
    sh = dict(B=B, N=N, V=V, tree=tree, max_depth=int(r.integers(1, 10)))
    w = tvgen.make_workload(1, seed=9000 + i, with_kv=False, overrides=sh)
    tvgen.plant_random(w, float(r.choice([0.0, 0.5, 0.9])), seed=9000 + i)
    greedy_compare(w, f"case {i}: {sh}")
