"""GPU parity: tv_build_tree (dynamic draft-tree construction) against the
oracle. Integer outputs and the fp64 scores (products of the same fp32
probabilities in the same order) must match bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, dev, host

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("parents", "tokens", "depth", "mask", "scores", "n_nodes")


def gpu_tree(roots, toks, probs, k_root, threshold, max_depth):
    out = tv.tv_build_tree(dev(roots), dev(toks), dev(probs), k_root, threshold, max_depth)
    r = {key: host(v) for key, v in out.items()}
    r["mask"] = r["mask"].view(np.uint64)
    return r


def compare(roots, toks, probs, what, k_root, threshold, max_depth, expect_error=0):
    print(f"[tree] {what}: B={toks.shape[0]} N={toks.shape[1]} k={toks.shape[2]} k_root={k_root} "
          f"threshold={threshold} depth<={max_depth}", flush=True)
    got = gpu_tree(roots, toks, probs, k_root, threshold, max_depth)
    assert tv.tv_device_error(DEV) == expect_error, what
    st, ref = oracle.status_build_tree(roots, toks, probs, k_root=k_root, threshold=threshold, max_depth=max_depth)
    assert st == (oracle.OK if expect_error == 0 else oracle.INVALID_ARG)
    for key in KEYS:
        g, r = got[key], ref[key]
        same = (g.view(np.uint64) == r.view(np.uint64)) if key == "scores" else (g == r)
        assert same.all(), f"{what}: {key} differs at {np.argwhere(~same)[:5].tolist()}"
    return ref


def generator_tables(seed, B, N, max_depth, topk, V):
    toks, probs = np.zeros((B, N, topk), np.int32), np.zeros((B, N, topk), np.float32)
    roots = np.zeros(B, np.int32)
    for b in range(B):
        rec = {}
        _, t = tvgen.dynamic_tree(seed, b, N, max_depth, topk, V, record=rec)
        roots[b] = t[0]
        for node, (tk, sc) in rec.items():
            if node < N:
                toks[b, node] = tk
                probs[b, node] = sc
    return roots, toks, probs


@pytest.mark.parametrize("cfg", [2, 3, 4])
@pytest.mark.parametrize("threshold", [0.0, 1e-3])
def test_build_tree_workload_shapes(cfg, threshold):
    c = tvgen.CONFIGS[cfg]
    roots, toks, probs = generator_tables(100 + cfg, c["B"], c["N"], c["max_depth"], c["topk"], c["V"])
    ref = compare(roots, toks, probs, f"cfg{cfg}", c["topk"], threshold, c["max_depth"])
    if threshold == 0.0:
        assert (ref["n_nodes"] == c["N"]).all()


def test_build_tree_page_parameters():
    # the page's reference code: top-4 at the root, top-3 below, threshold
    # 0.05, depth limit 6, budget 64
    B, N, k = 64, 64, 4
    probs = tvgen.uniform_f32(301, 1, (B, N, k))
    probs = (probs / probs.sum(-1, keepdims=True)).astype(np.float32)
    probs = -np.sort(-probs, -1)  # top-k proposals come in decreasing order
    toks = (tvgen.u64(301, 2, B * N * k) % 128256).astype(np.int32).reshape(B, N, k)
    ref = compare(np.arange(B, dtype=np.int32), toks, probs, "page-parameters", 4, 0.05, 6)
    assert (ref["n_nodes"] < N).any()  # the threshold cuts some trees short


@pytest.mark.parametrize("seed", range(3))
def test_build_tree_exact_ties(seed):
    # probabilities in eighths: many equal cumulative scores, so the
    # earliest-queued rule decides
    B, N, k = 200, 48, 5
    probs = (1 + tvgen.u64(400 + seed, 1, B * N * k) % 8).astype(np.float32).reshape(B, N, k) / 8
    toks = (tvgen.u64(400 + seed, 2, B * N * k) % 1000).astype(np.int32).reshape(B, N, k)
    compare(np.zeros(B, np.int32), toks, probs, f"ties-{seed}", 3, 0.0, 5 + seed)


def test_build_tree_fixture_and_edges():
    g = json.load(open(os.path.join(GOLD, "tree_build_hand.json")))
    got = gpu_tree(np.array(g["root_tokens"], np.int32), np.array(g["cand_tokens"], np.int32),
                   np.array(g["cand_probs"], np.float32), g["k_root"], g["threshold"], g["max_depth"])
    assert tv.tv_device_error(DEV) == 0
    for key, v in g["expect"].items():
        assert got[key].tolist() == v, key
    # budget 1, the largest k, a large batch, a threshold above every score
    rng_t = (tvgen.u64(5, 1, 3000 * 64 * 32) % 50000).astype(np.int32).reshape(3000, 64, 32)
    rng_p = tvgen.uniform_f32(5, 2, (3000, 64, 32))
    compare(np.arange(3000, dtype=np.int32), rng_t, rng_p, "k32-B3000", 32, 0.0, 8)
    compare(np.arange(7, dtype=np.int32), rng_t[:7, :1], rng_p[:7, :1], "N1", 1, 0.0, 3)
    ref = compare(np.arange(7, dtype=np.int32), rng_t[:7], rng_p[:7], "short", 3, 2.0, 8)
    assert (ref["n_nodes"] == 4).all()  # the root and its three proposals only


def test_build_tree_bad_probability():
    toks = np.zeros((3, 10, 4), np.int32)
    probs = np.full((3, 10, 4), 0.25, np.float32)
    probs[1, 7, 2] = np.nan
    probs[2, 0, 0] = -1.0
    compare(np.array([1, 2, 3], np.int32), toks, probs, "bad-probability", 2, 0.0, 4, expect_error=tv.INVALID_ARG)


def test_build_tree_host_errors_and_mask_consistency():
    roots, toks, probs = generator_tables(7, 4, 64, 6, 10, 1000)
    lib = tv.library()
    d_r, d_t, d_p = dev(roots), dev(toks), dev(probs)
    outs = [torch.empty((4, 64), dtype=torch.int32, device=DEV) for _ in range(2)]
    p = tv._ptr

    def call(N=64, k=10, k_root=10, thr=0.0, md=6, B=4):
        return lib.tv_build_tree(tv._ctx(DEV), p(d_r), p(d_t), p(d_p), B, N, k, k_root, thr, md, p(outs[0]),
                                 p(outs[1]), None, None, None, None)

    assert call(N=129) == tv.UNSUPPORTED
    assert call(k=33, k_root=3) == tv.UNSUPPORTED
    assert call(k_root=11) == tv.INVALID_ARG
    assert call(md=0) == tv.INVALID_ARG
    assert call(thr=float("nan")) == tv.INVALID_ARG
    assert call(N=0) == tv.INVALID_ARG
    assert call(B=0) == tv.OK
    assert call() == tv.OK
    torch.cuda.synchronize()
    assert tv.tv_device_error(DEV) == 0
    # the builder's masks are the masks tv_build_mask derives from its parents
    out = tv.tv_build_tree(d_r, d_t, d_p, 10, 0.0, 6)
    mask, depth = tv.tv_build_mask(out["parents"])
    assert torch.equal(mask, out["mask"]) and torch.equal(depth, out["depth"])
