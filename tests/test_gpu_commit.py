"""GPU parity: tv_commit (accepted-path KV commit and next-root insertion)
against the oracle.

Everything is integer or byte movement, so the bar is bit-exact: the whole
K and V pools after the commit, new prefix lengths, emitted tokens and next
roots. Paths come from the oracle's greedy acceptance on planted logits, or
from seeded root-to-node walks (inputs, not results of the HIP path).
"""
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


def walk_paths(parents, seed):
    """Seeded accepted paths: the root-to-node walk of a uniformly drawn node."""
    B, N = parents.shape
    s = tvgen.Stream(seed, 77)
    path = np.full((B, N), -1, np.int32)
    lens = np.zeros(B, np.int32)
    for b in range(B):
        c, p = s.randint(N), []
        while c >= 0:
            p.append(c)
            c = parents[b, c]
        if p[-1] != 0:  # forest node: only the root is accepted
            p = [0]
        p = p[::-1]
        path[b, :len(p)] = p
        lens[b] = len(p)
    bonus = np.array([s.randint(1 << 20) for _ in range(B)], np.int32)
    return path, lens, bonus


def run_commit(k_pages, v_pages, page_table, prefix_lens, max_prefix_len, draft_tokens, path, lens, bonus,
               want_emitted=True):
    k, v = dev(k_pages, torch.bfloat16), dev(v_pages, torch.bfloat16)
    out = tv.tv_commit(k, v, dev(page_table), dev(prefix_lens), max_prefix_len, dev(draft_tokens), dev(path),
                       dev(lens), dev(bonus), want_emitted=want_emitted)
    return k, v, out


def compare(w, path, lens, bonus, what, expect_error=0, prefix_lens=None, page_table=None):
    prefix_lens = w.prefix_lens if prefix_lens is None else prefix_lens
    page_table = w.page_table if page_table is None else page_table
    mpl = max(int(w.max_prefix_len), 0)
    print(f"[commit] {what} B={w.B} N={w.N} Hkv={w.Hkv} D={w.D} pages={w.num_pages}", flush=True)
    k, v, got = run_commit(w.k_pages, w.v_pages, page_table, prefix_lens, mpl, w.draft_tokens, path, lens, bonus)
    assert tv.tv_device_error(DEV) == expect_error, what
    st, k_ref, v_ref, ref = oracle.status_commit(w.k_pages, w.v_pages, page_table, prefix_lens, w.draft_tokens, path,
                                                 lens, bonus, B=w.B, N=w.N, Hkv=w.Hkv, D=w.D,
                                                 num_pages=w.num_pages, max_prefix_len=mpl)
    assert st == (oracle.OK if expect_error == 0 else oracle.INVALID_ARG)
    for key in ("new_prefix_lens", "emitted", "next_root"):
        g = host(got[key])
        assert (g == ref[key]).all(), f"{what}: {key} differs at {np.argwhere(g != ref[key])[:5].tolist()}"
    assert torch.equal(k.view(torch.int16), dev(k_ref).view(torch.int16)), f"{what}: K pool differs"
    assert torch.equal(v.view(torch.int16), dev(v_ref).view(torch.int16)), f"{what}: V pool differs"
    moved = int(((path >= 0) & (path != np.arange(w.N)[None, :])).sum())
    return moved


@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_commit_full_size(cfg):
    w = tvgen.make_workload(cfg)
    if w.mode == "greedy":
        tvgen.plant_random(w, 0.7, seed=cfg)
        acc = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
        path, lens, bonus = acc["path"], acc["accept_len"], acc["bonus"]
    else:
        path, lens, bonus = walk_paths(w.parents, cfg)
    moved = compare(w, path, lens, bonus, f"cfg{cfg}")
    # cfg1's one accepted path and every chain path are identity prefixes
    assert moved > 0 or cfg in (1, 5)


@pytest.mark.parametrize("cfg", [2, 3])
def test_commit_walk_paths(cfg):
    # random root-to-node walks: every depth, deep dynamic-tree paths (cfg3's
    # KV pool is reduced to short prefixes to keep the host side quick)
    ov = dict(L=(0, 300)) if cfg == 3 else None
    w = tvgen.make_workload(cfg, seed=2000 + cfg, with_logits=False, overrides=ov)
    path, lens, bonus = walk_paths(w.parents, 10 + cfg)
    compare(w, path, lens, bonus, f"walk-cfg{cfg}")


def test_commit_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLD, "commit_hand.json")))
    D, Hkv, P = g["D"], g["Hkv"], g["num_pages"]
    rng = tvgen.u64(31, 1, 2 * P * Hkv * 16 * D).astype(np.uint16).reshape(2, P, Hkv, 16, D)
    table = np.array(g["page_table"], np.int32)
    lens = np.array(g["prefix_lens"], np.int32)
    k, v, got = run_commit(rng[0], rng[1], table, lens, int(lens.max()), np.array(g["draft_tokens"], np.int32),
                           np.array(g["path"], np.int32), np.array(g["accept_len"], np.int32),
                           np.array(g["bonus"], np.int32))
    assert tv.tv_device_error(DEV) == 0
    for key in ("new_prefix_lens", "emitted", "next_root"):
        assert host(got[key]).tolist() == g["expect"][key], key
    kh, vh = host(k.view(torch.int16)).view(np.uint16), host(v.view(torch.int16)).view(np.uint16)
    N = len(g["parents"][0])
    for b in range(len(lens)):
        moved = dict((d, s) for d, s in g["expect"]["moved_rows"][str(b)])
        for t in range(lens[b] + N):
            s = moved.get(t, t)
            pd, ps = table[b, t // 16], table[b, s // 16]
            assert np.array_equal(kh[pd, :, t % 16], rng[0][ps, :, s % 16]), (b, t)
            assert np.array_equal(vh[pd, :, t % 16], rng[1][ps, :, s % 16]), (b, t)


@pytest.mark.parametrize("D", [64, 128])
def test_commit_largest_move(D):
    # N = 64 and path 0, 2, 3, ..., 63: 62 rows move, the most a 64-node tree
    # allows; prefixes put the tree across page boundaries
    w = tvgen.make_workload(2, seed=3100 + D, with_logits=False,
                            overrides=dict(B=5, N=64, D=D, Hkv=2, Hq=4, L=(0, 40), tree="chain"))
    path = np.tile(np.concatenate([[0], np.arange(2, 64)]).astype(np.int32), (w.B, 1))
    path = np.concatenate([path, np.full((w.B, 1), -1, np.int32)], 1)
    lens = np.full(w.B, 63, np.int32)
    moved = compare(w, path, lens, np.arange(w.B, dtype=np.int32), f"largest-D{D}")
    assert moved == 62 * w.B


def test_commit_root_only_and_full_chain():
    w = tvgen.make_workload(5, seed=3200, with_logits=False, overrides=dict(B=6, L=(0, 70)))
    path = np.tile(np.arange(w.N, dtype=np.int32), (w.B, 1))
    lens = np.array([1, w.N, 1, w.N, 2, 3], np.int32)
    for b in range(w.B):
        path[b, lens[b]:] = -1
    assert compare(w, path, lens, np.arange(w.B, dtype=np.int32) + 7, "identity") == 0


def test_commit_without_emitted_and_empty_batch():
    w = tvgen.make_workload(1, seed=3300, with_logits=False)
    path, lens, bonus = walk_paths(w.parents, 3)
    k, v, got = run_commit(w.k_pages, w.v_pages, w.page_table, w.prefix_lens, w.max_prefix_len, w.draft_tokens,
                           path, lens, bonus, want_emitted=False)
    assert tv.tv_device_error(DEV) == 0
    _, k_ref, _, ref = oracle.status_commit(w.k_pages, w.v_pages, w.page_table, w.prefix_lens, w.draft_tokens, path,
                                            lens, bonus, B=w.B, N=w.N, Hkv=w.Hkv, D=w.D, num_pages=w.num_pages)
    assert "emitted" not in got
    assert (host(got["new_prefix_lens"]) == ref["new_prefix_lens"]).all()
    assert torch.equal(k.view(torch.int16), dev(k_ref).view(torch.int16))
    e = torch.empty((0, w.N), dtype=torch.int32, device=DEV)
    z = torch.empty(0, dtype=torch.int32, device=DEV)
    out = tv.tv_commit(k, v, dev(w.page_table), z, 0, e, e, z, z)
    assert out["new_prefix_lens"].numel() == 0


@pytest.mark.parametrize("bad", ["len0", "len_big", "root", "order", "node_big", "bonus", "page", "page_big",
                                 "prefix_neg", "prefix_over_max"])
def test_commit_bad_sequence(bad):
    w = tvgen.make_workload(2, seed=3400, with_logits=False, overrides=dict(B=3, N=8, L=(20, 60), tree="chain"))
    path = np.full((w.B, w.N), -1, np.int32)
    path[:, :4] = [0, 2, 5, 7]
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
    elif bad == "prefix_neg":
        prefix[b] = -1
    elif bad == "prefix_over_max":
        prefix[b] = w.max_prefix_len + 1
    compare(w, path, lens, bonus, f"bad-{bad}", expect_error=tv.INVALID_ARG, prefix_lens=prefix, page_table=table)


def test_commit_host_errors():
    w = tvgen.make_workload(1, seed=3500, with_logits=False)
    path, lens, bonus = walk_paths(w.parents, 4)
    k, v = dev(w.k_pages, torch.bfloat16), dev(w.v_pages, torch.bfloat16)
    lib = tv.library()
    args = [dev(a) for a in (w.page_table, w.prefix_lens, w.draft_tokens, path, lens, bonus)]
    outs = [torch.empty(w.B, dtype=torch.int32, device=DEV), torch.empty((w.B, w.N), dtype=torch.int32, device=DEV),
            torch.empty(w.B, dtype=torch.int32, device=DEV)]
    p = tv._ptr
    ctx = tv._ctx(DEV)

    def call(B=w.B, N=w.N, Hkv=w.Hkv, D=w.D, maxp=w.maxp, mpl=w.max_prefix_len):
        return lib.tv_commit(ctx, p(k), p(v), w.num_pages, p(args[0]), maxp, p(args[1]), mpl, p(args[2]),
                             p(args[3]), p(args[4]), p(args[5]), B, N, Hkv, D, p(outs[0]), p(outs[1]), p(outs[2]))

    assert call(D=96) == tv.UNSUPPORTED
    assert call(N=129) == tv.UNSUPPORTED
    assert call(N=0) == tv.INVALID_ARG
    assert call(Hkv=0) == tv.INVALID_ARG
    assert call(maxp=0) == tv.INVALID_ARG
    assert call(mpl=w.maxp * 16) == tv.INVALID_ARG
    torch.cuda.synchronize()
    assert tv.tv_device_error(DEV) == 0
    assert torch.equal(k.view(torch.int16), dev(w.k_pages).view(torch.int16))


def test_commit_pool_above_2gib():
    # the touched pages sit above byte offset 2 GiB of a pool of 66000 pages
    small = tvgen.make_workload(2, seed=3600, with_logits=False, overrides=dict(B=4, L=(30, 200)))
    path, lens, bonus = walk_paths(small.parents, 5)
    _, k_ref, v_ref, ref = oracle.status_commit(small.k_pages, small.v_pages, small.page_table, small.prefix_lens,
                                                small.draft_tokens, path, lens, bonus, B=small.B, N=small.N,
                                                Hkv=small.Hkv, D=small.D, num_pages=small.num_pages)
    P_big = 66000
    base = P_big - small.num_pages
    print(f"[commit] pool-above-2GiB P={P_big} base={base}", flush=True)
    shape = (P_big, small.Hkv, 16, small.D)
    k = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
    assert base * small.Hkv * 16 * small.D * 2 > 2 ** 31
    k[base:] = dev(small.k_pages, torch.bfloat16)
    v[base:] = dev(small.v_pages, torch.bfloat16)
    table = np.where(small.page_table >= 0, small.page_table + base, -1).astype(np.int32)
    out = tv.tv_commit(k, v, dev(table), dev(small.prefix_lens), small.max_prefix_len, dev(small.draft_tokens),
                       dev(path), dev(lens), dev(bonus))
    assert tv.tv_device_error(DEV) == 0
    for key in ("new_prefix_lens", "emitted", "next_root"):
        assert (host(out[key]) == ref[key]).all(), key
    assert torch.equal(k[base:].view(torch.int16), dev(k_ref).view(torch.int16))
    assert torch.equal(v[base:].view(torch.int16), dev(v_ref).view(torch.int16))
    assert not k[:base].view(torch.int16).any()
    del k, v
    torch.cuda.empty_cache()
