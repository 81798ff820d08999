"""GPU: several draft/verify cycles in a row through the whole library.

Each cycle builds the dynamic tree from the draft head's proposals
(tv_build_tree), writes the tree nodes' K/V into the paged cache, runs
tv_build_mask, tv_attention and tv_accept (greedy, or sampled with uniforms
passed in), and commits the accepted path (tv_commit). The next cycle starts from what the commit left on the
device: the compacted cache, the grown prefix lengths and the next root
token. Every step is compared with the oracle run on the same state: trees,
masks, acceptance, committed pools and commit outputs bit-exact, attention
within the usual tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, TIGHT, check_attention, dev, host, mask_np

pytestmark = pytest.mark.gpu


def proposals(seed, B, N, depth, k, V):
    """The draft head's proposal rows (by creation order) of generator trees."""
    toks, probs = np.zeros((B, N, k), np.int32), np.zeros((B, N, k), np.float32)
    roots = np.zeros(B, np.int32)
    for b in range(B):
        rec = {}
        _, t = tvgen.dynamic_tree(seed, b, N, depth, k, V, record=rec)
        roots[b] = t[0]
        for node, (tk, sc) in rec.items():
            if node < N:
                toks[b, node], probs[b, node] = tk, sc
    return roots, toks, probs


@pytest.mark.parametrize("D,mode", [(64, "greedy"), (128, "greedy"), (128, "stochastic")])
def test_draft_verify_cycles(D, mode):
    B, N, Hq, Hkv, V, k, depth, cycles = 3, 24, 8, 2, 600, 4, 5, 3
    w = tvgen.make_workload(2, seed=4242 + D, with_kv=False, with_logits=False,
                            overrides=dict(B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, L=(20, 90), tree="chain"))
    # a page pool with room for every cycle's tree
    cap = w.prefix_lens + (cycles + 1) * N
    table, P = tvgen.make_pages(77 + D, cap, permuted=True)
    host_k = tvgen.normal_bf16(78 + D, 1, (P, Hkv, 16, D))
    host_v = tvgen.normal_bf16(78 + D, 2, (P, Hkv, 16, D))
    kp, vp = dev(host_k, torch.bfloat16), dev(host_v, torch.bfloat16)
    d_table = dev(table)
    max_len = int(w.prefix_lens.max()) + cycles * N
    lens = w.prefix_lens.copy()
    d_lens = dev(lens)
    roots = None
    accepted = 0
    for c in range(cycles):
        print(f"[loop] D={D} {mode} cycle {c}: prefix lengths {lens.tolist()}", flush=True)
        # 1. the dynamic tree, from this cycle's proposals and the last cycle's next root
        r0, toks, probs = proposals(900 + 10 * D + c, B, N, depth, k, V)
        roots = r0 if roots is None else roots
        tree = tv.tv_build_tree(dev(roots), dev(toks), dev(probs), k, 0.0, depth)
        assert tv.tv_device_error(DEV) == 0
        ref_tree = oracle.build_tree(roots, toks, probs, k_root=k, threshold=0.0, max_depth=depth)
        for key in ("parents", "tokens", "depth", "n_nodes"):
            assert (host(tree[key]) == ref_tree[key]).all(), (c, key)
        parents, tokens = ref_tree["parents"], ref_tree["tokens"]
        # 2. the tree nodes' K/V (the target's forward pass) at positions L_b .. L_b + N - 1
        pos = lens[:, None] + np.arange(N)[None, :]
        pages = np.take_along_axis(table, pos // 16, 1).reshape(-1)
        slots = (pos % 16).reshape(-1)
        nk = tvgen.normal_bf16(500 + c, 1 + D, (B * N, Hkv, D))
        nv = tvgen.normal_bf16(500 + c, 2 + D, (B * N, Hkv, D))
        host_k[pages, :, slots, :] = nk
        host_v[pages, :, slots, :] = nv
        ip, isl = torch.from_numpy(pages.astype(np.int64)).to(DEV), torch.from_numpy(slots.astype(np.int64)).to(DEV)
        kp[ip, :, isl, :] = dev(nk, torch.bfloat16)
        vp[ip, :, isl, :] = dev(nv, torch.bfloat16)
        # 3. attention over the cache as the previous cycles left it
        q = tvgen.normal_bf16(600 + c, 3 + D, (B, N, Hq, D))
        mask, _ = tv.tv_build_mask(dev(parents))
        assert (mask_np(mask) == ref_tree["mask"]).all()
        assert torch.equal(mask, tree["mask"])
        out = tv.tv_attention(dev(q, torch.bfloat16), kp, vp, d_table, d_lens, max_len, mask, float(w.sm_scale))
        assert tv.tv_device_error(DEV) == 0
        cw = dataclasses.replace(w, parents=parents, draft_tokens=tokens, prefix_lens=lens.copy(),
                                 max_prefix_len=max_len, page_table=table, num_pages=P, q=q, k_pages=host_k,
                                 v_pages=host_v)
        check_attention(host(out), oracle.attention(cw, ref_tree["mask"]), tight=TIGHT, what=f"cycle {c}")
        # 4. acceptance: greedy on logits that follow the tree part of the time;
        # sampled with each node's draft row close to its parent's target row
        cw.target_logits = tvgen.normal_f32(700 + c, 4 + D, (B, N, V))
        if mode == "greedy":
            tvgen.plant_random(cw, 0.7, seed=c + D)
            got = tv.tv_accept(dev(cw.target_logits), dev(tokens), dev(parents))
            ref = oracle.accept_greedy(cw.target_logits, tokens, parents)
        else:
            near = tvgen.normal_f32(701 + c, 5 + D, (B, N, V), sigma=0.3)
            draft = cw.target_logits[np.arange(B)[:, None], np.maximum(parents, 0)] + near
            uni = tvgen.uniform_f32(702 + c, 6 + D, (B, N))
            got = tv.tv_accept(dev(cw.target_logits), dev(tokens), dev(parents), mode=tv.STOCHASTIC,
                               draft_logits=dev(draft), uniforms=dev(uni), temperature=1.0)
            ref = oracle.accept_stochastic(cw.target_logits, draft, tokens, parents, uni, 1.0)
            assert (ref["margins"] > 1e-9).all(), "a decision too close to call"
        assert tv.tv_device_error(DEV) == 0
        for key in ("accept_len", "path", "bonus"):
            assert (host(got[key]) == ref[key]).all(), (c, key)
        accepted += int((ref["accept_len"] - 1).sum())
        # 5. commit on the device; the oracle commits the host mirror
        com = tv.tv_commit(kp, vp, d_table, d_lens, max_len, dev(tokens), got["path"], got["accept_len"], got["bonus"])
        assert tv.tv_device_error(DEV) == 0
        host_k, host_v, cref = oracle.commit(cw, ref["path"], ref["accept_len"], ref["bonus"])
        assert torch.equal(kp.view(torch.int16), dev(host_k).view(torch.int16)), c
        assert torch.equal(vp.view(torch.int16), dev(host_v).view(torch.int16)), c
        for key in ("new_prefix_lens", "emitted", "next_root"):
            assert (host(com[key]) == cref[key]).all(), (c, key)
        # the next cycle starts from the device's own outputs
        d_lens = com["new_prefix_lens"]
        lens = host(d_lens).astype(np.int32)
        roots = host(com["next_root"]).astype(np.int32)
        assert (lens == cref["new_prefix_lens"]).all()
    assert accepted >= cycles  # drafts were accepted, so rows really moved
