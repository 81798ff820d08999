"""GPU parity: tv_accept (greedy and stochastic) and tv_tau against the oracle.

Greedy outputs (accept_len, path, bonus, per-row argmax) must be bit-exact.
Stochastic decisions are taken in fp64 on both sides; they must agree
exactly wherever the oracle's decision margin exceeds 1e-9 (every seeded case
here), and the test reports the margins so a near-tie is visible.
"""
import numpy as np
import pytest

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, KEYS, DevWorkload, dev, greedy_compare, host, stochastic_compare

pytestmark = pytest.mark.gpu



@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("variant", ["random", "planted-full", "planted-partial"])
def test_greedy_full_size(cfg, variant):
    w = tvgen.make_workload(cfg, with_kv=False)
    print(f"[accept] cfg{cfg} {variant} B={w.B} N={w.N} V={w.V}", flush=True)
    if variant == "planted-full":
        for b in range(w.B):
            d = tvgen.tree_depths(w.parents[b])
            tvgen.plant_full_path(w, b, int(np.argmax(d)))
    elif variant == "planted-partial":
        tvgen.plant_random(w, 0.5, seed=cfg)
    ref = greedy_compare(w, f"cfg{cfg}-{variant}")
    if variant == "planted-full":
        depth = np.stack([tvgen.tree_depths(p) for p in w.parents])
        assert (ref["accept_len"] == depth.max(1) + 1).all()


@pytest.mark.parametrize("seed", range(4))
def test_greedy_ties_and_duplicate_siblings(seed):
    # tiny vocab and half-integer logits: exact ties, repeated sibling tokens
    w = tvgen.make_workload(1, seed=900 + seed, with_kv=False,
                            overrides=dict(B=200, N=3 + 15 * seed, V=6, max_depth=4))
    w.target_logits = np.round(w.target_logits * 2) / 2
    greedy_compare(w, f"ties-{seed}")


def test_greedy_odd_vocab_and_nan():
    # V not a multiple of 4 takes the scalar path; NaN ranks below every number
    w = tvgen.make_workload(2, with_kv=False, overrides=dict(B=3, V=10007))
    w.target_logits[0, 0, :50] = np.nan
    w.target_logits[1, 3, :] = np.nan
    tvgen.plant_random(w, 0.6)
    greedy_compare(w, "odd-V-nan")


def test_greedy_large_batch():
    # 70000 sequences of three nodes over a tiny vocabulary: grid dimensions
    # beyond 65536 rows and many path-pass workgroups
    w = tvgen.make_workload(1, seed=77, with_kv=False, overrides=dict(B=70000, N=3, V=8, max_depth=2))
    tvgen.plant_random(w, 0.7, seed=3)
    greedy_compare(w, "B70000")


@pytest.mark.parametrize("B,N,V", [(128, 2, 8), (129, 2, 8), (2, 128, 8193), (2, 128, 16384), (2, 128, 16385),
                                   (1, 15, 1024), (3, 64, 24577)])
def test_greedy_one_launch_limit(B, N, V):
    # with at most 256 argmax workgroups (rows x 16384-token chunks), the
    # argmax pass's last workgroup of each sequence runs the path logic (one
    # launch); above, the path pass runs on its own
    w = tvgen.make_workload(1, seed=B + N + V, with_kv=False,
                            overrides=dict(B=B, N=N, V=V, max_depth=min(N - 1, 9), tree="random"))
    tvgen.plant_random(w, 0.6, seed=5)
    print(f"[accept] greedy B={B} N={N} V={V}", flush=True)
    ref = greedy_compare(w, f"B{B}-N{N}-V{V}")
    assert (ref["accept_len"] >= 2).any()


def test_greedy_consecutive_calls_of_different_shapes():
    # the per-sequence arrival counters are left at zero by every call, so
    # calls of any shape can follow each other (several chunks per row, node
    # counts, 65-128 nodes)
    shapes = [dict(B=5, N=64, V=3000), dict(B=3, N=100, V=20000), dict(B=7, N=10, V=24577),
              dict(B=5, N=64, V=3000), dict(B=40, N=128, V=100)]
    for i, sh in enumerate(shapes):
        w = tvgen.make_workload(2, seed=40 + i, with_kv=False, overrides=dict(tree="random", max_depth=9, **sh))
        tvgen.plant_random(w, 0.7, seed=i)
        print(f"[accept] consecutive call {i}: {sh}", flush=True)
        greedy_compare(w, f"call{i}")
        sizes = np.array([1 + (7 * b) % sh["N"] for b in range(sh["B"])], np.int32)
        got = tv.tv_accept(dev(w.target_logits), dev(w.draft_tokens), dev(w.parents), tree_sizes=dev(sizes))
        assert tv.tv_device_error(DEV) == 0
        ref = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents, tree_sizes=sizes)
        for k in KEYS:
            assert (host(got[k]) == ref[k]).all(), (i, k)


def test_calls_on_two_streams_are_ordered():
    # one context rebound from stream to stream: the second call starts after
    # the first, so the two never share the arrival counters at once
    import torch
    # a one-launch shape (60 argmax workgroups) and a two-launch shape
    ws = [tvgen.make_workload(2, seed=60 + i, with_kv=False, overrides=sh)
          for i, sh in enumerate([dict(B=4, N=15, V=1024, max_depth=5), dict(B=8, N=64, V=128256)])]
    for i, w in enumerate(ws):
        tvgen.plant_random(w, 0.8, seed=i)
    dws = [DevWorkload(w, kv=False) for w in ws]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for dw, st in zip(dws, streams):
            with torch.cuda.stream(st):
                outs.append((dw.w, dw.accept(tv.GREEDY)))
    torch.cuda.synchronize()
    assert tv.tv_device_error(DEV) == 0
    for w, got in outs:
        ref = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
        for k in KEYS:
            assert (host(got[k]) == ref[k]).all(), k


def test_greedy_grid_limit_is_reported():
    # one workgroup per (row, 16384-token chunk) on a 1-D grid of at most
    # 2^32 - 1 work-items: larger calls are refused before any launch
    w = tvgen.make_workload(1, with_kv=False, overrides=dict(B=2, N=4, V=16))
    dw = DevWorkload(w, kv=False)
    lib, p = tv.library(), tv._ptr
    out = [dev(np.zeros(8, np.int32)) for _ in range(4)]
    ws = dev(np.zeros(64, np.uint8))
    st = lib.tv_accept(tv._ctx(DEV), p(dw.target_logits), None, p(dw.draft_tokens), p(dw.parents), None, None,
                       1 << 20, 128, 128256, tv.GREEDY, 1.0, p(out[0]), p(out[1]), p(out[2]), p(out[3]), p(ws), 64)
    assert st == tv.UNSUPPORTED
    # 2^24 - 1 rows of 16384 tokens: one greedy chunk per row fits the grid
    # (the call then stops at the too-small workspace), two stochastic chunks
    # per row do not
    rows, V = (1 << 24) - 1, 16384
    st = lib.tv_accept(tv._ctx(DEV), p(dw.target_logits), None, p(dw.draft_tokens), p(dw.parents), None, None,
                       rows, 1, V, tv.GREEDY, 1.0, p(out[0]), p(out[1]), p(out[2]), p(out[3]), p(ws), 64)
    assert st == tv.WORKSPACE
    st = lib.tv_accept(tv._ctx(DEV), p(dw.target_logits), p(dw.target_logits), p(dw.draft_tokens), p(dw.parents),
                       None, p(ws), rows, 1, V, tv.STOCHASTIC, 1.0, p(out[0]), p(out[1]), p(out[2]), None, p(ws), 64)
    assert st == tv.UNSUPPORTED
    # 2^23 sequences of one node over a 16-token vocabulary: the chunk grid
    # fits, the path pass's one 512-thread workgroup per sequence does not
    st = lib.tv_accept(tv._ctx(DEV), p(dw.target_logits), p(dw.target_logits), p(dw.draft_tokens), p(dw.parents),
                       None, p(ws), 1 << 23, 1, 16, tv.STOCHASTIC, 1.0, p(out[0]), p(out[1]), p(out[2]), None, p(ws),
                       64)
    assert st == tv.UNSUPPORTED


@pytest.mark.parametrize("N,V", [(1, 50), (6, 1), (1, 1), (1, 128256)])
def test_degenerate_shapes_both_modes(N, V):
    # root only (nothing to verify: the bonus is the root row's argmax or a
    # draw from it), a one-token vocabulary (every draft matches, every
    # distribution is the point mass), both
    w = tvgen.make_workload(5, seed=N * 10 + V, with_kv=False, overrides=dict(B=5, N=N, V=V))
    w.draft_tokens[:, :] = np.minimum(w.draft_tokens, V - 1)
    print(f"[accept] degenerate N={N} V={V}", flush=True)
    ref = greedy_compare(w, f"N{N}-V{V}")
    assert (ref["accept_len"] == N).all() if V == 1 else (ref["accept_len"] == 1).all()
    stochastic_compare(w, f"N{N}-V{V}-stochastic")


def test_empty_batch_launches_nothing():
    lib, p = tv.library(), tv._ptr
    w = tvgen.make_workload(1, with_kv=False, overrides=dict(B=1, N=2, V=4))
    dw = DevWorkload(w, kv=False)
    out = [dev(np.full(4, 7, np.int32)) for _ in range(4)]
    for mode in (tv.GREEDY, tv.STOCHASTIC):
        st = lib.tv_accept(tv._ctx(DEV), p(dw.target_logits), p(dw.draft_logits), p(dw.draft_tokens), p(dw.parents),
                           None, p(dw.uniforms), 0, 2, 4, mode, 1.0, p(out[0]), p(out[1]), p(out[2]), p(out[3]), None, 0)
        assert st == tv.OK
    assert all((host(o) == 7).all() for o in out)
    assert tv.tv_device_error(DEV) == 0


def test_greedy_forest_nodes_never_accepted():
    w = tvgen.make_workload(1, with_kv=False, overrides=dict(B=8, N=12, tree="forest", V=64))
    w.parents[:, 0] = -1
    w.parents[:, 1] = 0
    w.parents[:, 2] = 1
    greedy_compare(w, "forest")


def test_stochastic_cfg5_full_size():
    w = tvgen.make_workload(5, with_kv=False)
    dw = DevWorkload(w, kv=False)
    got = dw.accept(tv.STOCHASTIC)
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms,
                                   w.temperature)
    m = ref["margins"]
    print(f"[accept] cfg5 stochastic: min decision margin {np.nanmin(m):.3e}, "
          f"accept_len histogram {np.bincount(ref['accept_len']).tolist()}", flush=True)
    assert (m > 1e-9).all()
    for k in ("accept_len", "path", "bonus"):
        assert (host(got[k]) == ref[k]).all(), k


@pytest.mark.parametrize("variant", ["p-equals-q", "small-vocab", "temperature", "odd-vocab", "masked-vocab",
                                     "masked-vocab-temperature"])
def test_stochastic_variants(variant):
    over = dict(B=64)
    T = 1.0
    if variant == "small-vocab":
        over.update(V=7, N=9)
    if variant == "odd-vocab":
        over.update(V=12345, N=3)
    if variant == "temperature":
        over.update(V=5000)
    if variant.startswith("masked-vocab"):
        over.update(V=20000, N=5)
    w = tvgen.make_workload(5, seed=55, with_kv=False, overrides=over)
    if variant == "p-equals-q":
        w.draft_logits[:, 1:] = w.target_logits[:, :-1]
    if variant in ("temperature", "masked-vocab-temperature"):
        T = 0.7
        w.temperature = T
    if variant.startswith("masked-vocab"):
        # every seventh token banned (-inf in both distributions) in every
        # other sequence, and in the others one token per row far below the
        # row's maximum, so that its exponential underflows; neither is ever
        # a drafted token
        for b in range(w.B):
            if b % 2 == 0:
                ban = np.arange(3, w.V, 7)
                ban = ban[~np.isin(ban, w.draft_tokens[b])]
                w.target_logits[b][:, ban] = -np.inf
                w.draft_logits[b][:, ban] = -np.inf
            else:
                low = next(x for x in range(11, w.V) if x not in w.draft_tokens[b])
                w.target_logits[b][:, low] = -1e4
                w.draft_logits[b][:, low] = -1e4
    dw = DevWorkload(w, kv=False)
    got = dw.accept(tv.STOCHASTIC)
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms, T)
    m = ref["margins"]
    print(f"[accept] variant {variant}: min decision margin {np.nanmin(m):.3e}", flush=True)
    # every decision of the seeded inputs is far from a coin flip, so any
    # difference is a bug, not rounding
    assert (m > 1e-9).all(), variant
    for k in ("accept_len", "path", "bonus"):
        assert (host(got[k]) == ref[k]).all(), k
    if variant == "p-equals-q":
        assert (ref["accept_len"] == w.N).all()


def test_stochastic_tree_full_size():
    # the Llama-3-8B EAGLE-2 shape (64-node dynamic trees, V = 128256) with
    # sampled acceptance; each node's token drawn from its own draft row
    w = tvgen.make_workload(2, with_kv=False, overrides=dict(mode="stochastic"))
    ref = stochastic_compare(w, "cfg2-stochastic")
    assert ref["accept_len"].max() >= 2


@pytest.mark.parametrize("tree", ["random", "dynamic", "star", "forest"])
def test_stochastic_tree_shapes(tree):
    over = dict(B=48, N=40, V=3000, tree=tree, mode="stochastic")
    if tree in ("random", "dynamic"):
        over.update(max_depth=5, topk=6)
    w = tvgen.make_workload(2, seed=61, with_kv=False, overrides=over)
    if tree == "forest":
        w.parents[:, 1:8] = 0  # a root with seven children, the rest unreachable
    # draft rows close to the target rows make long accepted paths; far ones
    # make many rejected siblings (stored residuals)
    near = tvgen.normal_f32(61, 95, w.draft_logits.shape, sigma=0.3)
    for b in range(0, w.B, 2):
        for c in range(1, w.N):
            pr = w.parents[b, c]
            if pr >= 0:
                w.draft_logits[b, c] = w.target_logits[b, pr] + near[b, c]
    stochastic_compare(w, f"tree-{tree}")


@pytest.mark.parametrize("T", [0.6, 1.7])
def test_stochastic_tree_temperatures(T):
    # sampled acceptance on dynamic trees away from T = 1 (logits divided by
    # T in fp64 on both sides)
    w = tvgen.make_workload(2, seed=62, with_kv=False,
                            overrides=dict(B=24, N=40, V=5000, tree="dynamic", max_depth=5, topk=6, mode="stochastic"))
    near = tvgen.normal_f32(62, 96, w.draft_logits.shape, sigma=0.3)
    for b in range(w.B):
        for c in range(1, w.N):
            w.draft_logits[b, c] = w.target_logits[b, w.parents[b, c]] + near[b, c]
    w.temperature = T
    ref = stochastic_compare(w, f"tree-T{T}")
    assert ref["accept_len"].max() >= 3


def test_stochastic_tree_hand_worked_fixture():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "stochastic_tree_hand.json")))
    B = len(g["parents"])
    tl = np.tile(np.array(g["target_rows"], np.float32)[None], (B, 1, 1))
    dl = np.tile(np.array(g["draft_rows"], np.float32)[None], (B, 1, 1))
    got = tv.tv_accept(dev(tl), dev(np.array(g["draft_tokens"], np.int32)), dev(np.array(g["parents"], np.int32)),
                       mode=tv.STOCHASTIC, draft_logits=dev(dl), uniforms=dev(np.array(g["uniforms"], np.float32)),
                       temperature=g["temperature"])
    assert tv.tv_device_error(DEV) == 0
    for k, v in g["expect"].items():
        assert host(got[k]).tolist() == v, k


def test_stochastic_star_every_sibling_rejected():
    # 63 siblings under the root, draft rows far from the target: most
    # sequences reject many siblings in a row (one stored residual each)
    w = tvgen.make_workload(5, seed=62, with_kv=False, overrides=dict(B=16, N=64, V=2048, tree="star"))
    w.draft_logits *= 3.0
    w.draft_tokens[:, 1:] = tvgen.gumbel_argmax(62, 96, w.draft_logits, 1.0)[:, 1:]
    ref = stochastic_compare(w, "star-63")
    assert (ref["accept_len"] == 1).any()


@pytest.mark.parametrize("B,V", [(4, 65536), (3, 50001)])
def test_stochastic_star_sliced_vocab(B, V):
    # few sequences over a large vocabulary: each sequence's sweeps are split
    # over many workgroups that exchange their slice sums; 63 siblings give
    # long runs of stored residuals (an odd V takes the scalar loads)
    w = tvgen.make_workload(5, seed=63, with_kv=False, overrides=dict(B=B, N=64, V=V, tree="star"))
    w.draft_logits *= 2.5
    w.draft_tokens[:, 1:] = tvgen.gumbel_argmax(63, 97, w.draft_logits, 1.0)[:, 1:]
    stochastic_compare(w, f"star-sliced-B{B}-V{V}")


@pytest.mark.parametrize("V", [300000, 266241])
def test_stochastic_one_slice_many_rounds(V):
    # enough sequences that each one's vocabulary is one workgroup's slice,
    # and a vocabulary long enough that a wavefront sweeps more than 64 rounds
    # of 512 tokens: the final draw finds its round among records of two
    # rounds and recomputes the lanes' block sums (kept in LDS only for the
    # first rounds); an odd V takes the scalar loads
    w = tvgen.make_workload(5, seed=64, with_kv=False, overrides=dict(B=136, N=2, V=V))
    ref = stochastic_compare(w, f"one-slice-B136-V{V}")
    assert (ref["accept_len"] == 1).any() and (ref["accept_len"] == 2).any()


@pytest.mark.parametrize("B,N,V", [(130, 16, 20000), (100, 8, 100000)])
def test_stochastic_star_multi_round_slices(B, N, V):
    # stored residuals swept in several rounds per wavefront: one workgroup
    # per sequence with 5 rounds (B = 130), and two per sequence with 13
    # rounds, past the rounds whose lane sums the sweep keeps (B = 100); the
    # first round of a stored residual comes from registers, the others from
    # memory
    w = tvgen.make_workload(5, seed=65, with_kv=False, overrides=dict(B=B, N=N, V=V, tree="star"))
    w.draft_logits *= 2.5
    w.draft_tokens[:, 1:] = tvgen.gumbel_argmax(65, 98, w.draft_logits, 1.0)[:, 1:]
    ref = stochastic_compare(w, f"star-rounds-B{B}-N{N}-V{V}")
    assert (ref["accept_len"] == 1).any()


def test_tau_accumulates_over_calls():
    tv.tv_tau_reset(DEV)
    lens = []
    for cfg, seed in ((1, 3), (2, 4), (1, 5)):
        w = tvgen.make_workload(cfg, seed=seed, with_kv=False, overrides=dict(V=512))
        tvgen.plant_random(w, 0.7, seed=seed)
        lens.append(greedy_compare(w, f"tau-{cfg}")["accept_len"])
    w = tvgen.make_workload(5, with_kv=False, overrides=dict(B=16, V=300))
    DevWorkload(w, kv=False).accept(tv.STOCHASTIC)
    lens.append(oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms,
                                         1.0)["accept_len"])
    tau, cycles = tv.tv_tau(DEV)
    all_lens = np.concatenate(lens)
    assert cycles == all_lens.size
    assert tau == oracle.tau(all_lens)
    tv.tv_tau_reset(DEV)
    assert tv.tv_tau(DEV) == (0.0, 0)


def test_device_detected_errors():
    w = tvgen.make_workload(1, with_kv=False, overrides=dict(B=2, V=100))
    # bad parent
    p = w.parents.copy()
    p[1, 4] = 9
    st, _ = oracle.status_accept_greedy(w.target_logits, w.draft_tokens, p, w.B, w.N, w.V)
    dw = DevWorkload(w, kv=False)
    dw.parents = dev(p)
    got = dw.accept(tv.GREEDY)
    assert tv.tv_device_error(DEV) == st == oracle.INVALID_TREE
    assert host(got["accept_len"])[1] == -1
    # token out of range
    t = w.draft_tokens.copy()
    t[0, 2] = w.V
    st, _ = oracle.status_accept_greedy(w.target_logits, t, w.parents, w.B, w.N, w.V)
    dw = DevWorkload(w, kv=False)
    dw.draft_tokens = dev(t)
    dw.accept(tv.GREEDY)
    assert tv.tv_device_error(DEV) == st == oracle.INVALID_ARG
    # stochastic with a parent not earlier than its child
    w5 = tvgen.make_workload(5, with_kv=False, overrides=dict(B=2, V=100))
    p5 = w5.parents.copy()
    p5[:, 3] = 3
    st, _ = oracle.status_accept_stochastic(w5.target_logits, w5.draft_logits, w5.draft_tokens, p5, w5.uniforms,
                                            w5.B, w5.N, w5.V, 1.0)
    dw = DevWorkload(w5, kv=False)
    dw.parents = dev(p5)
    got = dw.accept(tv.STOCHASTIC)
    assert tv.tv_device_error(DEV) == st == oracle.INVALID_TREE
    assert (host(got["accept_len"]) == -1).all()


def test_host_detected_errors():
    w = tvgen.make_workload(5, with_kv=False, overrides=dict(B=2, V=100))
    dw = DevWorkload(w, kv=False)
    with pytest.raises(tv.TVError) as e:
        tv.tv_accept(dw.target_logits, dw.draft_tokens, dw.parents, mode=tv.STOCHASTIC, draft_logits=dw.draft_logits,
                     uniforms=dw.uniforms, temperature=0.0)
    assert e.value.status == tv.INVALID_ARG
    with pytest.raises(tv.TVError) as e:
        tv.tv_accept(dw.target_logits, dw.draft_tokens, dw.parents, mode=tv.STOCHASTIC)
    assert e.value.status == tv.INVALID_ARG
    import torch
    with pytest.raises(tv.TVError) as e:
        tv.tv_accept(dw.target_logits, dw.draft_tokens, dw.parents,
                     workspace=torch.empty(8, dtype=torch.uint8, device=DEV))
    assert e.value.status == tv.WORKSPACE
