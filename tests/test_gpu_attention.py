"""GPU parity: tv_attention against the fp64 oracle on the same seeded inputs.

Small cases are compared in full (several tiles, ragged tails, special
trees, edge shapes); the five full-size configurations are compared on
sampled rows in the launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, TIGHT, DevWorkload, check_attention, dev, host

pytestmark = pytest.mark.gpu


def small(tree, *, B=3, Hq=8, Hkv=2, D=128, L=(0, 300), N=20, seed=5, max_depth=5):
    return tvgen.make_workload(1, seed=seed, with_logits=False,
                               overrides=dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, N=N, tree=tree, pages="permuted",
                                              max_depth=max_depth))


def run_full(w, use_mask=True, out_dtype=torch.float32):
    dw = DevWorkload(w, logits=False)
    mask = tv.tv_build_mask(dw.parents)[0] if use_mask else None
    out = dw.attention(mask, out_dtype=out_dtype)
    om = oracle.build_mask(w.parents)[0] if use_mask else None
    ref = oracle.attention(w, om)
    assert tv.tv_device_error(DEV) == 0
    return host(out.float()), ref


SMALL_CASES = [
    ("random-D128-G4", dict(tree="random")),
    ("random-D64-G1", dict(tree="random", D=64, Hq=4, Hkv=4)),
    ("random-D64-G8", dict(tree="random", D=64, Hq=16, Hkv=2, N=33)),
    ("chain", dict(tree="chain", N=16)),
    ("star", dict(tree="star", N=31)),
    ("forest", dict(tree="forest", N=12)),
    ("dynamic-N64", dict(tree="random", N=64, max_depth=8, L=(100, 700))),
    ("prefix-0", dict(tree="random", L=0)),
    ("decode-N1", dict(tree="chain", N=1, L=(1, 200))),
    ("ragged-long", dict(tree="random", B=5, L=(1, 3000), N=7)),
]


@pytest.mark.parametrize("name,kw", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_small_cases_full_compare(name, kw):
    w = small(**kw)
    print(f"[attn] {name} B={w.B} N={w.N} Hq={w.Hq} Hkv={w.Hkv} D={w.D} L={w.prefix_lens.tolist()}", flush=True)
    got, ref = run_full(w)
    check_attention(got, ref, what=name)


def test_all_visible_baseline():
    w = small("random", N=24)
    got, ref = run_full(w, use_mask=False)
    check_attention(got, ref, what="mask=NULL")


def test_bf16_output():
    w = small("random", N=24)
    got, ref = run_full(w, out_dtype=torch.bfloat16)
    check_attention(got, ref, what="bf16 out")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 1e-3, 2.0])
def test_unusual_scales(scale):
    # a negative scale (Q is negated, |scale| used), zero (every visible key
    # weighs the same), tiny, and large (a peaked softmax whose running max
    # keeps jumping, so the lazy rescale runs)
    import dataclasses
    w = small("random", N=24, L=(100, 900), seed=11)
    w = dataclasses.replace(w, sm_scale=np.float32(scale))
    print(f"[attn] sm_scale={scale}", flush=True)
    got, ref = run_full(w)
    check_attention(got, ref, what=f"scale {scale}")


def test_many_short_row_groups_of_mixed_lengths():
    # more one-workgroup units than CUs (the MTP-chain shape: at most 32 rows
    # per KV head) with prefixes from 0 to 3000: the units are dispatched
    # longest first; every row against the oracle
    w = small("chain", B=300, Hq=4, Hkv=1, D=128, L=(0, 3000), N=3, seed=21)
    print(f"[attn] mixed lengths B={w.B} rows/unit={w.N * w.Hq // w.Hkv}", flush=True)
    got, ref = run_full(w)
    check_attention(got, ref, what="mixed lengths")


def test_deterministic_and_page_permutation_invariant():
    w = small("random", N=30, L=(500, 900), seed=8)
    dw = DevWorkload(w, logits=False)
    mask = tv.tv_build_mask(dw.parents)[0]
    a = host(dw.attention(mask))
    b = host(dw.attention(mask))
    assert np.array_equal(a, b), "two identical calls differ"
    rng = np.random.default_rng(1)
    perm = rng.permutation(w.num_pages).astype(np.int32)
    k2, v2 = np.empty_like(w.k_pages), np.empty_like(w.v_pages)
    k2[perm], v2[perm] = w.k_pages, w.v_pages
    w.k_pages, w.v_pages = k2, v2
    w.page_table = np.where(w.page_table >= 0, perm[np.maximum(w.page_table, 0)], -1).astype(np.int32)
    c = host(DevWorkload(w, logits=False).attention(mask))
    assert np.array_equal(a, c), "page relocation changed the result"


@pytest.mark.parametrize("D,Hkv,Hq", [(128, 2, 8), (64, 4, 16)])
def test_kv_pool_above_2gib(D, Hkv, Hq):
    """Pages placed past the first 2 GiB of a KV pool take the per-page buffer
    resource path (smaller pools share one resource with 32-bit offsets)."""
    w = small("random", N=24, L=(300, 700), D=D, Hkv=Hkv, Hq=Hq, seed=12)
    page_bytes = Hkv * 16 * D * 2
    offset = (2 ** 31) // page_bytes + 3000
    print(f"[attn] KV pool above 2 GiB, D{D} Hkv{Hkv}, page offset {offset}", flush=True)
    dw = DevWorkload(w, logits=False)
    big_k = torch.empty((offset + w.num_pages, Hkv, 16, D), dtype=torch.bfloat16, device=DEV)
    big_v = torch.empty_like(big_k)
    big_k[offset:] = dw.k
    big_v[offset:] = dw.v
    table = torch.where(dw.page_table >= 0, dw.page_table + offset, dw.page_table)
    mask = tv.tv_build_mask(dw.parents)[0]
    out = tv.tv_attention(dw.q, big_k, big_v, table, dw.prefix_lens, w.max_prefix_len, mask, float(w.sm_scale))
    assert tv.tv_device_error(DEV) == 0
    ref = oracle.attention(w, oracle.build_mask(w.parents)[0])
    check_attention(host(out), ref, tight=TIGHT, what=f"pool above 2 GiB, D{D}")
    del big_k, big_v


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_full_size_configs_every_element(cfg):
    # every output element of each workload at full size, in the launch
    # configuration the bench times, against the fp64 oracle (multithreaded:
    # a few seconds of host time for the largest)
    w = tvgen.make_workload(cfg, with_logits=False)
    print(f"[attn] cfg{cfg} full size, every row: {w.B * w.N * w.Hq} rows", flush=True)
    dw = DevWorkload(w, logits=False)
    mask = tv.tv_build_mask(dw.parents)[0]
    out = host(dw.attention(mask))
    assert tv.tv_device_error(DEV) == 0
    om = oracle.build_mask(w.parents)[0]
    check_attention(out, oracle.attention(w, om), tight=TIGHT, what=f"cfg{cfg}")


def test_device_detected_bad_page_and_length():
    w = small("random", N=10, L=(40, 90), B=2)
    bad = w.page_table.copy()
    bad[1, 1] = w.num_pages + 5
    st, _ = oracle.status_attention(w.q, w.k_pages, w.v_pages, bad, w.prefix_lens, None, B=w.B, N=w.N, Hq=w.Hq,
                                    Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale)
    dw = DevWorkload(w, logits=False)
    dw.page_table = dev(bad)
    out = host(dw.attention(None))
    assert tv.tv_device_error(DEV) == st == oracle.INVALID_ARG
    assert np.isnan(out[1]).all()
    assert np.isfinite(out[0]).all()
    dw = DevWorkload(w, logits=False)
    pl = w.prefix_lens.copy()
    pl[0] = w.max_prefix_len + 1
    dw.prefix_lens = dev(pl)
    out = host(dw.attention(None))
    assert tv.tv_device_error(DEV) == oracle.INVALID_ARG
    assert np.isnan(out[0]).all()


def test_host_detected_errors():
    w = small("random", N=10, L=(40, 90), B=2)
    dw = DevWorkload(w, logits=False)

    def call(**kw):
        args = dict(q=dw.q, k_pages=dw.k, v_pages=dw.v, page_table=dw.page_table, prefix_lens=dw.prefix_lens,
                    max_prefix_len=w.max_prefix_len, tree_mask=None, sm_scale=float(w.sm_scale))
        args.update(kw)
        with pytest.raises(tv.TVError) as e:
            tv.tv_attention(**args)
        return e.value.status

    assert call(max_prefix_len=w.page_table.shape[1] * 16) == tv.INVALID_ARG  # pages cannot hold L + N
    assert call(q=dw.q[:, :, :7].contiguous()) == tv.INVALID_ARG  # Hq % Hkv != 0
    q96 = torch.zeros((w.B, w.N, w.Hq, 96), dtype=torch.bfloat16, device=DEV)
    k96 = torch.zeros((w.num_pages, w.Hkv, 16, 96), dtype=torch.bfloat16, device=DEV)
    assert call(q=q96, k_pages=k96, v_pages=k96) == tv.UNSUPPORTED
    assert call(sm_scale=float("nan")) == tv.INVALID_ARG
    need = tv.tv_attention_workspace_bytes(DEV, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
    if need > 0:
        assert call(workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV)) == tv.WORKSPACE
    assert tv.tv_device_error(DEV) == 0


def test_size_limits_are_reported():
    # token positions and key counts are int32 inside the kernels: a prefix
    # bound above 2^30 is refused before any launch, by tv_attention and by
    # tv_commit, and the workspace query returns 0 for it
    lib, p = tv.library(), tv._ptr
    ctx = tv._ctx(DEV)
    big = (1 << 30) + 1
    maxp = (big + 16 + 15) // 16
    buf = dev(np.zeros(64, np.int32))
    assert lib.tv_attention_workspace_bytes(ctx, 1, 2, 4, 1, 64, big) == 0
    assert lib.tv_attention_workspace_bytes(ctx, 1, 2, 4, 1, 64, 1 << 30) > 0
    st = lib.tv_attention(ctx, p(buf), p(buf), p(buf), 1, p(buf), maxp, p(buf), big, None, None, 1, 2, 4, 1, 64,
                          1.0, p(buf), tv.F32, None, 0)
    assert st == tv.UNSUPPORTED
    st = lib.tv_commit(ctx, p(buf), p(buf), 1, p(buf), maxp, p(buf), big, p(buf), p(buf), p(buf), p(buf), 1, 2, 1, 64,
                       p(buf), None, p(buf))
    assert st == tv.UNSUPPORTED
    assert tv.tv_device_error(DEV) == 0


def test_binding_checks_arguments():
    # mixed devices, wrong dtypes and wrong shapes are refused by the binding
    # before any pointer reaches the library
    w = small("random", N=10, L=(40, 90), B=2)
    dw = DevWorkload(w, logits=False)
    mask, _ = tv.tv_build_mask(dw.parents)
    base = dict(q=dw.q, k_pages=dw.k, v_pages=dw.v, page_table=dw.page_table, prefix_lens=dw.prefix_lens,
                max_prefix_len=w.max_prefix_len, tree_mask=mask, sm_scale=float(w.sm_scale))

    def refused(exc, **kw):
        args = dict(base)
        args.update(kw)
        with pytest.raises(exc):
            tv.tv_attention(**args)

    refused(ValueError, prefix_lens=dw.prefix_lens.cpu())
    refused(TypeError, page_table=dw.page_table.long())
    refused(ValueError, prefix_lens=dw.prefix_lens[:1].contiguous())
    refused(ValueError, tree_mask=torch.zeros((w.B, w.N, 2), dtype=torch.int64, device=DEV))
    refused(ValueError, v_pages=dw.v[:, :, :8].contiguous())
    refused(ValueError, out=torch.empty((w.B, w.N, w.Hq, w.D + 1), dtype=torch.float32, device=DEV))
    refused(TypeError, out=torch.empty((w.B, w.N, w.Hq, w.D), dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        tv.tv_build_mask(dw.parents, mask=torch.zeros((w.B, w.N, 2), dtype=torch.int64, device=DEV))
    assert tv.tv_device_error(DEV) == 0


@pytest.mark.parametrize("N,L,slot,split", [(10, (38, 40), 1, False), (10, (38, 40), 2, False),
                                             (10, (400, 450), 1, True), (10, (400, 450), 2, True),
                                             (40, (10, 20), 2, False), (40, (400, 450), 2, True)],
                         ids=["one-split-first-half", "one-split-second-half", "split-first-half",
                              "split-second-half", "8-waves-one-split-second-half", "8-waves-split-second-half"])
def test_bad_page_seen_by_either_half(N, L, slot, split):
    # a bad page id is found by the wavefronts whose share of the tile it
    # falls in: page slot 1 of a tile by the first half of the workgroup,
    # slot 2 by the second. The first half writes its rows before the final
    # barrier, so a bad page found by the second half must still turn every
    # row of the sequence into NaN, for one key split (outputs written
    # directly) and for several (partials merged afterwards), with two
    # wavefronts per workgroup (40 rows) and with eight (160 rows)
    w = small("random", N=N, L=L, B=2)
    # the plan splits keys exactly when it asks for a workspace
    need = tv.tv_attention_workspace_bytes(DEV, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
    assert (need > 0) == split, need
    bad = w.page_table.copy()
    bad[1, slot] = w.num_pages + 5
    st, _ = oracle.status_attention(w.q, w.k_pages, w.v_pages, bad, w.prefix_lens, None, B=w.B, N=w.N, Hq=w.Hq,
                                    Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale)
    assert st == oracle.INVALID_ARG
    dw = DevWorkload(w, logits=False)
    dw.page_table = dev(bad)
    print(f"[attention] bad page slot {slot}, prefix lengths {w.prefix_lens.tolist()}", flush=True)
    out = host(dw.attention(None))
    assert tv.tv_device_error(DEV) == oracle.INVALID_ARG
    assert np.isnan(out[1]).all()
    assert np.isfinite(out[0]).all()


@pytest.mark.parametrize("case", ["key-split-one-split", "key-split-last-split", "negative-id", "last-split"])
def test_bad_page_variants(case):
    # a bad page id turns every row of its sequence into NaN and reports
    # INVALID_ARG: in the key-split template (at most 32 rows per KV head:
    # the two wavefronts merge through LDS after the bad page is seen), with
    # one key split and with the bad page in the last of several splits; a
    # negative id (-1) inside the sequence's pages; and a bad page in the last
    # split of the ping-pong template
    if case.startswith("key-split"):
        L = (38, 40) if case == "key-split-one-split" else (900, 1000)
        w = small("random", N=5, Hq=4, Hkv=1, L=L, B=2)
    elif case == "negative-id":
        w = small("random", N=10, L=(150, 200), B=2)
    else:
        w = small("random", N=40, L=(900, 1000), B=2)
    bad = w.page_table.copy()
    last = (int(w.prefix_lens[1]) + w.N - 1) // 16
    slot = {"key-split-one-split": 1, "key-split-last-split": last, "negative-id": 2, "last-split": last}[case]
    bad[1, slot] = -1 if case == "negative-id" else w.num_pages + 7
    st, _ = oracle.status_attention(w.q, w.k_pages, w.v_pages, bad, w.prefix_lens, None, B=w.B, N=w.N, Hq=w.Hq,
                                    Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale)
    assert st == oracle.INVALID_ARG
    plan_ws = tv.tv_attention_workspace_bytes(DEV, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
    print(f"[attention] bad page case {case}: slot {slot} of {last + 1}, prefix lengths {w.prefix_lens.tolist()}, "
          f"rows per KV head {w.N * w.Hq // w.Hkv}, workspace {plan_ws} B", flush=True)
    dw = DevWorkload(w, logits=False)
    dw.page_table = dev(bad)
    out = host(dw.attention(None))
    assert tv.tv_device_error(DEV) == oracle.INVALID_ARG
    assert np.isnan(out[1]).all()
    assert np.isfinite(out[0]).all()


@pytest.mark.parametrize("case", ["ping-pong", "key-split", "splits"])
def test_entries_past_each_sequence_are_ignored(case):
    # page-table entries past a sequence's last page (L_b + N keys) are never
    # read: filling them with ids outside the pool, negative ids or the
    # largest int changes neither the status nor a bit of the output, in the
    # ping-pong template, the key-split template and a plan with key splits
    if case == "ping-pong":
        w = small("random", N=40, L=(100, 400), B=3, seed=11)
    elif case == "key-split":
        w = small("random", N=5, Hq=4, Hkv=1, L=(30, 700), B=3, seed=12)
    else:
        w = small("random", N=20, L=(1500, 3000), B=2, seed=13)
    dw = DevWorkload(w, logits=False)
    mask = tv.tv_build_mask(dw.parents)[0]
    clean = host(dw.attention(mask))
    assert tv.tv_device_error(DEV) == 0
    junk = w.page_table.copy()
    fills = np.array([w.num_pages + 1000, -7, 2**31 - 1], np.int64)
    planted = 0
    for b in range(w.B):
        used = (int(w.prefix_lens[b]) + w.N + 15) // 16
        n = junk.shape[1] - used
        junk[b, used:] = np.resize(fills, n).astype(np.int32)
        planted += n
    assert planted > 0
    st, _ = oracle.status_attention(w.q, w.k_pages, w.v_pages, junk, w.prefix_lens, None, B=w.B, N=w.N, Hq=w.Hq,
                                    Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale)
    assert st == oracle.OK
    print(f"[attention] entries past each sequence, {case}: {planted} planted, prefix lengths "
          f"{w.prefix_lens.tolist()}", flush=True)
    dw.page_table = dev(junk)
    got = host(dw.attention(mask))
    assert tv.tv_device_error(DEV) == 0
    assert np.array_equal(got, clean), "entries past the sequence changed the output"


def test_split_partials_wide_rows():
    # a split plan (several key splits per sequence) where the KV head 1's
    # values are scaled by 64 (exact in bf16): its rows' partials O/l exceed
    # the fp16 bound and go to HBM in fp32, the other head's in fp16; both
    # must merge to the oracle's output
    w = small("random", N=24, L=(900, 1000), B=2, Hq=8, Hkv=2, seed=17)
    v = tvgen.bf16_to_f32(w.v_pages)
    v[:, 1] *= 64.0
    w.v_pages = (v.view(np.uint32) >> 16).astype(np.uint16)
    need = tv.tv_attention_workspace_bytes(DEV, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
    print(f"[attn] wide partials: L={w.prefix_lens.tolist()}, workspace {need} B", flush=True)
    assert need > 0
    got, ref = run_full(w)
    assert np.abs(ref[:, :, 4:]).max() > 4.0  # head group 1 is wide
    check_attention(got[:, :, :4], ref[:, :, :4], what="fp16 partials")
    # the outputs are linear in V: the scaled group, brought back to the
    # unscaled values' size, meets the same bar (the bf16 rounding of P
    # moves outputs in proportion to |V|)
    check_attention(got[:, :, 4:] / 64.0, ref[:, :, 4:] / 64.0, what="fp32 partials")
