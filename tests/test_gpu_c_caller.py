"""The C ABI from plain C, with no Python in the calling process: the test
writes a seeded workload to files, runs tests/_build/c_caller (built by
__graft_entry__.build() from tests/c_caller.c), which makes tv_build_mask,
tv_attention, tv_accept (greedy, or sampled) and tv_commit calls on device 0
and writes their outputs, and compares those with the oracle: masks, depths,
paths, lengths, bonus, argmax and the committed pools, lengths, emitted
tokens and next roots bit-exact, attention within the usual tolerance, tau
exact."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import tvgen
from gpu_util import check_attention

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "_build", "c_caller")

SHAPES = {
    # several key tiles per sequence, a ragged tail, GQA group 4, 24 nodes
    "d128": dict(B=3, Hq=8, Hkv=2, D=128, L=(300, 700), N=24, V=5000, tree="random", max_depth=6, pages="permuted"),
    # head dim 64, a 70-node tree (two mask words), one sequence with an empty prefix
    "d64-70-nodes": dict(B=2, Hq=4, Hkv=1, D=64, L=(0, 200), N=70, V=777, tree="random", max_depth=9,
                         pages="permuted"),
    # sampled acceptance on random trees at temperature 0.8, each node's token
    # drawn from its draft row
    "sampled-tree": dict(B=4, Hq=8, Hkv=2, D=128, L=(100, 500), N=20, V=3000, tree="random", max_depth=5,
                         pages="permuted", mode="stochastic", T=0.8),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_c_caller_matches_oracle(name, tmp_path):
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build() first"
    sampled = SHAPES[name].get("mode") == "stochastic"
    w = tvgen.make_workload(2 if sampled else 1, seed=3100 + len(name), overrides=SHAPES[name])
    if name.startswith("d64"):
        w.prefix_lens[0] = 0
    if not sampled:
        tvgen.plant_random(w, 0.7, seed=31)
    d = str(tmp_path)
    with open(os.path.join(d, "shape.txt"), "w") as f:
        f.write(f"{w.B} {w.N} {w.Hq} {w.Hkv} {w.D} {w.k_pages.shape[0]} {w.page_table.shape[1]} "
                f"{w.max_prefix_len} {w.V} {repr(float(w.sm_scale))}" +
                (f" {repr(float(np.float32(w.temperature)))}" if sampled else "") + "\n")
    files = [("q.bin", w.q), ("k.bin", w.k_pages), ("v.bin", w.v_pages), ("table.bin", w.page_table),
             ("plens.bin", w.prefix_lens), ("parents.bin", w.parents), ("tokens.bin", w.draft_tokens),
             ("logits.bin", w.target_logits)]
    if sampled:
        files += [("draft.bin", w.draft_logits), ("uniforms.bin", w.uniforms)]
    for fname, arr in files:
        np.ascontiguousarray(arr).tofile(os.path.join(d, fname))
    print(f"[c caller] {name}: B{w.B} Hq{w.Hq}/Hkv{w.Hkv} D{w.D} N{w.N} V{w.V} "
          f"prefix lengths {w.prefix_lens.tolist()}", flush=True)
    r = subprocess.run([BIN, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"c_caller failed ({r.returncode}): {r.stderr}"
    fields = r.stdout.split()
    assert fields[0] == "tau" and fields[2] == "cycles" and fields[4] == "device_error", r.stdout
    assert int(fields[5]) == 0, "device error flag raised"

    def got(fname, dtype, shape):
        return np.fromfile(os.path.join(d, fname), dtype=dtype).reshape(shape)

    W = (w.N + 63) // 64
    omask, odepth = oracle.build_mask(w.parents)
    assert (got("mask.bin", np.uint64, (w.B, w.N, W)) == omask).all()
    assert (got("depth.bin", np.int32, (w.B, w.N)) == odepth).all()
    check_attention(got("out.bin", np.float32, (w.B, w.N, w.Hq, w.D)), oracle.attention(w, omask), what=name)
    if sampled:
        ref = oracle.accept_stochastic(w.target_logits, w.draft_logits, w.draft_tokens, w.parents, w.uniforms,
                                       np.float32(w.temperature))
        # every decision of the seeded input is far from a coin flip
        assert (ref["margins"] > 1e-9).all()
    else:
        ref = oracle.accept_greedy(w.target_logits, w.draft_tokens, w.parents)
        assert (got("argmax.bin", np.int32, (w.B, w.N)) == ref["target_argmax"]).all()
    assert (got("accept_len.bin", np.int32, (w.B,)) == ref["accept_len"]).all()
    assert (got("path.bin", np.int32, (w.B, w.N)) == ref["path"]).all()
    assert (got("bonus.bin", np.int32, (w.B,)) == ref["bonus"]).all()
    assert int(fields[3]) == w.B and float(fields[1]) == oracle.tau(ref["accept_len"])
    assert (ref["accept_len"] >= 2).any()
    # the commit of the accepted paths, on the pools as the call found them
    k_ref, v_ref, cref = oracle.commit(w, ref["path"], ref["accept_len"], ref["bonus"])
    assert (got("k_new.bin", np.uint16, w.k_pages.shape) == k_ref).all()
    assert (got("v_new.bin", np.uint16, w.v_pages.shape) == v_ref).all()
    assert (got("new_lens.bin", np.int32, (w.B,)) == cref["new_prefix_lens"]).all()
    assert (got("emitted.bin", np.int32, (w.B, w.N)) == cref["emitted"]).all()
    assert (got("next_root.bin", np.int32, (w.B,)) == cref["next_root"]).all()
