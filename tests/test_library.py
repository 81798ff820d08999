"""CPU-only checks of the C ABI library: it loads, exports every function
include/treeverify.h declares, answers host-only queries, and the product
path never reaches the oracle. No compute call is made (no GPU here)."""
import glob
import os
import re

import pytest

import tree_verify_attention_attn_amd as tv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        names |= set(re.findall(r"\b(tv_[a-z_]+)\s*\(", open(h).read()))
    return names


def test_library_exports_every_declared_symbol():
    lib = tv.library()
    names = declared_functions()
    assert {"tv_create", "tv_build_mask", "tv_attention", "tv_accept", "tv_commit", "tv_build_tree", "tv_tau"} <= names
    missing = [n for n in sorted(names) if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_host_queries():
    lib = tv.library()
    for s in range(6):
        assert lib.tv_status_string(s)
    # accept workspace: greedy = B*N*chunks 64-bit keys (16384-token chunks),
    # stochastic = B*N*2*chunks*(m, Z) doubles (8192-token chunks)
    chunks = (128256 + 16383) // 16384
    assert tv.tv_accept_workspace_bytes(8, 64, 128256, tv.GREEDY) == 8 * 64 * chunks * 8
    assert tv.tv_accept_workspace_bytes(128, 5, 32000, tv.STOCHASTIC) == \
        (128 * 5 * 2 * 4 * 2 + 128 * 2 * 32000) * 8 + (128 * 16 + 128 * 256 * 4) * 8
    assert tv.tv_accept_workspace_bytes(0, 5, 32000, tv.GREEDY) == 0
    # a NULL context is rejected before anything touches a device
    assert lib.tv_build_mask(None, None, None, 1, 1, None, None) == tv.INVALID_ARG
    assert lib.tv_tau_reset(None) == tv.INVALID_ARG
    assert lib.tv_commit(None, None, None, 0, None, 0, None, 0, None, None, None, None, 1, 4, 1, 128, None, None,
                         None) == tv.INVALID_ARG


def test_product_path_never_loads_the_oracle():
    pkg = os.path.join(ROOT, "tree_verify_attention_attn_amd")
    for f in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if f.endswith((".py", ".hip", ".h", ".cpp")):
            text = open(f).read()
            assert not re.search(r"\boracle\b", text), f
            assert "tvgen" not in text, f


def test_tree_budget_follows_the_concurrency_schedule():
    # the page's schedule: the full tree up to 32 concurrent requests, then
    # 64 -> 32 -> 16, and plain decoding (the root alone) past 64
    cases = {(0, 64): 64, (1, 64): 64, (32, 64): 64, (33, 64): 32, (48, 64): 32, (49, 64): 16, (64, 64): 16,
             (65, 64): 1, (4096, 64): 1, (1, 128): 128, (40, 128): 64, (50, 128): 32, (60, 2): 1, (40, 1): 1}
    for (c, n), want in cases.items():
        assert tv.tv_tree_budget(c, n) == want, (c, n)
    for c, n in ((-1, 64), (10, 0), (10, 129)):
        assert tv.tv_tree_budget(c, n) == -1


def test_binding_refuses_host_tensors():
    # a host tensor's address means nothing to the kernels: the binding
    # refuses it before the library is called (no GPU needed)
    import torch
    import tree_verify_attention_attn_amd as tv
    q = torch.zeros((1, 2, 4, 64), dtype=torch.bfloat16)
    kv = torch.zeros((2, 1, 16, 64), dtype=torch.bfloat16)
    i32 = torch.zeros((1, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        tv.tv_attention(q, kv, kv, i32, torch.zeros(1, dtype=torch.int32), 8, None, 1.0)
    with pytest.raises(ValueError, match="GPU"):
        tv.tv_build_mask(i32)
    with pytest.raises(ValueError, match="GPU"):
        tv.tv_accept(torch.zeros((1, 2, 8)), i32, i32)
    with pytest.raises(ValueError, match="GPU"):
        tv.tv_commit(kv, kv, i32, torch.zeros(1, dtype=torch.int32), 8, i32, i32, torch.zeros(1, dtype=torch.int32),
                     torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        tv.tv_build_tree(torch.zeros(1, dtype=torch.int32), torch.zeros((1, 2, 3), dtype=torch.int32),
                         torch.zeros((1, 2, 3)), 3, 0.0, 2)


def test_header_compiles_as_c_and_cpp(tmp_path):
    # include/treeverify.h is a plain C header: C99, C11 and C++17, pedantic,
    # every warning an error
    import subprocess

    src = tmp_path / "uses_header.c"
    src.write_text('#include "treeverify.h"\n'
                   "int main(void) {\n"
                   "  tv_ctx *ctx = 0;\n"
                   "  (void)ctx;\n"
                   "  return tv_status_string(TV_OK)[0] == 0 && tv_tree_budget(1, 64) == 0;\n"
                   "}\n")
    inc = os.path.join(ROOT, "include")
    for cmd in (["gcc", "-std=c99"], ["gcc", "-std=c11"], ["g++", "-std=c++17", "-x", "c++"]):
        r = subprocess.run(cmd + ["-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-I", inc, str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, (cmd, r.stderr)


def test_c_caller_links_and_reports_usage(tmp_path):
    # the plain-C caller the GPU tests run builds against the library and the
    # HIP runtime; without arguments it prints its usage before any HIP call
    import subprocess

    import c_caller_build

    out = str(tmp_path / "c_caller")
    r = subprocess.run(c_caller_build.command(out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_LIBRARY_PATH=c_caller_build.LIBDIR)
    r = subprocess.run([out], capture_output=True, text=True, timeout=60, env=env)
    assert r.returncode == 2 and "usage" in r.stderr
