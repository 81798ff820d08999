"""TEST INFRASTRUCTURE ONLY: ctypes wrapper around the fp64 CPU oracle.

Only tests/, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package. The product library never loads it, and it shares no
code with the GPU path. All arrays are host numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# an alternative build (the sanitizer test loads ASan/UBSan builds this way)
_LIB_OVERRIDE = os.environ.get("TVO_LIB")
_lib = None

OK, INVALID_ARG, INVALID_TREE, UNSUPPORTED, WORKSPACE, RUNTIME = range(6)


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"oracle {what} returned status {status}")
        self.status = status


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_OVERRIDE or _LIB_PATH)
        vp, i32, i64, f32, c_int = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        lib.tvo_build_mask.argtypes = [vp, vp, i32, i32, vp, vp]
        lib.tvo_attention.argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, f32, vp,
                                      i64, vp, c_int]
        lib.tvo_accept_greedy.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, c_int]
        lib.tvo_accept_stochastic.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, c_int]
        lib.tvo_commit.argtypes = [vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        lib.tvo_build_tree.argtypes = [vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp]
        lib.tvo_tau.argtypes = [vp, i64]
        lib.tvo_tau.restype = ctypes.c_double
        for f in ("tvo_build_mask", "tvo_attention", "tvo_accept_greedy", "tvo_accept_stochastic", "tvo_commit",
                  "tvo_build_tree"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def status_build_mask(parents, B=None, N=None, tree_sizes=None):
    parents = _c(parents, np.int32)
    tree_sizes = _c(tree_sizes, np.int32)
    B = parents.shape[0] if B is None else B
    N = parents.shape[1] if N is None else N
    W = max((N + 63) // 64, 1)
    mask = np.zeros((max(B, 0), max(N, 0), W), np.uint64)
    depth = np.zeros((max(B, 0), max(N, 0)), np.int32)
    st = _load().tvo_build_mask(_p(parents), _p(tree_sizes), B, N, _p(mask), _p(depth))
    return st, mask, depth


def build_mask(parents, tree_sizes=None):
    """parents int32 [B][N] -> (mask uint64 [B][N][ceil(N/64)], depth int32 [B][N])."""
    st, mask, depth = status_build_mask(parents, tree_sizes=tree_sizes)
    if st != OK:
        raise OracleError(st, "build_mask")
    return mask, depth


def status_attention(q, k_pages, v_pages, page_table, prefix_lens, tree_mask, *, B, N, Hq, Hkv, D, sm_scale,
                     num_pages=None, maxp=None, max_prefix_len=None, rows=None, nthreads=0, tree_sizes=None):
    q = _c(q, np.uint16)
    k_pages = _c(k_pages, np.uint16)
    v_pages = _c(v_pages, np.uint16)
    page_table = _c(page_table, np.int32)
    prefix_lens = _c(prefix_lens, np.int32)
    tree_mask = _c(tree_mask, np.uint64)
    tree_sizes = _c(tree_sizes, np.int32)
    if num_pages is None:
        num_pages = k_pages.shape[0]
    if maxp is None:
        maxp = page_table.shape[1]
    if max_prefix_len is None:
        max_prefix_len = int(prefix_lens.max()) if prefix_lens.size else 0
    rows = _c(rows, np.int32)
    n_rows = rows.shape[0] if rows is not None else max(B, 0) * max(N, 0) * max(Hq, 0)
    out = np.zeros((n_rows, max(D, 1)), np.float64)
    st = _load().tvo_attention(_p(q), _p(k_pages), _p(v_pages), num_pages, _p(page_table), maxp, _p(prefix_lens),
                               max_prefix_len, _p(tree_mask), _p(tree_sizes), B, N, Hq, Hkv, D, np.float32(sm_scale),
                               _p(rows),
                               n_rows, _p(out), nthreads)
    return st, out


def attention(w, tree_mask, rows=None, nthreads=0, tree_sizes=None):
    """fp64 attention for workload `w` (see tvgen.Workload).

    rows: optional int32 [n][3] (b, i, h) list; default every row. Returns
    [n][D] (rows given) or [B][N][Hq][D] (all rows).
    """
    st, out = status_attention(w.q, w.k_pages, w.v_pages, w.page_table, w.prefix_lens, tree_mask, B=w.B, N=w.N,
                               Hq=w.Hq, Hkv=w.Hkv, D=w.D, sm_scale=w.sm_scale, num_pages=w.num_pages,
                               max_prefix_len=w.max_prefix_len, rows=rows, nthreads=nthreads, tree_sizes=tree_sizes)
    if st != OK:
        raise OracleError(st, "attention")
    if rows is None:
        return out.reshape(w.B, w.N, w.Hq, w.D)
    return out


def status_accept_greedy(target_logits, draft_tokens, parents, B, N, V, nthreads=0, tree_sizes=None):
    target_logits = _c(target_logits, np.float32)
    draft_tokens = _c(draft_tokens, np.int32)
    parents = _c(parents, np.int32)
    Bn, Nn = max(B, 0), max(N, 1)
    accept_len = np.zeros(Bn, np.int32)
    path = np.zeros((Bn, Nn), np.int32)
    bonus = np.zeros(Bn, np.int32)
    y = np.zeros((Bn, Nn), np.int32)
    tree_sizes = _c(tree_sizes, np.int32)
    st = _load().tvo_accept_greedy(_p(target_logits), _p(draft_tokens), _p(parents), _p(tree_sizes), B, N, V,
                                   _p(accept_len), _p(path), _p(bonus), _p(y), nthreads)
    return st, dict(accept_len=accept_len, path=path, bonus=bonus, target_argmax=y)


def accept_greedy(target_logits, draft_tokens, parents, nthreads=0, tree_sizes=None):
    B, N, V = target_logits.shape
    st, r = status_accept_greedy(target_logits, draft_tokens, parents, B, N, V, nthreads, tree_sizes=tree_sizes)
    if st != OK:
        raise OracleError(st, "accept_greedy")
    return r


def status_accept_stochastic(target_logits, draft_logits, draft_tokens, parents, uniforms, B, N, V, temperature,
                             nthreads=0, tree_sizes=None):
    target_logits = _c(target_logits, np.float32)
    draft_logits = _c(draft_logits, np.float32)
    draft_tokens = _c(draft_tokens, np.int32)
    parents = _c(parents, np.int32)
    uniforms = _c(uniforms, np.float32)
    Bn, Nn = max(B, 0), max(N, 1)
    accept_len = np.zeros(Bn, np.int32)
    path = np.zeros((Bn, Nn), np.int32)
    bonus = np.zeros(Bn, np.int32)
    margins = np.zeros((Bn, Nn), np.float64)
    tree_sizes = _c(tree_sizes, np.int32)
    st = _load().tvo_accept_stochastic(_p(target_logits), _p(draft_logits), _p(draft_tokens), _p(parents),
                                       _p(tree_sizes), _p(uniforms), B, N, V, np.float32(temperature), _p(accept_len), _p(path),
                                       _p(bonus), _p(margins), nthreads)
    return st, dict(accept_len=accept_len, path=path, bonus=bonus, margins=margins)


def accept_stochastic(target_logits, draft_logits, draft_tokens, parents, uniforms, temperature, nthreads=0,
                      tree_sizes=None):
    B, N, V = target_logits.shape
    st, r = status_accept_stochastic(target_logits, draft_logits, draft_tokens, parents, uniforms, B, N, V,
                                     temperature, nthreads, tree_sizes=tree_sizes)
    if st != OK:
        raise OracleError(st, "accept_stochastic")
    return r


def tau(accept_lens) -> float:
    a = _c(np.asarray(accept_lens).reshape(-1), np.int32)
    return _load().tvo_tau(_p(a), a.size)


def status_commit(k_pages, v_pages, page_table, prefix_lens, draft_tokens, path, accept_len, bonus, *, B, N, Hkv,
                  D, num_pages=None, maxp=None, max_prefix_len=None, with_emitted=True):
    """Accepted-path commit on copies of k_pages / v_pages.

    Returns (status, k_new, v_new, dict(new_prefix_lens, emitted, next_root)).
    """
    k = np.array(k_pages, dtype=np.uint16, order="C", copy=True)
    v = np.array(v_pages, dtype=np.uint16, order="C", copy=True)
    page_table = _c(page_table, np.int32)
    prefix_lens = _c(prefix_lens, np.int32)
    draft_tokens = _c(draft_tokens, np.int32)
    path = _c(path, np.int32)
    accept_len = _c(accept_len, np.int32)
    bonus = _c(bonus, np.int32)
    if num_pages is None:
        num_pages = k.shape[0]
    if maxp is None:
        maxp = page_table.shape[1]
    if max_prefix_len is None:
        max_prefix_len = int(prefix_lens.max()) if prefix_lens.size else 0
    new_lens = np.full(max(B, 0), -2, np.int32)
    emitted = np.full((max(B, 0), max(N, 0)), -2, np.int32) if with_emitted else None
    next_root = np.full(max(B, 0), -2, np.int32)
    st = _load().tvo_commit(_p(k), _p(v), num_pages, _p(page_table), maxp, _p(prefix_lens), max_prefix_len,
                            _p(draft_tokens), _p(path), _p(accept_len), _p(bonus), B, N, Hkv, D, _p(new_lens),
                            _p(emitted), _p(next_root))
    return st, k, v, dict(new_prefix_lens=new_lens, emitted=emitted, next_root=next_root)


def commit(w, path, accept_len, bonus):
    """Commit the accepted paths of workload `w` (see tvgen.Workload) on copies
    of its pages. Returns (k_new, v_new, dict(new_prefix_lens, emitted, next_root))."""
    st, k, v, r = status_commit(w.k_pages, w.v_pages, w.page_table, w.prefix_lens, w.draft_tokens, path,
                                accept_len, bonus, B=w.B, N=w.N, Hkv=w.Hkv, D=w.D, num_pages=w.num_pages,
                                max_prefix_len=w.max_prefix_len)
    if st != OK:
        raise OracleError(st, "commit")
    return k, v, r


def status_build_tree(root_tokens, cand_tokens, cand_probs, *, k_root, threshold, max_depth, B=None, N=None, k=None):
    """Returns (status, dict(parents, tokens, depth, mask, scores, n_nodes))."""
    cand_tokens = _c(cand_tokens, np.int32)
    cand_probs = _c(cand_probs, np.float32)
    root_tokens = _c(root_tokens, np.int32)
    B = cand_tokens.shape[0] if B is None else B
    N = cand_tokens.shape[1] if N is None else N
    k = cand_tokens.shape[2] if k is None else k
    shp = (max(B, 0), max(N, 0))
    W = max((N + 63) // 64, 1)
    out = dict(parents=np.full(shp, -2, np.int32), tokens=np.full(shp, -2, np.int32), depth=np.full(shp, -2, np.int32),
               mask=np.zeros(shp + (W,), np.uint64), scores=np.full(shp, np.nan),
               n_nodes=np.full(shp[0], -2, np.int32))
    st = _load().tvo_build_tree(_p(root_tokens), _p(cand_tokens), _p(cand_probs), B, N, k, k_root,
                                np.float32(threshold), max_depth, _p(out["parents"]), _p(out["tokens"]),
                                _p(out["depth"]), _p(out["mask"]), _p(out["scores"]), _p(out["n_nodes"]))
    return st, out


def build_tree(root_tokens, cand_tokens, cand_probs, *, k_root, threshold, max_depth):
    st, out = status_build_tree(root_tokens, cand_tokens, cand_probs, k_root=k_root, threshold=threshold,
                                max_depth=max_depth)
    if st != OK:
        raise OracleError(st, "build_tree")
    return out
