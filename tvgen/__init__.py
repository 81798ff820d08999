"""Seeded synthetic workloads for tree-verify attention and acceptance.

This module is the only code shared by the oracle tests and the GPU path. It
makes inputs - draft trees, paged bf16 Q/K/V, fp32 logits, uniforms - and holds
none of the verification arithmetic. Bulk random numbers come from the C
generator in ``tvgen.c`` (counter-based splitmix64 streams, Box-Muller normals,
bf16 by round-to-nearest-even), so every consumer sees bit-identical inputs.

Workload shapes follow the five verification configurations of the task
(tiny greedy tree; Llama-3-8B, Llama-3.1-70B and 32K long-context layer shapes
with EAGLE-2/EAGLE-3 dynamic trees; a 4-draft MTP chain with stochastic
acceptance). The dynamic tree is a host rendition of the EAGLE-2 expansion
described on the EAGLE-2 deep-dive page ("dynamic draft tree" section and its
PyTorch sketch): node 0 is the root, candidates carry the cumulative product of
their per-step scores, and the best candidate is popped until the node budget
is reached. Scores here are synthetic: a softmax over the top-k candidates of
N(0, 2) draws, since no trained draft head exists in this build.
"""
from __future__ import annotations

import ctypes
import dataclasses
import heapq
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtvgen.so")
# an alternative build (the sanitizer test loads ASan/UBSan builds this way)
_LIB_OVERRIDE = os.environ.get("TVG_LIB")
_lib = None

# tensor ids: each tensor of a workload draws from its own stream
TID_Q, TID_K, TID_V = 1, 2, 3
TID_TREE, TID_TREE_NORMAL = 4, 5
TID_TOKENS = 6
TID_TLOGITS, TID_DLOGITS = 7, 8
TID_UNIFORMS = 9
TID_PAGES = 10
TID_PREFIX = 11
TID_GUMBEL = 12
TID_PLANT = 13

PAGE = 16


def build(force: bool = True) -> str:
    """Compile libtvgen.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB_PATH):
        src = os.path.join(_HERE, "tvgen.c")
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_OVERRIDE or _LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.tvg_key.restype = u64
        lib.tvg_key.argtypes = [u64, u64]
        lib.tvg_u64.argtypes = [u64, u64, u64, i64, vp]
        lib.tvg_uniform_f32.argtypes = [u64, u64, u64, i64, vp]
        lib.tvg_normal_f64.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.tvg_normal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.tvg_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.tvg_gumbel_argmax.argtypes = [u64, u64, vp, i64, i64, dbl, vp]
        for f in ("tvg_u64", "tvg_uniform_f32", "tvg_normal_f64", "tvg_normal_f32", "tvg_normal_bf16",
                  "tvg_gumbel_argmax"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def u64(seed: int, tid: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().tvg_u64(seed, tid, offset, n, _ptr(out))
    return out


def uniform_f32(seed: int, tid: int, shape, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().tvg_uniform_f32(seed, tid, offset, out.size, _ptr(out))
    return out


def normal_f64(seed: int, tid: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, np.float64)
    _load().tvg_normal_f64(seed, tid, offset, out.size, sigma, _ptr(out))
    return out


def normal_f32(seed: int, tid: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().tvg_normal_f32(seed, tid, offset, out.size, sigma, _ptr(out))
    return out


def normal_bf16(seed: int, tid: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    """bf16 normals returned as their uint16 bit patterns."""
    out = np.empty(shape, np.uint16)
    _load().tvg_normal_bf16(seed, tid, offset, out.size, sigma, _ptr(out))
    return out


def gumbel_argmax(seed: int, tid: int, logits: np.ndarray, temperature: float) -> np.ndarray:
    """One draw per row from softmax(logits / T) by the Gumbel-max trick."""
    logits = np.ascontiguousarray(logits, np.float32)
    V = logits.shape[-1]
    rows = logits.size // V
    out = np.empty(logits.shape[:-1], np.int32)
    _load().tvg_gumbel_argmax(seed, tid, _ptr(logits), rows, V, float(temperature), _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Stream:
    """Sequential consumer of one (seed, tid) stream, fetched in blocks."""

    def __init__(self, seed: int, tid: int, block: int = 4096):
        self.seed, self.tid, self.block = seed, tid, block
        self.pos = 0
        self.buf = np.empty(0, np.uint64)
        self.base = 0

    def next_u64(self) -> int:
        i = self.pos - self.base
        if i >= self.buf.size:
            self.base = self.pos
            self.buf = u64(self.seed, self.tid, self.block, offset=self.pos)
            i = 0
        self.pos += 1
        return int(self.buf[i])

    def randint(self, n: int) -> int:
        """Uniform integer in [0, n): floor(u * n) with u = top 53 bits / 2^53."""
        return ((self.next_u64() >> 11) * n) >> 53

    def uniform(self) -> float:
        return (self.next_u64() >> 11) * 2.0 ** -53


class NormalStream:
    """Sequential fp64 N(0, sigma^2) draws from one (seed, tid) stream."""

    def __init__(self, seed: int, tid: int, sigma: float = 1.0, block: int = 1024):
        self.seed, self.tid, self.sigma, self.block = seed, tid, sigma, block
        self.pos = 0
        self.buf = np.empty(0)
        self.base = 0

    def take(self, n: int) -> np.ndarray:
        out = normal_f64(self.seed, self.tid, (n,), self.sigma, offset=self.pos)
        self.pos += n
        return out


# ----------------------------------------------------------------------------
# draft trees: parents[i] < i, parents[0] = -1 (node 0 is the root, i.e. the
# last verified token, and counts toward the node budget)
# ----------------------------------------------------------------------------

def chain_tree(N: int) -> np.ndarray:
    return np.arange(-1, N - 1, dtype=np.int32)


def star_tree(N: int) -> np.ndarray:
    """Root plus N-1 children of the root."""
    p = np.zeros(N, np.int32)
    if N:
        p[0] = -1
    return p


def forest_tree(N: int) -> np.ndarray:
    """N separate roots: each node's only ancestor is itself."""
    return np.full(N, -1, np.int32)


def random_tree(seed: int, tid: int, N: int, max_depth: int) -> np.ndarray:
    """parent[i] uniform over earlier nodes j with depth[j] <= max_depth - 1."""
    s = Stream(seed, tid)
    parents = np.full(N, -1, np.int32)
    depth = [0] * N
    for i in range(1, N):
        cand = [j for j in range(i) if depth[j] <= max_depth - 1]
        j = cand[s.randint(len(cand))]
        parents[i] = j
        depth[i] = depth[j] + 1
    return parents


def dynamic_tree(seed: int, tid: int, N: int, max_depth: int, topk: int, V: int, record: Optional[dict] = None):
    """Best-first expansion by cumulative score, as in the EAGLE-2 page's
    dynamic-tree algorithm (no pruning threshold, budget N including the root).

    Returns (parents int32[N], tokens int32[N]); tokens[0] is the root token.
    Sibling tokens are distinct (drawn without replacement). If `record` is a
    dict, record[node] = (tokens, probabilities) of every node's proposals.
    """
    s = Stream(seed, tid)
    zs = NormalStream(seed, tid + (1 << 20), sigma=math.sqrt(2.0))
    parents = [-1]
    tokens = [s.randint(V)]
    depth = [0]
    cum = [1.0]
    heap = []
    seq = 0

    def push_children(node):
        nonlocal seq
        if depth[node] >= max_depth:
            return
        z = zs.take(topk)
        e = np.exp(z - z.max())
        sc = e / e.sum()
        toks = []
        while len(toks) < topk:
            t = s.randint(V)
            if t not in toks:
                toks.append(t)
        if record is not None:
            record[node] = (list(toks), sc.copy())
        for k in range(topk):
            heapq.heappush(heap, (-(cum[node] * sc[k]), seq, node, toks[k]))
            seq += 1

    push_children(0)
    while len(parents) < N and heap:
        negc, _, par, tok = heapq.heappop(heap)
        parents.append(par)
        tokens.append(tok)
        depth.append(depth[par] + 1)
        cum.append(-negc)
        push_children(len(parents) - 1)
    return np.asarray(parents, np.int32), np.asarray(tokens, np.int32)


def tree_depths(parents: np.ndarray) -> np.ndarray:
    d = np.zeros(len(parents), np.int32)
    for i, p in enumerate(parents):
        d[i] = 0 if p < 0 else d[p] + 1
    return d


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------

CONFIGS = {
    1: dict(name="tiny-greedy", B=1, Hq=4, Hkv=1, D=64, L=128, N=15, tree="random", max_depth=4,
            pages="contiguous", V=1024, mode="greedy", T=1.0),
    2: dict(name="llama3-8b-eagle2", B=8, Hq=32, Hkv=8, D=128, L=2048, N=64, tree="dynamic", max_depth=6,
            topk=10, pages="permuted", V=128256, mode="greedy", T=1.0),
    3: dict(name="llama31-70b-eagle3", B=32, Hq=64, Hkv=8, D=128, L=4096, N=60, tree="dynamic", max_depth=8,
            topk=10, pages="permuted", V=128256, mode="greedy", T=1.0),
    4: dict(name="long-context-32k", B=4, Hq=32, Hkv=8, D=128, L=32768, N=64, tree="dynamic", max_depth=8,
            topk=10, pages="permuted", V=128256, mode="greedy", T=1.0),
    5: dict(name="mtp-chain-stochastic", B=128, Hq=32, Hkv=8, D=128, L=(256, 4096), N=5, tree="chain",
            pages="permuted", V=32000, mode="stochastic", T=1.0),
}


@dataclasses.dataclass
class Workload:
    cfg: int
    seed: int
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    V: int
    mode: str
    temperature: float
    sm_scale: np.float32
    prefix_lens: np.ndarray  # int32 [B]
    max_prefix_len: int
    page_table: np.ndarray  # int32 [B][maxp], -1 beyond each sequence's pages
    num_pages: int
    parents: np.ndarray  # int32 [B][N]
    draft_tokens: np.ndarray  # int32 [B][N]
    q: Optional[np.ndarray] = None  # bf16 bits uint16 [B][N][Hq][D]
    k_pages: Optional[np.ndarray] = None  # bf16 bits uint16 [P][Hkv][16][D]
    v_pages: Optional[np.ndarray] = None
    target_logits: Optional[np.ndarray] = None  # f32 [B][N][V]
    draft_logits: Optional[np.ndarray] = None  # f32 [B][N][V]
    uniforms: Optional[np.ndarray] = None  # f32 [B][N]

    @property
    def maxp(self) -> int:
        return self.page_table.shape[1]


def sm_scale_for(D: int) -> np.float32:
    return np.float32(1.0) / np.sqrt(np.float32(D))


def make_pages(seed: int, lens_plus_n: np.ndarray, permuted: bool):
    npages = (lens_plus_n + PAGE - 1) // PAGE
    P = int(npages.sum())
    maxp = int(npages.max()) if len(npages) else 0
    if permuted:
        s = Stream(seed, TID_PAGES)
        perm = np.arange(P, dtype=np.int32)
        for i in range(P - 1, 0, -1):  # Fisher-Yates
            j = s.randint(i + 1)
            perm[i], perm[j] = perm[j], perm[i]
    else:
        perm = np.arange(P, dtype=np.int32)
    table = np.full((len(npages), max(maxp, 1)), -1, np.int32)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, P


def make_workload(cfg: int, seed: Optional[int] = None, *, with_kv: bool = True, with_logits: bool = True,
                  overrides: Optional[dict] = None) -> Workload:
    """Build configuration `cfg` (1..5) with stream seed `seed` (default 1000+cfg).

    `overrides` may replace any shape field (B, N, L, V, ...) to derive smaller
    cases with the same recipe.
    """
    c = dict(CONFIGS[cfg])
    if overrides:
        c.update(overrides)
    if seed is None:
        seed = 1000 + cfg
    B, N, Hq, Hkv, D, V = c["B"], c["N"], c["Hq"], c["Hkv"], c["D"], c["V"]

    L = c["L"]
    if isinstance(L, tuple):
        lo, hi = L
        s = Stream(seed, TID_PREFIX)
        prefix = np.array([lo + s.randint(hi - lo + 1) for _ in range(B)], np.int32)
    else:
        prefix = np.full(B, L, np.int32)

    parents = np.empty((B, N), np.int32)
    tokens = np.empty((B, N), np.int32)
    ts = Stream(seed, TID_TOKENS)
    for b in range(B):
        if c["tree"] == "random":
            parents[b] = random_tree(seed, (TID_TREE << 16) + b, N, c["max_depth"])
            tokens[b] = [ts.randint(V) for _ in range(N)]
        elif c["tree"] == "dynamic":
            p, t = dynamic_tree(seed, (TID_TREE << 16) + b, N, c["max_depth"], c["topk"], V)
            assert len(p) == N, "candidate pool exhausted before the node budget"
            parents[b], tokens[b] = p, t
        elif c["tree"] == "chain":
            parents[b] = chain_tree(N)
            tokens[b] = [ts.randint(V) for _ in range(N)]
        elif c["tree"] == "star":
            parents[b] = star_tree(N)
            tokens[b] = [ts.randint(V) for _ in range(N)]
        elif c["tree"] == "forest":
            parents[b] = forest_tree(N)
            tokens[b] = [ts.randint(V) for _ in range(N)]
        else:
            raise ValueError(c["tree"])

    table, P = make_pages(seed, prefix + N, c["pages"] == "permuted")
    w = Workload(cfg=cfg, seed=seed, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, mode=c["mode"], temperature=c["T"],
                 sm_scale=sm_scale_for(D), prefix_lens=prefix, max_prefix_len=int(prefix.max()) if B else 0,
                 page_table=table, num_pages=P, parents=parents, draft_tokens=tokens)
    if with_kv:
        w.q = normal_bf16(seed, TID_Q, (B, N, Hq, D))
        w.k_pages = normal_bf16(seed, TID_K, (P, Hkv, PAGE, D))
        w.v_pages = normal_bf16(seed, TID_V, (P, Hkv, PAGE, D))
    if with_logits:
        w.target_logits = normal_f32(seed, TID_TLOGITS, (B, N, V))
        if c["mode"] == "stochastic":
            w.draft_logits = normal_f32(seed, TID_DLOGITS, (B, N, V))
            w.uniforms = uniform_f32(seed, TID_UNIFORMS, (B, N))
            # draft tokens t_i ~ q_i = softmax(draft_logits[b][i] / T), i >= 1
            drawn = gumbel_argmax(seed, TID_GUMBEL, w.draft_logits, c["T"])
            w.draft_tokens[:, 1:] = drawn[:, 1:]
    return w


# ----------------------------------------------------------------------------
# planted acceptance variants (parity only): force target argmaxes by writing
# large logits at chosen draft tokens. Pure data edits; no acceptance logic.
# ----------------------------------------------------------------------------

def plant_full_path(w: Workload, b: int, leaf: int, value: float = 10.0) -> None:
    """Make every node on root->leaf the target's argmax at its parent."""
    c = leaf
    while w.parents[b, c] >= 0:
        p = w.parents[b, c]
        w.target_logits[b, p, w.draft_tokens[b, c]] = value
        c = p


def plant_random(w: Workload, rho: float, seed: int = 7) -> None:
    """Each non-root node, with probability rho, gets a large distinct logit
    (6 + 4u) at its token in its parent's row."""
    s = Stream(seed, TID_PLANT)
    for b in range(w.B):
        for c in range(1, w.N):
            u = s.uniform()
            v = s.uniform()
            p = w.parents[b, c]
            if p >= 0 and u < rho:
                w.target_logits[b, p, w.draft_tokens[b, c]] = np.float32(6.0 + 4.0 * v)
