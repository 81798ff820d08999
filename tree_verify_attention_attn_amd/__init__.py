"""Python binding of libtreeverify (tree-verify attention and acceptance on MI355X).

Argument marshalling only: every step of the verification pass runs in the
HIP kernels of ``libtreeverify.so``. torch supplies device memory and the
current HIP stream. Functions carry the C ABI's names (see
``include/treeverify.h``); each takes torch tensors on one GPU and raises
``TVError`` on a non-OK status. There is no CPU fallback: if the library is
not built, or no GPU is present, calls fail loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtreeverify.so")

OK, INVALID_ARG, INVALID_TREE, UNSUPPORTED, WORKSPACE, HIP_ERROR = range(6)
F32, BF16 = 0, 1
GREEDY, STOCHASTIC = 0, 1

_lib = None
_ctxs = {}


class TVError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _load().tv_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def build(force: bool = True) -> str:
    from . import hipbuild as _b
    return _b.build(force=force)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        st = ctypes.c_int
        lib.tv_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp]
        lib.tv_destroy.argtypes = [vp]
        lib.tv_set_stream.argtypes = [vp, vp]
        lib.tv_build_mask.argtypes = [vp, vp, vp, i32, i32, vp, vp]
        lib.tv_attention_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, i32]
        lib.tv_attention_workspace_bytes.restype = sz
        lib.tv_attention.argtypes = [vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32, f32,
                                     vp, ctypes.c_int, vp, sz]
        lib.tv_accept_workspace_bytes.argtypes = [i32, i32, i32, ctypes.c_int]
        lib.tv_accept_workspace_bytes.restype = sz
        lib.tv_accept.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_int, f32, vp, vp, vp, vp, vp,
                                  sz]
        lib.tv_build_tree.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp]
        lib.tv_commit.argtypes = [vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
        lib.tv_tau.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64)]
        lib.tv_tau_reset.argtypes = [vp]
        lib.tv_device_error.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
        lib.tv_status_string.argtypes = [ctypes.c_int]
        lib.tv_status_string.restype = ctypes.c_char_p
        lib.tv_tree_budget.argtypes = [i32, i32]
        lib.tv_tree_budget.restype = i32
        for f in ("tv_create", "tv_destroy", "tv_set_stream", "tv_build_mask", "tv_attention", "tv_accept",
                  "tv_commit", "tv_build_tree", "tv_tau", "tv_tau_reset", "tv_device_error"):
            getattr(lib, f).restype = st
        _lib = lib
    return _lib


def library() -> ctypes.CDLL:
    """The loaded libtreeverify (raises if it is not built)."""
    return _load()


def _ctx(device: torch.device):
    """Per-device context, rebound to torch's current stream on every call."""
    if device.type != "cuda":
        raise ValueError("libtreeverify runs on a GPU: pass tensors on a cuda (HIP) device")
    idx = device.index if device.index is not None else torch.cuda.current_device()
    lib = _load()
    if idx not in _ctxs:
        h = ctypes.c_void_p()
        s = lib.tv_create(ctypes.byref(h), idx, ctypes.c_void_p(torch.cuda.current_stream(idx).cuda_stream))
        if s != OK:
            raise TVError(s, "tv_create")
        _ctxs[idx] = h
    h = _ctxs[idx]
    s = lib.tv_set_stream(h, ctypes.c_void_p(torch.cuda.current_stream(idx).cuda_stream))
    if s != OK:
        raise TVError(s, "tv_set_stream")
    return h


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check(s: int, what: str):
    if s != OK:
        raise TVError(s, what)


def tv_build_mask(parents: torch.Tensor, mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
                  tree_sizes: Optional[torch.Tensor] = None):
    """parents int32 [B][N] (N <= 128), tree_sizes int32 [B] or None ->
    (mask uint64-as-int64 [B][N][ceil(N/64)], depth int32 [B][N])."""
    B, N = parents.shape
    dev = parents.device
    W = max((N + 63) // 64, 1)
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    assert parents.dtype == torch.int32
    _check(_load().tv_build_mask(_ctx(dev), _ptr(parents), _ptr(tree_sizes), B, N, _ptr(mask), _ptr(depth)),
           "tv_build_mask")
    return mask, depth


def tv_build_tree(root_tokens: torch.Tensor, cand_tokens: torch.Tensor, cand_probs: torch.Tensor, k_root: int,
                  threshold: float, max_depth: int, outputs: Optional[dict] = None) -> dict:
    """root_tokens int32 [B]; cand_tokens int32 / cand_probs fp32 [B][N][k] ->
    dict(parents, tokens, depth [B][N] int32, mask int64 [B][N][W], scores fp64 [B][N], n_nodes [B])."""
    B, N, k = cand_tokens.shape
    assert cand_probs.shape == cand_tokens.shape and cand_probs.dtype == torch.float32
    assert cand_tokens.dtype == torch.int32 and root_tokens.dtype == torch.int32
    dev = cand_tokens.device
    if outputs is None:
        outputs = dict(parents=torch.empty((B, N), dtype=torch.int32, device=dev),
                       tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                       depth=torch.empty((B, N), dtype=torch.int32, device=dev),
                       mask=torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=dev),
                       scores=torch.empty((B, N), dtype=torch.float64, device=dev),
                       n_nodes=torch.empty(B, dtype=torch.int32, device=dev))
    o = outputs
    _check(_load().tv_build_tree(_ctx(dev), _ptr(root_tokens), _ptr(cand_tokens), _ptr(cand_probs), B, N, k, k_root,
                                 float(threshold), max_depth, _ptr(o["parents"]), _ptr(o["tokens"]),
                                 _ptr(o.get("depth")), _ptr(o.get("mask")), _ptr(o.get("scores")),
                                 _ptr(o.get("n_nodes"))), "tv_build_tree")
    return outputs


def tv_attention_workspace_bytes(device, B, N, Hq, Hkv, D, max_prefix_len) -> int:
    return int(_load().tv_attention_workspace_bytes(_ctx(torch.device(device)), B, N, Hq, Hkv, D, max_prefix_len))


def tv_attention(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor,
                 prefix_lens: torch.Tensor, max_prefix_len: int, tree_mask: Optional[torch.Tensor], sm_scale: float,
                 out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
                 workspace: Optional[torch.Tensor] = None, tree_sizes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q bf16 [B][N][Hq][D]; k/v_pages bf16 [P][Hkv][16][D]; page_table int32 [B][maxp];
    prefix_lens int32 [B]; tree_mask int64 [B][N][W] or None; tree_sizes int32 [B] or None
    -> out [B][N][Hq][D] (rows of absent nodes are not written)."""
    B, N, Hq, D = q.shape
    P, Hkv, page, D2 = k_pages.shape
    assert page == 16 and D2 == D and q.dtype == torch.bfloat16 and k_pages.dtype == torch.bfloat16
    assert v_pages.shape == k_pages.shape and v_pages.dtype == torch.bfloat16
    assert page_table.dtype == torch.int32 and prefix_lens.dtype == torch.int32
    dev = q.device
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    odt = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    h = _ctx(dev)
    need = int(_load().tv_attention_workspace_bytes(h, B, N, Hq, Hkv, D, max_prefix_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().tv_attention(h, _ptr(q), _ptr(k_pages), _ptr(v_pages), P, _ptr(page_table), page_table.shape[1],
                                _ptr(prefix_lens), int(max_prefix_len), _ptr(tree_mask), _ptr(tree_sizes), B, N,
                                Hq, Hkv, D,
                                float(sm_scale), _ptr(out), odt, _ptr(workspace), ws_bytes), "tv_attention")
    return out


def tv_tree_budget(concurrency: int, max_nodes: int = 64) -> int:
    """Node budget of a draft tree at this concurrency (-1 for bad arguments)."""
    return int(_load().tv_tree_budget(concurrency, max_nodes))


def tv_accept_workspace_bytes(B, N, V, mode=GREEDY) -> int:
    return int(_load().tv_accept_workspace_bytes(B, N, V, mode))


def tv_accept(target_logits: torch.Tensor, draft_tokens: torch.Tensor, parents: torch.Tensor, mode: int = GREEDY,
              draft_logits: Optional[torch.Tensor] = None, uniforms: Optional[torch.Tensor] = None,
              temperature: float = 1.0, outputs: Optional[dict] = None, want_argmax: bool = True,
              workspace: Optional[torch.Tensor] = None, tree_sizes: Optional[torch.Tensor] = None) -> dict:
    """Returns dict(accept_len [B], path [B][N], bonus [B], target_argmax [B][N] (greedy))."""
    B, N, V = target_logits.shape
    dev = target_logits.device
    assert target_logits.dtype == torch.float32 and draft_tokens.dtype == torch.int32 and parents.dtype == torch.int32
    if outputs is None:
        outputs = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
                       path=torch.empty((B, N), dtype=torch.int32, device=dev),
                       bonus=torch.empty(B, dtype=torch.int32, device=dev))
        if mode == GREEDY and want_argmax:
            outputs["target_argmax"] = torch.empty((B, N), dtype=torch.int32, device=dev)
    need = tv_accept_workspace_bytes(B, N, V, mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_load().tv_accept(_ctx(dev), _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(parents),
                             _ptr(tree_sizes), _ptr(uniforms), B, N, V, mode, float(temperature), _ptr(outputs["accept_len"]),
                             _ptr(outputs["path"]), _ptr(outputs["bonus"]), _ptr(outputs.get("target_argmax")),
                             _ptr(workspace), ws_bytes), "tv_accept")
    return outputs


def tv_commit(k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor, prefix_lens: torch.Tensor,
              max_prefix_len: int, draft_tokens: torch.Tensor, path: torch.Tensor, accept_len: torch.Tensor,
              bonus: torch.Tensor, outputs: Optional[dict] = None, want_emitted: bool = True) -> dict:
    """Moves the accepted path's K/V rows in place (k/v_pages bf16 [P][Hkv][16][D]).

    Returns dict(new_prefix_lens [B], emitted [B][N] (if wanted), next_root [B]);
    outputs must not overlap any input."""
    B, N = draft_tokens.shape
    P, Hkv, page, D = k_pages.shape
    assert page == 16 and v_pages.shape == k_pages.shape
    assert k_pages.dtype == torch.bfloat16 and v_pages.dtype == torch.bfloat16
    for t in (page_table, prefix_lens, draft_tokens, path, accept_len, bonus):
        assert t.dtype == torch.int32
    dev = k_pages.device
    if outputs is None:
        outputs = dict(new_prefix_lens=torch.empty(B, dtype=torch.int32, device=dev),
                       next_root=torch.empty(B, dtype=torch.int32, device=dev))
        if want_emitted:
            outputs["emitted"] = torch.empty((B, N), dtype=torch.int32, device=dev)
    _check(_load().tv_commit(_ctx(dev), _ptr(k_pages), _ptr(v_pages), P, _ptr(page_table), page_table.shape[1],
                             _ptr(prefix_lens), int(max_prefix_len), _ptr(draft_tokens), _ptr(path),
                             _ptr(accept_len), _ptr(bonus), B, N, Hkv, D, _ptr(outputs["new_prefix_lens"]),
                             _ptr(outputs.get("emitted")), _ptr(outputs["next_root"])), "tv_commit")
    return outputs


def tv_tau(device="cuda:0"):
    """(tau, cycles) since the last reset; synchronises the stream."""
    tau = ctypes.c_double()
    cycles = ctypes.c_uint64()
    _check(_load().tv_tau(_ctx(torch.device(device)), ctypes.byref(tau), ctypes.byref(cycles)), "tv_tau")
    return tau.value, cycles.value


def tv_tau_reset(device="cuda:0"):
    _check(_load().tv_tau_reset(_ctx(torch.device(device))), "tv_tau_reset")


def tv_device_error(device="cuda:0") -> int:
    code = ctypes.c_int32()
    _check(_load().tv_device_error(_ctx(torch.device(device)), ctypes.byref(code)), "tv_device_error")
    return code.value
