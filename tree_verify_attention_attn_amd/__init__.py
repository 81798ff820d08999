"""Python binding of libtreeverify (tree-verify attention and acceptance on MI355X).

Argument marshalling only: every step of the verification pass runs in the
HIP kernels of ``libtreeverify.so``. torch supplies device memory and the
current HIP stream. Functions carry the C ABI's names (see
``include/treeverify.h``); each takes torch tensors on one GPU and raises
``TVError`` on a non-OK status. There is no CPU fallback: if the library is
not built, or no GPU is present, calls fail loudly.
"""
from __future__ import annotations

import atexit
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
_bound = {}  # device index -> stream handle the context is bound to


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
        lib.tv_attention_noalloc.argtypes = [vp, vp, vp, vp, i64, vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                             f32, vp, ctypes.c_int]
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
        for f in ("tv_create", "tv_destroy", "tv_set_stream", "tv_build_mask", "tv_attention", "tv_attention_noalloc",
                  "tv_accept",
                  "tv_commit", "tv_build_tree", "tv_tau", "tv_tau_reset", "tv_device_error"):
            getattr(lib, f).restype = st
        _lib = lib
    return _lib


def _teardown():
    """Destroys every context at interpreter exit, while the HIP runtime is
    still fully alive: each context's stream is synchronised, then its device
    counters and event are released by tv_destroy. Without it they are left
    to the runtime's own exit-time destructors."""
    if _lib is None:
        return
    for idx, h in list(_ctxs.items()):
        _lib.tv_destroy(h)
    _ctxs.clear()
    _bound.clear()


def library() -> ctypes.CDLL:
    """The loaded libtreeverify (raises if it is not built)."""
    return _load()


# the current stream's raw handle: torch's own fast accessor where it exists
# (about 0.1 us), else the public one, which builds a Stream object (about 1 us)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream(idx: int) -> int:
    if _raw_stream is not None:
        return _raw_stream(idx)
    return torch.cuda.current_stream(idx).cuda_stream


def _ctx(device: torch.device):
    """Per-device context, rebound to torch's current stream on every call."""
    if device.type != "cuda":
        raise ValueError("libtreeverify runs on a GPU: pass tensors on a cuda (HIP) device")
    idx = device.index if device.index is not None else torch.cuda.current_device()
    lib = _load()
    if idx not in _ctxs:
        h = ctypes.c_void_p()
        st0 = _current_stream(idx)
        s = lib.tv_create(ctypes.byref(h), idx, ctypes.c_void_p(st0))
        if s != OK:
            raise TVError(s, "tv_create")
        if not _ctxs:
            atexit.register(_teardown)
        _ctxs[idx] = h
        _bound[idx] = st0
    h = _ctxs[idx]
    st = _current_stream(idx)
    if _bound.get(idx) != st:  # rebinding orders the new stream after the old one's queued work
        s = lib.tv_set_stream(h, ctypes.c_void_p(st))
        if s != OK:
            raise TVError(s, "tv_set_stream")
        _bound[idx] = st
    return h


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _arg(t, name: str, dtype: torch.dtype, shape: tuple, dev: torch.device, optional: bool = False):
    """Checks a tensor argument before its pointer reaches the library: a
    contiguous tensor of this dtype and shape (None matches any extent) on the
    call's GPU. A host tensor or another device's would be read by the kernels
    at a meaningless address. The common case costs about a microsecond; the
    message is built only on failure."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    try:
        ok = t.dtype is dtype and t.get_device() == dev.index and t.is_contiguous()
        shp = t.shape
    except AttributeError:
        raise TypeError(f"{name} must be a torch.Tensor") from None
    if ok and len(shp) == len(shape):
        for e, x in zip(shape, shp):
            if e is not None and x != e:
                break
        else:
            return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    want = "[" + ", ".join("*" if e is None else str(e) for e in shape) + "]"
    raise ValueError(f"{name} has shape {list(t.shape)}, expected {want}")


def _device_of(t: torch.Tensor, name: str) -> torch.device:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, not {t.device}")
    return t.device if t.device.index is not None else torch.device("cuda", torch.cuda.current_device())


def _p(t: Optional[torch.Tensor]):
    """Pointer of a tensor that _arg has already checked."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(s: int, what: str):
    if s != OK:
        raise TVError(s, what)


def tv_build_mask(parents: torch.Tensor, mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
                  tree_sizes: Optional[torch.Tensor] = None):
    """parents int32 [B][N] (N <= 128), tree_sizes int32 [B] or None ->
    (mask uint64-as-int64 [B][N][ceil(N/64)], depth int32 [B][N])."""
    dev = _device_of(parents, "parents")
    if parents.dim() != 2:
        raise ValueError("parents must be [B][N]")
    B, N = parents.shape
    W = max((N + 63) // 64, 1)
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    _arg(parents, "parents", torch.int32, (B, N), dev)
    _arg(tree_sizes, "tree_sizes", torch.int32, (B,), dev, optional=True)
    _arg(mask, "mask", torch.int64, (B, N, W), dev)
    _arg(depth, "depth", torch.int32, (B, N), dev, optional=True)
    _check(_load().tv_build_mask(_ctx(dev), _p(parents), _p(tree_sizes), B, N, _p(mask), _p(depth)),
           "tv_build_mask")
    return mask, depth


def tv_build_tree(root_tokens: torch.Tensor, cand_tokens: torch.Tensor, cand_probs: torch.Tensor, k_root: int,
                  threshold: float, max_depth: int, outputs: Optional[dict] = None) -> dict:
    """root_tokens int32 [B]; cand_tokens int32 / cand_probs fp32 [B][N][k] ->
    dict(parents, tokens, depth [B][N] int32, mask int64 [B][N][W], scores fp64 [B][N], n_nodes [B])."""
    dev = _device_of(cand_tokens, "cand_tokens")
    if cand_tokens.dim() != 3:
        raise ValueError("cand_tokens must be [B][N][k]")
    B, N, k = cand_tokens.shape
    _arg(cand_tokens, "cand_tokens", torch.int32, (B, N, k), dev)
    _arg(cand_probs, "cand_probs", torch.float32, (B, N, k), dev)
    _arg(root_tokens, "root_tokens", torch.int32, (B,), dev)
    if outputs is None:
        outputs = dict(parents=torch.empty((B, N), dtype=torch.int32, device=dev),
                       tokens=torch.empty((B, N), dtype=torch.int32, device=dev),
                       depth=torch.empty((B, N), dtype=torch.int32, device=dev),
                       mask=torch.empty((B, N, (N + 63) // 64), dtype=torch.int64, device=dev),
                       scores=torch.empty((B, N), dtype=torch.float64, device=dev),
                       n_nodes=torch.empty(B, dtype=torch.int32, device=dev))
    o = outputs
    W = (N + 63) // 64
    _arg(o.get("parents"), "outputs['parents']", torch.int32, (B, N), dev)
    _arg(o.get("tokens"), "outputs['tokens']", torch.int32, (B, N), dev)
    _arg(o.get("depth"), "outputs['depth']", torch.int32, (B, N), dev, optional=True)
    _arg(o.get("mask"), "outputs['mask']", torch.int64, (B, N, W), dev, optional=True)
    _arg(o.get("scores"), "outputs['scores']", torch.float64, (B, N), dev, optional=True)
    _arg(o.get("n_nodes"), "outputs['n_nodes']", torch.int32, (B,), dev, optional=True)
    _check(_load().tv_build_tree(_ctx(dev), _p(root_tokens), _p(cand_tokens), _p(cand_probs), B, N, k, k_root,
                                 float(threshold), max_depth, _p(o["parents"]), _p(o["tokens"]),
                                 _p(o.get("depth")), _p(o.get("mask")), _p(o.get("scores")),
                                 _p(o.get("n_nodes"))), "tv_build_tree")
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
    dev = _device_of(q, "q")
    if q.dim() != 4 or not isinstance(k_pages, torch.Tensor) or k_pages.dim() != 4:
        raise ValueError("q must be [B][N][Hq][D] and k_pages [P][Hkv][16][D]")
    B, N, Hq, D = q.shape
    P, Hkv = k_pages.shape[0], k_pages.shape[1]
    _arg(q, "q", torch.bfloat16, (B, N, Hq, D), dev)
    _arg(k_pages, "k_pages", torch.bfloat16, (P, Hkv, 16, D), dev)
    _arg(v_pages, "v_pages", torch.bfloat16, (P, Hkv, 16, D), dev)
    _arg(page_table, "page_table", torch.int32, (None, None), dev)
    if page_table.shape[0] < B:  # rows past B (a larger table) are never read
        raise ValueError(f"page_table has {page_table.shape[0]} rows, fewer than the batch's {B}")
    _arg(prefix_lens, "prefix_lens", torch.int32, (B,), dev)
    _arg(tree_mask, "tree_mask", torch.int64, (B, N, max((N + 63) // 64, 1)), dev, optional=True)
    _arg(tree_sizes, "tree_sizes", torch.int32, (B,), dev, optional=True)
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=out_dtype, device=dev)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be a float32 or bfloat16 tensor")
    _arg(out, "out", out.dtype, (B, N, Hq, D), dev)
    _arg(workspace, "workspace", torch.uint8, (None,), dev, optional=True)
    odt = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    h = _ctx(dev)
    if workspace is None:  # a given workspace's size is checked by the library
        need = int(_load().tv_attention_workspace_bytes(h, B, N, Hq, Hkv, D, max_prefix_len))
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_load().tv_attention(h, _p(q), _p(k_pages), _p(v_pages), P, _p(page_table), page_table.shape[1],
                                _p(prefix_lens), int(max_prefix_len), _p(tree_mask), _p(tree_sizes), B, N,
                                Hq, Hkv, D,
                                float(sm_scale), _p(out), odt, _p(workspace), ws_bytes), "tv_attention")
    return out


def tv_attention_noalloc(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor,
                         prefix_lens: torch.Tensor, max_prefix_len: int, tree_mask: Optional[torch.Tensor],
                         sm_scale: float, out: torch.Tensor, tree_sizes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """tv_attention without a workspace and without any allocation: the
    library's per-device scratch (TV_NOALLOC_SCRATCH_BYTES) holds the plan's
    partials. `out` must be given. Calls that overlap on one GPU race on the
    scratch."""
    dev = _device_of(q, "q")
    if q.dim() != 4 or not isinstance(k_pages, torch.Tensor) or k_pages.dim() != 4:
        raise ValueError("q must be [B][N][Hq][D] and k_pages [P][Hkv][16][D]")
    B, N, Hq, D = q.shape
    P, Hkv = k_pages.shape[0], k_pages.shape[1]
    _arg(q, "q", torch.bfloat16, (B, N, Hq, D), dev)
    _arg(k_pages, "k_pages", torch.bfloat16, (P, Hkv, 16, D), dev)
    _arg(v_pages, "v_pages", torch.bfloat16, (P, Hkv, 16, D), dev)
    _arg(page_table, "page_table", torch.int32, (None, None), dev)
    if page_table.shape[0] < B:
        raise ValueError(f"page_table has {page_table.shape[0]} rows, fewer than the batch's {B}")
    _arg(prefix_lens, "prefix_lens", torch.int32, (B,), dev)
    _arg(tree_mask, "tree_mask", torch.int64, (B, N, max((N + 63) // 64, 1)), dev, optional=True)
    _arg(tree_sizes, "tree_sizes", torch.int32, (B,), dev, optional=True)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be a float32 or bfloat16 tensor")
    _arg(out, "out", out.dtype, (B, N, Hq, D), dev)
    odt = {torch.float32: F32, torch.bfloat16: BF16}[out.dtype]
    _check(_load().tv_attention_noalloc(_ctx(dev), _p(q), _p(k_pages), _p(v_pages), P, _p(page_table),
                                        page_table.shape[1], _p(prefix_lens), int(max_prefix_len), _p(tree_mask),
                                        _p(tree_sizes), B, N, Hq, Hkv, D, float(sm_scale), _p(out), odt),
           "tv_attention_noalloc")
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
    dev = _device_of(target_logits, "target_logits")
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B][N][V]")
    B, N, V = target_logits.shape
    _arg(target_logits, "target_logits", torch.float32, (B, N, V), dev)
    _arg(draft_tokens, "draft_tokens", torch.int32, (B, N), dev)
    _arg(parents, "parents", torch.int32, (B, N), dev)
    _arg(draft_logits, "draft_logits", torch.float32, (B, N, V), dev, optional=True)
    _arg(uniforms, "uniforms", torch.float32, (B, N), dev, optional=True)
    _arg(tree_sizes, "tree_sizes", torch.int32, (B,), dev, optional=True)
    if outputs is None:
        outputs = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
                       path=torch.empty((B, N), dtype=torch.int32, device=dev),
                       bonus=torch.empty(B, dtype=torch.int32, device=dev))
        if mode == GREEDY and want_argmax:
            outputs["target_argmax"] = torch.empty((B, N), dtype=torch.int32, device=dev)
    _arg(outputs.get("accept_len"), "outputs['accept_len']", torch.int32, (B,), dev)
    _arg(outputs.get("path"), "outputs['path']", torch.int32, (B, N), dev)
    _arg(outputs.get("bonus"), "outputs['bonus']", torch.int32, (B,), dev)
    _arg(outputs.get("target_argmax"), "outputs['target_argmax']", torch.int32, (B, N), dev, optional=True)
    if workspace is None:  # a given workspace's size is checked by the library
        workspace = torch.empty(max(tv_accept_workspace_bytes(B, N, V, mode), 1), dtype=torch.uint8, device=dev)
    _arg(workspace, "workspace", torch.uint8, (None,), dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_load().tv_accept(_ctx(dev), _p(target_logits), _p(draft_logits), _p(draft_tokens), _p(parents),
                             _p(tree_sizes), _p(uniforms), B, N, V, mode, float(temperature), _p(outputs["accept_len"]),
                             _p(outputs["path"]), _p(outputs["bonus"]), _p(outputs.get("target_argmax")),
                             _p(workspace), ws_bytes), "tv_accept")
    return outputs


def tv_commit(k_pages: torch.Tensor, v_pages: torch.Tensor, page_table: torch.Tensor, prefix_lens: torch.Tensor,
              max_prefix_len: int, draft_tokens: torch.Tensor, path: torch.Tensor, accept_len: torch.Tensor,
              bonus: torch.Tensor, outputs: Optional[dict] = None, want_emitted: bool = True) -> dict:
    """Moves the accepted path's K/V rows in place (k/v_pages bf16 [P][Hkv][16][D]).

    Returns dict(new_prefix_lens [B], emitted [B][N] (if wanted), next_root [B]);
    outputs must not overlap any input."""
    dev = _device_of(k_pages, "k_pages")
    if k_pages.dim() != 4 or not isinstance(draft_tokens, torch.Tensor) or draft_tokens.dim() != 2:
        raise ValueError("k_pages must be [P][Hkv][16][D] and draft_tokens [B][N]")
    B, N = draft_tokens.shape
    P, Hkv, D = k_pages.shape[0], k_pages.shape[1], k_pages.shape[3]
    _arg(k_pages, "k_pages", torch.bfloat16, (P, Hkv, 16, D), dev)
    _arg(v_pages, "v_pages", torch.bfloat16, (P, Hkv, 16, D), dev)
    _arg(page_table, "page_table", torch.int32, (None, None), dev)
    if page_table.shape[0] < B:  # rows past B (a larger table) are never read
        raise ValueError(f"page_table has {page_table.shape[0]} rows, fewer than the batch's {B}")
    _arg(prefix_lens, "prefix_lens", torch.int32, (B,), dev)
    _arg(draft_tokens, "draft_tokens", torch.int32, (B, N), dev)
    _arg(path, "path", torch.int32, (B, N), dev)
    _arg(accept_len, "accept_len", torch.int32, (B,), dev)
    _arg(bonus, "bonus", torch.int32, (B,), dev)
    if outputs is None:
        outputs = dict(new_prefix_lens=torch.empty(B, dtype=torch.int32, device=dev),
                       next_root=torch.empty(B, dtype=torch.int32, device=dev))
        if want_emitted:
            outputs["emitted"] = torch.empty((B, N), dtype=torch.int32, device=dev)
    _arg(outputs.get("new_prefix_lens"), "outputs['new_prefix_lens']", torch.int32, (B,), dev)
    _arg(outputs.get("next_root"), "outputs['next_root']", torch.int32, (B,), dev)
    _arg(outputs.get("emitted"), "outputs['emitted']", torch.int32, (B, N), dev, optional=True)
    _check(_load().tv_commit(_ctx(dev), _p(k_pages), _p(v_pages), P, _p(page_table), page_table.shape[1],
                             _p(prefix_lens), int(max_prefix_len), _p(draft_tokens), _p(path),
                             _p(accept_len), _p(bonus), B, N, Hkv, D, _p(outputs["new_prefix_lens"]),
                             _p(outputs.get("emitted")), _p(outputs["next_root"])), "tv_commit")
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
