"""GPU check of tv_attention_noalloc, the attention entry point that
allocates nothing (its split partials live in the library's per-device
scratch): called through the C ABI, its output must equal tv_attention's
(same plan, same kernels) bit for bit, on two calls in a row, the second with
a smaller input, and a plan larger than the scratch is refused."""
import ctypes

import numpy as np
import pytest
import torch

import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, DevWorkload, host

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def c_noalloc(dw, mask, out):
    """The raw C ABI call (no binding-side checks)."""
    w = dw.w
    p = tv._ptr
    return tv.library().tv_attention_noalloc(tv._ctx(DEV), p(dw.q), p(dw.k), p(dw.v), w.num_pages, p(dw.page_table),
                                             w.page_table.shape[1], p(dw.prefix_lens), w.max_prefix_len, p(mask), None,
                                             w.B, w.N, w.Hq, w.Hkv, w.D, ctypes.c_float(float(w.sm_scale)), p(out),
                                             tv.F32)


def test_noalloc_matches_tv_attention_twice_second_smaller():
    # first: the 32K-context shape (eight key splits: 34 MB of partials in
    # the scratch); second: a smaller shape whose plan also splits keys, so
    # the second call reuses the scratch the first left behind
    cases = [tvgen.make_workload(4, with_logits=False),
             tvgen.make_workload(2, with_logits=False, overrides=dict(B=4, L=1000))]
    for k, w in enumerate(cases):
        need = tv.tv_attention_workspace_bytes(DEV, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
        print(f"[noalloc] call {k}: B={w.B} N={w.N} L={w.max_prefix_len}, plan needs {need} bytes", flush=True)
        assert 0 < need <= SCRATCH_BYTES
        dw = DevWorkload(w, logits=False)
        mask = tv.tv_build_mask(dw.parents)[0]
        ref = host(dw.attention(mask))
        out = torch.full((w.B, w.N, w.Hq, w.D), float("nan"), dtype=torch.float32, device=DEV)
        assert c_noalloc(dw, mask, out) == tv.OK
        torch.cuda.synchronize()
        assert tv.tv_device_error(DEV) == 0
        got = host(out)
        assert np.array_equal(got, ref), f"call {k}: max abs diff {np.nanmax(np.abs(got - ref)):.3e}"


def test_noalloc_refuses_a_plan_beyond_the_scratch():
    # a batch whose split partials exceed 64 MiB: refused before any launch,
    # the output untouched
    w = tvgen.make_workload(2, with_kv=False, with_logits=False, overrides=dict(B=64, N=128, L=60000))
    need = tv.tv_attention_workspace_bytes(DEV, w.B, w.N, w.Hq, w.Hkv, w.D, w.max_prefix_len)
    print(f"[noalloc] oversized plan needs {need} bytes", flush=True)
    if need <= SCRATCH_BYTES:
        pytest.skip("this device's plan fits the scratch")
    z = torch.zeros(16, dtype=torch.int32, device=DEV)
    out = torch.zeros(4, dtype=torch.float32, device=DEV)
    p = tv._ptr
    st = tv.library().tv_attention_noalloc(tv._ctx(DEV), p(z), p(z), p(z), 1, p(z), (w.max_prefix_len + w.N + 15) // 16,
                                           p(z), w.max_prefix_len, None, None, w.B, w.N, w.Hq, w.Hkv, w.D,
                                           ctypes.c_float(1.0), p(out), tv.F32)
    assert st == tv.WORKSPACE
    torch.cuda.synchronize()
    assert (host(out) == 0).all()
    assert tv.tv_device_error(DEV) == 0
