"""GPU parity: tv_build_mask against the oracle, bit-exact (masks and depths)."""
import numpy as np
import pytest

import oracle
import tvgen
import tree_verify_attention_attn_amd as tv
from gpu_util import DEV, dev, host, mask_np

pytestmark = pytest.mark.gpu


def trees():
    out = []
    for cfg in (1, 2, 3, 4, 5):
        w = tvgen.make_workload(cfg, with_kv=False, with_logits=False)
        out.append((f"cfg{cfg}", w.parents))
    N = 64
    out.append(("chain64", tvgen.chain_tree(N)[None]))
    out.append(("star64", tvgen.star_tree(N)[None]))
    out.append(("forest64", tvgen.forest_tree(N)[None]))
    out.append(("single", np.array([[-1]], np.int32)))
    out.append(("random-many", np.stack([tvgen.random_tree(9, b, 37, 6) for b in range(300)])))
    return out


@pytest.mark.parametrize("name,parents", trees(), ids=[t[0] for t in trees()])
def test_mask_bit_exact(name, parents):
    print(f"[mask] {name} B={parents.shape[0]} N={parents.shape[1]}", flush=True)
    m, d = tv.tv_build_mask(dev(parents))
    om, od = oracle.build_mask(parents)
    assert (mask_np(m) == om).all()
    assert (host(d) == od).all()
    assert tv.tv_device_error(DEV) == 0


def test_empty_is_a_no_op():
    p = dev(np.zeros((0, 5), np.int32))
    m, d = tv.tv_build_mask(p)
    assert m.numel() == 0
    assert tv.tv_device_error(DEV) == 0


def test_bad_parent_sets_device_error():
    parents = np.stack([tvgen.chain_tree(8), tvgen.chain_tree(8)])
    parents[1, 5] = 6  # parent after child
    st, _, _ = oracle.status_build_mask(parents)
    m, d = tv.tv_build_mask(dev(parents))
    assert tv.tv_device_error(DEV) == st == oracle.INVALID_TREE
    assert (mask_np(m)[1] == 0).all() and (host(d)[1] == -1).all()
    om, od = oracle.build_mask(parents[:1])
    assert (mask_np(m)[:1] == om).all()


def test_host_detected_errors():
    with pytest.raises(tv.TVError) as e:
        tv.tv_build_mask(dev(np.full((1, 129), -1, np.int32)))
    assert e.value.status == tv.UNSUPPORTED
