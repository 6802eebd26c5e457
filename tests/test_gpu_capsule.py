"""GPU parity of ring capsules (rb_snapshot / rb_restore) against the ring oracle.

FlashRT article (PaperDaily), the section on what a capsule is and Fig. 2:
snapshot freezes the live buffer set, restore copies it back and rebinds the
metadata, fork restores one capsule into several sessions, rollback restores
an earlier capsule. Bars: capsule and ring bytes bit-exact against the
oracle's model; attention after a restore bit-identical to attention at the
snapshot (same kernels, same inputs).
"""

import numpy as np
import pytest
import torch

from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, host, lib, tdtype  # noqa: E402


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


def _capsule_words(cap_t, s):
    a = host(cap_t)
    return a.view(np.uint32) if s.dtype == "f32" else a


def _model_capsule_flat(model):
    c = model.capsule()
    return np.concatenate([c["k"].reshape(-1), c["v"].reshape(-1)]), c


def _alloc_capsule(ring, s, where="cuda"):
    nb = ring.capsule_bytes()
    n = nb // (4 if s.dtype == "f32" else 2)
    if where == "host":
        return torch.empty(max(n, 1), dtype=tdtype(s.dtype), pin_memory=True)
    return torch.empty(max(n, 1), dtype=tdtype(s.dtype), device="cuda")


@pytest.mark.parametrize("shape,t,more", [(configs.TINY, 3, 6), (configs.PI05_1L, 1, 3), (configs.TINY, 9, 2)])
def test_snapshot_then_rollback_is_bit_exact(shape, t, more):
    _banner(f"capsule rollback {shape.name} t={t} more={more}")
    sc = Scenario(shape)
    for f in range(t):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(shape, 0, 0)
    out_at_t = sc.run_step(q, kd, vd)
    cap = _alloc_capsule(sc.ring, shape)
    st = sc.ring.snapshot(cap, capsule_bytes=sc.ring.capsule_bytes())
    torch.cuda.synchronize()
    flat, mcap = _model_capsule_flat(sc.model)
    assert st == mcap["state"]
    assert np.array_equal(_capsule_words(cap, shape)[:flat.size], flat), "capsule bytes differ from the oracle's"
    window_at_t = list(sc.window)
    for f in range(t, t + more):              # move on (wrapping), then roll back
        sc.push(100 + f)
    sc.ring.restore(cap, st)
    sc.model.restore(mcap)
    sc.window = window_at_t
    sc.check_bytes()
    out_back = sc.run_step(q, kd, vd)
    assert np.array_equal(out_back, out_at_t), "attention after rollback differs from attention at the snapshot"


def test_fork_into_fresh_rings_and_host_capsule():
    s = configs.PI05_1L
    _banner("capsule fork pi05_1L, host-memory capsule")

    src = Scenario(s)
    for f in range(3):
        src.push(f)
    q, kd, vd = synth.suffix_qkv(s, 0, 2)
    ref = src.run_step(q, kd, vd)
    cap = _alloc_capsule(src.ring, s, where="host")
    st = src.ring.snapshot(cap)
    torch.cuda.synchronize()
    forks = []
    for i in range(2):
        fk = Scenario(s, pin_tokens=0)         # an unpinned ring of the same config
        fk.ring.restore(cap, st)
        fk.model.restore(src.model.capsule())
        fk.pin_k, fk.pin_v, fk.window = src.pin_k, src.pin_v, list(src.window)
        fk.check_bytes()
        assert np.array_equal(fk.run_step(q, kd, vd), ref)
        forks.append(fk)
    # the sessions are independent: different pushes, different results; the source is untouched
    forks[0].push(500)
    forks[1].push(501)
    a, b = forks[0].run_step(q, kd, vd), forks[1].run_step(q, kd, vd)
    assert not np.array_equal(a, b)
    for fk in forks:
        fk.check_bytes()
    src.check_bytes()
    assert np.array_equal(src.run_step(q, kd, vd), ref)

