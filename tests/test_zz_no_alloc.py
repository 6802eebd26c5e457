"""pattn_step_noalloc: the attention step with its split partials in the
library's fixed device scratch instead of a caller workspace. Its results
must equal pattn_step's bit for bit (the same kernels and plan), on two
calls in a row, the second smaller than the first, so a stale partial left
by the first would show."""

import numpy as np
import pytest
import torch

from partitioned_kv_cache_amd import configs, synth


def _fake(n):
    return 0x1000 * n                      # never dereferenced: the calls fail validation first


def test_noalloc_rejects_calls_beyond_its_scratch():
    from partitioned_kv_cache_amd import _lib as L
    s = configs.LONG_18L
    r = L.Ring(L.rb_config(s.num_layers, 1, s.head_dim, s.pin_tokens, s.num_slots, s.tokens_per_frame, L.PA_BF16),
               _fake(1), _fake(2))
    big = L.pattn_args(0, s.num_layers, s.n_q_heads, s.n_dyn, s.scale, L.PA_BF16, 16)
    assert L.pattn_workspace_bytes(r, big) > L.pattn_noalloc_scratch_bytes()
    with pytest.raises(L.PattnError) as e:
        L.pattn_step_noalloc(r, big, _fake(3), _fake(4), _fake(5), _fake(6), stream=0)
    assert e.value.status == L.PA_ERANGE and "scratch" in str(e.value)
    r.close()


@pytest.mark.gpu
def test_noalloc_matches_pattn_step_on_two_calls_in_a_row():
    from tests.gpu_helpers import Scenario, dev, lib
    L = lib()
    torch.cuda.synchronize()
    cases = [configs.LONG_18L, configs.PI05_1L]          # the second call is the smaller one
    for s in cases:
        print(f"[gpu] noalloc vs pattn_step: {s.name}", flush=True)
        sc = Scenario(s)
        for f in range(s.num_slots):
            sc.push(f)
        q, kd, vd = (dev(a) for a in synth.suffix_qkv(s, 1, 4))
        args = L.pattn_args(0, s.num_layers, s.n_q_heads, s.n_dyn, s.scale, L.PA_F32, 0)
        wsb = L.pattn_workspace_bytes(sc.ring, args)
        assert wsb <= L.pattn_noalloc_scratch_bytes()
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        shape = (s.num_layers, s.n_dyn, s.n_q_heads, s.head_dim)
        want = torch.empty(shape, dtype=torch.float32, device="cuda")
        got = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        L.pattn_step(sc.ring, args, q, kd, vd, want, ws, wsb)
        L.pattn_step_noalloc(sc.ring, args, q, kd, vd, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{s.name}: pattn_step_noalloc differs from pattn_step"
        assert bool(torch.isfinite(got).all())
        sc.ring.close()
