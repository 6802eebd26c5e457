"""GPU checks of asynchronous pushes through a spare slot (rb_stage_frame /
rb_commit_frame).

Reflex review, system architecture (Figure 3): the vision thread pushes new
frames into the shared cache while the policy thread denoises from it. Here
the producer stages frame f+1 on its own stream while the consumer's steps
of frame f run; the commit makes the staged frame visible to later steps.
Bars: ring bytes bit-exact against the oracle's model; attention against the
oracle (fp32 max-abs 1e-5, bf16 2e-2 relative); the overlapped run
bit-identical to the same frames pushed synchronously.
"""

import numpy as np
import pytest
import torch

from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, lib, max_abs, rel_err  # noqa: E402


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("shape", [configs.TINY, configs.PI05_1L])
def test_spare_slot_ring_bytes_and_attention(shape):
    _banner(f"spare slot ring {shape.name}")
    sc = Scenario(shape, spare_slots=1)
    producer = torch.cuda.Stream()
    consumer = torch.cuda.current_stream()
    W = shape.num_slots
    q, kd, vd = synth.suffix_qkv(shape, 0, 1)
    for f in range(2 * (W + 1) + 1):
        sc.stage(f, producer)
        sc.commit(consumer)
        sc.check_bytes()
        assert sc.ring.state()["head"] == (f + 1) % (W + 1)
        if f % 2 == 0 or f >= W:
            got = sc.run_step(q, kd, vd)
            for layer in range(shape.num_layers):
                ref = sc.oracle_step(q, kd, vd, layer)
                if shape.dtype == "f32":
                    assert max_abs(got[layer], ref) <= 1e-5
                else:
                    assert rel_err(got[layer], ref) <= 2e-2


def test_overlapped_pushes_match_synchronous_pushes():
    s = configs.PI05_1L
    _banner("overlapped stage/commit vs synchronous push, pi05_1L, 6 frames x 10 steps")
    L = lib()
    n_frames, steps = 6, s.steps_per_frame
    frames = [tuple(dev(a) for a in synth.frame_kv(s, f)) for f in range(n_frames + 1)]
    qkv = [tuple(dev(a) for a in synth.suffix_qkv(s, 0, k)) for k in range(steps)]
    a_sc, b_sc = Scenario(s, spare_slots=1), Scenario(s, spare_slots=1)
    args = L.pattn_args(0, s.num_layers, s.n_q_heads, s.n_dyn, s.scale, L.PA_BF16, 0)
    wsb = L.pattn_workspace_bytes(a_sc.ring, args)
    producer, consumer = torch.cuda.Stream(), torch.cuda.current_stream()
    ws_a = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    shape = (s.num_layers, s.n_dyn, s.n_q_heads, s.head_dim)
    out_a = [torch.empty(shape, dtype=torch.int16, device="cuda") for _ in range(n_frames * steps)]
    out_b = [torch.empty(shape, dtype=torch.int16, device="cuda") for _ in range(n_frames * steps)]
    torch.cuda.synchronize()
    # A: frame f+1 is staged on the producer stream while frame f's steps run
    a_sc.ring.stage_frame(*frames[0], producer)
    a_sc.ring.commit_frame(consumer)
    for f in range(n_frames):
        a_sc.ring.stage_frame(*frames[f + 1], producer)
        for k in range(steps):
            L.pattn_step(a_sc.ring, args, *qkv[k], out_a[f * steps + k], ws_a, wsb, consumer)
        a_sc.ring.commit_frame(consumer)
    # B: the same frames pushed synchronously on one stream
    b_sc.ring.push_frame(*frames[0], consumer)
    for f in range(n_frames):
        for k in range(steps):
            L.pattn_step(b_sc.ring, args, *qkv[k], out_b[f * steps + k], ws_b, wsb, consumer)
        b_sc.ring.push_frame(*frames[f + 1], consumer)
    torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(out_a, out_b)):
        assert torch.equal(x, y), f"step {i}: overlapped result differs from the synchronous one"
    assert torch.equal(a_sc.k_buf, b_sc.k_buf) and torch.equal(a_sc.v_buf, b_sc.v_buf)
    assert a_sc.ring.state() == b_sc.ring.state()
