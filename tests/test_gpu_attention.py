"""GPU parity of the ring buffer and partitioned attention against the oracle.

Bars (written in each test): ring bytes bit-exact; fp32 attention max-abs
<= 1e-5; bf16 attention max|gpu - ref| / max|ref| <= 2e-2 per layer output.
The oracle attends over the chronological [pin; window; suffix] context in
float64; the kernels read the ring in physical slot order.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import full_attention
from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, host, lib, max_abs, rel_err  # noqa: E402

F32_ATOL = 1e-5
BF16_REL = 2e-2


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


# ------------------------------------------------------------------ ring ----

@pytest.mark.parametrize("shape,frames", [(configs.TINY, 10), (configs.PI05_1L, 5), (configs.LONG_18L, 10)])
def test_ring_bytes_bit_exact(shape, frames):
    _banner(f"ring bytes {shape.name} frames={frames}")
    sc = Scenario(shape)
    sc.check_bytes()
    for f in range(frames):
        sc.push(f)
        sc.check_bytes()


def test_ring_500_frames_wraps_and_counts():
    """500 pushes on the Pi0.5-like ring; frames are cheap device patterns."""
    _banner("ring 500 frames")
    s = configs.PI05_1L
    shp = (s.num_layers, s.tokens_per_frame, s.n_kv_heads, s.head_dim)
    base = np.arange(np.prod(shp), dtype=np.int64).reshape(shp)

    def frame(f):
        return ((base * 3 + f * 7919) % 65521).astype(np.uint16), ((base * 5 + f * 104729) % 65519).astype(np.uint16)

    sc = Scenario(s, frame_fn=frame)
    for f in range(500):
        ev = sc.push(f)
        assert ev == (f - s.num_slots if f >= s.num_slots else -1)
    sc.check_bytes()
    assert sc.ring.state() == {"head": 500 % s.num_slots, "count": s.num_slots, "pinned": s.pin_tokens,
                               "frames_pushed": 500}


def _unaligned(a: np.ndarray, shift: int) -> torch.Tensor:
    """A device view of `a` whose first element sits `shift` elements past a
    16-byte boundary (the frame copy then takes the 2-D copy path)."""
    t = dev(a).reshape(-1)
    buf = torch.empty(t.numel() + shift, dtype=t.dtype, device="cuda")
    buf[shift:].copy_(t)
    return buf[shift:].view(a.shape)


@pytest.mark.parametrize("shape", [configs.PI05_1L, configs.TINY], ids=lambda s: s.name)
def test_push_and_pin_from_unaligned_sources(shape):
    """Sources off a 16-byte boundary: ring bytes stay bit-exact (pin and
    pushes past a wrap), alternating with aligned pushes."""
    _banner(f"unaligned sources {shape.name}")
    sc = Scenario(shape, pin_tokens=0)
    if shape.pin_tokens:
        pk, pv = synth.pin_kv(shape)
        sc.ring.pin_prefix(_unaligned(pk, 1), _unaligned(pv, 1), shape.pin_tokens)
        sc.model.pin(sc._words(pk), sc._words(pv))
        sc.pin_k, sc.pin_v = pk, pv
        sc.check_bytes()
    for f in range(shape.num_slots + 3):
        k, v = sc.frame_fn(f)
        shift = f % 3          # 0: aligned (the kernel path), 1 and 2: not
        ev = sc.ring.push_frame(_unaligned(k, shift) if shift else dev(k), _unaligned(v, shift) if shift else dev(v))
        assert ev == sc.model.push(sc._words(k), sc._words(v))
        sc._enter(f, k, v)
        sc.check_bytes()


# ------------------------------------------------------------- attention ----

def test_attention_tiny_fp32_every_frame_and_step():
    s = configs.TINY
    _banner(f"attention {s.name}")
    sc = Scenario(s)
    worst = 0.0
    for f in range(s.frames):
        sc.push(f)
        for k in range(s.steps_per_frame):
            q, kd, vd = synth.suffix_qkv(s, f, k)
            for splits in (0, 1, 2, 3):
                out = sc.run_step(q, kd, vd, num_splits=splits)
                ref = sc.oracle_step(q, kd, vd, 0)
                worst = max(worst, max_abs(out[0], ref))
    _banner(f"tiny fp32 worst max-abs {worst:.3e}")
    assert worst <= F32_ATOL


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_attention_pi05_single_layer(splits):
    s = configs.PI05_1L
    _banner(f"attention {s.name} splits={splits}")
    sc = Scenario(s)
    worst = 0.0
    checked = {0: (0, 9), 1: (0,), 2: (5,), 7: (9,), 30: (0, 9)}
    for f in range(max(checked) + 1):
        sc.push(f)
        for k in checked.get(f, ()):
            q, kd, vd = synth.suffix_qkv(s, f, k)
            out = sc.run_step(q, kd, vd, num_splits=splits)
            worst = max(worst, rel_err(out[0], sc.oracle_step(q, kd, vd, 0)))
    _banner(f"pi05 1L worst rel {worst:.3e}")
    assert worst <= BF16_REL


def test_attention_long_history_18_layers_bench_launch():
    """Full long-history shape, default splits (the launch the benchmark times)."""
    s = configs.LONG_18L
    _banner(f"attention {s.name}")
    sc = Scenario(s)
    worst = 0.0
    for f in range(10):
        sc.push(f)
        if f in (0, 7, 9):               # partly filled, just full, wrapped once
            for k in (0, 9):
                q, kd, vd = synth.suffix_qkv(s, f, k)
                out = sc.run_step(q, kd, vd)
                for l in (0, 5, 17):
                    worst = max(worst, rel_err(out[l], sc.oracle_step(q, kd, vd, l)))
    _banner(f"long 18L worst rel {worst:.3e}")
    assert worst <= BF16_REL


@pytest.mark.parametrize("shape,q_layout", [(configs.LONG_18L, 0), (configs.LONG_18L, 1), (configs.PI05_1L, 0),
                                            (configs.PI05_1L, 1)])
def test_fp32_partials(shape, q_layout):
    """partials_f32 = 1 keeps the split partials' accumulator in FP32 between
    the per-split sum and the FP32 combine (the default rounds it to bf16).
    Both meet the bar; the FP32 form is at least as close to the oracle."""
    s = shape
    _banner(f"fp32 partials {s.name} q_layout={q_layout}")
    sc = Scenario(s)
    for f in range(s.num_slots + 1):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s, s.num_slots, 6)
    o16 = sc.run_step(q, kd, vd, q_layout=q_layout)
    o32 = sc.run_step(q, kd, vd, q_layout=q_layout, partials_f32=1)
    e16 = e32 = 0.0
    for l in sorted({0, s.num_layers // 2, s.num_layers - 1}):
        ref = sc.oracle_step(q, kd, vd, l)
        e16, e32 = max(e16, rel_err(o16[l], ref)), max(e32, rel_err(o32[l], ref))
    _banner(f"  rel err: bf16 partials {e16:.3e}, fp32 partials {e32:.3e}")
    assert e16 <= BF16_REL and e32 <= BF16_REL
    assert e32 <= e16 * 1.05
    assert not np.array_equal(o16, o32)           # the option really changes the partials


@pytest.mark.parametrize("splits,f32p", [(0, 0), (100, 0), (20, 1), (0, 1)])
def test_single_layer_long_history_many_splits(splits, f32p):
    """One layer of the long-history cache: the library picks ~50 splits, so
    the combine merges more partials than one batch of loads holds and
    splits each slice's merge over four waves (also with 100 splits, and
    FP32 partials past 8 splits)."""
    s = configs.LONG_18L.with_(name="lh_1L", cfg_id=48, num_layers=3)
    _banner(f"long-history single layer splits={splits} f32 partials={f32p}")
    sc = Scenario(s)
    for f in range(s.num_slots + 2):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s.with_(num_layers=1), 3, 2)
    out = sc.run_step(q, kd, vd, num_splits=splits, layer_begin=1, num_layers=1, partials_f32=f32p)
    ck, cv = sc.cached_context(1)
    ref = full_attention(synth.widen(q[0]), np.concatenate([ck, synth.widen(kd[0])]),
                         np.concatenate([cv, synth.widen(vd[0])]), s.scale)
    err = rel_err(out[0], ref)
    _banner(f"  rel {err:.3e}")
    assert err <= BF16_REL


@pytest.mark.parametrize("frames,splits,f32p", [(4, 22, 0), (4, 22, 1), (3, 10, 0)])
def test_single_layer_key_halves_ragged_splits(frames, splits, f32p):
    """A single layer of the long-history cache runs 128-row workgroups in
    two key halves that take alternate tiles and merge through LDS. These
    fills and split counts give every split an odd tile count (5 or 9: the
    halves walk 3 and 2, or 5 and 4 tiles) and leave a last split of 19 keys,
    one ragged tile, so that its second half sees no key at all."""
    s = configs.LONG_18L.with_(name="lh_1L", cfg_id=48, num_layers=3)
    total = s.pin_tokens + frames * s.tokens_per_frame + s.n_dyn
    chunk = -(-(-(-total // splits)) // 32) * 32
    parts = -(-total // chunk)
    assert chunk // 32 in (5, 9) and total - (parts - 1) * chunk == 19      # the shapes named above
    _banner(f"key halves: frames={frames} splits={splits} ({parts} parts of {chunk} keys) f32 partials={f32p}")
    sc = Scenario(s)
    for f in range(frames):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s.with_(num_layers=1), frames, 1)
    out = sc.run_step(q, kd, vd, num_splits=splits, layer_begin=1, num_layers=1, partials_f32=f32p)
    ck, cv = sc.cached_context(1)
    ref = full_attention(synth.widen(q[0]), np.concatenate([ck, synth.widen(kd[0])]),
                         np.concatenate([cv, synth.widen(vd[0])]), s.scale)
    err = rel_err(out[0], ref)
    _banner(f"  rel {err:.3e}")
    assert err <= BF16_REL


# (layers, splits, fp32 partials): split counts at the edges of the combine's
# choices on the long-history cache (6451 keys, where each count here is the
# number of parts the call makes). bf16 partials: a wave merges up to 8
# splits in a batch of 8, up to 16 in a batch of 16; past 16 two waves share
# a slice, past 32 four; 68 splits leave 17 per wave, a second batch with one
# real split. FP32 partials: batches of 8, two waves past 8, four past 16.
# One layer merges in quarter-slices (a small launch), three in whole blocks.
COMBINE_EDGES = [(1, 8, 0), (1, 9, 0), (1, 16, 0), (1, 17, 0), (1, 29, 0), (1, 34, 0), (1, 68, 0),
                 (3, 9, 0), (3, 17, 0), (3, 68, 0),
                 (1, 9, 1), (1, 16, 1), (1, 17, 1), (1, 34, 1), (3, 34, 1)]


@pytest.mark.parametrize("layers,splits,f32p", COMBINE_EDGES)
def test_combine_split_count_edges(layers, splits, f32p):
    s = configs.LONG_18L.with_(name="lh_3L", cfg_id=49, num_layers=3)
    _banner(f"combine edges: layers={layers} splits={splits} f32 partials={f32p}")
    sc = Scenario(s)
    for f in range(s.num_slots + 1):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s.with_(num_layers=layers), 1, 5)
    out = sc.run_step(q, kd, vd, num_splits=splits, layer_begin=3 - layers, num_layers=layers, partials_f32=f32p)
    worst = 0.0
    for i in range(layers):
        ck, cv = sc.cached_context(3 - layers + i)
        ref = full_attention(synth.widen(q[i]), np.concatenate([ck, synth.widen(kd[i])]),
                             np.concatenate([cv, synth.widen(vd[i])]), s.scale)
        worst = max(worst, rel_err(out[i], ref))
    _banner(f"  rel {worst:.3e}")
    assert worst <= BF16_REL


def test_attention_bf16_output_dtype():
    s = configs.PI05_1L
    sc = Scenario(s)
    for f in range(3):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s, 2, 4)
    out32 = sc.run_step(q, kd, vd)
    out16 = sc.run_step(q, kd, vd, out_dtype=lib().PA_BF16)
    ref = sc.oracle_step(q, kd, vd, 0)
    assert rel_err(out16[0], ref) <= BF16_REL
    # the bf16 output is the fp32 result rounded once
    assert np.max(np.abs(out16 - out32)) <= np.max(np.abs(out32)) * 2 ** -8


EDGE = [
    # (D, Hq, Hkv, P, pinned, W, F, N, frames, splits)
    (64, 1, 1, 0, 0, 3, 5, 1, 4, 0),          # no pin, a single suffix token
    (128, 4, 2, 7, 3, 2, 33, 5, 3, 0),         # grouped heads, pin gap, ragged tiles
    (256, 8, 1, 1, 1, 1, 1, 51, 2, 0),         # one-token window, one-slot ring
    (256, 2, 1, 40, 40, 4, 100, 3, 9, 7),      # ragged split tails
    (64, 6, 3, 5, 5, 5, 7, 17, 1, 3),          # one frame only (partly filled ring)
    (128, 8, 1, 300, 300, 2, 64, 51, 0, 0),    # nothing pushed yet: pin + suffix only
]


@pytest.mark.parametrize("D,hq,hkv,P,pinned,W,F,N,frames,splits", EDGE)
def test_attention_edge_cases(D, hq, hkv, P, pinned, W, F, N, frames, splits):
    _banner(f"edge D={D} hq={hq} hkv={hkv} P={P}/{pinned} W={W} F={F} N={N} frames={frames} splits={splits}")
    s = configs.PI05_1L.with_(name="edge", cfg_id=40 + D + hq, num_layers=2, n_q_heads=hq, n_kv_heads=hkv,
                              head_dim=D, pin_tokens=P, num_slots=W, tokens_per_frame=F, n_dyn=N,
                              scale=1 / math.sqrt(D))
    sc = Scenario(s, pin_tokens=pinned)
    for f in range(frames):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s, frames, 3)
    out = sc.run_step(q, kd, vd, num_splits=splits)
    for l in range(2):
        assert rel_err(out[l], sc.oracle_step(q, kd, vd, l)) <= BF16_REL


def test_attention_layer_subrange():
    s = configs.LONG_18L.with_(name="sub", cfg_id=47, num_layers=4, num_slots=2, tokens_per_frame=96)
    sc = Scenario(s)
    for f in range(3):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s.with_(num_layers=2), 3, 1)
    out = sc.run_step(q, kd, vd, layer_begin=2, num_layers=2)
    for lb in range(2):
        ck, cv = sc.cached_context(2 + lb)
        ref = full_attention(synth.widen(q[lb]), np.concatenate([ck, synth.widen(kd[lb])]),
                             np.concatenate([cv, synth.widen(vd[lb])]), s.scale)
        assert rel_err(out[lb], ref) <= BF16_REL


def test_naive_cache_fails_parity():
    """Negative control (Table 4 of the Reflex review: the naive cache is wrong):
    reusing step 0's suffix K/V at step 9 must miss the oracle by far more than the bar."""
    s = configs.PI05_1L
    sc = Scenario(s)
    for f in range(2):
        sc.push(f)
    q9, kd9, vd9 = synth.suffix_qkv(s, 1, 9)
    _, kd0, vd0 = synth.suffix_qkv(s, 1, 0)
    ref = sc.oracle_step(q9, kd9, vd9, 0)
    good = sc.run_step(q9, kd9, vd9)
    naive = sc.run_step(q9, kd0, vd0)
    assert rel_err(good[0], ref) <= BF16_REL
    assert rel_err(naive[0], ref) > 5 * BF16_REL


def test_repeat_calls_are_deterministic():
    s = configs.PI05_1L
    sc = Scenario(s)
    sc.push(0)
    q, kd, vd = synth.suffix_qkv(s, 0, 0)
    a = sc.run_step(q, kd, vd)
    b = sc.run_step(q, kd, vd)
    assert np.array_equal(a, b)
