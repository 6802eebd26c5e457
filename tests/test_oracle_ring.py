"""Pins of the ring model: a deque FIFO, the slot closed form, byte contents.

Reference: the Reflex paper review, §3 Architecture (pinned prefix + FIFO
window: enqueue the newest frame, evict the oldest) and §5 Code analysis
(zeroed static buffers with a write pointer).
"""

from collections import deque

import numpy as np
import pytest

from oracle.ring import RingModel


def _frame(L, F, H, D, f, salt):
    """Frame f's words: every element encodes (frame, salt) so bytes identify it."""
    return np.full((L, F, H, D), (f * 2 + salt) % 65000 + 1, dtype=np.uint16)


@pytest.mark.parametrize("L,P,W,F", [(1, 16, 4, 16), (3, 5, 2, 7), (2, 0, 1, 3), (18, 256, 8, 4)])
def test_fifo_against_deque_and_closed_form(L, P, W, F):
    H, D = 1, 2
    ring = RingModel(L, H, D, P, W, F)
    fifo = deque(maxlen=W)
    for f in range(3 * W + 2):
        ev = ring.push(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1))
        evicted_by_deque = fifo[0] if len(fifo) == W else -1
        fifo.append(f)
        assert ev == evicted_by_deque == (f - W if f >= W else -1)
        assert ring.window_frames() == list(fifo)
        assert ring.count == min(f + 1, W) == len(fifo)
        assert ring.head == (f + 1) % W
        # every frame in the window sits in slot f mod W and nowhere else
        for g in fifo:
            lo = P + (g % W) * F
            assert np.all(ring.k[:, lo:lo + F] == _frame(L, F, H, D, g, 0))
            assert np.all(ring.v[:, lo:lo + F] == _frame(L, F, H, D, g, 1))


def test_unwritten_slots_and_pin_gap_stay_zero():
    L, H, D, P, W, F = 2, 1, 3, 8, 4, 5
    ring = RingModel(L, H, D, P, W, F)
    pk = np.arange(L * 3 * H * D, dtype=np.uint16).reshape(L, 3, H, D) + 1
    ring.pin(pk, pk + 100)
    ring.push(_frame(L, F, H, D, 0, 0), _frame(L, F, H, D, 0, 1))
    assert np.array_equal(ring.k[:, :3], pk) and np.array_equal(ring.v[:, :3], pk + 100)
    assert not ring.k[:, 3:P].any()                      # pin gap: capacity 8, pinned 3
    assert not ring.k[:, P + F:].any()                   # slots 1..3 never written
    assert ring.state() == {"head": 1, "count": 1, "pinned": 3, "frames_pushed": 1}


def test_pin_errors():
    ring = RingModel(1, 1, 2, 4, 2, 2)
    with pytest.raises(ValueError):
        ring.pin(np.zeros((1, 5, 1, 2), np.uint16), np.zeros((1, 5, 1, 2), np.uint16))
    ring.pin(np.zeros((1, 4, 1, 2), np.uint16), np.zeros((1, 4, 1, 2), np.uint16))
    with pytest.raises(RuntimeError):
        ring.pin(np.zeros((1, 1, 1, 2), np.uint16), np.zeros((1, 1, 1, 2), np.uint16))


def test_layout_matches_the_pages_buffer():
    """[num_layers][max_seq_len][num_heads][head_dim], zero-initialised."""
    ring = RingModel(18, 1, 256, 48, 2, 768)
    assert ring.k.shape == (18, 48 + 2 * 768, 1, 256) and ring.k.dtype == np.uint16
    assert not ring.k.any() and not ring.v.any()


# ---------------------------------------------------------------- capsules ----
# FlashRT article (PaperDaily), the section on what a capsule is and Fig. 2:
# a restore must give back exactly the state frozen at the snapshot. The
# expected state is rebuilt independently, by replaying the same pushes into
# a fresh ring, never by the capsule code itself.

def _replay(L, H, D, P, W, F, pin_n, n_frames):
    r = RingModel(L, H, D, P, W, F)
    if pin_n:
        r.pin(np.full((L, pin_n, H, D), 60001, np.uint16), np.full((L, pin_n, H, D), 60002, np.uint16))
    for f in range(n_frames):
        r.push(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1))
    return r


def _context(r):
    """Chronological [pin; window] K and V of every layer, read through the slot map."""
    ks = [r.k[:, :r.pinned]] + [r.k[:, r.P + r.slot_of(g) * r.F:r.P + (r.slot_of(g) + 1) * r.F] for g in r.window_frames()]
    vs = [r.v[:, :r.pinned]] + [r.v[:, r.P + r.slot_of(g) * r.F:r.P + (r.slot_of(g) + 1) * r.F] for g in r.window_frames()]
    return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)


@pytest.mark.parametrize("L,P,pin_n,W,F,t,more", [(2, 8, 8, 4, 3, 2, 7), (1, 5, 3, 3, 2, 5, 4), (3, 0, 0, 2, 4, 0, 3),
                                                   (3, 6, 6, 4, 2, 9, 1)])
def test_capsule_round_trip_equals_replay(L, P, pin_n, W, F, t, more):
    H, D = 1, 2
    live = _replay(L, H, D, P, W, F, pin_n, t)
    cap = live.capsule()
    # the compact layout: per layer the pinned tokens, then slots 0 .. count-1
    ntok = pin_n + min(t, W) * F
    assert cap["k"].shape == cap["v"].shape == (L, ntok, H, D)
    assert np.all(cap["k"][:, :pin_n] == 60001) and np.all(cap["v"][:, :pin_n] == 60002)
    for slot in range(min(t, W)):
        f = max(g for g in range(t) if g % W == slot)          # the newest frame written to that slot
        seg = slice(pin_n + slot * F, pin_n + (slot + 1) * F)
        assert np.array_equal(cap["k"][:, seg], _frame(L, F, H, D, f, 0))
        assert np.array_equal(cap["v"][:, seg], _frame(L, F, H, D, f, 1))
    for f in range(t, t + more):                              # move on, wrapping the window
        live.push(_frame(L, F, H, D, f + 100, 0), _frame(L, F, H, D, f + 100, 1))
    live.restore(cap)                                          # rollback
    ref = _replay(L, H, D, P, W, F, pin_n, t)
    assert live.state() == ref.state() and live.window_frames() == ref.window_frames()
    for a, b in zip(_context(live), _context(ref)):
        assert np.array_equal(a, b)
    # the restored ring keeps evolving like the original: same eviction ids, same bytes
    for f in range(t, t + W + 1):
        assert live.push(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1)) == \
            ref.push(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1))
        for a, b in zip(_context(live), _context(ref)):
            assert np.array_equal(a, b)


def test_fork_gives_independent_sessions():
    L, H, D, P, W, F = 2, 1, 2, 4, 3, 2
    src = _replay(L, H, D, P, W, F, 4, 5)
    cap = src.capsule()
    a, b = RingModel(L, H, D, P, W, F), RingModel(L, H, D, P, W, F)
    a.restore(cap)
    b.restore(cap)
    for x in (a, b):
        assert x.state() == src.state()
        for u, w in zip(_context(x), _context(src)):
            assert np.array_equal(u, w)
    a.push(_frame(L, F, H, D, 900, 0), _frame(L, F, H, D, 900, 1))
    b.push(_frame(L, F, H, D, 901, 0), _frame(L, F, H, D, 901, 1))
    assert not np.array_equal(_context(a)[0], _context(b)[0])        # diverged
    assert np.array_equal(_context(src)[0], _context(_replay(L, H, D, P, W, F, 4, 5))[0])   # source untouched


def test_restore_rejects_unreachable_states():
    r = RingModel(1, 1, 2, 4, 3, 2)
    cap = r.capsule()
    for bad in ({"head": 1, "count": 0, "pinned": 0, "frames_pushed": 0},
                {"head": 0, "count": 3, "pinned": 0, "frames_pushed": 2},
                {"head": 0, "count": 0, "pinned": 5, "frames_pushed": 0}):
        with pytest.raises(ValueError):
            r.restore({"k": cap["k"], "v": cap["v"], "state": bad})


# ----------------------------------------------------- spare slot (staging) ----
# Reflex review, system architecture (Figure 3): a producer pushes frames while
# the consumer denoises. The safety property of the spare slot: staging the
# next frame never changes a byte the current window reads, and a commit is
# exactly a push.

@pytest.mark.parametrize("L,P,W,F", [(1, 4, 3, 2), (2, 0, 1, 3), (3, 5, 4, 1)])
def test_spare_slot_window_against_deque(L, P, W, F):
    H, D = 1, 2
    ring = RingModel(L, H, D, P, W, F, spare_slots=1)
    assert ring.S == W + 1 and ring.max_seq_len == P + (W + 1) * F
    fifo = deque(maxlen=W)
    for f in range(3 * (W + 1) + 2):
        before = _context(ring)
        ring.stage(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1))
        assert ring.window_frames() == list(fifo)                    # staging changes no window
        for a, b in zip(_context(ring), before):
            assert np.array_equal(a, b)
        assert all(ring.slot_of(g) != ring.head for g in fifo)       # the staged slot is outside the window
        ev = ring.commit()
        assert ev == (fifo[0] if len(fifo) == W else -1)
        fifo.append(f)
        assert ring.window_frames() == list(fifo) and ring.count == len(fifo)
        assert ring.head == (f + 1) % (W + 1)
        for g in fifo:
            lo = P + (g % (W + 1)) * F
            assert np.array_equal(ring.k[:, lo:lo + F], _frame(L, F, H, D, g, 0))


def test_spare_slot_push_equals_stage_commit_and_guards():
    L, H, D, P, W, F = 2, 1, 2, 3, 2, 2
    a, b = RingModel(L, H, D, P, W, F, spare_slots=1), RingModel(L, H, D, P, W, F, spare_slots=1)
    for f in range(7):
        assert a.push(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1)) == \
            (b.stage(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1)) or b.commit())
        assert np.array_equal(a.k, b.k) and a.state() == b.state()
    b.stage(_frame(L, F, H, D, 9, 0), _frame(L, F, H, D, 9, 1))
    with pytest.raises(RuntimeError):
        b.stage(_frame(L, F, H, D, 9, 0), _frame(L, F, H, D, 9, 1))
    with pytest.raises(RuntimeError):
        b.push(_frame(L, F, H, D, 9, 0), _frame(L, F, H, D, 9, 1))
    b.commit()
    with pytest.raises(RuntimeError):
        b.commit()


@pytest.mark.parametrize("t,more", [(2, 5), (7, 3)])
def test_spare_slot_capsule_round_trip_equals_replay(t, more):
    L, H, D, P, W, F = 2, 1, 2, 3, 3, 2

    def replay(n):
        r = RingModel(L, H, D, P, W, F, spare_slots=1)
        r.pin(np.full((L, P, H, D), 7, np.uint16), np.full((L, P, H, D), 8, np.uint16))
        for f in range(n):
            r.push(_frame(L, F, H, D, f, 0), _frame(L, F, H, D, f, 1))
        return r

    live = replay(t)
    cap = live.capsule()
    assert cap["k"].shape[1] == P + min(t, W) * F
    for f in range(t, t + more):
        live.push(_frame(L, F, H, D, f + 50, 0), _frame(L, F, H, D, f + 50, 1))
    live.restore(cap)
    ref = replay(t)
    assert live.state() == ref.state()
    for a, b in zip(_context(live), _context(ref)):
        assert np.array_equal(a, b)
