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
