"""Byte-level model of the static ring-buffer KV cache.

Test infrastructure (see ``oracle/__init__``).

Reference: "Reflex: Real-Time VLA Control through Streaming Inference" paper
review:
* §3 Architecture, ring-buffer diagram and Eq. 1 text: a pinned instruction
  prefix computed once at t = 0, then a sliding FIFO window where each frame
  enqueues the newest frame and evicts the oldest;
* §3 component table: buffer_k is num_layers x max_seq_len x num_heads x
  head_dim in BF16, allocated statically so no allocation happens later;
* §5 Code analysis: the buffers are created zeroed next to a write pointer
  ``ptr = 0``; ``add_new_prefix`` adds the new observation and reports the
  eviction; ``evict_source_prefix`` removes the oldest frame from all layers.

Capsules follow the FlashRT article (PaperDaily, "FlashRT开源：27倍加速…"),
the section on what a capsule is and Fig. 2: the live state at a commit
boundary is a fixed set of buffers plus metadata; snapshot freezes it,
restore copies it back and rebinds the metadata, fork restores one capsule
into several sessions, rollback restores an earlier one. For the ring the
live state is the valid region (pinned tokens and the first ``count`` slots
of every layer) and (head, count, pinned, frames_pushed).

Readings taken:
* the pin occupies tokens [0, P) of the same buffer, so max_seq_len = P + W*F;
* ``ptr`` is a slot index that advances by one per frame, modulo W;
* a push overwrites slot ``head`` in every layer (that overwrite *is* the
  eviction of the frame pushed W frames earlier) and nothing else moves;
* a capsule stores the valid region compactly, K then V, each
  ``[L][pinned + count*F][Hkv][D]``; a restore writes it back in place and
  leaves every other token as it was (no call reads those);
* asynchronous pushes (Reflex review, system architecture, Figure 3: the
  vision thread pushes into the shared cache while the policy thread
  denoises) need a slot no running step reads: with ``spare_slots = 1`` the
  ring has S = W + 1 physical slots, frame f goes to slot f mod S, and the
  window (the newest W frames) never includes slot ``head``, which a
  staged frame fills before its commit. A frame "evicted" is the one that
  leaves the window.

The model stores raw words (``uint16`` for bf16 bits, ``uint32`` for fp32
bits) so that device buffers can be compared with ``array_equal``.
"""

from __future__ import annotations

import numpy as np


class RingModel:
    """Expected contents and metadata of the ring after each call."""

    def __init__(self, num_layers, num_kv_heads, head_dim, pin_capacity, num_slots,
                 tokens_per_frame, word_dtype=np.uint16, spare_slots=0):
        if min(num_layers, num_kv_heads, head_dim, num_slots, tokens_per_frame) <= 0 or pin_capacity < 0:
            raise ValueError("ring dimensions must be positive (pin capacity >= 0)")
        if spare_slots not in (0, 1):
            raise ValueError("spare_slots must be 0 or 1")
        self.L, self.Hkv, self.D = num_layers, num_kv_heads, head_dim
        self.P, self.W, self.F = pin_capacity, num_slots, tokens_per_frame
        self.spare = spare_slots
        self.S = self.W + spare_slots          # physical slots
        self.staged = False
        self.max_seq_len = self.P + self.S * self.F
        shape = (self.L, self.max_seq_len, self.Hkv, self.D)
        self.k = np.zeros(shape, dtype=word_dtype)   # zeroed at creation (§5 code)
        self.v = np.zeros(shape, dtype=word_dtype)
        self.head = 0          # next slot to write (the page's ``ptr``)
        self.count = 0         # valid slots, saturates at W
        self.pinned = 0        # pinned prefix tokens
        self.frames_pushed = 0
        self.slot_frame = [-1] * self.S   # which frame id sits in each slot

    # -- the pinned prefix: written once, at t = 0 ---------------------------
    def pin(self, k_words: np.ndarray, v_words: np.ndarray) -> None:
        """Write ``[L][n][Hkv][D]`` into tokens [0, n) of every layer, once."""
        n = k_words.shape[1]
        if self.pinned:
            raise RuntimeError("prefix already pinned")
        if n > self.P:
            raise ValueError("prefix longer than the pin capacity")
        self.k[:, :n] = k_words
        self.v[:, :n] = v_words
        self.pinned = n

    # -- one frame: enqueue newest, evict oldest ------------------------------
    def push(self, k_words: np.ndarray, v_words: np.ndarray) -> int:
        """Overwrite slot ``head``; return the id of the frame that left the window, or -1."""
        if self.staged:
            raise RuntimeError("a staged frame is pending")
        self.stage(k_words, v_words)
        return self.commit()

    def stage(self, k_words: np.ndarray, v_words: np.ndarray) -> None:
        """Write the next frame into slot ``head`` without changing the window."""
        if self.staged:
            raise RuntimeError("a staged frame is pending")
        lo = self.P + self.head * self.F
        self.k[:, lo:lo + self.F] = k_words
        self.v[:, lo:lo + self.F] = v_words
        self.staged = True

    def commit(self) -> int:
        """The staged frame becomes the newest of the window; return the frame that left it, or -1."""
        if not self.staged:
            raise RuntimeError("nothing staged")
        self.staged = False
        evicted = self.frames_pushed - self.W if self.frames_pushed >= self.W else -1
        self.slot_frame[self.head] = self.frames_pushed
        self.frames_pushed += 1
        self.head = self.frames_pushed % self.S
        self.count = min(self.count + 1, self.W)
        return evicted

    # -- views used by the attention oracle -----------------------------------
    def window_frames(self) -> list[int]:
        """Frame ids in the window, oldest first (FIFO order)."""
        return [f for f in range(max(0, self.frames_pushed - self.W), self.frames_pushed)]

    def slot_of(self, frame_id: int) -> int:
        return frame_id % self.S

    def state(self) -> dict:
        return {"head": self.head, "count": self.count, "pinned": self.pinned,
                "frames_pushed": self.frames_pushed}

    # -- capsules: snapshot / restore (fork and rollback are restores) --------
    def valid_tokens(self) -> list[int]:
        """Token indices of the valid region of a layer, in capsule order: the
        pinned tokens, then the window's slots in physical order."""
        slots = sorted(self.slot_of(f) for f in self.window_frames())
        return list(range(self.pinned)) + [self.P + s * self.F + t for s in slots for t in range(self.F)]

    def capsule(self) -> dict:
        """The valid region, compact, plus the metadata."""
        idx = self.valid_tokens()
        return {"k": self.k[:, idx].copy(), "v": self.v[:, idx].copy(), "state": self.state()}

    def restore(self, cap: dict) -> None:
        st = cap["state"]
        fp, count, head, pinned = st["frames_pushed"], st["count"], st["head"], st["pinned"]
        if self.staged:
            raise RuntimeError("a staged frame is pending")
        if not (0 <= pinned <= self.P and fp >= 0 and count == min(fp, self.W) and head == fp % self.S):
            raise ValueError(f"state {st} is not reachable by this ring")
        self.pinned, self.count, self.head, self.frames_pushed = pinned, count, head, fp
        idx = self.valid_tokens()
        self.k[:, idx] = cap["k"]
        self.v[:, idx] = cap["v"]
        # slot s holds the latest frame f < frames_pushed with f = s (mod S)
        self.slot_frame = [-1] * self.S
        for f in range(max(0, fp - self.S), fp):
            self.slot_frame[f % self.S] = f

