"""Shared-KV multi-reader attention: decode streams with private KV tails.

Test infrastructure (see ``oracle/__init__``). Float64.

Reference: "OxyGen: Unified KV Cache Management for Vision-Language-Action
Models under Multi-Task Parallelism" review, core method and method details:
one prefill cache per frame is handed to the action expert as a read-only
context and to the language expert, which appends the KV of every decoded
token; the active requests are stacked along the batch dimension and advance
k decode steps per frame; a request ends at EOS or at a maximum length N.

Readings taken:
* all readers share one live cache (pin + sliding window); a decode stream's
  appended tokens live in a private tail that no other reader sees, and the
  action suffix never sees any private tail;
* a decode step first appends the stream's new token to its tail, then the
  stream's single query token attends over [pin; window; tail];
* a request that reached the maximum length N (a full tail) has ended; when
  retiring is on, the stream's next append starts a new request, whose tail
  holds only that token.
"""

from __future__ import annotations

import numpy as np

from .attention import full_attention


class PrivateTails:
    """Per-stream appended KV: [streams][capacity][Hkv][D] plus lengths."""

    def __init__(self, n_streams, capacity, n_kv_heads, head_dim):
        shape = (n_streams, capacity, n_kv_heads, head_dim)
        self.k = np.zeros(shape, np.float64)
        self.v = np.zeros(shape, np.float64)
        self.length = np.zeros(n_streams, np.int64)
        self.capacity = capacity

    def append(self, stream, k_tok, v_tok, retire_full=False):
        """Append one token ([Hkv][D]) to a stream's tail; with retire_full a
        full tail (a finished request) restarts with this token."""
        n = int(self.length[stream])
        if n >= self.capacity and retire_full:
            self.reset(stream)
            n = 0
        if n >= self.capacity:
            raise ValueError("private tail full")
        self.k[stream, n] = k_tok
        self.v[stream, n] = v_tok
        self.length[stream] = n + 1

    def reset(self, stream):
        """Retire a finished request: its tail becomes empty."""
        self.length[stream] = 0


def decode_attention(q_streams, shared_k, shared_v, tails: PrivateTails, scale):
    """Each stream's query [Hq][D] over [shared context; its own tail].

    q_streams [G][Hq][D]; shared_k/v [T][Hkv][D] chronological. Returns [G][Hq][D].
    """
    out = []
    for j in range(q_streams.shape[0]):
        n = int(tails.length[j])
        ck = np.concatenate([np.asarray(shared_k, np.float64), tails.k[j, :n]], axis=0)
        cv = np.concatenate([np.asarray(shared_v, np.float64), tails.v[j, :n]], axis=0)
        out.append(full_attention(np.asarray(q_streams[j:j + 1], np.float64), ck, cv, scale)[0])
    return np.stack(out)
