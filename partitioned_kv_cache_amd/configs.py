"""Workload shapes: five synthetic configurations of the denoising hot path.

Pure data. Shapes follow the pages' workloads: a 50-action chunk plus one
state token as the dynamic suffix, ten denoising steps per frame, three
cameras x 256 tokens per visual frame, a Pi0.5-like action expert with eight
query heads sharing one KV head of width 256.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Shape:
    name: str
    cfg_id: int              # seeds every tensor of this workload
    num_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str               # "f32" or "bf16" storage; accumulation is fp32
    pin_tokens: int          # P: pinned instruction prefix
    num_slots: int           # W: frames in the sliding window
    tokens_per_frame: int    # F
    n_dyn: int               # N: dynamic suffix tokens (actions + state)
    steps_per_frame: int
    frames: int
    scale: float
    # layer glue (only the full stack uses these)
    model_dim: int = 0
    cond_emb: int = 128
    state_dim: int = 32
    hidden_dim: int = 0
    ffn_dim: int = 0         # SwiGLU FFN width of the full action-expert layer (0: none)
    eps: float = 1e-6
    # shared-KV decode streams (only the multi-reader workload)
    n_streams: int = 0
    tail_capacity: int = 0
    extras: dict = field(default_factory=dict)

    @property
    def max_seq_len(self) -> int:
        return self.pin_tokens + self.num_slots * self.tokens_per_frame

    @property
    def cached_tokens_full(self) -> int:
        return self.max_seq_len

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


TINY = Shape("tiny_f32_1L", 1, num_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=64, dtype="f32",
             pin_tokens=16, num_slots=4, tokens_per_frame=16, n_dyn=8, steps_per_frame=3,
             frames=10, scale=1.0 / 8.0)

PI05_1L = Shape("pi05_like_1L", 2, num_layers=1, n_q_heads=8, n_kv_heads=1, head_dim=256, dtype="bf16",
                pin_tokens=48, num_slots=2, tokens_per_frame=768, n_dyn=51, steps_per_frame=10,
                frames=200, scale=1.0 / 16.0)

PI05_18L = PI05_1L.with_(name="pi05_like_18L_stack", cfg_id=3, num_layers=18, frames=10_000,
                         model_dim=1024, hidden_dim=1024)

LONG_18L = Shape("long_history_18L", 4, num_layers=18, n_q_heads=8, n_kv_heads=1, head_dim=256,
                 dtype="bf16", pin_tokens=256, num_slots=8, tokens_per_frame=768, n_dyn=51,
                 steps_per_frame=10, frames=500, scale=1.0 / 16.0)

SHARED_KV = LONG_18L.with_(name="shared_kv_multitask", cfg_id=5, frames=100, n_streams=16,
                           tail_capacity=30)

# The full denoising step (norm + QKV + attention + out-projection, chained
# layer by layer) on the long-history cache: the layer dims of the 18-layer
# stack over the long-history ring. The benchmark reports its microseconds
# per step beside the layer-batched attention step.
LONG_18L_FULL = LONG_18L.with_(name="long_history_18L_full_step", cfg_id=6, model_dim=1024,
                               hidden_dim=1024)

# The full action-expert layer: the 18-layer stack plus a SwiGLU FFN of
# width 4 x model per layer.
PI05_18L_FFN = PI05_18L.with_(name="pi05_like_18L_full_layer", cfg_id=7, ffn_dim=4096)

ALL = {s.name: s for s in (TINY, PI05_1L, PI05_18L, LONG_18L, SHARED_KV, LONG_18L_FULL, PI05_18L_FFN)}
