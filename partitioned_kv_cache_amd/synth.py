"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no arithmetic of the method: it draws numbers and converts
storage types. Every tensor comes from its own NumPy generator keyed by
``SeedSequence([0, cfg_id, tensor_id, layer, frame, step])``, so any frame or
step can be regenerated on its own. Draws are float32 and, for bf16
workloads, rounded once to bf16 (round to nearest, ties to even) on the host.

bf16 tensors are returned as ``uint16`` bit patterns, fp32 tensors as
``float32``. ``widen`` turns either into exact float64 for the oracle.

Distributions follow the workloads on the pages: K, V, Q and the flow state
x ~ N(0, 1) (the flow starts at x ~ N(0, I)); the robot state ~ N(0, 1);
weights ~ U(-1/sqrt(fan_in), 1/sqrt(fan_in)), nn.Linear's default range.
"""

from __future__ import annotations

import numpy as np

from .configs import Shape

# tensor ids (second-level seed keys)
T_Q, T_KPIN, T_VPIN, T_KFRAME, T_VFRAME, T_KDYN, T_VDYN = 1, 2, 3, 4, 5, 6, 7
T_X, T_STATE, T_W1, T_B1, T_W2, T_B2, T_WQKV, T_WO = 8, 9, 10, 11, 12, 13, 14, 15
T_TAILK, T_TAILV, T_DECQ = 16, 17, 18
T_WGATE, T_WUP, T_WDOWN, T_W1F, T_B1F, T_W2F, T_B2F = 19, 20, 21, 22, 23, 24, 25


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, *[int(k) for k in key]]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 view of a bf16-bits (uint16) or float32 array."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x)


def normal(shape, dtype: str, *key: int) -> np.ndarray:
    return _store(_rng(*key).standard_normal(shape, dtype=np.float32), dtype)


def uniform(shape, bound: float, dtype: str, *key: int) -> np.ndarray:
    x = _rng(*key).uniform(-bound, bound, size=shape).astype(np.float32)
    return _store(x, dtype)


# -- attention inputs ----------------------------------------------------------

def pin_kv(s: Shape, n_tokens: int | None = None):
    """K and V of the pinned prefix, [L][n][Hkv][D] (n defaults to P)."""
    n = s.pin_tokens if n_tokens is None else n_tokens
    shp = (s.num_layers, n, s.n_kv_heads, s.head_dim)
    return normal(shp, s.dtype, s.cfg_id, T_KPIN), normal(shp, s.dtype, s.cfg_id, T_VPIN)


def frame_kv(s: Shape, frame: int):
    """K and V of one visual frame, [L][F][Hkv][D]."""
    shp = (s.num_layers, s.tokens_per_frame, s.n_kv_heads, s.head_dim)
    return (normal(shp, s.dtype, s.cfg_id, T_KFRAME, 0, frame),
            normal(shp, s.dtype, s.cfg_id, T_VFRAME, 0, frame))


def suffix_qkv(s: Shape, frame: int, step: int):
    """Q [L][N][Hq][D] and the dynamic K, V [L][N][Hkv][D] of one step."""
    qs = (s.num_layers, s.n_dyn, s.n_q_heads, s.head_dim)
    ks = (s.num_layers, s.n_dyn, s.n_kv_heads, s.head_dim)
    return (normal(qs, s.dtype, s.cfg_id, T_Q, 0, frame, step),
            normal(ks, s.dtype, s.cfg_id, T_KDYN, 0, frame, step),
            normal(ks, s.dtype, s.cfg_id, T_VDYN, 0, frame, step))


# -- layer glue inputs -----------------------------------------------------------

def flow_x(s: Shape, frame: int):
    """Flow initialisation x ~ N(0, I), [N][model] bf16."""
    return normal((s.n_dyn, s.model_dim), "bf16", s.cfg_id, T_X, 0, frame)


def robot_state(s: Shape, frame: int):
    """Proprioceptive state ~ N(0, 1), [state_dim] bf16."""
    return normal((s.state_dim,), "bf16", s.cfg_id, T_STATE, 0, frame)


def mlp_weights(s: Shape, layer: int):
    """gamma-MLP weights of one layer in nn.Linear layout (bf16 bits).

    w1 [hidden][cond], b1 [hidden], w2 [model][hidden], b2 [model].
    """
    cond = s.cond_emb + s.state_dim
    b1 = 1.0 / np.sqrt(cond)
    b2 = 1.0 / np.sqrt(s.hidden_dim)
    return (uniform((s.hidden_dim, cond), b1, "bf16", s.cfg_id, T_W1, layer),
            uniform((s.hidden_dim,), b1, "bf16", s.cfg_id, T_B1, layer),
            uniform((s.model_dim, s.hidden_dim), b2, "bf16", s.cfg_id, T_W2, layer),
            uniform((s.model_dim,), b2, "bf16", s.cfg_id, T_B2, layer))


def proj_weights(s: Shape, layer: int):
    """Packed W_qkv [(Hq+2Hkv)D][model] and W_o [model][Hq D] (bf16 bits)."""
    wq = uniform((s.qkv_out, s.model_dim), 1.0 / np.sqrt(s.model_dim), "bf16", s.cfg_id, T_WQKV, layer)
    hd = s.n_q_heads * s.head_dim
    wo = uniform((s.model_dim, hd), 1.0 / np.sqrt(hd), "bf16", s.cfg_id, T_WO, layer)
    return wq, wo


def ffn_weights(s: Shape, layer: int):
    """SwiGLU FFN weights of one layer (bf16 bits): W_gate and W_up
    [ffn][model], W_down [model][ffn], U(+-1/sqrt(fan_in))."""
    bm, bf = 1.0 / np.sqrt(s.model_dim), 1.0 / np.sqrt(s.ffn_dim)
    return (uniform((s.ffn_dim, s.model_dim), bm, "bf16", s.cfg_id, T_WGATE, layer),
            uniform((s.ffn_dim, s.model_dim), bm, "bf16", s.cfg_id, T_WUP, layer),
            uniform((s.model_dim, s.ffn_dim), bf, "bf16", s.cfg_id, T_WDOWN, layer))


def ffn_mlp_weights(s: Shape, layer: int):
    """The FFN norm's own gamma-MLP weights (same shapes as mlp_weights)."""
    cond = s.cond_emb + s.state_dim
    b1 = 1.0 / np.sqrt(cond)
    b2 = 1.0 / np.sqrt(s.hidden_dim)
    return (uniform((s.hidden_dim, cond), b1, "bf16", s.cfg_id, T_W1F, layer),
            uniform((s.hidden_dim,), b1, "bf16", s.cfg_id, T_B1F, layer),
            uniform((s.model_dim, s.hidden_dim), b2, "bf16", s.cfg_id, T_W2F, layer),
            uniform((s.model_dim,), b2, "bf16", s.cfg_id, T_B2F, layer))


# -- shared-KV decode streams ------------------------------------------------------

def decode_q(s: Shape, frame: int, step: int):
    """One query token per stream, [L][G][Hq][D]."""
    return normal((s.num_layers, s.n_streams, s.n_q_heads, s.head_dim), s.dtype,
                  s.cfg_id, T_DECQ, 0, frame, step)


def decode_kv(s: Shape, frame: int, step: int):
    """The token each stream appends to its private tail, [L][G][Hkv][D]."""
    shp = (s.num_layers, s.n_streams, s.n_kv_heads, s.head_dim)
    return (normal(shp, s.dtype, s.cfg_id, T_TAILK, 0, frame, step),
            normal(shp, s.dtype, s.cfg_id, T_TAILV, 0, frame, step))
