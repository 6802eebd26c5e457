"""AdaRMSNorm: sinusoidal timestep embedding, gamma MLP and the normalisation.

Test infrastructure (see ``oracle/__init__``). Float64 arithmetic; values are
rounded to bf16 only where the module's dtype puts a bf16 tensor.

Reference: "Reflex: Real-Time VLA Control through Streaming Inference" paper
review:
* §3 Architecture, Eq. 2: AdaRMSNorm(x, c) = x / RMS(x) * gamma(c),
  gamma(c) = 1 + MLP(c), RMS(x) = sqrt(mean_i x_i^2 + eps); c concatenates
  a sinusoidal embedding of t_k with the proprioceptive state s_t; the RMS is
  taken in FP32 and the gating MLP runs in BF16 to save memory bandwidth.
* §3 component table: MLP = Linear(cond_dim -> hidden) -> SiLU ->
  Linear(hidden -> model_dim).
* §5 Code analysis, the AdaRMSNorm module: mean of squares of x.float(),
  x * rsqrt(ms + eps), times 1 + dense(cond).

Readings taken where the pages are silent:
* embedding: 128 dims, [sin(t w_i)]_{i<64} ++ [cos(t w_i)]_{i<64} with
  w_i = 10000^(-i/64) (the Transformer sinusoid); t_k = 1 - k/10;
* the Linear layers carry biases (nn.Linear's default); weights are stored
  bf16 in nn.Linear's [out][in] layout;
* the bf16 MLP rounds its input c and its hidden activation to bf16 and
  accumulates in wide precision; gamma = 1 + g is kept wide;
* the normalised output is computed wide and rounded to bf16 once, where it
  becomes the bf16 input of the following projection (done by the caller).
"""

from __future__ import annotations

import numpy as np

EMB_DIM = 128


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits. Write x = m * 2^e with 0.5 <= |m| < 1,
    round m * 256 to an integer (ties to even), scale back. Exact for the
    normal range used here; values are returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    r = np.rint(m * 256.0)            # numpy rint rounds half to even
    return np.ldexp(r / 256.0, e)


def timestep_embedding(t: float, dim: int = EMB_DIM) -> np.ndarray:
    """Sinusoidal embedding of one timestep: [sin(t w_i)] ++ [cos(t w_i)]."""
    half = dim // 2
    i = np.arange(half, dtype=np.float64)
    w = 10000.0 ** (-i / half)
    return np.concatenate([np.sin(t * w), np.cos(t * w)])


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def condition(t: float, state: np.ndarray) -> np.ndarray:
    """c = [emb(t); s], rounded to bf16 as the input of the bf16 MLP."""
    c = np.concatenate([timestep_embedding(t), np.asarray(state, dtype=np.float64)])
    return round_bf16(c)


def gamma(w1, b1, w2, b2, t: float, state) -> np.ndarray:
    """gamma(c) = 1 + W2 bf16(SiLU(W1 c + b1)) + b2 (Eq. 2, §3 component table).

    w1 [hidden][cond], b1 [hidden], w2 [model][hidden], b2 [model]; float64
    arrays holding bf16 values. Returns [model] float64.
    """
    c = condition(t, state)
    h1 = np.asarray(w1, np.float64) @ c + np.asarray(b1, np.float64)
    a = round_bf16(silu(h1))
    g = np.asarray(w2, np.float64) @ a + np.asarray(b2, np.float64)
    return 1.0 + g


def rmsnorm_scaled(x: np.ndarray, gamma_vec: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma, row-wise over the last axis (Eq. 2)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma_vec, dtype=np.float64)


def ada_rmsnorm(x, w1, b1, w2, b2, t: float, state, eps: float) -> np.ndarray:
    """AdaRMSNorm(x, c) with c = [emb(t); state] (Eq. 2), float64 output."""
    return rmsnorm_scaled(x, gamma(w1, b1, w2, b2, t, state), eps)
