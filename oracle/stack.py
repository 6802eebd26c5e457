"""One layer of the denoising stack, and the Euler update of the flow state.

Test infrastructure (see ``oracle/__init__``). Float64 arithmetic; tensors are
rounded to bf16 exactly where the stack stores them as bf16 between ops.

References: "Reflex: Real-Time VLA Control through Streaming Inference" paper
review, §2 Core idea (the flow starts from x ~ N(0, I) at t = 1 and is
denoised over K steps), §3 Architecture (Eq. 1 attention, Eq. 2 AdaRMSNorm),
§4 Innovations / §2 (a packed QKV kernel is one of the fused operators), and
§6 Table 7 (ten denoising steps per action chunk).

The pages give no layer glue, so everything below is a reading. Each op is
pinned on its own, and the end-to-end step (``denoise_step``, with and
without the FFN block) is pinned against the same step written with torch's
float64 operators (rms_norm, matmul, scaled_dot_product_attention, silu, bf16
conversion) on inputs where a miswired chain -- the wrong stream fed to the
next layer, one gamma for every layer, the velocity from another layer, a
dropped attention region -- fails the comparison:
* layer l at step k: y = bf16(AdaRMSNorm(h, gamma_{l,k})); [q|k|v] = y W_qkv^T
  with W_qkv packed [(Hq + 2 Hkv) * D][model] as q heads, then k heads, then
  v heads, each stored bf16; o = Eq. 1 attention over [cache; k_dyn] stored
  bf16; h <- bf16(h + o W_o^T) with W_o [model][Hq * D]; no bias (the FFN
  block below is optional);
* the velocity is the last layer's stream, v = h_L, and the Euler step with
  dt = 1/10 is x_{k+1} = bf16(x_k - v / 10);
* the full action-expert layer (the pages name SwiGLU fusion, FlashNorm and
  FusedAdaLN among the fused operators of §2 / the §3 system-optimisation
  row and Fig. 11, but give no FFN) adds, after the attention residual,
  y2 = bf16(AdaRMSNorm(h, gamma_ffn)) with its own gamma, act =
  bf16(SiLU(y2 W_gate^T) * (y2 W_up^T)) and h <- bf16(h + act W_down^T);
  no biases; the products before SiLU are wide (unrounded).
"""

from __future__ import annotations

import numpy as np

from .adanorm import rmsnorm_scaled, round_bf16, silu
from .attention import full_attention


def qkv_projection(y, w_qkv, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """[q|k|v] = y W_qkv^T, split into q [N][Hq][D], k and v [N][Hkv][D]."""
    y = np.asarray(y, np.float64)
    out = y @ np.asarray(w_qkv, np.float64).T
    n = y.shape[0]
    nq, nk = n_q_heads * head_dim, n_kv_heads * head_dim
    q = out[:, :nq].reshape(n, n_q_heads, head_dim)
    k = out[:, nq:nq + nk].reshape(n, n_kv_heads, head_dim)
    v = out[:, nq + nk:nq + 2 * nk].reshape(n, n_kv_heads, head_dim)
    return q, k, v


def out_projection_residual(h, o, w_o):
    """h + o W_o^T, with o flattened to [N][Hq * D]. Float64, unrounded."""
    o = np.asarray(o, np.float64).reshape(o.shape[0], -1)
    return np.asarray(h, np.float64) + o @ np.asarray(w_o, np.float64).T


def ffn_swiglu(h, gamma_vec, eps, w_gate, w_up, w_down):
    """The SwiGLU FFN block with its AdaRMSNorm; returns the stored
    intermediates y (bf16), act (bf16) and the new h (bf16)."""
    h = np.asarray(h, np.float64)
    y = round_bf16(rmsnorm_scaled(h, gamma_vec, eps))
    g = y @ np.asarray(w_gate, np.float64).T
    u = y @ np.asarray(w_up, np.float64).T
    act = round_bf16(silu(g) * u)
    h_new = round_bf16(h + act @ np.asarray(w_down, np.float64).T)
    return {"y2": y, "act": act, "h": h_new}


def layer(h, gamma_vec, eps, w_qkv, cache_k, cache_v, w_o, scale,
          n_q_heads, n_kv_heads, head_dim, ffn=None):
    """One layer; returns every stored intermediate (bf16-valued float64).

    ``cache_k`` / ``cache_v`` are the layer's cached context [T][Hkv][D] in
    chronological order (pin then window frames); the step's own k/v are
    appended after them, as Eq. 1 orders the regions. ``ffn`` (optional) is
    (gamma_ffn, w_gate, w_up, w_down) of the layer's SwiGLU FFN block.
    """
    y = round_bf16(rmsnorm_scaled(h, gamma_vec, eps))
    q, k, v = qkv_projection(y, w_qkv, n_q_heads, n_kv_heads, head_dim)
    q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    ctx_k = np.concatenate([np.asarray(cache_k, np.float64), k], axis=0)
    ctx_v = np.concatenate([np.asarray(cache_v, np.float64), v], axis=0)
    o = round_bf16(full_attention(q, ctx_k, ctx_v, scale))
    h_new = round_bf16(out_projection_residual(h, o, w_o))
    r = {"y": y, "q": q, "k": k, "v": v, "o": o, "h_attn": h_new, "h": h_new}
    if ffn is not None:
        f = ffn_swiglu(h_new, ffn[0], eps, ffn[1], ffn[2], ffn[3])
        r.update(y2=f["y2"], act=f["act"], h=f["h"])
    return r


def euler(x, v, dt: float = 0.1):
    """x_{k+1} = bf16(x_k - dt * v)."""
    return round_bf16(np.asarray(x, np.float64) - dt * np.asarray(v, np.float64))


def timesteps(n_steps: int = 10):
    """t_k = 1 - k / n_steps for k = 0 .. n_steps - 1 (flow starts at t = 1)."""
    return [1.0 - k / n_steps for k in range(n_steps)]


def denoise_step(x, gammas, eps, w_qkv, w_o, caches_k, caches_v, scale,
                 n_q_heads, n_kv_heads, head_dim, ffns=None):
    """All layers at one step, then the Euler update (pinned end to end against
    a torch float64 chain of the same step).

    ``gammas[l]`` is gamma_{l,k}; ``caches_k[l]`` the chronological cached
    context of layer l; ``ffns[l]`` (optional) layer l's FFN block as in
    ``layer``. Returns (x_next, per-layer intermediates).
    """
    h = np.asarray(x, np.float64)
    trace = []
    for l in range(len(w_qkv)):
        r = layer(h, gammas[l], eps, w_qkv[l], caches_k[l], caches_v[l], w_o[l], scale,
                  n_q_heads, n_kv_heads, head_dim, None if ffns is None else ffns[l])
        trace.append(r)
        h = r["h"]
    return euler(x, h), trace
