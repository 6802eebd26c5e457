"""Full-batch softmax attention over an explicitly concatenated context.

Test infrastructure (see ``oracle/__init__``). Float64 throughout.

Reference: "Reflex: Real-Time VLA Control through Streaming Inference" paper
review, §3 Architecture, Eq. 1: the dynamic-suffix queries Q^(k) attend over
the concatenation [K_pin; K_slide(t); K_dyn(k)] (and the matching values),
softmax(Q K^T / sqrt(d)) V, with no mask inside the formula. Prop. A.1 on the
same page states that the partitioned computation equals this full-batch one
on every dynamic-suffix token, which is why the oracle is simply the
full-batch definition.

Readings taken where the page is silent:
* d is the head dimension; the scale is applied once and passed explicitly.
* grouped heads: query head h reads KV head floor(h / (Hq / Hkv)).
* positions are baked into K before it is written, so no rotary step here.
"""

from __future__ import annotations

import numpy as np


def build_context(pin: np.ndarray, frames: list[np.ndarray], dyn: np.ndarray) -> np.ndarray:
    """Concatenate [pin; frame_oldest; ...; frame_newest; dyn] along tokens.

    Each argument is ``[tokens][Hkv][D]``; ``frames`` is in chronological
    order, oldest first (Eq. 1's K_slide(t) is the FIFO window of the most
    recent frames). Returns a float64 copy.
    """
    parts = [np.asarray(pin, dtype=np.float64)]
    parts += [np.asarray(f, dtype=np.float64) for f in frames]
    parts.append(np.asarray(dyn, dtype=np.float64))
    return np.concatenate(parts, axis=0)


def full_attention(q: np.ndarray, ctx_k: np.ndarray, ctx_v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for every query token and head (Eq. 1).

    q      [N][Hq][D]  queries of the dynamic suffix
    ctx_k  [T][Hkv][D] keys of the whole context, chronological
    ctx_v  [T][Hkv][D] values, same order
    scale  the 1/sqrt(d) factor of Eq. 1, given explicitly
    returns [N][Hq][D] float64

    For each (token i, head h) with KV head g: z_j = scale * <q_ih, k_jg>,
    m = max_j z_j, p_j = exp(z_j - m), out = sum_j p_j v_jg / sum_j p_j.
    Subtracting m is exact in real arithmetic (softmax is shift invariant)
    and keeps exp in range.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(ctx_k, dtype=np.float64)
    v = np.asarray(ctx_v, dtype=np.float64)
    n_tok, n_qh, d = q.shape
    t, n_kvh, d2 = k.shape
    if d2 != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    if n_qh % n_kvh:
        raise ValueError("query heads must be a multiple of kv heads")
    if t == 0:
        raise ValueError("empty context: softmax over no keys is undefined")
    group = n_qh // n_kvh
    out = np.empty((n_tok, n_qh, d), dtype=np.float64)
    for h in range(n_qh):
        g = h // group
        z = scale * (q[:, h, :] @ k[:, g, :].T)          # [N][T]
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        out[:, h, :] = (p @ v[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def partitioned_reference(q, pin_k, pin_v, frames_k, frames_v, dyn_k, dyn_v, scale):
    """Eq. 1 written as the page writes it: concatenate the three regions, attend.

    ``frames_k`` / ``frames_v`` are the window's frames oldest first.
    """
    ck = build_context(pin_k, frames_k, dyn_k)
    cv = build_context(pin_v, frames_v, dyn_v)
    return full_attention(q, ck, cv, scale)
