"""Pins of the attention oracle against things other than itself.

* brute force in pure Python (math.fsum) on tiny shapes, grouped heads included;
* closed forms: zero keys, constant values, one key, two keys, a dominant
  logit, a constant shift of every logit;
* the library special case: torch's scaled_dot_product_attention in float64;
* Prop. A.1 of the Reflex paper review (§3): permuting the cached tokens and
  merging per-region partial softmaxes by log-sum-exp both reproduce the
  full-batch result;
* Table 4 of the same review (§6): partitioned = full recompute (MSE 0.00),
  while the naive cache that reuses an earlier step's suffix KV is far off.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle.attention import build_context, full_attention, partitioned_reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute(q, k, v, scale):
    """Pure-Python loops, exactly summed with math.fsum."""
    n, hq, d = q.shape
    t, hkv, _ = k.shape
    grp = hq // hkv
    out = np.zeros((n, hq, d))
    for i in range(n):
        for h in range(hq):
            g = h // grp
            z = [scale * math.fsum(float(q[i, h, e]) * float(k[j, g, e]) for e in range(d)) for j in range(t)]
            m = max(z)
            p = [math.exp(x - m) for x in z]
            zsum = math.fsum(p)
            for e in range(d):
                out[i, h, e] = math.fsum(p[j] * float(v[j, g, e]) for j in range(t)) / zsum
    return out


@pytest.mark.parametrize("seed,n,hq,hkv,t,d", [
    (0, 3, 1, 1, 7, 4), (1, 2, 4, 2, 12, 8), (2, 5, 8, 1, 9, 3), (3, 1, 2, 2, 1, 5), (4, 4, 6, 3, 11, 6)])
def test_brute_force(seed, n, hq, hkv, t, d):
    r = np.random.default_rng(seed)
    q, k, v = r.normal(size=(n, hq, d)), r.normal(size=(t, hkv, d)), r.normal(size=(t, hkv, d))
    scale = 1 / math.sqrt(d)
    np.testing.assert_allclose(full_attention(q, k, v, scale), brute(q, k, v, scale), rtol=0, atol=1e-12)


def test_zero_keys_give_mean_of_values():
    r = np.random.default_rng(5)
    q, v = r.normal(size=(3, 2, 4)), r.normal(size=(9, 1, 4))
    out = full_attention(q, np.zeros((9, 1, 4)), v, 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, 0].mean(axis=0), out.shape), atol=1e-14)


def test_constant_values_give_the_constant():
    r = np.random.default_rng(6)
    q, k = r.normal(size=(4, 2, 5)), r.normal(size=(13, 2, 5))
    c = r.normal(size=5)
    out = full_attention(q, k, np.broadcast_to(c, (13, 2, 5)).copy(), 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), atol=1e-14)


def test_single_key_returns_its_value():
    r = np.random.default_rng(7)
    q, k, v = r.normal(size=(2, 3, 4)), r.normal(size=(1, 1, 4)), r.normal(size=(1, 1, 4))
    np.testing.assert_allclose(full_attention(q, k, v, 1.0), np.broadcast_to(v[0, 0], (2, 3, 4)), atol=1e-15)


def test_two_keys_sigmoid_form():
    r = np.random.default_rng(8)
    q, k, v = r.normal(size=(3, 1, 6)), r.normal(size=(2, 1, 6)), r.normal(size=(2, 1, 6))
    s = 0.7
    z = s * q[:, 0] @ k[:, 0].T
    sig = 1 / (1 + np.exp(-(z[:, 0] - z[:, 1])))
    want = sig[:, None] * v[0, 0] + (1 - sig)[:, None] * v[1, 0]
    np.testing.assert_allclose(full_attention(q, k, v, s)[:, 0], want, atol=1e-14)


def test_dominant_logit_selects_its_value():
    r = np.random.default_rng(9)
    k, v = r.normal(size=(10, 1, 8)), r.normal(size=(10, 1, 8))
    k[3, 0] *= 3.0                       # make key 3 the longest so q = lam * k_3 favours it
    q = (200.0 * k[3, 0])[None, None, :]
    np.testing.assert_allclose(full_attention(q, k, v, 1.0)[0, 0], v[3, 0], atol=1e-12)


def test_constant_logit_shift_changes_nothing():
    r = np.random.default_rng(10)
    q, k, v = r.normal(size=(4, 2, 6)), r.normal(size=(15, 1, 6)), r.normal(size=(15, 1, 6))
    base = full_attention(q, k, v, 0.5)
    # an extra coordinate with value a in q and 1 in every key adds 0.5 * a to every logit
    q2 = np.concatenate([q, np.full((4, 2, 1), 3000.0)], axis=2)
    k2 = np.concatenate([k, np.ones((15, 1, 1))], axis=2)
    v2 = np.concatenate([v, np.zeros((15, 1, 1))], axis=2)
    np.testing.assert_allclose(full_attention(q2, k2, v2, 0.5)[..., :6], base, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (8, 1), (4, 2)])
def test_torch_sdpa_float64(hq, hkv):
    r = np.random.default_rng(11 + hq)
    n, t, d = 7, 40, 16
    q, k, v = r.normal(size=(n, hq, d)), r.normal(size=(t, hkv, d)), r.normal(size=(t, hkv, d))
    tq = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq][N][D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(full_attention(q, k, v, 0.25), want, atol=1e-13)


def _partial(q, k, v, scale):
    """Unnormalised partial softmax of one region: (m, l, o) per (token, head)."""
    grp = q.shape[1] // k.shape[1]
    kk = np.repeat(k, grp, axis=1)
    vv = np.repeat(v, grp, axis=1)
    z = scale * np.einsum("nhd,thd->nht", q, kk)
    m = z.max(axis=2)
    p = np.exp(z - m[..., None])
    return m, p.sum(axis=2), np.einsum("nht,thd->nhd", p, vv)


def test_prop_a1_lse_merge_of_regions_equals_full():
    r = np.random.default_rng(12)
    hq, hkv, d, n = 4, 1, 8, 5
    pin = [r.normal(size=(6, hkv, d)) for _ in range(2)]
    frames = [[r.normal(size=(5, hkv, d)) for _ in range(3)] for _ in range(2)]
    dyn = [r.normal(size=(n, hkv, d)) for _ in range(2)]
    q = r.normal(size=(n, hq, d))
    full = partitioned_reference(q, pin[0], pin[1], frames[0], frames[1], dyn[0], dyn[1], 0.35)
    regions = [(pin[0], pin[1])] + list(zip(frames[0], frames[1])) + [(dyn[0], dyn[1])]
    parts = [_partial(q, a, b, 0.35) for a, b in regions]
    m = np.max([p[0] for p in parts], axis=0)
    lsum = sum(p[1] * np.exp(p[0] - m) for p in parts)
    osum = sum(p[2] * np.exp(p[0] - m)[..., None] for p in parts)
    np.testing.assert_allclose(osum / lsum[..., None], full, atol=1e-13)


def test_prop_a1_slot_order_does_not_matter():
    """The ring stores frames in slot order, not chronological order."""
    r = np.random.default_rng(13)
    hq, hkv, d, n = 8, 1, 16, 4
    pk, pv = r.normal(size=(3, hkv, d)), r.normal(size=(3, hkv, d))
    fk = [r.normal(size=(4, hkv, d)) for _ in range(5)]
    fv = [r.normal(size=(4, hkv, d)) for _ in range(5)]
    dk, dv = r.normal(size=(n, hkv, d)), r.normal(size=(n, hkv, d))
    q = r.normal(size=(n, hq, d))
    chrono = partitioned_reference(q, pk, pv, fk, fv, dk, dv, 0.25)
    order = [3, 4, 0, 1, 2]                           # a wrapped ring: head at slot 3
    slotted = partitioned_reference(q, pk, pv, [fk[i] for i in order], [fv[i] for i in order], dk, dv, 0.25)
    np.testing.assert_allclose(slotted, chrono, atol=1e-13)
    perm = r.permutation(3 + 20 + n)                  # any token permutation at all
    ck = build_context(pk, fk, dk)[perm]
    cv = build_context(pv, fv, dv)[perm]
    np.testing.assert_allclose(full_attention(q, ck, cv, 0.25), chrono, atol=1e-13)


def test_build_context_order_and_length():
    a = np.zeros((2, 1, 1)); b = np.ones((3, 1, 1)); c = 2 * np.ones((1, 1, 1)); e = 3 * np.ones((4, 1, 1))
    ctx = build_context(a, [b, c], e)
    assert ctx.shape == (10, 1, 1)
    assert list(ctx[:, 0, 0]) == [0, 0, 1, 1, 1, 2, 3, 3, 3, 3]


def _table4():
    rows = {}
    with open(os.path.join(GOLDEN, "reflex_table4_mse.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, val = line.split(",")
                rows[name.strip()] = float(val)
    return rows


def test_table4_partitioned_equals_full_and_naive_cache_does_not():
    """Table 4: partitioned MSE prints as 0.00, the naive cache as 1.42 (> 1.0).

    The naive cache reuses the suffix KV of step 0 at a later step; with
    unit-variance synthetic values its error is of order one, the same
    order as the page's 1.42, while the partitioned result is exact.
    """
    t4 = _table4()
    r = np.random.default_rng(14)
    hq, hkv, d, n = 8, 1, 32, 51
    pk, pv = r.normal(size=(16, hkv, d)), r.normal(size=(16, hkv, d))
    fk = [r.normal(size=(32, hkv, d)) for _ in range(2)]
    fv = [r.normal(size=(32, hkv, d)) for _ in range(2)]
    # step k: queries and the suffix's own k/v change with the step
    q0, q5 = r.normal(size=(n, hq, d)), r.normal(size=(n, hq, d))
    dk0, dv0 = r.normal(size=(n, hkv, d)), r.normal(size=(n, hkv, d))
    dk5, dv5 = r.normal(size=(n, hkv, d)), r.normal(size=(n, hkv, d))
    full = full_attention(q5, build_context(pk, fk, dk5), build_context(pv, fv, dv5), 1 / math.sqrt(d))
    part = partitioned_reference(q5, pk, pv, fk, fv, dk5, dv5, 1 / math.sqrt(d))
    naive = partitioned_reference(q5, pk, pv, fk, fv, dk0, dv0, 1 / math.sqrt(d))
    mse_part = float(np.mean((part - full) ** 2))
    mse_naive = float(np.mean((naive - full) ** 2))
    assert t4["partitioned"] == 0.0 and mse_part < 0.005
    assert t4["naive_cache"] > 1.0
    assert mse_naive > 1e3 * max(mse_part, 1e-30)
    assert mse_naive > 1e-3
    del q0
