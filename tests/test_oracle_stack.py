"""Pins of the layer glue oracle (QKV split, out-projection, Euler) and of the
shared-KV decode oracle. The end-to-end denoising step chains pinned ops and
is itself "parity unpinned" (the pages give no layer glue); the checks here
fix its wiring with cases whose answer is known in closed form.
"""

import numpy as np
import pytest

from oracle import stack, decode
from oracle.adanorm import round_bf16
from oracle.attention import full_attention


def test_qkv_split_order_by_unit_vectors():
    hq, hkv, d, model = 3, 1, 4, 6
    rows = (hq + 2 * hkv) * d
    w = np.arange(rows * model, dtype=np.float64).reshape(rows, model)
    for j in range(model):
        y = np.zeros((1, model)); y[0, j] = 1.0
        q, k, v = stack.qkv_projection(y, w, hq, hkv, d)
        for h in range(hq):
            for e in range(d):
                assert q[0, h, e] == w[h * d + e, j]
        for e in range(d):
            assert k[0, 0, e] == w[hq * d + e, j]
            assert v[0, 0, e] == w[(hq + hkv) * d + e, j]


def test_out_projection_flattens_heads_in_order():
    r = np.random.default_rng(1)
    o = r.normal(size=(2, 3, 4))
    w = r.normal(size=(5, 12))
    h = r.normal(size=(2, 5))
    want = np.array([[h[i, m] + sum(o[i, hh, e] * w[m, hh * 4 + e] for hh in range(3) for e in range(4))
                      for m in range(5)] for i in range(2)])
    np.testing.assert_allclose(stack.out_projection_residual(h, o, w), want, atol=1e-12)


def test_euler_closed_forms():
    x = round_bf16(np.random.default_rng(2).normal(size=(4, 8)))
    assert np.array_equal(stack.euler(x, np.zeros_like(x)), x)
    assert np.array_equal(stack.euler(x, x), round_bf16(0.9 * x))
    assert stack.timesteps(10) == [1.0, 0.9, 0.8, 0.7, 0.6, 0.5, 0.4, 0.30000000000000004, 0.19999999999999996,
                                   0.09999999999999998]


def test_layer_with_zero_out_projection_keeps_the_stream():
    r = np.random.default_rng(3)
    hq, hkv, d, model, n = 2, 1, 8, 16, 5
    h = round_bf16(r.normal(size=(n, model)))
    res = stack.layer(h, np.ones(model), 1e-6, r.normal(size=((hq + 2) * d, model)) * 0.1,
                      r.normal(size=(7, hkv, d)), r.normal(size=(7, hkv, d)), np.zeros((model, hq * d)),
                      0.3, hq, hkv, d)
    assert np.array_equal(res["h"], h)
    assert res["o"].shape == (n, hq, d)


def test_denoise_step_with_zero_out_projection_is_x_times_0_9():
    r = np.random.default_rng(4)
    L, hq, hkv, d, model, n = 3, 2, 1, 4, 8, 3
    x = round_bf16(r.normal(size=(n, model)))
    x1, trace = stack.denoise_step(
        x, [np.ones(model)] * L, 1e-6, [r.normal(size=((hq + 2) * d, model)) for _ in range(L)],
        [np.zeros((model, hq * d))] * L, [r.normal(size=(6, hkv, d))] * L, [r.normal(size=(6, hkv, d))] * L,
        0.5, hq, hkv, d)
    assert len(trace) == L
    assert np.array_equal(x1, round_bf16(0.9 * x))


def test_layer_attention_appends_step_kv_after_cache():
    """With the cache's values all equal to c, and W_v producing c too, o = c."""
    hq, hkv, d, model, n = 2, 1, 4, 4, 3
    c = np.array([0.5, -1.0, 2.0, 0.25])
    w = np.zeros(((hq + 2) * d, model))
    w[(hq + hkv) * d:, :] = 0.0
    # y has unit RMS rows; make v = y @ Wv^T = const c by using a row-constant y
    h = np.ones((n, model))
    w[(hq + hkv) * d:, 0] = c              # v = c * y[:, 0] = c * 1
    res = stack.layer(h, np.ones(model), 0.0, w, np.zeros((5, hkv, d)), np.broadcast_to(c, (5, hkv, d)),
                      np.zeros((model, hq * d)), 1.0, hq, hkv, d)
    np.testing.assert_allclose(res["o"], np.broadcast_to(round_bf16(c), (n, hq, d)))


def test_decode_streams_see_only_their_own_tail():
    r = np.random.default_rng(5)
    hq, hkv, d, g = 4, 1, 8, 3
    shared_k, shared_v = r.normal(size=(10, hkv, d)), r.normal(size=(10, hkv, d))
    tails = decode.PrivateTails(g, 4, hkv, d)
    for j in range(g):
        for _ in range(j + 1):
            tails.append(j, r.normal(size=(hkv, d)), r.normal(size=(hkv, d)))
    q = r.normal(size=(g, hq, d))
    out = decode.decode_attention(q, shared_k, shared_v, tails, 0.3)
    for j in range(g):
        n = j + 1
        want = full_attention(q[j:j + 1], np.concatenate([shared_k, tails.k[j, :n]]),
                              np.concatenate([shared_v, tails.v[j, :n]]), 0.3)[0]
        np.testing.assert_allclose(out[j], want, atol=1e-14)
    # changing stream 0's tail leaves stream 1 alone
    tails.k[0, 0] += 5.0
    out2 = decode.decode_attention(q, shared_k, shared_v, tails, 0.3)
    assert np.array_equal(out2[1], out[1]) and not np.allclose(out2[0], out[0])


def test_decode_tail_capacity_and_retire():
    tails = decode.PrivateTails(1, 2, 1, 2)
    tails.append(0, np.zeros((1, 2)), np.zeros((1, 2)))
    tails.append(0, np.zeros((1, 2)), np.zeros((1, 2)))
    with pytest.raises(ValueError):
        tails.append(0, np.zeros((1, 2)), np.zeros((1, 2)))
    tails.reset(0)
    assert tails.length[0] == 0


def test_retire_full_starts_a_new_request():
    """OxyGen review, method details: a request ends at its maximum length. With
    retiring on, a full stream's next token starts a new request: its query sees
    the shared context plus that one token only (checked against the plain
    definition, full attention over [shared; new token])."""
    rng = np.random.default_rng(7)
    shared_k, shared_v = rng.standard_normal((5, 1, 4)), rng.standard_normal((5, 1, 4))
    tails = decode.PrivateTails(2, 3, 1, 4)
    for _ in range(3):
        tails.append(0, rng.standard_normal((1, 4)), rng.standard_normal((1, 4)))
    tails.append(1, rng.standard_normal((1, 4)), rng.standard_normal((1, 4)))
    kn, vn = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    tails.append(0, kn, vn, retire_full=True)          # full: a new request
    tails.append(1, kn, vn, retire_full=True)          # not full: an ordinary append
    assert list(tails.length) == [1, 2]
    q = rng.standard_normal((2, 2, 4))
    got = decode.decode_attention(q, shared_k, shared_v, tails, 0.5)
    want0 = full_attention(q[0:1], np.concatenate([shared_k, kn[None]]), np.concatenate([shared_v, vn[None]]), 0.5)[0]
    assert np.allclose(got[0], want0, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------- SwiGLU FFN ----
# The FFN block is a reading (the pages name "SwiGLU fusion" among the fused
# operators but give no layer): pinned against torch's own rms_norm, silu,
# matmul and bf16 conversion in float64, plus identities.

def _torch_ffn(h, gamma, eps, wg, wu, wd):
    import torch
    t = lambda a: torch.tensor(a, dtype=torch.float64)          # noqa: E731
    bf = lambda v: v.to(torch.bfloat16).to(torch.float64)       # noqa: E731
    y = bf(torch.nn.functional.rms_norm(t(h), (h.shape[1],), weight=t(gamma), eps=eps))
    act = bf(torch.nn.functional.silu(y @ t(wg).T) * (y @ t(wu).T))
    return bf(t(h) + act @ t(wd).T).numpy(), act.numpy()


@pytest.mark.parametrize("n,d,f", [(5, 8, 16), (51, 64, 256)])
def test_ffn_swiglu_against_torch(n, d, f):
    rng = np.random.default_rng(11 + n)
    h = round_bf16(rng.standard_normal((n, d)))
    gamma = 1.0 + 0.1 * rng.standard_normal(d)
    wg, wu = rng.uniform(-1, 1, (f, d)) / np.sqrt(d), rng.uniform(-1, 1, (f, d)) / np.sqrt(d)
    wd = rng.uniform(-1, 1, (d, f)) / np.sqrt(f)
    wg, wu, wd = round_bf16(wg), round_bf16(wu), round_bf16(wd)
    got = stack.ffn_swiglu(h, gamma, 1e-6, wg, wu, wd)
    want_h, want_act = _torch_ffn(h, gamma, 1e-6, wg, wu, wd)
    assert np.array_equal(got["act"], want_act) or np.max(np.abs(got["act"] - want_act)) <= 2.0 ** -7 * np.max(np.abs(want_act))
    assert np.max(np.abs(got["h"] - want_h)) <= 2.0 ** -7 * np.max(np.abs(want_h))
    # gate and up are not interchangeable: swapping them changes the result
    swapped = stack.ffn_swiglu(h, gamma, 1e-6, wu, wg, wd)
    assert not np.allclose(swapped["act"], got["act"])


def test_ffn_swiglu_identities():
    rng = np.random.default_rng(3)
    h = round_bf16(rng.standard_normal((4, 8)))
    gamma = np.ones(8)
    wg, wu, wd = rng.standard_normal((16, 8)), rng.standard_normal((16, 8)), rng.standard_normal((8, 16))
    for g_, u_, d_ in ((wg, wu, 0 * wd), (0 * wg, wu, wd), (wg, 0 * wu, wd)):
        r = stack.ffn_swiglu(h, gamma, 1e-6, g_, u_, d_)
        assert np.array_equal(r["h"], h)            # a zero factor leaves the stream alone
    # SiLU(g) * u with one-hot rows: act = silu(y_i) * y_j exactly before rounding
    e = np.eye(8)
    r = stack.ffn_swiglu(h, gamma, 1e-6, e[[0, 1]], e[[2, 3]], np.zeros((8, 2)))
    y = r["y2"]
    want = round_bf16(y[:, [0, 1]] / (1 + np.exp(-y[:, [0, 1]])) * y[:, [2, 3]])
    assert np.array_equal(r["act"], want)


def test_layer_with_ffn_chains_after_the_attention_residual():
    rng = np.random.default_rng(5)
    n, d, hd = 3, 256, 64
    h = round_bf16(rng.standard_normal((n, d)))
    wqkv = round_bf16(rng.uniform(-1, 1, ((4 + 2) * hd, d)) / 16)
    wo = round_bf16(rng.uniform(-1, 1, (d, 4 * hd)) / 16)
    ck, cv = rng.standard_normal((5, 1, hd)), rng.standard_normal((5, 1, hd))
    ffn = (np.ones(d), round_bf16(rng.uniform(-1, 1, (512, d)) / 16), round_bf16(rng.uniform(-1, 1, (512, d)) / 16),
           round_bf16(rng.uniform(-1, 1, (d, 512)) / 22))
    r = stack.layer(h, np.ones(d), 1e-6, wqkv, ck, cv, wo, 0.125, 4, 1, hd, ffn=ffn)
    plain = stack.layer(h, np.ones(d), 1e-6, wqkv, ck, cv, wo, 0.125, 4, 1, hd)
    assert np.array_equal(r["h_attn"], plain["h"])
    assert np.array_equal(r["h"], stack.ffn_swiglu(plain["h"], *ffn[:1], 1e-6, *ffn[1:])["h"])
