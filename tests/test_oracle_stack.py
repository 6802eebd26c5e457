"""Pins of the layer glue oracle (QKV split, out-projection, Euler) and of the
shared-KV decode oracle. The end-to-end denoising step is pinned against the
same step written with torch's own float64 operators, on inputs chosen so
that a wiring mistake (wrong stream fed forward, wrong gamma, wrong velocity,
a dropped attention region) fails it; closed forms fix the pieces.
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
    """All keys zero, so every logit is 0 and attention is the plain mean of
    the values over the whole context [cache; step]. The cache's values are
    c1 (T rows) and the step's own values are c2 (n rows, produced by W_v from
    a row-constant y), so o = (T c1 + n c2) / (T + n). Dropping the step's
    K/V would give c1, dropping the cache c2."""
    hq, hkv, d, model, n, T = 2, 1, 4, 4, 3, 5
    c1 = np.array([0.5, -1.0, 2.0, 0.25])
    c2 = np.array([-2.0, 1.5, 0.75, 3.0])
    w = np.zeros(((hq + 2) * d, model))
    h = np.ones((n, model))                 # unit RMS, so y = 1 in every column
    w[(hq + hkv) * d:, 0] = c2              # v_step = c2 * y[:, 0] = c2
    res = stack.layer(h, np.ones(model), 0.0, w, np.zeros((T, hkv, d)), np.broadcast_to(c1, (T, hkv, d)),
                      np.zeros((model, hq * d)), 1.0, hq, hkv, d)
    want = round_bf16((T * c1 + n * c2) / (T + n))
    np.testing.assert_allclose(res["o"], np.broadcast_to(want, (n, hq, d)))
    assert not np.allclose(want, round_bf16(c1)) and not np.allclose(want, round_bf16(c2))


# ------------------------------------------- the denoising step end to end ----
# An independent pin of the layer glue: the same step written with torch's
# own float64 operators (F.rms_norm with the gamma as its weight, a matmul
# for the packed projection, F.scaled_dot_product_attention over
# cat([cache, step K/V]) with the KV heads repeated for their query heads,
# F.silu for the FFN, and torch's bf16 conversion at every bf16 store). The
# inputs make every part of the wiring matter: a nonzero out-projection,
# a different gamma per layer, different cache and step K/V, two KV heads.

def _torch_denoise_step(x, gammas, eps, wqkv, wo, ck, cv, scale, hq, hkv, d, ffns=None, dt=0.1):
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)   # noqa: E731
    bf = lambda v: v.to(torch.bfloat16).to(torch.float64)                          # noqa: E731
    n, model = x.shape
    h = t(x)
    hs, os_ = [], []
    for l in range(len(wqkv)):
        y = bf(F.rms_norm(h, (model,), weight=t(gammas[l]), eps=eps))
        qkv = y @ t(wqkv[l]).T
        q = bf(qkv[:, :hq * d]).reshape(n, hq, d)
        k = bf(qkv[:, hq * d:(hq + hkv) * d]).reshape(n, hkv, d)
        v = bf(qkv[:, (hq + hkv) * d:]).reshape(n, hkv, d)
        K = torch.cat([t(ck[l]), k], 0).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        V = torch.cat([t(cv[l]), v], 0).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        o = F.scaled_dot_product_attention(q.permute(1, 0, 2), K, V, scale=scale)
        o = bf(o.permute(1, 0, 2).reshape(n, hq * d))
        h = bf(h + o @ t(wo[l]).T)
        if ffns is not None:
            g2, wg, wu, wd = ffns[l]
            y2 = bf(F.rms_norm(h, (model,), weight=t(g2), eps=eps))
            act = bf(F.silu(y2 @ t(wg).T) * (y2 @ t(wu).T))
            h = bf(h + act @ t(wd).T)
        os_.append(o.numpy().reshape(n, hq, d))
        hs.append(h.numpy())
    return bf(t(x) - dt * h).numpy(), hs, os_


def _glue_case(L=3, n=5, model=32, hq=4, hkv=2, d=8, T=7, ffn=0, seed=21):
    rng = np.random.default_rng(seed)
    r = lambda *s: rng.standard_normal(s)          # noqa: E731
    x = round_bf16(r(n, model))
    gammas = [1.0 + 0.4 * r(model) for _ in range(L)]
    wqkv = [round_bf16(r((hq + 2 * hkv) * d, model) / np.sqrt(model)) for _ in range(L)]
    wo = [round_bf16(r(model, hq * d) / np.sqrt(hq * d)) for _ in range(L)]
    ck = [round_bf16(r(T, hkv, d)) for _ in range(L)]
    cv = [round_bf16(r(T, hkv, d)) for _ in range(L)]
    ffns = None
    if ffn:
        ffns = [(1.0 + 0.3 * r(model), round_bf16(r(ffn, model) / np.sqrt(model)),
                 round_bf16(r(ffn, model) / np.sqrt(model)), round_bf16(r(model, ffn) / np.sqrt(ffn)))
                for _ in range(L)]
    return dict(x=x, gammas=gammas, eps=1e-6, wqkv=wqkv, wo=wo, ck=ck, cv=cv, scale=1 / np.sqrt(d), hq=hq,
                hkv=hkv, d=d, ffns=ffns)


def _oracle_step(c):
    x1, trace = stack.denoise_step(c["x"], c["gammas"], c["eps"], c["wqkv"], c["wo"], c["ck"], c["cv"], c["scale"],
                                   c["hq"], c["hkv"], c["d"], c["ffns"])
    return x1, [tr["h"] for tr in trace], [tr["o"] for tr in trace]


def _glue_error(c):
    """Worst relative difference (per tensor, max|a - b| / max|b|) between the
    oracle's step and the torch chain over x_{k+1}, every layer's h and o."""
    x1, hs, os_ = _oracle_step(c)
    tx1, ths, tos = _torch_denoise_step(c["x"], c["gammas"], c["eps"], c["wqkv"], c["wo"], c["ck"], c["cv"],
                                        c["scale"], c["hq"], c["hkv"], c["d"], c["ffns"])
    rel = lambda a, b: float(np.max(np.abs(a - b)) / np.max(np.abs(b)))   # noqa: E731
    return max([rel(x1, tx1)] + [rel(a, b) for a, b in zip(hs, ths)] + [rel(a, b) for a, b in zip(os_, tos)])


# Both sides compute in float64 and round to bf16 at the same points, so they
# differ only where a float64 summation-order difference flips a bf16
# rounding; one flip moves a value by at most 2^-8 of itself.
GLUE_TOL = 2.0 ** -8


@pytest.mark.parametrize("ffn", [0, 64])
def test_denoise_step_matches_a_torch_float64_chain(ffn):
    c = _glue_case(ffn=ffn)
    assert _glue_error(c) <= GLUE_TOL


def test_denoise_step_pin_catches_planted_wiring_mistakes(monkeypatch):
    """Each mistake below is planted in the oracle (by patching the names the
    oracle's step calls) and must make the torch-chain pin fail."""
    c = _glue_case()
    assert _glue_error(c) <= GLUE_TOL
    real_layer, real_attn, real_euler = stack.layer, stack.full_attention, stack.euler

    def plant(name, fn):
        with monkeypatch.context() as m:
            m.setattr(stack, name, fn)
            err = _glue_error(c)
        assert err > 10 * GLUE_TOL, f"the pin did not catch the planted mistake ({name}): {err:.3g}"

    first = {}

    def layer_fed_x(h, *a, **k):               # every layer reads x instead of h_{l-1}
        first.setdefault("h", h)
        return real_layer(first["h"], *a, **k)
    plant("layer", layer_fed_x)

    first.clear()

    def layer_gamma0(h, g, *a, **k):            # every layer uses gamma_0
        first.setdefault("g", g)
        return real_layer(h, first["g"], *a, **k)
    plant("layer", layer_gamma0)

    hist = []

    def layer_rec(*a, **k):
        r = real_layer(*a, **k)
        hist.append(r["h"])
        return r

    def euler_h1(x, v, dt=0.1):                 # velocity taken from h_1
        return real_euler(x, hist[0], dt)
    with monkeypatch.context() as m:
        m.setattr(stack, "layer", layer_rec)
        m.setattr(stack, "euler", euler_h1)
        err = _glue_error(c)
    assert err > 10 * GLUE_TOL

    n = c["x"].shape[0]
    plant("full_attention", lambda q, k, v, s: real_attn(q, k[:-n], v[:-n], s))    # step K/V dropped
    plant("full_attention", lambda q, k, v, s: real_attn(q, k[-n:], v[-n:], s))    # cache dropped
    plant("full_attention", lambda q, k, v, s: real_attn(q, k, v, s * 2))          # scale applied twice


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
