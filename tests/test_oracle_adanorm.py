"""Pins of the AdaRMSNorm oracle (Eq. 2 of the Reflex paper review, §3; the
module in §5): torch's rms_norm and nn.Linear/SiLU in float64, torch's own
bf16 conversion, closed forms of the embedding and of constant rows, and
scale invariance.
"""

import math

import numpy as np
import pytest
import torch

from oracle import adanorm
from partitioned_kv_cache_amd import synth


def test_round_bf16_matches_torch_on_float32_values():
    r = np.random.default_rng(0)
    x = np.concatenate([r.normal(size=5000), r.normal(size=5000) * 1e-3, r.normal(size=5000) * 1e4]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(adanorm.round_bf16(x.astype(np.float64)), want)


def test_round_bf16_ties_to_even():
    ulp = 2.0 ** -7                   # bf16 spacing in [1, 2)
    assert adanorm.round_bf16(np.array([1 + ulp / 2]))[0] == 1.0             # tie -> even (1.0)
    assert adanorm.round_bf16(np.array([1 + 1.5 * ulp]))[0] == 1 + 2 * ulp   # tie -> even
    assert adanorm.round_bf16(np.array([1 + ulp / 2 + 1e-9]))[0] == 1 + ulp


def test_round_bf16_agrees_with_the_input_generator():
    x = np.random.default_rng(1).normal(size=4096).astype(np.float32)
    assert np.array_equal(adanorm.round_bf16(x.astype(np.float64)), synth.widen(synth.f32_to_bf16_bits(x)))


def test_embedding_closed_forms():
    e0 = adanorm.timestep_embedding(0.0)
    assert e0.shape == (128,) and np.all(e0[:64] == 0.0) and np.all(e0[64:] == 1.0)
    for t in (1.0, 0.3, 0.9):
        e = adanorm.timestep_embedding(t)
        np.testing.assert_allclose(e[:64] ** 2 + e[64:] ** 2, 1.0, atol=1e-15)
        assert e[0] == math.sin(t) and e[64] == math.cos(t)          # lowest frequency is 1
        assert abs(e[63] - math.sin(t * 10000 ** (-63 / 64))) < 1e-16  # highest index, slowest


def test_gamma_identity_reduces_to_torch_rms_norm():
    r = np.random.default_rng(2)
    x = r.normal(size=(51, 64)) * 3
    w1, b1 = r.normal(size=(32, 160)), r.normal(size=32)
    g = adanorm.gamma(w1, b1, np.zeros((64, 32)), np.zeros(64), 0.5, r.normal(size=32))
    assert np.all(g == 1.0)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), eps=1e-6).numpy()
    np.testing.assert_allclose(adanorm.rmsnorm_scaled(x, g, 1e-6), want, atol=1e-13)


def test_constant_row_closed_form():
    gam = np.linspace(0.5, 1.5, 16)
    for a in (1e-4, 0.5, -7.0):
        y = adanorm.rmsnorm_scaled(np.full((2, 16), a), gam, 1e-6)
        np.testing.assert_allclose(y, np.broadcast_to(a / math.sqrt(a * a + 1e-6) * gam, (2, 16)), rtol=1e-14)


def test_scale_invariance_when_eps_is_negligible():
    r = np.random.default_rng(3)
    x, gam = r.normal(size=(4, 1024)), r.normal(size=1024)
    np.testing.assert_allclose(adanorm.rmsnorm_scaled(1e3 * x, gam, 1e-6),
                               adanorm.rmsnorm_scaled(x, gam, 1e-6), rtol=1e-6)


def test_eps_sits_inside_the_square_root():
    # one nonzero element: RMS = sqrt(a^2/d + eps)
    x = np.zeros((1, 4)); x[0, 0] = 0.01
    y = adanorm.rmsnorm_scaled(x, np.ones(4), 1e-4)
    assert abs(y[0, 0] - 0.01 / math.sqrt(0.01 ** 2 / 4 + 1e-4)) < 1e-15


def test_gamma_matches_torch_linear_silu_linear():
    """1 + Linear(SiLU(Linear(c))) in float64 with bf16 rounding of c and the hidden layer."""
    r = np.random.default_rng(4)
    cond, hid, model = 160, 96, 80
    w1 = synth.widen(synth.f32_to_bf16_bits(r.uniform(-0.08, 0.08, (hid, cond)).astype(np.float32)))
    b1 = synth.widen(synth.f32_to_bf16_bits(r.uniform(-0.08, 0.08, hid).astype(np.float32)))
    w2 = synth.widen(synth.f32_to_bf16_bits(r.uniform(-0.1, 0.1, (model, hid)).astype(np.float32)))
    b2 = synth.widen(synth.f32_to_bf16_bits(r.uniform(-0.1, 0.1, model).astype(np.float32)))
    state = synth.widen(synth.f32_to_bf16_bits(r.normal(size=32).astype(np.float32)))
    l1 = torch.nn.Linear(cond, hid, dtype=torch.float64)
    l2 = torch.nn.Linear(hid, model, dtype=torch.float64)
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(w1)); l1.bias.copy_(torch.from_numpy(b1))
        l2.weight.copy_(torch.from_numpy(w2)); l2.bias.copy_(torch.from_numpy(b2))
        for t in (1.0, 0.6, 0.1):
            c = adanorm.condition(t, state)
            a = torch.nn.functional.silu(l1(torch.from_numpy(c)))
            a = a.to(torch.float32).to(torch.bfloat16).to(torch.float64)
            want = 1.0 + l2(a).numpy()
            np.testing.assert_allclose(adanorm.gamma(w1, b1, w2, b2, t, state), want, atol=1e-12)


def test_condition_layout_is_embedding_then_state():
    s = np.arange(32) / 8.0
    c = adanorm.condition(0.0, s)
    assert c.shape == (160,)
    assert np.all(c[:64] == 0) and np.all(c[64:128] == 1) and np.array_equal(c[128:], s)


@pytest.mark.parametrize("t", [1.0, 0.0])
def test_ada_rmsnorm_composes_gamma_and_norm(t):
    r = np.random.default_rng(5)
    x = r.normal(size=(3, 24))
    w1, b1, w2, b2 = r.normal(size=(8, 160)) * 0.1, r.normal(size=8) * 0.1, r.normal(size=(24, 8)) * 0.1, r.normal(size=24) * 0.1
    s = r.normal(size=32)
    g = adanorm.gamma(w1, b1, w2, b2, t, s)
    rms = np.sqrt(np.mean(x ** 2, axis=1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(adanorm.ada_rmsnorm(x, w1, b1, w2, b2, t, s, 1e-6), x / rms * g, rtol=1e-14)
