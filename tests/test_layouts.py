"""The element-index formulas include/pattn.h documents for the
fragment-packed weights (pa_pack_weight) and for operand-order queries
(PA_Q_OPERAND), written out per element here, against the numpy reshapes
that the GPU tests compare the kernels with. Host-only."""

import numpy as np
import pytest


def weight_index(r, c, k):
    # (((r / 32) * (k / 16) + c / 16) * 64 + ((c / 8) % 2) * 32 + r % 32) * 8 + c % 8
    return (((r // 32) * (k // 16) + c // 16) * 64 + ((c // 8) % 2) * 32 + r % 32) * 8 + c % 8


def weight_reshape(w):
    n, k = w.shape
    return w.reshape(n // 32, 32, k // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("n,k", [(32, 16), (64, 48), (96, 128)])
def test_weight_formula_matches_reshape(n, k):
    w = np.arange(n * k, dtype=np.int64).reshape(n, k)
    out = np.empty(n * k, dtype=np.int64)
    for r in range(n):
        for c in range(k):
            out[weight_index(r, c, k)] = w[r, c]
    np.testing.assert_array_equal(out, weight_reshape(w))


def test_stacked_layers_pack_in_place():
    L_, n, k = 3, 64, 32
    w = np.arange(L_ * n * k, dtype=np.int64).reshape(L_ * n, k)
    whole = weight_reshape(w)
    for l in range(L_):
        np.testing.assert_array_equal(whole[l * n * k:(l + 1) * n * k], weight_reshape(w[l * n:(l + 1) * n]))


def q_index(l, g, r, d, hkv, nb, D):
    # ((((l*Hkv + g)*nb + r/32)*(D/16) + d/16)*64 + ((d/8)%2)*32 + r%32)*8 + d%8
    return ((((l * hkv + g) * nb + r // 32) * (D // 16) + d // 16) * 64 + ((d // 8) % 2) * 32 + r % 32) * 8 + d % 8


def q_reshape(q, hkv):
    lb, n, hq, d = q.shape
    g = hq // hkv
    nb = (n * g + 31) // 32
    out = []
    for l in range(lb):
        for h in range(hkv):
            rows = q[l, :, h * g:(h + 1) * g, :].reshape(n * g, d)
            pad = np.zeros((nb * 32, d), dtype=q.dtype)
            pad[:n * g] = rows
            out.append(pad.reshape(nb, 32, d // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1))
    return np.concatenate(out)


@pytest.mark.parametrize("lb,n,hq,hkv,D", [(2, 5, 4, 2, 32), (1, 51, 8, 1, 64), (2, 3, 6, 3, 16)])
def test_operand_q_formula_matches_reshape(lb, n, hq, hkv, D):
    q = np.arange(1, lb * n * hq * D + 1, dtype=np.int64).reshape(lb, n, hq, D)
    g = hq // hkv
    nb = (n * g + 31) // 32
    out = np.zeros(lb * hkv * nb * 32 * D, dtype=np.int64)
    for l in range(lb):
        for t in range(n):
            for h in range(hq):
                r = t * g + h % g            # row r of KV head h / G is (token r / G, head g*G + r % G)
                for d in range(D):
                    out[q_index(l, h // g, r, d, hkv, nb, D)] = q[l, t, h, d]
    np.testing.assert_array_equal(out, q_reshape(q, hkv))
