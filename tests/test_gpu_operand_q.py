"""GPU tests of the PA_Q_OPERAND query layout (q already in the order the
matrix-core kernel consumes it).

pattn_pack_q is a permutation of bf16 words, checked bit for bit against the
layout written out here with numpy reshapes. pattn_step on the converted q
feeds the kernel exactly the same operands as on token-major q, so its output
must be bit-identical; it also meets the oracle bar (2e-2 relative).
"""

import math

import numpy as np
import pytest
import torch

from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, host, lib, rel_err  # noqa: E402

BF16_REL = 2e-2


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


def _operand_numpy(q: np.ndarray, hkv: int) -> np.ndarray:
    """[Lb][N][Hq][D] -> [Lb*Hkv][nb][D/16][2][32][8], flattened (padding rows zero)."""
    lb, n, hq, d = q.shape
    g = hq // hkv
    nb = (n * g + 31) // 32
    out = []
    for l in range(lb):
        for h in range(hkv):
            rows = q[l, :, h * g:(h + 1) * g, :].reshape(n * g, d)          # row r = token * G + head within group
            pad = np.zeros((nb * 32, d), dtype=q.dtype)
            pad[:n * g] = rows
            out.append(pad.reshape(nb, 32, d // 16, 2, 8).transpose(0, 2, 3, 1, 4).reshape(-1))
    return np.concatenate(out)


def _shape(D, hq, hkv, N, L=2):
    return configs.PI05_1L.with_(name="opq", cfg_id=60 + D + hq + N, num_layers=L, n_q_heads=hq, n_kv_heads=hkv,
                                 head_dim=D, pin_tokens=16, num_slots=2, tokens_per_frame=64, n_dyn=N,
                                 scale=1 / math.sqrt(D))


@pytest.mark.parametrize("D,hq,hkv,N", [(256, 8, 1, 51), (128, 4, 2, 5), (64, 6, 3, 17), (256, 8, 1, 64)])
def test_pack_q_matches_layout(D, hq, hkv, N):
    L = lib()
    s = _shape(D, hq, hkv, N)
    _banner(f"pattn_pack_q D={D} hq={hq} hkv={hkv} N={N}")
    sc = Scenario(s)
    q = synth.suffix_qkv(s, 0, 0)[0]
    args = L.pattn_args(0, s.num_layers, hq, N, s.scale, L.PA_BF16, 0, L.PA_Q_OPERAND)
    nbytes = L.pattn_operand_q_bytes(sc.ring, args)
    ref = _operand_numpy(q, hkv)
    assert nbytes == ref.size * 2
    out = torch.full((nbytes // 2,), -1, dtype=torch.int16, device="cuda")      # padding must come back zero
    L.pattn_pack_q(sc.ring, args, dev(q), out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), ref)


EDGE = [
    # (D, Hq, Hkv, P, pinned, W, F, N, frames, splits)
    (64, 1, 1, 0, 0, 3, 5, 1, 4, 0),
    (128, 4, 2, 7, 3, 2, 33, 5, 3, 0),
    (256, 2, 1, 40, 40, 4, 100, 3, 9, 7),
    (128, 8, 1, 300, 300, 2, 64, 51, 0, 0),
]


@pytest.mark.parametrize("D,hq,hkv,P,pinned,W,F,N,frames,splits", EDGE)
def test_operand_q_bit_identical_to_token_major(D, hq, hkv, P, pinned, W, F, N, frames, splits):
    L = lib()
    _banner(f"operand-order q D={D} hq={hq} hkv={hkv} N={N} frames={frames} splits={splits}")
    s = configs.PI05_1L.with_(name="opq_edge", cfg_id=70 + D + hq, num_layers=2, n_q_heads=hq, n_kv_heads=hkv,
                              head_dim=D, pin_tokens=P, num_slots=W, tokens_per_frame=F, n_dyn=N,
                              scale=1 / math.sqrt(D))
    sc = Scenario(s, pin_tokens=pinned)
    for f in range(frames):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s, frames, 3)
    a = sc.run_step(q, kd, vd, num_splits=splits)
    b = sc.run_step(q, kd, vd, num_splits=splits, q_layout=L.PA_Q_OPERAND)
    np.testing.assert_array_equal(a, b)
    for l in range(2):
        assert rel_err(b[l], sc.oracle_step(q, kd, vd, l)) <= BF16_REL


def test_operand_q_long_history_bench_launch():
    """The 18-layer long-history shape in the benchmark's launch configuration."""
    L = lib()
    s = configs.LONG_18L
    _banner("operand-order q, long history 18 layers")
    sc = Scenario(s)
    for f in range(9):
        sc.push(f)
    q, kd, vd = synth.suffix_qkv(s, 8, 5)
    a = sc.run_step(q, kd, vd, out_dtype=L.PA_BF16)
    b = sc.run_step(q, kd, vd, out_dtype=L.PA_BF16, q_layout=L.PA_Q_OPERAND)
    np.testing.assert_array_equal(a, b)
    for l in (0, 17):
        assert rel_err(b[l], sc.oracle_step(q, kd, vd, l)) <= BF16_REL
