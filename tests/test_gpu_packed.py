"""GPU tests of the fragment-packed weight path of the denoising stack.

pa_pack_weight is integer work (a permutation of bf16 words), so it is
checked bit for bit against the layout written out here with numpy reshapes.
The packed stack (pa_stack.packed = 1) computes the same products in the same
order as the unpacked one, so its x must equal the unpacked step's bit for
bit; against the oracle chain it meets the stack's bar, max|gpu - ref| /
max|ref| <= 2e-2 (bf16 storage, FP32 accumulation).
"""

import numpy as np
import pytest
import torch

from oracle import stack
from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, host, lib, rel_err  # noqa: E402

BAR = 2e-2


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


def _pack_numpy(w: np.ndarray) -> np.ndarray:
    """[n][k] -> [n/32][k/16][2 (k/8 mod 2)][32 (n mod 32)][8 (k mod 8)], flattened."""
    n, k = w.shape
    return np.ascontiguousarray(w.reshape(n // 32, 32, k // 16, 2, 8).transpose(0, 2, 3, 1, 4)).reshape(-1)


def _pack_dev(w_d: torch.Tensor, n: int, k: int) -> torch.Tensor:
    out = torch.empty_like(w_d)
    lib().pa_pack_weight(w_d, n, k, out)
    return out


@pytest.mark.parametrize("n,k", [(32, 16), (64, 48), (2560, 1024), (1024, 2048), (96, 4096)])
def test_pack_weight_matches_layout(n, k):
    _banner(f"pa_pack_weight {n} x {k}")
    w = synth._rng(901, n, k).integers(0, 1 << 16, size=(n, k), dtype=np.uint16)
    got = host(_pack_dev(dev(w), n, k)).reshape(-1)
    np.testing.assert_array_equal(got, _pack_numpy(w))


def test_pack_weight_of_a_layer_stack_packs_each_layer():
    L_, n, k = 3, 96, 64
    w = synth._rng(902).integers(0, 1 << 16, size=(L_, n, k), dtype=np.uint16)
    got = host(_pack_dev(dev(w), L_ * n, k)).reshape(L_, -1)
    for l in range(L_):
        np.testing.assert_array_equal(got[l], _pack_numpy(w[l]))


def test_pack_weight_rejects_bad_arguments():
    L = lib()
    w = torch.zeros(64 * 64, dtype=torch.int16, device="cuda")
    out = torch.empty_like(w)
    for n, k in [(48, 64), (64, 24), (0, 64)]:
        with pytest.raises(L.PattnError):
            L.pa_pack_weight(w, n, k, out)
    with pytest.raises(L.PattnError):
        L.pa_pack_weight(w, 64, 64, w)                  # in place
    with pytest.raises(L.PattnError):
        L.pa_pack_weight(w[1:], 32, 64, out)            # 2-byte aligned


class PackedRig:
    """One ring, the stack's weights in both layouts, and the two pa_stack views."""

    def __init__(self, s, frames, ffn=False):
        L = lib()
        self.s = s
        self.sc = Scenario(s)
        for f in range(frames):
            self.sc.push(f)
        self.wq = [synth.proj_weights(s, l) for l in range(s.num_layers)]
        self.wf = [synth.ffn_weights(s, l) for l in range(s.num_layers)] if ffn else None
        wqkv, wo = dev(np.stack([w[0] for w in self.wq])), dev(np.stack([w[1] for w in self.wq]))
        hd = s.n_q_heads * s.head_dim
        self.plain = [wqkv, wo]
        self.packed = [_pack_dev(wqkv, s.num_layers * s.qkv_out, s.model_dim),
                       _pack_dev(wo, s.num_layers * s.model_dim, hd)]
        fd = 0
        if ffn:
            fd = s.ffn_dim
            g, u, d = (dev(np.stack([w[i] for w in self.wf])) for i in range(3))
            self.plain += [g, u, d]
            self.packed += [_pack_dev(g, s.num_layers * fd, s.model_dim), _pack_dev(u, s.num_layers * fd, s.model_dim),
                            _pack_dev(d, s.num_layers * s.model_dim, fd)]
        args = (s.num_layers, s.n_dyn, s.model_dim, s.n_q_heads)
        tail = (s.eps, s.scale, 0.1, 0, fd)
        ws = self.plain
        self.st_plain = L.pa_stack(*args, ws[0], ws[1], *tail, *(ws[2:] if ffn else (None, None, None)))
        ws = self.packed
        self.st_packed = L.pa_stack(*args, ws[0], ws[1], *tail, *(ws[2:] if ffn else (None, None, None)), packed=1)
        self.ws_plain = L.pa_denoise_step_workspace_bytes(self.sc.ring, self.st_plain)
        self.ws_packed = L.pa_denoise_step_workspace_bytes(self.sc.ring, self.st_packed)
        assert self.ws_plain > 0 and self.ws_packed > 0
        self.ws = torch.empty(max(self.ws_plain, self.ws_packed), dtype=torch.uint8, device="cuda")
        rng = synth._rng(s.cfg_id, 905)
        self.gamma = (1.0 + 0.2 * rng.standard_normal((s.num_layers, s.model_dim))).astype(np.float32)
        self.gamma_ffn = (1.0 + 0.2 * rng.standard_normal((s.num_layers, s.model_dim))).astype(np.float32)
        self.g_d, self.gf_d = dev(self.gamma), dev(self.gamma_ffn)

    def run(self, x: np.ndarray, packed: bool):
        L = lib()
        x_d = dev(x)
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        st, wsb = (self.st_packed, self.ws_packed) if packed else (self.st_plain, self.ws_plain)
        L.pa_denoise_step(self.sc.ring, st, x_d, self.g_d, self.s.model_dim, flag, self.ws, wsb,
                          gamma_ffn=self.gf_d if self.wf else None)
        torch.cuda.synchronize()
        rows, model = self.s.n_dyn, self.s.model_dim
        self.last_h = host(self.ws[: rows * model * 2].view(torch.int16).reshape(rows, model)).copy()
        return host(x_d), int(host(flag)[0])

    def oracle(self, x: np.ndarray):
        s = self.s
        caches = [self.sc.cached_context(l) for l in range(s.num_layers)]
        ffns = None
        if self.wf:
            ffns = [(self.gamma_ffn[l].astype(np.float64), *(synth.widen(w) for w in self.wf[l]))
                    for l in range(s.num_layers)]
        x1, trace = stack.denoise_step(synth.widen(x), [g.astype(np.float64) for g in self.gamma], s.eps,
                                       [synth.widen(w[0]) for w in self.wq], [synth.widen(w[1]) for w in self.wq],
                                       [c[0] for c in caches], [c[1] for c in caches], s.scale, s.n_q_heads,
                                       s.n_kv_heads, s.head_dim, ffns=ffns)
        return x1, trace[-1]["h"]


CASES = {
    # name: (shape, frames, ffn, check against the oracle)
    "stack_51x1024": (configs.PI05_18L.with_(name="pk_a", cfg_id=910, num_layers=3), 3, False, True),
    "stack_7x512": (configs.PI05_18L.with_(name="pk_b", cfg_id=911, num_layers=2, n_dyn=7, model_dim=512), 2,
                    False, True),
    "stack_64x1024_hq4": (configs.PI05_18L.with_(name="pk_c", cfg_id=912, num_layers=2, n_dyn=64, n_q_heads=4), 1,
                          False, False),
    "full_51x1024_ffn4096": (configs.PI05_18L_FFN.with_(name="pk_d", cfg_id=913, num_layers=3), 3, True, True),
    "full_33x512_ffn3072": (configs.PI05_18L_FFN.with_(name="pk_e", cfg_id=914, num_layers=2, n_dyn=33,
                                                       model_dim=512, ffn_dim=3072), 2, True, False),
    # the long-history cache (6,400 cached keys per layer, wrapped once): each
    # layer's attention runs the key-halves launch, with Q in operand order
    # (packed) and token-major (unpacked)
    "long_51x1024": (configs.LONG_18L_FULL.with_(name="pk_f", cfg_id=915, num_layers=2), 9, False, True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_packed_stack_is_bit_identical_to_unpacked(case):
    s, frames, ffn, check_oracle = CASES[case]
    _banner(f"packed stack {case}: rows={s.n_dyn} model={s.model_dim} Hq={s.n_q_heads} L={s.num_layers} ffn={ffn}")
    rig = PackedRig(s, frames, ffn)
    x = synth.flow_x(s, 1)
    x_plain, f_plain = rig.run(x, packed=False)
    h_plain = rig.last_h
    x_packed, f_packed = rig.run(x, packed=True)
    np.testing.assert_array_equal(x_packed, x_plain)
    np.testing.assert_array_equal(rig.last_h, h_plain)        # the velocity h_L, bit for bit
    assert f_plain == 0 and f_packed == 0
    if check_oracle:
        x1, h_last = rig.oracle(x)
        err = rel_err(synth.widen(x_packed), x1)
        err_h = rel_err(synth.widen(rig.last_h), h_last)
        _banner(f"  packed x rel {err:.3e}, h_L rel {err_h:.3e}")
        assert err <= BAR and err_h <= BAR


def test_packed_stack_flags_nonfinite_input():
    s, frames, ffn, _ = CASES["full_51x1024_ffn4096"]
    rig = PackedRig(s.with_(num_layers=1), 1, ffn)
    x = synth.flow_x(rig.s, 0)
    x[5, 100] = 0x7F80                                  # +Inf in bf16
    _, flag = rig.run(x, packed=True)
    assert flag == 1


def test_packed_stack_rejects_unsupported_shapes():
    L = lib()
    s = configs.PI05_18L.with_(name="pk_bad", cfg_id=915, num_layers=1, model_dim=768)
    sc = Scenario(s)
    w = torch.zeros(s.qkv_out * s.model_dim + s.model_dim * s.n_q_heads * s.head_dim, dtype=torch.int16,
                    device="cuda")
    st = L.pa_stack(1, s.n_dyn, s.model_dim, s.n_q_heads, w, w, s.eps, s.scale, 0.1, packed=1)
    assert L.pa_denoise_step_workspace_bytes(sc.ring, st) == 0       # model_dim 768 has no packed kernels
    st = L.pa_stack(1, s.n_dyn, s.model_dim, s.n_q_heads, w, w, s.eps, s.scale, 0.1, packed=2)
    assert L.pa_denoise_step_workspace_bytes(sc.ring, st) == 0


def test_packed_stack_graph_replays_match_eager():
    """Two packed steps captured in a graph; frames pushed eagerly between
    replays; every replay equals the eager run bit for bit."""
    L = lib()
    s, _, ffn, _ = CASES["full_51x1024_ffn4096"]
    s = s.with_(name="pk_graph", cfg_id=916, num_layers=2)
    rig = PackedRig(s, s.num_slots, ffn)
    x0 = dev(synth.flow_x(s, 0))
    x = x0.clone()
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")

    def two_steps():
        for _ in range(2):
            L.pa_denoise_step(rig.sc.ring, rig.st_packed, x, rig.g_d, s.model_dim, flag, rig.ws, rig.ws_packed,
                              gamma_ffn=rig.gf_d)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        two_steps()
    for rep in range(3):
        rig.sc.push(s.num_slots + rep)
        torch.cuda.synchronize()
        x.copy_(x0)
        two_steps()
        torch.cuda.synchronize()
        eager = host(x).copy()
        x.copy_(x0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(x), eager)
