"""Helpers for the GPU tests: device buffers from seeded host arrays, a ring
scenario that keeps the library's ring and the oracle's model in step, and
the parity measures. Imported by ``test_gpu_*.py`` only."""

from __future__ import annotations

import numpy as np
import torch

from oracle.attention import full_attention
from oracle.ring import RingModel
from partitioned_kv_cache_amd import synth
from partitioned_kv_cache_amd.configs import Shape


def lib():
    from partitioned_kv_cache_amd import _lib
    return _lib


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array in storage dtype (uint16 bf16 bits / float32 / int32) -> device tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def tdtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.int16


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| over one output tensor."""
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def max_abs(gpu: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)))


class Scenario:
    """A ring on the GPU plus the oracle's model of it, fed the same frames."""

    def __init__(self, s: Shape, pin_tokens: int | None = None, frame_fn=None, spare_slots: int = 0):
        L = lib()
        self.s = s
        self.dt = L.PA_F32 if s.dtype == "f32" else L.PA_BF16
        seq = s.pin_tokens + (s.num_slots + spare_slots) * s.tokens_per_frame
        shp = (s.num_layers, seq, s.n_kv_heads, s.head_dim)
        self.k_buf = torch.zeros(shp, dtype=tdtype(s.dtype), device="cuda")
        self.v_buf = torch.zeros(shp, dtype=tdtype(s.dtype), device="cuda")
        self.ring = L.Ring(L.rb_config(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                                       s.tokens_per_frame, self.dt, spare_slots), self.k_buf, self.v_buf)
        word = np.uint32 if s.dtype == "f32" else np.uint16
        self.model = RingModel(s.num_layers, s.n_kv_heads, s.head_dim, s.pin_tokens, s.num_slots,
                               s.tokens_per_frame, word, spare_slots=spare_slots)
        self.frame_fn = frame_fn or (lambda f: synth.frame_kv(s, f))
        self.pin_k = self.pin_v = None
        n_pin = s.pin_tokens if pin_tokens is None else pin_tokens
        if n_pin > 0:
            self.pin_k, self.pin_v = synth.pin_kv(s, n_pin)
            self.ring.pin_prefix(dev(self.pin_k), dev(self.pin_v), n_pin)
            self.model.pin(self._words(self.pin_k), self._words(self.pin_v))
        self.window: list[tuple[int, np.ndarray, np.ndarray]] = []   # (frame, k, v), oldest first

    def _words(self, a):
        return a.view(np.uint32) if a.dtype == np.float32 else a

    def push(self, f: int) -> int:
        k, v = self.frame_fn(f)
        ev = self.ring.push_frame(dev(k), dev(v))
        ev_model = self.model.push(self._words(k), self._words(v))
        assert ev == ev_model
        self._enter(f, k, v)
        return ev

    def _enter(self, f, k, v):
        self.window.append((f, k, v))
        if len(self.window) > self.s.num_slots:
            self.window.pop(0)

    def stage(self, f: int, stream):
        """Stage frame f on `stream` (device tensors kept alive until the commit)."""
        k, v = self.frame_fn(f)
        self._staged = (f, k, v, dev(k), dev(v))
        self.ring.stage_frame(self._staged[3], self._staged[4], stream)
        self.model.stage(self._words(k), self._words(v))

    def commit(self, stream) -> int:
        f, k, v, _, _ = self._staged
        ev = self.ring.commit_frame(stream)
        assert ev == self.model.commit()
        self._enter(f, k, v)
        self._staged = None
        return ev

    def check_bytes(self):
        torch.cuda.synchronize()
        gk, gv = host(self.k_buf), host(self.v_buf)
        if gk.dtype == np.float32:
            gk, gv = gk.view(np.uint32), gv.view(np.uint32)
        assert np.array_equal(gk, self.model.k), "K ring bytes differ from the ring model"
        assert np.array_equal(gv, self.model.v), "V ring bytes differ from the ring model"
        st = self.ring.state()
        m = self.model.state()
        assert st == m, (st, m)

    def cached_context(self, layer: int):
        """Chronological [pin; window frames] of one layer, float64."""
        parts_k, parts_v = [], []
        if self.pin_k is not None:
            parts_k.append(synth.widen(self.pin_k[layer]))
            parts_v.append(synth.widen(self.pin_v[layer]))
        for _, k, v in self.window:
            parts_k.append(synth.widen(k[layer]))
            parts_v.append(synth.widen(v[layer]))
        d, h = self.s.head_dim, self.s.n_kv_heads
        if not parts_k:
            return np.zeros((0, h, d)), np.zeros((0, h, d))
        return np.concatenate(parts_k), np.concatenate(parts_v)

    def run_step(self, q, k_dyn, v_dyn, out_dtype=None, num_splits=0, layer_begin=0, num_layers=None, q_layout=0,
                 partials_f32=0):
        """pattn_step on host arrays; returns the output as float64 [Lb][N][Hq][D].
        With q_layout = PA_Q_OPERAND the token-major q is converted by pattn_pack_q first."""
        L = lib()
        s = self.s
        nl = s.num_layers if num_layers is None else num_layers
        od = L.PA_F32 if out_dtype is None else out_dtype
        args = L.pattn_args(layer_begin, nl, s.n_q_heads, q.shape[1], s.scale, od, num_splits, q_layout,
                            partials_f32)
        ws_bytes = L.pattn_workspace_bytes(self.ring, args)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        out = torch.empty((nl, q.shape[1], s.n_q_heads, s.head_dim),
                          dtype=torch.float32 if od == L.PA_F32 else torch.int16, device="cuda")
        q_d = dev(q)
        if q_layout == L.PA_Q_OPERAND:
            q_op = torch.empty(L.pattn_operand_q_bytes(self.ring, args) // 2, dtype=torch.int16, device="cuda")
            L.pattn_pack_q(self.ring, args, q_d, q_op)
            q_d = q_op
        L.pattn_step(self.ring, args, q_d, dev(k_dyn), dev(v_dyn), out, ws, ws_bytes)
        torch.cuda.synchronize()
        return synth.widen(host(out))

    def oracle_step(self, q, k_dyn, v_dyn, layer: int):
        ck, cv = self.cached_context(layer)
        ck = np.concatenate([ck, synth.widen(k_dyn[layer])])
        cv = np.concatenate([cv, synth.widen(v_dyn[layer])])
        return full_attention(synth.widen(q[layer]), ck, cv, self.s.scale)
