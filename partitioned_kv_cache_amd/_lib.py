"""ctypes binding of libpattn.so: the C ABI of include/pattn.h, same names.

Argument marshalling only: tensors become device pointers, the stream is
torch's current stream unless one is given, and a non-OK status raises
``PattnError`` with the library's message. Every computation runs in the
HIP library. If the library is missing this module raises at import time;
there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os

# torch first: its HIP runtime is then the one this library binds to, so
# torch's streams, events and allocations are valid handles here.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m partitioned_kv_cache_amd.build` "
                      "(or __graft_entry__.build()); there is no CPU fallback")

_lib = C.CDLL(LIB_PATH)

PA_OK, PA_EINVAL, PA_ESHAPE, PA_ESTATE, PA_EDEVICE, PA_ERANGE = range(6)
PA_F32, PA_BF16 = 0, 1
PA_Q_TOKEN_MAJOR, PA_Q_OPERAND = 0, 1
STATUS_NAMES = {0: "PA_OK", 1: "PA_EINVAL", 2: "PA_ESHAPE", 3: "PA_ESTATE", 4: "PA_EDEVICE", 5: "PA_ERANGE"}

# every symbol the header declares
EXPORTS = (
    "pa_last_error", "rb_create", "rb_destroy", "rb_pin_prefix", "rb_push_frame", "rb_get_state",
    "pattn_workspace_bytes", "pattn_step", "pattn_append_private", "pattn_decode_workspace_bytes",
    "pattn_decode", "ada_gamma_workspace_bytes", "ada_gamma", "ada_rmsnorm_workspace_bytes", "ada_rmsnorm",
    "ada_rmsnorm_qkv_workspace_bytes", "ada_rmsnorm_qkv", "oproj_residual", "pattn_step_timed",
    "pa_denoise_step_workspace_bytes", "pa_denoise_step", "rb_capsule_bytes", "rb_snapshot", "rb_restore",
    "rb_stage_frame", "rb_commit_frame", "ffn_swiglu_workspace_bytes", "ffn_swiglu", "pattn_fused_workspace_bytes",
    "pattn_fused_step", "pa_pack_weight", "pattn_operand_q_bytes", "pattn_pack_q", "rb_bind_state_word",
    "pattn_noalloc_scratch_bytes", "pattn_step_noalloc",
)


class PattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.pa_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


class RbConfig(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("pin_capacity", C.c_int32), ("num_slots", C.c_int32), ("tokens_per_frame", C.c_int32),
                ("dtype", C.c_int32), ("spare_slots", C.c_int32)]


class RbState(C.Structure):
    _fields_ = [("head", C.c_int32), ("count", C.c_int32), ("pinned", C.c_int32), ("reserved", C.c_int32),
                ("frames_pushed", C.c_int64)]


class PattnArgs(C.Structure):
    _fields_ = [("layer_begin", C.c_int32), ("num_layers", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_dyn", C.c_int32), ("scale", C.c_float), ("out_dtype", C.c_int32), ("num_splits", C.c_int32),
                ("q_layout", C.c_int32), ("partials_f32", C.c_int32)]


class PattnDecodeArgs(C.Structure):
    _fields_ = [("layer_begin", C.c_int32), ("num_layers", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_streams", C.c_int32), ("tail_capacity", C.c_int32), ("scale", C.c_float),
                ("out_dtype", C.c_int32), ("num_splits", C.c_int32), ("retire_full", C.c_int32)]


class AdaMlp(C.Structure):
    _fields_ = [("w1", C.c_void_p), ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p),
                ("num_layers", C.c_int32), ("cond_emb", C.c_int32), ("state_dim", C.c_int32),
                ("hidden_dim", C.c_int32), ("model_dim", C.c_int32)]


class PaStack(C.Structure):
    _fields_ = [("num_layers", C.c_int32), ("rows", C.c_int32), ("model_dim", C.c_int32), ("n_q_heads", C.c_int32),
                ("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("eps", C.c_float), ("scale", C.c_float),
                ("dt", C.c_float), ("num_splits", C.c_int32), ("ffn_dim", C.c_int32), ("w_gate", C.c_void_p),
                ("w_up", C.c_void_p), ("w_down", C.c_void_p), ("packed", C.c_int32)]


_vp, _i32, _f32, _sz = C.c_void_p, C.c_int32, C.c_float, C.c_size_t


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype, f.argtypes = res, list(args)
    return f


_sig("pa_last_error", C.c_char_p)
_sig("rb_create", _i32, C.POINTER(RbConfig), _vp, _vp, C.POINTER(_vp))
_sig("rb_destroy", _i32, _vp)
_sig("rb_pin_prefix", _i32, _vp, _vp, _vp, _i32, _vp)
_sig("rb_push_frame", _i32, _vp, _vp, _vp, _vp, C.POINTER(C.c_int64))
_sig("rb_get_state", _i32, _vp, C.POINTER(RbState))
_sig("rb_stage_frame", _i32, _vp, _vp, _vp, _vp)
_sig("rb_commit_frame", _i32, _vp, _vp, C.POINTER(C.c_int64))
_sig("rb_bind_state_word", _i32, _vp, _vp, _vp)
_sig("rb_capsule_bytes", _sz, _vp)
_sig("rb_snapshot", _i32, _vp, _vp, _sz, C.POINTER(RbState), _vp)
_sig("rb_restore", _i32, _vp, _vp, _sz, C.POINTER(RbState), _vp)
_sig("pattn_workspace_bytes", _sz, _vp, C.POINTER(PattnArgs))
_sig("pattn_step", _i32, _vp, C.POINTER(PattnArgs), _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("pattn_noalloc_scratch_bytes", _sz)
_sig("pattn_step_noalloc", _i32, _vp, C.POINTER(PattnArgs), _vp, _vp, _vp, _vp, _vp)
_sig("pattn_step_timed", _i32, _vp, C.POINTER(PattnArgs), _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp, _vp)
_sig("pa_denoise_step_workspace_bytes", _sz, _vp, C.POINTER(PaStack))
_sig("pa_denoise_step", _i32, _vp, C.POINTER(PaStack), _vp, _vp, _vp, C.c_int64, _vp, _vp, _sz, _vp)
_sig("ffn_swiglu_workspace_bytes", _sz, _i32, _i32, _i32)
_sig("ffn_swiglu", _i32, _vp, _i32, _i32, _i32, _vp, _f32, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _sz, _vp)
_sig("pa_pack_weight", _i32, _vp, _i32, _i32, _vp, _vp)
_sig("pattn_operand_q_bytes", _sz, _vp, C.POINTER(PattnArgs))
_sig("pattn_pack_q", _i32, _vp, C.POINTER(PattnArgs), _vp, _vp, _vp)
_sig("pattn_append_private", _i32, _vp, C.POINTER(PattnDecodeArgs), _vp, _vp, _vp, _vp, _vp, _vp, _vp)
_sig("pattn_decode_workspace_bytes", _sz, _vp, C.POINTER(PattnDecodeArgs))
_sig("pattn_decode", _i32, _vp, C.POINTER(PattnDecodeArgs), _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("pattn_fused_workspace_bytes", _sz, _vp, C.POINTER(PattnArgs), C.POINTER(PattnDecodeArgs))
_sig("pattn_fused_step", _i32, _vp, C.POINTER(PattnArgs), _vp, _vp, _vp, _vp, C.POINTER(PattnDecodeArgs), _vp, _vp, _vp,
     _vp, _vp, _vp, _sz, _vp)
_sig("ada_gamma_workspace_bytes", _sz, C.POINTER(AdaMlp), _i32)
_sig("ada_gamma", _i32, C.POINTER(AdaMlp), C.POINTER(C.c_float), _i32, _vp, _vp, _vp, _sz, _vp)
_sig("ada_rmsnorm_workspace_bytes", _sz, C.POINTER(AdaMlp))
_sig("ada_rmsnorm", _i32, _vp, _i32, C.POINTER(AdaMlp), _i32, _f32, _vp, _f32, _vp, _i32, _vp, _vp, _sz, _vp)
_sig("ada_rmsnorm_qkv_workspace_bytes", _sz, _i32, _i32)
_sig("ada_rmsnorm_qkv", _i32, _vp, _i32, _i32, _vp, _f32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp)
_sig("oproj_residual", _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _f32, _vp, _vp)


def _check(st: int, where: str):
    if st != PA_OK:
        raise PattnError(st, where)


def ptr(t) -> int | None:
    """Device pointer of a tensor (or an int / None passed through)."""
    if t is None or isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------- ring ------

class Ring:
    """Handle over caller-owned K/V buffers [L][P + W*F][Hkv][D] (rb_*)."""

    def __init__(self, cfg: RbConfig, k_buf, v_buf):
        self.cfg = cfg
        self.k_buf, self.v_buf = k_buf, v_buf        # keep the tensors alive
        h = _vp()
        _check(_lib.rb_create(C.byref(cfg), ptr(k_buf), ptr(v_buf), C.byref(h)), "rb_create")
        self.handle = h.value

    def close(self):
        if self.handle:
            _lib.rb_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pin_prefix(self, k, v, n_tokens: int, stream=None):
        _check(_lib.rb_pin_prefix(self.handle, ptr(k), ptr(v), n_tokens, _stream(stream)), "rb_pin_prefix")

    def push_frame(self, k, v, stream=None) -> int:
        ev = C.c_int64(0)
        _check(_lib.rb_push_frame(self.handle, ptr(k), ptr(v), _stream(stream), C.byref(ev)), "rb_push_frame")
        return ev.value

    def stage_frame(self, k, v, stream=None):
        """Copy the next frame into the spare slot on the producer's stream (rb_stage_frame)."""
        _check(_lib.rb_stage_frame(self.handle, ptr(k), ptr(v), _stream(stream)), "rb_stage_frame")

    def commit_frame(self, stream=None) -> int:
        """Make the staged frame the newest of the window for work enqueued on `stream` (rb_commit_frame)."""
        ev = C.c_int64(0)
        _check(_lib.rb_commit_frame(self.handle, _stream(stream), C.byref(ev)), "rb_commit_frame")
        return ev.value

    def bind_state_word(self, word, stream=None):
        """Keep {head, count, pinned, 0} in a device int32[4] the kernels read (rb_bind_state_word)."""
        self.state_word = word                     # keep the tensor alive
        _check(_lib.rb_bind_state_word(self.handle, ptr(word), _stream(stream)), "rb_bind_state_word")

    def state(self) -> dict:
        s = RbState()
        _check(_lib.rb_get_state(self.handle, C.byref(s)), "rb_get_state")
        return {"head": s.head, "count": s.count, "pinned": s.pinned, "frames_pushed": s.frames_pushed}

    # capsules: the valid K/V region plus the metadata (rb_snapshot / rb_restore)
    def capsule_bytes(self) -> int:
        return _lib.rb_capsule_bytes(self.handle)

    def snapshot(self, capsule, capsule_bytes: int | None = None, stream=None) -> dict:
        s = RbState()
        nb = capsule.numel() * capsule.element_size() if capsule_bytes is None else capsule_bytes
        _check(_lib.rb_snapshot(self.handle, ptr(capsule), nb, C.byref(s), _stream(stream)), "rb_snapshot")
        return {"head": s.head, "count": s.count, "pinned": s.pinned, "frames_pushed": s.frames_pushed}

    def restore(self, capsule, state: dict, capsule_bytes: int | None = None, stream=None):
        s = RbState(state["head"], state["count"], state["pinned"], 0, state["frames_pushed"])
        nb = capsule.numel() * capsule.element_size() if capsule_bytes is None else capsule_bytes
        _check(_lib.rb_restore(self.handle, ptr(capsule), nb, C.byref(s), _stream(stream)), "rb_restore")


def rb_config(num_layers, num_kv_heads, head_dim, pin_capacity, num_slots, tokens_per_frame, dtype,
              spare_slots=0) -> RbConfig:
    return RbConfig(num_layers, num_kv_heads, head_dim, pin_capacity, num_slots, tokens_per_frame, dtype, spare_slots)


# ------------------------------------------------------------ attention ------

def pattn_args(layer_begin, num_layers, n_q_heads, n_dyn, scale, out_dtype=PA_F32, num_splits=0,
               q_layout=0, partials_f32=0) -> PattnArgs:
    return PattnArgs(layer_begin, num_layers, n_q_heads, n_dyn, scale, out_dtype, num_splits, q_layout, partials_f32)


def pattn_operand_q_bytes(ring: Ring, args: PattnArgs) -> int:
    return _lib.pattn_operand_q_bytes(ring.handle, C.byref(args))


def pattn_pack_q(ring: Ring, args: PattnArgs, q, q_operand, stream=None):
    """Token-major q -> the PA_Q_OPERAND order pattn_step reads with q_layout = PA_Q_OPERAND."""
    _check(_lib.pattn_pack_q(ring.handle, C.byref(args), ptr(q), ptr(q_operand), _stream(stream)), "pattn_pack_q")


def pattn_workspace_bytes(ring: Ring, args: PattnArgs) -> int:
    return _lib.pattn_workspace_bytes(ring.handle, C.byref(args))


def pattn_step(ring: Ring, args: PattnArgs, q, k_dyn, v_dyn, out, workspace, ws_bytes: int, stream=None):
    _check(_lib.pattn_step(ring.handle, C.byref(args), ptr(q), ptr(k_dyn), ptr(v_dyn), ptr(out), ptr(workspace),
                           ws_bytes, _stream(stream)), "pattn_step")


def pattn_noalloc_scratch_bytes() -> int:
    return _lib.pattn_noalloc_scratch_bytes()


def pattn_step_noalloc(ring: Ring, args: PattnArgs, q, k_dyn, v_dyn, out, stream=None):
    """pattn_step with the partials in the library's fixed device scratch (no workspace, no allocation)."""
    _check(_lib.pattn_step_noalloc(ring.handle, C.byref(args), ptr(q), ptr(k_dyn), ptr(v_dyn), ptr(out),
                                   _stream(stream)), "pattn_step_noalloc")


def pattn_step_timed(ring: Ring, args: PattnArgs, q, k_dyn, v_dyn, out, workspace, ws_bytes: int, stream=None,
                     ev_begin=None, ev_end=None):
    """pattn_step plus HIP events recorded around its split-KV partial kernel (raw hipEvent_t ints)."""
    _check(_lib.pattn_step_timed(ring.handle, C.byref(args), ptr(q), ptr(k_dyn), ptr(v_dyn), ptr(out),
                                 ptr(workspace), ws_bytes, _stream(stream), ev_begin, ev_end), "pattn_step_timed")


def decode_args(layer_begin, num_layers, n_q_heads, n_streams, tail_capacity, scale, out_dtype=PA_F32,
                num_splits=0, retire_full=0) -> PattnDecodeArgs:
    return PattnDecodeArgs(layer_begin, num_layers, n_q_heads, n_streams, tail_capacity, scale, out_dtype, num_splits,
                           retire_full)


def pattn_append_private(ring: Ring, args: PattnDecodeArgs, tail_k, tail_v, tail_len, k_new, v_new,
                         overflow=None, stream=None):
    _check(_lib.pattn_append_private(ring.handle, C.byref(args), ptr(tail_k), ptr(tail_v), ptr(tail_len),
                                     ptr(k_new), ptr(v_new), ptr(overflow), _stream(stream)), "pattn_append_private")


def pattn_decode_workspace_bytes(ring: Ring, args: PattnDecodeArgs) -> int:
    return _lib.pattn_decode_workspace_bytes(ring.handle, C.byref(args))


def pattn_decode(ring: Ring, args: PattnDecodeArgs, q, tail_k, tail_v, tail_len, out, workspace, ws_bytes: int,
                 stream=None):
    _check(_lib.pattn_decode(ring.handle, C.byref(args), ptr(q), ptr(tail_k), ptr(tail_v), ptr(tail_len), ptr(out),
                             ptr(workspace), ws_bytes, _stream(stream)), "pattn_decode")


# ------------------------------------------------------------- adanorm -------

def ada_mlp(w1, b1, w2, b2, num_layers, cond_emb, state_dim, hidden_dim, model_dim) -> AdaMlp:
    m = AdaMlp(ptr(w1), ptr(b1), ptr(w2), ptr(b2), num_layers, cond_emb, state_dim, hidden_dim, model_dim)
    m._keep = (w1, b1, w2, b2)
    return m


def ada_gamma_workspace_bytes(mlp: AdaMlp, n_t: int) -> int:
    return _lib.ada_gamma_workspace_bytes(C.byref(mlp), n_t)


def ada_gamma(mlp: AdaMlp, t: list[float], state, gamma, workspace, ws_bytes: int, stream=None):
    arr = (C.c_float * len(t))(*t)
    _check(_lib.ada_gamma(C.byref(mlp), arr, len(t), ptr(state), ptr(gamma), ptr(workspace), ws_bytes,
                          _stream(stream)), "ada_gamma")


def ada_rmsnorm_workspace_bytes(mlp: AdaMlp) -> int:
    return _lib.ada_rmsnorm_workspace_bytes(C.byref(mlp))


def ada_rmsnorm(x, rows: int, mlp: AdaMlp, layer: int, t: float, state, eps: float, y, y_dtype: int,
                nonfinite, workspace, ws_bytes: int, stream=None):
    _check(_lib.ada_rmsnorm(ptr(x), rows, C.byref(mlp), layer, t, ptr(state), eps, ptr(y), y_dtype,
                            ptr(nonfinite), ptr(workspace), ws_bytes, _stream(stream)), "ada_rmsnorm")


def ada_rmsnorm_qkv_workspace_bytes(rows: int, model_dim: int) -> int:
    return _lib.ada_rmsnorm_qkv_workspace_bytes(rows, model_dim)


def ada_rmsnorm_qkv(x, rows, model_dim, gamma, eps, w_qkv, n_q_heads, n_kv_heads, head_dim, q, k_dyn, v_dyn,
                    nonfinite, workspace, ws_bytes, stream=None):
    _check(_lib.ada_rmsnorm_qkv(ptr(x), rows, model_dim, ptr(gamma), eps, ptr(w_qkv), n_q_heads, n_kv_heads,
                                head_dim, ptr(q), ptr(k_dyn), ptr(v_dyn), ptr(nonfinite), ptr(workspace), ws_bytes,
                                _stream(stream)), "ada_rmsnorm_qkv")


def oproj_residual(o, w_o, h, rows, in_dim, model_dim, x=None, dt=0.1, nonfinite=None, stream=None):
    _check(_lib.oproj_residual(ptr(o), ptr(w_o), ptr(h), rows, in_dim, model_dim, ptr(x), dt, ptr(nonfinite),
                               _stream(stream)), "oproj_residual")


# ----------------------------------------------------------- denoise step ----

def pa_stack(num_layers, rows, model_dim, n_q_heads, w_qkv, w_o, eps, scale, dt, num_splits=0, ffn_dim=0,
             w_gate=None, w_up=None, w_down=None, packed=0) -> PaStack:
    st = PaStack(num_layers, rows, model_dim, n_q_heads, ptr(w_qkv), ptr(w_o), eps, scale, dt, num_splits, ffn_dim,
                 ptr(w_gate), ptr(w_up), ptr(w_down), int(packed))
    st._keep = (w_qkv, w_o, w_gate, w_up, w_down)
    return st


def pa_denoise_step_workspace_bytes(ring: Ring, st: PaStack) -> int:
    return _lib.pa_denoise_step_workspace_bytes(ring.handle, C.byref(st))


def pa_denoise_step(ring: Ring, st: PaStack, x, gamma, gamma_layer_stride: int, nonfinite, workspace, ws_bytes: int,
                    stream=None, gamma_ffn=None):
    _check(_lib.pa_denoise_step(ring.handle, C.byref(st), ptr(x), ptr(gamma), ptr(gamma_ffn), gamma_layer_stride,
                                ptr(nonfinite), ptr(workspace), ws_bytes, _stream(stream)), "pa_denoise_step")


def pa_pack_weight(w, n: int, k: int, w_packed, stream=None):
    """Rewrite an nn.Linear weight bf16 [n][k] into the fragment-packed order (pa_pack_weight)."""
    _check(_lib.pa_pack_weight(ptr(w), n, k, ptr(w_packed), _stream(stream)), "pa_pack_weight")


def ffn_swiglu_workspace_bytes(rows: int, model_dim: int, ffn_dim: int) -> int:
    return _lib.ffn_swiglu_workspace_bytes(rows, model_dim, ffn_dim)


def ffn_swiglu(h, rows: int, model_dim: int, ffn_dim: int, gamma, eps: float, w_gate, w_up, w_down, x=None,
               dt: float = 0.0, nonfinite=None, workspace=None, ws_bytes: int = 0, stream=None):
    """h <- bf16(h + SwiGLU-FFN(AdaRMSNorm(h, gamma))); x <- bf16(x - dt h) when x is given."""
    _check(_lib.ffn_swiglu(ptr(h), rows, model_dim, ffn_dim, ptr(gamma), eps, ptr(w_gate), ptr(w_up), ptr(w_down),
                           ptr(x), dt, ptr(nonfinite), ptr(workspace), ws_bytes, _stream(stream)), "ffn_swiglu")


def raw():
    """The ctypes CDLL itself (for the symbol-export test)."""
    return _lib


def pattn_fused_workspace_bytes(ring: Ring, args: PattnArgs, dec: PattnDecodeArgs) -> int:
    return _lib.pattn_fused_workspace_bytes(ring.handle, C.byref(args), C.byref(dec))


def pattn_fused_step(ring: Ring, args: PattnArgs, q, k_dyn, v_dyn, out, dec: PattnDecodeArgs, q_dec, tail_k, tail_v,
                     tail_len, out_dec, workspace, ws_bytes: int, stream=None):
    """The action suffix and the decode streams in one pass over the shared cache (pattn_fused_step)."""
    _check(_lib.pattn_fused_step(ring.handle, C.byref(args), ptr(q), ptr(k_dyn), ptr(v_dyn), ptr(out), C.byref(dec),
                                 ptr(q_dec), ptr(tail_k), ptr(tail_v), ptr(tail_len), ptr(out_dec), ptr(workspace),
                                 ws_bytes, _stream(stream)), "pattn_fused_step")

