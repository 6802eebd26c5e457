"""The C-ABI library loads and exports every entry point include/pattn.h
declares; host-side argument validation returns the documented status codes
without touching a device (no compute call runs here)."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pattn.h")
LIB = os.path.join(ROOT, "partitioned_kv_cache_amd", "libpattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libpattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:pa_status|size_t|const char\*|char\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for n in ("rb_create", "rb_pin_prefix", "rb_push_frame", "rb_get_state", "pattn_step", "ada_rmsnorm",
              "ada_gamma", "ada_rmsnorm_qkv", "pattn_decode", "pattn_append_private", "oproj_residual",
              "pa_last_error", "rb_capsule_bytes", "rb_snapshot", "rb_restore"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    from partitioned_kv_cache_amd import _lib
    assert sorted(_lib.EXPORTS) == declared_functions()


def _fake(n):
    return 0x10000 * n      # non-null, never dereferenced on these paths


def test_rb_create_validation_and_state_without_device():
    from partitioned_kv_cache_amd import _lib as L
    bad = L.rb_config(1, 1, 64, 16, 4, 16, 7)
    with pytest.raises(L.PattnError) as e:
        L.Ring(bad, _fake(1), _fake(2))
    assert e.value.status == L.PA_EINVAL and "dtype" in str(e.value)
    with pytest.raises(L.PattnError) as e:
        L.Ring(L.rb_config(1, 1, 60, 16, 4, 16, L.PA_F32), _fake(1), _fake(2))
    assert e.value.status == L.PA_ESHAPE
    with pytest.raises(L.PattnError) as e:
        L.Ring(L.rb_config(0, 1, 64, 16, 4, 16, L.PA_F32), _fake(1), _fake(2))
    assert e.value.status == L.PA_ESHAPE
    r = L.Ring(L.rb_config(1, 1, 64, 16, 4, 16, L.PA_F32), _fake(1), _fake(2))
    assert r.state() == {"head": 0, "count": 0, "pinned": 0, "frames_pushed": 0}
    with pytest.raises(L.PattnError) as e:
        r.pin_prefix(_fake(3), _fake(4), 17, stream=0)       # > P
    assert e.value.status == L.PA_ESHAPE
    with pytest.raises(L.PattnError) as e:
        r.pin_prefix(None, _fake(4), 4, stream=0)
    assert e.value.status == L.PA_EINVAL
    r.close()


def test_pattn_step_validation_without_device():
    from partitioned_kv_cache_amd import _lib as L
    r = L.Ring(L.rb_config(2, 1, 256, 48, 2, 768, L.PA_BF16), _fake(1), _fake(2))
    a = L.pattn_args(0, 2, 8, 51, 1 / 16, L.PA_F32)
    ws = L.pattn_workspace_bytes(r, a)
    assert ws > 0 and ws % 256 == 0
    # not pinned yet, P > 0: state error, raised before any launch
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r, a, _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), ws, stream=0)
    assert e.value.status == L.PA_ESTATE
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r, L.pattn_args(1, 2, 8, 51, 1 / 16), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), ws, 0)
    assert e.value.status == L.PA_ESHAPE                      # layers [1, 3) outside 2 layers
    r2 = L.Ring(L.rb_config(1, 2, 64, 0, 2, 8, L.PA_BF16), _fake(1), _fake(2))
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r2, L.pattn_args(0, 1, 7, 5, 1 / 8), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), ws, 0)
    assert e.value.status == L.PA_ESHAPE                      # 7 query heads over 2 KV heads
    r2.close()
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r, L.pattn_args(0, 2, 8, 0, 1 / 16), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), ws, 0)
    assert e.value.status == L.PA_ESHAPE                      # n_dyn = 0
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r, L.pattn_args(0, 2, 8, 51, -1.0), _fake(3), _fake(4), _fake(5), _fake(6), _fake(7), ws, 0)
    assert e.value.status == L.PA_EINVAL
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r, a, 0x10001, _fake(4), _fake(5), _fake(6), _fake(7), ws, 0)
    assert e.value.status == L.PA_EINVAL and "aligned" in str(e.value)
    assert L.pattn_workspace_bytes(r, L.pattn_args(0, 3, 8, 51, 1.0)) == 0
    r.close()


def test_workspace_grows_with_splits():
    from partitioned_kv_cache_amd import _lib as L
    r = L.Ring(L.rb_config(18, 1, 256, 256, 8, 768, L.PA_BF16), _fake(1), _fake(2))
    w4 = L.pattn_workspace_bytes(r, L.pattn_args(0, 18, 8, 51, 1 / 16, L.PA_F32, 4))
    w8 = L.pattn_workspace_bytes(r, L.pattn_args(0, 18, 8, 51, 1 / 16, L.PA_F32, 8))
    assert w8 > w4 > 0
    # 408 rows pad to 416; 8 splits x 18 layers x 416 rows x 256 dims of bf16 partial O
    # (a bf16 ring), plus FP32 (m, l)
    ml = ((8 * 18 * 416 * 8 + 255) // 256) * 256
    assert w8 == 8 * 18 * 416 * 256 * 2 + ml
    r.close()
    # an f32 ring keeps FP32 partial O
    r = L.Ring(L.rb_config(18, 1, 256, 256, 8, 768, L.PA_F32), _fake(1), _fake(2))
    assert L.pattn_workspace_bytes(r, L.pattn_args(0, 18, 8, 51, 1 / 16, L.PA_F32, 8)) == 8 * 18 * 416 * 256 * 4 + ml
    r.close()


def test_ada_validation_without_device():
    from partitioned_kv_cache_amd import _lib as L
    m = L.ada_mlp(_fake(1), _fake(2), _fake(3), _fake(4), 18, 128, 32, 1024, 1024)
    assert L.ada_gamma_workspace_bytes(m, 10) == 18 * 10 * 1024 * 2
    assert L.ada_gamma_workspace_bytes(m, 17) == 0
    with pytest.raises(L.PattnError) as e:
        L.ada_gamma(m, [0.5] * 17, _fake(5), _fake(6), _fake(7), 1 << 30, stream=0)
    assert e.value.status == L.PA_ESHAPE
    with pytest.raises(L.PattnError) as e:
        L.ada_rmsnorm_qkv(_fake(1), 65, 1024, _fake(2), 1e-6, _fake(3), 8, 1, 256, _fake(4), _fake(5), _fake(6),
                          None, _fake(7), 1 << 20, stream=0)
    assert e.value.status == L.PA_ESHAPE
    with pytest.raises(L.PattnError) as e:
        L.oproj_residual(_fake(1), _fake(2), _fake(3), 51, 2000, 1024, stream=0)
    assert e.value.status == L.PA_ESHAPE


def test_capsule_validation_without_device():
    """Sizes and state checks of rb_snapshot / rb_restore run on the host before any copy."""
    from partitioned_kv_cache_amd import _lib as L
    r = L.Ring(L.rb_config(2, 1, 64, 16, 4, 16, L.PA_F32), _fake(1), _fake(2))
    assert r.capsule_bytes() == 0                     # nothing pinned or pushed: an empty capsule
    st = r.snapshot(None, capsule_bytes=0, stream=0)
    assert st == {"head": 0, "count": 0, "pinned": 0, "frames_pushed": 0}
    r.restore(None, st, capsule_bytes=0, stream=0)
    # a full 4-slot window with 16 pinned tokens: 2 x 2 layers x (16 + 4 x 16) tokens x 64 x 4 bytes
    full = {"head": 1, "count": 4, "pinned": 16, "frames_pushed": 9}
    need = 2 * 2 * (16 + 4 * 16) * 64 * 4
    with pytest.raises(L.PattnError) as e:
        r.restore(_fake(3), full, capsule_bytes=need - 1, stream=0)
    assert e.value.status == L.PA_ERANGE
    for bad in ({"head": 2, "count": 4, "pinned": 16, "frames_pushed": 9},      # head != 9 mod 4
                {"head": 1, "count": 3, "pinned": 16, "frames_pushed": 9},      # count != min(9, 4)
                {"head": 0, "count": 0, "pinned": 17, "frames_pushed": 0},      # pinned > P
                {"head": 0, "count": 0, "pinned": 0, "frames_pushed": -1}):
        with pytest.raises(L.PattnError) as e:
            r.restore(_fake(3), bad, capsule_bytes=need, stream=0)
        assert e.value.status == L.PA_EINVAL
    assert r.state() == {"head": 0, "count": 0, "pinned": 0, "frames_pushed": 0}   # rejected restores change nothing
    r.close()



def test_staging_guards_without_device():
    """rb_stage_frame / rb_commit_frame reject misuse on the host, before any copy."""
    from partitioned_kv_cache_amd import _lib as L
    with pytest.raises(L.PattnError) as e:
        L.Ring(L.rb_config(1, 1, 64, 4, 2, 8, L.PA_F32, spare_slots=2), _fake(1), _fake(2))
    assert e.value.status == L.PA_EINVAL
    classic = L.Ring(L.rb_config(1, 1, 64, 4, 2, 8, L.PA_F32), _fake(1), _fake(2))
    with pytest.raises(L.PattnError) as e:
        classic.stage_frame(_fake(3), _fake(4), stream=0)
    assert e.value.status == L.PA_ESTATE and "spare" in str(e.value)
    spare = L.Ring(L.rb_config(1, 1, 64, 4, 2, 8, L.PA_F32, spare_slots=1), _fake(1), _fake(2))
    with pytest.raises(L.PattnError) as e:
        spare.commit_frame(stream=0)
    assert e.value.status == L.PA_ESTATE
    # the spare slot adds one frame to the buffers' layout: capsule of an empty ring stays empty
    assert spare.capsule_bytes() == 0 and spare.state()["head"] == 0
    classic.close()
    spare.close()


def test_pack_weight_validation_without_device():
    from partitioned_kv_cache_amd import _lib as L
    for args, status in [((None, 64, 64, _fake(2)), L.PA_EINVAL), ((_fake(1), 64, 64, _fake(1)), L.PA_EINVAL),
                         ((_fake(1) + 8, 64, 64, _fake(2)), L.PA_EINVAL), ((_fake(1), 48, 64, _fake(2)), L.PA_ESHAPE),
                         ((_fake(1), 64, 24, _fake(2)), L.PA_ESHAPE), ((_fake(1), 0, 64, _fake(2)), L.PA_ESHAPE)]:
        with pytest.raises(L.PattnError) as e:
            L.pa_pack_weight(*args, stream=0)
        assert e.value.status == status


def test_packed_stack_workspace_and_shape_checks_without_device():
    from partitioned_kv_cache_amd import _lib as L
    r = L.Ring(L.rb_config(18, 1, 256, 48, 2, 768, L.PA_BF16), _fake(1), _fake(2))
    w = [_fake(3 + i) for i in range(5)]
    full = dict(ffn_dim=4096, w_gate=w[2], w_up=w[3], w_down=w[4])
    plain = L.pa_denoise_step_workspace_bytes(r, L.pa_stack(18, 51, 1024, 8, w[0], w[1], 1e-6, 1 / 16, 0.1, **full))
    packed = L.pa_denoise_step_workspace_bytes(r, L.pa_stack(18, 51, 1024, 8, w[0], w[1], 1e-6, 1 / 16, 0.1,
                                                             packed=1, **full))
    # packed operands span all 64 row slots: the normalised GEMM operand
    # (model 1024), the attention output (Hq D = 2048) and the SwiGLU
    # activation (4096) each take 13 more rows of bf16; packed Q pads
    # 51 x 8 = 408 query rows to 13 blocks of 32 (416 rows of D = 256)
    up = lambda b: (b + 255) // 256 * 256
    assert packed - plain == (up(64 * 1024 * 2) - up(51 * 1024 * 2) + up(64 * 2048 * 2) - up(51 * 2048 * 2)
                              + up(64 * 4096 * 2) - up(51 * 4096 * 2) + up(416 * 256 * 2) - up(408 * 256 * 2))
    for kw in (dict(packed=2), dict(packed=1, model_dim=768), dict(packed=1, ffn_dim=5120)):
        md = kw.pop("model_dim", 1024)
        f = dict(full, ffn_dim=kw.pop("ffn_dim", 4096))
        assert L.pa_denoise_step_workspace_bytes(r, L.pa_stack(18, 51, md, 8, w[0], w[1], 1e-6, 1 / 16, 0.1,
                                                               **f, **kw)) == 0
    # 4 query heads of 256: Hq D = 1024 is a packed size; 3 heads (768) is not
    assert L.pa_denoise_step_workspace_bytes(r, L.pa_stack(18, 51, 1024, 4, w[0], w[1], 1e-6, 1 / 16, 0.1,
                                                           packed=1)) > 0
    assert L.pa_denoise_step_workspace_bytes(r, L.pa_stack(18, 51, 1024, 3, w[0], w[1], 1e-6, 1 / 16, 0.1,
                                                           packed=1)) == 0
    r.close()


def test_split_k_workspace_sizes_without_device():
    """The FFN workspace holds the bf16 activation and FP32 partials of the
    down projection per 512-wide chunk of ffn_dim; the stack adds partials of
    the out-projection when Hq * D is a multiple of 512."""
    from partitioned_kv_cache_amd import _lib as L
    up = lambda b: (b + 255) // 256 * 256  # noqa: E731
    for rows, model, ffn in [(51, 1024, 4096), (1, 256, 1024), (64, 768, 8192), (33, 512, 3072)]:
        assert L.ffn_swiglu_workspace_bytes(rows, model, ffn) == up(rows * ffn * 2) + up(ffn // 512 * rows * model * 4)
    r = L.Ring(L.rb_config(18, 1, 256, 48, 2, 768, L.PA_BF16), _fake(1), _fake(2))
    w = [_fake(3), _fake(4)]
    st = lambda hq: L.pa_stack(18, 51, 1024, hq, w[0], w[1], 1e-6, 1 / 16, 0.1)  # noqa: E731
    attn = lambda hq: L.pattn_workspace_bytes(r, L.pattn_args(0, 1, hq, 51, 1 / 16, L.PA_BF16))  # noqa: E731
    # h, normalised operand y, q, k, v, o, attention, out-projection partials (Hq D = 2048: 4 chunks)
    base = lambda hq: (2 * up(51 * 1024 * 2) + up(51 * hq * 256 * 2) + 2 * up(51 * 256 * 2)  # noqa: E731
                       + up(51 * hq * 256 * 2) + up(attn(hq)))
    assert L.pa_denoise_step_workspace_bytes(r, st(8)) == base(8) + up(4 * 51 * 1024 * 4)
    # Hq D = 768 is not a whole number of chunks: no partials, single-kernel out-projection
    assert L.pa_denoise_step_workspace_bytes(r, st(3)) == base(3)
    r.close()


def test_operand_q_validation_without_device():
    from partitioned_kv_cache_amd import _lib as L
    r = L.Ring(L.rb_config(18, 1, 256, 256, 8, 768, L.PA_BF16), _fake(1), _fake(2))
    a = L.pattn_args(0, 18, 8, 51, 1 / 16, L.PA_BF16, 0, L.PA_Q_OPERAND)
    # 51 tokens x 8 heads = 408 rows -> 13 blocks of 32, 18 layers, D = 256, bf16
    assert L.pattn_operand_q_bytes(r, a) == 18 * 13 * 32 * 256 * 2
    with pytest.raises(L.PattnError) as e:
        L.pattn_pack_q(r, a, _fake(3), _fake(3), stream=0)        # in place
    assert e.value.status == L.PA_EINVAL
    with pytest.raises(L.PattnError) as e:
        L.pattn_step(r, L.pattn_args(0, 18, 8, 51, 1 / 16, L.PA_BF16, 0, 2), _fake(3), _fake(4), _fake(5), _fake(6),
                     _fake(7), 1 << 30, 0)
    assert e.value.status == L.PA_EINVAL and "q_layout" in str(e.value)
    r.close()
    rf = L.Ring(L.rb_config(1, 1, 64, 16, 4, 16, L.PA_F32), _fake(1), _fake(2))
    af = L.pattn_args(0, 1, 1, 8, 1 / 8, L.PA_F32, 0, L.PA_Q_OPERAND)
    assert L.pattn_operand_q_bytes(rf, af) == 0                         # f32 rings take token-major q
    with pytest.raises(L.PattnError) as e:
        L.pattn_pack_q(rf, af, _fake(3), _fake(4), stream=0)
    assert e.value.status == L.PA_EINVAL
    rf.close()
