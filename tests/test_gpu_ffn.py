"""GPU parity of the SwiGLU FFN block (fused AdaRMSNorm + gate/up projection
with SiLU(gate) * up in the epilogue, then the down projection with the
residual and, optionally, the Euler update) and of the denoising step of the
full action-expert layer (attention block + FFN block per layer).

Bar: max|gpu - ref| / max|ref| <= 2e-2 per output tensor (bf16 storage, FP32
accumulation); expected values come from the oracle only.
"""

import numpy as np
import pytest
import torch

from oracle import adanorm, stack
from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, host, lib, rel_err  # noqa: E402

BAR = 2e-2


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


def _case(rows, model, ffn, seed):
    s = configs.PI05_18L_FFN.with_(name=f"ffn_{rows}_{model}_{ffn}", cfg_id=200 + seed, model_dim=model,
                                   ffn_dim=ffn, num_layers=1)
    wg, wu, wd = synth.ffn_weights(s, 0)
    h = synth.normal((rows, model), "bf16", s.cfg_id, synth.T_X, 1)
    gamma = (1.0 + 0.2 * synth._rng(s.cfg_id, 999).standard_normal(model)).astype(np.float32)
    return s, h, gamma, wg, wu, wd


@pytest.mark.parametrize("rows,model,ffn", [(51, 1024, 4096), (7, 256, 1024), (33, 512, 3072), (64, 768, 2048),
                                            (1, 1024, 8192)])
def test_ffn_swiglu_matches_oracle(rows, model, ffn):
    L = lib()
    _banner(f"ffn_swiglu rows={rows} model={model} ffn={ffn}")
    s, h, gamma, wg, wu, wd = _case(rows, model, ffn, rows)
    h_d = dev(h)
    wsb = L.ffn_swiglu_workspace_bytes(rows, model, ffn)
    up = lambda n: (n + 255) // 256 * 256  # noqa: E731
    # the bf16 activation, then FP32 partials of the down projection per 512-wide chunk of ffn
    assert wsb == up(rows * ffn * 2) + up(ffn // 512 * rows * model * 4)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.ffn_swiglu(h_d, rows, model, ffn, dev(gamma), s.eps, dev(wg), dev(wu), dev(wd), None, 0.0, flag, ws, wsb)
    torch.cuda.synchronize()
    ref = stack.ffn_swiglu(synth.widen(h), gamma.astype(np.float64), s.eps, synth.widen(wg), synth.widen(wu),
                           synth.widen(wd))
    act = synth.widen(host(ws[:rows * ffn * 2].view(torch.int16)).reshape(rows, ffn))
    e_act, e_h = rel_err(act, ref["act"]), rel_err(synth.widen(host(h_d)), ref["h"])
    _banner(f"  act rel {e_act:.2e}, h rel {e_h:.2e}")
    assert e_act <= BAR and e_h <= BAR
    assert int(host(flag)[0]) == 0


def test_ffn_swiglu_euler_update_and_nonfinite_flag():
    L = lib()
    s, h, gamma, wg, wu, wd = _case(51, 1024, 4096, 5)
    x = synth.normal((51, 1024), "bf16", s.cfg_id, synth.T_X, 2)
    h_d, x_d = dev(h), dev(x)
    wsb = L.ffn_swiglu_workspace_bytes(51, 1024, 4096)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.ffn_swiglu(h_d, 51, 1024, 4096, dev(gamma), s.eps, dev(wg), dev(wu), dev(wd), x_d, 0.1, flag, ws, wsb)
    torch.cuda.synchronize()
    ref = stack.ffn_swiglu(synth.widen(h), gamma.astype(np.float64), s.eps, synth.widen(wg), synth.widen(wu),
                           synth.widen(wd))
    assert rel_err(synth.widen(host(x_d)), stack.euler(synth.widen(x), ref["h"], 0.1)) <= BAR
    assert int(host(flag)[0]) == 0
    for row in (3, 40):                     # in either 32-row half of the operand
        bad = h.copy()
        bad[row, 17] = 0x7F80               # +Inf in bf16
        flag.zero_()
        L.ffn_swiglu(dev(bad), 51, 1024, 4096, dev(gamma), s.eps, dev(wg), dev(wu), dev(wd), None, 0.0, flag, ws, wsb)
        torch.cuda.synchronize()
        assert int(host(flag)[0]) == 1, row


def test_ffn_rejects_unsupported_sizes():
    L = lib()
    assert L.ffn_swiglu_workspace_bytes(51, 1536, 4096) == 0      # model_dim beyond 1024
    assert L.ffn_swiglu_workspace_bytes(51, 1024, 5120) == 0      # ffn_dim 5 x 1024
    assert L.ffn_swiglu_workspace_bytes(65, 1024, 4096) == 0      # more than 64 rows


def test_denoise_step_with_ffn_matches_oracle_chain():
    L = lib()
    s = configs.PI05_18L_FFN.with_(name="ffn_stack", cfg_id=210, num_layers=3)
    _banner("denoise step, full layer (attention + SwiGLU FFN), 3 layers")
    sc = Scenario(s)
    for f in range(3):
        sc.push(f)
    wq = [synth.proj_weights(s, l) for l in range(s.num_layers)]
    wf = [synth.ffn_weights(s, l) for l in range(s.num_layers)]
    keep = [dev(np.stack([w[i] for w in wq])) for i in range(2)] + [dev(np.stack([w[i] for w in wf])) for i in range(3)]
    st = L.pa_stack(s.num_layers, s.n_dyn, s.model_dim, s.n_q_heads, keep[0], keep[1], s.eps, s.scale, 0.1, 0,
                    s.ffn_dim, keep[2], keep[3], keep[4])
    wsb = L.pa_denoise_step_workspace_bytes(sc.ring, st)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    state = synth.robot_state(s, 2)
    t = stack.timesteps(10)[3]
    ga, gf = [], []
    for l in range(s.num_layers):
        ga.append(adanorm.gamma(*(synth.widen(a) for a in synth.mlp_weights(s, l)), t, synth.widen(state)))
        gf.append(adanorm.gamma(*(synth.widen(a) for a in synth.ffn_mlp_weights(s, l)), t, synth.widen(state)))
    ga32, gf32 = np.stack(ga).astype(np.float32), np.stack(gf).astype(np.float32)
    x = synth.flow_x(s, 2)
    x_d = dev(x)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.pa_denoise_step(sc.ring, st, x_d, dev(ga32), s.model_dim, flag, ws, wsb, gamma_ffn=dev(gf32))
    torch.cuda.synchronize()
    caches = [sc.cached_context(l) for l in range(s.num_layers)]
    ffns = [(gf32[l].astype(np.float64), *(synth.widen(w) for w in wf[l])) for l in range(s.num_layers)]
    x1, trace = stack.denoise_step(synth.widen(x), [g.astype(np.float64) for g in ga32], s.eps,
                                   [synth.widen(w[0]) for w in wq], [synth.widen(w[1]) for w in wq],
                                   [c[0] for c in caches], [c[1] for c in caches], s.scale, s.n_q_heads,
                                   s.n_kv_heads, s.head_dim, ffns=ffns)
    err = rel_err(synth.widen(host(x_d)), x1)
    _banner(f"  full-layer step x rel {err:.3e}")
    assert err <= BAR
    assert int(host(flag)[0]) == 0
    # every layer's stream (after its FFN): an l-layer step leaves h_l at the
    # head of the workspace
    rows, model = s.n_dyn, s.model_dim
    for nl in range(1, s.num_layers + 1):
        st_l = L.pa_stack(nl, s.n_dyn, s.model_dim, s.n_q_heads, keep[0], keep[1], s.eps, s.scale, 0.1, 0,
                          s.ffn_dim, keep[2], keep[3], keep[4])
        L.pa_denoise_step(sc.ring, st_l, dev(x), dev(ga32), s.model_dim, flag, ws, wsb, gamma_ffn=dev(gf32))
        torch.cuda.synchronize()
        h_l = synth.widen(host(ws[: rows * model * 2].view(torch.int16).reshape(rows, model)))
        e = rel_err(h_l, trace[nl - 1]["h"])
        _banner(f"  full-layer step h_{nl} rel {e:.3e}")
        assert e <= BAR
