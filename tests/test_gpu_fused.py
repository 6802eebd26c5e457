"""GPU parity of the fused reader pass (pattn_fused_step): the action
suffix's rows and the decode streams' rows in one pass over the shared
[pin; window] keys (OxyGen review, core method).

Expected values come from the oracle: the action rows attend over
[pin; window; suffix] (Eq. 1), each decode row over [pin; window; its own
tail] and never the suffix. Bar: max|gpu - ref| / max|ref| <= 2e-2 per output
tensor; the fused results also agree with the two separate passes within
that bar (they differ in rounding order only).
"""

import numpy as np
import pytest
import torch

from oracle import decode
from oracle.attention import full_attention
from partitioned_kv_cache_amd import configs, synth

pytestmark = pytest.mark.gpu

from tests.gpu_helpers import Scenario, dev, host, lib, rel_err, tdtype  # noqa: E402

BAR = 2e-2


def _banner(msg):
    print(f"[gpu] {msg}", flush=True)


# The last case is the benchmark's launch: 18 layers, 16 streams, bf16 outputs.
@pytest.mark.parametrize("layers,G,n_act,cap,frames,splits,odt", [(3, 16, 51, 30, 9, 0, "f32"),
                                                                     (2, 1, 1, 4, 2, 0, "f32"),
                                                                     (2, 5, 17, 8, 3, 3, "f32"),
                                                                     (18, 16, 51, 30, 9, 0, "f32"),
                                                                     (18, 16, 51, 30, 9, 0, "bf16")])
def test_fused_pass_matches_oracle_and_separate_passes(layers, G, n_act, cap, frames, splits, odt):
    L = lib()
    s = configs.SHARED_KV.with_(name=f"fused_{layers}_{G}_{n_act}", cfg_id=300 + layers + G, num_layers=layers,
                                n_streams=G, tail_capacity=cap, n_dyn=n_act)
    _banner(f"fused pass layers={layers} streams={G} action tokens={n_act} cap={cap} splits={splits} out={odt}")
    sc = Scenario(s)
    for f in range(frames):
        sc.push(f)
    hkv, D = s.n_kv_heads, s.head_dim
    lens = np.array([(3 * j) % (cap + 1) for j in range(G)], dtype=np.int32)     # includes 0 and cap
    tk = synth.normal((layers, G, cap, hkv, D), "bf16", s.cfg_id, synth.T_TAILK, 5)
    tv = synth.normal((layers, G, cap, hkv, D), "bf16", s.cfg_id, synth.T_TAILV, 5)
    q, kd, vd = synth.suffix_qkv(s, 0, 3)
    qd = synth.decode_q(s, frames, 0)
    od = L.PA_F32 if odt == "f32" else L.PA_BF16
    a = L.pattn_args(0, layers, s.n_q_heads, n_act, s.scale, od, splits)
    d = L.decode_args(0, layers, s.n_q_heads, G, cap, s.scale, od, splits)
    wsb = L.pattn_fused_workspace_bytes(sc.ring, a, d)
    assert wsb > 0
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((layers, n_act, s.n_q_heads, D), dtype=tdtype(odt), device="cuda")
    out_d = torch.empty((layers, G, s.n_q_heads, D), dtype=tdtype(odt), device="cuda")
    tk_d, tv_d, len_d = dev(tk), dev(tv), dev(lens)
    L.pattn_fused_step(sc.ring, a, dev(q), dev(kd), dev(vd), out, d, dev(qd), tk_d, tv_d, len_d, out_d, ws, wsb)
    # the two separate passes on the same inputs
    sep = sc.run_step(q, kd, vd, out_dtype=od, num_splits=splits)
    dwsb = L.pattn_decode_workspace_bytes(sc.ring, d)
    dws = torch.empty(dwsb, dtype=torch.uint8, device="cuda")
    out_d2 = torch.empty_like(out_d)
    L.pattn_decode(sc.ring, d, dev(qd), tk_d, tv_d, len_d, out_d2, dws, dwsb)
    torch.cuda.synchronize()
    got_a, got_d, sep_d = (synth.widen(host(t)) for t in (out, out_d, out_d2))
    worst = 0.0
    for l in sorted({0, layers // 2, layers - 1}):
        ref_a = sc.oracle_step(q, kd, vd, l)
        tails = decode.PrivateTails(G, cap, hkv, D)
        for j in range(G):
            for t in range(int(lens[j])):
                tails.append(j, synth.widen(tk[l, j, t]), synth.widen(tv[l, j, t]))
        ck, cv = sc.cached_context(l)
        ref_d = decode.decode_attention(synth.widen(qd[l]), ck, cv, tails, s.scale)
        e = max(rel_err(got_a[l], ref_a), rel_err(got_d[l], ref_d), rel_err(got_a[l], sep[l]),
                rel_err(got_d[l], sep_d[l]))
        worst = max(worst, e)
    _banner(f"  fused worst rel {worst:.3e}")
    assert worst <= BAR


def test_fused_rejects_mismatched_arguments():
    L = lib()
    s = configs.SHARED_KV.with_(name="fused_bad", cfg_id=320, num_layers=2)
    sc = Scenario(s)
    a = L.pattn_args(0, 2, s.n_q_heads, s.n_dyn, s.scale, L.PA_F32)
    d = L.decode_args(0, 2, s.n_q_heads, 4, 8, s.scale * 2, L.PA_F32)
    assert L.pattn_fused_workspace_bytes(sc.ring, a, d) == 0
    d2 = L.decode_args(1, 1, s.n_q_heads, 4, 8, s.scale, L.PA_F32)
    assert L.pattn_fused_workspace_bytes(sc.ring, a, d2) == 0
