"""No write lands outside the buffers the library is given: every output,
state and workspace is a view into a larger buffer whose margins hold a
sentinel byte; after the call the margins are unchanged, and the results are
the bits of the same call on plain buffers."""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import act_dtype, make_layer, to_dev, workspace_for_window  # noqa: E402

GUARD = 4096          # bytes on each side of a buffer
SENTINEL = 0xA5


class Guarded:
    """A tensor of `shape` and `dtype` with GUARD sentinel bytes either side."""

    def __init__(self, shape, dtype, init=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((GUARD + n + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)
        if init is not None:
            self.t.copy_(init)

    def intact(self):
        return bool((self.raw[:GUARD] == SENTINEL).all()) and bool((self.raw[GUARD + self.n:] == SENTINEL).all())


def _prefill_case():
    sh = synth.FULL
    case = synth.prefill_case(sh, [130, 0, 67, 1, 200], seed=71, with_state=True, with_conv_state=True)
    ad = act_dtype(sh)
    layer = make_layer(sh, case.params)
    x = {k: to_dev(v, ad) for k, v in case.inputs.items()}
    return sh, case, ad, layer, x


@pytest.mark.parametrize("window_slots, want_core, in_place", [(2, True, False), (None, False, True)],
                         ids=["windows-core", "default-in-place"])
def test_prefill_writes_stay_inside(window_slots, want_core, in_place):
    sh, case, ad, layer, x = _prefill_case()
    cu = to_dev(case.cu_seqlens)
    N, T = len(case.cu_seqlens) - 1, int(case.cu_seqlens[-1])
    S0, C0 = to_dev(case.initial_state), to_dev(case.conv_state, ad)
    wsb = (workspace_for_window(layer, N, T, window_slots, want_core) if window_slots
           else gdn.prefill_workspace_bytes(layer, N, T))

    def call(out, core, si, so, ci, co, ws):
        gdn.prefill_raw(layer, N=N, T_total=T, cu_seqlens=cu, q=x["q"], k=x["k"], v=x["v"], z=x["z"],
                        a=x["a"], b=x["b"], out=out, core_out=core, initial_state=si, final_state=so,
                        conv_state_in=ci, conv_state_out=co, workspace=ws)
        torch.cuda.synchronize()

    ref = {"out": torch.empty((T, sh.Hv, sh.dv), dtype=torch.float32, device="cuda"),
           "core": torch.empty((T, sh.Hv, sh.dv), dtype=torch.float32, device="cuda") if want_core else None,
           "fs": torch.empty_like(S0), "cs": torch.empty_like(C0)}
    call(ref["out"], ref["core"], S0, ref["fs"], C0, ref["cs"],
         torch.empty(wsb, dtype=torch.uint8, device="cuda"))

    out = Guarded((T, sh.Hv, sh.dv), torch.float32)
    core = Guarded((T, sh.Hv, sh.dv), torch.float32) if want_core else None
    st = Guarded(tuple(S0.shape), torch.float32, S0)
    cs = Guarded(tuple(C0.shape), ad, C0)
    fs = st if in_place else Guarded(tuple(S0.shape), torch.float32)
    co = cs if in_place else Guarded(tuple(C0.shape), ad)
    ws = Guarded((wsb,), torch.uint8)
    call(out.t, core.t if core else None, st.t, fs.t, cs.t, co.t, ws.t)
    for name, g in (("out", out), ("core_out", core), ("state", st), ("final_state", fs), ("conv", cs),
                    ("conv_out", co), ("workspace", ws)):
        if g is not None:
            assert g.intact(), name
    assert torch.equal(out.t, ref["out"])
    if want_core:
        assert torch.equal(core.t, ref["core"])
    assert torch.equal(fs.t, ref["fs"]) and torch.equal(co.t, ref["cs"])


def test_decode_writes_stay_inside():
    sh = synth.FULL
    B = 5
    ad = act_dtype(sh)
    layer = make_layer(sh, synth.layer_params(sh, 72))
    x = {k: to_dev(v, ad) for k, v in synth.token_inputs(sh, B, 73).items()}
    S0 = to_dev(synth.initial_states(sh, B, 74))
    C0 = to_dev(synth.conv_states(sh, B, 75), ad)
    out = Guarded((B, sh.Hv, sh.dv), torch.float32)
    core = Guarded((B, sh.Hv, sh.dv), torch.float32)
    st = Guarded(tuple(S0.shape), torch.float32, S0)
    cs = Guarded(tuple(C0.shape), ad, C0)
    ws_ref = gdn.decode_workspace(layer, B)
    ws = Guarded(tuple(ws_ref.shape), ws_ref.dtype, ws_ref)
    gdn.decode_raw(layer, B=B, q=x["q"], k=x["k"], v=x["v"], z=x["z"], a=x["a"], b=x["b"], out=out.t,
                   core_out=core.t, state_in=st.t, state_out=st.t, conv_state_in=cs.t, conv_state_out=cs.t,
                   workspace=ws.t)
    torch.cuda.synchronize()
    for name, g in (("out", out), ("core_out", core), ("state", st), ("conv", cs), ("workspace", ws)):
        assert g.intact(), name
    ref = gdn.decode(layer, x["q"], x["k"], x["v"], x["z"], x["a"], x["b"], S0.clone(), C0.clone(),
                     want_core=True)
    torch.cuda.synchronize()
    assert torch.equal(out.t, ref["out"]) and torch.equal(core.t, ref["core_out"])
    assert torch.equal(st.t, ref["final_state"]) and torch.equal(cs.t, ref["conv_state_out"])


def test_layer_writes_stay_inside():
    """The layer entry points (in_proj, the layer, out_proj) on guarded y,
    states and workspaces, prefill then decode."""
    sh = synth.FULL
    hidden = 2048
    p = synth.layer_params(sh, 76)
    w_in, w_out = synth.proj_weights(sh, hidden, 76)
    layer = make_layer(sh, p)
    bf = lambda a: to_dev(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)  # noqa: E731
    proj = gdn.Proj(hidden=hidden, w_in=bf(w_in), w_out=bf(w_out))
    lens = [90, 0, 33]
    cu_np = synth.cu_from_lengths(lens)
    T, N = int(cu_np[-1]), len(lens)
    cu = to_dev(cu_np)
    x = bf(synth.hidden_inputs(T, hidden, 77))
    y = Guarded((T, hidden), torch.float32)
    fs = Guarded((N, sh.Hv, sh.dk, sh.dv), torch.float32)
    cs = Guarded((N, sh.K - 1, sh.Cc), torch.bfloat16)
    wsb = gdn.layer_prefill_workspace_bytes(layer, proj, N, T)
    ws = Guarded((wsb,), torch.uint8)
    gdn.layer_prefill_raw(layer, proj, N=N, T_total=T, cu_seqlens=cu, x=x, y=y.t, final_state=fs.t,
                          conv_state_out=cs.t, workspace=ws.t)
    torch.cuda.synchronize()
    for name, g in (("y", y), ("final_state", fs), ("conv_out", cs), ("workspace", ws)):
        assert g.intact(), name
    # one decode step from those states, in place
    xd = bf(synth.hidden_inputs(N, hidden, 78))
    yd = Guarded((N, hidden), torch.float32)
    dws_b = gdn.layer_decode_workspace_bytes(layer, proj, N)
    dws = Guarded((dws_b,), torch.uint8, torch.zeros(dws_b, dtype=torch.uint8, device="cuda"))
    gdn.layer_decode_raw(layer, proj, B=N, x=xd, y=yd.t, state_in=fs.t, state_out=fs.t,
                         conv_state_in=cs.t, conv_state_out=cs.t, workspace=dws.t)
    torch.cuda.synchronize()
    for name, g in (("y", yd), ("state", fs), ("conv", cs), ("workspace", dws)):
        assert g.intact(), name
    assert bool(torch.isfinite(yd.t).all())


def test_verify_writes_stay_inside():
    """Multi-token verify with per-token state snapshots (the largest writes
    of a decode step) on guarded buffers, states in place."""
    sh = synth.FULL
    B, tok = 3, 4
    ad = act_dtype(sh)
    layer = make_layer(sh, synth.layer_params(sh, 79))
    x = {k: to_dev(v, ad) for k, v in synth.token_inputs(sh, B * tok, 80).items()}
    S0 = to_dev(synth.initial_states(sh, B, 81))
    C0 = to_dev(synth.conv_states(sh, B, 82), ad)
    out = Guarded((B * tok, sh.Hv, sh.dv), torch.float32)
    core = Guarded((B * tok, sh.Hv, sh.dv), torch.float32)
    st = Guarded(tuple(S0.shape), torch.float32, S0)
    cs = Guarded(tuple(C0.shape), ad, C0)
    snap = Guarded((B, tok, sh.Hv, sh.dk, sh.dv), torch.float32)
    gdn.decode_multi_raw(layer, B=B, tokens=tok, q=x["q"], k=x["k"], v=x["v"], z=x["z"], a=x["a"], b=x["b"],
                         out=out.t, core_out=core.t, state_in=st.t, state_out=st.t, conv_state_in=cs.t,
                         conv_state_out=cs.t, state_snapshots=snap.t)
    torch.cuda.synchronize()
    for name, g in (("out", out), ("core_out", core), ("state", st), ("conv", cs), ("snapshots", snap)):
        assert g.intact(), name
    ref = gdn.decode_multi(layer, x["q"], x["k"], x["v"], x["z"], x["a"], x["b"], S0.clone(), C0.clone(),
                           tok, want_core=True, want_snapshots=True)
    torch.cuda.synchronize()
    assert torch.equal(out.t, ref["out"]) and torch.equal(st.t, ref["final_state"])
    assert torch.equal(snap.t, ref["state_snapshots"])
