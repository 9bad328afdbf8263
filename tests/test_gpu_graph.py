"""Decode steps captured in a HIP graph (torch.cuda.CUDAGraph): every replay,
with eager work and synchronisations between replays, gives the same bits as
the eager step from the same state (the graph holds no memset nodes: the
library records only kernel launches)."""
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import act_dtype, make_layer, to_dev  # noqa: E402


@pytest.mark.parametrize("use_ws", [False, True])
def test_decode_graph_replays_match_eager(use_ws):
    """use_ws: the graph's steps run one work-group per value head with one
    shared decode workspace (its arrival counters reset themselves, so the
    graph needs no fill node); the eager reference runs without one."""
    sh = synth.FULL
    L, B, reps = 3, 4, 4
    ad = act_dtype(sh)
    layers = [make_layer(sh, synth.layer_params(sh, 300 + l)) for l in range(L)]
    toks = [{k: to_dev(v, ad) for k, v in synth.token_inputs(sh, B, 310 + l).items()} for l in range(L)]
    S0 = [to_dev(synth.initial_states(sh, B, 320 + l)) for l in range(L)]
    C0 = [to_dev(synth.conv_states(sh, B, 330 + l), ad) for l in range(L)]
    outs = [torch.empty((B, sh.Hv, sh.dv), dtype=torch.float32, device="cuda") for _ in range(L)]
    st = [s.clone() for s in S0]
    cs = [c.clone() for c in C0]
    ws = gdn.decode_workspace(layers[0], B)

    def step(state, conv, workspace=None):
        for l in range(L):
            t = toks[l]
            gdn.decode_raw(layers[l], B=B, q=t["q"], k=t["k"], v=t["v"], z=t["z"], a=t["a"],
                           b=t["b"], out=outs[l], state_in=state[l], state_out=state[l],
                           conv_state_in=conv[l], conv_state_out=conv[l], workspace=workspace)

    # eager reference: reps successive steps from S0, C0
    ref_st = [s.clone() for s in S0]
    ref_cs = [c.clone() for c in C0]
    ref = []
    for _ in range(reps):
        step(ref_st, ref_cs)
        ref.append(([o.clone() for o in outs], [s.clone() for s in ref_st]))
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(st, cs, ws if use_ws else None)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    # capturing did not run the step: restart from S0, C0 and replay
    for l in range(L):
        st[l].copy_(S0[l])
        cs[l].copy_(C0[l])
    torch.cuda.synchronize()
    for r in range(reps):
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(outs[l], ref[r][0][l]), (r, l)
            assert torch.equal(st[l], ref[r][1][l]), (r, l)
        del junk
