"""State pools (state_slots) and the mixed serving step (gdn_step): results
through a pool match the fp64 oracle run on the pool entries' states and are
bit-identical to the dense layout, pool entries nobody names stay untouched,
and one gdn_step matches the oracle and equals the separate decode and
prefill calls (llmxabe README, status paragraph: prefill and decode batched
across parallel sequences)."""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import (act_dtype, check_against_oracle, make_layer, oracle_layer,  # noqa: E402
                         to_dev, workspace_for_window)


def _pool_np(sh, S, seed):
    return synth.initial_states(sh, S, seed), synth.conv_states(sh, S, seed + 1)


def _pool(sh, S, seed, ad):
    st, cs = _pool_np(sh, S, seed)
    return to_dev(st), to_dev(cs, ad)


def _np(t):
    return t.float().cpu().numpy()


def test_decode_through_a_pool_bitwise():
    sh = synth.FULL
    ad = act_dtype(sh)
    layer = make_layer(sh, synth.layer_params(sh, 401))
    S, slots = 9, [7, 2, 5, 0]
    B = len(slots)
    pst, pcs = _pool(sh, S, 402, ad)
    tn = synth.token_inputs(sh, B, 403)
    t = {k: to_dev(v, ad) for k, v in tn.items()}
    idx = torch.tensor(slots, device="cuda")
    dense = gdn.decode(layer, *(t[n] for n in "qkvzab"), pst[idx].clone(), pcs[idx].clone(),
                       in_place=True, want_core=True)
    before_st, before_cs = pst.clone(), pcs.clone()
    out = torch.empty_like(dense["out"])
    core = torch.empty_like(dense["core_out"])
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    gdn.decode_raw(layer, B=B, q=t["q"], k=t["k"], v=t["v"], z=t["z"], a=t["a"], b=t["b"],
                   out=out, core_out=core, state_in=pst, state_out=pst, conv_state_in=pcs,
                   conv_state_out=pcs, state_slots=sl, num_slots=S)
    torch.cuda.synchronize()
    assert torch.equal(out, dense["out"]) and torch.equal(core, dense["core_out"])
    assert torch.equal(pst[idx], dense["final_state"])
    assert torch.equal(pcs[idx], dense["conv_state_out"])
    rest = [i for i in range(S) if i not in slots]
    assert torch.equal(pst[rest], before_st[rest]) and torch.equal(pcs[rest], before_cs[rest])
    # the oracle on the named entries' states, one token per sequence
    S_np, C_np = _pool_np(sh, S, 402)
    ref = oracle_layer(sh, synth.layer_params(sh, 401), np.arange(B + 1), tn, S_np[slots], C_np[slots])
    check_against_oracle(np.arange(B + 1), ref, _np(out), _np(core), _np(pst[idx]), _np(pcs[idx]),
                         label="pool decode")


@pytest.mark.parametrize("window_slots", [None, 1])
def test_prefill_through_a_pool_bitwise(window_slots):
    sh = synth.TINY
    ad = act_dtype(sh)
    lens = [37, 0, 27, 1, 16]
    case = synth.prefill_case(sh, lens, seed=404)
    layer = make_layer(sh, case.params)
    S, slots = 8, [6, 1, 3, 7, 0]
    N = len(lens)
    pst, pcs = _pool(sh, S, 405, ad)
    x = {k: to_dev(v, ad) for k, v in case.inputs.items()}
    cu = to_dev(case.cu_seqlens)
    T = int(case.cu_seqlens[-1])
    idx = torch.tensor(slots, device="cuda")
    ws_bytes = (gdn.prefill_workspace_bytes(layer, N, T) if window_slots is None
                else workspace_for_window(layer, N, T, window_slots, with_core_out=False))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dense = gdn.prefill(layer, *(x[n] for n in "qkvzab"), cu, initial_state=pst[idx].clone(),
                        conv_state_in=pcs[idx].clone(), want_core=True, workspace=ws)
    before_st, before_cs = pst.clone(), pcs.clone()
    out = torch.empty_like(dense["out"])
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    gdn.prefill_raw(layer, N=N, T_total=T, cu_seqlens=cu, q=x["q"], k=x["k"], v=x["v"],
                    z=x["z"], a=x["a"], b=x["b"], out=out, initial_state=pst, final_state=pst,
                    conv_state_in=pcs, conv_state_out=pcs, workspace=ws, state_slots=sl,
                    num_slots=S)
    torch.cuda.synchronize()
    assert torch.equal(out, dense["out"])
    assert torch.equal(pst[idx], dense["final_state"])
    assert torch.equal(pcs[idx], dense["conv_state_out"])
    rest = [i for i in range(S) if i not in slots]
    assert torch.equal(pst[rest], before_st[rest]) and torch.equal(pcs[rest], before_cs[rest])
    S_np, C_np = _pool_np(sh, S, 405)
    ref = oracle_layer(sh, case.params, case.cu_seqlens, case.inputs, S_np[slots], C_np[slots])
    check_against_oracle(case.cu_seqlens, ref, _np(out), None, _np(pst[idx]), _np(pcs[idx]),
                         label=f"pool prefill w={window_slots}")


def test_step_mixed_equals_separate_calls():
    """One serving step over one pool: 3 prefill sequences and 4 decode
    sequences with disjoint entries."""
    sh = synth.FULL
    ad = act_dtype(sh)
    layer = make_layer(sh, synth.layer_params(sh, 406))
    S = 10
    pslots, dslots = [4, 9, 1], [0, 6, 2, 8]
    lens = [70, 5, 130]
    pcase = synth.prefill_case(sh, lens, seed=407)
    x = {k: to_dev(v, ad) for k, v in pcase.inputs.items()}
    cu = to_dev(pcase.cu_seqlens)
    T = int(pcase.cu_seqlens[-1])
    tn = synth.token_inputs(sh, len(dslots), 408)
    t = {k: to_dev(v, ad) for k, v in tn.items()}
    pst0, pcs0 = _pool(sh, S, 409, ad)
    ws = torch.empty(gdn.prefill_workspace_bytes(layer, len(lens), T), dtype=torch.uint8, device="cuda")

    def run(pst, pcs, mixed):
        pout = torch.empty((T, sh.Hv, sh.dv), dtype=torch.float32, device="cuda")
        dout = torch.empty((len(dslots), sh.Hv, sh.dv), dtype=torch.float32, device="cuda")
        pre = dict(N=len(lens), T_total=T, cu_seqlens=cu, q=x["q"], k=x["k"], v=x["v"], z=x["z"],
                   a=x["a"], b=x["b"], out=pout, initial_state=pst, final_state=pst,
                   conv_state_in=pcs, conv_state_out=pcs,
                   state_slots=torch.tensor(pslots, dtype=torch.int32, device="cuda"), num_slots=S)
        dec = dict(B=len(dslots), q=t["q"], k=t["k"], v=t["v"], z=t["z"], a=t["a"], b=t["b"],
                   out=dout, state_in=pst, state_out=pst, conv_state_in=pcs, conv_state_out=pcs,
                   state_slots=torch.tensor(dslots, dtype=torch.int32, device="cuda"), num_slots=S)
        if mixed:
            gdn.step_raw(layer, prefill=pre, decode=dec, workspace=ws)
        else:
            gdn.decode_raw(layer, **dec)
            gdn.prefill_raw(layer, workspace=ws, **pre)
        torch.cuda.synchronize()
        return pout, dout

    a_st, a_cs = pst0.clone(), pcs0.clone()
    b_st, b_cs = pst0.clone(), pcs0.clone()
    pa, da = run(a_st, a_cs, True)
    pb, db = run(b_st, b_cs, False)
    assert torch.equal(pa, pb) and torch.equal(da, db)
    assert torch.equal(a_st, b_st) and torch.equal(a_cs, b_cs)
    untouched = [i for i in range(S) if i not in pslots + dslots]
    assert torch.equal(a_st[untouched], pst0[untouched])
    # both halves of the step against the oracle on the entries' states
    params = synth.layer_params(sh, 406)
    S_np, C_np = _pool_np(sh, S, 409)
    ref_p = oracle_layer(sh, params, pcase.cu_seqlens, pcase.inputs, S_np[pslots], C_np[pslots])
    check_against_oracle(pcase.cu_seqlens, ref_p, _np(pa), None, _np(a_st[pslots]),
                         _np(a_cs[pslots]), label="step prefill")
    B = len(dslots)
    ref_d = oracle_layer(sh, params, np.arange(B + 1), tn, S_np[dslots], C_np[dslots])
    check_against_oracle(np.arange(B + 1), ref_d, _np(da), None, _np(a_st[dslots]),
                         _np(a_cs[dslots]), label="step decode")
