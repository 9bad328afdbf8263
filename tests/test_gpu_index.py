"""Device-side indices that break their contract are rejected on the GPU,
with no memory touched through them.

- prefill: cu_seqlens must start at 0, never decrease and end at T_total,
  and state_slots entries must lie in [0, num_slots).  A bad call writes
  nothing and sets GDN_STATUS_BAD_INDEX; the next good call on the same
  workspace is unaffected.
- decode: a sequence whose pool entry is out of range is skipped (its rows
  and every pool entry it would name keep their contents) and reported; the
  other sequences get the same bits as a batch without it."""
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import act_dtype, make_layer, to_dev  # noqa: E402

LENS = [100, 20, 50]          # cu_seqlens 0, 100, 120, 170
SLOTS = [3, 1, 2]
POOL = 4


def _prefill_setup(seed):
    sh = synth.FULL
    ad = act_dtype(sh)
    case = synth.prefill_case(sh, LENS, seed=seed)
    layer = make_layer(sh, case.params)
    x = {k: to_dev(v, ad) for k, v in case.inputs.items()}
    pst = to_dev(synth.initial_states(sh, POOL, seed + 1))
    pcs = to_dev(synth.conv_states(sh, POOL, seed + 2), ad)
    T, N = case.T, case.N
    ws = torch.zeros(gdn.prefill_workspace_bytes(layer, N, T), dtype=torch.uint8, device="cuda")
    return sh, layer, x, pst, pcs, T, N, ws


def _run_prefill(layer, x, sh, T, N, cu, slots, pst, pcs, ws, status):
    out = torch.full((T, sh.Hv, sh.dv), float("nan"), device="cuda")
    core = torch.full((T, sh.Hv, sh.dv), float("nan"), device="cuda")
    gdn.prefill_raw(layer, N=N, T_total=T, cu_seqlens=cu, q=x["q"], k=x["k"], v=x["v"], z=x["z"],
                    a=x["a"], b=x["b"], out=out, core_out=core, initial_state=pst, final_state=pst,
                    conv_state_in=pcs, conv_state_out=pcs, workspace=ws, state_slots=slots,
                    num_slots=POOL, status=status)
    torch.cuda.synchronize()
    return out, core


BAD = {
    "decreasing": ([0, 130, 120, 170], SLOTS),
    "end_short": ([0, 100, 120, 160], SLOTS),
    "end_long": ([0, 100, 120, 180], SLOTS),
    "start": ([4, 100, 120, 170], SLOTS),
    "slot_high": ([0, 100, 120, 170], [3, 4, 2]),
    "slot_negative": ([0, 100, 120, 170], [3, -1, 2]),
}


@pytest.mark.parametrize("kind", sorted(BAD))
def test_prefill_rejects_bad_device_indices(kind):
    sh, layer, x, pst, pcs, T, N, ws = _prefill_setup(61)
    cu_bad, slots_bad = BAD[kind]
    print(f"bad {kind}: cu {cu_bad} slots {slots_bad}", flush=True)
    st0, cs0 = pst.clone(), pcs.clone()
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    cu = torch.tensor(cu_bad, dtype=torch.int32, device="cuda")
    sl = torch.tensor(slots_bad, dtype=torch.int32, device="cuda")
    out, core = _run_prefill(layer, x, sh, T, N, cu, sl, pst, pcs, ws, status)
    assert int(status.item()) == gdn.GDN_STATUS_BAD_INDEX
    assert torch.isnan(out).all() and torch.isnan(core).all()
    assert torch.equal(pst, st0) and torch.equal(pcs, cs0)
    # the same without a status word: still nothing written
    out2, core2 = _run_prefill(layer, x, sh, T, N, cu, sl, pst, pcs, ws, None)
    assert torch.isnan(out2).all() and torch.isnan(core2).all()
    assert torch.equal(pst, st0) and torch.equal(pcs, cs0)
    # a good call on the same workspace afterwards: status cleared, results
    # equal to those of a fresh workspace
    cu_ok = torch.tensor([0, 100, 120, 170], dtype=torch.int32, device="cuda")
    sl_ok = torch.tensor(SLOTS, dtype=torch.int32, device="cuda")
    p1, c1 = pst.clone(), pcs.clone()
    o1, k1 = _run_prefill(layer, x, sh, T, N, cu_ok, sl_ok, p1, c1, ws, status)
    assert int(status.item()) == 0
    p2, c2 = pst.clone(), pcs.clone()
    o2, k2 = _run_prefill(layer, x, sh, T, N, cu_ok, sl_ok, p2, c2, torch.zeros_like(ws), None)
    for a, b in ((o1, o2), (k1, k2), (p1, p2), (c1, c2)):
        assert torch.equal(a, b)
    assert not torch.isnan(o1).any()


@pytest.mark.parametrize("use_ws", [False, True])
def test_decode_skips_out_of_range_slot(use_ws):
    sh = synth.FULL
    ad = act_dtype(sh)
    layer = make_layer(sh, synth.layer_params(sh, 71))
    S, slots, bad_row = 6, [4, 9, 0, 2], 1
    B = len(slots)
    pst = to_dev(synth.initial_states(sh, S, 72))
    pcs = to_dev(synth.conv_states(sh, S, 73), ad)
    tok = {k: to_dev(v, ad) for k, v in synth.token_inputs(sh, B, 74).items()}
    st0, cs0 = pst.clone(), pcs.clone()
    out = torch.full((B, sh.Hv, sh.dv), float("nan"), device="cuda")
    core = torch.full((B, sh.Hv, sh.dv), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = gdn.decode_workspace(layer, B) if use_ws else None
    print(f"decode slots {slots} pool {S} workspace {use_ws}", flush=True)
    gdn.decode_raw(layer, B=B, q=tok["q"], k=tok["k"], v=tok["v"], z=tok["z"], a=tok["a"], b=tok["b"],
                   out=out, core_out=core, state_in=pst, state_out=pst, conv_state_in=pcs,
                   conv_state_out=pcs, state_slots=torch.tensor(slots, dtype=torch.int32, device="cuda"),
                   num_slots=S, workspace=ws, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == gdn.GDN_STATUS_BAD_INDEX
    assert torch.isnan(out[bad_row]).all() and torch.isnan(core[bad_row]).all()
    # the batch without the bad sequence, from the same pool: the same bits
    keep = [i for i in range(B) if i != bad_row]
    rst, rcs = st0.clone(), cs0.clone()
    rout = torch.empty((len(keep), sh.Hv, sh.dv), device="cuda")
    rcore = torch.empty_like(rout)
    gdn.decode_raw(layer, B=len(keep), q=tok["q"][keep], k=tok["k"][keep], v=tok["v"][keep],
                   z=tok["z"][keep], a=tok["a"][keep], b=tok["b"][keep], out=rout, core_out=rcore,
                   state_in=rst, state_out=rst, conv_state_in=rcs, conv_state_out=rcs,
                   state_slots=torch.tensor([slots[i] for i in keep], dtype=torch.int32, device="cuda"),
                   num_slots=S)
    torch.cuda.synchronize()
    assert torch.equal(out[keep], rout) and torch.equal(core[keep], rcore)
    assert torch.equal(pst, rst) and torch.equal(pcs, rcs)
    untouched = [e for e in range(S) if e not in slots]
    assert torch.equal(pst[untouched], st0[untouched]) and torch.equal(pcs[untouched], cs0[untouched])
    if use_ws:
        # the skipped sequence counted no arrivals: the workspace is still
        # zero where it must be, and a good call through it gives the bits
        # of a call without one
        assert int(ws.count_nonzero().item()) == 0
        good = [4, 3, 0, 2]
        a_st, a_cs = st0.clone(), cs0.clone()
        b_st, b_cs = st0.clone(), cs0.clone()
        o_a = torch.empty((B, sh.Hv, sh.dv), device="cuda")
        o_b = torch.empty_like(o_a)
        for o_, s_, c_, w_ in ((o_a, a_st, a_cs, ws), (o_b, b_st, b_cs, None)):
            gdn.decode_raw(layer, B=B, q=tok["q"], k=tok["k"], v=tok["v"], z=tok["z"], a=tok["a"],
                           b=tok["b"], out=o_, state_in=s_, state_out=s_, conv_state_in=c_,
                           conv_state_out=c_, num_slots=S, workspace=w_,
                           state_slots=torch.tensor(good, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(o_a, o_b) and torch.equal(a_st, b_st) and torch.equal(a_cs, b_cs)
