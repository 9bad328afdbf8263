"""Session snapshots: park a sequence's state in host memory, clobber the
device copy, restore it (into another pool entry) and continue -- the
continuation must be bit-identical to the run that never stopped (skindeep.ai
"Our own inference runtime", "Session swap": restart-and-continue reproduces
the output exactly), and match the fp64 oracle's uninterrupted run over both
segments."""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import act_dtype, check_against_oracle, make_layer, oracle_layer, to_dev  # noqa: E402


@pytest.mark.parametrize("shape", ["full", "tiny"])
def test_restart_and_continue_bitwise(shape):
    sh = synth.FULL if shape == "full" else synth.TINY
    ad = act_dtype(sh)
    C = sh.chunk
    lens_a, lens_b = [3 * C + 5], [2 * C + 7]
    case_a = synth.prefill_case(sh, lens_a, seed=501)
    case_b = synth.prefill_case(sh, lens_b, seed=502)
    layer = make_layer(sh, case_a.params)
    S = 4
    S_np = synth.initial_states(sh, S, 503)
    C_np = synth.conv_states(sh, S, 504)
    pst0 = to_dev(S_np)
    pcs0 = to_dev(C_np, ad)

    def run(case, pst, pcs, slot):
        x = {k: to_dev(v, ad) for k, v in case.inputs.items()}
        T = int(case.cu_seqlens[-1])
        out = torch.empty((T, sh.Hv, sh.dv), dtype=torch.float32, device="cuda")
        ws = torch.empty(gdn.prefill_workspace_bytes(layer, 1, T), dtype=torch.uint8, device="cuda")
        sl = torch.tensor([slot], dtype=torch.int32, device="cuda")
        gdn.prefill_raw(layer, N=1, T_total=T, cu_seqlens=to_dev(case.cu_seqlens), q=x["q"],
                        k=x["k"], v=x["v"], z=x["z"], a=x["a"], b=x["b"], out=out,
                        initial_state=pst, final_state=pst, conv_state_in=pcs,
                        conv_state_out=pcs, workspace=ws, state_slots=sl, num_slots=S)
        torch.cuda.synchronize()
        return out

    # uninterrupted: A then B on entry 2
    ref_st, ref_cs = pst0.clone(), pcs0.clone()
    run(case_a, ref_st, ref_cs, 2)
    out_ref = run(case_b, ref_st, ref_cs, 2)

    # A, park entry 2, clobber the pools, resume into entry 1, then B
    st, cs = pst0.clone(), pcs0.clone()
    run(case_a, st, cs, 2)
    buf = gdn.snapshot_save(layer, st, cs, slot=2)
    hd = gdn.snapshot_inspect(buf)
    assert (hd["Hk"], hd["Hv"], hd["dk"], hd["dv"]) == (sh.Hk, sh.Hv, sh.dk, sh.dv)
    assert hd["state_bytes"] == sh.Hv * sh.dk * sh.dv * 4
    saved_state = st[2].clone()
    st.normal_()
    cs.copy_(torch.randn(cs.shape, device="cuda").to(cs.dtype))
    gdn.snapshot_restore(layer, buf, st, cs, slot=1)
    assert torch.equal(st[1], saved_state)
    out = run(case_b, st, cs, 1)
    assert torch.equal(out, out_ref)
    assert torch.equal(st[1], ref_st[2]) and torch.equal(cs[1], ref_cs[2])

    # the oracle without interruption: one sequence of both segments from
    # entry 2's original states; the resumed segment's outputs and the
    # states after it must match its tail
    La, Lb = lens_a[0], lens_b[0]
    xab = {k: np.concatenate([case_a.inputs[k], case_b.inputs[k]]) for k in case_a.inputs}
    ref = oracle_layer(sh, case_a.params, np.array([0, La + Lb]), xab, S_np[2:3], C_np[2:3])
    tail = {"out": ref["out"][La:], "core_out": ref["core_out"][La:],
            "final_state": ref["final_state"], "conv_state_out": ref["conv_state_out"]}
    check_against_oracle(np.array([0, Lb]), tail, out.cpu().numpy(), None, st[1:2].cpu().numpy(),
                         cs[1:2].float().cpu().numpy(), label=f"snapshot resume {shape}")

    # and a decode step from the restored entry matches one from the original
    t = {k: to_dev(v, ad) for k, v in synth.token_inputs(sh, 1, 505).items()}
    d_ref = gdn.decode(layer, *(t[n] for n in "qkvzab"), ref_st[2:3].clone(), ref_cs[2:3].clone())
    d = gdn.decode(layer, *(t[n] for n in "qkvzab"), st[1:2].clone(), cs[1:2].clone())
    torch.cuda.synchronize()
    assert torch.equal(d["out"], d_ref["out"]) and torch.equal(d["final_state"], d_ref["final_state"])
