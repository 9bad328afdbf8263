"""The prefill scan's fp16 operand range.

Between chunks the scan feeds the state S and the pseudo-values
u = beta (v - e^g S k) to the matrix cores as fp16, which holds magnitudes
below 65504.  Inside that range the result meets the usual bar against the
fp64 oracle, whatever the scale; beyond it a conversion rounds to inf, and
the call reports that through its status word (GDN_STATUS_NONFINITE) rather
than passing a non-finite result on silently.  The layer is close to linear
in (S, v) jointly (the q/k norms do not see v; the output norm divides the
scale out), so scaling v and the initial state by a power of two moves the
scan's operands by that factor while the inputs stay exact in bf16."""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
import oracle
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import act_dtype, check_prefill, gpu_prefill, oracle_prefill, to_dev  # noqa: E402


def _scaled_case(scale, seed):
    case = synth.prefill_case(synth.FULL, [300, 130], seed=seed, with_state=True)
    case.inputs = dict(case.inputs)
    case.inputs["v"] = case.inputs["v"] * np.float32(scale)
    case.initial_state = case.initial_state * np.float32(scale)
    return case


def test_scaled_values_within_fp16_range_meet_the_bar():
    """v and S scaled by 2^10 (state entries up to ~1e3-1e4): parity with the
    oracle at the usual bar and a clear status word (set to 7 beforehand)."""
    case = _scaled_case(2.0 ** 10, 901)
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    res = gpu_prefill(case, status=status)
    smax = float(res["final_state"].abs().max())
    print(f"scaled 2^10: max |final state| {smax:.3e}, status {int(status.item())}", flush=True)
    assert int(status.item()) == 0
    check_prefill(case, res, oracle_prefill(case), label="scaled 2^10")


def test_beyond_fp16_range_is_reported():
    """v and S scaled by 2^17 push the scan's fp16 operands past 65504: the
    status word reports it; the next in-range call clears it again."""
    case = _scaled_case(2.0 ** 17, 902)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = gpu_prefill(case, status=status)
    finite = bool(torch.isfinite(res["out"]).all()) and bool(torch.isfinite(res["final_state"]).all())
    print(f"scaled 2^17: status {int(status.item())}, all finite {finite}", flush=True)
    assert int(status.item()) & gdn.GDN_STATUS_NONFINITE
    assert not finite
    gpu_prefill(_scaled_case(1.0, 903), status=status)
    assert int(status.item()) == 0


@pytest.mark.parametrize("want_core", [False, True], ids=["workspace-o", "core_out"])
def test_pre_norm_output_beyond_fp16_is_reported(want_core):
    """The prefill hands o to the gated norm as fp16, so o itself must stay
    below 65504 too.  A q scale of 2^14 with the state scaled by 2^6 keeps
    every fp16 operand of the scan in range (|q^| = 2^14, P and Q_G no
    larger, state entries below ~1e2) while some entries of o pass 65504
    (the oracle's o is checked for that).  The final state is still exact to the
    bar; `out` is not finite there, and the status word says so.  core_out,
    when asked for, keeps o in fp32 and stays finite."""
    sh = synth.FULL
    case = synth.prefill_case(sh, [300, 130], seed=904, with_state=True)
    case.initial_state = case.initial_state * np.float32(64.0)
    qscale = 2.0 ** 14
    d = oracle.Dims(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.K, qscale, sh.eps_l2, sh.eps_rms)
    x, p = case.inputs, case.params
    ref = oracle.gdn_forward(d, case.cu_seqlens, x["q"], x["k"], x["v"], x["z"], x["a"], x["b"],
                             p["conv_w"], p["A_log"], p["dt_bias"], p["norm_w"], case.initial_state, None)
    omax = float(np.abs(ref["core_out"]).max())
    assert omax > 65504 * 1.5, omax
    ad = act_dtype(sh)
    layer = gdn.Layer(Hk=sh.Hk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv, chunk=sh.chunk,
                      conv_w=to_dev(p["conv_w"]), A_log=to_dev(p["A_log"]), dt_bias=to_dev(p["dt_bias"]),
                      norm_w=to_dev(p["norm_w"]), act_dtype=gdn.GDN_DTYPE_BF16, out_dtype=gdn.GDN_DTYPE_FP32,
                      scale=qscale, eps_l2=sh.eps_l2, eps_rms=sh.eps_rms)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = gdn.prefill(layer, *(to_dev(x[n], ad) for n in "qkvzab"), to_dev(case.cu_seqlens),
                      initial_state=to_dev(case.initial_state), want_core=want_core, status=status)
    torch.cuda.synchronize()
    fs = res["final_state"].double().cpu().numpy()
    err = np.abs(fs - ref["final_state"]).max() / np.abs(ref["final_state"]).max()
    print(f"o beyond fp16 ({'core_out' if want_core else 'workspace'}): max |o| {omax:.3e}, "
          f"status {int(status.item())}, state err {err:.2e}", flush=True)
    assert int(status.item()) & gdn.GDN_STATUS_NONFINITE
    assert not bool(torch.isfinite(res["out"]).all())
    assert err < 2e-3
    if want_core:
        assert bool(torch.isfinite(res["core_out"]).all())
