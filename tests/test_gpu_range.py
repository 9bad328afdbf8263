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
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import check_prefill, gpu_prefill, oracle_prefill  # noqa: E402


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
