"""gdn_prefill_noalloc, the prefill entry point that allocates nothing (its
workspace is the library's static device scratch array): through the C ABI
it gives the same bits as gdn_prefill with an allocated workspace, on two
calls in a row (the second smaller, so it runs over what the first left in
the shared array), and it refuses sizes that do not fit the array before
enqueueing anything."""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import act_dtype, make_layer, to_dev  # noqa: E402


def _buffers(sh, T, N, want_core):
    dev = "cuda"
    odt = torch.float32
    adt = act_dtype(sh)
    out = torch.full((T, sh.Hv, sh.dv), float("nan"), dtype=odt, device=dev)
    core = torch.full((T, sh.Hv, sh.dv), float("nan"), dtype=torch.float32, device=dev) if want_core else None
    fs = torch.full((N, sh.Hv, sh.dk, sh.dv), float("nan"), dtype=torch.float32, device=dev)
    cs = torch.zeros((N, sh.K - 1, sh.Cc), dtype=adt, device=dev)
    return out, core, fs, cs


def _run(sh, layer, case, noalloc, want_core):
    ad = act_dtype(sh)
    x = {k: to_dev(v, ad) for k, v in case.inputs.items()}
    cu = to_dev(case.cu_seqlens)
    N, T = case.N, case.T
    S0 = None if case.initial_state is None else to_dev(case.initial_state)
    C0 = None if case.conv_state is None else to_dev(case.conv_state, ad)
    out, core, fs, cs = _buffers(sh, T, N, want_core)
    kw = dict(N=N, T_total=T, cu_seqlens=cu, q=x["q"], k=x["k"], v=x["v"], z=x["z"], a=x["a"],
              b=x["b"], out=out, core_out=core, initial_state=S0, final_state=fs,
              conv_state_in=C0, conv_state_out=cs)
    if noalloc:
        gdn.prefill_noalloc_raw(layer, **kw)
    else:
        ws = torch.empty(gdn.prefill_workspace_bytes(layer, N, T), dtype=torch.uint8, device="cuda")
        gdn.prefill_raw(layer, workspace=ws, **kw)
    torch.cuda.synchronize()
    return out, core, fs, cs


@pytest.mark.parametrize("shape", ["full", "tiny"])
def test_noalloc_prefill_matches_prefill_twice(shape):
    sh = synth.FULL if shape == "full" else synth.TINY
    C = sh.chunk
    # first call: two sequences with states and the pre-norm output; second:
    # one shorter sequence without core_out (the array then also holds the
    # pre-norm output), over the first call's leftovers
    calls = [dict(lens=[11 * C + 5, 3 * C + 1], want_core=True, seed=701),
             dict(lens=[2 * C + 9], want_core=False, seed=702)]
    for i, c in enumerate(calls):
        print(f"noalloc {shape} call {i}: lens {c['lens']} core {c['want_core']}", flush=True)
        case = synth.prefill_case(sh, c["lens"], seed=c["seed"], with_state=True,
                                  with_conv_state=True, norm_w_jitter=True)
        layer = make_layer(sh, case.params)
        got = _run(sh, layer, case, True, c["want_core"])
        ref = _run(sh, layer, case, False, c["want_core"])
        for g, r, name in zip(got, ref, ("out", "core_out", "final_state", "conv_state_out")):
            if r is None:
                continue
            assert not torch.isnan(g).any(), name
            assert torch.equal(g, r), (i, name)


def test_noalloc_prefill_refuses_what_does_not_fit():
    """Without core_out the pre-norm output (fp16) must fit the array too:
    a 4096-token batch of the full shape needs 32 MiB for it plus the carry
    slots and one chunk slot, which fits; 16384 tokens need 128 MiB for it
    alone, which does not, and nothing is enqueued (the output keeps its
    poison)."""
    sh = synth.FULL
    layer = make_layer(sh, synth.layer_params(sh, 703))
    T = 16384
    ad = act_dtype(sh)
    x = torch.zeros((T, sh.Hv, sh.dv), dtype=ad, device="cuda")
    qk = torch.zeros((T, sh.Hk, sh.dk), dtype=ad, device="cuda")
    ab = torch.zeros((T, sh.Hv), dtype=ad, device="cuda")
    out = torch.full((T, sh.Hv, sh.dv), float("nan"), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GdnError) as ei:
        gdn.prefill_noalloc_raw(layer, N=1, T_total=T, cu_seqlens=cu, q=qk, k=qk, v=x, z=x, a=ab,
                                b=ab, out=out)
    assert ei.value.status == gdn.GDN_ERR_WORKSPACE and "noalloc" in ei.value.detail
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
