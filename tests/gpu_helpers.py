"""Shared helpers of the GPU parity tests: move a synthetic case to the
device, run the HIP path through the C ABI, run the fp64 oracle on the same
bits, and compute the error metric.

Error metric (per output tensor and per sequence): max|y - r| / max|r|, the
worst absolute error scaled by the largest reference magnitude of that
sequence's tensor.  The bar is 2e-3 for fp32 outputs from bf16 inputs with
fp32 state; conv states must match exactly."""
from __future__ import annotations

import numpy as np
import torch

import gated_deltanet_linear_03_amd as gdn
import oracle

TOL = 2e-3


def dev():
    return torch.device("cuda:0")


def to_dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(dev())
    return t if dtype is None else t.to(dtype)


def act_dtype(shape):
    return torch.bfloat16 if shape.act_dtype == "bf16" else torch.float32


def make_layer(case_or_shape, params, out_dtype=gdn.GDN_DTYPE_FP32):
    sh = case_or_shape
    return gdn.Layer(Hk=sh.Hk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv, chunk=sh.chunk,
                     conv_w=to_dev(params["conv_w"]), A_log=to_dev(params["A_log"]),
                     dt_bias=to_dev(params["dt_bias"]), norm_w=to_dev(params["norm_w"]),
                     act_dtype=gdn.GDN_DTYPE_BF16 if sh.act_dtype == "bf16" else gdn.GDN_DTYPE_FP32,
                     out_dtype=out_dtype, scale=sh.scale, eps_l2=sh.eps_l2,
                     eps_rms=sh.eps_rms)


def dims(sh):
    return oracle.Dims(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.K, sh.scale, sh.eps_l2, sh.eps_rms)


def chunk_slot_bytes(Hv, dk, dv, C):
    """Operand-block bytes of one chunk slot (all value heads): -W and K_d^T
    as fp16 fragments, Q_G and P as fp16 hi + lo fragments, U~ as fp32
    fragments."""
    CK = max(C, 32)
    return Hv * (2 * C * dk + 4 * C * dk + 2 * dk * CK + 4 * C * CK + 4 * C * dv)


def workspace_for_window(layer, N, T, window_slots, with_core_out=True):
    """Workspace bytes that make gdn_prefill run windows of window_slots
    chunk slots (fewer, if that is more than the default), asking the
    library for the window each size gives: the default workspace less the
    slots beyond those, less more slots while the call's window (with core_out,
    the pre-norm output's share of the workspace is free for slots) is still
    wider."""
    slot = chunk_slot_bytes(layer.Hv, layer.dk, layer.dv, layer.chunk)
    full = gdn.prefill_workspace_bytes(layer, N, T)
    default = gdn.prefill_window_slots(layer, N, T, full)
    want = min(window_slots, default)
    nb = full - (default - want) * slot
    while gdn.prefill_window_slots(layer, N, T, nb, with_core_out) > want:
        nb -= slot
    assert gdn.prefill_window_slots(layer, N, T, nb, with_core_out) == want
    return nb


def gpu_prefill(case, out_dtype=gdn.GDN_DTYPE_FP32, want_core=True, in_place=False,
                window_slots=None, status=None):
    """window_slots: run with a workspace that holds only this many chunk
    slots of operand blocks (more, smaller windows); None = default."""
    sh = case.shape
    ad = act_dtype(sh)
    layer = make_layer(sh, case.params, out_dtype)
    x = {k: to_dev(v, ad) for k, v in case.inputs.items()}
    cu = to_dev(case.cu_seqlens)
    S0 = None if case.initial_state is None else to_dev(case.initial_state)
    C0 = None if case.conv_state is None else to_dev(case.conv_state, ad)
    ws = None
    if window_slots is not None:
        N, T = len(case.cu_seqlens) - 1, int(case.cu_seqlens[-1])
        ws = torch.empty(workspace_for_window(layer, N, T, window_slots, want_core), dtype=torch.uint8,
                         device="cuda")
    res = gdn.prefill(layer, x["q"], x["k"], x["v"], x["z"], x["a"], x["b"], cu,
                      initial_state=S0, conv_state_in=C0, want_core=want_core,
                      in_place=in_place, workspace=ws, status=status)
    torch.cuda.synchronize()
    return res


def oracle_prefill(case, heads_of_key=None, nthreads=0):
    """fp64 oracle on the same bits.  heads_of_key: restrict to the listed
    key heads (and their value heads), returning arrays for those heads."""
    sh = case.shape
    x = case.inputs
    p = case.params
    if heads_of_key is None:
        return oracle.gdn_forward(dims(sh), case.cu_seqlens, x["q"], x["k"], x["v"],
                                  x["z"], x["a"], x["b"], p["conv_w"], p["A_log"],
                                  p["dt_bias"], p["norm_w"], case.initial_state,
                                  case.conv_state, nthreads=nthreads)
    G = sh.Hv // sh.Hk
    hk = list(heads_of_key)
    hv = [h for k in hk for h in range(k * G, (k + 1) * G)]
    qk = sh.Hk * sh.dk
    ch = ([k * sh.dk + i for k in hk for i in range(sh.dk)] +
          [qk + k * sh.dk + i for k in hk for i in range(sh.dk)] +
          [2 * qk + h * sh.dv + j for h in hv for j in range(sh.dv)])
    d = oracle.Dims(len(hk), len(hv), sh.dk, sh.dv, sh.K, sh.scale, sh.eps_l2, sh.eps_rms)
    S0 = None if case.initial_state is None else case.initial_state[:, hv]
    C0 = None if case.conv_state is None else case.conv_state[:, :, ch]
    r = oracle.gdn_forward(d, case.cu_seqlens, x["q"][:, hk], x["k"][:, hk], x["v"][:, hv],
                           x["z"][:, hv], x["a"][:, hv], x["b"][:, hv], p["conv_w"][ch],
                           p["A_log"][hv], p["dt_bias"][hv], p["norm_w"], S0, C0,
                           nthreads=nthreads)
    r["heads"] = hv
    r["channels"] = ch
    return r


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    if den == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def per_seq_errors(cu, got, ref):
    """Token tensors [T, ...]: max over sequences of the metric."""
    errs = []
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b > a:
            errs.append(rel_err(got[a:b], ref[a:b]))
    return max(errs) if errs else 0.0


def state_errors(got, ref):
    return max(rel_err(got[n], ref[n]) for n in range(got.shape[0])) if got.shape[0] else 0.0


def oracle_layer(sh, params, cu, x, S0=None, C0=None, nthreads=0):
    """fp64 oracle over numpy token inputs x (dict q, k, v, z, a, b) with
    per-sequence states S0 [N, Hv, dk, dv] and C0 [N, K-1, Cc] (None =
    zeros)."""
    return oracle.gdn_forward(dims(sh), cu, x["q"], x["k"], x["v"], x["z"], x["a"], x["b"],
                              params["conv_w"], params["A_log"], params["dt_bias"],
                              params["norm_w"], S0, C0, nthreads=nthreads)


def check_against_oracle(cu, ref, out, core=None, state=None, conv=None, tol=TOL, label=""):
    """Per-sequence metric of out (and core_out, final states) against the
    oracle's dict; conv states exact.  Arrays are numpy, rows as in ref."""
    e_out = per_seq_errors(cu, np.asarray(out, dtype=np.float64), ref["out"])
    e_core = 0.0 if core is None else per_seq_errors(cu, core, ref["core_out"])
    e_state = 0.0 if state is None else state_errors(state, ref["final_state"])
    print(f"{label} vs oracle: out {e_out:.3e} core {e_core:.3e} state {e_state:.3e}", flush=True)
    assert e_out < tol and e_core < tol and e_state < tol, (label, e_out, e_core, e_state)
    if conv is not None:
        assert np.array_equal(np.asarray(conv, dtype=np.float64), ref["conv_state_out"]), label
    return e_out, e_core, e_state


def check_prefill(case, res, ref, tol=TOL, heads=None, label=""):
    cu = case.cu_seqlens
    sel = slice(None) if heads is None else heads
    out = res["out"].float().cpu().numpy()[:, sel]
    e_out = per_seq_errors(cu, out, ref["out"])
    e_core = per_seq_errors(cu, res["core_out"].cpu().numpy()[:, sel], ref["core_out"]) \
        if "core_out" in res else 0.0
    e_state = state_errors(res["final_state"].cpu().numpy()[:, sel], ref["final_state"])
    print(f"{label} out {e_out:.3e} core {e_core:.3e} state {e_state:.3e}", flush=True)
    assert e_out < tol and e_core < tol and e_state < tol, (e_out, e_core, e_state)
    cs = res["conv_state_out"].float().cpu().numpy()
    if heads is not None:
        cs = cs[:, :, ref["channels"]]
    assert np.array_equal(cs, ref["conv_state_out"]), "conv state differs"
    return e_out, e_core, e_state
