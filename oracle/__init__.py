"""fp64 CPU oracle for one Gated DeltaNet layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  It shares no code with the HIP library in
``gated_deltanet_linear_03_amd`` and neither side imports the other; the only
thing both sides use is the seeded input generator, which holds none of the
layer's arithmetic.

``gdn_oracle.c`` is the token-by-token fp64 definition (conv1d + SiLU, L2
norm, gates, the gated delta rule of Yang, Kautz and Hatamizadeh, "Gated
Delta Networks", ICLR 2025, and the SiLU(z)-gated RMSNorm).  ``layer_forward``
adds the projections either side (matrix products in fp64).  ``chunked.py``
is a second, chunk-parallel fp64 form of the same recurrence that exists only
to pin the chunk algebra against the sequential definition.

Every input is widened exactly to float64 before it reaches the C code
(bf16 and fp32 values are exactly representable in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("Hk", ctypes.c_int), ("Hv", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("K", ctypes.c_int), ("scale", ctypes.c_double),
                ("eps_l2", ctypes.c_double), ("eps_rms", ctypes.c_double)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_softplus.restype = ctypes.c_double
        L.oracle_softplus.argtypes = [ctypes.c_double]
        L.oracle_sigmoid.restype = ctypes.c_double
        L.oracle_sigmoid.argtypes = [ctypes.c_double]
        L.oracle_gates.restype = None
        L.oracle_gates.argtypes = [ctypes.c_double] * 4 + [dp, dp]
        L.oracle_l2norm.restype = None
        L.oracle_l2norm.argtypes = [ctypes.c_int, dp, ctypes.c_double,
                                    ctypes.c_double, dp]
        L.oracle_rmsnorm_gate.restype = None
        L.oracle_rmsnorm_gate.argtypes = [ctypes.c_int, dp, dp, dp,
                                          ctypes.c_double, dp]
        L.oracle_delta_rule.restype = None
        L.oracle_delta_rule.argtypes = ([ctypes.c_int] * 3 + [dp] * 5 +
                                        [dp, dp])
        L.oracle_gdn_forward.restype = ctypes.c_int
        L.oracle_gdn_forward.argtypes = (
            [ctypes.POINTER(_Dims), ctypes.c_int,
             ctypes.POINTER(ctypes.c_int64)] + [dp] * 16 + [ctypes.c_int])
        _lib = L
    return _lib


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


# ---- scalar and per-vector pieces (exposed for the pins) -----------------

def silu(x: float) -> float:
    return lib().oracle_silu(float(x))


def softplus(x: float) -> float:
    return lib().oracle_softplus(float(x))


def sigmoid(x: float) -> float:
    return lib().oracle_sigmoid(float(x))


def gates(a, b, A_log, dt_bias):
    g = ctypes.c_double()
    be = ctypes.c_double()
    lib().oracle_gates(float(a), float(b), float(A_log), float(dt_bias),
                       ctypes.byref(g), ctypes.byref(be))
    return g.value, be.value


def l2norm(x, eps: float, scale: float = 1.0):
    x = _f64(x)
    y = np.empty_like(x)
    lib().oracle_l2norm(x.size, _p(x), float(eps), float(scale), _p(y))
    return y


def rmsnorm_gate(o, z, w, eps: float):
    o, z, w = _f64(o), _f64(z), _f64(w)
    y = np.empty_like(o)
    lib().oracle_rmsnorm_gate(o.size, _p(o), _p(z), _p(w), float(eps), _p(y))
    return y


def delta_rule(q, k, v, g, beta, S0=None):
    """Bare gated delta rule for one head on normalised inputs.

    q, k [T, dk]; v [T, dv]; g, beta [T]; S0 [dv, dk] (S, not its transpose).
    Returns (o [T, dv], S_T [dv, dk]).
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else _f64(S0).copy()
    o = np.empty((T, dv))
    lib().oracle_delta_rule(T, dk, dv, _p(q), _p(k), _p(v), _p(g), _p(beta),
                            _p(S), _p(o))
    return o, S


@dataclass
class Dims:
    Hk: int
    Hv: int
    dk: int
    dv: int
    K: int = 4
    scale: float = 1.0
    eps_l2: float = 1e-6
    eps_rms: float = 1e-6

    @property
    def Cc(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


def gdn_forward(dims: Dims, cu_seqlens, q, k, v, z, a, b, conv_w, A_log,
                dt_bias, norm_w, state_in=None, conv_state_in=None,
                nthreads: int = 0):
    """The whole layer in fp64.  Shapes: q, k [T, Hk, dk]; v, z [T, Hv, dv];
    a, b [T, Hv]; conv_w [Cc, K]; A_log, dt_bias [Hv]; norm_w [dv];
    state_in [N, Hv, dk, dv] (S transposed); conv_state_in [N, K-1, Cc].

    Returns dict(out, core_out, final_state, conv_state_out), all float64.
    """
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.size - 1
    T = int(cu[-1]) if N > 0 else 0
    q, k, v, z, a, b = (_f64(x) for x in (q, k, v, z, a, b))
    conv_w, A_log, dt_bias, norm_w = (_f64(x) for x in
                                      (conv_w, A_log, dt_bias, norm_w))
    state_in = _f64(state_in)
    conv_state_in = _f64(conv_state_in)
    out = np.zeros((T, dims.Hv, dims.dv))
    core = np.zeros((T, dims.Hv, dims.dv))
    fs = np.zeros((N, dims.Hv, dims.dk, dims.dv))
    cs = np.zeros((N, dims.K - 1, dims.Cc))
    if nthreads <= 0:
        nthreads = os.cpu_count() or 1
    cd = _Dims(dims.Hk, dims.Hv, dims.dk, dims.dv, dims.K, dims.scale,
               dims.eps_l2, dims.eps_rms)
    rc = lib().oracle_gdn_forward(
        ctypes.byref(cd), N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        _p(q), _p(k), _p(v), _p(z), _p(a), _p(b), _p(conv_w), _p(A_log),
        _p(dt_bias), _p(norm_w), _p(state_in), _p(conv_state_in),
        _p(out), _p(core), _p(fs), _p(cs), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gdn_forward rejected its arguments")
    return {"out": out, "core_out": core, "final_state": fs,
            "conv_state_out": cs}


def round_bf16(x):
    """Round to the nearest bf16 value, ties to even (the dtype the layer's
    projection and gated output are handed over in), from float64 through
    float32: fp64 -> fp32 rounds to nearest, then the 16 low bits of the fp32
    pattern are rounded off to nearest-even."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def layer_forward(dims: Dims, cu_seqlens, x, w_in, w_out, conv_w, A_log, dt_bias,
                  norm_w, state_in=None, conv_state_in=None, nthreads: int = 0):
    """The layer with its projections: proj = x w_in^T handed over in bf16,
    split into q | k | v | z | a | b, the layer above, its gated output handed
    over in bf16, y = out w_out^T.  x [T, hidden]; w_in [P, hidden]; w_out
    [hidden, Hv*dv].  Returns gdn_forward's dict plus y (float64)."""
    x, w_in, w_out = _f64(x), _f64(w_in), _f64(w_out)
    T = x.shape[0]
    qk, hd = dims.Hk * dims.dk, dims.Hv * dims.dv
    proj = round_bf16(x @ w_in.T)
    q = proj[:, :qk].reshape(T, dims.Hk, dims.dk)
    k = proj[:, qk:2 * qk].reshape(T, dims.Hk, dims.dk)
    v = proj[:, 2 * qk:2 * qk + hd].reshape(T, dims.Hv, dims.dv)
    z = proj[:, 2 * qk + hd:2 * qk + 2 * hd].reshape(T, dims.Hv, dims.dv)
    a = proj[:, 2 * qk + 2 * hd:2 * qk + 2 * hd + dims.Hv]
    b = proj[:, 2 * qk + 2 * hd + dims.Hv:]
    res = gdn_forward(dims, cu_seqlens, q, k, v, z, a, b, conv_w, A_log, dt_bias, norm_w,
                      state_in=state_in, conv_state_in=conv_state_in, nthreads=nthreads)
    res["y"] = round_bf16(res["out"]).reshape(T, hd) @ w_out.T
    res["proj"] = proj
    return res
