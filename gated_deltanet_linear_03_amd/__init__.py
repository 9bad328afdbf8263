"""MI355X (gfx950) Gated DeltaNet layer: thin Python binding of ``libgdn.so``.

Every step of the layer runs in the HIP kernels behind the C ABI declared in
``include/gdn.h``; this module only marshals torch tensors (device memory)
and the current HIP stream into that ABI.  There is no fallback: if the
library is missing the import of the binding raises.

    import torch, gated_deltanet_linear_03_amd as gdn
    layer = gdn.Layer(Hk=16, Hv=32, dk=128, dv=128, chunk=64,
                      conv_w=..., A_log=..., dt_bias=..., norm_w=...)
    res = gdn.prefill(layer, q, k, v, z, a, b, cu_seqlens,
                      initial_state=None, conv_state_in=None)
    dec = gdn.decode(layer, q1, k1, v1, z1, a1, b1, state, conv_state)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARGUMENT = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE = 3
GDN_ERR_HIP = 4
GDN_DTYPE_FP32 = 0
GDN_DTYPE_BF16 = 1
GDN_STATUS_NONFINITE = 1
GDN_STATUS_BAD_INDEX = 2
GDN_GEMM_AUTO = 0
GDN_GEMM_TILED = 1
GDN_GEMM_FEW_ROWS = 2
GDN_GEMM_LIBRARY = 3
GDN_GEMM_LIBRARY_FEW_ROWS = 4

EXPORTS = ("gdn_abi_version", "gdn_prefill_workspace_bytes", "gdn_prefill",
           "gdn_prefill_timed", "gdn_prefill_launches", "gdn_decode", "gdn_decode_multi",
           "gdn_step", "gdn_snapshot_bytes", "gdn_snapshot_save", "gdn_snapshot_inspect",
           "gdn_snapshot_restore", "gdn_gemm_bf16", "gdn_layer_prefill_workspace_bytes",
           "gdn_layer_prefill", "gdn_layer_decode_workspace_bytes", "gdn_layer_decode",
           "gdn_status_string", "gdn_last_error", "gdn_selftest_mfma", "gdn_prefill_noalloc",
           "gdn_prefill_window_slots", "gdn_decode_workspace_bytes", "gdn_gemm_bf16_path")
NOALLOC_SCRATCH_BYTES = 128 << 20       # GDN_NOALLOC_SCRATCH_BYTES
SNAPSHOT_MAGIC = 0x50534E47
SNAPSHOT_VERSION = 1
PREFILL_KERNELS = ("prep", "scan", "epi")


class GdnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"gdn status {status}: {detail}")
        self.status = status
        self.detail = detail


class CSnapshotHeader(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("Hk", ctypes.c_int32), ("Hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("conv_K", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("state_bytes", ctypes.c_uint64), ("conv_bytes", ctypes.c_uint64),
                ("checksum", ctypes.c_uint64), ("reserved", ctypes.c_uint64)]


class CProj(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("w_in", ctypes.c_void_p), ("w_out", ctypes.c_void_p)]


class CLayerIO(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("T_total", ctypes.c_int64),
                ("cu_seqlens", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("y_dtype", ctypes.c_int32), ("initial_state", ctypes.c_void_p),
                ("final_state", ctypes.c_void_p), ("conv_state_in", ctypes.c_void_p),
                ("conv_state_out", ctypes.c_void_p), ("state_slots", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32), ("status", ctypes.c_void_p)]


class CLayerDecodeIO(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("y_dtype", ctypes.c_int32), ("state_in", ctypes.c_void_p),
                ("state_out", ctypes.c_void_p), ("conv_state_in", ctypes.c_void_p),
                ("conv_state_out", ctypes.c_void_p), ("state_slots", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32), ("status", ctypes.c_void_p)]


class CLayer(ctypes.Structure):
    _fields_ = [("Hk", ctypes.c_int32), ("Hv", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("conv_K", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("eps_l2", ctypes.c_float),
                ("eps_rms", ctypes.c_float),
                ("conv_w", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("norm_w", ctypes.c_void_p)]


_TOKEN_FIELDS = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                 ("v", ctypes.c_void_p), ("z", ctypes.c_void_p),
                 ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                 ("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
                 ("v_stride", ctypes.c_int64), ("z_stride", ctypes.c_int64),
                 ("a_stride", ctypes.c_int64), ("b_stride", ctypes.c_int64)]


class CPrefillIO(ctypes.Structure):
    _fields_ = ([("N", ctypes.c_int32), ("T_total", ctypes.c_int64),
                 ("cu_seqlens", ctypes.c_void_p)] + _TOKEN_FIELDS +
                [("initial_state", ctypes.c_void_p),
                 ("final_state", ctypes.c_void_p),
                 ("conv_state_in", ctypes.c_void_p),
                 ("conv_state_out", ctypes.c_void_p),
                 ("out", ctypes.c_void_p), ("core_out", ctypes.c_void_p),
                 ("state_slots", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
                 ("status", ctypes.c_void_p)])


class CDecodeIO(ctypes.Structure):
    _fields_ = ([("B", ctypes.c_int32)] + _TOKEN_FIELDS +
                [("state_in", ctypes.c_void_p), ("state_out", ctypes.c_void_p),
                 ("conv_state_in", ctypes.c_void_p),
                 ("conv_state_out", ctypes.c_void_p),
                 ("out", ctypes.c_void_p), ("core_out", ctypes.c_void_p),
                 ("state_slots", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
                 ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                 ("status", ctypes.c_void_p)])


_lib = None


def lib():
    """Load ``libgdn.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m gated_deltanet_linear_03_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_abi_version.argtypes = []
        L.gdn_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(CLayer),
                                                  ctypes.c_int32, ctypes.c_int64]
        L.gdn_prefill.restype = ctypes.c_int
        L.gdn_prefill.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CPrefillIO),
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.gdn_prefill_noalloc.restype = ctypes.c_int
        L.gdn_prefill_noalloc.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CPrefillIO),
                                          ctypes.c_void_p]
        L.gdn_step.restype = ctypes.c_int
        L.gdn_step.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CPrefillIO),
                               ctypes.POINTER(CDecodeIO), ctypes.c_void_p, ctypes.c_size_t,
                               ctypes.c_void_p]
        L.gdn_decode_multi.restype = ctypes.c_int
        L.gdn_decode_multi.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CDecodeIO),
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.gdn_prefill_launches.restype = ctypes.c_int64
        L.gdn_prefill_launches.argtypes = [ctypes.POINTER(CLayer), ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32]
        L.gdn_prefill_window_slots.restype = ctypes.c_int64
        L.gdn_prefill_window_slots.argtypes = [ctypes.POINTER(CLayer), ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_size_t, ctypes.c_int32]
        L.gdn_prefill_timed.restype = ctypes.c_int
        L.gdn_prefill_timed.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CPrefillIO),
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
        L.gdn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_decode_workspace_bytes.argtypes = [ctypes.POINTER(CLayer), ctypes.c_int32]
        L.gdn_decode.restype = ctypes.c_int
        L.gdn_decode.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CDecodeIO),
                                 ctypes.c_void_p]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_selftest_mfma.restype = ctypes.c_int
        L.gdn_selftest_mfma.argtypes = [ctypes.c_void_p] * 4
        L.gdn_gemm_bf16.restype = ctypes.c_int
        L.gdn_gemm_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.gdn_gemm_bf16_path.restype = ctypes.c_int
        L.gdn_gemm_bf16_path.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        L.gdn_layer_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_layer_prefill_workspace_bytes.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CProj),
                                                        ctypes.c_int32, ctypes.c_int64]
        L.gdn_layer_prefill.restype = ctypes.c_int
        L.gdn_layer_prefill.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CProj),
                                        ctypes.POINTER(CLayerIO), ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
        L.gdn_layer_decode_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_layer_decode_workspace_bytes.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CProj),
                                                       ctypes.c_int32]
        L.gdn_layer_decode.restype = ctypes.c_int
        L.gdn_layer_decode.argtypes = [ctypes.POINTER(CLayer), ctypes.POINTER(CProj),
                                       ctypes.POINTER(CLayerDecodeIO), ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        L.gdn_snapshot_bytes.restype = ctypes.c_size_t
        L.gdn_snapshot_bytes.argtypes = [ctypes.POINTER(CLayer)]
        L.gdn_snapshot_save.restype = ctypes.c_int
        L.gdn_snapshot_save.argtypes = [ctypes.POINTER(CLayer), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.gdn_snapshot_inspect.restype = ctypes.c_int
        L.gdn_snapshot_inspect.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.POINTER(CSnapshotHeader)]
        L.gdn_snapshot_restore.restype = ctypes.c_int
        L.gdn_snapshot_restore.argtypes = [ctypes.POINTER(CLayer), ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p]
        _lib = L
    return _lib


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, lib().gdn_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t, name, rows, row_elems, esize=None, whole=False):
    """Raise ValueError unless t (None passes) is a device tensor of at least
    `rows` rows, each of at least `row_elems` elements stored densely, with
    element size `esize`.  whole=True is for buffers the library addresses
    as packed rows of exactly `row_elems` elements (it takes no row stride
    for them): each row must then hold exactly that many elements and the
    rows must follow each other with no gap.  The library trusts the sizes
    it is given, so buffers are measured here, before any launch, rather
    than read or written out of bounds or at the wrong place."""
    if t is None:
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: a device tensor is required")
    if t.dim() < 1 or int(t.shape[0]) < rows:
        raise ValueError(f"{name}: {rows} rows needed, shape is {tuple(t.shape)}")
    if t.is_contiguous() and (esize is None or t.element_size() == esize):
        # the common case, in a few calls: dense rows packed back to back
        n0 = int(t.shape[0])
        if n0 == 0:
            return
        per = t.numel() // n0
        if per == row_elems or (per > row_elems and not whole):
            return
    per_row = 1
    for d in t.shape[1:]:
        per_row *= int(d)
    if per_row < row_elems:
        raise ValueError(f"{name}: rows of {row_elems} elements needed, shape is {tuple(t.shape)}")
    if whole and per_row != row_elems:
        raise ValueError(f"{name}: rows of exactly {row_elems} elements needed (the library takes "
                         f"no row stride for it), shape is {tuple(t.shape)}")
    if esize is not None and t.element_size() != esize:
        raise ValueError(f"{name}: {esize}-byte elements needed, not {t.element_size()}")
    step = 1
    for d in range(t.dim() - 1, 0, -1):
        if int(t.shape[d]) != 1 and int(t.stride(d)) != step:
            raise ValueError(f"{name}: the elements of a row must be contiguous")
        step *= int(t.shape[d])
    if whole and t.dim() > 1 and int(t.shape[0]) > 1 and int(t.stride(0)) != step:
        raise ValueError(f"{name}: rows must be packed back to back")


def _act_size(layer) -> int:
    return 2 if layer.act_dtype == GDN_DTYPE_BF16 else 4


def _out_size(layer) -> int:
    return 2 if layer.out_dtype == GDN_DTYPE_BF16 else 4


def _check_tokens(layer, rows, q, k, v, z, a, b, out, core_out):
    asz = _act_size(layer)
    _need(q, "q", rows, layer.Hk * layer.dk, asz)
    _need(k, "k", rows, layer.Hk * layer.dk, asz)
    _need(v, "v", rows, layer.Hv * layer.dv, asz)
    _need(z, "z", rows, layer.Hv * layer.dv, asz)
    _need(a, "a", rows, layer.Hv, asz)
    _need(b, "b", rows, layer.Hv, asz)
    _need(out, "out", rows, layer.Hv * layer.dv, _out_size(layer), whole=True)
    _need(core_out, "core_out", rows, layer.Hv * layer.dv, 4, whole=True)


def _check_states(layer, rows, state_in, state_out, conv_state_in, conv_state_out,
                  names=("state_in", "state_out")):
    se = layer.Hv * layer.dk * layer.dv
    ce = (layer.conv_K - 1) * layer.Cc
    _need(state_in, names[0], rows, se, 4, whole=True)
    _need(state_out, names[1], rows, se, 4, whole=True)
    _need(conv_state_in, "conv_state_in", rows, ce, _act_size(layer), whole=True)
    _need(conv_state_out, "conv_state_out", rows, ce, _act_size(layer), whole=True)


def _check_index(t, name, n):
    if t is None:
        return
    if not getattr(t, "is_cuda", False) or t.element_size() != 4 or t.numel() < n \
            or not t.is_contiguous():
        raise ValueError(f"{name}: a contiguous device int32 tensor of {n} entries is required")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class Layer:
    """Shape and parameters of one layer.  Parameters are fp32 device
    tensors: conv_w [Cc, 4], A_log [Hv], dt_bias [Hv], norm_w [dv]."""
    Hk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    conv_w: object
    A_log: object
    dt_bias: object
    norm_w: object
    act_dtype: int = GDN_DTYPE_BF16
    out_dtype: int = GDN_DTYPE_FP32
    scale: float | None = None
    eps_l2: float = 1e-6
    eps_rms: float = 1e-6
    conv_K: int = 4

    @property
    def Cc(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv

    def c(self) -> CLayer:
        # the parameters are measured once per set of tensors and shapes
        key = tuple((t.data_ptr(), t.numel()) if t is not None else None
                    for t in (self.conv_w, self.A_log, self.dt_bias, self.norm_w)) + \
            (self.Hk, self.Hv, self.dk, self.dv, self.conv_K)
        if getattr(self, "_checked", None) != key:
            _need(self.conv_w, "conv_w", self.Cc, self.conv_K, 4, whole=True)
            _need(self.A_log, "A_log", self.Hv, 1, 4, whole=True)
            _need(self.dt_bias, "dt_bias", self.Hv, 1, 4, whole=True)
            _need(self.norm_w, "norm_w", self.dv, 1, 4, whole=True)
            self._checked = key
        scale = self.scale if self.scale is not None else self.dk ** -0.5
        return CLayer(self.Hk, self.Hv, self.dk, self.dv, self.conv_K, self.chunk,
                      self.act_dtype, self.out_dtype, scale, self.eps_l2,
                      self.eps_rms, _ptr(self.conv_w), _ptr(self.A_log),
                      _ptr(self.dt_bias), _ptr(self.norm_w))


def _tok_stride(t):
    return 0 if t is None else int(t.stride(0))


def prefill_workspace_bytes(layer: Layer, N: int, T_total: int) -> int:
    cl = layer.c()
    n = lib().gdn_prefill_workspace_bytes(ctypes.byref(cl), int(N), int(T_total))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return int(n)


def prefill_launches(layer: Layer, N: int, T_total: int, workspace_bytes: int | None = None,
                     with_core_out: bool = False):
    """Names of the kernels gdn_prefill enqueues, in order, for these sizes
    and workspace size (default: gdn_prefill_workspace_bytes), with or
    without core_out: prep and scan per window of chunks, then epi."""
    if workspace_bytes is None:
        workspace_bytes = prefill_workspace_bytes(layer, N, T_total)
    cl = layer.c()
    n = lib().gdn_prefill_launches(ctypes.byref(cl), int(N), int(T_total), int(workspace_bytes),
                                   int(bool(with_core_out)))
    if n < 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return ["prep", "scan"] * ((n - 1) // 2) + ["epi"]


def prefill_window_slots(layer: Layer, N: int, T_total: int, workspace_bytes: int | None = None,
                         with_core_out: bool = False) -> int:
    """Chunk slots per window gdn_prefill runs with for these sizes and
    workspace size (default: gdn_prefill_workspace_bytes), with or without
    core_out."""
    if workspace_bytes is None:
        workspace_bytes = prefill_workspace_bytes(layer, N, T_total)
    cl = layer.c()
    n = lib().gdn_prefill_window_slots(ctypes.byref(cl), int(N), int(T_total), int(workspace_bytes),
                                       int(bool(with_core_out)))
    if n < 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return int(n)


def _status_ptr(status):
    """Pointer of an optional device int32 status word (checked)."""
    _check_index(status, "status", 1)
    return _ptr(status)


def _prefill_io(layer, N, T_total, cu_seqlens, q, k, v, z, a, b, out, core_out, initial_state,
                final_state, conv_state_in, conv_state_out, state_slots, num_slots, status=None):
    _check_tokens(layer, int(T_total), q, k, v, z, a, b, out, core_out)
    _check_index(cu_seqlens, "cu_seqlens", int(N) + 1)
    _check_index(state_slots, "state_slots", int(N))
    _check_index(status, "status", 1)
    _check_states(layer, int(num_slots) if state_slots is not None else int(N), initial_state,
                  final_state, conv_state_in, conv_state_out, ("initial_state", "final_state"))
    return CPrefillIO(int(N), int(T_total), _ptr(cu_seqlens),
                      _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(a), _ptr(b),
                      _tok_stride(q), _tok_stride(k), _tok_stride(v),
                      _tok_stride(z), _tok_stride(a), _tok_stride(b),
                      _ptr(initial_state), _ptr(final_state), _ptr(conv_state_in),
                      _ptr(conv_state_out), _ptr(out), _ptr(core_out), _ptr(state_slots),
                      int(num_slots), _ptr(status))


def _decode_io(layer, B, q, k, v, z, a, b, out, core_out, state_in, state_out, conv_state_in,
               conv_state_out, state_slots, num_slots, tokens=1, workspace=None, status=None):
    _check_tokens(layer, int(B) * int(tokens), q, k, v, z, a, b, out, core_out)
    _check_index(state_slots, "state_slots", int(B))
    _check_states(layer, int(num_slots) if state_slots is not None else int(B), state_in,
                  state_out, conv_state_in, conv_state_out)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return CDecodeIO(int(B), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(a), _ptr(b),
                     _tok_stride(q), _tok_stride(k), _tok_stride(v), _tok_stride(z),
                     _tok_stride(a), _tok_stride(b), _ptr(state_in), _ptr(state_out),
                     _ptr(conv_state_in), _ptr(conv_state_out), _ptr(out),
                     _ptr(core_out), _ptr(state_slots), int(num_slots), _ptr(workspace), int(wsb),
                     _status_ptr(status))


def prefill_raw(layer: Layer, *, N, T_total, cu_seqlens, q, k, v, z, a, b,
                out, core_out=None, initial_state=None, final_state=None,
                conv_state_in=None, conv_state_out=None, workspace=None,
                workspace_bytes=None, stream=None, events=None, state_slots=None,
                num_slots=0, status=None):
    """Call ``gdn_prefill`` on caller-provided buffers (no allocation).
    events: optional list of len(prefill_launches(...)) + 1 recorded
    torch.cuda.Event(enable_timing=True) objects; the call then goes through
    ``gdn_prefill_timed`` and consecutive events bracket each kernel.
    status: optional device int32 tensor, 0 after the call, or with bit
    GDN_STATUS_NONFINITE set when an output or final state is not finite,
    GDN_STATUS_BAD_INDEX when cu_seqlens or state_slots break their contract
    (nothing is then written)."""
    cl = layer.c()
    io = _prefill_io(layer, N, T_total, cu_seqlens, q, k, v, z, a, b, out, core_out, initial_state,
                     final_state, conv_state_in, conv_state_out, state_slots, num_slots, status)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is None:
        _check(lib().gdn_prefill(ctypes.byref(cl), ctypes.byref(io), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream)))
    else:
        arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        _check(lib().gdn_prefill_timed(ctypes.byref(cl), ctypes.byref(io), _ptr(workspace),
                                       int(workspace_bytes), _stream(stream), arr,
                                       len(events)))


def prefill_noalloc_raw(layer: Layer, *, N, T_total, cu_seqlens, q, k, v, z, a, b, out,
                        core_out=None, initial_state=None, final_state=None,
                        conv_state_in=None, conv_state_out=None, stream=None,
                        state_slots=None, num_slots=0, status=None):
    """Call ``gdn_prefill_noalloc``: gdn_prefill on caller-provided buffers
    with the library's static device scratch as the workspace."""
    cl = layer.c()
    io = _prefill_io(layer, N, T_total, cu_seqlens, q, k, v, z, a, b, out, core_out, initial_state,
                     final_state, conv_state_in, conv_state_out, state_slots, num_slots, status)
    _check(lib().gdn_prefill_noalloc(ctypes.byref(cl), ctypes.byref(io), _stream(stream)))


def prefill(layer: Layer, q, k, v, z, a, b, cu_seqlens, initial_state=None,
            conv_state_in=None, want_core=False, in_place=False, workspace=None,
            stream=None, status=None):
    """Allocate outputs with torch and run ``gdn_prefill``.

    q, k [T, Hk, dk]; v, z [T, Hv, dv]; a, b [T, Hv] (act dtype, may be
    token-strided views); cu_seqlens int32 [N+1] on the device.  Returns a
    dict with out, final_state, conv_state_out and (if asked) core_out.
    With in_place=True the states are updated in the given tensors."""
    import torch
    dev = q.device
    T = int(q.shape[0])
    N = int(cu_seqlens.numel() - 1)
    odt = torch.bfloat16 if layer.out_dtype == GDN_DTYPE_BF16 else torch.float32
    adt = torch.bfloat16 if layer.act_dtype == GDN_DTYPE_BF16 else torch.float32
    out = torch.empty((T, layer.Hv, layer.dv), dtype=odt, device=dev)
    core = torch.empty((T, layer.Hv, layer.dv), dtype=torch.float32, device=dev) if want_core else None
    if in_place and initial_state is not None:
        fs = initial_state
    else:
        fs = torch.empty((N, layer.Hv, layer.dk, layer.dv), dtype=torch.float32, device=dev)
    if in_place and conv_state_in is not None:
        cs = conv_state_in
    else:
        cs = torch.empty((N, layer.conv_K - 1, layer.Cc), dtype=adt, device=dev)
    if workspace is None:
        nb = prefill_workspace_bytes(layer, N, T)
        workspace = torch.empty(nb, dtype=torch.uint8, device=dev)
    prefill_raw(layer, N=N, T_total=T, cu_seqlens=cu_seqlens, q=q, k=k, v=v, z=z,
                a=a, b=b, out=out, core_out=core, initial_state=initial_state,
                final_state=fs, conv_state_in=conv_state_in, conv_state_out=cs,
                workspace=workspace, stream=stream, status=status)
    res = {"out": out, "final_state": fs, "conv_state_out": cs}
    if want_core:
        res["core_out"] = core
    return res


def decode_workspace_bytes(layer: Layer, B: int) -> int:
    """Bytes of a ``gdn_decode`` workspace for up to B sequences."""
    n = lib().gdn_decode_workspace_bytes(ctypes.byref(layer.c()), int(B))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return int(n)


def decode_workspace(layer: Layer, B: int, device="cuda"):
    """A zero-filled ``gdn_decode`` workspace for up to B sequences (every
    call leaves it zero-filled where it must be)."""
    import torch
    return torch.zeros(decode_workspace_bytes(layer, B), dtype=torch.uint8, device=device)


def decode_raw(layer: Layer, *, B, q, k, v, z, a, b, out, state_in, state_out,
               conv_state_in, conv_state_out, core_out=None, stream=None, state_slots=None,
               num_slots=0, workspace=None, status=None):
    """Call ``gdn_decode`` on caller-provided buffers (no allocation).  With
    state_slots (device int32 [B]) the states are pools of num_slots entries;
    with a workspace (``decode_workspace``) one work-group per value head
    (same bits).  status: optional device int32 tensor into which
    GDN_STATUS_BAD_INDEX is ORed when a pool entry is out of range (that
    sequence is skipped); the call never clears it."""
    cl = layer.c()
    io = _decode_io(layer, B, q, k, v, z, a, b, out, core_out, state_in, state_out, conv_state_in,
                    conv_state_out, state_slots, num_slots, workspace=workspace, status=status)
    _check(lib().gdn_decode(ctypes.byref(cl), ctypes.byref(io), _stream(stream)))


def step_raw(layer: Layer, *, prefill=None, decode=None, workspace=None, workspace_bytes=None,
             stream=None):
    """Call ``gdn_step``: prefill and decode are dicts of the keyword
    arguments prefill_raw / decode_raw take (buffers only), or None."""
    cl = layer.c()
    pio = dio = None
    if prefill is not None:
        f = dict(core_out=None, initial_state=None, final_state=None, conv_state_in=None,
                 conv_state_out=None, state_slots=None, num_slots=0, status=None)
        f.update(prefill)
        pio = _prefill_io(layer, f["N"], f["T_total"], f["cu_seqlens"], f["q"], f["k"], f["v"], f["z"],
                          f["a"], f["b"], f["out"], f["core_out"], f["initial_state"],
                          f["final_state"], f["conv_state_in"], f["conv_state_out"],
                          f["state_slots"], f["num_slots"], f["status"])
    if decode is not None:
        f = dict(core_out=None, state_slots=None, num_slots=0, workspace=None, status=None)
        f.update(decode)
        dio = _decode_io(layer, f["B"], f["q"], f["k"], f["v"], f["z"], f["a"], f["b"], f["out"],
                         f["core_out"], f["state_in"], f["state_out"], f["conv_state_in"],
                         f["conv_state_out"], f["state_slots"], f["num_slots"],
                         workspace=f["workspace"], status=f["status"])
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_step(ctypes.byref(cl), ctypes.byref(pio) if pio is not None else None,
                          ctypes.byref(dio) if dio is not None else None, _ptr(workspace),
                          int(workspace_bytes), _stream(stream)))


MAX_VERIFY_TOKENS = 16


def decode_multi_raw(layer: Layer, *, B, tokens, q, k, v, z, a, b, out, state_in, state_out,
                     conv_state_in, conv_state_out, core_out=None, state_snapshots=None,
                     stream=None):
    """Call ``gdn_decode_multi``: `tokens` tokens for each of B sequences
    (token tensors with B * tokens rows, sequence-major)."""
    cl = layer.c()
    io = _decode_io(layer, B, q, k, v, z, a, b, out, core_out, state_in, state_out, conv_state_in,
                    conv_state_out, None, 0, tokens=tokens)
    _need(state_snapshots, "state_snapshots", int(B),
          int(tokens) * layer.Hv * layer.dk * layer.dv, 4, whole=True)
    _check(lib().gdn_decode_multi(ctypes.byref(cl), ctypes.byref(io), int(tokens),
                                  _ptr(state_snapshots), _stream(stream)))


def decode_multi(layer: Layer, q, k, v, z, a, b, state, conv_state, tokens, in_place=True,
                 want_core=False, want_snapshots=False, stream=None):
    """Multi-token verify: q, k [B*tokens, Hk, dk]; v, z [B*tokens, Hv, dv];
    a, b [B*tokens, Hv]; state [B, Hv, dk, dv]; conv_state [B, 3, Cc].
    Returns out (and core_out, per-token state snapshots [B, tokens, Hv, dk,
    dv] if asked) plus the final states."""
    import torch
    dev = q.device
    B = int(state.shape[0])
    odt = torch.bfloat16 if layer.out_dtype == GDN_DTYPE_BF16 else torch.float32
    out = torch.empty((B * tokens, layer.Hv, layer.dv), dtype=odt, device=dev)
    core = torch.empty((B * tokens, layer.Hv, layer.dv), dtype=torch.float32, device=dev) if want_core else None
    snap = (torch.empty((B, tokens, layer.Hv, layer.dk, layer.dv), dtype=torch.float32, device=dev)
            if want_snapshots else None)
    st_out = state if in_place else torch.empty_like(state)
    cs_out = conv_state if in_place else torch.empty_like(conv_state)
    decode_multi_raw(layer, B=B, tokens=tokens, q=q, k=k, v=v, z=z, a=a, b=b, out=out,
                     state_in=state, state_out=st_out, conv_state_in=conv_state,
                     conv_state_out=cs_out, core_out=core, state_snapshots=snap, stream=stream)
    res = {"out": out, "final_state": st_out, "conv_state_out": cs_out}
    if want_core:
        res["core_out"] = core
    if want_snapshots:
        res["state_snapshots"] = snap
    return res


def decode(layer: Layer, q, k, v, z, a, b, state, conv_state, in_place=True,
           want_core=False, stream=None, workspace=None):
    """One token per sequence: q, k [B, Hk, dk]; v, z [B, Hv, dv]; a, b
    [B, Hv]; state [B, Hv, dk, dv] fp32; conv_state [B, 3, Cc].  Updates
    the states in place by default.  Returns a dict like ``prefill``."""
    import torch
    B = int(q.shape[0])
    odt = torch.bfloat16 if layer.out_dtype == GDN_DTYPE_BF16 else torch.float32
    out = torch.empty((B, layer.Hv, layer.dv), dtype=odt, device=q.device)
    core = torch.empty((B, layer.Hv, layer.dv), dtype=torch.float32, device=q.device) if want_core else None
    so = state if in_place else torch.empty_like(state)
    co = conv_state if in_place else torch.empty_like(conv_state)
    decode_raw(layer, B=B, q=q, k=k, v=v, z=z, a=a, b=b, out=out, state_in=state,
               state_out=so, conv_state_in=conv_state, conv_state_out=co,
               core_out=core, stream=stream, workspace=workspace)
    res = {"out": out, "final_state": so, "conv_state_out": co}
    if want_core:
        res["core_out"] = core
    return res


def gemm_bf16(A, B, C, stream=None, path=None):
    """C[M, N] = A[M, K] @ B[N, K]^T on the matrix cores: A, B bf16 device
    tensors (rows may be strided), C bf16 or fp32.  path: None (as
    gdn_gemm_bf16) or one of GDN_GEMM_AUTO / TILED / FEW_ROWS / LIBRARY /
    LIBRARY_FEW_ROWS."""
    import torch
    M, K = int(A.shape[0]), int(A.shape[1])
    N = int(B.shape[0])
    _need(A, "A", M, K, 2)
    _need(B, "B", N, K, 2)
    _need(C, "C", M, N)
    cd = GDN_DTYPE_BF16 if C.dtype == torch.bfloat16 else GDN_DTYPE_FP32
    if path is None:
        _check(lib().gdn_gemm_bf16(_ptr(A), int(A.stride(0)), _ptr(B), int(B.stride(0)), _ptr(C),
                                   int(C.stride(0)), cd, M, N, K, _stream(stream)))
    else:
        _check(lib().gdn_gemm_bf16_path(_ptr(A), int(A.stride(0)), _ptr(B), int(B.stride(0)), _ptr(C),
                                        int(C.stride(0)), cd, M, N, K, int(path), _stream(stream)))


@dataclass
class Proj:
    """The projections either side of the layer: w_in [P, hidden] and w_out
    [hidden, Hv*dv], bf16 device tensors (P = 2 Hk dk + 2 Hv dv + 2 Hv, rows
    q | k | v | z | a | b)."""
    hidden: int
    w_in: object
    w_out: object

    def check(self, layer: Layer):
        P = 2 * layer.Hk * layer.dk + 2 * layer.Hv * layer.dv + 2 * layer.Hv
        _need(self.w_in, "w_in", P, self.hidden, 2, whole=True)
        _need(self.w_out, "w_out", self.hidden, layer.Hv * layer.dv, 2, whole=True)

    def c(self) -> CProj:
        return CProj(self.hidden, _ptr(self.w_in), _ptr(self.w_out))


def layer_prefill_workspace_bytes(layer: Layer, proj: Proj, N: int, T_total: int) -> int:
    cl, cp = layer.c(), proj.c()
    n = lib().gdn_layer_prefill_workspace_bytes(ctypes.byref(cl), ctypes.byref(cp), int(N), int(T_total))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return int(n)


def layer_prefill_raw(layer: Layer, proj: Proj, *, N, T_total, cu_seqlens, x, y,
                      initial_state=None, final_state=None, conv_state_in=None,
                      conv_state_out=None, workspace=None, workspace_bytes=None,
                      state_slots=None, num_slots=0, stream=None, status=None):
    """Call ``gdn_layer_prefill``: x [T, hidden] bf16 -> y [T, hidden] (bf16
    or fp32), through in_proj, the layer and out_proj."""
    import torch
    cl, cp = layer.c(), proj.c()
    proj.check(layer)
    _need(x, "x", int(T_total), proj.hidden, 2, whole=True)
    _need(y, "y", int(T_total), proj.hidden, None, whole=True)
    _check_index(cu_seqlens, "cu_seqlens", int(N) + 1)
    _check_index(state_slots, "state_slots", int(N))
    _check_states(layer, int(num_slots) if state_slots is not None else int(N), initial_state,
                  final_state, conv_state_in, conv_state_out, ("initial_state", "final_state"))
    yd = GDN_DTYPE_BF16 if y is not None and y.dtype == torch.bfloat16 else GDN_DTYPE_FP32
    io = CLayerIO(int(N), int(T_total), _ptr(cu_seqlens), _ptr(x), _ptr(y), yd,
                  _ptr(initial_state), _ptr(final_state), _ptr(conv_state_in),
                  _ptr(conv_state_out), _ptr(state_slots), int(num_slots), _status_ptr(status))
    nb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    _check(lib().gdn_layer_prefill(ctypes.byref(cl), ctypes.byref(cp), ctypes.byref(io),
                                   _ptr(workspace), nb, _stream(stream)))


def layer_decode_workspace_bytes(layer: Layer, proj: Proj, B: int) -> int:
    cl, cp = layer.c(), proj.c()
    n = lib().gdn_layer_decode_workspace_bytes(ctypes.byref(cl), ctypes.byref(cp), int(B))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return int(n)


def layer_decode_raw(layer: Layer, proj: Proj, *, B, x, y, state_in, state_out, conv_state_in,
                     conv_state_out, workspace, workspace_bytes=None, state_slots=None, num_slots=0,
                     stream=None, status=None):
    """Call ``gdn_layer_decode``: x [B, hidden] bf16 -> y [B, hidden], one
    token per sequence through in_proj, the decode step and out_proj."""
    import torch
    cl, cp = layer.c(), proj.c()
    proj.check(layer)
    _need(x, "x", int(B), proj.hidden, 2, whole=True)
    _need(y, "y", int(B), proj.hidden, None, whole=True)
    _check_index(state_slots, "state_slots", int(B))
    _check_states(layer, int(num_slots) if state_slots is not None else int(B), state_in,
                  state_out, conv_state_in, conv_state_out)
    yd = GDN_DTYPE_BF16 if y is not None and y.dtype == torch.bfloat16 else GDN_DTYPE_FP32
    io = CLayerDecodeIO(int(B), _ptr(x), _ptr(y), yd, _ptr(state_in), _ptr(state_out),
                        _ptr(conv_state_in), _ptr(conv_state_out), _ptr(state_slots), int(num_slots),
                        _status_ptr(status))
    nb = workspace_bytes if workspace_bytes is not None else (
        workspace.numel() * workspace.element_size() if workspace is not None else 0)
    _check(lib().gdn_layer_decode(ctypes.byref(cl), ctypes.byref(cp), ctypes.byref(io),
                                  _ptr(workspace), nb, _stream(stream)))


def snapshot_bytes(layer: Layer) -> int:
    cl = layer.c()
    n = lib().gdn_snapshot_bytes(ctypes.byref(cl))
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, lib().gdn_last_error().decode())
    return int(n)


def snapshot_save(layer: Layer, state, conv_state, slot: int = 0, num_slots=None, stream=None):
    """Park pool entry `slot` of state [num_slots, Hv, dk, dv] and conv_state
    [num_slots, K-1, Cc] (device tensors) into a new host buffer (a numpy
    uint8 array holding the header and the payload).  Synchronises the
    stream."""
    import numpy as np
    if num_slots is None:
        num_slots = int(state.shape[0])
    buf = np.zeros(snapshot_bytes(layer), dtype=np.uint8)
    cl = layer.c()
    _check_states(layer, int(num_slots), state, None, conv_state, None)
    _check(lib().gdn_snapshot_save(ctypes.byref(cl), _ptr(state), _ptr(conv_state), int(slot),
                                   int(num_slots), buf.ctypes.data, buf.nbytes, _stream(stream)))
    return buf


def snapshot_inspect(buf) -> dict:
    """Validate a snapshot held in a host bytes-like object; return its header."""
    import numpy as np
    arr = np.frombuffer(buf, dtype=np.uint8)
    hd = CSnapshotHeader()
    _check(lib().gdn_snapshot_inspect(arr.ctypes.data if arr.size else None, arr.nbytes,
                                      ctypes.byref(hd)))
    return {name: getattr(hd, name) for name, _ in CSnapshotHeader._fields_}


def snapshot_restore(layer: Layer, buf, state, conv_state, slot: int = 0, num_slots=None,
                     stream=None):
    """Write a snapshot back into pool entry `slot` of state / conv_state
    after checking it belongs to this layer.  Synchronises the stream."""
    import numpy as np
    if num_slots is None:
        num_slots = int(state.shape[0])
    arr = np.frombuffer(buf, dtype=np.uint8)
    cl = layer.c()
    _check_states(layer, int(num_slots), state, None, conv_state, None)
    _check(lib().gdn_snapshot_restore(ctypes.byref(cl), arr.ctypes.data if arr.size else None,
                                      arr.nbytes, _ptr(state), _ptr(conv_state), int(slot),
                                      int(num_slots), _stream(stream)))


def selftest_mfma(A, B, C, stream=None):
    _check(lib().gdn_selftest_mfma(_ptr(A), _ptr(B), _ptr(C), _stream(stream)))
