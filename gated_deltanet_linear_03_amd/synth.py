"""Seeded synthetic inputs for the Gated DeltaNet layer.

This module is shared by the HIP path's tests/benchmark and by the fp64
oracle's tests; it therefore holds none of the layer's arithmetic -- only
random draws, bf16 rounding of the drawn values and the workload shapes.

Workloads (the layer shape is the 35B-A3B one described on the llmxabe
README, model section: 16 key heads, 32 value heads, 128-wide heads, a
fixed-size state of 32x128x128 fp32 per sequence and layer):

* ``tiny``     1 sequence of 64 tokens, 2 key / 4 value heads, dk = dv = 32,
               chunk 16, fp32 everywhere, zero initial state;
* ``prefill``  1 sequence of 4096 tokens, 16 / 32 heads, dk = dv = 128,
               chunk 64, bf16 activations, zero initial state;
* ``decode``   B sequences x one bf16 token, 30 stacked layers, carried fp32
               state and conv state;
* ``long``     1 sequence of 131072 tokens resuming from a random state;
* ``varlen``   8 packed sequences, lengths log-uniform in [512, 32768],
               per-sequence random initial states.

Distributions: q, k, v, z ~ N(0, 1); gate logits a, b ~ N(0, 1); conv
weights ~ N(0, 1/4); A_log ~ U(log 1, log 16); dt_bias ~ N(0, 0.1);
initial states ~ N(0, 0.02).  The second argument of N(., .) is read as the
variance.  Values are drawn in fp32 and rounded to nearest-even bf16 where
the workload is bf16, so the GPU and the oracle see identical bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32
    arrays whose values are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                                  # wraps only for NaN payloads
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclass
class LayerShape:
    Hk: int = 16
    Hv: int = 32
    dk: int = 128
    dv: int = 128
    K: int = 4
    chunk: int = 64
    act_dtype: str = "bf16"      # "bf16" or "fp32" for q/k/v/z/a/b, conv state
    eps_l2: float = 1e-6
    eps_rms: float = 1e-6

    @property
    def Cc(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)


TINY = LayerShape(Hk=2, Hv=4, dk=32, dv=32, K=4, chunk=16, act_dtype="fp32")
FULL = LayerShape()


def _act(x: np.ndarray, shape: LayerShape) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return bf16_round(x) if shape.act_dtype == "bf16" else x


def _normal(rng, size, std=1.0):
    return (rng.standard_normal(size, dtype=np.float32) * np.float32(std))


def layer_params(shape: LayerShape, seed: int, norm_w_jitter: bool = False,
                 A_log_range=(0.0, math.log(16.0))):
    """conv_w [Cc, K], A_log [Hv], dt_bias [Hv], norm_w [dv]; all fp32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    conv_w = _normal(rng, (shape.Cc, shape.K), 0.5)
    A_log = rng.uniform(A_log_range[0], A_log_range[1], shape.Hv).astype(np.float32)
    dt_bias = _normal(rng, (shape.Hv,), math.sqrt(0.1))
    if norm_w_jitter:
        norm_w = (1.0 + 0.1 * rng.standard_normal(shape.dv)).astype(np.float32)
    else:
        norm_w = np.ones(shape.dv, dtype=np.float32)
    return {"conv_w": conv_w, "A_log": A_log, "dt_bias": dt_bias,
            "norm_w": norm_w}


HIDDEN = 2048        # model width of the 35B-A3B shape (see the projection docs)


def proj_rows(shape: LayerShape) -> int:
    """Output rows of in_proj: q | k | v | z | a | b."""
    return 2 * shape.Hk * shape.dk + 2 * shape.Hv * shape.dv + 2 * shape.Hv


def proj_weights(shape: LayerShape, hidden: int, seed: int):
    """w_in [P, hidden] and w_out [hidden, Hv*dv], N(0, 1/fan_in), rounded to
    bf16 (values held as fp32 arrays), so projections of N(0, 1) inputs have
    unit variance like the token inputs."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 6])))
    w_in = bf16_round(_normal(rng, (proj_rows(shape), hidden), 1.0 / math.sqrt(hidden)))
    w_out = bf16_round(_normal(rng, (hidden, shape.Hv * shape.dv), 1.0 / math.sqrt(shape.Hv * shape.dv)))
    return w_in, w_out


def proj_weights_floored(shape: LayerShape, hidden: int, seed: int, floor: float = 2.0 ** -10):
    """proj_weights with every |w_in| raised to at least `floor` (sign
    kept): dense N(0, 1/fan_in) weights whose magnitudes span at most ~8
    binades, so that with sparse_hidden_inputs every in_proj sum is exact
    in fp32."""
    w_in, w_out = proj_weights(shape, hidden, seed)
    w_in = np.where(np.abs(w_in) < floor, np.where(w_in < 0, -floor, floor), w_in).astype(np.float32)
    return w_in, w_out


def sparse_hidden_inputs(T: int, hidden: int, seed: int, nnz: int = 8):
    """x [T, hidden] with nnz nonzeros per row at random columns, each one
    of +-1/2, +-1, +-2.  Against bf16 weights of magnitude in [2^-10, 1)
    each product has at most 9 significant bits and every partial sum of a
    row fits in 24 bits, so in_proj is exact in fp32 in any summation
    order: both sides of a parity test see the same projection bits."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 9])))
    x = np.zeros((T, hidden), dtype=np.float32)
    vals = np.array([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], dtype=np.float32)
    for t in range(T):
        cols = rng.choice(hidden, nnz, replace=False)
        x[t, cols] = rng.choice(vals, nnz)
    return x


def proj_weights_exact(shape: LayerShape, hidden: int, seed: int):
    """w_in with one nonzero per row, +-1 or +-1/2 at a random column, so a
    projection of bf16 inputs is exact in bf16 whatever the summation order
    (both sides of a parity test then see the same projection bits); w_out as
    in proj_weights."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 8])))
    P = proj_rows(shape)
    w_in = np.zeros((P, hidden), dtype=np.float32)
    cols = rng.integers(0, hidden, P)
    vals = rng.choice(np.array([-1.0, -0.5, 0.5, 1.0], dtype=np.float32), P)
    w_in[np.arange(P), cols] = vals
    _, w_out = proj_weights(shape, hidden, seed)
    return w_in, w_out


def hidden_inputs(T: int, hidden: int, seed: int):
    """x [T, hidden] ~ N(0, 1), rounded to bf16 (as fp32 values)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return bf16_round(_normal(rng, (T, hidden)))


TOKEN_BLOCK = 4096


def token_inputs(shape: LayerShape, T: int, seed: int):
    """q, k [T, Hk, dk]; v, z [T, Hv, dv]; a, b [T, Hv] in the activation
    dtype's values (held as fp32 arrays).  Each tensor is drawn in blocks of
    TOKEN_BLOCK tokens, block j of tensor i from its own stream
    SeedSequence([seed, 2, i, j]), so values do not depend on how many
    threads fill them."""
    import concurrent.futures as cf
    import os
    inner = {"q": (shape.Hk, shape.dk), "k": (shape.Hk, shape.dk),
             "v": (shape.Hv, shape.dv), "z": (shape.Hv, shape.dv),
             "a": (shape.Hv,), "b": (shape.Hv,)}
    out = {n: np.empty((T,) + s, dtype=np.float32) for n, s in inner.items()}
    jobs = [(i, n, j) for i, n in enumerate(inner) for j in range(0, T, TOKEN_BLOCK)]

    def fill(job):
        i, n, j = job
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2, i, j // TOKEN_BLOCK])))
        t1 = min(T, j + TOKEN_BLOCK)
        out[n][j:t1] = _act(_normal(rng, (t1 - j,) + inner[n]), shape)

    if len(jobs) > 8:
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, jobs))
    else:
        for job in jobs:
            fill(job)
    return out


def initial_states(shape: LayerShape, N: int, seed: int, var: float = 0.02):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    return _normal(rng, (N, shape.Hv, shape.dk, shape.dv), math.sqrt(var))


def conv_states(shape: LayerShape, N: int, seed: int):
    """Random carried conv states [N, K-1, Cc] (raw inputs ~ N(0,1))."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
    return _act(_normal(rng, (N, shape.K - 1, shape.Cc)), shape)


def varlen_lengths(N: int, seed: int, lo: int = 512, hi: int = 32768):
    """Lengths floor(exp(U(ln lo, ln hi))), one per sequence."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 5])))
    return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), N))).astype(np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@dataclass
class PrefillCase:
    shape: LayerShape
    cu_seqlens: np.ndarray
    inputs: dict
    params: dict
    initial_state: np.ndarray | None = None
    conv_state: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.size - 1)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])


def prefill_case(shape: LayerShape, lengths, seed: int, with_state=False,
                 with_conv_state=False, norm_w_jitter=False,
                 A_log_range=(0.0, math.log(16.0))) -> PrefillCase:
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    N = len(lengths)
    return PrefillCase(
        shape=shape, cu_seqlens=cu,
        inputs=token_inputs(shape, T, seed),
        params=layer_params(shape, seed, norm_w_jitter, A_log_range),
        initial_state=initial_states(shape, N, seed) if with_state else None,
        conv_state=conv_states(shape, N, seed) if with_conv_state else None,
        meta={"seed": seed})


def tiny_case(seed: int = 0) -> PrefillCase:
    """1 x 64 tokens, fp32, zero initial state."""
    return prefill_case(TINY, [64], seed)


def prefill_4k_case(seed: int = 1) -> PrefillCase:
    """1 x 4096 tokens at the 35B-A3B layer shape, zero initial state."""
    return prefill_case(FULL, [4096], seed)


def long_case(seed: int = 3, T: int = 131072) -> PrefillCase:
    """1 x 131072 tokens resuming from a N(0, 0.02) state, zero conv state."""
    return prefill_case(FULL, [T], seed, with_state=True)


def varlen_case(seed: int = 4, N: int = 8) -> PrefillCase:
    """8 packed sequences, log-uniform lengths, random initial states."""
    return prefill_case(FULL, varlen_lengths(N, seed), seed, with_state=True)
