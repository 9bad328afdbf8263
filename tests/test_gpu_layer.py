"""The projections either side of the layer: the bf16 matrix-core GEMM
against fp64 products of the same bf16 values, and gdn_layer_prefill /
gdn_layer_decode (in_proj -> layer -> out_proj) against the oracle's
layer_forward.  The layer tests take in_proj weights whose products are
exact in bf16, so both sides feed the layer identical bits (a projection
rounded from an fp32 and from an fp64 sum may differ by one bf16 ulp, and
one ulp in a gate input moves e^g by up to ~3% at A_log = ln 16); the GEMM
tests cover realistic weights."""
import numpy as np
import pytest
import torch

import gated_deltanet_linear_03_amd as gdn
import oracle
from gated_deltanet_linear_03_amd import synth

pytestmark = pytest.mark.gpu

from gpu_helpers import TOL, dims, make_layer, per_seq_errors, state_errors, to_dev  # noqa: E402


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


PATHS = [None, gdn.GDN_GEMM_TILED, gdn.GDN_GEMM_FEW_ROWS, gdn.GDN_GEMM_LIBRARY, gdn.GDN_GEMM_LIBRARY_FEW_ROWS]
PATH_IDS = ["auto", "tiled", "few_rows", "library", "library_few"]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("M, N, K", [(300, 200, 136), (1, 392, 64), (257, 12352, 2048),
                                     (64, 2048, 4096), (17, 12352, 2048), (40, 100, 200),
                                     (3, 2056, 4104)])
def test_gemm_matches_fp64(M, N, K, path):
    r = np.random.default_rng(M + N + K)
    A = synth.bf16_round(r.standard_normal((M, K)).astype(np.float32))
    B = synth.bf16_round((r.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32))
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    C32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    gdn.gemm_bf16(_bf16(A), _bf16(B), C32, path=path)
    gdn.gemm_bf16(_bf16(A), _bf16(B), C16, path=path)
    torch.cuda.synchronize()
    got = C32.cpu().numpy().astype(np.float64)
    # fp32 accumulation of K exact products: a few ulp of the largest partial sum
    bound = 4 * K * 2.0 ** -24 * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    if path in (gdn.GDN_GEMM_LIBRARY, gdn.GDN_GEMM_LIBRARY_FEW_ROWS) or path is None:
        # the library may pick another algorithm for a bf16 C: its result is
        # a rounding of some fp32 sum within the same bound
        g16 = C16.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g16 - ref) <= bound + 2.0 ** -8 * np.abs(ref) + 1e-30)
    else:
        # bf16 output: the nearest bf16 of the fp32 result
        assert torch.equal(C16.float(), C32.to(torch.bfloat16).float())


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("M", [130, 7])
def test_gemm_strided_rows(M, path):
    """Row strides beyond K (views into wider buffers), on every kernel
    family; by default 7 rows take the library's 64-row choice and 130 rows
    its 4096-row one."""
    r = np.random.default_rng(3)
    N, K = 70, 96
    Aw = _bf16(r.standard_normal((M, K + 24)))
    Bw = _bf16(r.standard_normal((N, K + 8)))
    A, B = Aw[:, 8:8 + K], Bw[:, :K]
    Cw = torch.zeros((M, N + 5), dtype=torch.float32, device="cuda")
    gdn.gemm_bf16(A, B, Cw[:, :N], path=path)
    torch.cuda.synchronize()
    ref = A.float().cpu().double() @ B.float().cpu().double().T
    assert torch.allclose(Cw[:, :N].cpu().double(), ref, rtol=1e-5, atol=1e-5)
    assert not Cw[:, N:].any()


def test_gemm_few_rows_batch_invariant():
    """Up to 64 rows (the default path's 64-row family): each output row's
    bits depend on its own A row only, not on how many rows are in the call."""
    r = np.random.default_rng(11)
    N, K = 12352, 2048
    A = _bf16(r.standard_normal((64, K)))
    B = _bf16(r.standard_normal((N, K)) / np.sqrt(K))
    full = torch.empty((64, N), dtype=torch.float32, device="cuda")
    gdn.gemm_bf16(A, B, full)
    for rows in ((0, 1), (5, 8), (16, 33), (60, 64)):
        part = torch.empty((rows[1] - rows[0], N), dtype=torch.float32, device="cuda")
        gdn.gemm_bf16(A[rows[0]:rows[1]], B, part)
        torch.cuda.synchronize()
        assert torch.equal(part, full[rows[0]:rows[1]]), rows


@pytest.mark.parametrize("path", [gdn.GDN_GEMM_LIBRARY, gdn.GDN_GEMM_LIBRARY_FEW_ROWS],
                         ids=["library", "library_few"])
@pytest.mark.parametrize("out", ["fp32", "bf16"])
@pytest.mark.parametrize("N, K", [(12352, 2048), (2048, 4096)])
def test_gemm_library_rows_do_not_depend_on_m(N, K, out, path):
    """The library paths (the layer's prefill and decode projections) keep
    one algorithm per shape: every row's bits are those of the largest
    product (more rows than either path's algorithm was chosen at, so it
    runs in row blocks), at any number of rows, and repeat calls give the
    same bits."""
    r = np.random.default_rng(N + K)
    M = 4096 + 97
    A = _bf16(r.standard_normal((M, K)))
    B = _bf16(r.standard_normal((N, K)) / np.sqrt(K))
    dt = torch.float32 if out == "fp32" else torch.bfloat16
    print(f"gemm rows case N={N} K={K} out={out} path={path}", flush=True)
    full = torch.empty((M, N), dtype=dt, device="cuda")
    gdn.gemm_bf16(A, B, full, path=path)
    again = torch.empty_like(full)
    gdn.gemm_bf16(A, B, again, path=path)
    torch.cuda.synchronize()
    assert torch.equal(full, again)
    for m in (1, 3, 64, 65, 300, 4095, 4096):
        part = torch.empty((m, N), dtype=dt, device="cuda")
        gdn.gemm_bf16(A[:m], B, part, path=path)
        torch.cuda.synchronize()
        assert torch.equal(part, full[:m]), m


_CHILD_GEMM = """
import hashlib, sys
import numpy as np, torch
sys.path.insert(0, sys.argv[1])
import gated_deltanet_linear_03_amd as gdn
M, N, K, path, f32 = (int(v) for v in sys.argv[2:7])
r = np.random.default_rng(M + N + K)
A = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).cuda().to(torch.bfloat16)
B = torch.from_numpy((r.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)).cuda().to(torch.bfloat16)
C = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
gdn.gemm_bf16(A, B, C, path=path)
torch.cuda.synchronize()
print(hashlib.sha256(C.cpu().contiguous().view(torch.uint8).numpy().tobytes()).hexdigest())
"""


@pytest.mark.parametrize("M, N, K, path, f32", [
    (300, 12352, 2048, gdn.GDN_GEMM_LIBRARY, 0),          # in_proj, split into 12288 + 64 columns
    (300, 2048, 4096, gdn.GDN_GEMM_LIBRARY, 1),           # out_proj, fp32 out
    (5, 12352, 2048, gdn.GDN_GEMM_LIBRARY_FEW_ROWS, 0),   # the decode projections' pin
])
def test_gemm_library_bits_same_in_another_process(M, N, K, path, f32):
    """The library path's algorithm is chosen without timing (the first
    no-workspace candidate the library ranks), so a second process on the
    same library and device computes the same bits."""
    import hashlib
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = np.random.default_rng(M + N + K)
    A = torch.from_numpy(r.standard_normal((M, K)).astype(np.float32)).cuda().to(torch.bfloat16)
    B = torch.from_numpy((r.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)).cuda().to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    gdn.gemm_bf16(A, B, C, path=path)
    torch.cuda.synchronize()
    mine = hashlib.sha256(C.cpu().contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
    print(f"child process: gemm M={M} N={N} K={K} path={path}", flush=True)
    out = subprocess.run([sys.executable, "-c", _CHILD_GEMM, root, str(M), str(N), str(K), str(path), str(f32)],
                         capture_output=True, text=True, timeout=90)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.split()[-1] == mine


def _layer_case(sh, hidden, lens, seed, with_states):
    p = synth.layer_params(sh, seed)
    # in_proj exact in bf16 (see proj_weights_exact): both sides hand the
    # layer the same projection bits
    w_in, w_out = synth.proj_weights_exact(sh, hidden, seed)
    cu = synth.cu_from_lengths(lens)
    T, N = int(cu[-1]), len(lens)
    x = synth.hidden_inputs(T, hidden, seed)
    S0 = synth.initial_states(sh, N, seed) if with_states else None
    C0 = synth.conv_states(sh, N, seed) if with_states else None
    return p, w_in, w_out, cu, x, S0, C0


def _run_layer(sh, hidden, p, w_in, w_out, cu, x, S0, C0):
    layer = make_layer(sh, p)
    proj = gdn.Proj(hidden=hidden, w_in=_bf16(w_in), w_out=_bf16(w_out))
    T, N = int(cu[-1]), len(cu) - 1
    y = torch.empty((T, hidden), dtype=torch.float32, device="cuda")
    fs = torch.empty((N, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device="cuda")
    cs = torch.empty((N, sh.K - 1, sh.Cc), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.layer_prefill_workspace_bytes(layer, proj, N, T), dtype=torch.uint8,
                     device="cuda")
    gdn.layer_prefill_raw(layer, proj, N=N, T_total=T, cu_seqlens=to_dev(cu), x=_bf16(x), y=y,
                          initial_state=None if S0 is None else to_dev(S0), final_state=fs,
                          conv_state_in=None if C0 is None else _bf16(C0), conv_state_out=cs,
                          workspace=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy(), fs.cpu().numpy(), cs.float().cpu().numpy()


@pytest.mark.parametrize("shape, hidden, lens, states", [
    ("small", 64, [37, 0, 27, 1, 16], True),
    ("full", 2048, [200], False),
    ("full", 2048, [70, 5, 130], True),
])
def test_layer_prefill_parity(shape, hidden, lens, states):
    sh = synth.FULL if shape == "full" else synth.LayerShape(Hk=2, Hv=4, dk=32, dv=32, chunk=16)
    p, w_in, w_out, cu, x, S0, C0 = _layer_case(sh, hidden, lens, 601, states)
    y, fs, cs = _run_layer(sh, hidden, p, w_in, w_out, cu, x, S0, C0)
    ref = oracle.layer_forward(dims(sh), cu, x, w_in, w_out, p["conv_w"], p["A_log"],
                               p["dt_bias"], p["norm_w"], state_in=S0, conv_state_in=C0)
    e_y = per_seq_errors(cu, y, ref["y"])
    e_s = state_errors(fs, ref["final_state"])
    print(f"layer {shape} {lens}: y {e_y:.3e} state {e_s:.3e}", flush=True)
    assert e_s < TOL
    # y: the gated output is handed to out_proj in bf16 on both sides, from
    # values that differ within the layer's tolerance, so an element may round
    # one bf16 ulp (2^-8 relative) apart; bound each y by that over its
    # |products| plus the layer tolerance of the sequence's largest |y|
    T = int(cu[-1])
    g = np.abs(oracle.round_bf16(ref["out"]).reshape(T, -1))
    handover = 2.0 ** -8 * (g @ np.abs(w_out.astype(np.float64)).T)
    for n_ in range(len(cu) - 1):
        a, b = int(cu[n_]), int(cu[n_ + 1])
        if b > a:
            scale = np.abs(ref["y"][a:b]).max()
            assert np.all(np.abs(y[a:b] - ref["y"][a:b]) <= handover[a:b] + TOL * scale), n_
    # the conv state holds raw projection values, exact on both sides
    assert np.array_equal(cs, ref["conv_state_out"])


@pytest.mark.parametrize("shape, hidden, B", [("small", 64, 5), ("full", 2048, 3), ("full", 2048, 64)])
def test_layer_decode_parity(shape, hidden, B):
    """One token per sequence through in_proj, the decode step and out_proj,
    against the oracle's layer on one-token sequences from the same states."""
    sh = synth.FULL if shape == "full" else synth.LayerShape(Hk=2, Hv=4, dk=32, dv=32, chunk=16)
    p = synth.layer_params(sh, 611)
    w_in, w_out = synth.proj_weights_exact(sh, hidden, 611)
    x = synth.hidden_inputs(B, hidden, 612)
    S0 = synth.initial_states(sh, B, 613)
    C0 = synth.conv_states(sh, B, 614)
    layer = make_layer(sh, p)
    proj = gdn.Proj(hidden=hidden, w_in=_bf16(w_in), w_out=_bf16(w_out))
    y = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    st = to_dev(S0)
    cs = _bf16(C0)
    ws = torch.zeros(gdn.layer_decode_workspace_bytes(layer, proj, B), dtype=torch.uint8, device="cuda")
    gdn.layer_decode_raw(layer, proj, B=B, x=_bf16(x), y=y, state_in=st, state_out=st,
                         conv_state_in=cs, conv_state_out=cs, workspace=ws)
    torch.cuda.synchronize()
    cu = np.arange(B + 1)
    ref = oracle.layer_forward(dims(sh), cu, x, w_in, w_out, p["conv_w"], p["A_log"],
                               p["dt_bias"], p["norm_w"], state_in=S0, conv_state_in=C0)
    yg = y.cpu().numpy()
    e_s = state_errors(st.cpu().numpy(), ref["final_state"])
    print(f"layer decode {shape} B={B}: y {per_seq_errors(cu, yg, ref['y']):.3e} state {e_s:.3e}",
          flush=True)
    assert e_s < TOL
    g = np.abs(oracle.round_bf16(ref["out"]).reshape(B, -1))
    handover = 2.0 ** -8 * (g @ np.abs(w_out.astype(np.float64)).T)
    for b in range(B):
        scale = np.abs(ref["y"][b]).max()
        assert np.all(np.abs(yg[b] - ref["y"][b]) <= handover[b] + TOL * scale), b


def test_layer_prefill_random_weights_elementwise():
    """Realistic dense in_proj weights (N(0, 1/fan_in), bf16, magnitudes
    floored at 2^-10) against sparse hidden inputs (8 nonzeros of +-1/2, +-1,
    +-2 per token): every projection sum is exact in fp32, so both sides hand
    the layer the same bits, and y is bounded element by element as in the
    other layer tests."""
    sh = synth.FULL
    hidden = 2048
    p = synth.layer_params(sh, 621)
    w_in, w_out = synth.proj_weights_floored(sh, hidden, 621)
    lens = [300, 45]
    cu = synth.cu_from_lengths(lens)
    T = int(cu[-1])
    x = synth.sparse_hidden_inputs(T, hidden, 622)
    S0 = synth.initial_states(sh, len(lens), 623)
    C0 = synth.conv_states(sh, len(lens), 624)
    y, fs, cs = _run_layer(sh, hidden, p, w_in, w_out, cu, x, S0, C0)
    ref = oracle.layer_forward(dims(sh), cu, x, w_in, w_out, p["conv_w"], p["A_log"],
                               p["dt_bias"], p["norm_w"], state_in=S0, conv_state_in=C0)
    e_y = per_seq_errors(cu, y, ref["y"])
    e_s = state_errors(fs, ref["final_state"])
    print(f"layer realistic weights: y {e_y:.3e} state {e_s:.3e}", flush=True)
    assert e_s < TOL
    g = np.abs(oracle.round_bf16(ref["out"]).reshape(T, -1))
    handover = 2.0 ** -8 * (g @ np.abs(w_out.astype(np.float64)).T)
    for n_ in range(len(lens)):
        a, b = int(cu[n_]), int(cu[n_ + 1])
        scale = np.abs(ref["y"][a:b]).max()
        assert np.all(np.abs(y[a:b] - ref["y"][a:b]) <= handover[a:b] + TOL * scale), n_
    assert np.array_equal(cs, ref["conv_state_out"])


def test_sparse_inputs_make_in_proj_exact():
    """The premise of the test above, on the GPU GEMM: its bf16 projection of
    sparse inputs against floored realistic weights equals the fp64 product
    rounded once to bf16, element for element."""
    sh = synth.FULL
    hidden = 2048
    w_in, _ = synth.proj_weights_floored(sh, hidden, 621)
    x = synth.sparse_hidden_inputs(64, hidden, 625)
    ref = oracle.round_bf16(x.astype(np.float64) @ w_in.astype(np.float64).T)
    C16 = torch.empty((64, w_in.shape[0]), dtype=torch.bfloat16, device="cuda")
    gdn.gemm_bf16(_bf16(x), _bf16(w_in), C16)
    torch.cuda.synchronize()
    assert np.array_equal(C16.float().cpu().numpy().astype(np.float64), ref)


def _layer_decode(sh, hidden, p, w_in, w_out, x, S0, C0):
    layer = make_layer(sh, p)
    proj = gdn.Proj(hidden=hidden, w_in=_bf16(w_in), w_out=_bf16(w_out))
    B = x.shape[0]
    y = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    st = to_dev(S0)
    cs = _bf16(C0)
    ws = torch.zeros(gdn.layer_decode_workspace_bytes(layer, proj, B), dtype=torch.uint8, device="cuda")
    gdn.layer_decode_raw(layer, proj, B=B, x=_bf16(x), y=y, state_in=st, state_out=st,
                         conv_state_in=cs, conv_state_out=cs, workspace=ws)
    torch.cuda.synchronize()
    return y, st, cs


def test_layer_decode_batch_invariant_across_64_rows():
    """The decode layer's projections stay on one kernel family at every
    batch size: a sequence's y and states are the same bits at B = 1, 64, 65
    and 130."""
    sh = synth.FULL
    hidden = 2048
    p = synth.layer_params(sh, 631)
    w_in, w_out = synth.proj_weights(sh, hidden, 631)
    Bmax = 130
    x = synth.hidden_inputs(Bmax, hidden, 632)
    S0 = synth.initial_states(sh, Bmax, 633)
    C0 = synth.conv_states(sh, Bmax, 634)
    ref_y, ref_st, ref_cs = _layer_decode(sh, hidden, p, w_in, w_out, x, S0, C0)
    for B in (1, 64, 65):
        y, st, cs = _layer_decode(sh, hidden, p, w_in, w_out, x[:B], S0[:B], C0[:B])
        assert torch.equal(y, ref_y[:B]), B
        assert torch.equal(st, ref_st[:B]) and torch.equal(cs, ref_cs[:B]), B


def test_layer_decode_graph_replays_match_eager():
    """gdn_layer_decode (in_proj, the decode step, out_proj; the projections
    through hipBLASLt with no workspace) captured in a HIP graph after eager
    calls have chosen the GEMM algorithms: every replay, with eager work
    between replays, gives the bits of the same eager step."""
    sh = synth.FULL
    hidden, B, reps = 2048, 5, 4
    p = synth.layer_params(sh, 640)
    w_in, w_out = synth.proj_weights(sh, hidden, 640)
    layer = make_layer(sh, p)
    proj = gdn.Proj(hidden=hidden, w_in=_bf16(w_in), w_out=_bf16(w_out))
    xs = [_bf16(synth.hidden_inputs(B, hidden, 641 + r)) for r in range(reps)]
    x = torch.empty_like(xs[0])
    S0 = to_dev(synth.initial_states(sh, B, 650))
    C0 = _bf16(synth.conv_states(sh, B, 651))
    y = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    st, cs = S0.clone(), C0.clone()
    ws = torch.zeros(gdn.layer_decode_workspace_bytes(layer, proj, B), dtype=torch.uint8, device="cuda")

    def step():
        gdn.layer_decode_raw(layer, proj, B=B, x=x, y=y, state_in=st, state_out=st,
                             conv_state_in=cs, conv_state_out=cs, workspace=ws)

    ref = []
    for r in range(reps):
        x.copy_(xs[r])
        step()
        torch.cuda.synchronize()
        ref.append((y.clone(), st.clone(), cs.clone()))
    st.copy_(S0)
    cs.copy_(C0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    st.copy_(S0)
    cs.copy_(C0)
    torch.cuda.synchronize()
    for r in range(reps):
        x.copy_(xs[r])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, ref[r][0]), r
        assert torch.equal(st, ref[r][1]) and torch.equal(cs, ref[r][2]), r
        del junk


def test_layer_prefill_graph_replays_match_eager():
    """gdn_layer_prefill (in_proj, the three prefill kernels, out_proj)
    captured in a HIP graph after an eager call: every replay, with eager work
    between replays and new inputs copied in before each, gives the eager
    call's bits."""
    sh = synth.FULL
    hidden, lens, reps = 2048, [300, 0, 77], 3
    p = synth.layer_params(sh, 660)
    w_in, w_out = synth.proj_weights(sh, hidden, 660)
    layer = make_layer(sh, p)
    proj = gdn.Proj(hidden=hidden, w_in=_bf16(w_in), w_out=_bf16(w_out))
    cu_np = synth.cu_from_lengths(lens)
    T, N = int(cu_np[-1]), len(lens)
    cu = to_dev(cu_np)
    xs = [_bf16(synth.hidden_inputs(T, hidden, 661 + r)) for r in range(reps)]
    x = torch.empty_like(xs[0])
    S0 = to_dev(synth.initial_states(sh, N, 670))
    y = torch.empty((T, hidden), dtype=torch.float32, device="cuda")
    fs = torch.empty((N, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device="cuda")
    cs = torch.empty((N, sh.K - 1, sh.Cc), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.layer_prefill_workspace_bytes(layer, proj, N, T), dtype=torch.uint8, device="cuda")

    def step():
        gdn.layer_prefill_raw(layer, proj, N=N, T_total=T, cu_seqlens=cu, x=x, y=y, initial_state=S0,
                              final_state=fs, conv_state_out=cs, workspace=ws)

    ref = []
    for r in range(reps):
        x.copy_(xs[r])
        step()
        torch.cuda.synchronize()
        ref.append((y.clone(), fs.clone(), cs.clone()))
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for r in range(reps):
        x.copy_(xs[r])
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, ref[r][0]), r
        assert torch.equal(fs, ref[r][1]) and torch.equal(cs, ref[r][2]), r
        del junk


def test_layer_prefill_short_sequence_alone_vs_packed():
    """The prefill layer's projections keep one kernel family at every token
    count: a 40-token sequence gives the same bits alone (40 rows) and packed
    behind a 300-token one."""
    sh = synth.FULL
    hidden = 2048
    p = synth.layer_params(sh, 641)
    w_in, w_out = synth.proj_weights(sh, hidden, 641)
    x = synth.hidden_inputs(340, hidden, 642)
    S0 = synth.initial_states(sh, 2, 643)
    C0 = synth.conv_states(sh, 2, 644)
    y2, fs2, cs2 = _run_layer(sh, hidden, p, w_in, w_out, synth.cu_from_lengths([300, 40]), x, S0, C0)
    y1, fs1, cs1 = _run_layer(sh, hidden, p, w_in, w_out, synth.cu_from_lengths([40]), x[300:],
                              S0[1:], C0[1:])
    assert np.array_equal(y1, y2[300:])
    assert np.array_equal(fs1[0], fs2[1]) and np.array_equal(cs1[0], cs2[1])
