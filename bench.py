#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer hot path on one MI355X.

Headline (``value``): prefill tokens/s of one layer at the 35B-A3B shape
(1 sequence x 4096 tokens, 16 key / 32 value heads, dk = dv = 128, chunk
64, bf16 activations, fp32 state from zero), one ``gdn_prefill`` call per
step with inputs resident in HBM.  The same JSON line carries

* ``roofline``      the dominant prefill kernel against its peak, with its
                    duration from HIP events recorded between the kernels
                    inside the timed region (``gdn_prefill_timed``);
* ``decode``        one decode step (one token per sequence) through 30
                    stacked layers at B = 64 (plus B = 1 and 3): state GB/s
                    against the 8 TB/s HBM peak, states carried in place;
* ``long_prefill``  1 x 131072 tokens resuming from a N(0, 0.02) state;
* ``varlen_prefill`` 8 packed sequences with log-uniform lengths;
* ``cpu_baseline``  the fp64 oracle on the host cores over the same 4096
                    token workload (a reported baseline, not a target).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--decode-batches", default="64,3,1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer-with-projections line")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (3 times): "
                         "the reference for scaling HBM byte counters")
    return ap.parse_args()


# ---- algorithmic work per token / per sequence ---------------------------------

def prefill_flops_per_token(Hk, Hv, dk, dv, C):
    """Matrix products of the chunked form, counted once (triangles at
    half): per value head, the scan's W H, Q H, K_d^T U (2 dk dv each) and
    P U ((C+1) dv); the prep's Grams per key head ((C-1) dk + (C+1) dk),
    the triangular solve (C^2/3), W and U~ ((C+1)(dk + dv))."""
    scan = Hv * (3 * 2 * dk * dv + (C + 1) * dv)
    prep = Hk * ((C - 1) * dk + (C + 1) * dk) + Hv * (C * C / 3 + (C + 1) * (dk + dv))
    return scan, prep


def decode_bytes_per_seq(Hk, Hv, dk, dv, act_bytes=2, out_bytes=4):
    Cc = 2 * Hk * dk + Hv * dv
    state = 2 * Hv * dk * dv * 4
    conv = 2 * 3 * Cc * act_bytes
    tok = (2 * Hk * dk + 2 * Hv * dv + 2 * Hv) * act_bytes
    out = Hv * dv * out_bytes
    return state + conv + tok + out, state


def measured_traffic(key):
    """HBM bytes per dispatch recorded in profiles/hbm_traffic.json for this
    kernel, or None once the kernel sources differ from the ones measured."""
    import glob
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_deltanet_linear_03_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    if h.hexdigest() != data.get("source_sha256"):
        return None
    k = data["kernels"].get(key)
    return None if k is None else k["read_bytes"] + k["write_bytes"]


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer's data-parallel hot path "
              "runs on a single MI355X (sequences shard across GPUs with no "
              "exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_deltanet_linear_03_amd as gdn
    from gated_deltanet_linear_03_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.calib_copy_mb:
        nbytes = args.calib_copy_mb << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": nbytes, "copies": 3}), flush=True)
        return
    sh = synth.FULL

    def layer_from(params):
        t = {k: torch.from_numpy(v).to(dev) for k, v in params.items()}
        return gdn.Layer(Hk=sh.Hk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv, chunk=sh.chunk,
                         act_dtype=gdn.GDN_DTYPE_BF16, out_dtype=gdn.GDN_DTYPE_FP32,
                         scale=sh.scale, eps_l2=sh.eps_l2, eps_rms=sh.eps_rms, **t)

    def bf16_dev(a):
        return torch.from_numpy(a).to(dev).to(torch.bfloat16)

    def gpu_inputs(T, gen):
        """Seeded device-side draws with the workload's distributions."""
        def n(*s):
            return torch.randn(*s, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        return {"q": n(T, sh.Hk, sh.dk), "k": n(T, sh.Hk, sh.dk), "v": n(T, sh.Hv, sh.dv),
                "z": n(T, sh.Hv, sh.dv), "a": n(T, sh.Hv), "b": n(T, sh.Hv)}

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)       # creates the underlying HIP event
        return evs

    # ---------------- prefill, 1 x 4096 (headline) ----------------
    case = synth.prefill_4k_case(1)
    T = case.T
    layer = layer_from(case.params)
    x = {k: bf16_dev(v) for k, v in case.inputs.items()}
    cu = torch.from_numpy(case.cu_seqlens).to(dev)
    out = torch.empty((T, sh.Hv, sh.dv), dtype=torch.float32, device=dev)
    fs = torch.empty((1, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
    cs = torch.empty((1, 3, sh.Cc), dtype=torch.bfloat16, device=dev)
    nb = gdn.prefill_workspace_bytes(layer, 1, T)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)

    def prefill_step(lay, xx, cuu, NN, TT, oo, ff, cc, S0=None, events=None):
        gdn.prefill_raw(lay, N=NN, T_total=TT, cu_seqlens=cuu, q=xx["q"], k=xx["k"],
                        v=xx["v"], z=xx["z"], a=xx["a"], b=xx["b"], out=oo,
                        initial_state=S0, final_state=ff, conv_state_out=cc,
                        workspace=ws, events=events)

    K, W = args.steps, args.warmup
    names = gdn.prefill_launches(layer, 1, T, nb)

    def kernel_ms(evl, reps):
        """Per-step time of each kernel kind (summed over its launches), and
        the launch count of each kind per step."""
        tot, cnt = {}, {}
        for j, name in enumerate(names):
            tot[name] = tot.get(name, 0.0) + sum(evl[i][j].elapsed_time(evl[i][j + 1])
                                                 for i in range(reps)) / reps
            cnt[name] = cnt.get(name, 0) + 1
        return tot, cnt

    # Rotate over NSET independent input sets (~100 MB each), so the 256 MiB
    # Infinity Cache does not hold a step's inputs from an earlier step; set
    # 0 is the seeded host-side case, the others device-side draws.
    NSET = 5
    gen_in = torch.Generator(device=dev)
    gen_in.manual_seed(11)
    sets = [x] + [gpu_inputs(T, gen_in) for _ in range(NSET - 1)]
    for i in range(W):
        prefill_step(layer, sets[i % NSET], cu, 1, T, out, fs, cs)
    torch.cuda.synchronize()
    # timed region: K plain steps between two events (an event recorded
    # between launches costs several microseconds of its own, so the
    # per-kernel times come from a second, instrumented pass below)
    e0, e1 = new_events(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        prefill_step(layer, sets[i % NSET], cu, 1, T, out, fs, cs)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / K
    tok_s = T / (ms_step * 1e-3)
    # instrumented pass: the same K steps with an event before every launch
    evs = [new_events(len(names) + 1) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        prefill_step(layer, sets[i % NSET], cu, 1, T, out, fs, cs, events=evs[i])
    torch.cuda.synchronize()
    steps_ms = sorted(evs[i][0].elapsed_time(evs[i][-1]) for i in range(K))
    pct = lambda q: steps_ms[min(K - 1, int(round(q * (K - 1))))]
    kern_ms, kern_n = kernel_ms(evs, K)
    log(f"prefill 4k: {ms_step:.3f} ms/step ({wall / K * 1e3:.3f} wall) {tok_s:.4g} tok/s; with an event "
        f"between launches: median {pct(0.5):.3f}, p10 {pct(0.1):.3f}, p90 {pct(0.9):.3f} ms, "
        f"kernels {kern_ms} launches {kern_n}")
    # the same with one input set: Infinity-Cache-warm inputs (context only)
    w0, w1 = new_events(2)
    torch.cuda.synchronize()
    w0.record(stream)
    for i in range(K):
        prefill_step(layer, x, cu, 1, T, out, fs, cs)
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / K
    log(f"prefill 4k, one input set (cache-warm): {warm_ms:.3f} ms/step")
    del sets

    scan_f, prep_f = prefill_flops_per_token(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.chunk)
    epi_bytes = sh.Hv * sh.dv * (4 + 2 + 4)
    path_bytes = (T * ((2 * sh.Hk * sh.dk + 2 * sh.Hv * sh.dv + 2 * sh.Hv) * 2 + sh.Hv * sh.dv * 4)
                  + sh.Hv * sh.dk * sh.dv * 4)
    rl = {}
    for name, ms in kern_ms.items():
        if name == "scan":
            a = scan_f * T / (ms * 1e-3) / 1e12
            rl[name] = {"bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        elif name == "prep":
            a = prep_f * T / (ms * 1e-3) / 1e12
            rl[name] = {"bound": "mfma", "achieved": a, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        elif name == "epi":
            a = epi_bytes * T / (ms * 1e-3) / 1e9
            rl[name] = {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    dominant = max(("prep", "scan", "epi"), key=lambda n: kern_ms[n])
    roof = dict(rl[dominant])
    roof["kernel"] = dominant
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(f"prefill_4k/{dominant}")
    roof["avg_ms"] = kern_ms[dominant] / kern_n[dominant]      # per launch
    roof["launches_per_step"] = kern_n[dominant]
    del out, fs, cs, x
    torch.cuda.empty_cache()

    result = {
        "metric": "GDN prefill tokens/s (MFMA % peak) + decode state GB/s (% HBM peak), 1 GPU",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gdn_prefill 1x4096 tokens, Hk=16 Hv=32 dk=dv=128, chunk 64, "
                               "bf16 inputs, fp32 state from zero, fp32 out",
                   "N": 1, "T": T, "Hk": sh.Hk, "Hv": sh.Hv, "dk": sh.dk, "dv": sh.dv,
                   "chunk": sh.chunk, "parallelism": "single GPU"},
        "roofline": roof,
        "prefill_kernels_ms": kern_ms,
        "prefill_kernel_launches": kern_n,
        "instrumented_ms_per_step_median_p10_p90": [pct(0.5), pct(0.1), pct(0.9)],
        "input_sets": NSET,
        "ms_per_step_one_input_set": warm_ms,
        "prefill_kernel_roofline": {k: dict(v, frac=v["achieved"] / v["peak"]) for k, v in rl.items()},
        "prefill_alg_tflops": (scan_f + prep_f) * T / (ms_step * 1e-3) / 1e12,
        # the whole path against HBM: compulsory bytes (q, k, v, z, a, b in,
        # out, the final state) over the step time
        "prefill_path_roofline": {
            "bound": "hbm", "bytes_per_step": path_bytes,
            "achieved": path_bytes / (ms_step * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": path_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }

    # ---------------- context: measured device-copy bandwidth ----------------
    cp_src = torch.empty(1 << 29, dtype=torch.float32, device=dev)     # 2 GiB
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    c0, c1 = new_events(2)
    c0.record(stream)
    for _ in range(5):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * cp_src.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    result["hbm_copy_GBps"] = copy_gbs      # read + write bytes of a 2 GiB device copy
    log(f"device copy: {copy_gbs:.1f} GB/s (read + write)")
    del cp_src, cp_dst
    torch.cuda.empty_cache()

    # ---------------- decode, 30 layers x B ----------------
    if not args.no_decode:
        L = args.layers
        # multi-token verify below: VB sequences x VT draft tokens, on the
        # same state pool, which therefore holds at least VB sequences
        VB, VT = 8, 4
        Bmax = max([int(b) for b in args.decode_batches.split(",")] + [VB])
        gen = torch.Generator(device=dev)
        layers, states, convs, toks = [], [], [], []
        Tpre = 2048
        for l in range(L):
            lay = layer_from(synth.layer_params(sh, 100 + l))
            gen.manual_seed(1000 + l)
            xp = gpu_inputs(Bmax * Tpre, gen)
            cup = torch.arange(0, Bmax * Tpre + 1, Tpre, dtype=torch.int32, device=dev)
            st = torch.empty((Bmax, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
            cv = torch.empty((Bmax, 3, sh.Cc), dtype=torch.bfloat16, device=dev)
            nbp = gdn.prefill_workspace_bytes(lay, Bmax, Bmax * Tpre)
            if ws.numel() < nbp:
                ws = torch.empty(nbp, dtype=torch.uint8, device=dev)
            outp = torch.empty((Bmax * Tpre, sh.Hv, sh.dv), dtype=torch.float32, device=dev)
            # the carried state is the one a 2048-token prefill leaves behind
            prefill_step(lay, xp, cup, Bmax, Bmax * Tpre, outp, st, cv)
            torch.cuda.synchronize()
            del xp, outp
            layers.append(lay)
            states.append(st)
            convs.append(cv)
            toks.append(gpu_inputs(Bmax, gen))
        log(f"decode setup: {L} layers x B={Bmax} states from a {Tpre}-token prefill")
        dec = {}
        per_seq, state_per_seq = decode_bytes_per_seq(sh.Hk, sh.Hv, sh.dk, sh.dv)
        for B in [int(b) for b in args.decode_batches.split(",")]:
            outs = [torch.empty((B, sh.Hv, sh.dv), dtype=torch.float32, device=dev) for _ in range(L)]

            def dstep(events=None):
                for l in range(L):
                    t = toks[l]
                    if events is not None:
                        events[l][0].record(stream)
                    gdn.decode_raw(layers[l], B=B, q=t["q"][:B], k=t["k"][:B], v=t["v"][:B],
                                   z=t["z"][:B], a=t["a"][:B], b=t["b"][:B], out=outs[l],
                                   state_in=states[l][:B], state_out=states[l][:B],
                                   conv_state_in=convs[l][:B], conv_state_out=convs[l][:B])
                    if events is not None:
                        events[l][1].record(stream)
            for _ in range(W):
                dstep()
            torch.cuda.synchronize()
            d0, d1 = new_events(2)
            torch.cuda.synchronize()
            d0.record(stream)
            for i in range(K):
                dstep()
            d1.record(stream)
            torch.cuda.synchronize()
            eager_ms = d0.elapsed_time(d1) / K
            # kernel times from a second pass with events around each launch
            devs = [[new_events(2) for _ in range(L)] for _ in range(K)]
            torch.cuda.synchronize()
            for i in range(K):
                dstep(devs[i])
            torch.cuda.synchronize()
            kms = sum(devs[i][l][0].elapsed_time(devs[i][l][1]) for i in range(K) for l in range(L)) / (K * L)
            kern_gbs = B * per_seq / (kms * 1e-3) / 1e9
            dec[f"B{B}"] = {"layers": L, "eager_ms_per_step": eager_ms,
                            "eager_state_GBps": L * B * state_per_seq / (eager_ms * 1e-3) / 1e9,
                            "kernel_avg_ms": kms,
                            "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": kern_gbs / PEAK_HBM_GBS,
                                         "traffic": measured_traffic("decode_b64/decode") if B == 64 else None,
                                         "bytes_per_launch": B * per_seq}}
            # the same 30-layer step replayed from a HIP graph (launch gaps
            # removed; the states keep advancing exactly as eager steps do)
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                dstep()                       # warm the capture stream
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=cap):
                    dstep()
            torch.cuda.current_stream().wait_stream(cap)
            torch.cuda.synchronize()
            g0, g1 = new_events(2)
            g0.record(stream)
            for i in range(K):
                g.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            gms = g0.elapsed_time(g1) / K
            # the step as a serving loop runs it, replayed from a graph: the
            # headline decode figures (the eager loop above also pays the
            # Python binding's per-call cost, which B = 64 no longer hides)
            state_gbs = L * B * state_per_seq / (gms * 1e-3) / 1e9
            dec[f"B{B}"].update({"ms_per_step": gms, "state_GBps": state_gbs,
                                 "all_bytes_GBps": L * B * per_seq / (gms * 1e-3) / 1e9,
                                 "state_frac_hbm": state_gbs / PEAK_HBM_GBS})
            del g
            log(f"decode B={B}: {gms:.3f} ms/step from a graph ({eager_ms:.3f} eager), state "
                f"{state_gbs:.1f} GB/s, kernel {kms * 1e3:.1f} us = {kern_gbs:.1f} GB/s")
        result["decode"] = dec

        # multi-token verify: VB sequences x VT draft tokens x the same layers
        vt = []
        for l in range(L):
            gen.manual_seed(2000 + l)
            vt.append(gpu_inputs(VB * VT, gen))
        vouts = [torch.empty((VB * VT, sh.Hv, sh.dv), dtype=torch.float32, device=dev) for _ in range(L)]

        def vstep(events=None):
            for l in range(L):
                t = vt[l]
                if events is not None:
                    events[l][0].record(stream)
                gdn.decode_multi_raw(layers[l], B=VB, tokens=VT, q=t["q"], k=t["k"], v=t["v"],
                                     z=t["z"], a=t["a"], b=t["b"], out=vouts[l],
                                     state_in=states[l][:VB], state_out=states[l][:VB],
                                     conv_state_in=convs[l][:VB], conv_state_out=convs[l][:VB])
                if events is not None:
                    events[l][1].record(stream)
        for _ in range(W):
            vstep()
        torch.cuda.synchronize()
        v0, v1 = new_events(2)
        v0.record(stream)
        for i in range(K):
            vstep()
        v1.record(stream)
        torch.cuda.synchronize()
        vms = v0.elapsed_time(v1) / K
        vevs = [[new_events(2) for _ in range(L)] for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            vstep(vevs[i])
        torch.cuda.synchronize()
        vkms = sum(vevs[i][l][0].elapsed_time(vevs[i][l][1]) for i in range(K) for l in range(L)) / (K * L)
        result["verify"] = {"B": VB, "tokens": VT, "layers": L, "ms_per_step": vms,
                            "tokens_per_s": VB * VT / (vms * 1e-3),
                            "kernel_avg_ms": vkms,
                            "state_GBps": L * VB * state_per_seq / (vms * 1e-3) / 1e9}
        log(f"verify B={VB} x {VT} tokens: {vms:.3f} ms/step, kernel {vkms * 1e3:.1f} us")
        del layers, states, convs, toks, vt, vouts
        torch.cuda.empty_cache()

    # ---------------- long prefill, 1 x 131072 from a random state ----------------
    def timed_prefill(name, lengths, seed, reps):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        TT = int(sum(lengths))
        NN = len(lengths)
        lay = layer_from(synth.layer_params(sh, seed))
        xx = gpu_inputs(TT, gen)
        cuu = torch.from_numpy(synth.cu_from_lengths(lengths)).to(dev)
        S0 = (torch.randn((NN, sh.Hv, sh.dk, sh.dv), generator=gen, device=dev) * math.sqrt(0.02))
        oo = torch.empty((TT, sh.Hv, sh.dv), dtype=torch.float32, device=dev)
        ff = torch.empty_like(S0)
        cc = torch.empty((NN, 3, sh.Cc), dtype=torch.bfloat16, device=dev)
        nonlocal_ws = gdn.prefill_workspace_bytes(lay, NN, TT)
        nonlocal ws
        if ws.numel() < nonlocal_ws:
            ws = torch.empty(nonlocal_ws, dtype=torch.uint8, device=dev)
        prefill_step(lay, xx, cuu, NN, TT, oo, ff, cc, S0=S0)
        torch.cuda.synchronize()
        lnames = gdn.prefill_launches(lay, NN, TT, ws.numel())
        a0, a1 = new_events(2)
        a0.record(stream)
        for i in range(reps):
            prefill_step(lay, xx, cuu, NN, TT, oo, ff, cc, S0=S0)
        a1.record(stream)
        torch.cuda.synchronize()
        ms = a0.elapsed_time(a1) / reps
        # kernel times from a second pass with an event before every launch
        ev = [new_events(len(lnames) + 1) for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            prefill_step(lay, xx, cuu, NN, TT, oo, ff, cc, S0=S0, events=ev[i])
        torch.cuda.synchronize()
        km = {}
        for j, n in enumerate(lnames):
            km[n] = km.get(n, 0.0) + sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(reps)) / reps
        alg = (scan_f + prep_f) * TT / (ms * 1e-3) / 1e12
        r = {"N": NN, "T": TT, "ms": ms, "tokens_per_s": TT / (ms * 1e-3), "kernels_ms": km,
             "alg_tflops": alg, "alg_mfma_frac": alg / PEAK_BF16_TFLOPS,
             "scan_tflops": scan_f * TT / (km["scan"] * 1e-3) / 1e12}
        log(f"{name}: {ms:.3f} ms, {r['tokens_per_s']:.4g} tok/s, kernels {km}")
        del xx, oo, ff, cc, S0
        torch.cuda.empty_cache()
        return r

    if not args.no_long:
        result["long_prefill"] = timed_prefill("long prefill 1x131072", [131072], 3, 3)
    if not args.no_varlen:
        lens = [int(v) for v in synth.varlen_lengths(8, 4)]
        r = timed_prefill("varlen prefill 8 seqs", lens, 4, 3)
        r["lengths"] = lens
        result["varlen_prefill"] = r

    # ---------------- the layer with its projections, 1 x 4096 ----------------
    if not args.no_layer:
        H = synth.HIDDEN
        gen = torch.Generator(device=dev)
        gen.manual_seed(21)
        P = synth.proj_rows(sh)
        HD = sh.Hv * sh.dv
        lay = layer_from(case.params)
        w_in = (torch.randn((P, H), generator=gen, device=dev) / math.sqrt(H)).to(torch.bfloat16)
        w_out = (torch.randn((H, HD), generator=gen, device=dev) / math.sqrt(HD)).to(torch.bfloat16)
        proj = gdn.Proj(hidden=H, w_in=w_in, w_out=w_out)
        xs = [torch.randn((T, H), generator=gen, device=dev).to(torch.bfloat16) for _ in range(3)]
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        lws = torch.empty(gdn.layer_prefill_workspace_bytes(lay, proj, 1, T), dtype=torch.uint8,
                          device=dev)
        lfs = torch.empty((1, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
        lcs = torch.empty((1, 3, sh.Cc), dtype=torch.bfloat16, device=dev)

        def layer_step(xx):
            gdn.layer_prefill_raw(lay, proj, N=1, T_total=T, cu_seqlens=cu, x=xx, y=y,
                                  final_state=lfs, conv_state_out=lcs, workspace=lws)

        for i in range(W):
            layer_step(xs[i % 3])
        l0, l1 = new_events(2)
        l0.record(stream)
        for i in range(K):
            layer_step(xs[i % 3])
        l1.record(stream)
        torch.cuda.synchronize()
        lms = l0.elapsed_time(l1) / K
        # the two GEMMs alone, same shapes and buffers
        pbuf = torch.empty((T, P), dtype=torch.bfloat16, device=dev)
        gbuf = torch.empty((T, HD), dtype=torch.bfloat16, device=dev)

        def gemm_ms(A, B, C):
            for _ in range(2):
                gdn.gemm_bf16(A, B, C)
            g0, g1 = new_events(2)
            g0.record(stream)
            for _ in range(K):
                gdn.gemm_bf16(A, B, C)
            g1.record(stream)
            torch.cuda.synchronize()
            return g0.elapsed_time(g1) / K

        in_ms = gemm_ms(xs[0], w_in, pbuf)
        out_ms = gemm_ms(gbuf, w_out, y)
        in_tf = 2 * T * P * H / (in_ms * 1e-3) / 1e12
        out_tf = 2 * T * HD * H / (out_ms * 1e-3) / 1e12
        result["layer_with_projections"] = {
            "hidden": H, "T": T, "ms_per_step": lms, "tokens_per_s": T / (lms * 1e-3),
            "in_proj_ms": in_ms, "out_proj_ms": out_ms,
            "in_proj": {"bound": "mfma", "achieved": in_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": in_tf / PEAK_BF16_TFLOPS, "shape": [T, P, H]},
            "out_proj": {"bound": "mfma", "achieved": out_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": out_tf / PEAK_BF16_TFLOPS, "shape": [T, H, HD]}}
        log(f"layer with projections (hidden {H}) 1x{T}: {lms:.3f} ms/step "
            f"({T / (lms * 1e-3):.4g} tok/s); in_proj {in_ms * 1e3:.1f} us = {in_tf:.0f} TFLOP/s, "
            f"out_proj {out_ms * 1e3:.1f} us = {out_tf:.0f} TFLOP/s")
        del xs, y, lws, lfs, lcs, pbuf, gbuf, w_in, w_out
        torch.cuda.empty_cache()

        # decode with projections: 8 layers' weights (~540 MB, more than the
        # Infinity Cache holds) rotated, one token per sequence
        NL = 8
        projs = [gdn.Proj(hidden=H,
                          w_in=(torch.randn((P, H), generator=gen, device=dev) / math.sqrt(H)).to(torch.bfloat16),
                          w_out=(torch.randn((H, HD), generator=gen, device=dev) / math.sqrt(HD)).to(torch.bfloat16))
                 for _ in range(NL)]
        dec = {}
        for Bd in (1, 64):
            xd = torch.randn((Bd, H), generator=gen, device=dev).to(torch.bfloat16)
            yd = torch.empty((Bd, H), dtype=torch.bfloat16, device=dev)
            sd = [torch.randn((Bd, sh.Hv, sh.dk, sh.dv), generator=gen, device=dev) * 0.1 for _ in range(NL)]
            cd = [torch.zeros((Bd, 3, sh.Cc), dtype=torch.bfloat16, device=dev) for _ in range(NL)]
            dws = torch.empty(gdn.layer_decode_workspace_bytes(lay, projs[0], Bd), dtype=torch.uint8, device=dev)

            def dstep(l):
                gdn.layer_decode_raw(lay, projs[l], B=Bd, x=xd, y=yd, state_in=sd[l], state_out=sd[l],
                                     conv_state_in=cd[l], conv_state_out=cd[l], workspace=dws)

            for l in range(NL):
                dstep(l)
            d0, d1 = new_events(2)
            d0.record(stream)
            R = 3
            for _ in range(R):
                for l in range(NL):
                    dstep(l)
            d1.record(stream)
            torch.cuda.synchronize()
            ms_l = d0.elapsed_time(d1) / (R * NL)
            wbytes = 2 * (P * H + H * HD)
            sbytes = Bd * 2 * sh.Hv * sh.dk * sh.dv * 4
            dec[f"B{Bd}"] = {"ms_per_layer": ms_l, "weight_and_state_GBps": (wbytes + sbytes) / (ms_l * 1e-3) / 1e9}
            log(f"layer decode with projections B={Bd}: {ms_l * 1e3:.1f} us per layer, weights + state "
                f"{(wbytes + sbytes) / (ms_l * 1e-3) / 1e9:.0f} GB/s")
            del xd, yd, sd, cd, dws
        result["layer_with_projections"]["decode"] = dec
        del projs
        torch.cuda.empty_cache()

    # ---------------- CPU baseline: the fp64 oracle on the host ----------------
    if not args.no_cpu_baseline:
        import oracle
        cores = min(os.cpu_count() or 1, 16)
        d = oracle.Dims(sh.Hk, sh.Hv, sh.dk, sh.dv, 4, sh.scale, sh.eps_l2, sh.eps_rms)
        reps, t_cpu = 0, 0.0
        while t_cpu < 10.0 and reps < 200:
            tc = time.perf_counter()
            oracle.gdn_forward(d, case.cu_seqlens, *(case.inputs[n] for n in "qkvzab"),
                               case.params["conv_w"], case.params["A_log"],
                               case.params["dt_bias"], case.params["norm_w"], nthreads=cores)
            t_cpu += time.perf_counter() - tc
            reps += 1
        result["cpu_baseline"] = {"value": T * reps / t_cpu, "unit": "tokens/s", "cores": cores,
                                  "kind": "oracle",
                                  "sample": f"the whole 1x{T}-token workload, all 32 heads, "
                                            f"fp64 token-by-token, {reps} runs ({t_cpu:.1f} s)"}
        log(f"cpu baseline: {result['cpu_baseline']['value']:.1f} tok/s on {cores} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
