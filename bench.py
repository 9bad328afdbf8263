#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer hot path on one MI355X.

Headline (``value``): prefill tokens/s of one layer at the 35B-A3B shape on
the long-context workload -- 1 sequence x 131072 tokens in 64-token chunks,
16 key / 32 value heads, dk = dv = 128, bf16 activations, resuming from a
N(0, 0.02) fp32 state, fp32 out -- one ``gdn_prefill`` call per step with
inputs resident in HBM.  The same JSON line carries

* ``roofline``        the step's dominant kernel against its binding ceiling
                      (the larger of its matrix-core time for its
                      algorithmic flops and its HBM time for its compulsory
                      bytes), its duration from HIP events recorded between
                      the kernels inside the timed region
                      (``gdn_prefill_timed``, on the kernels' own stream);
* ``prefill_4k``      1 x 4096 tokens from a zero state (inputs rotated over
                      five sets, so the Infinity Cache does not hold them);
* ``varlen_prefill``  8 packed sequences with log-uniform lengths;
* ``decode``          one decode step (one token per sequence) through 30
                      stacked layers at B = 64 (plus B = 1 and 3): state GB/s
                      against the 8 TB/s HBM peak, states carried in place;
* ``cpu_baseline``    the fp64 oracle on the host's cores over a bounded
                      sample of the headline workload (a reported baseline,
                      not a target), plus a single-thread figure.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only]
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
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix-core peak, TFLOP/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed steps of the headline")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--headline-only", action="store_true",
                    help="only the 131072-token headline (for profiling)")
    ap.add_argument("--only", choices=["4k", "varlen", "decode", "layer"], default=None,
                    help="only this extra workload, no headline and no JSON line (for profiling)")
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--decode-batches", default="64,3,1")
    ap.add_argument("--decode-compare", action="store_true",
                    help="also time decode without a workspace (the one-work-group kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="about this much oracle work for the all-threads CPU baseline")
    ap.add_argument("--no-4k", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer-with-projections lines")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (3 times): "
                         "the reference for scaling HBM byte counters")
    return ap.parse_args(argv)


# ---- algorithmic work per token / per sequence ---------------------------------

def prefill_flops_per_token(Hk, Hv, dk, dv, C):
    """Matrix products of the chunked form, counted once (triangles at
    half): per value head, the scan's W H, Q H, K_d^T U (2 dk dv each) and
    P U ((C+1) dv); the prep's Grams per key head ((C-1) dk + (C+1) dk),
    the triangular solve (C^2/3), W and U~ ((C+1)(dk + dv))."""
    scan = Hv * (3 * 2 * dk * dv + (C + 1) * dv)
    prep = Hk * ((C - 1) * dk + (C + 1) * dk) + Hv * (C * C / 3 + (C + 1) * (dk + dv))
    return scan, prep


def prefill_bytes_per_token(Hk, Hv, dk, dv, act_bytes=2, out_bytes=4):
    """Compulsory HBM bytes per token: what prep must read (q, k, v, a, b),
    what the epilogue must read and write (z in, out out), and the whole
    path (every input read once, out written once); the states (read and
    written once per sequence) come on top."""
    prep = (2 * Hk * dk + Hv * dv + 2 * Hv) * act_bytes
    epi = Hv * dv * (act_bytes + out_bytes)
    return {"prep": prep, "scan": 0, "epi": epi, "path": prep + epi}


def decode_bytes_per_seq(Hk, Hv, dk, dv, act_bytes=2, out_bytes=4):
    Cc = 2 * Hk * dk + Hv * dv
    state = 2 * Hv * dk * dv * 4
    conv = 2 * 3 * Cc * act_bytes
    tok = (2 * Hk * dk + 2 * Hv * dv + 2 * Hv) * act_bytes
    out = Hv * dv * out_bytes
    return state + conv + tok + out, state


def binding_roofline(flops, nbytes, seconds):
    """A kernel's work against its binding ceiling: the larger of the
    matrix-core time for `flops` at the bf16 peak and the HBM time for
    `nbytes` at the HBM peak.  Returns the roofline block (achieved in the
    binding unit; frac = ceiling time / measured time)."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_hbm >= t_mfma:
        r = {"bound": "hbm", "achieved": nbytes / seconds / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": flops / seconds / 1e12, "peak": PEAK_BF16_TFLOPS,
             "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["ceiling_ms"] = max(t_mfma, t_hbm) * 1e3
    r["mfma_ms_at_peak"] = t_mfma * 1e3
    r["hbm_ms_at_peak"] = t_hbm * 1e3
    return r


def sources_sha():
    """Hash of the kernel sources, recorded with the counter profiles."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "gated_deltanet_linear_03_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _profile_entry(fname, key):
    """Entry `key` of profiles/<fname> while the kernel sources still hash to
    the value recorded with it, else None."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    if data.get("source_sha256") != sources_sha():
        return None
    return data["kernels"].get(key)


def measured_traffic(key):
    """HBM bytes per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/hbm_traffic.json), or None once the sources changed."""
    k = _profile_entry("hbm_traffic.json", key)
    return None if k is None else k["read_bytes"] + k["write_bytes"]


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer's data-parallel hot path "
              "runs on a single MI355X (sequences shard across GPUs with no "
              "exchange); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

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
    K, W = args.steps, args.warmup
    scan_f, prep_f = prefill_flops_per_token(sh.Hk, sh.Hv, sh.dk, sh.dv, sh.chunk)
    bpt = prefill_bytes_per_token(sh.Hk, sh.Hv, sh.dk, sh.dv)
    state_bytes = sh.Hv * sh.dk * sh.dv * 4

    def layer_from(params):
        t = {k: torch.from_numpy(v).to(dev) for k, v in params.items()}
        return gdn.Layer(Hk=sh.Hk, Hv=sh.Hv, dk=sh.dk, dv=sh.dv, chunk=sh.chunk,
                         act_dtype=gdn.GDN_DTYPE_BF16, out_dtype=gdn.GDN_DTYPE_FP32,
                         scale=sh.scale, eps_l2=sh.eps_l2, eps_rms=sh.eps_rms, **t)

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

    ws_holder = {"ws": torch.empty(0, dtype=torch.uint8, device=dev)}

    def workspace(nbytes):
        if ws_holder["ws"].numel() < nbytes:
            ws_holder["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return ws_holder["ws"]

    def time_prefill(lay, sets, lengths, S0, reps, warm):
        """reps plain steps between two events (the headline figure), then
        reps instrumented steps with an event before every launch (kernel
        times and per-step spread); input sets rotate per step."""
        NN, TT = len(lengths), int(sum(lengths))
        cu = torch.from_numpy(synth.cu_from_lengths(lengths)).to(dev)
        out = torch.empty((TT, sh.Hv, sh.dv), dtype=torch.float32, device=dev)
        fs = torch.empty((NN, sh.Hv, sh.dk, sh.dv), dtype=torch.float32, device=dev)
        cs = torch.empty((NN, 3, sh.Cc), dtype=torch.bfloat16, device=dev)
        ws = workspace(gdn.prefill_workspace_bytes(lay, NN, TT))
        names = gdn.prefill_launches(lay, NN, TT, ws.numel())

        def step(x, events=None):
            gdn.prefill_raw(lay, N=NN, T_total=TT, cu_seqlens=cu, q=x["q"], k=x["k"], v=x["v"],
                            z=x["z"], a=x["a"], b=x["b"], out=out, initial_state=S0,
                            final_state=fs, conv_state_out=cs, workspace=ws, events=events)

        for i in range(warm):
            step(sets[i % len(sets)])
        torch.cuda.synchronize()
        e0, e1 = new_events(2)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(reps):
            step(sets[i % len(sets)])
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = e0.elapsed_time(e1) / reps
        evs = [new_events(len(names) + 1) for _ in range(reps)]
        torch.cuda.synchronize()
        for i in range(reps):
            step(sets[i % len(sets)], events=evs[i])
        torch.cuda.synchronize()
        steps_ms = sorted(evs[i][0].elapsed_time(evs[i][-1]) for i in range(reps))
        pct = lambda q: steps_ms[min(reps - 1, int(round(q * (reps - 1))))]
        kern, cnt = {}, {}
        for j, name in enumerate(names):
            kern[name] = kern.get(name, 0.0) + sum(evs[i][j].elapsed_time(evs[i][j + 1])
                                                   for i in range(reps)) / reps
            cnt[name] = cnt.get(name, 0) + 1
        del out, fs, cs
        return {"N": NN, "T": TT, "ms": ms, "wall_ms": wall / reps * 1e3,
                "tokens_per_s": TT / (ms * 1e-3), "kernels_ms": kern, "kernel_launches": cnt,
                "instrumented_ms_median_p10_p90": [pct(0.5), pct(0.1), pct(0.9)]}

    def kernel_rooflines(r, traffic_prefix=None):
        """Each prefill kernel of a timed prefill against its binding
        ceiling, per step (the same ratio as per launch)."""
        T = r["T"]
        work = {"prep": (prep_f * T, bpt["prep"] * T),
                "scan": (scan_f * T, 2 * r["N"] * state_bytes),
                "epi": (0.0, bpt["epi"] * T)}
        out = {}
        for name, ms in r["kernels_ms"].items():
            fl, by = work[name]
            rl = binding_roofline(fl, by, ms * 1e-3)
            n = r["kernel_launches"][name]
            rl.update({"kernel": name, "avg_ms": ms / n, "launches_per_step": n,
                       "alg_flops_per_launch": fl / n, "alg_bytes_per_launch": by / n,
                       "traffic": (measured_traffic(f"{traffic_prefix}/{name}")
                                   if traffic_prefix else None)})
            out[name] = rl
        return out

    def mfma_block(head, alg_tflops):
        """Algorithmic matrix-core flops of the step over the bf16 peak, and
        the executed ones (split-precision products count three times) from
        the MFMA counters in profiles/mfma_util.json while the sources match:
        executed flops per launch x launches per step over the step time."""
        b = {"alg_tflops": alg_tflops, "peak": PEAK_BF16_TFLOPS, "alg_frac": alg_tflops / PEAK_BF16_TFLOPS,
             "alg_flops_per_token": scan_f + prep_f}
        ex = [_profile_entry("mfma_util.json", f"prefill_long/{k}") for k in ("prep", "scan")]
        if all(e is not None for e in ex):
            fl = sum(e["exec_flops"] * head["kernel_launches"][k] for e, k in zip(ex, ("prep", "scan")))
            t = fl / (head["ms"] * 1e-3) / 1e12
            b.update({"executed_tflops": t, "executed_frac": t / PEAK_BF16_TFLOPS,
                      "mfma_busy_prep": ex[0]["mfma_busy"], "mfma_busy_scan": ex[1]["mfma_busy"]})
        return b

    # ---------------- headline: prefill 1 x 131072 from a random state ----------------
    def headline(T_long):
        gen = torch.Generator(device=dev)
        gen.manual_seed(3)
        lay_long = layer_from(synth.layer_params(sh, 3))
        x_long = gpu_inputs(T_long, gen)
        S0_long = torch.randn((1, sh.Hv, sh.dk, sh.dv), generator=gen, device=dev) * math.sqrt(0.02)
        torch.cuda.synchronize()
        head = time_prefill(lay_long, [x_long], [T_long], S0_long, K, W)
        rls = kernel_rooflines(head, "prefill_long")
        dominant = max(head["kernels_ms"], key=lambda n: head["kernels_ms"][n])
        ms_step = head["ms"]
        tok_s = head["tokens_per_s"]
        path_bytes = bpt["path"] * T_long + 2 * state_bytes
        alg_tflops = (scan_f + prep_f) * T_long / (ms_step * 1e-3) / 1e12
        log(f"prefill 1x{T_long}: {ms_step:.3f} ms/step, {tok_s:.4g} tok/s, kernels {head['kernels_ms']} "
            f"launches {head['kernel_launches']}; dominant {dominant}: {rls[dominant]['frac']:.3f} of its "
            f"{rls[dominant]['bound']} ceiling")
        del x_long
        torch.cuda.empty_cache()
        return {
            "metric": "GDN prefill tokens/s (MFMA % peak) + decode state GB/s (% HBM peak), 1 GPU",
            "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "gdn_prefill 1x131072 tokens (64-token chunks) resuming from a "
                                   "N(0,0.02) fp32 state, zero conv state, Hk=16 Hv=32 dk=dv=128, "
                                   "bf16 inputs N(0,1), fp32 out",
                       "N": 1, "T": T_long, "Hk": sh.Hk, "Hv": sh.Hv, "dk": sh.dk, "dv": sh.dv,
                       "chunk": sh.chunk, "parallelism": "single GPU"},
            "roofline": rls[dominant],
            "prefill_kernel_roofline": rls,
            "prefill_kernels_ms": head["kernels_ms"],
            "prefill_kernel_launches": head["kernel_launches"],
            "instrumented_ms_per_step_median_p10_p90": head["instrumented_ms_median_p10_p90"],
            # the benchmark spec's figure: algorithmic matrix-core flops of the step
            # over the bf16 peak (executed-MFMA counters: profiles/)
            "mfma": mfma_block(head, alg_tflops),
            # the whole path against HBM: compulsory bytes (q, k, v, z, a, b
            # in, out, the state in and out) over the step time
            "prefill_path_roofline": {
                "bound": "hbm", "bytes_per_step": path_bytes,
                "achieved": path_bytes / (ms_step * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": path_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "ceiling_ms": path_bytes / (PEAK_HBM_GBS * 1e9) * 1e3},
        }

    if args.only:
        # one extra workload alone, for a profiler run
        args.headline_only = False
        args.no_4k, args.no_varlen, args.no_decode = (args.only != "4k", args.only != "varlen",
                                                      args.only != "decode")
        args.no_layer = args.only != "layer"
        args.no_cpu_baseline = True
        result = {}
    else:
        result = headline(131072)

    if not args.headline_only and not args.only:
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

    # ---------------- prefill 1 x 4096 from zero, five rotated input sets ----------------
    if not args.headline_only and not args.no_4k:
        case = synth.prefill_4k_case(1)
        lay4 = layer_from(case.params)
        x4 = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in case.inputs.items()}
        g4 = torch.Generator(device=dev)
        g4.manual_seed(11)
        sets = [x4] + [gpu_inputs(case.T, g4) for _ in range(4)]
        r4 = time_prefill(lay4, sets, [case.T], None, 50, 20)
        r4["kernel_roofline"] = kernel_rooflines(r4, "prefill_4k")
        r4["input_sets"] = len(sets)
        warm = time_prefill(lay4, [x4], [case.T], None, 50, 5)
        r4["ms_one_input_set"] = warm["ms"]
        result["prefill_4k"] = r4
        log(f"prefill 1x4096: {r4['ms']:.3f} ms/step ({r4['tokens_per_s']:.4g} tok/s), one input set "
            f"{warm['ms']:.3f}; kernels {r4['kernels_ms']}")
        del sets, x4
        torch.cuda.empty_cache()

    # ---------------- varlen prefill, 8 sequences ----------------
    if not args.headline_only and not args.no_varlen:
        lens = [int(v) for v in synth.varlen_lengths(8, 4)]
        gv = torch.Generator(device=dev)
        gv.manual_seed(4)
        layv = layer_from(synth.layer_params(sh, 4))
        xv = gpu_inputs(sum(lens), gv)
        S0v = torch.randn((8, sh.Hv, sh.dk, sh.dv), generator=gv, device=dev) * math.sqrt(0.02)
        rv = time_prefill(layv, [xv], lens, S0v, 5, 2)
        rv["lengths"] = lens
        rv["kernel_roofline"] = kernel_rooflines(rv)
        result["varlen_prefill"] = rv
        log(f"varlen prefill {lens}: {rv['ms']:.3f} ms ({rv['tokens_per_s']:.4g} tok/s), kernels "
            f"{rv['kernels_ms']}")
        del xv, S0v
        torch.cuda.empty_cache()

    # ---------------- decode, 30 layers x B ----------------
    if not args.headline_only and not args.no_decode:
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
            ws = workspace(gdn.prefill_workspace_bytes(lay, Bmax, Bmax * Tpre))
            outp = torch.empty((Bmax * Tpre, sh.Hv, sh.dv), dtype=torch.float32, device=dev)
            # the carried state is the one a 2048-token prefill leaves behind
            gdn.prefill_raw(lay, N=Bmax, T_total=Bmax * Tpre, cu_seqlens=cup, q=xp["q"], k=xp["k"],
                            v=xp["v"], z=xp["z"], a=xp["a"], b=xp["b"], out=outp, final_state=st,
                            conv_state_out=cv, workspace=ws)
            torch.cuda.synchronize()
            del xp, outp
            layers.append(lay)
            states.append(st)
            convs.append(cv)
            toks.append(gpu_inputs(Bmax, gen))
        log(f"decode setup: {L} layers x B={Bmax} states from a {Tpre}-token prefill")
        dec = {}
        per_seq, state_per_seq = decode_bytes_per_seq(sh.Hk, sh.Hv, sh.dk, sh.dv)
        DK = 20
        dws = gdn.decode_workspace(layers[0], Bmax)     # zero-filled once, shared by the layers

        def decode_variant(B, ws):
            """Eager and graph-replayed 30-layer steps and the kernel time per
            layer, with the decode workspace `ws` (the library then picks the
            column-split kernel for small batches) or without (one
            work-group per sequence and key head)."""
            outs = [torch.empty((B, sh.Hv, sh.dv), dtype=torch.float32, device=dev) for _ in range(L)]

            def dstep(events=None):
                for l in range(L):
                    t = toks[l]
                    if events is not None:
                        events[l][0].record(stream)
                    gdn.decode_raw(layers[l], B=B, q=t["q"][:B], k=t["k"][:B], v=t["v"][:B],
                                   z=t["z"][:B], a=t["a"][:B], b=t["b"][:B], out=outs[l],
                                   state_in=states[l][:B], state_out=states[l][:B],
                                   conv_state_in=convs[l][:B], conv_state_out=convs[l][:B], workspace=ws)
                    if events is not None:
                        events[l][1].record(stream)
            for _ in range(5):
                dstep()
            torch.cuda.synchronize()
            d0, d1 = new_events(2)
            torch.cuda.synchronize()
            d0.record(stream)
            for i in range(DK):
                dstep()
            d1.record(stream)
            torch.cuda.synchronize()
            eager_ms = d0.elapsed_time(d1) / DK
            # kernel times from a second pass with events around each launch
            devs = [[new_events(2) for _ in range(L)] for _ in range(DK)]
            torch.cuda.synchronize()
            for i in range(DK):
                dstep(devs[i])
            torch.cuda.synchronize()
            kms = sum(devs[i][l][0].elapsed_time(devs[i][l][1]) for i in range(DK) for l in range(L)) / (DK * L)
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
            for i in range(DK):
                g.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            gms = g0.elapsed_time(g1) / DK
            del g
            return eager_ms, kms, gms

        for B in [int(b) for b in args.decode_batches.split(",")]:
            eager_ms, kms, gms = decode_variant(B, dws)
            kern_gbs = B * per_seq / (kms * 1e-3) / 1e9
            dec[f"B{B}"] = {"layers": L, "eager_ms_per_step": eager_ms,
                            "eager_state_GBps": L * B * state_per_seq / (eager_ms * 1e-3) / 1e9,
                            "kernel_avg_ms": kms,
                            "roofline": {"bound": "hbm", "achieved": kern_gbs, "peak": PEAK_HBM_GBS,
                                         "unit": "GB/s", "frac": kern_gbs / PEAK_HBM_GBS,
                                         "traffic": measured_traffic(f"decode_b{B}/decode"),
                                         "bytes_per_launch": B * per_seq}}
            # the step as a serving loop runs it, replayed from a graph: the
            # headline decode figures (the eager loop above also pays the
            # Python binding's per-call cost, which B = 64 no longer hides)
            state_gbs = L * B * state_per_seq / (gms * 1e-3) / 1e9
            dec[f"B{B}"].update({"ms_per_step": gms, "state_GBps": state_gbs,
                                 "all_bytes_GBps": L * B * per_seq / (gms * 1e-3) / 1e9,
                                 "state_frac_hbm": state_gbs / PEAK_HBM_GBS})
            log(f"decode B={B}: {gms:.3f} ms/step from a graph ({eager_ms:.3f} eager), state "
                f"{state_gbs:.1f} GB/s, kernel {kms * 1e3:.1f} us = {kern_gbs:.1f} GB/s")
            if args.decode_compare:
                e2, k2, g2 = decode_variant(B, None)
                dec[f"B{B}"]["without_workspace"] = {"ms_per_step": g2, "eager_ms_per_step": e2,
                                                     "kernel_avg_ms": k2}
                log(f"  without a workspace (one work-group per key head): {g2:.3f} ms/step from a graph, "
                    f"kernel {k2 * 1e3:.1f} us")
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
        for _ in range(5):
            vstep()
        torch.cuda.synchronize()
        v0, v1 = new_events(2)
        v0.record(stream)
        for i in range(DK):
            vstep()
        v1.record(stream)
        torch.cuda.synchronize()
        vms = v0.elapsed_time(v1) / DK
        vevs = [[new_events(2) for _ in range(L)] for _ in range(DK)]
        torch.cuda.synchronize()
        for i in range(DK):
            vstep(vevs[i])
        torch.cuda.synchronize()
        vkms = sum(vevs[i][l][0].elapsed_time(vevs[i][l][1]) for i in range(DK) for l in range(L)) / (DK * L)
        result["verify"] = {"B": VB, "tokens": VT, "layers": L, "ms_per_step": vms,
                            "tokens_per_s": VB * VT / (vms * 1e-3),
                            "kernel_avg_ms": vkms,
                            "state_GBps": L * VB * state_per_seq / (vms * 1e-3) / 1e9}
        log(f"verify B={VB} x {VT} tokens: {vms:.3f} ms/step, kernel {vkms * 1e3:.1f} us")
        del layers, states, convs, toks, vt, vouts
        torch.cuda.empty_cache()

    # ---------------- the layer with its projections, 1 x 4096 ----------------
    if not args.headline_only and not args.no_layer:
        T = 4096
        H = synth.HIDDEN
        gen = torch.Generator(device=dev)
        gen.manual_seed(21)
        P = synth.proj_rows(sh)
        HD = sh.Hv * sh.dv
        lay = layer_from(synth.layer_params(sh, 1))
        cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
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

        LK = 20
        for i in range(5):
            layer_step(xs[i % 3])
        l0, l1 = new_events(2)
        l0.record(stream)
        for i in range(LK):
            layer_step(xs[i % 3])
        l1.record(stream)
        torch.cuda.synchronize()
        lms = l0.elapsed_time(l1) / LK
        # the two GEMMs alone, same shapes and buffers
        pbuf = torch.empty((T, P), dtype=torch.bfloat16, device=dev)
        gbuf = torch.empty((T, HD), dtype=torch.bfloat16, device=dev)

        def gemm_ms(A, B, C):
            for _ in range(2):
                gdn.gemm_bf16(A, B, C)
            g0, g1 = new_events(2)
            g0.record(stream)
            for _ in range(LK):
                gdn.gemm_bf16(A, B, C)
            g1.record(stream)
            torch.cuda.synchronize()
            return g0.elapsed_time(g1) / LK

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
            dws = torch.zeros(gdn.layer_decode_workspace_bytes(lay, projs[0], Bd), dtype=torch.uint8, device=dev)

            def ldstep(l):
                gdn.layer_decode_raw(lay, projs[l], B=Bd, x=xd, y=yd, state_in=sd[l], state_out=sd[l],
                                     conv_state_in=cd[l], conv_state_out=cd[l], workspace=dws)

            for l in range(NL):
                ldstep(l)
            d0, d1 = new_events(2)
            d0.record(stream)
            R = 3
            for _ in range(R):
                for l in range(NL):
                    ldstep(l)
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
        host_cpus = os.cpu_count() or 1
        cores = min(host_cpus, 16)
        d = oracle.Dims(sh.Hk, sh.Hv, sh.dk, sh.dv, 4, sh.scale, sh.eps_l2, sh.eps_rms)

        def oracle_rate(Ts, threads):
            """tokens/s of the oracle on the first Ts tokens of a seeded
            sample of the headline workload (its shape and distributions,
            an N(0, 0.02) initial state), all 32 value heads."""
            c = synth.prefill_case(sh, [Ts], seed=3, with_state=True)
            t0 = time.perf_counter()
            oracle.gdn_forward(d, c.cu_seqlens, *(c.inputs[n] for n in "qkvzab"), c.params["conv_w"],
                               c.params["A_log"], c.params["dt_bias"], c.params["norm_w"],
                               c.initial_state, nthreads=threads)
            return Ts / (time.perf_counter() - t0)

        probe = oracle_rate(256, cores)
        Ts = int(min(131072, max(256, probe * args.cpu_seconds)) // 64 * 64)
        rate = oracle_rate(Ts, cores)
        probe1 = oracle_rate(64, 1)
        T1 = int(min(4096, max(64, probe1 * args.cpu_seconds / 2)) // 64 * 64)
        rate1 = oracle_rate(T1, 1)
        result["cpu_baseline"] = {
            "value": rate, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {Ts} of the 131072 tokens of a seeded host-side draw of the headline "
                      f"workload (same shape and distributions, N(0,0.02) initial state), all 32 value "
                      f"heads, fp64 token by token on {cores} threads",
            "single_thread_tokens_per_s": rate1, "single_thread_sample_tokens": T1,
            "host_cpus": host_cpus, "cpu_model": cpu_model()}
        log(f"cpu baseline: {rate:.1f} tok/s on {cores} threads ({Ts} tokens), {rate1:.1f} tok/s on one "
            f"thread ({T1} tokens); host has {host_cpus} CPUs ({cpu_model()})")

    if not args.only:
        print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
