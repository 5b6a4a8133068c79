"""Benchmark of the Gated DeltaNet token mixer on one MI355X.

A step is one pass of the prefill token mixer over the bf16 workload B=4, H=16, T=4096,
d_k=d_v=128 (preprocess -> chunked prefill -> output gate), inputs resident in HBM.
`value` is that pipeline's throughput in Mtok/s (a token spans all 16 heads), from K steps
timed with nothing but a synchronisation on either side. The steps rotate over several
complete sets of input and output buffers (together larger than the 256 MB Infinity Cache), so
no step finds the previous step's data in that cache. Per-step percentiles and per-kernel
durations come from two further passes of K steps, each with events between calls.

Beside it, in the same JSON line:
  long_context     one sequence B=1, H=32, T=65536 with an initial and a final state (the
                   1024-step inter-chunk scan), gdn_chunk_prefill alone;
  varlen           64 packed sequences, log-uniform lengths in [128, 32768], H=16, through the
                   whole pipeline with per-sequence initial and final states;
  decode           256 sequences x 32 heads, 100 steps, fp32 state updated in place (and the
                   multi-token and fused forms);
  ceilings         the HBM stream and bf16 matrix-core rates measured on this device;
  cpu_baseline     the fp64 oracle on a bounded sample, on the host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                       [--no-backward] [--no-extra-configs] [--rotate R]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak, TFLOP/s
CHUNK = 64


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def prefill_algorithmic(H, dk, dv, ntok, nseq, s0, st, in_bytes=2, y_bytes=2):
    """Algorithmic bytes and flops of one chunked-prefill launch.
    bytes per token-head: q, k, v read + g, beta (fp32) + y written; per (seq, head): states.
    flops per token-head: 6 dk dv (Q S, K S (W S), K^T U) + C(2dk + dv) (causal halves of
    Q K^T, K K^T, P U) + C(dk + dv) (T applied to both sides) + C^2/3 (triangular solve)."""
    th = ntok * H
    per_th_bytes = (2 * dk + dv) * in_bytes + 8 + dv * y_bytes
    state_bytes = nseq * H * dk * dv * 4 * (int(s0) + int(st))
    per_th_flops = 6 * dk * dv + CHUNK * (2 * dk + dv) + CHUNK * (dk + dv) + CHUNK * CHUNK / 3
    return th * per_th_bytes + state_bytes, th * per_th_flops


def preprocess_bytes(ntok, H, dk, dv, nseq=1):
    """x streams read (bf16) + q, k, v written (bf16) + a_raw, b_raw read and g, beta written
    (fp32) + conv taps and per-head vectors."""
    return ntok * H * (2 * dk + dv) * (2 + 2) + ntok * H * 16 + 3 * H * 128 * 4 * 4


def gate_bytes(ntok, H, dv):
    """y and z read, o written (bf16)."""
    return ntok * H * dv * (2 + 2 + 2)


def pct(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "p50": round(float(np.median(a)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


TRAFFIC_RECORD = "traffic_bench_kernels_B4_H16_T4096_d128_and_decode_N256_H32.json"
MFMA_RECORD = "mfma_bench_kernels_B4_H16_T4096_d128_and_decode_N256_H32.json"


def counter_record(name, sources):
    """A committed counter summary under profiles/, if every source file in `sources` is
    unchanged since the counters were taken (else None: the figures no longer apply)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    from gated_deltanet_recurrence_chunked_amd import rocprof_summary
    with open(path) as f:
        rec = json.load(f)
    now = rocprof_summary.source_shas()
    then = rec.get("source_sha256", {})
    if any(then.get(f) != now.get(f) for f in sources):
        return None
    return rec


def counted_bytes(rec, kernel):
    """FETCH + WRITE bytes per dispatch of `kernel` in a traffic record, for its largest launch
    (the record's workloads: prefill B=4 H=16 T=4096 and decode N=256 H=32; the decode forms
    launch the streaming kernels on far smaller grids)."""
    if rec is None:
        return None
    hits = [e["bytes"] for k, e in rec["kernels"].items() if k.startswith(kernel)]
    return max(hits) if hits else None


PREFILL_SRC = ("chunk_bf16.hip", "gdn_device.h", "gdn_inverse.h", "gdn_mfma.h")


class Timer:
    """HIP events on one stream: `total` brackets a region, `between` marks call boundaries."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def region(self, fn, n):
        """ms per call of fn() over n calls, events only around the whole region."""
        self.torch.cuda.synchronize()
        e0 = self.event()
        for i in range(n):
            fn(i)
        e1 = self.event()
        self.torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def per_call(self, fn, n):
        """ms of each of n calls (an event between consecutive calls)."""
        self.torch.cuda.synchronize()
        evs = [self.event()]
        for i in range(n):
            fn(i)
            evs.append(self.event())
        self.torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(evs[:-1], evs[1:])]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=3,
                    help="buffer sets the pipeline steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB stream copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.rotate < 1:
        print("--steps and --rotate must be >= 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    from gated_deltanet_recurrence_chunked_amd import inputs as gi

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    bf = torch.bfloat16
    stream = torch.cuda.current_stream()
    tm = Timer(torch, stream)

    def d(a, bf16=False):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(bf).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # ------------------------------------------------------------------ prefill workload
    log("[bench] generating bf16 prefill inputs B=4 H=16 T=4096 d=128")
    inp = gi.make_inputs(gi.PREFILL, seed=0)
    sh = inp["shape"]
    H, dk, dv, ntok, nseq = sh.H, sh.dk, sh.dv, sh.ntok, sh.num_seqs
    W = dict(wq=d(inp["wq"]), wk=d(inp["wk"]), wv=d(inp["wv"]), A_log=d(inp["A_log"]),
             dt_bias=d(inp["dt_bias"]), nw=d(inp["norm_weight"]))
    base = dict(xq=d(inp["xq"], True), xk=d(inp["xk"], True), xv=d(inp["xv"], True),
                a_raw=d(inp["a_raw"]), b_raw=d(inp["b_raw"]), z=d(inp["z"], True))

    def new_set(first):
        X = {k_: (t if first else t.clone()) for k_, t in base.items()}
        outs = dict(q=torch.empty((ntok, H, dk), dtype=bf, device=dev),
                    k=torch.empty((ntok, H, dk), dtype=bf, device=dev),
                    v=torch.empty((ntok, H, dv), dtype=bf, device=dev),
                    g=torch.empty((ntok, H), dtype=torch.float32, device=dev),
                    beta=torch.empty((ntok, H), dtype=torch.float32, device=dev))
        return dict(X=X, outs=outs, y=torch.empty((ntok, H, dv), dtype=bf, device=dev),
                    o=torch.empty((ntok, H, dv), dtype=bf, device=dev))
    sets = [new_set(i == 0) for i in range(args.rotate)]
    set_bytes = sum(t.numel() * t.element_size() for s_ in sets[:1]
                    for t in list(s_["X"].values()) + list(s_["outs"].values()) + [s_["y"], s_["o"]])
    ws_n = gdn.gdn_chunk_prefill_workspace_size(ntok, nseq, H, dk, dv, bf)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def preprocess(s_):
        X = s_["X"]
        gdn.gdn_preprocess(X["xq"], X["xk"], X["xv"], W["wq"], W["wk"], W["wv"], X["a_raw"],
                           X["b_raw"], W["A_log"], W["dt_bias"], H=H, num_seqs=nseq,
                           out_dtype=bf, outs=s_["outs"])

    def prefill(s_):
        o_ = s_["outs"]
        gdn.gdn_chunk_prefill(o_["q"], o_["k"], o_["v"], o_["g"], o_["beta"], num_seqs=nseq,
                              y=s_["y"], workspace=ws, output_final_state=False)

    def gate(s_):
        gdn.gdn_output_gate(s_["y"], s_["X"]["z"], W["nw"], eps=1e-6, o=s_["o"])

    def step(i):
        s_ = sets[i % len(sets)]
        preprocess(s_)
        prefill(s_)
        gate(s_)

    log(f"[bench] warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps over {len(sets)} rotating buffer sets "
        f"({set_bytes / 1e6:.0f} MB each)")
    ms_step = tm.region(step, args.steps)
    mtoks = ntok / (ms_step * 1e-3) / 1e6
    step_ms = tm.per_call(step, args.steps)
    # per-kernel durations: a third pass, an event between consecutive calls
    kt = {"pre": [], "pf": [], "og": []}

    def kstep(i):
        s_ = sets[i % len(sets)]
        evs = [tm.event()]
        preprocess(s_)
        evs.append(tm.event())
        prefill(s_)
        evs.append(tm.event())
        gate(s_)
        evs.append(tm.event())
        kt.setdefault("ev", []).append(evs)
    tm.region(kstep, args.steps)
    for evs in kt.pop("ev"):
        kt["pre"].append(evs[0].elapsed_time(evs[1]))
        kt["pf"].append(evs[1].elapsed_time(evs[2]))
        kt["og"].append(evs[2].elapsed_time(evs[3]))
    t_pre, t_pf, t_og = (float(np.mean(kt[x])) for x in ("pre", "pf", "og"))
    log(f"[bench] pipeline {ms_step * 1e3:.1f} us/step = {mtoks:.1f} Mtok/s "
        f"(median step {np.median(step_ms) * 1e3:.1f} us; preprocess {t_pre * 1e3:.1f} us, "
        f"prefill {t_pf * 1e3:.1f} us, gate {t_og * 1e3:.1f} us)")

    pf_bytes, pf_flops = prefill_algorithmic(H, dk, dv, ntok, nseq, False, False)
    pre_b, og_b = preprocess_bytes(ntok, H, dk, dv), gate_bytes(ntok, H, dv)
    kernels = {
        "gdn_preprocess": dict(us=round(t_pre * 1e3, 2), **{"us_" + k_: v_ for k_, v_ in pct([x * 1e3 for x in kt["pre"]]).items()},
                               GBs=round(pre_b / (t_pre * 1e-3) / 1e9, 1), bytes=pre_b),
        "gdn_chunk_prefill": dict(us=round(t_pf * 1e3, 2), **{"us_" + k_: v_ for k_, v_ in pct([x * 1e3 for x in kt["pf"]]).items()},
                                  GBs=round(pf_bytes / (t_pf * 1e-3) / 1e9, 1),
                                  TFLOPs=round(pf_flops / (t_pf * 1e-3) / 1e12, 1),
                                  Mtok_s=round(ntok / (t_pf * 1e-3) / 1e6, 2)),
        "gdn_output_gate": dict(us=round(t_og * 1e3, 2), **{"us_" + k_: v_ for k_, v_ in pct([x * 1e3 for x in kt["og"]]).items()},
                                GBs=round(og_b / (t_og * 1e-3) / 1e9, 1), bytes=og_b),
    }
    pf_gbs = pf_bytes / (t_pf * 1e-3) / 1e9
    traffic_rec = counter_record(TRAFFIC_RECORD, PREFILL_SRC)
    mfma_rec = counter_record(MFMA_RECORD, PREFILL_SRC)
    stream_rec = counter_record(TRAFFIC_RECORD, ("preprocess.hip", "gdn_device.h"))
    for name, kern, t_ms in (("gdn_preprocess", "preprocess_kernel<unsigned short, unsigned short>", t_pre),
                             ("gdn_output_gate", "output_gate_kernel<unsigned short", t_og)):
        cb = counted_bytes(stream_rec, kern)
        if cb is not None:
            kernels[name]["counted_bytes"] = int(cb)
            kernels[name]["counted_GBs"] = round(cb / (t_ms * 1e-3) / 1e9, 1)
    roofline = {"kernel": "gdn_chunk_prefill (chunk_prep_kernel + chunk_scan_fwd_kernel)",
                "bound": "hbm", "achieved": round(pf_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(pf_gbs / HBM_PEAK_GBS, 4),
                "traffic": (int(traffic_rec["gdn_chunk_prefill_bytes_per_call"])
                            if traffic_rec else None),
                "algorithmic_bytes_per_launch": pf_bytes,
                "launch_us": round(t_pf * 1e3, 2),
                "mfma": {"achieved_TFLOPs": round(pf_flops / (t_pf * 1e-3) / 1e12, 1),
                         "peak_TFLOPs": BF16_PEAK_TFLOPS,
                         "frac": round(pf_flops / (t_pf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops_per_launch": pf_flops}}
    if mfma_rec:
        # flops the matrix cores executed (counted), over the same live launch time
        cf = float(mfma_rec["gdn_chunk_prefill_mfma_flops_per_call"])
        roofline["mfma"]["counted_flops_per_launch"] = int(cf)
        roofline["mfma"]["counted_TFLOPs"] = round(cf / (t_pf * 1e-3) / 1e12, 1)
        roofline["mfma"]["counted_frac"] = round(cf / (t_pf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    del kt

    # the same token mixer through the fused entry point (one call: the preprocess kernel, the
    # chunked prefill, and the gated RMSNorm, which runs in the scan's epilogue only where the
    # full-row scan runs, from 256 (sequence, head) pairs of equal length; here it launches the
    # same kernels as the separate calls). The clock drifts over a run, so the ratio comes from rounds that time
    # the fused call and the separate calls in turn (median of each).
    ws_f = torch.empty(gdn.gdn_fused_prefill_workspace_size(ntok, nseq, H, dk, dv),
                       dtype=torch.uint8, device=dev)

    def fstep(i):
        s_ = sets[i % len(sets)]
        X = s_["X"]
        gdn.gdn_fused_prefill(X["xq"], X["xk"], X["xv"], W["wq"], W["wk"], W["wv"], X["a_raw"],
                              X["b_raw"], W["A_log"], W["dt_bias"], X["z"], W["nw"], H=H,
                              num_seqs=nseq, output_final_state=False, o=s_["o"], workspace=ws_f)
    for i in range(5):
        fstep(i)
    ms_fused = tm.region(fstep, args.steps)
    n_r = max(1, args.steps // 5)
    rounds_f, rounds_s = [], []
    for _ in range(5):
        rounds_f.append(tm.region(fstep, n_r))
        rounds_s.append(tm.region(step, n_r))
    ratio = float(np.median(rounds_s) / np.median(rounds_f))
    fused_prefill = {"workload": "gdn_fused_prefill at B=4 H=16 T=4096 d=128 (bf16 x, z, o)",
                     "calls": args.steps, "us_per_call": round(ms_fused * 1e3, 1),
                     "Mtok_s": round(ntok / (ms_fused * 1e-3) / 1e6, 2),
                     "vs_separate_kernels": round(ratio, 3),
                     "rounds_us": {"fused": [round(x * 1e3, 1) for x in rounds_f],
                                   "separate": [round(x * 1e3, 1) for x in rounds_s]}}
    log(f"[bench] fused prefill {ms_fused * 1e3:.1f} us/call = {fused_prefill['Mtok_s']} Mtok/s "
        f"({ratio:.2f}x the separate kernels, timed in turn)")
    del ws_f

    # ------------------------------------------------------------------ backward (training)
    outs = sets[0]["outs"]
    y = sets[0]["y"]
    backward = None
    if not args.no_backward:
        gen = torch.Generator(device=dev).manual_seed(0)
        dy = torch.randn((ntok, H, dv), generator=gen, device=dev).to(bf)
        ws_b = torch.empty(gdn.gdn_chunk_backward_workspace_size(ntok, nseq, H, dk, dv),
                           dtype=torch.uint8, device=dev)

        def bstep(i):
            gdn.gdn_chunk_backward(outs["q"], outs["k"], outs["v"], outs["g"], outs["beta"], dy,
                                   num_seqs=nseq, workspace=ws_b, want_dinitial_state=False)
        for i in range(3):
            bstep(i)
        bms = tm.region(bstep, 10)
        backward = {"workload": "gdn_chunk_backward at B=4 H=16 T=4096 d=128 (bf16 q, k, v, dy; "
                                "fp32 gradients of q, k, v, g, beta)",
                    "calls": 10, "us_per_call": round(bms * 1e3, 1),
                    "Mtok_s": round(ntok / (bms * 1e-3) / 1e6, 2),
                    "workspace_bytes": ws_b.numel(),
                    "vs_forward_prefill": round(bms / t_pf, 2)}
        log(f"[bench] backward {bms * 1e3:.1f} us/call ({backward['Mtok_s']} Mtok/s, "
            f"{bms / t_pf:.1f}x the forward prefill)")
        del dy, ws_b

    # ------------------------------------------------------------------ per-channel decay variant
    kda = None
    if not args.no_backward:
        gen = torch.Generator(device=dev).manual_seed(1)
        gk = -torch.clamp(torch.exp(torch.randn((ntok, H, dk), generator=gen, device=dev) - 2.0),
                          max=5.0)
        ws_k = torch.empty(int(gdn.lib().gdn_kda_chunk_prefill_bounded_workspace_size(ntok, nseq, H)),
                           dtype=torch.uint8, device=dev)
        ws_f = torch.empty(int(gdn.lib().gdn_kda_chunk_prefill_workspace_size(ntok, nseq, H, dk)),
                           dtype=torch.uint8, device=dev)

        def kstep_(i):   # log-decays in [-5, 0): the bf16 matrix-core path
            gdn.gdn_kda_chunk_prefill_bounded(outs["q"], outs["k"], outs["v"], gk, outs["beta"],
                                              num_seqs=nseq, y=y, workspace=ws_k,
                                              output_final_state=False)

        def fstep_(i):   # the same call on the fp32 path (any log-decay <= 0)
            gdn.gdn_kda_chunk_prefill(outs["q"], outs["k"], outs["v"], gk, outs["beta"],
                                      num_seqs=nseq, y=y, workspace=ws_f, output_final_state=False)
        for i in range(3):
            kstep_(i)
            fstep_(i)
        kms = tm.region(kstep_, 10)
        fms_ = tm.region(fstep_, 5)
        kda = {"workload": "gdn_kda_chunk_prefill_bounded at B=4 H=16 T=4096 d=128 (bf16 q, k, v, "
                           "y; per-channel fp32 log-decays in [-5, 0))",
               "calls": 10, "us_per_call": round(kms * 1e3, 1),
               "Mtok_s": round(ntok / (kms * 1e-3) / 1e6, 2),
               "vs_scalar_decay_prefill": round(kms / t_pf, 2),
               "fp32_path_us_per_call": round(fms_ * 1e3, 1)}
        log(f"[bench] per-channel-decay prefill {kms * 1e3:.1f} us/call ({kda['Mtok_s']} Mtok/s); "
            f"fp32 path {fms_ * 1e3:.1f} us/call")
        del ws_f
        del gk, ws_k

    del sets, outs, y, ws, base
    torch.cuda.empty_cache()

    long_context = varlen = None
    if not args.no_extra_configs:
        long_context = bench_long_context(torch, gdn, gi, dev, tm)
        varlen = bench_varlen(torch, gdn, gi, dev, tm)

    decode = None if args.no_decode else bench_decode(torch, gdn, gi, dev, tm, d, args)
    ceilings = bench_ceilings(torch, gdn, dev, tm)

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        gdn.gdn_mb_stream(src, dst)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import gdn_cases as C
        sub = C.subset(inp, seqs=list(range(nseq)))
        threads = oracle.default_threads()
        log(f"[bench] timing the fp64 oracle on {nseq} sequences x {H} heads x {sh.lengths[0]} "
            f"tokens with {threads} threads")
        # the whole workload, repeated until about 10 s of work have been timed
        runs, t0 = 0, time.perf_counter()
        while True:
            C.oracle_run(sub, nthreads=threads)
            runs += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or runs >= 50:
                break
        ntok_s = int(sub["cu"][-1])
        cpu = {"value": round(ntok_s * runs / dt / 1e6, 6), "unit": "Mtok/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{nseq} of {nseq} sequences ({ntok_s} tokens x {H} heads, d=128): "
                         f"preprocess + gates + recurrence + output gate in fp64, {runs} runs in "
                         f"{dt:.1f} s",
               "cpu": cpu_model()}
        log(f"[bench] oracle {runs} runs in {dt:.1f} s -> {cpu['value']} Mtok/s")

    out = {
        "metric": "GDN prefill Mtok/s (H16,d128,T4096) + decode state-update HBM GB/s",
        "value": round(mtoks, 2), "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "step_us": pct([x * 1e3 for x in step_ms]),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 GDN prefill token mixer: preprocess + chunked prefill "
                               "(C=64) + output gate", "B": 4, "H": H, "T": sh.lengths[0],
                   "d_k": dk, "d_v": dv, "tokens_per_step": ntok,
                   "rotating_buffer_sets": args.rotate,
                   "timing": "value from K steps between two synchronisations; step_us from a "
                             "second pass with an event between steps; kernels from a third "
                             "pass with events between calls"},
        "kernels": kernels, "roofline": roofline, "decode": decode,
        "long_context": long_context, "varlen": varlen, "backward": backward,
        "per_channel_decay": kda, "fused_prefill": fused_prefill, "ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def bench_long_context(torch, gdn, gi, dev, tm):
    """One sequence B=1, H=32, T=65536, d=128 with S0 ~ N(0, 0.01) and the final state:
    gdn_chunk_prefill alone (q, k unit rows, v ~ N(0,1), bf16; gates drawn as in the small
    configurations and turned into g, beta by the gates-only preprocess)."""
    bf = torch.bfloat16
    L, H, dk, dv = 65536, 32, 128, 128
    log(f"[bench] long-context prefill B=1 H={H} T={L} (inputs drawn on the device)")
    g = torch.Generator(device=dev).manual_seed(2)

    def unit(shape):
        x = torch.randn(shape, generator=g, device=dev)
        return (x / x.norm(dim=-1, keepdim=True)).to(bf)
    q, k = unit((L, H, dk)), unit((L, H, dk))
    v = torch.randn((L, H, dv), generator=g, device=dev).to(bf)
    a_raw = torch.randn((L, H), generator=g, device=dev)
    b_raw = torch.randn((L, H), generator=g, device=dev)
    A_log = torch.log(1.0 + 15.0 * torch.rand((H,), generator=g, device=dev))
    dt_bias = torch.full((H,), -4.6, device=dev)
    _, _, _, gg, beta = gdn.gdn_preprocess(None, None, None, None, None, None, a_raw, b_raw,
                                           A_log, dt_bias, H=H)
    S0 = torch.randn((1, H, dk, dv), generator=g, device=dev) * 0.1
    ST = torch.empty_like(S0)
    y = torch.empty((L, H, dv), dtype=bf, device=dev)
    ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(L, 1, H, dk, dv, bf),
                     dtype=torch.uint8, device=dev)

    def call(i):
        gdn.gdn_chunk_prefill(q, k, v, gg, beta, initial_state=S0, final_state=ST, y=y,
                              workspace=ws)
    call(0)
    n = 5
    times = tm.per_call(call, n)
    ms = float(np.mean(times))
    b, f = prefill_algorithmic(H, dk, dv, L, 1, True, True)
    res = {"workload": "gdn_chunk_prefill B=1 H=32 T=65536 d=128, bf16 q, k, v, y, fp32 S0 and "
                       "S_T (1024 chunks in sequence)",
           "calls": n, "us_per_call": round(ms * 1e3, 1), "us": pct([t * 1e3 for t in times]),
           "Mtok_s": round(L / (ms * 1e-3) / 1e6, 3),
           "GBs": round(b / (ms * 1e-3) / 1e9, 1), "hbm_frac": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "TFLOPs": round(f / (ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "algorithmic_bytes": b, "algorithmic_flops": f}
    log(f"[bench] long-context prefill {ms * 1e3:.1f} us/call = {res['Mtok_s']} Mtok/s "
        f"({res['hbm_frac']:.1%} HBM, {res['mfma_frac']:.1%} MFMA)")
    del q, k, v, a_raw, b_raw, gg, beta, S0, ST, y, ws
    torch.cuda.empty_cache()
    return res


def bench_varlen(torch, gdn, gi, dev, tm):
    """64 packed sequences with the seeded log-uniform lengths of the varlen workload, H=16,
    d=128, through preprocess (conv reset at each start) -> prefill (S0, S_T) -> output gate.
    Values are drawn on the device with the distributions of the small configurations."""
    bf = torch.bfloat16
    sh = gi.make_shape(gi.VARLEN)
    H, dk, dv, ntok, nseq = sh.H, sh.dk, sh.dv, sh.ntok, sh.num_seqs
    log(f"[bench] varlen pipeline {nseq} sequences, {ntok} tokens, H={H} (inputs drawn on the device)")
    cu_host = sh.cu_seqlens()
    cu = torch.from_numpy(cu_host).to(dev)
    g = torch.Generator(device=dev).manual_seed(4)

    def bfn(shape, std=1.0):
        return (torch.randn(shape, generator=g, device=dev) * std).to(bf)
    xq, xk, xv, z = bfn((ntok, H, dk)), bfn((ntok, H, dk)), bfn((ntok, H, dv)), bfn((ntok, H, dv))
    wq = torch.randn((H * dk, 4), generator=g, device=dev) * 0.5
    wk = torch.randn((H * dk, 4), generator=g, device=dev) * 0.5
    wv = torch.randn((H * dv, 4), generator=g, device=dev) * 0.5
    a_raw = torch.randn((ntok, H), generator=g, device=dev)
    b_raw = torch.randn((ntok, H), generator=g, device=dev)
    A_log = torch.log(1.0 + 15.0 * torch.rand((H,), generator=g, device=dev))
    dt_bias = torch.full((H,), -4.6, device=dev)
    nw = torch.randn((dv,), generator=g, device=dev) * math.sqrt(0.02)
    S0 = torch.randn((nseq, H, dk, dv), generator=g, device=dev) * 0.1
    ST = torch.empty_like(S0)
    outs = dict(q=torch.empty((ntok, H, dk), dtype=bf, device=dev),
                k=torch.empty((ntok, H, dk), dtype=bf, device=dev),
                v=torch.empty((ntok, H, dv), dtype=bf, device=dev),
                g=torch.empty((ntok, H), dtype=torch.float32, device=dev),
                beta=torch.empty((ntok, H), dtype=torch.float32, device=dev))
    y = torch.empty((ntok, H, dv), dtype=bf, device=dev)
    o = torch.empty((ntok, H, dv), dtype=bf, device=dev)
    ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(ntok, nseq, H, dk, dv, bf),
                     dtype=torch.uint8, device=dev)
    kt = []

    def step(i, timed=False):
        e = [tm.event()] if timed else None
        gdn.gdn_preprocess(xq, xk, xv, wq, wk, wv, a_raw, b_raw, A_log, dt_bias, H=H,
                           cu_seqlens=cu, num_seqs=nseq, out_dtype=bf, outs=outs)
        if timed:
            e.append(tm.event())
        gdn.gdn_chunk_prefill(outs["q"], outs["k"], outs["v"], outs["g"], outs["beta"],
                              initial_state=S0, final_state=ST, cu_seqlens=cu,
                              cu_seqlens_host=cu_host, num_seqs=nseq, y=y, workspace=ws)
        if timed:
            e.append(tm.event())
        gdn.gdn_output_gate(y, z, nw, eps=1e-6, o=o)
        if timed:
            e.append(tm.event())
            kt.append(e)
    step(0)
    n = 5
    times = tm.per_call(step, n)
    ms = float(np.mean(times))
    tm.region(lambda i: step(i, True), n)
    t_pre = float(np.mean([e[0].elapsed_time(e[1]) for e in kt]))
    t_pf = float(np.mean([e[1].elapsed_time(e[2]) for e in kt]))
    t_og = float(np.mean([e[2].elapsed_time(e[3]) for e in kt]))
    # the same token mixer through the fused entry point (packed sequences of unequal lengths
    # take the sliced scan and the output-gate kernel, as the separate calls do)
    wsf = torch.empty(gdn.gdn_fused_prefill_workspace_size(ntok, nseq, H, dk, dv),
                      dtype=torch.uint8, device=dev)

    def fstep(i):
        gdn.gdn_fused_prefill(xq, xk, xv, wq, wk, wv, a_raw, b_raw, A_log, dt_bias, z, nw, H=H,
                              initial_state=S0, cu_seqlens=cu, cu_seqlens_host=cu_host,
                              num_seqs=nseq, o=o, workspace=wsf)
    fstep(0)
    fms = tm.region(fstep, n)
    # the ratio from rounds that time the two forms in turn (the clock drifts over a run)
    rf, rs = [], []
    for _ in range(3):
        rf.append(tm.region(fstep, 2))
        rs.append(tm.region(step, 2))
    fratio = float(np.median(rs) / np.median(rf))
    del wsf
    b, f = prefill_algorithmic(H, dk, dv, ntok, nseq, True, True)
    res = {"workload": f"varlen pipeline: {nseq} packed sequences (seeded log-uniform lengths in "
                       f"[128, 32768], {ntok} tokens), H=16 d=128, bf16, per-sequence S0 and S_T",
           "steps": n, "us_per_step": round(ms * 1e3, 1), "step_us": pct([t * 1e3 for t in times]),
           "Mtok_s": round(ntok / (ms * 1e-3) / 1e6, 2),
           "kernels_us": {"gdn_preprocess": round(t_pre * 1e3, 1),
                          "gdn_chunk_prefill": round(t_pf * 1e3, 1),
                          "gdn_output_gate": round(t_og * 1e3, 1)},
           "prefill_hbm_frac": round(b / (t_pf * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "prefill_mfma_frac": round(f / (t_pf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "longest_sequence": int(max(sh.lengths)),
           "fused_us_per_step": round(fms * 1e3, 1),
           "fused_Mtok_s": round(ntok / (fms * 1e-3) / 1e6, 2),
           "fused_vs_separate_kernels": round(fratio, 3)}
    log(f"[bench] varlen pipeline {ms * 1e3:.1f} us/step = {res['Mtok_s']} Mtok/s "
        f"(prefill {t_pf * 1e3:.1f} us); fused {fms * 1e3:.1f} us/step ({fratio:.2f}x, timed in turn)")
    del xq, xk, xv, z, outs, y, o, ws, S0, ST, a_raw, b_raw
    torch.cuda.empty_cache()
    return res


def bench_decode(torch, gdn, gi, dev, tm, d, args):
    bf = torch.bfloat16
    S_ = args.decode_steps
    log(f"[bench] generating decode inputs N=256 H=32 d=128, {S_} steps")
    di = gi.make_inputs(gi.DECODE, seed=0, steps=S_)
    dsh = di["shape"]
    N, DH = dsh.num_seqs, dsh.H
    state = d(di["state"])
    qd, kd, vd = d(di["q"], True), d(di["k"], True), d(di["v"], True)
    _, _, _, gd, bd = gdn.gdn_preprocess(None, None, None, None, None, None,
                                         d(di["a_raw"].reshape(S_ * N, DH)),
                                         d(di["b_raw"].reshape(S_ * N, DH)),
                                         d(di["A_log"]), d(di["dt_bias"]), H=DH)
    gd = gd.view(S_, N, DH)
    bd = bd.view(S_, N, DH)
    yd = torch.empty((S_, N, DH, dsh.dv), dtype=bf, device=dev)

    def dstep(s):
        gdn.gdn_decode_step(qd[s], kd[s], vd[s], gd[s], bd[s], state, y=yd[s])
    for s in range(min(3, S_)):      # warm-up (advances the state; timing is unaffected)
        dstep(s)
    dms = tm.region(dstep, S_)
    dper = tm.per_call(dstep, S_)
    heads = N * DH
    state_bytes = heads * dsh.dk * dsh.dv * 4 * 2
    tok_bytes = heads * ((2 * dsh.dk + dsh.dv) * 2 + 8 + dsh.dv * 2)
    gbs = (state_bytes + tok_bytes) / (dms * 1e-3) / 1e9
    decode = {"workload": "decode N=256 H=32 d_k=d_v=128, fp32 state in place, bf16 tokens",
              "steps": S_, "us_per_step": round(dms * 1e3, 2),
              "step_us": pct([x * 1e3 for x in dper]), "GB_s": round(gbs, 1),
              "state_only_GB_s": round(state_bytes / (dms * 1e-3) / 1e9, 1),
              "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
              "bytes_per_step": state_bytes + tok_bytes}
    rec = counter_record(TRAFFIC_RECORD, ("decode.hip", "gdn_device.h"))
    cb = counted_bytes(rec, "decode_pipe_kernel<")
    if cb is not None:
        decode["counted_bytes"] = int(cb)
        decode["counted_GBs"] = round(cb / (dms * 1e-3) / 1e9, 1)
    log(f"[bench] decode {dms * 1e3:.1f} us/step, {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM)")
    del state, qd, kd, vd, gd, bd, yd
    torch.cuda.empty_cache()

    # multi-token decode (MTP verify): the same sequences and heads, T = 4 tokens per step,
    # a quarter as many steps (the same number of tokens)
    T4, S4 = 4, max(1, S_ // 4)
    log(f"[bench] generating multi-token decode inputs N=256 H=32 d=128 T={T4}, {S4} steps")
    mi = gi.make_inputs(gi.DECODE, seed=1, steps=S4, tokens=T4)
    state = d(mi["state"])
    qm, km, vm = d(mi["q"], True), d(mi["k"], True), d(mi["v"], True)
    _, _, _, gm, bm = gdn.gdn_preprocess(None, None, None, None, None, None,
                                         d(mi["a_raw"].reshape(S4 * N * T4, DH)),
                                         d(mi["b_raw"].reshape(S4 * N * T4, DH)),
                                         d(mi["A_log"]), d(mi["dt_bias"]), H=DH)
    gm = gm.view(S4, N, T4, DH)
    bm = bm.view(S4, N, T4, DH)
    ym = torch.empty((S4, N, T4, DH, dsh.dv), dtype=bf, device=dev)

    def mstep(s):
        gdn.gdn_decode_multi(qm[s], km[s], vm[s], gm[s], bm[s], state, y=ym[s])
    for s in range(min(3, S4)):
        mstep(s)
    mms = tm.region(mstep, S4)
    mtok_bytes = T4 * tok_bytes
    mgbs = (state_bytes + mtok_bytes) / (mms * 1e-3) / 1e9
    decode["multi_token"] = {
        "workload": f"decode N=256 H=32 d_k=d_v=128, {T4} tokens per sequence per step "
                    "(gdn_decode_multi), fp32 state in place, bf16 tokens",
        "tokens_per_step": T4, "steps": S4, "us_per_step": round(mms * 1e3, 2),
        "Mtok_s": round(N * T4 / (mms * 1e-3) / 1e6, 3), "GB_s": round(mgbs, 1),
        "hbm_frac": round(mgbs / HBM_PEAK_GBS, 4), "bytes_per_step": state_bytes + mtok_bytes,
        "vs_single_token_steps": round(T4 * dms / mms, 2)}
    cb = counted_bytes(rec, "decode_multi_kernel<128, 128, 4, unsigned short, unsigned short, false>")
    if cb is not None:
        decode["multi_token"]["counted_bytes"] = int(cb)
        decode["multi_token"]["counted_GBs"] = round(cb / (mms * 1e-3) / 1e9, 1)
    log(f"[bench] multi-token decode T={T4}: {mms * 1e3:.1f} us/step, {mgbs:.0f} GB/s "
        f"({mgbs / HBM_PEAK_GBS:.1%} of HBM), {T4 * dms / mms:.2f}x the tokens/s of T=1 steps")
    del state, qm, km, vm, gm, bm, ym
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ fused decode step
    log(f"[bench] generating fused decode inputs N=256 H=32 d=128, {S_} steps")
    fi = gi.decode_layer_draws(0, S_, 256, 32)
    N, DH, fdk, fdv = fi["N"], fi["H"], fi["dk"], fi["dv"]
    F = {x: d(fi[x], True) for x in ("xq", "xk", "xv", "z", "conv_state")}
    F.update({x: d(fi[x]) for x in ("wq", "wk", "wv", "a_raw", "b_raw", "A_log", "dt_bias",
                                    "norm_weight", "state")})
    of = torch.empty((N, DH, fdv), dtype=bf, device=dev)

    def fdec(s):
        gdn.gdn_fused_decode(F["xq"][s], F["xk"][s], F["xv"][s], F["wq"], F["wk"], F["wv"],
                             F["conv_state"], F["a_raw"][s], F["b_raw"][s], F["A_log"],
                             F["dt_bias"], F["state"], F["z"][s], F["norm_weight"], o=of)
    for s in range(min(3, S_)):
        fdec(s)
    fms = tm.region(fdec, S_)
    # the same step through the separate kernels: preprocess with the conv history carried
    # (double-buffered), the single-token update, the output gate
    hist = [F["conv_state"], torch.empty_like(F["conv_state"])]
    qkv = dict(q=torch.empty((N, DH, fdk), dtype=bf, device=dev),
               k=torch.empty((N, DH, fdk), dtype=bf, device=dev),
               v=torch.empty((N, DH, fdv), dtype=bf, device=dev),
               g=torch.empty((N, DH), dtype=torch.float32, device=dev),
               beta=torch.empty((N, DH), dtype=torch.float32, device=dev))
    ysep = torch.empty((N, DH, fdv), dtype=bf, device=dev)

    def sdec(s):
        gdn.gdn_preprocess_stateful(F["xq"][s], F["xk"][s], F["xv"][s], F["wq"], F["wk"],
                                    F["wv"], F["a_raw"][s], F["b_raw"][s], F["A_log"],
                                    F["dt_bias"], H=DH, num_seqs=N, out_dtype=bf, outs=qkv,
                                    conv_state_in=hist[s % 2], conv_state_out=hist[1 - s % 2])
        gdn.gdn_decode_step(qkv["q"], qkv["k"], qkv["v"], qkv["g"], qkv["beta"], F["state"],
                            y=ysep)
        gdn.gdn_output_gate(ysep, F["z"][s], F["norm_weight"], eps=1e-6, o=of)
    for s in range(min(2, S_)):
        sdec(s)
    sms = tm.region(sdec, S_)
    heads = N * DH
    f_state = heads * fdk * fdv * 4 * 2
    f_tok = heads * ((2 * fdk + fdv) * 2 * (1 + 3 + 3) + 8 + fdv * (2 + 2))
    fgbs = (f_state + f_tok) / (fms * 1e-3) / 1e9
    decode["fused"] = {
        "workload": "gdn_fused_decode N=256 H=32 d_k=d_v=128: conv with carried history, "
                    "gates, state update and output gate in one kernel (bf16 x, z, o)",
        "steps": S_, "us_per_step": round(fms * 1e3, 2), "GB_s": round(fgbs, 1),
        "hbm_frac": round(fgbs / HBM_PEAK_GBS, 4), "bytes_per_step": f_state + f_tok,
        "separate_kernels_us_per_step": round(sms * 1e3, 2),
        "vs_separate_kernels": round(sms / fms, 3)}
    log(f"[bench] fused decode {fms * 1e3:.1f} us/step ({fgbs:.0f} GB/s, {fgbs / HBM_PEAK_GBS:.1%} "
        f"of HBM); separate kernels {sms * 1e3:.1f} us/step")
    del F, of, hist, qkv, ysep
    torch.cuda.empty_cache()

    # the same with 4 tokens per sequence per step (MTP verify from the projected streams)
    fm = gi.decode_layer_draws(1, S4, 256, 32, tokens=T4)
    F = {x: d(fm[x], True) for x in ("xq", "xk", "xv", "z", "conv_state")}
    F.update({x: d(fm[x]) for x in ("wq", "wk", "wv", "a_raw", "b_raw", "A_log", "dt_bias",
                                    "norm_weight", "state")})
    of = torch.empty((N, T4, DH, fdv), dtype=bf, device=dev)

    def fmdec(s):
        gdn.gdn_fused_decode_multi(F["xq"][s], F["xk"][s], F["xv"][s], F["wq"], F["wk"],
                                   F["wv"], F["conv_state"], F["a_raw"][s], F["b_raw"][s],
                                   F["A_log"], F["dt_bias"], F["state"], F["z"][s],
                                   F["norm_weight"], o=of)
    for s in range(min(3, S4)):
        fmdec(s)
    fmms = tm.region(fmdec, S4)
    hist = [F["conv_state"], torch.empty_like(F["conv_state"])]
    qkv = dict(q=torch.empty((N * T4, DH, fdk), dtype=bf, device=dev),
               k=torch.empty((N * T4, DH, fdk), dtype=bf, device=dev),
               v=torch.empty((N * T4, DH, fdv), dtype=bf, device=dev),
               g=torch.empty((N * T4, DH), dtype=torch.float32, device=dev),
               beta=torch.empty((N * T4, DH), dtype=torch.float32, device=dev))
    ysep = torch.empty((N, T4, DH, fdv), dtype=bf, device=dev)

    def smdec(s):
        gdn.gdn_preprocess_stateful(
            F["xq"][s].view(N * T4, DH, fdk), F["xk"][s].view(N * T4, DH, fdk),
            F["xv"][s].view(N * T4, DH, fdv), F["wq"], F["wk"], F["wv"],
            F["a_raw"][s].view(N * T4, DH), F["b_raw"][s].view(N * T4, DH), F["A_log"],
            F["dt_bias"], H=DH, num_seqs=N, out_dtype=bf, outs=qkv,
            conv_state_in=hist[s % 2], conv_state_out=hist[1 - s % 2])
        gdn.gdn_decode_multi(qkv["q"].view(N, T4, DH, fdk), qkv["k"].view(N, T4, DH, fdk),
                             qkv["v"].view(N, T4, DH, fdv), qkv["g"].view(N, T4, DH),
                             qkv["beta"].view(N, T4, DH), F["state"], y=ysep)
        gdn.gdn_output_gate(ysep.view(N * T4, DH, fdv), F["z"][s].view(N * T4, DH, fdv),
                            F["norm_weight"], eps=1e-6, o=of.view(N * T4, DH, fdv))
    for s in range(min(2, S4)):
        smdec(s)
    smms = tm.region(smdec, S4)
    fm_tok = T4 * heads * ((2 * fdk + fdv) * 2 + 8 + fdv * (2 + 2)) + 2 * heads * 3 * (2 * fdk + fdv) * 2
    fmgbs = (f_state + fm_tok) / (fmms * 1e-3) / 1e9
    decode["fused_multi_token"] = {
        "workload": f"gdn_fused_decode_multi N=256 H=32 d_k=d_v=128, {T4} tokens per sequence "
                    "per step from the projected streams (bf16 x, z, o)",
        "tokens_per_step": T4, "steps": S4, "us_per_step": round(fmms * 1e3, 2),
        "GB_s": round(fmgbs, 1), "hbm_frac": round(fmgbs / HBM_PEAK_GBS, 4),
        "separate_kernels_us_per_step": round(smms * 1e3, 2),
        "vs_separate_kernels": round(smms / fmms, 3)}
    log(f"[bench] fused multi-token decode T={T4}: {fmms * 1e3:.1f} us/step ({fmgbs:.0f} GB/s); "
        f"separate kernels {smms * 1e3:.1f} us/step")
    del F, of, hist, qkv, ysep
    torch.cuda.empty_cache()
    return decode


def bench_ceilings(torch, gdn, dev, tm):
    """The HBM stream (1 GiB copy, and in place) and the bf16 matrix-core issue rate, measured
    with the library's own measurement kernels on this device."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    gdn.gdn_mb_stream(a, b)
    copy_ms = tm.region(lambda i: gdn.gdn_mb_stream(a, b), 10)
    inpl_ms = tm.region(lambda i: gdn.gdn_mb_stream(a, a), 10)
    del a, b
    sink = torch.empty(256 * 8, dtype=torch.float32, device=dev)
    iters = 4096
    flops = gdn.gdn_mb_mfma_bf16(sink, iters)
    mf_ms = tm.region(lambda i: gdn.gdn_mb_mfma_bf16(sink, iters), 5)
    res = {"hbm_copy_GBs": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
           "hbm_in_place_GBs": round(2 * n / (inpl_ms * 1e-3) / 1e9, 1),
           "bf16_mfma_TFLOPs": round(flops / (mf_ms * 1e-3) / 1e12, 1),
           "note": "1 GiB read + 1 GiB written per stream call (16-byte nontemporal accesses); "
                   "the matrix-core figure is 2048 workgroups x 4 waves of independent "
                   "32x32x16 bf16 products"}
    log(f"[bench] ceilings: copy {res['hbm_copy_GBs']} GB/s, in place {res['hbm_in_place_GBs']} "
        f"GB/s, bf16 MFMA {res['bf16_mfma_TFLOPs']} TFLOP/s")
    return res


if __name__ == "__main__":
    main()
