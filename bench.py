"""Benchmark of the Gated DeltaNet token mixer on one MI355X.

A step is one pass of the prefill token mixer over the bf16 workload B=4, H=16, T=4096,
d_k=d_v=128 (preprocess -> chunked prefill -> output gate), inputs resident in HBM.
`value` is that pipeline's throughput in Mtok/s (a token spans all 16 heads). The decode
half of the metric (256 sequences x 32 heads, d=128, 100 steps with fresh tokens, fp32 state
updated in place) is timed in the same run and reported under "decode", with the
multi-token decode (4 tokens per sequence per step, as in MTP verification) beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    from gated_deltanet_recurrence_chunked_amd import inputs as gi

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def d(a, bf16=False):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # ------------------------------------------------------------------ prefill workload
    log("[bench] generating bf16 prefill inputs B=4 H=16 T=4096 d=128")
    inp = gi.make_inputs(gi.PREFILL, seed=0)
    sh = inp["shape"]
    H, dk, dv, ntok, nseq = sh.H, sh.dk, sh.dv, sh.ntok, sh.num_seqs
    X = dict(xq=d(inp["xq"], True), xk=d(inp["xk"], True), xv=d(inp["xv"], True),
             wq=d(inp["wq"]), wk=d(inp["wk"]), wv=d(inp["wv"]), a_raw=d(inp["a_raw"]),
             b_raw=d(inp["b_raw"]), A_log=d(inp["A_log"]), dt_bias=d(inp["dt_bias"]),
             z=d(inp["z"], True), nw=d(inp["norm_weight"]))
    bf = torch.bfloat16
    outs = dict(q=torch.empty((ntok, H, dk), dtype=bf, device=dev),
                k=torch.empty((ntok, H, dk), dtype=bf, device=dev),
                v=torch.empty((ntok, H, dv), dtype=bf, device=dev),
                g=torch.empty((ntok, H), dtype=torch.float32, device=dev),
                beta=torch.empty((ntok, H), dtype=torch.float32, device=dev))
    y = torch.empty((ntok, H, dv), dtype=bf, device=dev)
    o = torch.empty((ntok, H, dv), dtype=bf, device=dev)
    ws_n = gdn.gdn_chunk_prefill_workspace_size(ntok, nseq, H, dk, dv, bf)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    ev = {}

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(name, []).append(e)

    def step(timed):
        if timed:
            mark("pre0")
        gdn.gdn_preprocess(X["xq"], X["xk"], X["xv"], X["wq"], X["wk"], X["wv"], X["a_raw"],
                           X["b_raw"], X["A_log"], X["dt_bias"], H=H, num_seqs=nseq,
                           out_dtype=bf, outs=outs)
        if timed:
            mark("pre1")
        gdn.gdn_chunk_prefill(outs["q"], outs["k"], outs["v"], outs["g"], outs["beta"],
                              num_seqs=nseq, y=y, workspace=ws, output_final_state=False)
        if timed:
            mark("pf1")
        gdn.gdn_output_gate(y, X["z"], X["nw"], eps=1e-6, o=o)
        if timed:
            mark("og1")

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step(True)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    def avg(a, b):
        return float(np.mean([x.elapsed_time(y_) for x, y_ in zip(ev[a], ev[b])]))

    t_pre = avg("pre0", "pre1")
    t_pf = avg("pre1", "pf1")
    t_og = avg("pf1", "og1")
    mtoks = ntok / (ms_step * 1e-3) / 1e6
    log(f"[bench] pipeline {ms_step * 1e3:.1f} us/step = {mtoks:.1f} Mtok/s "
        f"(preprocess {t_pre * 1e3:.1f} us, prefill {t_pf * 1e3:.1f} us, gate {t_og * 1e3:.1f} us)")

    # the same token mixer through the fused entry point (conv, SiLU, L2Norm and gates inside
    # the per-chunk kernel; bit-identical outputs)
    ws_f = torch.empty(gdn.gdn_fused_prefill_workspace_size(ntok, nseq, H, dk, dv),
                       dtype=torch.uint8, device=dev)
    o_f = torch.empty_like(o)

    def fstep():
        gdn.gdn_fused_prefill(X["xq"], X["xk"], X["xv"], X["wq"], X["wk"], X["wv"], X["a_raw"],
                              X["b_raw"], X["A_log"], X["dt_bias"], X["z"], X["nw"], H=H,
                              num_seqs=nseq, output_final_state=False, o=o_f, workspace=ws_f)
    for _ in range(10):
        fstep()
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        fstep()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_fused = t_start.elapsed_time(t_end) / args.steps
    fused_prefill = {"workload": "gdn_fused_prefill at B=4 H=16 T=4096 d=128 (bf16 x, z, o)",
                     "calls": args.steps, "us_per_call": round(ms_fused * 1e3, 1),
                     "Mtok_s": round(ntok / (ms_fused * 1e-3) / 1e6, 2),
                     "vs_separate_kernels": round(ms_step / ms_fused, 3)}
    log(f"[bench] fused prefill {ms_fused * 1e3:.1f} us/call = {fused_prefill['Mtok_s']} Mtok/s "
        f"({ms_step / ms_fused:.2f}x the separate kernels)")
    del ws_f, o_f

    pf_bytes, pf_flops = prefill_algorithmic(H, dk, dv, ntok, nseq, False, False)
    pre_bytes = ntok * H * (2 * dk + dv) * (2 + 2) + ntok * H * 16 + 3 * H * 128 * 4 * 4
    og_bytes = ntok * H * dv * (2 + 2 + 2)
    kernels = {
        "gdn_preprocess": dict(us=t_pre * 1e3, GBs=pre_bytes / (t_pre * 1e-3) / 1e9),
        "gdn_chunk_prefill": dict(us=t_pf * 1e3, GBs=pf_bytes / (t_pf * 1e-3) / 1e9,
                                  TFLOPs=pf_flops / (t_pf * 1e-3) / 1e12,
                                  mfma_frac=pf_flops / (t_pf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                  Mtok_s=ntok / (t_pf * 1e-3) / 1e6),
        "gdn_output_gate": dict(us=t_og * 1e3, GBs=og_bytes / (t_og * 1e-3) / 1e9),
    }
    pf_gbs = pf_bytes / (t_pf * 1e-3) / 1e9
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_gdn_chunk_prefill_B4_H16_T4096_d128.json")
    if os.path.exists(tpath):
        from gated_deltanet_recurrence_chunked_amd import rocprof_summary
        with open(tpath) as f:
            rec = json.load(f)
        if rec.get("kernel_source_sha256") == rocprof_summary.prefill_source_sha():
            traffic = int(rec["gdn_chunk_prefill_bytes_per_call"])
    roofline = {"kernel": "gdn_chunk_prefill (chunk_prep_kernel + chunk_scan_kernel)",
                "bound": "hbm", "achieved": round(pf_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(pf_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "algorithmic_bytes_per_launch": pf_bytes,
                "mfma": {"achieved_TFLOPs": round(pf_flops / (t_pf * 1e-3) / 1e12, 1),
                         "peak_TFLOPs": BF16_PEAK_TFLOPS,
                         "frac": round(pf_flops / (t_pf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "algorithmic_flops_per_launch": pf_flops}}
    # ------------------------------------------------------------------ backward (training)
    backward = None
    if not args.no_backward:
        gen = torch.Generator(device=dev).manual_seed(0)
        dy = torch.randn((ntok, H, dv), generator=gen, device=dev).to(bf)
        ws_b = torch.empty(gdn.gdn_chunk_backward_workspace_size(ntok, nseq, H, dk, dv),
                           dtype=torch.uint8, device=dev)

        def bstep():
            return gdn.gdn_chunk_backward(outs["q"], outs["k"], outs["v"], outs["g"],
                                          outs["beta"], dy, num_seqs=nseq, workspace=ws_b,
                                          want_dinitial_state=False)
        for _ in range(3):
            bstep()
        torch.cuda.synchronize()
        nb = 10
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(nb):
            bstep()
        b1.record(stream)
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / nb
        backward = {"workload": "gdn_chunk_backward at B=4 H=16 T=4096 d=128 (bf16 q, k, v, dy; "
                                "fp32 gradients of q, k, v, g, beta)",
                    "calls": nb, "us_per_call": round(bms * 1e3, 1),
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
        ws_k = torch.empty(int(gdn.lib().gdn_kda_chunk_prefill_workspace_size(ntok, nseq, H, dk)),
                           dtype=torch.uint8, device=dev)

        def kstep():
            return gdn.gdn_kda_chunk_prefill(outs["q"], outs["k"], outs["v"], gk, outs["beta"],
                                             num_seqs=nseq, y=y, workspace=ws_k,
                                             output_final_state=False)
        for _ in range(3):
            kstep()
        torch.cuda.synchronize()
        nk = 10
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(nk):
            kstep()
        b1.record(stream)
        torch.cuda.synchronize()
        kms = b0.elapsed_time(b1) / nk
        kda = {"workload": "gdn_kda_chunk_prefill at B=4 H=16 T=4096 d=128 (bf16 q, k, v, y; "
                           "per-channel fp32 log-decays)",
               "calls": nk, "us_per_call": round(kms * 1e3, 1),
               "Mtok_s": round(ntok / (kms * 1e-3) / 1e6, 2),
               "vs_scalar_decay_prefill": round(kms / t_pf, 2)}
        log(f"[bench] per-channel-decay prefill {kms * 1e3:.1f} us/call ({kda['Mtok_s']} Mtok/s)")
        del gk, ws_k

    del X, outs, y, o, ws
    torch.cuda.empty_cache()

    # ------------------------------------------------------------------ decode workload
    decode = None
    if not args.no_decode:
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
        for s in range(min(3, S_)):      # warm-up (advances the state; timing is unaffected)
            gdn.gdn_decode_step(qd[s], kd[s], vd[s], gd[s], bd[s], state, y=yd[s])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(S_):
            gdn.gdn_decode_step(qd[s], kd[s], vd[s], gd[s], bd[s], state, y=yd[s])
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / S_
        heads = N * DH
        state_bytes = heads * dsh.dk * dsh.dv * 4 * 2
        tok_bytes = heads * ((2 * dsh.dk + dsh.dv) * 2 + 8 + dsh.dv * 2)
        gbs = (state_bytes + tok_bytes) / (dms * 1e-3) / 1e9
        decode = {"workload": "decode N=256 H=32 d_k=d_v=128, fp32 state in place, bf16 tokens",
                  "steps": S_, "us_per_step": round(dms * 1e3, 2), "GB_s": round(gbs, 1),
                  "state_only_GB_s": round(state_bytes / (dms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                  "bytes_per_step": state_bytes + tok_bytes}
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
        for s in range(min(3, S4)):
            gdn.gdn_decode_multi(qm[s], km[s], vm[s], gm[s], bm[s], state, y=ym[s])
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(S4):
            gdn.gdn_decode_multi(qm[s], km[s], vm[s], gm[s], bm[s], state, y=ym[s])
        e1.record(stream)
        torch.cuda.synchronize()
        mms = e0.elapsed_time(e1) / S4
        mtok_bytes = T4 * tok_bytes
        mgbs = (state_bytes + mtok_bytes) / (mms * 1e-3) / 1e9
        decode["multi_token"] = {
            "workload": f"decode N=256 H=32 d_k=d_v=128, {T4} tokens per sequence per step "
                        "(gdn_decode_multi), fp32 state in place, bf16 tokens",
            "tokens_per_step": T4, "steps": S4, "us_per_step": round(mms * 1e3, 2),
            "Mtok_s": round(N * T4 / (mms * 1e-3) / 1e6, 3), "GB_s": round(mgbs, 1),
            "hbm_frac": round(mgbs / HBM_PEAK_GBS, 4), "bytes_per_step": state_bytes + mtok_bytes,
            "vs_single_token_steps": round(T4 * dms / mms, 2)}
        log(f"[bench] multi-token decode T={T4}: {mms * 1e3:.1f} us/step, {mgbs:.0f} GB/s "
            f"({mgbs / HBM_PEAK_GBS:.1%} of HBM), {T4 * dms / mms:.2f}x the tokens/s of T=1 steps")
        del state, qm, km, vm, gm, bm, ym
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ fused decode step
    if decode is not None:
        S_ = args.decode_steps
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
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(S_):
            fdec(s)
        e1.record(stream)
        torch.cuda.synchronize()
        fms = e0.elapsed_time(e1) / S_
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
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(S_ - S_ % 2):
            sdec(s)
        e1.record(stream)
        torch.cuda.synchronize()
        sms = e0.elapsed_time(e1) / max(1, S_ - S_ % 2)
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
        T4, S4 = 4, max(1, S_ // 4)
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
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(S4):
            fmdec(s)
        e1.record(stream)
        torch.cuda.synchronize()
        fmms = e0.elapsed_time(e1) / S4
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
        torch.cuda.synchronize()
        e0.record(stream)
        for s in range(S4 - S4 % 2):
            smdec(s)
        e1.record(stream)
        torch.cuda.synchronize()
        smms = e0.elapsed_time(e1) / max(1, S4 - S4 % 2)
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

    if args.calibrate_copy:
        n = 1 << 28
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import gdn_cases as C
        nseq_s = nseq
        sub = C.subset(inp, seqs=list(range(nseq_s)))
        threads = oracle.default_threads()
        log(f"[bench] timing the fp64 oracle on {nseq_s} sequence x {H} heads x {sh.lengths[0]} "
            f"tokens with {threads} threads")
        t0 = time.perf_counter()
        C.oracle_run(sub, nthreads=threads)
        dt = time.perf_counter() - t0
        ntok_s = int(sub["cu"][-1])
        cpu = {"value": round(ntok_s / dt / 1e6, 6), "unit": "Mtok/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{nseq_s} of {nseq} sequences ({ntok_s} tokens x {H} heads, d=128): "
                         f"preprocess + gates + recurrence + output gate in fp64, {dt:.1f} s",
               "cpu": platform.processor() or platform.machine()}
        log(f"[bench] oracle {dt:.1f} s -> {cpu['value']} Mtok/s")

    out = {
        "metric": "GDN prefill Mtok/s (H16,d128,T4096) + decode state-update HBM GB/s",
        "value": round(mtoks, 2), "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "bf16 GDN prefill token mixer: preprocess + chunked prefill "
                               "(C=64) + output gate", "B": 4, "H": H, "T": sh.lengths[0],
                   "d_k": dk, "d_v": dv, "tokens_per_step": ntok},
        "kernels": kernels, "roofline": roofline, "decode": decode, "backward": backward,
        "per_channel_decay": kda, "fused_prefill": fused_prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
