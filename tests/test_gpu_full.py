"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark
uses (one call over the whole packed batch). The HIP path computes every output once; the fp64
oracle then checks every (sequence, head) slice, in batches of heads (a slice depends on nothing
outside it, and batching bounds the host memory of the fp64 copies). Each batch prints a line,
so a long comparison is never silent."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _every_slice(inp, res, head_batch):
    sh = inp["shape"]
    seqs = list(range(sh.num_seqs))
    for h0 in range(0, sh.H, head_batch):
        heads = list(range(h0, min(sh.H, h0 + head_batch)))
        print(f"  heads {heads[0]}-{heads[-1]} of {sh.H}, all {len(seqs)} sequences:", flush=True)
        C.check_prefill_sampled(inp, res, seqs=seqs, heads=heads, y_bf16=True)


def test_prefill_pipeline_b4_h16_t4096_full(gpu):
    _announce("bf16 prefill pipeline full: B=4 H=16 T=4096 d=128 bf16, preprocess + prefill + "
              "output gate, every (sequence, head) slice")
    inp = gi.make_inputs(gi.PREFILL, seed=0)
    res = C.gpu_run(inp, y_dtype="bf16")
    _every_slice(inp, res, head_batch=4)


def test_long_context_t65536_full(gpu):
    _announce("long-context prefill full: B=1 H=32 T=65536 d=128 bf16, S0 ~ N(0, 0.01), "
              "every head")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=0)
    res = C.gpu_run(inp, y_dtype="bf16")
    _every_slice(inp, res, head_batch=16)


def test_varlen_64_seqs_full(gpu):
    _announce("varlen prefill full: 64 packed sequences, log-uniform lengths [128, 32768], H=16, "
              "every (sequence, head) slice")
    inp = gi.make_inputs(gi.VARLEN, seed=0)
    res = C.gpu_run(inp, y_dtype="bf16")
    _every_slice(inp, res, head_batch=2)


def test_decode_n256_100_steps_full(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("batched decode full: N=256 H=32 d=128, 100 steps, fp32 state in place, every head")
    inp = gi.make_inputs(gi.DECODE, seed=0)
    sh = inp["shape"]
    S_, N, H = sh.steps, sh.num_seqs, sh.H
    state = C.dev(inp["state"])
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))  # noqa: E731
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None,
                                          f32(inp["a_raw"].reshape(S_ * N, H)),
                                          f32(inp["b_raw"].reshape(S_ * N, H)),
                                          f32(inp["A_log"]), f32(inp["dt_bias"]), H=H)
    g = g.view(S_, N, H)
    beta = beta.view(S_, N, H)
    q, k, v = C.dev(inp["q"], True), C.dev(inp["k"], True), C.dev(inp["v"], True)
    y = torch.empty((S_, N, H, sh.dv), dtype=torch.bfloat16, device="cuda")
    for s in range(S_):
        gdn.gdn_decode_step(q[s], k[s], v[s], g[s], beta[s], state, y=y[s])
    torch.cuda.synchronize()
    y_all = y.view(torch.int16).cpu().numpy().view(np.uint16)      # [S, N, H, dv] bf16 bits
    S_all = state.cpu().numpy()
    del q, k, v, y, state
    # the oracle: sequence n is its S_ decode tokens in order
    cu = np.arange(0, N * S_ + 1, S_).astype(np.int32)
    hb = 8
    for h0 in range(0, H, hb):
        hs = slice(h0, h0 + hb)
        perm = lambda a: np.ascontiguousarray(np.swapaxes(a[:, :, hs], 0, 1).reshape(N * S_, -1, *a.shape[3:]))  # noqa
        qq = gi.as_f64(perm(inp["q"]), True)
        kk = gi.as_f64(perm(inp["k"]), True)
        vv = gi.as_f64(perm(inp["v"]), True)
        _, al, be = C.oracle.gates(perm(inp["a_raw"]).astype(np.float64),
                                   perm(inp["b_raw"]).astype(np.float64),
                                   inp["A_log"][hs].astype(np.float64),
                                   inp["dt_bias"][hs].astype(np.float64))
        y_ref, S_ref = C.oracle.recurrence(qq, kk, vv, al, be,
                                           inp["state"][:, hs].astype(np.float64), cu)
        y_got = gi.as_f64(perm(y_all), True)
        ey = C.assert_close("y", y_got, y_ref, True, stored_bf16=True, cu=cu, H=hb)
        es = C.assert_close("S", S_all[:, hs].astype(np.float64), S_ref, True, state=True)
        print(f"  heads {h0}-{h0 + hb - 1}: every sequence, max slice rel L2 y {ey:.2e} "
              f"S {es:.2e}, max |y - y_ref| {C.max_abs(y_got, y_ref):.3e}", flush=True)
