"""GPU parity of the HIP path against the fp64 oracle (reduced sizes: several chunks,
ragged tails, empty and short sequences). Every case prints its name before touching the GPU."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _compare_prefill(inp, res, ref, sub, y_bf16):
    sh = inp["shape"]
    bf = sh.bf16
    tok, heads, seqs = sub["tok"], sub["heads"], sub["seqs"]
    cu, H = sub["cu"], sub["H"]
    report = {}
    if sh.conv:
        for key in ("q", "k", "v"):
            report[key] = C.assert_close(key, C.gpu_slice(res[key], tok, heads), ref[key], True,
                                         stored_bf16=True, cu=cu, H=H)
    for key in ("g", "beta"):
        got = C.gpu_slice(res[key], tok, heads)
        err = np.abs(got - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30)
        assert err < 1e-5, f"{key}: {err}"
    report["y"] = C.assert_close("y", C.gpu_slice(res["y"], tok, heads), ref["y"], bf,
                                 stored_bf16=y_bf16, cu=cu, H=H)
    if res.get("ST") is not None:
        report["ST"] = C.assert_close("ST", C.gpu_state_slice(res["ST"], seqs, heads), ref["ST"], bf,
                                      state=True)
    if "o" in res:
        # against the plain oracle; the allowance for the pipeline's bf16 storage of q, k, v
        # and y is derived in gdn_cases.o_allowance
        report["o"], report["o_max_abs"] = C.check_o(C.gpu_slice(res["o"], tok, heads), sub,
                                                     ref, y_bf16)
    print("  max slice rel L2:", {k: f"{v:.2e}" for k, v in report.items()}, flush=True)


CASES = [
    # (workload, overrides, y dtype)
    (gi.TINY_FP32, {}, "f32"),
    (gi.TINY_FP32, dict(T=200, d=128), "f32"),
    (gi.TINY_FP32, dict(B=3, T=130, d=64), "f32"),
    (gi.PREFILL, dict(B=2, H=3, T=200), "f32"),
    (gi.PREFILL, dict(B=2, H=3, T=200), "bf16"),
    (gi.PREFILL, dict(B=1, H=2, T=70, d=64), "f32"),
    (gi.LONG_CONTEXT, dict(H=2, T=1000), "f32"),
    # d_k = 128, d_v = 64 on the matrix-core path: two 32-column slices per head
    (gi.PREFILL, dict(B=2, H=2, T=150, dv=64), "bf16"),
    (gi.LONG_CONTEXT, dict(H=3, T=330, dv=64), "f32"),
    (gi.VARLEN, dict(H=2, lengths=[0, 1, 3, 63, 64, 65, 200, 0, 130]), "f32"),
    (gi.VARLEN, dict(H=2, nseq=5, lmax=600), "bf16"),
    # 256 or more (sequence, head) pairs: the sliced scan's largest grids (the full-row scan runs
    # these only with the output gate in the fused prefill)
    (gi.PREFILL, dict(B=64, H=4, T=200), "bf16"),
    (gi.PREFILL, dict(B=64, H=4, T=260), "f32"),
    (gi.VARLEN, dict(H=8, nseq=40, lmax=400), "bf16"),
]


@pytest.mark.parametrize("workload,ov,ydt", CASES,
                         ids=[f"{gi.TAGS[w]}-{o}-{y}" for w, o, y in CASES])
def test_prefill_pipeline_parity(gpu, workload, ov, ydt):
    _announce(f"prefill {gi.TAGS[workload]} {ov} y={ydt}")
    inp = gi.make_inputs(workload, seed=0, **ov)
    res = C.gpu_run(inp, y_dtype=ydt)
    sub = C.subset(inp)
    ref = C.oracle_run(sub)
    _compare_prefill(inp, res, ref, sub, ydt == "bf16")


@pytest.mark.parametrize("ov,ydt", [(dict(N=8, H=2, steps=6), "f32"),
                                    (dict(N=5, H=3, steps=4, d=64), "bf16")])
def test_decode_steps_parity(gpu, ov, ydt):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce(f"decode {ov} y={ydt}")
    inp = gi.make_inputs(gi.DECODE, seed=0, **ov)
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
    ys = []
    for s in range(S_):
        ys.append(gdn.gdn_decode_step(C.dev(inp["q"][s], True), C.dev(inp["k"][s], True),
                                      C.dev(inp["v"][s], True), g[s].contiguous(),
                                      beta[s].contiguous(), state, y_dtype=ydt))
    torch.cuda.synchronize()
    # oracle: each sequence is the S-token sequence of its decode steps
    perm = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape(N * S_, *a.shape[2:]))  # noqa
    q = perm(gi.as_f64(inp["q"], True))
    k = perm(gi.as_f64(inp["k"], True))
    v = perm(gi.as_f64(inp["v"], True))
    og, al, be = C.oracle.gates(perm(inp["a_raw"].astype(np.float64)),
                                perm(inp["b_raw"].astype(np.float64)),
                                inp["A_log"].astype(np.float64), inp["dt_bias"].astype(np.float64))
    cu = np.arange(0, N * S_ + 1, S_)
    y_ref, S_ref = C.oracle.recurrence(q, k, v, al, be, inp["state"].astype(np.float64), cu)
    y_gpu = np.stack([C.host(y) for y in ys], axis=1).reshape(N * S_, H, sh.dv)
    C.assert_close("y", y_gpu, y_ref, True, stored_bf16=(ydt == "bf16"), cu=cu, H=H)
    C.assert_close("S", C.host(state), S_ref, True, state=True)


def test_prefill_is_deterministic(gpu):
    _announce("determinism: bf16 prefill pipeline B=2 H=2 T=150")
    inp = gi.make_inputs(gi.PREFILL, seed=3, B=2, H=2, T=150)
    a = C.gpu_run(inp, y_dtype="f32")
    b = C.gpu_run(inp, y_dtype="f32")
    for key in ("q", "k", "v", "y", "ST", "o"):
        assert np.array_equal(C.host(a[key]), C.host(b[key])), key


@pytest.mark.parametrize("nseq,bf16", [(300, True), (1300, True), (1300, False)])
def test_prefill_many_sequences(gpu, nseq, bf16):
    """Many short packed sequences (empty ones included): more than 256 runs the chunk
    table's scan over several rounds, more than 1024 skips its longest-first ordering."""
    L = C.many_short_lengths(11, nseq)
    _announce(f"prefill {nseq} packed sequences, lengths 0..70, H=2, bf16={bf16}")
    if bf16:   # the full pipeline on the matrix-core path, with S0
        inp = gi.make_inputs(gi.VARLEN, seed=12, H=2, lengths=L)
    else:      # fp32 q, k, v with d = 64 on the fp32 path
        inp = gi.make_inputs(gi.TINY_FP32, seed=12, H=2, lengths=L)
    res = C.gpu_run(inp, y_dtype="bf16" if bf16 else "f32")
    C.check_prefill_sampled(inp, res, C.sampled_seqs(L, 12), [0, 1], y_bf16=bf16)


@pytest.mark.parametrize("bf16", [True, False])
def test_prefill_final_state_in_place(gpu, bf16):
    """final_state may be the initial_state buffer (updated in place): the same y and S_T, bit
    for bit, as with a separate output buffer (the scalar-decay and per-channel-decay
    prefills)."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    L = [130, 0, 64, 7]
    _announce(f"prefill with final_state = initial_state, lengths {L} H=2 bf16={bf16}")
    inp = gi.make_inputs(gi.LONG_CONTEXT if bf16 else gi.TINY_FP32, seed=15, H=2, lengths=L)
    sh = inp["shape"]
    S0 = gi.make_inputs(gi.LONG_CONTEXT, seed=15, B=len(L), H=2, T=1, d=sh.dk)["S0"]
    q, k, v = (C.dev(inp[x], bf16) for x in ("q", "k", "v"))
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))          # noqa: E731
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None, f32(inp["a_raw"]),
                                          f32(inp["b_raw"]), f32(inp["A_log"]),
                                          f32(inp["dt_bias"]), H=sh.H)
    cu = C.dev(inp["cu_seqlens"])
    kw = dict(cu_seqlens=cu, cu_seqlens_host=inp["cu_seqlens"], num_seqs=len(L))
    y1, ST1 = gdn.gdn_chunk_prefill(q, k, v, g, beta, initial_state=f32(S0), **kw)
    S = f32(S0)
    y2, ST2 = gdn.gdn_chunk_prefill(q, k, v, g, beta, initial_state=S, final_state=S, **kw)
    torch.cuda.synchronize()
    assert ST2.data_ptr() == S.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(ST1, S)
    # the per-channel-decay prefill likewise
    gk = f32(gi.kda_log_decay_draw(15, sh.ntok, sh.H, sh.dk))
    y1, ST1 = gdn.gdn_kda_chunk_prefill(q, k, v, gk, beta, initial_state=f32(S0), **kw)
    S = f32(S0)
    y2, ST2 = gdn.gdn_kda_chunk_prefill(q, k, v, gk, beta, initial_state=S, final_state=S, **kw)
    torch.cuda.synchronize()
    assert ST2.data_ptr() == S.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(ST1, S)


def test_full_row_scan_equals_sliced_scan(gpu):
    """The full-row scan (all 128 d_v columns per workgroup; the fused prefill takes it, with the
    output gate in its epilogue, for 256 or more (sequence, head) pairs of equal length) forms
    every product of the sliced scan that gdn_chunk_prefill runs from the same operands in the
    same order, so the y and final state the fused call exports equal, bit for bit,
    gdn_chunk_prefill's on the exported q, k, v, g, beta and the same S0."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("full-row scan (fused prefill, B=64 H=4, 256 pairs, S0) against the sliced scan")
    inp = gi.make_inputs(gi.PREFILL, seed=5, B=64, H=4, T=200)
    inp["S0"] = np.random.default_rng(5).standard_normal((64, 4, 128, 128)) * 0.1
    fused = C.gpu_run_fused(inp)
    y, st = gdn.gdn_chunk_prefill(fused["q"], fused["k"], fused["v"], fused["g"], fused["beta"],
                                  initial_state=C.dev(inp["S0"].astype(np.float32)),
                                  num_seqs=64, y_dtype="bf16")
    torch.cuda.synchronize()
    assert y.dtype == fused["y"].dtype and torch.equal(y, fused["y"]), "y differs"
    assert torch.equal(st, fused["ST"]), "final state differs"
    print("  full-row scan's y and S_T equal the sliced scan's bit for bit", flush=True)
