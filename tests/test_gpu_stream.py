"""GPU parity of the streaming entry points against the fp64 oracle:
  * gdn_preprocess_stateful (the conv with a carried history, in and out);
  * gdn_decode_multi (T tokens per sequence in one pass over each state, with the state
    after every token on request);
  * both chained after a prefill: a prompt prefilled with its conv history and state carried
    out, then multi-token decode steps, against the oracle over each whole sequence.
Sources: reading notes "Qwen3.8-Next 架构设计：评测、效率与训练稳定性", section 2.1.1,
eqs. (1)-(10); the design summary "设计 LLM 架构" (causal depthwise short conv; MTP drafts)."""
import sys

import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _f32(a):
    return C.dev(np.ascontiguousarray(a, dtype=np.float32))


# ----------------------------------------------------------------------------- preprocess
@pytest.mark.parametrize("with_hist", [True, False])
@pytest.mark.parametrize("dims", [(128, 128), (64, 128), (128, 64)])
def test_preprocess_stateful_varlen(gpu, with_hist, dims):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    dk, dv = dims
    lengths = [0, 1, 2, 3, 67, 130, 1, 64]      # empty and shorter-than-history sequences
    _announce(f"preprocess_stateful lengths={lengths} H=2 dk={dk} dv={dv} hist={with_hist}")
    inp = gi.make_inputs(gi.VARLEN, seed=3, H=2, dk=dk, dv=dv, lengths=lengths)
    sh = inp["shape"]
    H, cu = sh.H, inp["cu_seqlens"]
    hist = gi.conv_state_draw(5, sh.num_seqs, H, dk, dv) if with_hist else None
    q, k, v, g, beta, hout = gdn.gdn_preprocess_stateful(
        C.dev(inp["xq"], True), C.dev(inp["xk"], True), C.dev(inp["xv"], True),
        _f32(inp["wq"]), _f32(inp["wk"]), _f32(inp["wv"]), _f32(inp["a_raw"]),
        _f32(inp["b_raw"]), _f32(inp["A_log"]), _f32(inp["dt_bias"]), H=H,
        conv_state_in=None if hist is None else C.dev(hist, True), conv_state_out=True,
        cu_seqlens=C.dev(cu), num_seqs=sh.num_seqs, l2_eps=C.L2_EPS, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    xs = [gi.as_f64(inp[x], True) for x in ("xq", "xk", "xv")]
    hin = None if hist is None else gi.as_f64(hist, True)
    rq, rk, rv, rh = oracle.preprocess_stateful(*xs, inp["wq"], inp["wk"], inp["wv"], cu, H,
                                                conv_state_in=hin, l2_eps=C.L2_EPS)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        C.assert_close(name, C.host(got), ref, True, stored_bf16=True, cu=cu, H=H)
    rg, _, rb = oracle.gates(inp["a_raw"], inp["b_raw"], inp["A_log"], inp["dt_bias"])
    assert np.abs(C.host(g) - rg).max() / np.abs(rg).max() < 1e-5
    assert np.abs(C.host(beta) - rb).max() < 1e-5
    # the carried history is raw input moved, bit for bit
    assert np.array_equal(C.host(hout), rh)


# ----------------------------------------------------------------------------- decode
def _decode_case(N, T, H, dk, dv, bf16, seed):
    """Raw draws of one multi-token decode step (drawn as in the batched decode workload)."""
    inp = gi.make_inputs(gi.DECODE, seed=seed, N=N, H=H, dk=dk, dv=dv, steps=1, tokens=T)
    q, k, v = (inp[x][0].reshape(N, T, H, -1) for x in "qkv")   # [N, T, H, d] bf16 bits
    if not bf16:                                              # fp32 inputs: the same values
        q, k, v = (gi.bf16_bits_to_f32(x) for x in (q, k, v))
    return inp, q, k, v


@pytest.mark.parametrize("T", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("dims,bf16", [((128, 128), True), ((64, 128), True), ((128, 64), False),
                                       ((64, 64), False)])
def test_decode_multi_against_token_by_token(gpu, T, dims, bf16):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    dk, dv = dims
    N, H = 5, 3
    _announce(f"decode_multi N={N} T={T} H={H} dk={dk} dv={dv} bf16={bf16}")
    inp, q, k, v = _decode_case(N, T, H, dk, dv, bf16, seed=T)
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None,
                                          _f32(inp["a_raw"][0].reshape(N * T, H)),
                                          _f32(inp["b_raw"][0].reshape(N * T, H)),
                                          _f32(inp["A_log"]), _f32(inp["dt_bias"]), H=H)
    state = C.dev(inp["state"])
    y, steps = gdn.gdn_decode_multi(C.dev(q, bf16), C.dev(k, bf16), C.dev(v, bf16),
                                    g.view(N, T, H), beta.view(N, T, H), state,
                                    y_dtype=torch.float32, step_states=True)
    torch.cuda.synchronize()
    qq, kk, vv = (gi.as_f64(x, bf16).reshape(N * T, H, -1) for x in (q, k, v))
    _, al, be = oracle.gates(inp["a_raw"][0].reshape(N * T, H), inp["b_raw"][0].reshape(N * T, H),
                             inp["A_log"], inp["dt_bias"])
    cu = np.arange(0, N * T + 1, T)
    S0 = inp["state"].astype(np.float64)
    y_ref, S_ref = oracle.recurrence(qq, kk, vv, al, be, S0, cu)
    C.assert_close("y", C.host(y).reshape(N * T, H, dv), y_ref, bf16, cu=cu, H=H)
    C.assert_close("state", C.host(state), S_ref, bf16, state=True)
    got_steps = C.host(steps)                                  # [N, T, H, dk, dv]
    for t in range(T):                                         # state after the first t+1 tokens
        sel = (np.arange(N)[:, None] * T + np.arange(t + 1)[None, :]).ravel()
        _, S_t = oracle.recurrence(qq[sel], kk[sel], vv[sel], al[sel], be[sel], S0,
                                   np.arange(0, N * (t + 1) + 1, t + 1))
        C.assert_close(f"step_states[{t}]", got_steps[:, t], S_t, bf16, state=True)


def test_decode_multi_one_token_matches_decode_step(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    N, H = 16, 4
    _announce(f"decode_multi T=1 vs decode_step N={N} H={H}")
    inp, q, k, v = _decode_case(N, 1, H, 128, 128, True, seed=11)
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None,
                                          _f32(inp["a_raw"][0].reshape(N, H)),
                                          _f32(inp["b_raw"][0].reshape(N, H)),
                                          _f32(inp["A_log"]), _f32(inp["dt_bias"]), H=H)
    s1, s2 = C.dev(inp["state"]), C.dev(inp["state"])
    y1 = gdn.gdn_decode_step(C.dev(q[:, 0], True), C.dev(k[:, 0], True), C.dev(v[:, 0], True),
                             g.view(N, H), beta.view(N, H), s1, y_dtype=torch.float32)
    y2, _ = gdn.gdn_decode_multi(C.dev(q, True), C.dev(k, True), C.dev(v, True), g.view(N, 1, H),
                                 beta.view(N, 1, H), s2, y_dtype=torch.float32)
    torch.cuda.synchronize()
    # same arithmetic up to evaluation order: agreement far inside the parity bar
    assert np.abs(C.host(y1) - C.host(y2)[:, 0]).max() < 1e-5
    assert np.abs(C.host(s1) - C.host(s2)).max() < 1e-5


# ----------------------------------------------------------------------------- prefill + decode
def test_prefill_then_multi_token_decode_equals_whole_sequences(gpu):
    """Prompt prefilled with conv history and state carried out, then 3 decode steps of 4 tokens
    with both carried from step to step: every output equals the oracle's over the whole
    sequences (prompt + drafts) processed at once."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    N, H, steps, T = 3, 2, 3, 4
    prompts = [100, 64, 2]
    _announce(f"prefill {prompts} then {steps} decode steps of T={T}, H={H}, d=128")
    s = gi.make_stream_inputs(7, N, H, prompts, steps, T)
    cu = s["cu_seqlens"]
    bf = torch.bfloat16
    w = [_f32(s[x]) for x in ("wq", "wk", "wv")]
    gate_p = [_f32(s["A_log"]), _f32(s["dt_bias"])]
    # prompt: preprocess with the history carried out, prefill with the state carried out
    q, k, v, g, beta, hist = gdn.gdn_preprocess_stateful(
        C.dev(s["xq"], True), C.dev(s["xk"], True), C.dev(s["xv"], True), *w,
        _f32(s["a_raw"]), _f32(s["b_raw"]), *gate_p, H=H, conv_state_out=True,
        cu_seqlens=C.dev(cu), num_seqs=N, out_dtype=bf)
    y_p, state = gdn.gdn_chunk_prefill(q, k, v, g, beta, cu_seqlens=C.dev(cu), cu_seqlens_host=cu,
                                       num_seqs=N, y_dtype=torch.float32)
    ys = []
    for st in range(steps):
        dq, dk_, dv_, dg, db, hist_next = gdn.gdn_preprocess_stateful(
            C.dev(s["dxq"][st].reshape(N * T, H, -1), True),
            C.dev(s["dxk"][st].reshape(N * T, H, -1), True),
            C.dev(s["dxv"][st].reshape(N * T, H, -1), True), *w,
            _f32(s["da_raw"][st].reshape(N * T, H)), _f32(s["db_raw"][st].reshape(N * T, H)),
            *gate_p, H=H, conv_state_in=hist, conv_state_out=True, num_seqs=N, out_dtype=bf)
        hist = hist_next
        y_d, _ = gdn.gdn_decode_multi(dq.view(N, T, H, -1), dk_.view(N, T, H, -1),
                                      dv_.view(N, T, H, -1), dg.view(N, T, H), db.view(N, T, H),
                                      state, y_dtype=torch.float32)
        ys.append(C.host(y_d))
    torch.cuda.synchronize()

    # oracle: each sequence = prompt tokens then its decode tokens, in one pass
    rows_x = {x: [] for x in ("xq", "xk", "xv", "a_raw", "b_raw")}
    lens = []
    for n in range(N):
        lo, hi = cu[n], cu[n + 1]
        for x in rows_x:
            part = [s[x][lo:hi]] + [s["d" + x][st][n] for st in range(steps)]
            rows_x[x].append(np.concatenate(part, axis=0))
        lens.append(hi - lo + steps * T)
    whole = {x: np.concatenate(v, axis=0) for x, v in rows_x.items()}
    cu_w = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    xq, xk, xv = (gi.as_f64(whole[x], True) for x in ("xq", "xk", "xv"))
    rq, rk, rv = oracle.preprocess(xq, xk, xv, s["wq"], s["wk"], s["wv"], cu_w, H, C.L2_EPS)
    # the HIP path stores q, k, v in bf16 between its kernels: the oracle rounds them the same way
    rq, rk, rv = oracle.round_bf16(rq), oracle.round_bf16(rk), oracle.round_bf16(rv)
    _, al, be = oracle.gates(whole["a_raw"], whole["b_raw"], s["A_log"], s["dt_bias"])
    y_ref, S_ref = oracle.recurrence(rq, rk, rv, al, be, None, cu_w)
    # gather the HIP outputs in the same order
    y_got = []
    yp = C.host(y_p)
    for n in range(N):
        y_got.append(yp[cu[n]:cu[n + 1]])
        for st in range(steps):
            y_got.append(ys[st][n])
    y_got = np.concatenate(y_got, axis=0)
    C.assert_close("y (prompt + decode)", y_got, y_ref, True, cu=cu_w, H=H)
    C.assert_close("final state", C.host(state), S_ref, True, state=True)
