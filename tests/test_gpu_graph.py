"""The entry points inside a captured HIP graph: a serving loop captures a decode step (or a
prefill) once and replays it on new inputs copied into the same buffers. Each replay, with the
program's own eager work between the replays, must equal the same call run eagerly, bit for
bit (the library issues kernels only: no memset or copy nodes, no allocations)."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_fused_decode_replays(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    N, H, steps = 8, 4, 4
    _announce(f"graph replay of gdn_fused_decode N={N} H={H}, {steps} steps")
    d = gi.decode_layer_draws(31, steps, N, H)
    bf = lambda a: C.dev(a, True)                                              # noqa: E731
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))            # noqa: E731
    w = [f32(d[x]) for x in ("wq", "wk", "wv")]
    A_log, dt_bias, nw = f32(d["A_log"]), f32(d["dt_bias"]), f32(d["norm_weight"])
    # eager reference over the steps
    hist_e, state_e = bf(d["conv_state"]), f32(d["state"])
    o_ref = []
    for s in range(steps):
        o_ref.append(gdn.gdn_fused_decode(bf(d["xq"][s]), bf(d["xk"][s]), bf(d["xv"][s]), *w,
                                          hist_e, f32(d["a_raw"][s]), f32(d["b_raw"][s]), A_log,
                                          dt_bias, state_e, bf(d["z"][s]), nw))
    # captured step on static buffers
    xq, xk, xv, z = (bf(d[x][0]) for x in ("xq", "xk", "xv", "z"))
    ar, br = f32(d["a_raw"][0]), f32(d["b_raw"][0])
    hist, state = bf(d["conv_state"]), f32(d["state"])
    o = torch.empty_like(o_ref[0])
    step = lambda: gdn.gdn_fused_decode(xq, xk, xv, *w, hist, ar, br, A_log, dt_bias, state, z,  # noqa
                                        nw, o=o)
    hist0, state0 = hist.clone(), state.clone()
    g = _capture(step)           # the warm-up and the capture advanced the buffers: reset them
    hist.copy_(hist0)
    state.copy_(state0)
    for s in range(steps):
        for dst, src in ((xq, d["xq"][s]), (xk, d["xk"][s]), (xv, d["xv"][s]), (z, d["z"][s])):
            dst.copy_(bf(src))
        ar.copy_(f32(d["a_raw"][s]))
        br.copy_(f32(d["b_raw"][s]))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref[s]), f"replay {s}: o differs from the eager call"
    assert torch.equal(state, state_e) and torch.equal(hist, hist_e)


def test_decode_step_and_prefill_replay(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("graph replay of gdn_decode_step and of gdn_chunk_prefill (bf16, B=2 H=4 T=200)")
    di = gi.make_inputs(gi.DECODE, seed=32, N=8, H=4, steps=3)
    bf = lambda a: C.dev(a, True)                                              # noqa: E731
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))            # noqa: E731
    g_ = -torch.rand((3, 8, 4), device="cuda") * 0.3
    b_ = torch.rand((3, 8, 4), device="cuda")
    state_e = f32(di["state"])
    y_ref = [gdn.gdn_decode_step(bf(di["q"][s]), bf(di["k"][s]), bf(di["v"][s]), g_[s].contiguous(),
                                 b_[s].contiguous(), state_e) for s in range(3)]
    q, k, v = bf(di["q"][0]), bf(di["k"][0]), bf(di["v"][0])
    gs, bs = g_[0].clone(), b_[0].clone()
    state = f32(di["state"])
    y = torch.empty_like(y_ref[0])
    graph = _capture(lambda: gdn.gdn_decode_step(q, k, v, gs, bs, state, y=y))
    state.copy_(f32(di["state"]))
    for s in range(3):
        q.copy_(bf(di["q"][s]))
        k.copy_(bf(di["k"][s]))
        v.copy_(bf(di["v"][s]))
        gs.copy_(g_[s])
        bs.copy_(b_[s])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref[s]), f"decode replay {s}"
    assert torch.equal(state, state_e)

    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=33, B=2, H=4, T=200)
    sh = inp["shape"]
    qp, kp, vp = bf(inp["q"]), bf(inp["k"]), bf(inp["v"])
    _, _, _, gp, bp = gdn.gdn_preprocess(None, None, None, None, None, None, f32(inp["a_raw"]),
                                         f32(inp["b_raw"]), f32(inp["A_log"]),
                                         f32(inp["dt_bias"]), H=sh.H)
    S0 = f32(inp["S0"])
    y_e, st_e = gdn.gdn_chunk_prefill(qp, kp, vp, gp, bp, initial_state=S0, num_seqs=sh.num_seqs)
    ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(sh.ntok, sh.num_seqs, sh.H, 128, 128),
                     dtype=torch.uint8, device="cuda")
    yg, stg = torch.empty_like(y_e), torch.empty_like(st_e)
    graph = _capture(lambda: gdn.gdn_chunk_prefill(qp, kp, vp, gp, bp, initial_state=S0,
                                                   final_state=stg, num_seqs=sh.num_seqs, y=yg,
                                                   workspace=ws))
    for rep in range(3):
        yg.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y_e) and torch.equal(stg, st_e), f"prefill replay {rep}"
