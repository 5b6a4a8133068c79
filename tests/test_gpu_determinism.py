"""Run-to-run determinism of the entry points beyond the forward prefill (which
tests/test_gpu_parity.py covers): none of the kernels uses atomics or a reduction whose order
depends on scheduling, so two calls on the same inputs must agree bit for bit."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _f32(a):
    return C.dev(np.ascontiguousarray(a, dtype=np.float32))


def _same(a, b, name):
    import torch
    assert torch.equal(a, b), f"{name} differs between two identical calls"


def test_backward_and_kda_are_deterministic(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("determinism: backward and per-channel decay, lengths [130, 70, 1] H=3 d=128 bf16")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=5, H=3, lengths=[130, 70, 1])
    sh = inp["shape"]
    q, k, v = (C.dev(inp[x], True) for x in ("q", "k", "v"))
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None, _f32(inp["a_raw"]),
                                          _f32(inp["b_raw"]), _f32(inp["A_log"]),
                                          _f32(inp["dt_bias"]), H=sh.H)
    cu = C.dev(inp["cu_seqlens"])
    gd = gi.grad_draws(5, sh.ntok, sh.num_seqs, sh.H, sh.dk, sh.dv, bf16=True)
    dy, dST = C.dev(gd["dy"], True), _f32(gd["dST"])
    S0 = _f32(inp["S0"])
    runs = [gdn.gdn_chunk_backward(q, k, v, g, beta, dy, initial_state=S0, dfinal_state=dST,
                                   cu_seqlens=cu, num_seqs=sh.num_seqs) for _ in range(2)]
    torch.cuda.synchronize()
    for name in runs[0]:
        if runs[0][name] is not None:
            _same(runs[0][name], runs[1][name], name)
    gk = _f32(gi.kda_log_decay_draw(5, sh.ntok, sh.H, sh.dk))
    kda = [gdn.gdn_kda_chunk_prefill(q, k, v, gk, beta, initial_state=S0, cu_seqlens=cu,
                                     num_seqs=sh.num_seqs) for _ in range(2)]
    torch.cuda.synchronize()
    _same(kda[0][0], kda[1][0], "kda y")
    _same(kda[0][1], kda[1][1], "kda S_T")


@pytest.mark.parametrize("T", [1, 4])
def test_fused_and_multi_token_decode_are_deterministic(gpu, T):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    N, H = 16, 4
    _announce(f"determinism: fused decode and multi-token decode N={N} H={H} T={T}")
    d = gi.decode_layer_draws(6, 1, N, H, tokens=T)
    bf = lambda a: C.dev(a, True)                                              # noqa: E731
    outs = []
    for _ in range(2):
        hist, state = bf(d["conv_state"]), _f32(d["state"])
        args = (bf(d["xq"][0]), bf(d["xk"][0]), bf(d["xv"][0]), _f32(d["wq"]), _f32(d["wk"]),
                _f32(d["wv"]), hist, _f32(d["a_raw"][0]), _f32(d["b_raw"][0]), _f32(d["A_log"]),
                _f32(d["dt_bias"]), state, bf(d["z"][0]), _f32(d["norm_weight"]))
        if T == 1:
            o = gdn.gdn_fused_decode(*args)
        else:
            o, _, _ = gdn.gdn_fused_decode_multi(*args)
        outs.append((o, state, hist))
    torch.cuda.synchronize()
    for a, b, name in zip(outs[0], outs[1], ("o", "state", "conv history")):
        _same(a, b, name)
    if T > 1:   # the unfused multi-token step on prepared q, k, v
        q = C.dev(gi.f32_to_bf16_bits(np.tanh(gi.as_f64(d["xq"][0], True)).astype(np.float32)), True)
        k = C.dev(gi.f32_to_bf16_bits(np.tanh(gi.as_f64(d["xk"][0], True)).astype(np.float32)), True)
        v = bf(d["xv"][0])
        g = -torch.sigmoid(_f32(d["a_raw"][0]))
        beta = torch.sigmoid(_f32(d["b_raw"][0]))
        res = []
        for _ in range(2):
            state = _f32(d["state"])
            y, st = gdn.gdn_decode_multi(q, k, v, g, beta, state, step_states=True)
            res.append((y, st, state))
        torch.cuda.synchronize()
        for a, b, name in zip(res[0], res[1], ("y", "step states", "state")):
            _same(a, b, name)
