"""GPU parity of gdn_chunk_backward (gradients of the chunked prefill) against the fp64
oracle's reverse-mode gradients of eqs. (1)-(4), token by token. With fp32 inputs (or any
d_k, d_v other than 128) the backward computes in fp32 and is held to the fp32 bar (1e-4
relative L2 per (sequence, head)); bf16 q, k, v and dy at d_k = d_v = 128 take the bf16
matrix-core backward, held to the bf16 bar (gdn_cases.assert_close_grad)."""
import sys

import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _f32(a):
    return C.dev(np.ascontiguousarray(a, dtype=np.float32))


def _run(inp, grads, bf16_in, bf16_dy, seqs=None, heads=None, with_s0=True, with_dst=True):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    sh = inp["shape"]
    H, cu = sh.H, inp["cu_seqlens"]
    q, k, v = (C.dev(inp[x], bf16_in) for x in ("q", "k", "v"))
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None, _f32(inp["a_raw"]),
                                          _f32(inp["b_raw"]), _f32(inp["A_log"]),
                                          _f32(inp["dt_bias"]), H=H)
    S0 = inp.get("S0") if with_s0 else None
    dST = grads["dST"] if with_dst else None
    cu_d = None if sh.equal_lengths else C.dev(cu)
    out = gdn.gdn_chunk_backward(q, k, v, g, beta, C.dev(grads["dy"], bf16_dy),
                                 initial_state=None if S0 is None else _f32(S0),
                                 dfinal_state=None if dST is None else _f32(dST),
                                 cu_seqlens=cu_d, cu_seqlens_host=None if cu_d is None else cu,
                                 num_seqs=sh.num_seqs)
    torch.cuda.synchronize()
    seqs = list(range(sh.num_seqs)) if seqs is None else seqs
    heads = list(range(H)) if heads is None else heads
    sub = C.subset(inp, seqs=seqs, heads=heads)
    tok, scu = sub["tok"], sub["cu"]
    _, al, be = oracle.gates(sub["a_raw"], sub["b_raw"], sub["A_log"], sub["dt_bias"])
    dy = gi.as_f64(grads["dy"], bf16_dy)[tok][:, heads]
    s0 = None if S0 is None else S0.astype(np.float64)[seqs][:, heads]
    dst = None if dST is None else dST.astype(np.float64)[seqs][:, heads]
    ref = oracle.recurrence_backward(sub["q"], sub["k"], sub["v"], al, be, dy, s0, dst, scu)
    # bf16 q, k, v and dy at d_k = d_v = 128 take the bf16 matrix-core backward and its bar
    mfma = bf16_in and bf16_dy and sh.dk == 128 and sh.dv == 128
    rep = {}
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        got = C.gpu_slice(out[key], tok, heads)
        if mfma:
            rep[key] = C.assert_close_grad(key, got, ref[key], cu=scu, H=len(heads))
        else:
            rep[key] = C.assert_close(key, got, ref[key], False, cu=scu, H=len(heads))
    got = C.gpu_state_slice(out["dinitial_state"], seqs, heads)
    if mfma:
        rep["dS0"] = C.assert_close_grad("dS0", got, ref["dS0"], state=True)
    else:
        rep["dS0"] = C.assert_close("dS0", got, ref["dS0"], False, state=True)
    if mfma:
        print("  max slice rel L2 / elementwise ratio:",
              {k: f"{v[0]:.2e}/{v[1]:.2f}" for k, v in rep.items()}, flush=True)
    else:
        print("  max slice rel L2:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_backward_fp32_inputs_ragged(gpu, dims):
    dk, dv = dims
    _announce(f"backward fp32 inputs, lengths [70, 1, 129, 0, 64] H=2 dk={dk} dv={dv}")
    inp = gi.make_inputs(gi.TINY_FP32, seed=5, H=2, lengths=[70, 1, 129, 0, 64], dk=dk, dv=dv)
    inp["S0"] = gi.make_inputs(gi.LONG_CONTEXT, seed=5, H=2, T=1, dk=dk, dv=dv)["S0"].repeat(5, axis=0)
    sh = inp["shape"]
    grads = gi.grad_draws(5, sh.ntok, sh.num_seqs, sh.H, dk, dv)
    _run(inp, grads, bf16_in=False, bf16_dy=False)


@pytest.mark.parametrize("with_s0,with_dst", [(True, True), (False, False)])
def test_backward_bf16_inputs(gpu, with_s0, with_dst):
    _announce(f"backward bf16 inputs B=1 H=2 T=300 d=128 S0={with_s0} dST={with_dst}")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=6, H=2, T=300)
    grads = gi.grad_draws(6, 300, 1, 2, 128, 128, bf16=True)
    _run(inp, grads, bf16_in=True, bf16_dy=True, with_s0=with_s0, with_dst=with_dst)


def test_backward_b4_h16_t4096_sampled(gpu):
    _announce("backward at B=4 H=16 T=4096 d=128, sampled slices")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=7, B=4, H=16, T=4096)
    sh = inp["shape"]
    grads = gi.grad_draws(7, sh.ntok, sh.num_seqs, sh.H, 128, 128, bf16=True)
    _run(inp, grads, bf16_in=True, bf16_dy=True, seqs=[0, 3], heads=[2, 13])


def test_backward_of_no_tokens_passes_the_state_gradient_through(gpu):
    """ntok = 0: every sequence is empty, so dS0 = dS_T (zero without one). Called through the
    C ABI directly, the token inputs pointing at a small dummy buffer the kernels never touch."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("backward with no tokens (2 sequences of length 0)")
    L = gdn.lib()
    N, H, d = 2, 2, 64
    dummy = torch.zeros(64, dtype=torch.float32, device="cuda")
    dST = torch.randn(N, H, d, d, device="cuda")
    ws = torch.empty(max(int(L.gdn_chunk_backward_workspace_size(0, N, H, d, d)), 256),
                     dtype=torch.uint8, device="cuda")
    p = dummy.data_ptr()
    for src in (dST, None):
        dS0 = torch.full((N, H, d, d), 7.0, device="cuda")
        st = L.gdn_chunk_backward(p, p, p, 0, p, p, None, p, 0, None if src is None else src.data_ptr(),
                                  None, None, N, 0, H, d, d, p, p, p, p, p, dS0.data_ptr(),
                                  ws.data_ptr(), ws.numel(), None)
        torch.cuda.synchronize()
        assert st == 0, L.gdn_last_error()
        ref = torch.zeros_like(dS0) if src is None else src
        assert torch.equal(dS0, ref)


def test_backward_many_sequences(gpu):
    """1300 short packed sequences (empty ones included), fp32 inputs, sampled sequences."""
    L = C.many_short_lengths(14, 1300)
    _announce("backward 1300 packed sequences, lengths 0..70, H=2 d=64, fp32 inputs, S0, dS_T")
    inp = gi.make_inputs(gi.TINY_FP32, seed=14, H=2, lengths=L)
    inp["S0"] = gi.make_inputs(gi.LONG_CONTEXT, seed=14, B=len(L), H=2, T=1, d=64)["S0"]
    sh = inp["shape"]
    grads = gi.grad_draws(14, sh.ntok, sh.num_seqs, 2, 64, 64)
    _run(inp, grads, bf16_in=False, bf16_dy=False, seqs=C.sampled_seqs(L, 14))


def test_backward_bf16_varlen_ragged(gpu):
    """The bf16 matrix-core backward on packed sequences of ragged lengths (empty, 1 token, one
    past a chunk, a full chunk), with S0 and dS_T: the chain's longest-first order, the per-chunk
    kernel's chunk table and the ragged last chunks."""
    lengths = [70, 1, 129, 0, 64, 200, 65]
    _announce(f"backward bf16 inputs, lengths {lengths} H=2 d=128, S0, dS_T")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=15, H=2, lengths=lengths)
    sh = inp["shape"]
    grads = gi.grad_draws(15, sh.ntok, sh.num_seqs, sh.H, 128, 128, bf16=True)
    _run(inp, grads, bf16_in=True, bf16_dy=True)


def test_backward_bf16_many_sequences(gpu):
    """300 short packed sequences (empty ones, 64 and 65 tokens included) through the bf16
    matrix-core backward, sampled sequences on both sides of 256 (the chunk table's rounds)."""
    L = C.many_short_lengths(16, 300)
    _announce("backward bf16 inputs, 300 packed sequences of 0..70 tokens, H=2 d=128, S0, dS_T")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=16, H=2, lengths=L)
    sh = inp["shape"]
    grads = gi.grad_draws(16, sh.ntok, sh.num_seqs, sh.H, 128, 128, bf16=True)
    _run(inp, grads, bf16_in=True, bf16_dy=True, seqs=C.sampled_seqs(L, 16))
