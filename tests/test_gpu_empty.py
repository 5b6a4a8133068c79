"""Empty batches through the Python binding: no tokens (ntok = 0, every sequence empty) in the
prefill, preprocess, backward and per-channel-decay entry points, and no sequences (N = 0) in
decode. torch gives a zero-element device tensor a null data pointer, so these calls also
check that the C ABI takes NULL for arrays indexed by an empty token axis.

With no tokens the recurrence of eqs. (1)-(4) never runs: each final state is the initial one
(zero without one), each conv history out is the history in, and dS0 is dS_T. Those are
copies, so they are compared bit for bit."""
import sys

import pytest

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _empty(*shape, dtype=None):
    import torch
    return torch.empty(shape, dtype=dtype or torch.float32, device="cuda")


@pytest.mark.parametrize("dk,bf16,with_cu", [(128, True, True), (128, True, False),
                                             (64, False, True), (128, False, False)])
def test_prefill_kda_and_backward_of_no_tokens(gpu, dk, bf16, with_cu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    num_seqs, H, dv = 3, 2, 64
    _announce(f"no tokens: prefill, per-channel decay, backward num_seqs={num_seqs} H={H} "
              f"dk={dk} dv={dv} bf16={bf16} cu={with_cu}")
    dt = torch.bfloat16 if bf16 else torch.float32
    q, k = _empty(0, H, dk, dtype=dt), _empty(0, H, dk, dtype=dt)
    v = _empty(0, H, dv, dtype=dt)
    g, beta = _empty(0, H), _empty(0, H)
    cu = torch.zeros(num_seqs + 1, dtype=torch.int32, device="cuda") if with_cu else None
    S0 = torch.randn(num_seqs, H, dk, dv, device="cuda")
    kw = dict(cu_seqlens=cu, num_seqs=num_seqs)
    for init in (S0, None):
        ref = S0 if init is not None else torch.zeros_like(S0)
        y, ST = gdn.gdn_chunk_prefill(q, k, v, g, beta, initial_state=init, **kw)
        yk, STk = gdn.gdn_kda_chunk_prefill(q, k, v, _empty(0, H, dk), beta, initial_state=init,
                                            **kw)
        torch.cuda.synchronize()
        assert y.shape == (0, H, dv) and yk.shape == (0, H, dv)
        assert torch.equal(ST, ref), "prefill final state"
        assert torch.equal(STk, ref), "per-channel decay final state"
    dST = torch.randn(num_seqs, H, dk, dv, device="cuda")
    grads = gdn.gdn_chunk_backward(q, k, v, g, beta, _empty(0, H, dv, dtype=dt), initial_state=S0,
                                   dfinal_state=dST, **kw)
    torch.cuda.synchronize()
    assert torch.equal(grads["dinitial_state"], dST)
    assert grads["dq"].shape == (0, H, dk) and grads["dg"].shape == (0, H)


@pytest.mark.parametrize("with_cu", [True, False])
def test_preprocess_and_fused_prefill_of_no_tokens(gpu, with_cu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    num_seqs, H, dk, dv = 2, 4, 128, 128
    _announce(f"no tokens: preprocess (stateful) and fused prefill num_seqs={num_seqs} H={H} "
              f"cu={with_cu}")
    bf = torch.bfloat16
    xq, xk, xv, z = (_empty(0, H, d, dtype=bf) for d in (dk, dk, dv, dv))
    w = [torch.randn(H * d, 4, device="cuda") for d in (dk, dk, dv)]
    a_raw, b_raw = _empty(0, H), _empty(0, H)
    A_log, dt_bias = torch.randn(H, device="cuda"), torch.randn(H, device="cuda")
    cu = torch.zeros(num_seqs + 1, dtype=torch.int32, device="cuda") if with_cu else None
    hin = torch.randn(num_seqs, 3, H * (2 * dk + dv), device="cuda").to(bf)
    for src in (hin, None):
        q, k, v, g, beta, hout = gdn.gdn_preprocess_stateful(
            xq, xk, xv, *w, a_raw, b_raw, A_log, dt_bias, H=H, conv_state_in=src,
            conv_state_out=True, cu_seqlens=cu, num_seqs=num_seqs)
        torch.cuda.synchronize()
        assert q.shape == (0, H, dk) and g.shape == (0, H)
        assert torch.equal(hout, hin if src is not None else torch.zeros_like(hin)), "history"
    S0 = torch.randn(num_seqs, H, dk, dv, device="cuda")
    o, ST, ex = gdn.gdn_fused_prefill(xq, xk, xv, *w, a_raw, b_raw, A_log, dt_bias, z,
                                      torch.randn(dv, device="cuda"), H=H, initial_state=S0,
                                      cu_seqlens=cu, num_seqs=num_seqs, export=True)
    torch.cuda.synchronize()
    assert o.shape == (0, H, dv) and ex["y"].shape == (0, H, dv)
    assert torch.equal(ST, S0)


def test_decode_and_gate_of_no_sequences(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    H, dk, dv, T = 4, 128, 128, 4
    _announce(f"no sequences: decode step, multi-token decode, fused decodes, output gate H={H}")
    bf = torch.bfloat16
    q, k, v = _empty(0, H, dk, dtype=bf), _empty(0, H, dk, dtype=bf), _empty(0, H, dv, dtype=bf)
    state = _empty(0, H, dk, dv)
    y = gdn.gdn_decode_step(q, k, v, _empty(0, H), _empty(0, H), state)
    ym, steps = gdn.gdn_decode_multi(_empty(0, T, H, dk, dtype=bf), _empty(0, T, H, dk, dtype=bf),
                                     _empty(0, T, H, dv, dtype=bf),
                                     _empty(0, T, H), _empty(0, T, H), state, step_states=True)
    w = [torch.randn(H * d, 4, device="cuda") for d in (dk, dk, dv)]
    A_log, dt_bias = torch.randn(H, device="cuda"), torch.randn(H, device="cuda")
    nw = torch.randn(dv, device="cuda")
    hist = _empty(0, 3, H * (2 * dk + dv), dtype=bf)
    o = gdn.gdn_fused_decode(q, k, v, *w, hist, _empty(0, H), _empty(0, H), A_log, dt_bias, state,
                             _empty(0, H, dv, dtype=bf), nw)
    om, _, _ = gdn.gdn_fused_decode_multi(
        _empty(0, T, H, dk, dtype=bf), _empty(0, T, H, dk, dtype=bf), _empty(0, T, H, dv, dtype=bf),
        *w, hist, _empty(0, T, H), _empty(0, T, H), A_log, dt_bias, state,
        _empty(0, T, H, dv, dtype=bf), nw, step_states=True)
    og = gdn.gdn_output_gate(_empty(0, H, dv, dtype=bf), _empty(0, H, dv, dtype=bf), nw)
    torch.cuda.synchronize()
    assert y.shape == (0, H, dv) and ym.shape == (0, T, H, dv) and steps.shape == (0, T, H, dk, dv)
    assert o.shape == (0, H, dv) and om.shape == (0, T, H, dv) and og.shape == (0, H, dv)
