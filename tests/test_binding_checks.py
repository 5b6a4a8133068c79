"""Host-side checks of the Python binding: the kernels see bare pointers, so a tensor whose
extent or dtype does not match the call must be refused before anything reaches the device.
Runs on the CPU: the shape checks come before any device pointer is taken."""
import pytest
import torch

import gated_deltanet_recurrence_chunked_amd as gdn

bf, f32 = torch.bfloat16, torch.float32


def _t(*shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def _raises(match, fn, *args, **kw):
    with pytest.raises(gdn.GdnError, match=match):
        fn(*args, **kw)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        gdn.lib()
    except gdn.GdnError as e:
        pytest.skip(str(e))


def test_prefill_and_backward_shapes():
    n, H, dk, dv = 70, 2, 128, 64
    q, k, v = _t(n, H, dk, dtype=bf), _t(n, H, dk, dtype=bf), _t(n, H, dv, dtype=bf)
    g, beta = _t(n, H), _t(n, H)
    _raises("k has shape", gdn.gdn_chunk_prefill, q, _t(n - 1, H, dk, dtype=bf), v, g, beta)
    _raises("v has shape", gdn.gdn_chunk_prefill, q, k, _t(n + 1, H, dv, dtype=bf), g, beta)
    _raises("k must have the dtype of q", gdn.gdn_chunk_prefill, q, _t(n, H, dk), v, g, beta)
    _raises("beta has shape", gdn.gdn_chunk_prefill, q, k, v, g, _t(n, H + 1))
    _raises("initial_state has shape", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            initial_state=_t(1, H, dk, dk))
    _raises("cu_seqlens has shape", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            cu_seqlens=torch.zeros(3, dtype=torch.int32), num_seqs=3)
    _raises("cu_seqlens_host has 2 entries", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            cu_seqlens=torch.zeros(3, dtype=torch.int32), cu_seqlens_host=[0, 70], num_seqs=2)
    _raises("dy has shape", gdn.gdn_chunk_backward, q, k, v, g, beta, _t(n, H, dk, dtype=bf))
    _raises("dfinal_state has shape", gdn.gdn_chunk_backward, q, k, v, g, beta,
            _t(n, H, dv, dtype=bf), dfinal_state=_t(2, H, dk, dv))
    _raises("g has shape", gdn.gdn_kda_chunk_prefill, q, k, v, g, beta)   # per-channel g
    # everything consistent: the next complaint is that the tensors are not on the device
    _raises("must be a device tensor", gdn.gdn_chunk_prefill, q, k, v, g, beta)


def test_preprocess_decode_and_gate_shapes():
    n, H, d = 40, 2, 128
    x = _t(n, H, d, dtype=bf)
    w = _t(H * d, 4)
    a, b, hv = _t(n, H), _t(n, H), _t(H)
    _raises("wk has shape", gdn.gdn_preprocess, x, x, x, w, _t(H * d, 3), w, a, b, hv, hv, H=H)
    _raises("xv has shape", gdn.gdn_preprocess, x, x, _t(n, H + 1, d, dtype=bf), w, w, w, a, b,
            hv, hv, H=H)
    _raises("dt_bias has shape", gdn.gdn_preprocess, x, x, x, w, w, w, a, b, hv, _t(H + 1), H=H)
    _raises("conv_state_in has shape", gdn.gdn_preprocess_stateful, x, x, x, w, w, w, a, b, hv,
            hv, H=H, conv_state_in=_t(1, 2, 3 * H * d, dtype=bf))
    N, T = 4, 3
    _raises("state has shape", gdn.gdn_decode_step, _t(N, H, d, dtype=bf), _t(N, H, d, dtype=bf),
            _t(N, H, d, dtype=bf), _t(N, H), _t(N, H), _t(N, H, d, 64))
    _raises("g has shape", gdn.gdn_decode_multi, _t(N, T, H, d, dtype=bf),
            _t(N, T, H, d, dtype=bf), _t(N, T, H, d, dtype=bf), _t(N, H), _t(N, T, H),
            _t(N, H, d, d))
    _raises("step_states has shape", gdn.gdn_decode_multi, _t(N, T, H, d, dtype=bf),
            _t(N, T, H, d, dtype=bf), _t(N, T, H, d, dtype=bf), _t(N, T, H), _t(N, T, H),
            _t(N, H, d, d), step_states=_t(N, T + 1, H, d, d))
    _raises("norm_weight has shape", gdn.gdn_output_gate, _t(n, H, d, dtype=bf),
            _t(n, H, d, dtype=bf), _t(d + 1))
    _raises("z has shape", gdn.gdn_output_gate, _t(n, H, d, dtype=bf), _t(n, H, 64, dtype=bf),
            _t(d))


def test_fused_entry_point_shapes():
    n, H, d = 40, 4, 128
    x = _t(n, H, d, dtype=bf)
    w = _t(H * d, 4)
    hv = _t(H)
    _raises("z has shape", gdn.gdn_fused_prefill, x, x, x, w, w, w, _t(n, H), _t(n, H), hv, hv,
            _t(n - 1, H, d, dtype=bf), _t(d), H=H)
    _raises("a_raw has shape", gdn.gdn_fused_prefill, x, x, x, w, w, w, _t(n, 1), _t(n, H), hv,
            hv, x, _t(d), H=H)
    N, T = 3, 2
    xd = _t(N, H, d, dtype=bf)
    hist = _t(N, 3, H * 3 * d, dtype=bf)
    st = _t(N, H, d, d)
    _raises("conv_state has shape", gdn.gdn_fused_decode, xd, xd, xd, w, w, w,
            _t(N, 3, H * d, dtype=bf), _t(N, H), _t(N, H), hv, hv, st, xd, _t(d))
    _raises("z must have the dtype of xq", gdn.gdn_fused_decode, xd, xd, xd, w, w, w, hist,
            _t(N, H), _t(N, H), hv, hv, st, _t(N, H, d), _t(d))
    xm = _t(N, T, H, d, dtype=bf)
    _raises("b_raw has shape", gdn.gdn_fused_decode_multi, xm, xm, xm, w, w, w, hist,
            _t(N, T, H), _t(N, H), hv, hv, st, xm, _t(d))
    _raises("conv_state_out has shape", gdn.gdn_fused_decode_multi, xm, xm, xm, w, w, w, hist,
            _t(N, T, H), _t(N, T, H), hv, hv, st, xm, _t(d), conv_state_out=hist[:2])


def test_output_dtype_must_match_the_requested_dtype():
    """A caller-provided output whose dtype differs from the dtype the call writes (an explicit
    y_dtype / o_dtype / out_dtype, or the default) is refused: the kernel would write elements
    of the other size into it."""
    n, H, d = 64, 2, 128
    q = k = v = _t(n, H, d, dtype=bf)
    g, beta = _t(n, H), _t(n, H)
    _raises("y must be torch.float32", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            y=_t(n, H, d, dtype=bf), y_dtype=f32)
    _raises("y must be torch.bfloat16", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            y=_t(n, H, d), y_dtype=bf)
    _raises("final_state must be torch.float32", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            final_state=_t(1, H, d, d, dtype=bf))
    _raises("y must be torch.float32", gdn.gdn_kda_chunk_prefill, q, k, v, _t(n, H, d), beta,
            y=_t(n, H, d, dtype=bf), y_dtype=f32)
    N, T = 4, 2
    xd = _t(N, H, d, dtype=bf)
    _raises("y must be torch.float32", gdn.gdn_decode_step, xd, xd, xd, _t(N, H), _t(N, H),
            _t(N, H, d, d), y=xd, y_dtype=f32)
    xm = _t(N, T, H, d, dtype=bf)
    _raises("y must be torch.float32", gdn.gdn_decode_multi, xm, xm, xm, _t(N, T, H),
            _t(N, T, H), _t(N, H, d, d), y=xm, y_dtype=f32)
    _raises("o must be torch.float32", gdn.gdn_output_gate, _t(n, H, d, dtype=bf),
            _t(n, H, d, dtype=bf), _t(d), o=_t(n, H, d, dtype=bf), o_dtype=f32)
    x = _t(n, H, d, dtype=bf)
    w = _t(H * d, 4)
    hv = _t(H)
    for name in ("q", "k", "v"):
        outs = {name: _t(n, H, d, dtype=bf)}
        _raises(f"{name} must be torch.float32", gdn.gdn_preprocess, x, x, x, w, w, w, g, beta,
                hv, hv, H=H, out_dtype=f32, outs=outs)
        _raises(f"{name} must be torch.float32", gdn.gdn_preprocess_stateful, x, x, x, w, w, w,
                g, beta, hv, hv, H=H, out_dtype=f32, outs=outs)
    _raises("g must be torch.float32", gdn.gdn_preprocess, x, x, x, w, w, w, g, beta, hv, hv,
            H=H, outs={"g": _t(n, H, dtype=bf)})
    _raises("o must be torch.float32", gdn.gdn_fused_prefill, x, x, x, w, w, w, g, beta, hv, hv,
            x, _t(d), H=H, o=_t(n, H, d, dtype=bf), o_dtype=f32)
    hist = _t(N, 3, H * 3 * d, dtype=bf)
    _raises("o must be torch.float32", gdn.gdn_fused_decode, xd, xd, xd, w, w, w, hist,
            _t(N, H), _t(N, H), hv, hv, _t(N, H, d, d), xd, _t(d), o=xd, o_dtype=f32)
    _raises("o must be torch.float32", gdn.gdn_fused_decode_multi, xm, xm, xm, w, w, w, hist,
            _t(N, T, H), _t(N, T, H), hv, hv, _t(N, H, d, d), xm, _t(d), o=xm, o_dtype=f32)
    # a given output of the default dtype passes these checks (next: not on the device)
    _raises("must be a device tensor", gdn.gdn_chunk_prefill, q, k, v, g, beta,
            y=_t(n, H, d, dtype=bf))
