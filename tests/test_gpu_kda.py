"""GPU parity of gdn_kda_chunk_prefill (the delta rule with a per-channel decay) against the
fp64 oracle's token-by-token recurrence. The path computes in fp32, so fp32 inputs are held to
1e-4; bf16 inputs with a bf16-stored y to the bf16 bar."""
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


def _case(inp, g, bf16, y_dtype, seqs=None, heads=None, bounded=False):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    sh = inp["shape"]
    H, cu = sh.H, inp["cu_seqlens"]
    q, k, v = (C.dev(inp[x], bf16) for x in ("q", "k", "v"))
    _, _, _, _, beta = gdn.gdn_preprocess(None, None, None, None, None, None, _f32(inp["a_raw"]),
                                          _f32(inp["b_raw"]), _f32(inp["A_log"]),
                                          _f32(inp["dt_bias"]), H=H)
    cu_d = None if sh.equal_lengths else C.dev(cu)
    S0 = inp.get("S0")
    run = gdn.gdn_kda_chunk_prefill_bounded if bounded else gdn.gdn_kda_chunk_prefill
    y, ST = run(q, k, v, _f32(g), beta,
                                      initial_state=None if S0 is None else _f32(S0),
                                      cu_seqlens=cu_d, cu_seqlens_host=None if cu_d is None else cu,
                                      num_seqs=sh.num_seqs, y_dtype=y_dtype)
    torch.cuda.synchronize()
    seqs = list(range(sh.num_seqs)) if seqs is None else seqs
    heads = list(range(H)) if heads is None else heads
    sub = C.subset(inp, seqs=seqs, heads=heads)
    _, _, be = oracle.gates(sub["a_raw"], sub["b_raw"], sub["A_log"], sub["dt_bias"])
    al = np.exp(g.astype(np.float64)[sub["tok"]][:, heads])
    y_ref, S_ref = oracle.kda_recurrence(sub["q"], sub["k"], sub["v"], al, be, sub.get("S0"),
                                         sub["cu"])
    y_bf16 = y_dtype == "bf16"
    # the bounded path computes on the bf16 matrix cores: the bf16 bar whatever y's dtype
    ey = C.assert_close("y", C.gpu_slice(y, sub["tok"], heads), y_ref, y_bf16 or bounded,
                        stored_bf16=y_bf16, cu=sub["cu"], H=len(heads))
    # the fp32 path holds S_T to the fp32 bar; the bf16 matrix-core path to the bf16 one
    es = C.assert_close("S_T", C.gpu_state_slice(ST, seqs, heads), S_ref, bounded, state=True)
    print(f"  max slice rel L2: y {ey:.2e}, S_T {es:.2e}", flush=True)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_kda_fp32_ragged(gpu, dims):
    dk, dv = dims
    _announce(f"kda fp32 inputs, lengths [70, 1, 129, 0, 64] H=2 dk={dk} dv={dv}")
    inp = gi.make_inputs(gi.TINY_FP32, seed=8, H=2, lengths=[70, 1, 129, 0, 64], dk=dk, dv=dv)
    inp["S0"] = gi.make_inputs(gi.LONG_CONTEXT, seed=8, H=2, T=1, dk=dk, dv=dv)["S0"].repeat(5, axis=0)
    g = gi.kda_log_decay_draw(8, inp["shape"].ntok, 2, dk)
    _case(inp, g, bf16=False, y_dtype="f32")


def test_kda_steep_decays(gpu):
    """Log-decays far below the KDA bound (down to -60 per token): the kernels form only
    exponentials of non-positive differences, so nothing overflows however steep the decay."""
    _announce("kda fp32 inputs with steep per-channel decays, lengths [130, 64, 7] H=2 d=128")
    inp = gi.make_inputs(gi.TINY_FP32, seed=10, H=2, lengths=[130, 64, 7], d=128)
    g = gi.kda_log_decay_draw(10, inp["shape"].ntok, 2, 128, mean=1.0, cap=60.0)
    assert g.min() < -30.0
    _case(inp, g, False, "f32")


def test_kda_bf16_long(gpu):
    _announce("kda bf16 inputs B=1 H=2 T=1000 d=128, S0, bf16 y")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=9, H=2, T=1000)
    g = gi.kda_log_decay_draw(9, 1000, 2, 128)
    _case(inp, g, bf16=True, y_dtype="bf16")


def test_kda_equal_channel_decays_match_the_scalar_path(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("kda with one decay per head equals gdn_chunk_prefill (fp32 path)")
    inp = gi.make_inputs(gi.TINY_FP32, seed=10, H=2, lengths=[200, 77])
    sh = inp["shape"]
    q, k, v = (C.dev(inp[x]) for x in ("q", "k", "v"))
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None, _f32(inp["a_raw"]),
                                          _f32(inp["b_raw"]), _f32(inp["A_log"]),
                                          _f32(inp["dt_bias"]), H=sh.H)
    cu = C.dev(inp["cu_seqlens"])
    y1, s1 = gdn.gdn_chunk_prefill(q, k, v, g, beta, cu_seqlens=cu, num_seqs=2)
    gk = g[:, :, None].expand(-1, -1, 64).contiguous()
    y2, s2 = gdn.gdn_kda_chunk_prefill(q, k, v, gk, beta, cu_seqlens=cu, num_seqs=2)
    torch.cuda.synchronize()
    assert np.abs(C.host(y1) - C.host(y2)).max() / np.abs(C.host(y1)).max() < 1e-5
    assert np.abs(C.host(s1) - C.host(s2)).max() / np.abs(C.host(s1)).max() < 1e-5


def test_kda_b4_h16_t4096_sampled(gpu):
    _announce("kda at B=4 H=16 T=4096 d=128 (bf16), sampled slices")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=11, B=4, H=16, T=4096)
    g = gi.kda_log_decay_draw(11, 4 * 4096, 16, 128)
    _case(inp, g, bf16=True, y_dtype="bf16", seqs=[1, 2], heads=[0, 7])


def test_kda_many_sequences(gpu):
    """1300 short packed sequences (empty ones included), fp32 inputs, sampled sequences."""
    L = C.many_short_lengths(13, 1300)
    _announce("kda 1300 packed sequences, lengths 0..70, H=2 d=64, fp32 inputs, S0")
    inp = gi.make_inputs(gi.TINY_FP32, seed=13, H=2, lengths=L)
    inp["S0"] = gi.make_inputs(gi.LONG_CONTEXT, seed=13, B=len(L), H=2, T=1, d=64)["S0"]
    g = gi.kda_log_decay_draw(13, inp["shape"].ntok, 2, 64)
    _case(inp, g, False, "f32", seqs=C.sampled_seqs(L, 13))


# ----------------------------------------------------------------------------- bounded decays
# gdn_kda_chunk_prefill_bounded: log-decays in [-5, 0] on the bf16 matrix cores (bf16 q, k, v,
# d = 128), held to the bf16 bar.
BOUNDED = [
    (gi.LONG_CONTEXT, dict(H=2, T=1000), "bf16"),                               # S0, bf16 y
    (gi.LONG_CONTEXT, dict(B=2, H=3, T=200), "f32"),                            # ragged last chunk
    (gi.LONG_CONTEXT, dict(H=2, lengths=[0, 1, 3, 63, 64, 65, 200, 0, 130]), "bf16"),  # packed
    (gi.LONG_CONTEXT, dict(B=64, H=4, T=130), "bf16"),                          # 256 pairs
]


@pytest.mark.parametrize("workload,ov,ydt", BOUNDED, ids=[f"{gi.TAGS[w]}-{o}-{y}" for w, o, y in BOUNDED])
def test_kda_bounded(gpu, workload, ov, ydt):
    _announce(f"kda bounded (bf16 matrix cores) {gi.TAGS[workload]} {ov} y={ydt}")
    inp = gi.make_inputs(workload, seed=14, **ov)
    g = gi.kda_log_decay_draw(14, inp["shape"].ntok, inp["shape"].H, 128)
    assert g.min() >= -5.0
    _case(inp, g, bf16=True, y_dtype=ydt, bounded=True)


def test_kda_bounded_at_the_bound(gpu):
    """Every log-decay at the bound (-5 per token, 80 over a 16-token block): the scaled
    operands reach e^80 and e^-80 and stay finite; the result still meets the bf16 bar."""
    _announce("kda bounded with every log-decay = -5, B=2 H=2 T=300")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=15, B=2, H=2, T=300)
    g = np.full((inp["shape"].ntok, 2, 128), -5.0, dtype=np.float32)
    _case(inp, g, bf16=True, y_dtype="f32", bounded=True)


def test_kda_bounded_b4_h16_t4096_sampled(gpu):
    _announce("kda bounded at B=4 H=16 T=4096 d=128, sampled slices")
    inp = gi.make_inputs(gi.LONG_CONTEXT, seed=11, B=4, H=16, T=4096)
    g = gi.kda_log_decay_draw(11, 4 * 4096, 16, 128)
    _case(inp, g, bf16=True, y_dtype="bf16", seqs=[0, 3], heads=[0, 5, 15], bounded=True)
