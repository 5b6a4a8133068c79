"""GPU parity of the fused entry points against the fp64 oracle:
  * gdn_fused_prefill (conv, SiLU, L2Norm and gates inside the per-chunk kernel, then the scan
    and the output gate): against the oracle's eqs. (6)-(11), and element for element against
    the separate-kernel pipeline gdn_preprocess -> gdn_chunk_prefill -> gdn_output_gate;
  * gdn_fused_decode (one kernel per decode step from the projected streams, conv history and
    state carried in place) and gdn_fused_decode_multi (T tokens per sequence per step, with
    the state after each token on request): against the oracle over each sequence's whole
    token stream.
Sources: reading notes "Qwen3.8-Next 架构设计：评测、效率与训练稳定性", section 2.1.1,
eqs. (1)-(11); the design summary "设计 LLM 架构" (causal depthwise short conv)."""
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


def _compare_to_oracle(inp, res, sub):
    tok, heads, seqs, cu, H = sub["tok"], sub["heads"], sub["seqs"], sub["cu"], sub["H"]
    ref = C.oracle_run(sub)
    rep = {}
    for key in ("q", "k", "v"):
        rep[key] = C.assert_close(key, C.gpu_slice(res[key], tok, heads), ref[key], True,
                                  stored_bf16=True, cu=cu, H=H)
    for key in ("g", "beta"):
        got = C.gpu_slice(res[key], tok, heads)
        err = np.abs(got - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30)
        assert err < 1e-5, f"{key}: {err}"
    rep["y"] = C.assert_close("y", C.gpu_slice(res["y"], tok, heads), ref["y"], True,
                              stored_bf16=True, cu=cu, H=H)
    rep["ST"] = C.assert_close("ST", C.gpu_state_slice(res["ST"], seqs, heads), ref["ST"], True,
                               state=True)
    rep["o"], rep["o_max_abs"] = C.check_o(C.gpu_slice(res["o"], tok, heads), sub, ref, True)
    print("  max slice rel L2:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


def _equal_to_pipeline(fused, sep, gate_in_scan=False):
    """The fused path computes q, k, v and the gates with the preprocess kernel's arithmetic, so
    these, y and the final state equal the separate kernels' bit for bit. o does too when the
    output gate runs as its own kernel on the stored bf16 y; when the full-row scan applies the
    gate (gate_in_scan) it starts from the fp32 y, and o is held to the oracle instead."""
    import torch
    keys = ("q", "k", "v", "g", "beta", "y", "ST") + (() if gate_in_scan else ("o",))
    for key in keys:
        a, b = fused[key], sep[key]
        assert a.dtype == b.dtype and a.shape == b.shape, key
        if not torch.equal(a, b):
            d = (a.float() - b.float()).abs().max().item()
            raise AssertionError(f"{key}: fused differs from the separate kernels (max |diff| {d:.3e})")


PREFILL_CASES = [
    (gi.PREFILL, dict(B=2, H=3, T=200)),                                      # one head per workgroup
    (gi.PREFILL, dict(B=2, H=4, T=300)),                                      # four heads per workgroup
    (gi.PREFILL, dict(B=2, H=2, T=150, dv=64)),                               # two heads, dv = 64
    (gi.VARLEN, dict(H=2, lengths=[0, 1, 3, 63, 64, 65, 200, 0, 130])),      # empty/short seqs, S0
    (gi.VARLEN, dict(H=4, nseq=5, lmax=600)),
    # 256 or more (sequence, head) pairs of equal length: the gate runs in the full-row scan's
    # epilogue; packed sequences of unequal lengths take the sliced scan and the gate kernel
    (gi.PREFILL, dict(B=64, H=4, T=200)),
    (gi.VARLEN, dict(H=8, nseq=40, lmax=400)),
]


def _gate_in_scan(inp):
    sh = inp["shape"]
    return sh.equal_lengths and sh.num_seqs * sh.H >= 256 and sh.dv == 128


@pytest.mark.parametrize("workload,ov", PREFILL_CASES,
                         ids=[f"{gi.TAGS[w]}-{o}" for w, o in PREFILL_CASES])
def test_fused_prefill(gpu, workload, ov):
    _announce(f"fused prefill {gi.TAGS[workload]} {ov}")
    inp = gi.make_inputs(workload, seed=1, **ov)
    fused = C.gpu_run_fused(inp)
    _compare_to_oracle(inp, fused, C.subset(inp))
    _equal_to_pipeline(fused, C.gpu_run(inp, y_dtype="bf16"), _gate_in_scan(inp))


@pytest.mark.slow
def test_fused_prefill_b4_h16_t4096_full(gpu):
    _announce("fused prefill at B=4 H=16 T=4096 d=128 (bf16), sampled slices")
    inp = gi.make_inputs(gi.PREFILL, seed=0)
    fused = C.gpu_run_fused(inp)
    _compare_to_oracle(inp, fused, C.subset(inp, seqs=[0, 3], heads=[0, 9, 15]))
    _equal_to_pipeline(fused, C.gpu_run(inp, y_dtype="bf16"))


# ----------------------------------------------------------------------------- decode
DECODE_CASES = [
    # (N, H, dk, dv, x bf16, o bf16, steps)
    (8, 2, 128, 128, True, True, 5),
    (5, 3, 64, 128, False, False, 4),
    (4, 2, 128, 64, True, False, 3),
    (3, 1, 64, 64, False, True, 6),
    # around the persistent kernel's grid (one workgroup per compute unit, 256 on MI355X): one
    # head more than workgroups, and some workgroups with an odd, others an even head count
    (257, 1, 128, 128, True, True, 2),
    (769, 1, 128, 128, False, False, 2),
]


@pytest.mark.parametrize("N,H,dk,dv,xbf,obf,steps", DECODE_CASES,
                         ids=[f"N{c[0]}-H{c[1]}-dk{c[2]}-dv{c[3]}-x{'bf' if c[4] else 'f32'}-o{'bf' if c[5] else 'f32'}"
                              for c in DECODE_CASES])
def test_fused_decode_steps(gpu, N, H, dk, dv, xbf, obf, steps):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce(f"fused decode N={N} H={H} dk={dk} dv={dv} x_bf16={xbf} o_bf16={obf} steps={steps}")
    d = gi.decode_layer_draws(11, steps, N, H, dk, dv, bf16=xbf)
    xd = lambda a: C.dev(a, xbf)                                               # noqa: E731
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))            # noqa: E731
    w = [f32(d[x]) for x in ("wq", "wk", "wv")]
    conv_state = xd(d["conv_state"])
    state = f32(d["state"])
    os_, ys = [], []
    for s in range(steps):
        o, y = gdn.gdn_fused_decode(xd(d["xq"][s]), xd(d["xk"][s]), xd(d["xv"][s]), *w, conv_state,
                                    f32(d["a_raw"][s]), f32(d["b_raw"][s]), f32(d["A_log"]),
                                    f32(d["dt_bias"]), state, xd(d["z"][s]),
                                    f32(d["norm_weight"]), l2_eps=C.L2_EPS, rms_eps=C.RMS_EPS,
                                    o_dtype=torch.bfloat16 if obf else torch.float32, want_y=True)
        os_.append(C.host(o))
        ys.append(C.host(y))
    torch.cuda.synchronize()

    # oracle: sequence n is its `steps` tokens in order, starting from the carried history
    perm = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape(N * steps, *a.shape[2:]))  # noqa
    f64 = lambda a: gi.as_f64(a, xbf)                                          # noqa: E731
    cu = np.arange(0, N * steps + 1, steps).astype(np.int32)
    q, k, v, hist = oracle.preprocess_stateful(perm(f64(d["xq"])), perm(f64(d["xk"])),
                                               perm(f64(d["xv"])), d["wq"], d["wk"], d["wv"], cu,
                                               H, conv_state_in=f64(d["conv_state"]),
                                               l2_eps=C.L2_EPS)
    _, al, be = oracle.gates(perm(d["a_raw"].astype(np.float64)), perm(d["b_raw"].astype(np.float64)),
                             d["A_log"].astype(np.float64), d["dt_bias"].astype(np.float64))
    y_ref, S_ref = oracle.recurrence(q, k, v, al, be, d["state"].astype(np.float64), cu)
    o_ref = oracle.output_gate(y_ref, perm(f64(d["z"])), d["norm_weight"].astype(np.float64),
                               C.RMS_EPS)
    gather = lambda L: np.stack(L, axis=1).reshape(N * steps, H, dv)           # noqa: E731
    bf_path = xbf or obf
    rep = dict(
        y=C.assert_close("y", gather(ys), y_ref, bf_path, stored_bf16=obf, cu=cu, H=H),
        o=C.assert_close("o", gather(os_), o_ref, bf_path, stored_bf16=obf, cu=cu, H=H),
        S=C.assert_close("S", C.host(state), S_ref, bf_path, state=True))
    print("  max slice rel L2:", {k_: f"{v_:.2e}" for k_, v_ in rep.items()}, flush=True)
    # the carried history is raw input moved, bit for bit
    assert np.array_equal(C.host(conv_state), hist)


# ----------------------------------------------------------------------------- multi-token decode
MULTI_CASES = [
    # (N, H, dk, dv, x bf16, o bf16, T, steps, conv history out of place, step states)
    (5, 2, 128, 128, True, True, 4, 3, False, False),
    (3, 3, 64, 128, False, False, 2, 3, True, True),
    (4, 1, 128, 64, True, False, 8, 2, True, False),
    (2, 2, 64, 64, False, True, 3, 4, False, True),
]


@pytest.mark.parametrize("N,H,dk,dv,xbf,obf,T,steps,oop,want_steps", MULTI_CASES,
                         ids=[f"N{c[0]}-H{c[1]}-dk{c[2]}-dv{c[3]}-T{c[6]}" for c in MULTI_CASES])
def test_fused_decode_multi_steps(gpu, N, H, dk, dv, xbf, obf, T, steps, oop, want_steps):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce(f"fused multi-token decode N={N} H={H} dk={dk} dv={dv} T={T} steps={steps} "
              f"x_bf16={xbf} o_bf16={obf} out_of_place={oop} step_states={want_steps}")
    d = gi.decode_layer_draws(12, steps, N, H, dk, dv, bf16=xbf, tokens=T)
    xd = lambda a: C.dev(a, xbf)                                               # noqa: E731
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))            # noqa: E731
    w = [f32(d[x]) for x in ("wq", "wk", "wv")]
    hist = [xd(d["conv_state"])]
    if oop:
        hist.append(torch.empty_like(hist[0]))
    state = f32(d["state"])
    os_, ys, last_steps = [], [], None
    for s in range(steps):
        h_in = hist[s % len(hist)]
        h_out = hist[(s + 1) % len(hist)]
        o, y, st = gdn.gdn_fused_decode_multi(
            xd(d["xq"][s]), xd(d["xk"][s]), xd(d["xv"][s]), *w, h_in, f32(d["a_raw"][s]),
            f32(d["b_raw"][s]), f32(d["A_log"]), f32(d["dt_bias"]), state, xd(d["z"][s]),
            f32(d["norm_weight"]), conv_state_out=h_out, l2_eps=C.L2_EPS, rms_eps=C.RMS_EPS,
            o_dtype=torch.bfloat16 if obf else torch.float32, want_y=True,
            step_states=True if want_steps else None)
        os_.append(C.host(o))
        ys.append(C.host(y))
        if want_steps:
            last_steps = C.host(st)
    torch.cuda.synchronize()
    final_hist = C.host(hist[steps % len(hist)])

    # oracle: sequence n is its steps*T tokens in order, from the carried history and state
    L = steps * T
    perm = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape(N * L, *a.shape[3:]))  # noqa
    f64 = lambda a: gi.as_f64(a, xbf)                                          # noqa: E731
    cu = np.arange(0, N * L + 1, L).astype(np.int32)
    q, k, v, hist_ref = oracle.preprocess_stateful(perm(f64(d["xq"])), perm(f64(d["xk"])),
                                                   perm(f64(d["xv"])), d["wq"], d["wk"], d["wv"],
                                                   cu, H, conv_state_in=f64(d["conv_state"]),
                                                   l2_eps=C.L2_EPS)
    _, al, be = oracle.gates(perm(d["a_raw"].astype(np.float64)), perm(d["b_raw"].astype(np.float64)),
                             d["A_log"].astype(np.float64), d["dt_bias"].astype(np.float64))
    S0 = d["state"].astype(np.float64)
    y_ref, S_ref = oracle.recurrence(q, k, v, al, be, S0, cu)
    o_ref = oracle.output_gate(y_ref, perm(f64(d["z"])), d["norm_weight"].astype(np.float64),
                               C.RMS_EPS)
    gather = lambda Ls: np.stack(Ls, axis=1).reshape(N * L, H, dv)             # noqa: E731
    bf_path = xbf or obf
    rep = dict(
        y=C.assert_close("y", gather(ys), y_ref, bf_path, stored_bf16=obf, cu=cu, H=H),
        o=C.assert_close("o", gather(os_), o_ref, bf_path, stored_bf16=obf, cu=cu, H=H),
        S=C.assert_close("S", C.host(state), S_ref, bf_path, state=True))
    assert np.array_equal(final_hist, hist_ref)
    if want_steps:
        # the state after token t of the last step = the oracle's state after that many tokens
        # (the kernel evaluates the last token's state twice, for the step output and in place)
        fin = C.host(state)
        assert np.abs(last_steps[:, T - 1] - fin).max() <= 1e-6 * np.abs(fin).max()
        for t in range(T - 1):
            keep = (steps - 1) * T + t + 1
            idx = np.concatenate([np.arange(n * L, n * L + keep) for n in range(N)])
            cu_t = np.arange(0, N * keep + 1, keep).astype(np.int32)
            _, S_t = oracle.recurrence(q[idx], k[idx], v[idx], al[idx], be[idx], S0, cu_t)
            rep[f"S_step{t}"] = C.assert_close(f"state after token {t}", last_steps[:, t], S_t,
                                               bf_path, state=True)
    print("  max slice rel L2:", {k_: f"{v_:.2e}" for k_, v_ in rep.items()}, flush=True)


def test_fused_decode_multi_one_token_matches_fused_decode(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    N, H = 6, 2
    _announce(f"fused multi-token decode T=1 vs fused decode N={N} H={H}")
    d = gi.decode_layer_draws(13, 1, N, H, bf16=False)
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))            # noqa: E731
    args = lambda s: [f32(d[x][0]) for x in ("xq", "xk", "xv")] + [f32(d[x]) for x in ("wq", "wk", "wv")]  # noqa
    h1, h2 = f32(d["conv_state"]), f32(d["conv_state"])
    s1, s2 = f32(d["state"]), f32(d["state"])
    o1 = gdn.gdn_fused_decode(*args(0), h1, f32(d["a_raw"][0]), f32(d["b_raw"][0]),
                              f32(d["A_log"]), f32(d["dt_bias"]), s1, f32(d["z"][0]),
                              f32(d["norm_weight"]))
    xs = [f32(d[x][0]).view(N, 1, H, -1) for x in ("xq", "xk", "xv")]
    o2, _, _ = gdn.gdn_fused_decode_multi(*xs, *[f32(d[x]) for x in ("wq", "wk", "wv")], h2,
                                          f32(d["a_raw"][0]).view(N, 1, H),
                                          f32(d["b_raw"][0]).view(N, 1, H), f32(d["A_log"]),
                                          f32(d["dt_bias"]), s2,
                                          f32(d["z"][0]).view(N, 1, H, -1), f32(d["norm_weight"]))
    torch.cuda.synchronize()
    assert np.abs(C.host(o1) - C.host(o2)[:, 0]).max() < 1e-5
    assert np.abs(C.host(s1) - C.host(s2)).max() < 1e-5
    assert torch.equal(h1, h2)


# ----------------------------------------------------------------------------- full-size decode
def _subset_stream(d, seqs, heads, xbf):
    """The draws of decode_layer_draws restricted to some sequences and heads, as float64, with
    the token axes flattened per sequence (sequence-major): the oracle's packed streams."""
    H, dk, dv = d["H"], d["dk"], d["dv"]
    f64 = lambda a: gi.as_f64(np.ascontiguousarray(a), xbf)                    # noqa: E731
    multi = d["tokens"] > 1

    def pick(a, tail):   # [steps, N, (T,) H, ...] -> [ns * steps * T, nh, ...]
        a = a[:, seqs][:, :, :, heads] if multi else a[:, seqs][:, :, heads]
        if not multi:
            a = a[:, :, None]
        a = np.swapaxes(a, 0, 1)                          # [ns, steps, T, nh, ...]
        return a.reshape((-1, len(heads)) + tail)

    out = dict(xq=pick(f64(d["xq"]), (dk,)), xk=pick(f64(d["xk"]), (dk,)),
               xv=pick(f64(d["xv"]), (dv,)), z=pick(f64(d["z"]), (dv,)),
               a_raw=pick(d["a_raw"].astype(np.float64), ()),
               b_raw=pick(d["b_raw"].astype(np.float64), ()))
    for key, dd in (("wq", dk), ("wk", dk), ("wv", dv)):
        out[key] = d[key].astype(np.float64).reshape(H, dd, 4)[heads].reshape(-1, 4)
    cs = f64(d["conv_state"])[seqs]                                           # [ns, 3, C]
    parts, off = [], 0
    for dd in (dk, dk, dv):
        blk = cs[:, :, off:off + H * dd].reshape(len(seqs), 3, H, dd)[:, :, heads]
        parts.append(blk.reshape(len(seqs), 3, -1))
        off += H * dd
    out["conv_state"] = np.concatenate(parts, axis=2)
    out["state"] = d["state"].astype(np.float64)[seqs][:, heads]
    out["A_log"] = d["A_log"].astype(np.float64)[heads]
    out["dt_bias"] = d["dt_bias"].astype(np.float64)[heads]
    return out


@pytest.mark.slow
@pytest.mark.parametrize("T", [1, 4])
def test_fused_decode_full_size(gpu, T):
    """The fused decode step at N=256, H=32, d=128 (bf16 x, z, o), as the benchmark runs it, over
    2 steps; sampled (sequence, head) slices against the oracle."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    N, H, steps = 256, 32, 2
    _announce(f"fused decode full size N={N} H={H} d=128 T={T} steps={steps}")
    d = gi.decode_layer_draws(21, steps, N, H, tokens=T)
    bf = lambda a: C.dev(a, True)                                              # noqa: E731
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))            # noqa: E731
    w = [f32(d[x]) for x in ("wq", "wk", "wv")]
    hist, state = bf(d["conv_state"]), f32(d["state"])
    os_ = []
    for s in range(steps):
        args = (bf(d["xq"][s]), bf(d["xk"][s]), bf(d["xv"][s]), *w, hist, f32(d["a_raw"][s]),
                f32(d["b_raw"][s]), f32(d["A_log"]), f32(d["dt_bias"]), state, bf(d["z"][s]),
                f32(d["norm_weight"]))
        if T == 1:
            o = gdn.gdn_fused_decode(*args, l2_eps=C.L2_EPS, rms_eps=C.RMS_EPS)
        else:
            o, _, _ = gdn.gdn_fused_decode_multi(*args, l2_eps=C.L2_EPS, rms_eps=C.RMS_EPS)
        os_.append(o)
    torch.cuda.synchronize()
    seqs, heads = [0, 101, 255], [0, 17, 31]
    sub = _subset_stream(d, seqs, heads, True)
    L = steps * T
    cu = np.arange(0, len(seqs) * L + 1, L).astype(np.int32)
    q, k, v, hist_ref = oracle.preprocess_stateful(sub["xq"], sub["xk"], sub["xv"], sub["wq"],
                                                   sub["wk"], sub["wv"], cu, len(heads),
                                                   conv_state_in=sub["conv_state"],
                                                   l2_eps=C.L2_EPS)
    _, al, be = oracle.gates(sub["a_raw"], sub["b_raw"], sub["A_log"], sub["dt_bias"])
    y_ref, S_ref = oracle.recurrence(q, k, v, al, be, sub["state"], cu)
    o_ref = oracle.output_gate(y_ref, sub["z"], d["norm_weight"].astype(np.float64), C.RMS_EPS)
    # the GPU's o for the sampled slices, in the oracle's order
    got, oh = [], [C.host(o) for o in os_]
    for n in seqs:
        for s in range(steps):
            got.append(oh[s][n][heads] if T == 1 else oh[s][n][:, heads])
    got = np.concatenate([g.reshape(-1, len(heads), 128) for g in got], axis=0)
    rep = dict(o=C.assert_close("o", got, o_ref, True, stored_bf16=True, cu=cu, H=len(heads)),
               S=C.assert_close("S", C.host(state)[seqs][:, heads], S_ref, True, state=True))
    # the history of the sampled slices moved on by the steps' inputs, bit for bit
    hg = C.host(hist)[seqs]
    parts, off = [], 0
    for dd in (128, 128, 128):
        blk = hg[:, :, off:off + H * dd].reshape(len(seqs), 3, H, dd)[:, :, heads]
        parts.append(blk.reshape(len(seqs), 3, -1))
        off += H * dd
    assert np.array_equal(np.concatenate(parts, axis=2), hist_ref)
    print("  max slice rel L2:", {k_: f"{v_:.2e}" for k_, v_ in rep.items()}, flush=True)
