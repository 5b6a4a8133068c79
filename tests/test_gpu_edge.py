"""GPU tests of the method's special cases on the bf16 matrix-core prefill and on the decode step
(reading notes "Qwen3.8-Next 架构设计：评测、效率与训练稳定性", section 2.1.1, subsection "Gated Delta
递归": alpha, beta in (0, 1), the state erased along k and rewritten with v):
  * beta = 1 with unit-norm k and q = k: y_t = S_t^T k_t = v_t exactly (erase-then-write);
  * beta = 0 and g = 0 (alpha = 1): the state is untouched, S_T = S_0 bit for bit, y_t = S_0^T q_t;
  * beta = 0 with steep decays: pure decay, S_T = e^{sum g} S_0 and y_t = e^{G_t} S_0^T q_t;
  * alpha -> 0 at single tokens inside chunks (a huge decay rate): the state is forgotten there;
  * a NaN in one (sequence, head) slice stays in it: every other slice equals a clean run bit
    for bit (and, for a NaN in v, every other d_v column of the same slice too, since the
    columns of S, V, U and Y are independent).
The closed forms are computed here in numpy (fp64) from the inputs; the alpha -> 0 case is
checked against the fp64 oracle, which is pinned to the same special cases on the CPU."""
import sys

import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu

H, DK = 3, 128


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _unit_bf16_keys(rng, n, h, d):
    """Keys of exactly unit norm in bf16: four entries of +-1/2 at distinct random positions
    (4 * 1/4 = 1, every value exact in bf16), so overlapping supports make them non-orthogonal."""
    k = np.zeros((n, h, d), np.float32)
    for t in range(n):
        for j in range(h):
            idx = rng.choice(d, size=4, replace=False)
            k[t, j, idx] = rng.choice([-0.5, 0.5], size=4)
    return gi.f32_to_bf16_bits(k)


def _config_gates(rng, n, h):
    """g = log alpha as in the workloads: -e^A softplus(w - 4.6), e^A ~ U[1, 16], w ~ N(0, 1)."""
    eA = rng.uniform(1.0, 16.0, size=h)
    x = rng.standard_normal((n, h)) - 4.6
    sp = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
    return (-eA * sp).astype(np.float32)


def _prefill(q, k, v, g, beta, S0, cu, y_dtype="f32"):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    nseq = len(cu) - 1
    y, ST = gdn.gdn_chunk_prefill(
        C.dev(q, True), C.dev(k, True), C.dev(v, True), C.dev(g), C.dev(beta),
        initial_state=None if S0 is None else C.dev(S0), cu_seqlens=C.dev(cu),
        cu_seqlens_host=cu, num_seqs=nseq, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y, ST


def _lengths():
    return [200, 64, 131, 1]      # ragged tails, a whole chunk, a single token


def _cu(L):
    return np.concatenate([[0], np.cumsum(L)]).astype(np.int32)


@pytest.mark.parametrize("dv", [128, 64])
def test_erase_then_write_prefill(gpu, dv):
    """beta = 1, q = k with |k| = 1: y_t = v_t."""
    _announce(f"edge: beta=1, q=k unit (bf16-exact), prefill matrix path dv={dv}")
    rng = np.random.default_rng(101)
    L = _lengths()
    cu, n = _cu(L), sum(L)
    k = _unit_bf16_keys(rng, n, H, DK)
    v = gi.f32_to_bf16_bits(rng.standard_normal((n, H, dv)).astype(np.float32))
    g = _config_gates(rng, n, H)
    beta = np.ones((n, H), np.float32)
    S0 = (0.1 * rng.standard_normal((len(L), H, DK, dv))).astype(np.float32)
    y, _ = _prefill(k, k, v, g, beta, S0, cu)
    vf = gi.as_f64(v, True)
    e = C.assert_close("y = v", C.host(y), vf, True, cu=cu, H=H)
    print(f"  y = v: max slice rel L2 {e:.2e}, max |y - v| {C.max_abs(C.host(y), vf):.3e}")


def test_erase_then_write_decode(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("edge: beta=1, q=k unit (bf16-exact), decode steps")
    rng = np.random.default_rng(102)
    N, steps = 8, 5
    state = C.dev((0.1 * rng.standard_normal((N, H, DK, DK))).astype(np.float32))
    for s in range(steps):
        k = _unit_bf16_keys(rng, N, H, DK)
        v = gi.f32_to_bf16_bits(rng.standard_normal((N, H, DK)).astype(np.float32))
        g = _config_gates(rng, N, H)
        y = gdn.gdn_decode_step(C.dev(k, True), C.dev(k, True), C.dev(v, True), C.dev(g),
                                C.dev(np.ones((N, H), np.float32)), state, y_dtype="f32")
        torch.cuda.synchronize()
        vf = gi.as_f64(v, True)
        err = np.abs(C.host(y) - vf).max()
        assert err <= 1e-4 * max(1.0, np.abs(vf).max()), f"step {s}: max |y - v| {err:.3e}"
    print(f"  decode y = v: max |y - v| {err:.3e}")


@pytest.mark.parametrize("dv", [128, 64])
def test_identity_gates_keep_state_prefill(gpu, dv):
    """beta = 0, g = 0: S_T = S_0 bit for bit; y_t = S_0^T q_t."""
    _announce(f"edge: beta=0, g=0, prefill matrix path dv={dv}")
    rng = np.random.default_rng(103)
    L = _lengths()
    cu, n = _cu(L), sum(L)
    q = gi.f32_to_bf16_bits(rng.standard_normal((n, H, DK)).astype(np.float32) / np.sqrt(DK))
    k = gi.f32_to_bf16_bits(rng.standard_normal((n, H, DK)).astype(np.float32) / np.sqrt(DK))
    v = gi.f32_to_bf16_bits(rng.standard_normal((n, H, dv)).astype(np.float32))
    S0 = (0.1 * rng.standard_normal((len(L), H, DK, dv))).astype(np.float32)
    z = np.zeros((n, H), np.float32)
    y, ST = _prefill(q, k, v, z, z, S0, cu)
    assert np.array_equal(ST.cpu().numpy(), S0), "S_T differs from S_0"
    qf = gi.as_f64(q, True)
    y_ref = np.concatenate([np.einsum("thi,hij->thj", qf[cu[s]:cu[s + 1]], S0[s].astype(np.float64))
                            for s in range(len(L))])
    e = C.assert_close("y = S0^T q", C.host(y), y_ref, True, cu=cu, H=H)
    print(f"  S_T == S_0 bit for bit; y: max slice rel L2 {e:.2e}")


def test_identity_gates_keep_state_decode(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("edge: beta=0, g=0, decode steps")
    rng = np.random.default_rng(104)
    N = 8
    S0 = (0.1 * rng.standard_normal((N, H, DK, DK))).astype(np.float32)
    state = C.dev(S0)
    z = C.dev(np.zeros((N, H), np.float32))
    for s in range(4):
        q = gi.f32_to_bf16_bits(rng.standard_normal((N, H, DK)).astype(np.float32))
        k = gi.f32_to_bf16_bits(rng.standard_normal((N, H, DK)).astype(np.float32))
        v = gi.f32_to_bf16_bits(rng.standard_normal((N, H, DK)).astype(np.float32))
        y = gdn.gdn_decode_step(C.dev(q, True), C.dev(k, True), C.dev(v, True), z, z, state,
                                y_dtype="f32")
        torch.cuda.synchronize()
        y_ref = np.einsum("nhi,nhij->nhj", gi.as_f64(q, True), S0.astype(np.float64))
        err = np.abs(C.host(y) - y_ref).max() / np.abs(y_ref).max()
        assert err < 1e-5, f"step {s}: y rel err {err:.3e}"
    assert np.array_equal(state.cpu().numpy(), S0), "state changed"
    print("  decode state == S_0 bit for bit")


@pytest.mark.parametrize("dv", [128, 64])
def test_pure_decay_prefill(gpu, dv):
    """beta = 0, steep g: S_T = e^{sum g} S_0, y_t = e^{G_t} S_0^T q_t."""
    _announce(f"edge: beta=0, steep decays, prefill matrix path dv={dv}")
    rng = np.random.default_rng(105)
    L = _lengths()
    cu, n = _cu(L), sum(L)
    q = gi.f32_to_bf16_bits(rng.standard_normal((n, H, DK)).astype(np.float32) / np.sqrt(DK))
    k = gi.f32_to_bf16_bits(rng.standard_normal((n, H, DK)).astype(np.float32) / np.sqrt(DK))
    v = gi.f32_to_bf16_bits(rng.standard_normal((n, H, dv)).astype(np.float32))
    S0 = (0.1 * rng.standard_normal((len(L), H, DK, dv))).astype(np.float32)
    g = (-rng.uniform(0.0, 0.4, size=(n, H))).astype(np.float32)
    g[cu[0] + 70] = -15.0                     # one very steep step inside a chunk
    beta = np.zeros((n, H), np.float32)
    y, ST = _prefill(q, k, v, g, beta, S0, cu)
    qf = gi.as_f64(q, True)
    y_ref, S_ref = [], []
    for s in range(len(L)):
        G = np.cumsum(g[cu[s]:cu[s + 1]].astype(np.float64), axis=0)           # [L, H]
        S = S0[s].astype(np.float64)
        y_ref.append(np.exp(G)[:, :, None] * np.einsum("thi,hij->thj", qf[cu[s]:cu[s + 1]], S))
        S_ref.append(np.exp(G[-1] if len(G) else np.zeros(H))[:, None, None] * S)
    y_ref, S_ref = np.concatenate(y_ref), np.stack(S_ref)
    ey = C.assert_close("y", C.host(y), y_ref, True, cu=cu, H=H)
    es = C.assert_close("S_T", C.host(ST), S_ref, True, state=True)
    print(f"  pure decay: max slice rel L2 y {ey:.2e}, S_T {es:.2e}")


def _spiky_inputs(seed, dv, L, spikes=None):
    """Workload-distributed q, k (unit rows), v, gates, S0, with alpha -> 0 at a few tokens:
    a_raw = +40 there, so g = -e^A softplus(35.4) ~ -35 .. -570 and alpha = e^g underflows.
    Default spikes (for _lengths()): the first, middle and last token of chunks."""
    rng = np.random.default_rng(seed)
    cu, n = _cu(L), sum(L)
    if spikes is None:
        spikes = [cu[0] + 5, cu[0] + 64, cu[0] + 127, cu[0] + 150, cu[2] + 63, cu[2] + 100]
    assert max(spikes) < n
    q = gi.f32_to_bf16_bits(_unit(rng, n))
    k = gi.f32_to_bf16_bits(_unit(rng, n))
    v = gi.f32_to_bf16_bits(rng.standard_normal((n, H, dv)).astype(np.float32))
    a_raw = rng.standard_normal((n, H)).astype(np.float32)
    a_raw[spikes] = 40.0
    b_raw = rng.standard_normal((n, H)).astype(np.float32)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = np.full(H, -4.6, np.float32)
    g, _, beta = oracle.gates(a_raw.astype(np.float64), b_raw.astype(np.float64),
                              A_log.astype(np.float64), dt_bias.astype(np.float64))
    S0 = (0.1 * rng.standard_normal((len(L), H, DK, dv))).astype(np.float32)
    return cu, q, k, v, g.astype(np.float32), beta.astype(np.float32), S0


def _unit(rng, n):
    x = rng.standard_normal((n, H, DK))
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("dv", [128, 64])
def test_alpha_to_zero_inside_chunks_prefill(gpu, dv):
    _announce(f"edge: alpha -> 0 at single tokens (a_raw = 40), prefill matrix path dv={dv}")
    L = _lengths()
    cu, q, k, v, g, beta, S0 = _spiky_inputs(106, dv, L)
    assert g.min() < -30.0
    y, ST = _prefill(q, k, v, g, beta, S0, cu, y_dtype="bf16")
    al = np.exp(g.astype(np.float64))
    y_ref, S_ref = oracle.recurrence(gi.as_f64(q, True), gi.as_f64(k, True), gi.as_f64(v, True),
                                     al, beta.astype(np.float64), S0.astype(np.float64), cu)
    ey = C.assert_close("y", C.host(y), y_ref, True, stored_bf16=True, cu=cu, H=H)
    es = C.assert_close("S_T", C.host(ST), S_ref, True, state=True)
    print(f"  alpha -> 0: max slice rel L2 y {ey:.2e}, S_T {es:.2e}")


def test_alpha_to_zero_decode(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("edge: alpha -> 0 at some steps, decode")
    L = [6] * 8
    cu, q, k, v, g, beta, S0 = _spiky_inputs(107, DK, L, spikes=[2, 5, 8, 20, 33, 47])
    N, steps = len(L), L[0]
    state = C.dev(S0)
    ys = []
    for s in range(steps):
        idx = cu[:-1] + s                     # token s of every sequence
        ys.append(gdn.gdn_decode_step(C.dev(q[idx], True), C.dev(k[idx], True),
                                      C.dev(v[idx], True), C.dev(g[idx]), C.dev(beta[idx]),
                                      state, y_dtype="f32"))
    torch.cuda.synchronize()
    y = np.stack([C.host(t) for t in ys], axis=1).reshape(N * steps, H, DK)
    y_ref, S_ref = oracle.recurrence(gi.as_f64(q, True), gi.as_f64(k, True), gi.as_f64(v, True),
                                     np.exp(g.astype(np.float64)), beta.astype(np.float64),
                                     S0.astype(np.float64), cu)
    ey = C.assert_close("y", y, y_ref, True, cu=cu, H=H)
    es = C.assert_close("S", C.host(state), S_ref, True, state=True)
    print(f"  decode alpha -> 0: max slice rel L2 y {ey:.2e}, S {es:.2e}")


@pytest.mark.parametrize("where", ["k", "v"])
def test_nan_stays_in_its_slice_prefill(gpu, where):
    import torch
    _announce(f"edge: NaN in {where} of one (sequence, head), prefill matrix path")
    dv = 128
    L = _lengths()
    cu, q, k, v, g, beta, S0 = _spiky_inputs(108, dv, L)
    y0, S0_out = _prefill(q, k, v, g, beta, S0, cu, y_dtype="bf16")
    seq, t, h, c = 0, 70, 1, 37             # token 70 of sequence 0 (second chunk), head 1
    nan_bf16 = np.uint16(0x7FC0)
    if where == "k":
        k = k.copy()
        k[cu[seq] + t, h, c] = nan_bf16
    else:
        v = v.copy()
        v[cu[seq] + t, h, c] = nan_bf16
    y1, S1 = _prefill(q, k, v, g, beta, S0, cu, y_dtype="bf16")
    a, b = y0.view(torch.int16).cpu().numpy(), y1.view(torch.int16).cpu().numpy()
    sa, sb = S0_out.cpu().numpy(), S1.cpu().numpy()
    lo, hi = cu[seq], cu[seq + 1]
    chunk0 = lo + (t // 64) * 64            # the NaN's chunk: earlier chunks are untouched
    keep = np.ones(a.shape, bool)
    if where == "k":
        keep[chunk0:hi, h, :] = False
    else:
        keep[chunk0:hi, h, c] = False
    assert np.array_equal(a[keep], b[keep]), "a NaN leaked out of its slice (y)"
    assert np.isnan(C.host(y1)[~keep]).any(), "the NaN did not reach y"
    keep_s = np.ones(sa.shape, bool)
    if where == "k":
        keep_s[seq, h] = False
    else:
        keep_s[seq, h, :, c] = False
    assert np.array_equal(sa[keep_s], sb[keep_s]), "a NaN leaked out of its slice (S_T)"
    print(f"  NaN in {where}: every other slice{' and column' if where == 'v' else ''} "
          "unchanged bit for bit")


def test_nan_stays_in_its_slice_decode(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce("edge: NaN in one head's state, decode")
    rng = np.random.default_rng(109)
    N = 8
    S0 = (0.1 * rng.standard_normal((N, H, DK, DK))).astype(np.float32)
    q = gi.f32_to_bf16_bits(_unit(rng, N))
    k = gi.f32_to_bf16_bits(_unit(rng, N))
    v = gi.f32_to_bf16_bits(rng.standard_normal((N, H, DK)).astype(np.float32))
    g = _config_gates(rng, N, H)
    beta = rng.uniform(0.1, 0.9, size=(N, H)).astype(np.float32)
    outs = []
    for poison in (False, True):
        S = S0.copy()
        if poison:
            S[3, 1, 10, 20] = np.nan
        st = C.dev(S)
        y = gdn.gdn_decode_step(C.dev(q, True), C.dev(k, True), C.dev(v, True), C.dev(g),
                                C.dev(beta), st, y_dtype="f32")
        torch.cuda.synchronize()
        outs.append((y.cpu().numpy(), st.cpu().numpy()))
    (ya, sa), (yb, sb) = outs
    keep = np.ones(ya.shape, bool)
    keep[3, 1] = False
    assert np.array_equal(ya[keep], yb[keep])
    keep_s = np.ones(sa.shape, bool)
    keep_s[3, 1] = False
    assert np.array_equal(sa[keep_s], sb[keep_s])
    assert np.isnan(yb[3, 1]).any()
    print("  decode NaN: every other head unchanged bit for bit")
