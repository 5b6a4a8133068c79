"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check compares the oracle with something other than itself: the closed
form eq. (5), exact rational brute force of the product expansion, closed forms
for special gates, invariants the pages state (erase-then-write), library
routines (numpy.convolve, numpy matmul) and mpmath at high precision.
Source: reading notes of "On the Design of Qwen3.8-Next Architecture",
section 2.1.1, eqs. (1)-(11).
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(12345)


def _rand_case(T, H, dk, dv, unit_k=True, seed=0, nseq_cu=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    al = rng.uniform(0.3, 0.999, (T, H))
    be = rng.uniform(0.01, 0.99, (T, H))
    return q, k, v, al, be


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------- P1: eq. 5 == eqs. 1-3
@pytest.mark.parametrize("unit_k", [True, False])
def test_eq5_closed_form_equals_eqs_1_to_3(unit_k):
    q, k, v, al, be = _rand_case(80, 3, 16, 12, unit_k=unit_k, seed=1)
    S0 = np.random.default_rng(2).standard_normal((2, 3, 16, 12))
    cu = [0, 37, 80]
    y1, s1 = oracle.recurrence(q, k, v, al, be, S0, cu)
    y2, s2 = oracle.recurrence(q, k, v, al, be, S0, cu, closed_form=True)
    assert _rel(y1, y2) < 1e-13
    assert _rel(s1, s2) < 1e-13


# ---------------------------------------------------------------- P2: alpha = 1, beta = 0
def test_unit_decay_zero_write_leaves_state():
    q, k, v, al, be = _rand_case(40, 2, 8, 8, seed=3)
    al[:] = 1.0
    be[:] = 0.0
    S0 = np.random.default_rng(4).standard_normal((1, 2, 8, 8))
    y, ST = oracle.recurrence(q, k, v, al, be, S0)
    assert np.array_equal(ST, S0)
    for h in range(2):
        ref = q[:, h, :] @ S0[0, h]          # y_t = S0^T q_t  (numpy matmul)
        assert np.allclose(y[:, h, :], ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- P3: erase-then-write
def test_full_write_strength_stores_value_exactly():
    """beta = 1 and ||k|| = 1: eq. 2-3 give S_t^T k_t = alpha S^T k + (k.k)(v - alpha S^T k) = v_t.
    Reading with q_t = k_t returns v_t at every step."""
    q, k, v, al, be = _rand_case(60, 2, 32, 16, unit_k=True, seed=5)
    be[:] = 1.0
    S0 = np.random.default_rng(6).standard_normal((1, 2, 32, 16))
    y, _ = oracle.recurrence(k, k, v, al, be, S0)
    assert np.max(np.abs(y - v)) < 1e-12


# ---------------------------------------------------------------- P4: brute force
def _frac_matmul(A, B):
    return [[sum((A[i][l] * B[l][j] for l in range(len(B))), Fraction(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def _frac_add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _brute_force_state(alpha, beta, k, v, S0, t_end, one, matmul, add):
    """S_t = A_t ... A_1 S0 + sum_s A_t ... A_{s+1} beta_s k_s v_s^T with A_s = alpha_s (I - beta_s k_s k_s^T)."""
    dk = len(S0)

    def A(s):
        return [[alpha[s] * ((one if i == j else 0 * one) - beta[s] * k[s][i] * k[s][j])
                 for j in range(dk)] for i in range(dk)]

    def prod(lo, hi):  # A_hi ... A_lo (1-based inclusive), identity if empty
        P = [[one if i == j else 0 * one for j in range(dk)] for i in range(dk)]
        for s in range(lo, hi + 1):
            P = matmul(A(s - 1), P)
        return P

    S = matmul(prod(1, t_end), S0)
    for s in range(1, t_end + 1):
        outer = [[beta[s - 1] * k[s - 1][i] * v[s - 1][j] for j in range(len(S0[0]))]
                 for i in range(dk)]
        S = add(S, matmul(prod(s + 1, t_end), outer))
    return S


def test_bruteforce_exact_rationals():
    rng = np.random.default_rng(7)
    T, dk, dv = 7, 4, 3
    F = lambda x: Fraction(int(x), 64)  # noqa: E731
    k = [[F(rng.integers(-64, 65)) for _ in range(dk)] for _ in range(T)]      # not unit-norm
    q = [[F(rng.integers(-64, 65)) for _ in range(dk)] for _ in range(T)]
    v = [[F(rng.integers(-64, 65)) for _ in range(dv)] for _ in range(T)]
    alpha = [Fraction(int(rng.integers(20, 64)), 64) for _ in range(T)]
    beta = [Fraction(int(rng.integers(1, 64)), 64) for _ in range(T)]
    S0 = [[F(rng.integers(-64, 65)) for _ in range(dv)] for _ in range(dk)]

    to = lambda M: np.array([[float(x) for x in r] for r in M])  # noqa: E731
    y, ST = oracle.recurrence(to(q)[:, None, :], to(k)[:, None, :], to(v)[:, None, :],
                              np.array([[float(a)] for a in alpha]),
                              np.array([[float(b)] for b in beta]), to(S0)[None, None])
    for t in range(1, T + 1):
        St = _brute_force_state(alpha, beta, k, v, S0, t, Fraction(1), _frac_matmul, _frac_add)
        yt = [sum((St[i][j] * q[t - 1][i] for i in range(dk)), Fraction(0)) for j in range(dv)]
        ref = np.array([float(x) for x in yt])
        assert _rel(y[t - 1, 0], ref) < 1e-12
    assert _rel(ST[0, 0], to(St)) < 1e-12


def test_bruteforce_mpmath_50_digits():
    mpmath.mp.dps = 50
    q, k, v, al, be = _rand_case(9, 1, 12, 5, unit_k=True, seed=8)
    S0 = np.random.default_rng(9).standard_normal((1, 1, 12, 5))
    y, ST = oracle.recurrence(q, k, v, al, be, S0)
    mk = lambda a: mpmath.matrix(a.tolist())  # noqa: E731
    alpha = [mpmath.mpf(x) for x in al[:, 0]]
    beta = [mpmath.mpf(x) for x in be[:, 0]]
    kk = [[mpmath.mpf(x) for x in r] for r in k[:, 0]]
    vv = [[mpmath.mpf(x) for x in r] for r in v[:, 0]]
    one = mpmath.mpf(1)

    def mm(A, B):
        return (mpmath.matrix(A) * mpmath.matrix(B)).tolist()

    def add(A, B):
        return (mpmath.matrix(A) + mpmath.matrix(B)).tolist()

    S = _brute_force_state(alpha, beta, kk, vv, mk(S0[0, 0]).tolist(), 9, one, mm, add)
    ref = np.array([[float(x) for x in r] for r in S])
    assert _rel(ST[0, 0], ref) < 1e-13
    yt = np.array([float(x) for x in (mpmath.matrix(S).T * mpmath.matrix(q[8, 0].tolist()))])
    assert _rel(y[8, 0], yt) < 1e-13


# ---------------------------------------------------------------- P5: beta = 0
def test_zero_write_is_pure_decay():
    q, k, v, al, be = _rand_case(50, 2, 8, 6, seed=10)
    be[:] = 0.0
    S0 = np.random.default_rng(11).standard_normal((1, 2, 8, 6))
    y, ST = oracle.recurrence(q, k, v, al, be, S0)
    gam = np.cumprod(al, axis=0)
    for h in range(2):
        ref = gam[:, h, None] * (q[:, h, :] @ S0[0, h])
        assert np.allclose(y[:, h], ref, rtol=1e-12, atol=1e-14)
        assert _rel(ST[0, h], gam[-1, h] * S0[0, h]) < 1e-13


# ---------------------------------------------------------------- P6: orthonormal keys
def test_basis_keys_overwrite_rows():
    dk, dv, T = 10, 7, 6
    rng = np.random.default_rng(12)
    perm = rng.permutation(dk)[:T]
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, perm] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    _, ST = oracle.recurrence(q, k, v, np.ones((T, 1)), np.ones((T, 1)), S0)
    expect = S0[0, 0].copy()
    expect[perm] = v[:, 0, :]
    assert np.max(np.abs(ST[0, 0] - expect)) < 1e-14


# ---------------------------------------------------------------- P7: linearity in (v, S0)
def test_linear_in_values_and_initial_state():
    q, k, v1, al, be = _rand_case(30, 2, 8, 8, seed=13)
    v2 = np.random.default_rng(14).standard_normal(v1.shape)
    s1 = np.random.default_rng(15).standard_normal((1, 2, 8, 8))
    s2 = np.random.default_rng(16).standard_normal((1, 2, 8, 8))
    a, b = 0.7, -1.3
    y1, t1 = oracle.recurrence(q, k, v1, al, be, s1)
    y2, t2 = oracle.recurrence(q, k, v2, al, be, s2)
    y3, t3 = oracle.recurrence(q, k, a * v1 + b * v2, al, be, a * s1 + b * s2)
    assert _rel(y3, a * y1 + b * y2) < 1e-12
    assert _rel(t3, a * t1 + b * t2) < 1e-12


# ---------------------------------------------------------------- packing invariants
def test_packed_sequences_are_independent_and_empty_sequence_keeps_state():
    q, k, v, al, be = _rand_case(50, 2, 8, 4, seed=17)
    S0 = np.random.default_rng(18).standard_normal((3, 2, 8, 4))
    cu = [0, 20, 20, 50]        # middle sequence is empty
    y, ST = oracle.recurrence(q, k, v, al, be, S0, cu)
    assert np.array_equal(ST[1], S0[1])
    for s, (lo, hi) in enumerate([(0, 20), (20, 50)]):
        idx = 0 if s == 0 else 2
        ys, Ss = oracle.recurrence(q[lo:hi], k[lo:hi], v[lo:hi], al[lo:hi], be[lo:hi], S0[idx:idx + 1])
        assert np.array_equal(ys, y[lo:hi])
        assert np.array_equal(Ss[0], ST[idx])


def test_single_steps_chain_equals_one_call():
    """Decode semantics: feeding S_T back as S0 token by token equals one prefill call."""
    q, k, v, al, be = _rand_case(12, 2, 8, 4, seed=19)
    y, ST = oracle.recurrence(q, k, v, al, be)
    S = np.zeros((1, 2, 8, 4))
    for t in range(12):
        yt, S = oracle.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], al[t:t + 1], be[t:t + 1], S)
        assert np.array_equal(yt[0], y[t])
    assert np.array_equal(S, ST)


# ---------------------------------------------------------------- eqs. 6-8 pins
def test_conv_identity_and_shift_taps():
    rng = np.random.default_rng(20)
    x = rng.standard_normal((30, 5))
    cu = [0, 11, 30]
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (5, 1))
    assert np.array_equal(oracle.short_conv(x, ident, cu), x)
    shift = np.tile([1.0, 0.0, 0.0, 0.0], (5, 1))        # oldest tap: x[t-3], zero before start
    u = oracle.short_conv(x, shift, cu)
    for lo, hi in [(0, 11), (11, 30)]:
        assert np.all(u[lo:lo + 3] == 0.0)
        assert np.array_equal(u[lo + 3:hi], x[lo:hi - 3])


def test_conv_matches_numpy_convolve_with_resets():
    rng = np.random.default_rng(21)
    C, K = 6, 4
    x = rng.standard_normal((40, C))
    w = rng.standard_normal((C, K))
    cu = [0, 2, 17, 40]          # includes a sequence shorter than K
    u = oracle.short_conv(x, w, cu)
    for lo, hi in zip(cu[:-1], cu[1:]):
        for c in range(C):
            # causal cross-correlation == convolution with reversed taps, truncated to 'full'[:n]
            ref = np.convolve(x[lo:hi, c], w[c, ::-1], mode="full")[: hi - lo]
            assert np.allclose(u[lo:hi, c], ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------- conv with a carried history
def _joined(hist_rows, piece):
    return np.concatenate([hist_rows, piece], axis=0)


def test_conv_history_matches_numpy_convolve_over_the_joined_stream():
    rng = np.random.default_rng(22)
    C, K = 5, 4
    x = rng.standard_normal((23, C))
    w = rng.standard_normal((C, K))
    cu = [0, 0, 1, 3, 10, 23]      # empty, 1- and 2-token sequences keep part of the history
    hist = rng.standard_normal((len(cu) - 1, K - 1, C))
    u, hout = oracle.short_conv_hist(x, w, cu, hist)
    for s, (lo, hi) in enumerate(zip(cu[:-1], cu[1:])):
        ext = _joined(hist[s], x[lo:hi])
        for c in range(C):
            ref = np.convolve(ext[:, c], w[c, ::-1], mode="full")[K - 1: K - 1 + hi - lo]
            assert np.allclose(u[lo:hi, c], ref, rtol=1e-14, atol=1e-14)
        # the carried history is the last K-1 rows of the joined stream, oldest first
        assert np.array_equal(hout[s], ext[-(K - 1):])


def test_conv_history_oldest_tap_reads_history_rows_in_order():
    rng = np.random.default_rng(23)
    C = 3
    x = rng.standard_normal((6, C))
    hist = rng.standard_normal((1, 3, C))
    shift = np.tile([1.0, 0.0, 0.0, 0.0], (C, 1))        # u[t] = input three positions back
    u, _ = oracle.short_conv_hist(x, shift, [0, 6], hist)
    assert np.array_equal(u[:3], hist[0])                 # row 0 is the oldest input
    assert np.array_equal(u[3:], x[:3])


def test_conv_history_split_stream_equals_whole_sequence():
    rng = np.random.default_rng(24)
    C, K, n = 4, 4, 57
    x = rng.standard_normal((n, C))
    w = rng.standard_normal((C, K))
    whole = oracle.short_conv(x, w, [0, n])
    cuts = [0, 0, 1, 3, 4, 20, 21, 21, 40, n]            # pieces of 0, 1, 2, 1, 16, ... tokens
    hist = np.zeros((1, K - 1, C))
    parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        u, hist = oracle.short_conv_hist(x[lo:hi], w, [0, hi - lo], hist)
        parts.append(u)
    assert np.allclose(np.concatenate(parts), whole, rtol=0, atol=1e-15)
    assert np.array_equal(hist[0], x[-(K - 1):])
    # no history given == zero history == the resetting conv
    u0, h0 = oracle.short_conv_hist(x, w, [0, 30, n])
    assert np.array_equal(u0, oracle.short_conv(x, w, [0, 30, n]))
    assert np.array_equal(h0[0], x[27:30]) and np.array_equal(h0[1], x[n - 3:])


def test_activations_against_mpmath():
    mpmath.mp.dps = 40
    xs = np.array([-30.0, -7.5, -1.0, -1e-3, 0.0, 0.3, 2.0, 9.0, 25.0])
    a = oracle.silu(xs)
    for x, got in zip(xs, a):
        ref = mpmath.mpf(x) / (1 + mpmath.e ** (-mpmath.mpf(x)))
        assert abs(got - float(ref)) <= 1e-15 * max(1.0, abs(float(ref)))
    # gates: beta = sigmoid(b), alpha = exp(-exp(A) softplus(a + bias))
    A_log = np.array([0.0, np.log(7.0)])
    dt_bias = np.array([-4.6, -4.6])
    a_raw = np.array([[-3.0, 0.5], [4.6, 12.0], [40.0, -40.0]])
    b_raw = np.array([[0.0, -2.0], [3.0, 30.0], [-30.0, 1e-3]])
    g, al, be = oracle.gates(a_raw, b_raw, A_log, dt_bias)
    for t in range(3):
        for h in range(2):
            x = mpmath.mpf(a_raw[t, h]) + mpmath.mpf(dt_bias[h])
            sp = mpmath.log(1 + mpmath.e ** x)
            gr = -mpmath.e ** mpmath.mpf(A_log[h]) * sp
            assert abs(g[t, h] - float(gr)) <= 1e-14 * abs(float(gr))
            assert abs(al[t, h] - float(mpmath.e ** gr)) <= 1e-14 * float(mpmath.e ** gr)
            br = 1 / (1 + mpmath.e ** (-mpmath.mpf(b_raw[t, h])))
            assert abs(be[t, h] - float(br)) <= 1e-15
    assert be[0, 0] == 0.5


def test_gate_special_values():
    """softplus(0) = ln 2, so alpha = 2^(-exp(A)) when a_raw + b_alpha = 0; beta(0) = 1/2."""
    A_log = np.log(np.array([1.0, 3.0, 16.0]))
    dt = np.array([-4.6, -4.6, -4.6])
    g, al, be = oracle.gates(np.full((1, 3), 4.6), np.zeros((1, 3)), A_log, dt)
    assert np.allclose(al[0], 2.0 ** -np.exp(A_log), rtol=1e-14)
    assert np.all(be == 0.5)
    assert np.all((al > 0) & (al < 1))
    # far into the linear branch softplus(x) = x: no overflow of exp(x)
    g, _, _ = oracle.gates(np.full((1, 1), 800.0), np.zeros((1, 1)), np.zeros(1), np.zeros(1))
    assert g[0, 0] == -800.0


def test_l2norm_unit_and_epsilon():
    rng = np.random.default_rng(22)
    a = rng.standard_normal((7, 3, 64)) * 5
    assert np.allclose(np.linalg.norm(oracle.l2norm(a, eps=0.0), axis=-1), 1.0, rtol=1e-15, atol=0)
    out = oracle.l2norm(a, eps=1e-6)
    ss = np.sum(a * a, axis=-1)
    assert np.allclose(np.linalg.norm(out, axis=-1), np.sqrt(ss / (ss + 1e-6)), rtol=1e-14)
    assert np.array_equal(oracle.l2norm(np.zeros((1, 8)), eps=1e-6), np.zeros((1, 8)))


# ---------------------------------------------------------------- eq. 11 pins
def test_output_gate_constant_rows_and_scale_invariance():
    dv = 16
    w = np.random.default_rng(23).standard_normal(dv) * 0.1
    for c in [-3.0, 0.25, 7.0]:
        y = np.full((1, dv), c)
        z = np.zeros((1, dv))
        o = oracle.output_gate(y, z, w, eps=0.0)
        assert np.allclose(o[0], 0.5 * (1 + w) * np.sign(c), rtol=1e-15, atol=1e-15)
    rng = np.random.default_rng(24)
    y = rng.standard_normal((5, dv))
    z = rng.standard_normal((5, dv))
    o1 = oracle.output_gate(y, z, w, eps=0.0)
    o2 = oracle.output_gate(y * 37.0, z, w, eps=0.0)
    assert _rel(o1, o2) < 1e-14
    # w = 0 and a saturated gate: RMS of the output is one
    o3 = oracle.output_gate(y, np.full_like(y, 800.0), np.zeros(dv), eps=0.0)
    assert np.allclose(np.sqrt(np.mean(o3 * o3, axis=-1)), 1.0, rtol=1e-14)


def test_bf16_storage_rounding_matches_torch():
    import torch
    x = np.random.default_rng(25).standard_normal(50000) * 7
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.round_bf16(x), ref)


# ---------------------------------------------------------------- gradients of eqs. 1-4
def _fd_check(T, H, dk, dv, cu, seed, n_probe=None):
    """Central finite differences of L = <y, Wy> + <S_T, WS> against the oracle's reverse-mode
    gradients, for every input element (or n_probe random ones per input)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    al = rng.uniform(0.5, 0.99, (T, H))
    be = rng.uniform(0.1, 0.9, (T, H))
    nseq = len(cu) - 1
    S0 = rng.standard_normal((nseq, H, dk, dv))
    Wy = rng.standard_normal((T, H, dv))
    WS = rng.standard_normal((nseq, H, dk, dv))

    def loss():
        y, ST = oracle.recurrence(q, k, v, al, be, S0, cu, nthreads=1)
        return float((y * Wy).sum() + (ST * WS).sum())

    grads = oracle.recurrence_backward(q, k, v, al, be, Wy, S0, WS, cu, nthreads=1)
    h = 1e-6
    for arr, key in ((q, "dq"), (k, "dk"), (v, "dv"), (al, "dalpha"), (be, "dbeta"), (S0, "dS0")):
        idxs = list(np.ndindex(arr.shape))
        if n_probe is not None:
            idxs = [idxs[i] for i in rng.choice(len(idxs), min(n_probe, len(idxs)), replace=False)]
        for idx in idxs:
            a0 = arr[idx]
            arr[idx] = a0 + h
            lp = loss()
            arr[idx] = a0 - h
            lm = loss()
            arr[idx] = a0
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grads[key][idx]) <= 1e-6 * max(1.0, abs(fd)), (key, idx, fd, grads[key][idx])
    return grads


def test_backward_matches_finite_differences():
    _fd_check(T=9, H=2, dk=3, dv=4, cu=[0, 4, 4, 9], seed=30)     # includes an empty sequence


def test_backward_across_checkpoint_blocks_matches_finite_differences():
    # 150 tokens: the oracle recomputes states from checkpoints every 64 tokens
    _fd_check(T=150, H=1, dk=2, dv=3, cu=[0, 150], seed=31, n_probe=12)


def test_backward_zero_write_is_pure_decay():
    # beta = 0: S_T = (prod alpha) S0 and y_t = (prod_{i<=t} alpha_i) S0^T q_t, so with dy = 0
    # the state gradient is transported back with the same product
    rng = np.random.default_rng(32)
    T, dk, dv = 20, 4, 5
    q, k = rng.standard_normal((T, 1, dk)), rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    al = rng.uniform(0.6, 0.99, (T, 1))
    be = np.zeros((T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    dST = rng.standard_normal((1, 1, dk, dv))
    g = oracle.recurrence_backward(q, k, v, al, be, np.zeros((T, 1, dv)), S0, dST)
    assert np.allclose(g["dS0"], np.prod(al) * dST, rtol=1e-13, atol=0)
    assert np.all(g["dv"] == 0.0)
    assert np.allclose(g["dg"], np.full((T, 1), np.sum(dST * np.prod(al) * S0)), rtol=1e-12)


# ---------------------------------------------------------------- per-channel decay (KDA)
def _kda_case(T, H, dk, dv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    al = rng.uniform(0.3, 0.999, (T, H, dk))
    be = rng.uniform(0.05, 0.95, (T, H))
    return q, k, v, al, be


def test_kda_with_equal_channel_decays_is_gdn():
    q, k, v, _, be = _kda_case(50, 2, 8, 6, seed=40)
    al = np.random.default_rng(41).uniform(0.3, 0.999, (50, 2))
    S0 = np.random.default_rng(42).standard_normal((2, 2, 8, 6))
    cu = [0, 23, 50]
    y1, s1 = oracle.kda_recurrence(q, k, v, np.repeat(al[:, :, None], 8, axis=2), be, S0, cu)
    y2, s2 = oracle.recurrence(q, k, v, al, be, S0, cu)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_kda_zero_write_decays_each_row_by_its_own_product():
    q, k, v, al, be = _kda_case(30, 1, 5, 4, seed=43)
    be[:] = 0.0
    S0 = np.random.default_rng(44).standard_normal((1, 1, 5, 4))
    y, ST = oracle.kda_recurrence(q, k, v, al, be, S0)
    cum = np.cumprod(al[:, 0, :], axis=0)                     # [T, dk]
    assert np.allclose(ST[0, 0], cum[-1][:, None] * S0[0, 0], rtol=1e-13, atol=0)
    ref = np.einsum("ti,ti,ij->tj", q[:, 0], cum, S0[0, 0])
    assert np.allclose(y[:, 0], ref, rtol=1e-12, atol=1e-14)


def test_kda_channel_permutation_equivariance():
    q, k, v, al, be = _kda_case(40, 1, 7, 3, seed=45)
    S0 = np.random.default_rng(46).standard_normal((1, 1, 7, 3))
    perm = np.random.default_rng(47).permutation(7)
    y1, s1 = oracle.kda_recurrence(q, k, v, al, be, S0)
    y2, s2 = oracle.kda_recurrence(q[:, :, perm], k[:, :, perm], v, al[:, :, perm], be,
                                   S0[:, :, perm])
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-13)
    assert np.allclose(s1[:, :, perm], s2, rtol=1e-12, atol=1e-13)


def test_kda_full_write_strength_stores_value():
    q, k, v, al, be = _kda_case(25, 1, 6, 4, seed=48)
    be[:] = 1.0
    y, _ = oracle.kda_recurrence(k, k, v, al, be)            # read back with q = k
    assert np.allclose(y, v, rtol=1e-12, atol=1e-12)
