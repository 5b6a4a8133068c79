"""fp64 CPU oracle for the Gated DeltaNet token mixer (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library; both sides are fed the same raw draws from the input generator.

Every function follows the reading notes of "On the Design of Qwen3.8-Next
Architecture", section 2.1.1: eqs. (1)-(5) for the recurrence, eqs. (6)-(10) for
the pre-processing and gates, eq. (11) (without W_o) for the output gate; the
C source states the passage per function.

Parity status: the recurrence, conv (with and without a carried history), SiLU, L2Norm,
gates and output gate are all
pinned by the CPU tests (closed forms, invariants, exact-rational brute force,
library routines). The conventions the pages leave open (conv tap order, the
epsilons, RMSNorm scope) are pinned only by the stated readings.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

L2_EPS = 1e-6
RMS_EPS = 1e-6
CONV_K = 4

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.gdn_oracle_short_conv.argtypes = [_dp, _dp, ctypes.c_int, _ip, ctypes.c_int,
                                              ctypes.c_int, _dp]
        lib.gdn_oracle_short_conv_hist.argtypes = [_dp, _dp, ctypes.c_int, _ip, ctypes.c_int,
                                                   ctypes.c_int, _dp, _dp, _dp]
        lib.gdn_oracle_silu.argtypes = [_dp, ctypes.c_long, _dp]
        lib.gdn_oracle_l2norm.argtypes = [_dp, ctypes.c_long, ctypes.c_int, ctypes.c_double, _dp]
        lib.gdn_oracle_gates.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_long, ctypes.c_int,
                                         _dp, _dp, _dp]
        lib.gdn_oracle_recurrence.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_recurrence.restype = ctypes.c_int
        lib.gdn_oracle_kda_recurrence.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp,
                                                  _dp, ctypes.c_int]
        lib.gdn_oracle_kda_recurrence.restype = ctypes.c_int
        lib.gdn_oracle_recurrence_backward.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip,
                                                       ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_int, _dp, _dp, _dp, _dp, _dp,
                                                       _dp, _dp, _dp, ctypes.c_int]
        lib.gdn_oracle_recurrence_backward.restype = ctypes.c_int
        lib.gdn_oracle_output_gate.argtypes = [_dp, _dp, _dp, ctypes.c_long, ctypes.c_int,
                                               ctypes.c_double, _dp]
        _lib = lib
    return _lib


def _d(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(_dp)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ------------------------------------------------------------------ eqs. 6-8
def short_conv(x, w, cu_seqlens):
    """x: [ntok, C]; w: [C, K] (tap K-1 = current token); zero history per sequence."""
    x = _d(x)
    w = _d(w)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ntok, C = x.shape
    u = np.empty_like(x)
    _load().gdn_oracle_short_conv(_p(x), _p(w), w.shape[1], cu.ctypes.data_as(_ip),
                                  len(cu) - 1, C, _p(u))
    return u


def short_conv_hist(x, w, cu_seqlens, hist_in=None):
    """ShortConv continuing earlier input: x: [ntok, C]; w: [C, K]; hist_in: [nseq, K-1, C]
    (row K-2 = the input just before each sequence start) or None (zero history).
    Returns (u [ntok, C], hist_out [nseq, K-1, C]): hist_out holds the last K-1 inputs of
    history + sequence, ready to be the next call's hist_in."""
    x = _d(x)
    w = _d(w)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ntok, C = x.shape
    K = w.shape[1]
    nseq = len(cu) - 1
    hin = None if hist_in is None else _d(hist_in)
    u = np.empty_like(x)
    hout = np.empty((nseq, K - 1, C))
    _load().gdn_oracle_short_conv_hist(_p(x), _p(w), K, cu.ctypes.data_as(_ip), nseq, C,
                                       _p(hin), _p(u), _p(hout))
    return u, hout


def silu(u):
    u = _d(u)
    a = np.empty_like(u)
    _load().gdn_oracle_silu(_p(u), u.size, _p(a))
    return a


def l2norm(a, eps=L2_EPS):
    a = _d(a)
    d = a.shape[-1]
    out = np.empty_like(a)
    _load().gdn_oracle_l2norm(_p(a), a.size // d, d, eps, _p(out))
    return out


# ------------------------------------------------------------------ eqs. 9-10
def gates(a_raw, b_raw, A_log, dt_bias):
    """Returns (g = log alpha, alpha, beta), each shaped like a_raw ([..., H])."""
    a_raw = _d(a_raw)
    b_raw = _d(b_raw)
    H = a_raw.shape[-1]
    g = np.empty_like(a_raw)
    al = np.empty_like(a_raw)
    be = np.empty_like(a_raw)
    _load().gdn_oracle_gates(_p(a_raw), _p(b_raw), _p(_d(A_log)), _p(_d(dt_bias)),
                             a_raw.size // H, H, _p(g), _p(al), _p(be))
    return g, al, be


# ------------------------------------------------------------------ eqs. 1-5
def recurrence(q, k, v, alpha, beta, S0=None, cu_seqlens=None, closed_form=False, nthreads=None):
    """Token-by-token gated delta rule. q,k: [ntok,H,dk]; v: [ntok,H,dv]; alpha,beta: [ntok,H];
    S0: [nseq,H,dk,dv] or None. Returns (y [ntok,H,dv], S_T [nseq,H,dk,dv])."""
    q = _d(q)
    k = _d(k)
    v = _d(v)
    alpha = _d(alpha)
    beta = _d(beta)
    ntok, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = [0, ntok]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = len(cu) - 1
    s0 = None if S0 is None else _d(S0)
    y = np.zeros((ntok, H, dv))
    ST = np.zeros((nseq, H, dk, dv))
    _load().gdn_oracle_recurrence(_p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(s0),
                                  cu.ctypes.data_as(_ip), nseq, H, dk, dv, int(closed_form),
                                  _p(y), _p(ST), nthreads or default_threads())
    return y, ST


def kda_recurrence(q, k, v, alpha, beta, S0=None, cu_seqlens=None, nthreads=None):
    """The delta rule with a per-channel decay alpha [ntok, H, dk] (Kimi Delta Attention's
    diagonal gate in place of GDN's scalar): row i of the state decays by alpha_t[i].
    Returns (y [ntok,H,dv], S_T [nseq,H,dk,dv])."""
    q, k, v, alpha, beta = (_d(x) for x in (q, k, v, alpha, beta))
    ntok, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = [0, ntok]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = len(cu) - 1
    s0 = None if S0 is None else _d(S0)
    y = np.zeros((ntok, H, dv))
    ST = np.zeros((nseq, H, dk, dv))
    _load().gdn_oracle_kda_recurrence(_p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(s0),
                                      cu.ctypes.data_as(_ip), nseq, H, dk, dv, _p(y), _p(ST),
                                      nthreads or default_threads())
    return y, ST


def recurrence_backward(q, k, v, alpha, beta, dy, S0=None, dST=None, cu_seqlens=None,
                        nthreads=None):
    """Gradients of eqs. 1-4 (reverse mode, token by token). Shapes as recurrence(); dy like
    y, dST like S_T (None = zero). Returns dict(dq, dk, dv, dalpha, dbeta, dg, dS0) where
    dg = dalpha * alpha is the gradient with respect to g = log alpha."""
    q, k, v, alpha, beta, dy = (_d(x) for x in (q, k, v, alpha, beta, dy))
    ntok, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = [0, ntok]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    nseq = len(cu) - 1
    s0 = None if S0 is None else _d(S0)
    dst = None if dST is None else _d(dST)
    out = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               dalpha=np.zeros_like(alpha), dbeta=np.zeros_like(beta),
               dS0=np.zeros((nseq, H, dk, dv)))
    _load().gdn_oracle_recurrence_backward(
        _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(s0), cu.ctypes.data_as(_ip), nseq, H, dk,
        dv, _p(dy), _p(dst), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dalpha"]),
        _p(out["dbeta"]), _p(out["dS0"]), nthreads or default_threads())
    out["dg"] = out["dalpha"] * alpha
    return out


# ------------------------------------------------------------------ eq. 11 without W_o
def output_gate(y, z, w, eps=RMS_EPS):
    """o = sigmoid(z) * (1 + w) * y / sqrt(mean(y^2) + eps) over the last axis."""
    y = _d(y)
    z = _d(z)
    dv = y.shape[-1]
    o = np.empty_like(y)
    _load().gdn_oracle_output_gate(_p(y), _p(z), _p(_d(w)), y.size // dv, dv, eps, _p(o))
    return o


# ------------------------------------------------------------------ storage format
def round_bf16(x):
    """Values as stored in bfloat16: fp64 -> fp32 (round to nearest even) -> bf16 (round to
    nearest even), widened back to fp64. Models a path that keeps an intermediate in bf16."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    b = ((u + r) >> np.uint32(16)) << np.uint32(16)
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ whole token mixer
def preprocess(xq, xk, xv, wq, wk, wv, cu_seqlens, H, l2_eps=L2_EPS):
    """eqs. 6-8 on pre-conv streams x* [ntok,H,d] (float64 values); w* [H*d, K]."""
    ntok = xq.shape[0]

    def stream(x, w, norm):
        d = x.shape[2]
        a = silu(short_conv(x.reshape(ntok, H * d), w, cu_seqlens)).reshape(ntok, H, d)
        return l2norm(a, l2_eps) if norm else a

    return stream(xq, wq, True), stream(xk, wk, True), stream(xv, wv, False)


def preprocess_stateful(xq, xk, xv, wq, wk, wv, cu_seqlens, H, conv_state_in=None,
                        l2_eps=L2_EPS):
    """eqs. 6-8 for sequences that continue earlier input. conv_state_in: [nseq, K-1, C_all]
    or None, with C_all = H*(2 dk + dv) channels ordered q | k | v. Returns
    (q, k, v, conv_state_out) with conv_state_out in the same layout."""
    ntok = xq.shape[0]
    dk, dv = xq.shape[2], xv.shape[2]
    cuts = np.cumsum([0, H * dk, H * dk, H * dv])
    outs, hist = [], []
    for i, (x, w, norm) in enumerate(((xq, wq, True), (xk, wk, True), (xv, wv, False))):
        d = x.shape[2]
        hin = None if conv_state_in is None else conv_state_in[:, :, cuts[i]:cuts[i + 1]]
        u, hout = short_conv_hist(x.reshape(ntok, H * d), w, cu_seqlens, hin)
        a = silu(u).reshape(ntok, H, d)
        outs.append(l2norm(a, l2_eps) if norm else a)
        hist.append(hout)
    return outs[0], outs[1], outs[2], np.concatenate(hist, axis=2)


def forward(q, k, v, a_raw, b_raw, A_log, dt_bias, S0=None, cu_seqlens=None, nthreads=None):
    """eqs. 9-10 then eqs. 1-4: returns dict(g, alpha, beta, y, ST)."""
    g, al, be = gates(a_raw, b_raw, A_log, dt_bias)
    y, ST = recurrence(q, k, v, al, be, S0, cu_seqlens, nthreads=nthreads)
    return dict(g=g, alpha=al, beta=be, y=y, ST=ST)
