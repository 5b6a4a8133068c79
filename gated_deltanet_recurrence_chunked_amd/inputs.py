"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no convolution, activation, normalisation layer, gate
or recurrence). Both the HIP path and the fp64 oracle are fed from it, and
each applies the method to these raw draws on its own.

Two input-distribution steps look like method steps and are not:
  * "q, k ~ N(0,1) then L2-normalised" draws a direction uniformly on the unit
    sphere (a Gaussian vector divided by its exact fp64 norm, no epsilon). It
    describes the synthetic distribution; the method's own L2Norm (with its
    epsilon) is not applied here.
  * bf16 values are produced by one round-to-nearest-even cast of the fp32 draw,
    and are returned as raw uint16 bit patterns, so both sides see identical bits.

Workloads follow the five synthetic shapes of the Gated DeltaNet description
(the paper "On the Design of Qwen3.8-Next Architecture", section 2.1.1, eqs. 1-11):
"N(0, s)" is read as variance s.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np

SEED_TAG = 0x6D64


# --------------------------------------------------------------------------- bf16 bit helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray, is_bf16: bool) -> np.ndarray:
    return (bf16_bits_to_f32(a) if is_bf16 else np.asarray(a, dtype=np.float32)).astype(np.float64)


# --------------------------------------------------------------------------- workloads
# Workload ids. They also enter the seeds, so their values are fixed.
TINY_FP32 = 0       # fp32 recurrence, B=1 H=2 T=256 d=64, no conv, S0 = 0
PREFILL = 1         # bf16 prefill with conv preprocess and output gate, B=4 H=16 T=4096 d=128
LONG_CONTEXT = 2    # one bf16 sequence with S0, B=1 H=32 T=65536 d=128
DECODE = 3          # batched decode, N=256 H=32 d=128, 100 steps, fp32 state in place
VARLEN = 4          # 64 packed bf16 sequences, log-uniform lengths in [128, 32768], H=16 d=128

TAGS = {TINY_FP32: "tiny", PREFILL: "prefill", LONG_CONTEXT: "long", DECODE: "decode",
        VARLEN: "varlen"}


@dataclass
class Shape:
    """Sizes of one workload. `lengths` lists every packed sequence length."""
    workload: int
    H: int
    dk: int
    dv: int
    lengths: list[int]
    bf16: bool
    conv: bool            # inputs are pre-conv projected streams (full preprocess)
    has_s0: bool
    steps: int = 0        # decode steps (the decode workload only)
    equal_lengths: bool = True
    tokens: int = 1       # tokens per sequence per decode step (> 1: multi-token)

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)

    @property
    def ntok(self) -> int:
        return int(sum(self.lengths))

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


FULL_SIZES = {
    TINY_FP32: dict(B=1, H=2, T=256, d=64),
    PREFILL: dict(B=4, H=16, T=4096, d=128),
    LONG_CONTEXT: dict(B=1, H=32, T=65536, d=128),
    DECODE: dict(N=256, H=32, d=128, steps=100),
    VARLEN: dict(nseq=64, H=16, d=128, lmin=128, lmax=32768),
}

WORKLOAD_NAMES = {
    TINY_FP32: "tiny fp32 recurrence (B=1,H=2,T=256,d=64)",
    PREFILL: "bf16 prefill + preprocess + output gate (B=4,H=16,T=4096,d=128)",
    LONG_CONTEXT: "long-context prefill with S0 (B=1,H=32,T=65536,d=128)",
    DECODE: "batched decode, 100 steps (N=256,H=32,d=128)",
    VARLEN: "varlen packed prefill, 64 seqs log-uniform [128,32768] (H=16,d=128)",
}


def _varlen_lengths(rng: np.random.Generator, nseq: int, lmin: int, lmax: int) -> list[int]:
    u = rng.uniform(math.log(lmin), math.log(lmax), size=nseq)
    return [int(math.floor(math.exp(x))) for x in u]


def make_shape(workload: int, seed: int = 0, **ov) -> Shape:
    """Shape of `workload`; keyword overrides shrink it for fast tests
    (B, H, T, d, N, steps, nseq, lmin, lmax, lengths)."""
    p = dict(FULL_SIZES[workload])
    p.update({k: v for k, v in ov.items() if v is not None})
    d = p["d"]
    dk = p.get("dk", d)
    dv = p.get("dv", d)
    if workload in (TINY_FP32, PREFILL, LONG_CONTEXT):
        lengths = p.get("lengths") or [p["T"]] * p["B"]
        return Shape(workload, p["H"], dk, dv, list(lengths), bf16=(workload != TINY_FP32),
                     conv=(workload == PREFILL), has_s0=(workload == LONG_CONTEXT),
                     equal_lengths=len(set(lengths)) <= 1)
    if workload == DECODE:
        T = int(p.get("tokens", 1))
        return Shape(workload, p["H"], dk, dv, [T] * p["N"], bf16=True, conv=False, has_s0=True,
                     steps=p["steps"], tokens=T)
    if workload == VARLEN:
        if "lengths" in p and p["lengths"]:
            lengths = list(p["lengths"])
        else:
            rng = np.random.default_rng(np.random.SeedSequence([SEED_TAG, workload, seed, 99]))
            lengths = _varlen_lengths(rng, p["nseq"], p["lmin"], p["lmax"])
        return Shape(workload, p["H"], dk, dv, lengths, bf16=True, conv=True, has_s0=True,
                     equal_lengths=False)
    raise ValueError(f"unknown workload {workload}")


# --------------------------------------------------------------------------- draws
class _Streams:
    """One independent child generator per named tensor, in a fixed order."""
    NAMES = ["xq", "xk", "xv", "q", "k", "v", "wq", "wk", "wv", "a_raw", "b_raw", "A_log",
             "z", "norm_weight", "S0"]

    def __init__(self, workload: int, seed: int):
        kids = np.random.SeedSequence([SEED_TAG, workload, seed]).spawn(len(self.NAMES))
        self._kids = dict(zip(self.NAMES, kids))

    def rng(self, name: str) -> np.random.Generator:
        return np.random.default_rng(self._kids[name])


_BLOCK = 1 << 22


def _normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) drawn block by block (bounded temporary memory)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _BLOCK):
        e = min(n, s + _BLOCK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def _unit_rows(rng: np.random.Generator, shape, bf16: bool) -> np.ndarray:
    """Directions uniform on the unit sphere of the last axis (exact fp64 norm, then one cast)."""
    d = shape[-1]
    rows = int(np.prod(shape[:-1]))
    out = np.empty((rows, d), dtype=np.uint16 if bf16 else np.float32)
    step = max(1, _BLOCK // d)
    for s in range(0, rows, step):
        e = min(rows, s + step)
        x = rng.standard_normal((e - s, d))
        x /= np.sqrt(np.einsum("ij,ij->i", x, x))[:, None]
        x32 = x.astype(np.float32)
        out[s:e] = f32_to_bf16_bits(x32) if bf16 else x32
    return out.reshape(shape)


def _gate_draws(st: _Streams, lead_shape, H: int) -> dict:
    """Raw gate inputs: b_raw = u ~ N(0,1); a_raw = w ~ N(0,1) with bias b_alpha = -4.6;
    exp(A_h) ~ U[1,16] per head, stored as A_log = ln U."""
    a_raw = _normal(st.rng("a_raw"), tuple(lead_shape) + (H,))
    b_raw = _normal(st.rng("b_raw"), tuple(lead_shape) + (H,))
    A_log = np.log(st.rng("A_log").uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = np.full(H, -4.6, dtype=np.float32)
    return dict(a_raw=a_raw, b_raw=b_raw, A_log=A_log, dt_bias=dt_bias)


def make_inputs(workload: int, seed: int = 0, **ov) -> dict:
    """All inputs of `workload` as numpy arrays (bf16 tensors as uint16 bits).

    Keys: "shape" (Shape), "cu_seqlens" (int32 [num_seqs+1]), and per workload:
      TINY_FP32, LONG_CONTEXT: q, k (unit rows), v, a_raw, b_raw, A_log, dt_bias [, S0]
      PREFILL, VARLEN: xq, xk, xv, wq, wk, wv (conv taps [H*d, 4], tap 3 = current token),
            a_raw, b_raw, A_log, dt_bias, z, norm_weight [, S0]
      DECODE: state [N,H,dk,dv] and per-step q, k, v [steps,N,H,d], a_raw, b_raw [steps,N,H],
            A_log, dt_bias [H]
    """
    sh = make_shape(workload, seed, **ov)
    st = _Streams(workload, seed)
    H, dk, dv, ntok = sh.H, sh.dk, sh.dv, sh.ntok
    out: dict = {"shape": sh, "cu_seqlens": sh.cu_seqlens()}
    if workload in (TINY_FP32, LONG_CONTEXT):
        out["q"] = _unit_rows(st.rng("q"), (ntok, H, dk), sh.bf16)
        out["k"] = _unit_rows(st.rng("k"), (ntok, H, dk), sh.bf16)
        v = _normal(st.rng("v"), (ntok, H, dv))
        out["v"] = f32_to_bf16_bits(v) if sh.bf16 else v
        out.update(_gate_draws(st, (ntok,), H))
        if sh.has_s0:
            out["S0"] = _normal(st.rng("S0"), (sh.num_seqs, H, dk, dv), std=0.1)
    elif workload in (PREFILL, VARLEN):
        out["xq"] = _normal_bf16(st.rng("xq"), (ntok, H, dk))
        out["xk"] = _normal_bf16(st.rng("xk"), (ntok, H, dk))
        out["xv"] = _normal_bf16(st.rng("xv"), (ntok, H, dv))
        # depthwise conv taps ~ N(0, 1/4): std 0.5
        out["wq"] = _normal(st.rng("wq"), (H * dk, 4), std=0.5)
        out["wk"] = _normal(st.rng("wk"), (H * dk, 4), std=0.5)
        out["wv"] = _normal(st.rng("wv"), (H * dv, 4), std=0.5)
        out.update(_gate_draws(st, (ntok,), H))
        out["z"] = _normal_bf16(st.rng("z"), (ntok, H, dv))
        # zero-centred RMSNorm weight ~ N(0, 0.02): std sqrt(0.02)
        out["norm_weight"] = _normal(st.rng("norm_weight"), (dv,), std=math.sqrt(0.02))
        if sh.has_s0:
            out["S0"] = _normal(st.rng("S0"), (sh.num_seqs, H, dk, dv), std=0.1)
    elif workload == DECODE:
        N, S = sh.num_seqs, sh.steps
        lead = (S, N) if sh.tokens == 1 else (S, N, sh.tokens)   # multi-token: [S, N, T, ...]
        out["state"] = _normal(st.rng("S0"), (N, H, dk, dv), std=0.1)
        out["q"] = _unit_rows(st.rng("q"), lead + (H, dk), True)
        out["k"] = _unit_rows(st.rng("k"), lead + (H, dk), True)
        out["v"] = _normal_bf16(st.rng("v"), lead + (H, dv))
        out.update(_gate_draws(st, lead, H))
    return out


def kda_log_decay_draw(seed: int, ntok: int, H: int, dk: int, mean: float = -2.0,
                       cap: float = 5.0) -> np.ndarray:
    """Per-channel log-decays g [ntok, H, dk] fp32 for the per-channel-decay variant:
    g = -min(exp(N(mean, 1)), cap). The default is mostly mild decays (median alpha ~ 0.87)
    with a tail down to the lower bound -5 that the KDA-style gate imposes; mean=1, cap=60
    gives steep decays (median alpha ~ 0.07, some channels forgotten within one token)."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED_TAG, 55, seed]))
    x = _normal(rng, (ntok, H, dk)).astype(np.float64) + mean
    return (-np.minimum(np.exp(x), cap)).astype(np.float32)


def grad_draws(seed: int, ntok: int, num_seqs: int, H: int, dk: int, dv: int,
               bf16: bool = False) -> dict:
    """Upstream gradients for a backward pass: dy [ntok, H, dv] ~ N(0,1) (bf16 bits if bf16)
    and dST [num_seqs, H, dk, dv] ~ N(0,1) fp32."""
    kids = np.random.SeedSequence([SEED_TAG, 66, seed]).spawn(2)
    r1, r2 = (np.random.default_rng(k) for k in kids)
    dy = _normal_bf16(r1, (ntok, H, dv)) if bf16 else _normal(r1, (ntok, H, dv))
    return dict(dy=dy, dST=_normal(r2, (num_seqs, H, dk, dv)))


def conv_state_draw(seed: int, num_seqs: int, H: int, dk: int, dv: int,
                    conv_k: int = 4) -> np.ndarray:
    """A carried conv history [num_seqs, conv_k-1, H*(2dk+dv)] of bf16 N(0,1) bits, as if the
    sequences had seen earlier input (channels q | k | v)."""
    rng = np.random.default_rng(np.random.SeedSequence([SEED_TAG, 77, seed]))
    return _normal_bf16(rng, (num_seqs, conv_k - 1, H * (2 * dk + dv)))


def make_stream_inputs(seed: int, N: int, H: int, prompt_lengths, steps: int, tokens: int,
                       dk: int = 128, dv: int = 128) -> dict:
    """A prompt per sequence followed by `steps` decode steps of `tokens` tokens each, as the
    pre-conv projected streams drawn as in the bf16 prefill workload (bf16 bits).
      prompt: xq, xk [P, H, dk], xv [P, H, dv], a_raw, b_raw [P, H], packed by
              cu_seqlens (lengths prompt_lengths);
      decode: dxq, dxk [steps, N, tokens, H, dk], dxv [..., dv], da_raw, db_raw
              [steps, N, tokens, H];
      shared: wq, wk, wv [H*d, 4] conv taps, A_log, dt_bias [H]."""
    assert len(prompt_lengths) == N
    kids = dict(zip(["p", "d", "w", "g"],
                    np.random.SeedSequence([SEED_TAG, 88, seed]).spawn(4)))
    rp, rd, rw = (np.random.default_rng(kids[x]) for x in "pdw")
    P = int(sum(prompt_lengths))
    lead = (steps, N, tokens)
    out = dict(cu_seqlens=np.concatenate([[0], np.cumsum(prompt_lengths)]).astype(np.int32),
               H=H, dk=dk, dv=dv, N=N, steps=steps, tokens=tokens)
    out["xq"] = _normal_bf16(rp, (P, H, dk))
    out["xk"] = _normal_bf16(rp, (P, H, dk))
    out["xv"] = _normal_bf16(rp, (P, H, dv))
    out["a_raw"] = _normal(rp, (P, H))
    out["b_raw"] = _normal(rp, (P, H))
    out["dxq"] = _normal_bf16(rd, lead + (H, dk))
    out["dxk"] = _normal_bf16(rd, lead + (H, dk))
    out["dxv"] = _normal_bf16(rd, lead + (H, dv))
    out["da_raw"] = _normal(rd, lead + (H,))
    out["db_raw"] = _normal(rd, lead + (H,))
    out["wq"] = _normal(rw, (H * dk, 4), std=0.5)
    out["wk"] = _normal(rw, (H * dk, 4), std=0.5)
    out["wv"] = _normal(rw, (H * dv, 4), std=0.5)
    out["A_log"] = np.log(np.random.default_rng(kids["g"]).uniform(1.0, 16.0, size=H)).astype(np.float32)
    out["dt_bias"] = np.full(H, -4.6, dtype=np.float32)
    return out


def decode_layer_draws(seed: int, steps: int, N: int, H: int, dk: int = 128, dv: int = 128,
                       bf16: bool = True, tokens: int = 1) -> dict:
    """Raw inputs of `steps` decode steps of the whole token mixer (the fused decode step),
    drawn as in the bf16 prefill workload: per step xq, xk [steps, N, H, dk], xv, z [steps, N, H, dv]
    (bf16 bits, or float32 with bf16=False), a_raw, b_raw [steps, N, H] (with tokens > 1, a
    [tokens] axis after N: T tokens per sequence per step); conv taps
    wq, wk, wv [H*d, 4] ~ N(0, 1/4); A_log, dt_bias [H]; norm_weight [dv] ~ N(0, 0.02);
    a carried conv history conv_state [N, 3, H*(2dk+dv)] ~ N(0,1) in the x dtype and a
    state [N, H, dk, dv] ~ N(0, 0.01) fp32."""
    kids = dict(zip(["x", "g", "w", "z", "h", "s"],
                    np.random.SeedSequence([SEED_TAG, 99, seed]).spawn(6)))
    rx, rg, rw, rz, rh, rs = (np.random.default_rng(kids[c]) for c in "xgwzhs")
    draw = _normal_bf16 if bf16 else _normal
    lead = (steps, N, H) if tokens == 1 else (steps, N, tokens, H)
    out = dict(steps=steps, N=N, H=H, dk=dk, dv=dv, bf16=bf16, tokens=tokens)
    out["xq"] = draw(rx, lead + (dk,))
    out["xk"] = draw(rx, lead + (dk,))
    out["xv"] = draw(rx, lead + (dv,))
    out["a_raw"] = _normal(rg, lead)
    out["b_raw"] = _normal(rg, lead)
    out["A_log"] = np.log(rg.uniform(1.0, 16.0, size=H)).astype(np.float32)
    out["dt_bias"] = np.full(H, -4.6, dtype=np.float32)
    out["wq"] = _normal(rw, (H * dk, 4), std=0.5)
    out["wk"] = _normal(rw, (H * dk, 4), std=0.5)
    out["wv"] = _normal(rw, (H * dv, 4), std=0.5)
    out["z"] = draw(rz, lead + (dv,))
    out["norm_weight"] = _normal(rz, (dv,), std=math.sqrt(0.02))
    out["conv_state"] = draw(rh, (N, 3, H * (2 * dk + dv)))
    out["state"] = _normal(rs, (N, H, dk, dv), std=0.1)
    return out


def checksums(inp: dict) -> dict:
    """SHA-256 (first 16 hex digits) of every array, for the results record."""
    res = {}
    for k, a in inp.items():
        if isinstance(a, np.ndarray):
            res[k] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
    return res
