"""Shared drivers of the parity tests: run one workload through the HIP path (libgdn via the
Python binding) and through the fp64 oracle, on the same seeded raw draws.

The oracle side never sees a value produced by the HIP path: both start from the input
generator's arrays. Sampled comparisons restrict the oracle to a subset of (sequence, head)
slices; the recurrence of one slice depends on nothing outside it.
"""
from __future__ import annotations

import numpy as np

import oracle
from gated_deltanet_recurrence_chunked_amd import inputs as gi

L2_EPS = 1e-6
RMS_EPS = 1e-6

# Tolerances of the parity bar: max over (sequence, head) slices of ||a-b|| / ||b||, and
# an elementwise bound on the bf16-input path.
TOL_REL = {False: 1e-4, True: 5e-3}        # keyed by "bf16 path"
TOL_ABS = 2e-2
U_BF16 = 2.0 ** -8                         # unit roundoff of bf16 (8 significant bits, RNE)
BF16_HALF_ULP_REL = U_BF16                 # rounding bound of a bf16-stored output


# ----------------------------------------------------------------------------- host <-> device
def dev(a: np.ndarray, bf16: bool = False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


# ----------------------------------------------------------------------------- metrics
def slice_rel_errors(a: np.ndarray, b: np.ndarray, cu, H: int) -> np.ndarray:
    """Relative L2 error per (sequence, head) slice of token-major [ntok, H, ...] arrays."""
    errs = []
    for lo, hi in zip(cu[:-1], cu[1:]):
        if hi == lo:
            continue
        for h in range(H):
            x = a[lo:hi, h].ravel()
            y = b[lo:hi, h].ravel()
            errs.append(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-30))
    return np.array(errs)


def state_rel_errors(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per (sequence, head) relative L2 error of [nseq, H, dk, dv] states."""
    n = a.shape[0] * a.shape[1]
    x = a.reshape(n, -1)
    y = b.reshape(n, -1)
    return np.linalg.norm(x - y, axis=1) / np.maximum(np.linalg.norm(y, axis=1), 1e-30)


def o_allowance(o_ref, o_qkv, y_bf16):
    """Elementwise allowance of the output gate's o beyond the bar (2e-2 plus o's own bf16
    rounding), against the plain fp64 oracle o_ref. It is derived from the bf16 storage of the
    pipeline's intermediates, before any comparison:
      * y stored in bf16 before the gate (y_bf16): each element of a (token, head) row moves by
        at most u = 2^-8 relative, so the row's RMS moves by at most u as well (its square is a
        weighted mean of the elements' factors), and o_j = c_j y_j / rms(y) moves by at most
        (1+u)/(1-u) - 1 = 2u/(1-u) relative;
      * q, k, v stored in bf16 between the preprocess and the prefill: their effect on o is
        |o_qkv - o_ref|, where o_qkv is the oracle's own o with its q, k, v rounded to bf16
        (y left unrounded). It is computed by the oracle alone, exactly, with no GPU value.
    The RMSNorm maps each row to unit RMS, so in rows where y is small next to the terms that
    cancel in it (the first tokens of a sequence) the q, k, v storage shows up in o at full
    size; elsewhere this term is small."""
    a = np.abs(o_qkv - o_ref)
    if y_bf16:
        a = a + 2.0 * U_BF16 / (1.0 - U_BF16) * np.abs(o_ref)
    return a


def assert_close_grad(name, got, ref, cu=None, H=None, state=False):
    """The bf16 bar applied to a gradient of the bf16 matrix-core backward, against the fp64
    oracle's gradient: max slice relative L2 <= 5e-3 as for the forward's outputs, and
    elementwise |got - ref| <= 2e-2 s + 2^-8 |ref|, where s = max(1, RMS of the reference
    slice). A gradient is not an O(1) quantity like y: the 2e-2 of the forward's bar is taken in
    units of the slice's own scale once that scale exceeds 1, and 2^-8 |ref| is the relative
    precision of bf16 operands (the products' inputs are bf16 or hi + lo pairs)."""
    if state:
        errs = state_rel_errors(got, ref)
        n = ref.shape[0] * ref.shape[1]
        rms = np.sqrt(np.mean(ref.reshape(n, -1) ** 2, axis=1)).reshape(ref.shape[:2] + (1,) * (ref.ndim - 2))
        scale = np.broadcast_to(np.maximum(1.0, rms), ref.shape)
    else:
        errs = slice_rel_errors(got, ref, cu, H)
        scale = np.ones_like(ref)
        for lo, hi in zip(cu[:-1], cu[1:]):
            for h in range(H):
                x = ref[lo:hi, h]
                if x.size:
                    scale[lo:hi, h] = max(1.0, float(np.sqrt(np.mean(x * x))))
    worst = float(errs.max()) if errs.size else 0.0
    assert worst <= TOL_REL[True], f"{name}: max slice rel L2 {worst:.3e} > {TOL_REL[True]:.0e}"
    bound = TOL_ABS * scale + U_BF16 * np.abs(ref)
    ratio = np.abs(got - ref) / bound
    if ratio.size and not np.all(ratio <= 1.0):
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError(f"{name}: elementwise |diff| over the bound at {tuple(int(x) for x in i)}: "
                             f"got {got[i]:.6g} ref {ref[i]:.6g} bound {bound[i]:.4g}, "
                             f"{int(np.sum(ratio > 1))} elements over")
    return worst, float(ratio.max()) if ratio.size else 0.0


def max_abs(got, ref) -> float:
    return float(np.abs(got - ref).max()) if np.size(ref) else 0.0


def assert_close(name, got, ref, bf16_path, stored_bf16=False, cu=None, H=None, state=False,
                 allowance=None):
    """The parity bar: max slice relative L2 <= TOL_REL; on the bf16 path also
    |got - ref| <= 2e-2 (+ the output's own bf16 rounding if it is stored in bf16, + an
    elementwise allowance derived beforehand from the arithmetic, e.g. o_allowance)."""
    if state:
        errs = state_rel_errors(got, ref)
    else:
        errs = slice_rel_errors(got, ref, cu, H)
    worst = float(errs.max()) if errs.size else 0.0
    tol = TOL_REL[bf16_path]
    assert worst <= tol, f"{name}: max slice rel L2 {worst:.3e} > {tol:.0e}"
    if bf16_path:
        r = ref
        bound = TOL_ABS + (BF16_HALF_ULP_REL * np.abs(r) if stored_bf16 else 0.0)
        if allowance is not None:
            bound = bound + allowance
        excess = np.abs(got - r) - bound
        if not np.all(excess <= 0):
            i = np.unravel_index(np.argmax(excess), excess.shape)
            row = r[i[:-1]] if r.ndim > 1 else r
            raise AssertionError(
                f"{name}: max |diff| {np.abs(got - r).max():.3e} exceeds the elementwise bound; "
                f"worst at {tuple(int(x) for x in i)}: got {got[i]:.6g} ref {r[i]:.6g} "
                f"bound {bound[i] if np.ndim(bound) else bound:.4g}; row rms {np.sqrt(np.mean(row * row)):.4g}, "
                f"{int(np.sum(excess > 0))} elements over")
    return worst


# ----------------------------------------------------------------------------- oracle side
def subset(inp: dict, seqs=None, heads=None) -> dict:
    """Restrict a workload to some sequences and heads (the oracle evaluates only those).
    Returns a dict of float64 arrays plus cu_seqlens, H and the token index map."""
    sh = inp["shape"]
    cu = inp["cu_seqlens"]
    seqs = list(range(sh.num_seqs)) if seqs is None else list(seqs)
    heads = list(range(sh.H)) if heads is None else list(heads)
    tok = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64) \
        if seqs else np.zeros(0, np.int64)
    new_cu = np.concatenate([[0], np.cumsum([cu[s + 1] - cu[s] for s in seqs])]).astype(np.int32)
    out = dict(cu=new_cu, H=len(heads), tok=tok, seqs=seqs, heads=heads)
    every_token = len(tok) == sh.ntok and np.array_equal(tok, np.arange(sh.ntok))

    def pick(a):                                 # slice first, widen the slice only
        return a[:, heads] if every_token else a[tok][:, heads]
    for key in ("q", "k", "v", "xq", "xk", "xv", "z"):
        if key in inp:
            a = pick(inp[key])
            out[key] = gi.as_f64(a, a.dtype == np.uint16)
    for key in ("a_raw", "b_raw"):
        if key in inp:
            out[key] = pick(inp[key]).astype(np.float64)
    for key in ("A_log", "dt_bias"):
        out[key] = inp[key].astype(np.float64)[heads]
    for key, d in (("wq", sh.dk), ("wk", sh.dk), ("wv", sh.dv)):
        if key in inp:
            w = inp[key].astype(np.float64).reshape(sh.H, d, -1)
            out[key] = w[heads].reshape(len(heads) * d, -1)
    if "norm_weight" in inp:
        out["norm_weight"] = inp["norm_weight"].astype(np.float64)
    if inp.get("S0") is not None:
        out["S0"] = inp["S0"].astype(np.float64)[seqs][:, heads]
    return out


def oracle_run(sub: dict, nthreads=None, storage_bf16=False, y_bf16=True) -> dict:
    """The oracle's token mixer on a subset: eqs. 6-10 (if pre-conv streams), 1-4, 11.
    storage_bf16 rounds the intermediates the bf16 pipeline stores (q, k, v after the
    preprocess, and y before the output gate when y_bf16) to bf16, in the oracle's own
    arithmetic; the o of such a run with y_bf16=False is o_allowance's o_qkv."""
    H = sub["H"]
    res = {}
    if "xq" in sub:
        q, k, v = oracle.preprocess(sub["xq"], sub["xk"], sub["xv"], sub["wq"], sub["wk"],
                                    sub["wv"], sub["cu"], H, L2_EPS)
        if storage_bf16:
            q, k, v = oracle.round_bf16(q), oracle.round_bf16(k), oracle.round_bf16(v)
        res.update(q=q, k=k, v=v)
    else:
        q, k, v = sub["q"], sub["k"], sub["v"]
    g, al, be = oracle.gates(sub["a_raw"], sub["b_raw"], sub["A_log"], sub["dt_bias"])
    res.update(g=g, beta=be)
    y, ST = oracle.recurrence(q, k, v, al, be, sub.get("S0"), sub["cu"], nthreads=nthreads)
    res.update(y=y, ST=ST)
    if "z" in sub:
        yo = oracle.round_bf16(y) if (storage_bf16 and y_bf16) else y
        res["o"] = oracle.output_gate(yo, sub["z"], sub["norm_weight"], RMS_EPS)
    return res


# ----------------------------------------------------------------------------- HIP side
def gpu_run(inp: dict, y_dtype="bf16", state_out=True) -> dict:
    """The HIP path on the whole workload. Returns device tensors."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    sh = inp["shape"]
    bf = sh.bf16
    cu = inp["cu_seqlens"]
    cu_d = None if sh.equal_lengths else dev(cu)
    cu_h = None if sh.equal_lengths else cu
    f32 = lambda a: dev(np.asarray(a, dtype=np.float32))  # noqa: E731
    res = {}
    if sh.conv:
        q, k, v, g, beta = gdn.gdn_preprocess(
            dev(inp["xq"], True), dev(inp["xk"], True), dev(inp["xv"], True),
            f32(inp["wq"]), f32(inp["wk"]), f32(inp["wv"]), f32(inp["a_raw"]), f32(inp["b_raw"]),
            f32(inp["A_log"]), f32(inp["dt_bias"]), H=sh.H, cu_seqlens=cu_d,
            num_seqs=sh.num_seqs, l2_eps=L2_EPS, out_dtype=torch.bfloat16)
    else:
        q, k, v = dev(inp["q"], bf), dev(inp["k"], bf), dev(inp["v"], bf)
        _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None,
                                              f32(inp["a_raw"]), f32(inp["b_raw"]),
                                              f32(inp["A_log"]), f32(inp["dt_bias"]), H=sh.H,
                                              num_seqs=1)
    res.update(q=q, k=k, v=v, g=g, beta=beta)
    S0 = f32(inp["S0"]) if inp.get("S0") is not None else None
    y, ST = gdn.gdn_chunk_prefill(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu_d,
                                  cu_seqlens_host=cu_h, num_seqs=sh.num_seqs, y_dtype=y_dtype,
                                  output_final_state=state_out)
    res.update(y=y, ST=ST)
    if "z" in inp:
        res["o"] = gdn.gdn_output_gate(y, dev(inp["z"], True), f32(inp["norm_weight"]),
                                       eps=RMS_EPS, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    return res


def gpu_run_fused(inp: dict) -> dict:
    """The fused token mixer (gdn_fused_prefill) on the whole workload, with its intermediates
    exported. Returns device tensors under the keys gpu_run uses (y is bf16)."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    sh = inp["shape"]
    cu = inp["cu_seqlens"]
    cu_d = None if sh.equal_lengths else dev(cu)
    cu_h = None if sh.equal_lengths else cu
    f32 = lambda a: dev(np.asarray(a, dtype=np.float32))  # noqa: E731
    S0 = f32(inp["S0"]) if inp.get("S0") is not None else None
    o, ST, ex = gdn.gdn_fused_prefill(
        dev(inp["xq"], True), dev(inp["xk"], True), dev(inp["xv"], True), f32(inp["wq"]),
        f32(inp["wk"]), f32(inp["wv"]), f32(inp["a_raw"]), f32(inp["b_raw"]), f32(inp["A_log"]),
        f32(inp["dt_bias"]), dev(inp["z"], True), f32(inp["norm_weight"]), H=sh.H,
        initial_state=S0, cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=sh.num_seqs,
        l2_eps=L2_EPS, rms_eps=RMS_EPS, o_dtype=torch.bfloat16, export=True)
    torch.cuda.synchronize()
    return dict(o=o, ST=ST, **ex)


def gpu_slice(t, tok, heads):
    """Token/head subset of a device [ntok, H, ...] tensor, as float64 numpy."""
    import torch
    idx_t = torch.as_tensor(tok, device=t.device)
    idx_h = torch.as_tensor(heads, device=t.device)
    return host(t.index_select(0, idx_t).index_select(1, idx_h))


def gpu_state_slice(t, seqs, heads):
    import torch
    return host(t.index_select(0, torch.as_tensor(seqs, device=t.device))
                .index_select(1, torch.as_tensor(heads, device=t.device)))


# ----------------------------------------------------------------------------- many sequences
def many_short_lengths(seed: int, nseq: int, lmax: int = 70) -> list[int]:
    """nseq seeded lengths in [0, lmax], with an empty sequence first and lengths 64 and 65
    (a full chunk, one token past it) next: a packing of many short sequences, as in serving."""
    rng = np.random.default_rng(np.random.SeedSequence([0x6D616E79, seed, nseq]))
    L = [int(x) for x in rng.integers(0, lmax + 1, size=nseq)]
    L[0], L[1], L[2], L[-1] = 0, 64, 65, 1
    return L


def sampled_seqs(lengths, seed: int, extra: int = 6) -> list[int]:
    """Sequences to check against the oracle: the ends, both sides of 256 and 1024 (the chunk
    table's scan rounds and its longest-first limit), and a few seeded picks."""
    n = len(lengths)
    fixed = {0, 1, 2, 255, 256, 257, 1023, 1024, 1025, n - 1}
    rng = np.random.default_rng(np.random.SeedSequence([0x73656C, seed, n]))
    picks = set(int(x) for x in rng.integers(0, n, size=extra))
    return sorted(i for i in fixed | picks if 0 <= i < n)


def check_prefill_sampled(inp, res, seqs, heads, y_bf16):
    """Sampled (sequence, head) slices of a pipeline run against the oracle on just those."""
    sh = inp["shape"]
    sub = subset(inp, seqs=seqs, heads=heads)
    ref = oracle_run(sub)
    tok, cu, H = sub["tok"], sub["cu"], sub["H"]
    rep = {}
    if sh.conv:
        for key in ("q", "k", "v"):
            rep[key] = assert_close(key, gpu_slice(res[key], tok, heads), ref[key], True,
                                    stored_bf16=True, cu=cu, H=H)
    for key in ("g", "beta"):
        got = gpu_slice(res[key], tok, heads)
        assert np.abs(got - ref[key]).max() / np.abs(ref[key]).max() < 1e-5, key
    rep["y"] = assert_close("y", gpu_slice(res["y"], tok, heads), ref["y"], sh.bf16,
                            stored_bf16=y_bf16, cu=cu, H=H)
    rep["ST"] = assert_close("ST", gpu_state_slice(res["ST"], seqs, heads), ref["ST"], sh.bf16,
                             state=True)
    if "o" in res:
        rep["o"], rep["o_max_abs"] = check_o(gpu_slice(res["o"], tok, heads), sub, ref, y_bf16)
    print("  max slice rel L2:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


def check_o(got, sub, ref, y_bf16):
    """o against the plain fp64 oracle, to the bar plus o_allowance. Returns (max slice rel L2,
    raw max |o - o_ref|)."""
    qkv = oracle_run(sub, storage_bf16=True, y_bf16=False)
    err = assert_close("o", got, ref["o"], True, stored_bf16=True, cu=sub["cu"], H=sub["H"],
                       allowance=o_allowance(ref["o"], qkv["o"], y_bf16))
    return err, max_abs(got, ref["o"])
