"""GPU parity at the largest arrays the C ABI accepts: 2^31 - 1 elements per array, the limit
that keeps every token and state index inside the kernels within 32 bits. The slices checked
are the ones at the largest offsets (the last sequence, the last head), plus the first.

The arrays are too large to build on the host, so the inputs are drawn on the device with
torch's seeded generator (q, k ~ N(0, 1) normalised per (token, head), v ~ N(0, 1), g uniform in
[-0.15, -0.001], beta = sigmoid(N(0, 1)), states ~ N(0, 0.01)); the sampled slices are copied
back and the fp64 oracle evaluates them alone (a slice depends on nothing outside it)."""
import sys

import numpy as np
import pytest

import gdn_cases as C

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

LIMIT = 2 ** 31 - 1


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _tokens(torch, gen, shape, d):
    """bf16 q or k (normalised over the last axis) and v, drawn on the device."""
    bf = torch.bfloat16
    q = torch.randn(shape + (d,), generator=gen, device="cuda")
    q = (q / q.norm(dim=-1, keepdim=True)).to(bf)
    k = torch.randn(shape + (d,), generator=gen, device="cuda")
    k = (k / k.norm(dim=-1, keepdim=True)).to(bf)
    v = torch.randn(shape + (d,), generator=gen, device="cuda").to(bf)
    g = -(torch.rand(shape, generator=gen, device="cuda") * 0.149 + 0.001)
    beta = torch.sigmoid(torch.randn(shape, generator=gen, device="cuda"))
    return q, k, v, g, beta


def _f64(t):
    return t.double().cpu().numpy()


def test_decode_largest_state(gpu):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    H, d = 1, 128
    N = LIMIT // (H * d * d)                      # 131,071 states: 2^31 - 16,384 fp32 elements
    assert N * H * d * d <= LIMIT
    _announce(f"decode at the largest state array: N={N} H={H} d={d} ({N * H * d * d} elements, "
              "one step in place)")
    gen = torch.Generator(device="cuda").manual_seed(11)
    state = torch.randn((N, H, d, d), generator=gen, device="cuda") * 0.1
    q, k, v, g, beta = _tokens(torch, gen, (N, H), d)
    pick = [0, 1, N // 2, N - 2, N - 1]
    S_before = _f64(state[pick])
    y = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_step(q, k, v, g, beta, state, y=y)
    torch.cuda.synchronize()
    # each picked state is a one-token sequence for the oracle
    cu = np.arange(len(pick) + 1, dtype=np.int32)
    y_ref, S_ref = C.oracle.recurrence(_f64(q[pick]), _f64(k[pick]), _f64(v[pick]),
                                       np.exp(_f64(g[pick])), _f64(beta[pick]), S_before, cu)
    y_got = _f64(y[pick])
    ey = C.assert_close("y", y_got, y_ref, True, stored_bf16=True, cu=cu, H=H)
    es = C.assert_close("S", _f64(state[pick]), S_ref, True, state=True)
    print(f"  states {pick}: max rel L2 y {ey:.2e} S {es:.2e}, "
          f"max |y - y_ref| {C.max_abs(y_got, y_ref):.3e}", flush=True)


@pytest.mark.parametrize("B,H", [(4, 16), (64, 16)], ids=["64_pairs", "1024_pairs"])
def test_prefill_largest_token_arrays(gpu, B, H):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    d = 128
    L = LIMIT // (B * H * d)                      # tokens per sequence
    ntok = B * L
    assert ntok * H * d <= LIMIT
    _announce(f"prefill at the largest token arrays: B={B} H={H} L={L} d={d} "
              f"({ntok * H * d} elements per array), S0 and S_T")
    gen = torch.Generator(device="cuda").manual_seed(12)
    q, k, v, g, beta = _tokens(torch, gen, (ntok, H), d)
    S0 = torch.randn((B, H, d, d), generator=gen, device="cuda") * 0.1
    ws = torch.empty(gdn.gdn_chunk_prefill_workspace_size(ntok, B, H, d, d), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty((ntok, H, d), dtype=torch.bfloat16, device="cuda")
    y, ST = gdn.gdn_chunk_prefill(q, k, v, g, beta, initial_state=S0, num_seqs=B, y=y,
                                  workspace=ws)
    torch.cuda.synchronize()
    del ws
    for s, h in ((B - 1, H - 1), (B - 1, 0), (0, H - 1)):
        lo, hi = s * L, (s + 1) * L
        sl = lambda t: _f64(t[lo:hi, h:h + 1])   # noqa: E731
        cu = np.array([0, L], dtype=np.int32)
        y_ref, S_ref = C.oracle.recurrence(sl(q), sl(k), sl(v), np.exp(sl(g)), sl(beta),
                                           _f64(S0[s:s + 1, h:h + 1]), cu)
        y_got = sl(y)
        ey = C.assert_close("y", y_got, y_ref, True, stored_bf16=True, cu=cu, H=1)
        es = C.assert_close("S_T", _f64(ST[s:s + 1, h:h + 1]), S_ref, True, state=True)
        print(f"  sequence {s} head {h} (tokens {lo}..{hi - 1}): rel L2 y {ey:.2e} S_T {es:.2e}, "
              f"max |y - y_ref| {C.max_abs(y_got, y_ref):.3e}", flush=True)
