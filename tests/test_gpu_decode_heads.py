"""GPU parity of gdn_decode_step at d_k = d_v = 128 for head counts around the persistent
kernel's grid (one workgroup per compute unit, each walking heads blockIdx.x, + gridDim.x, ...):
fewer heads than workgroups, exactly as many, one more, and counts that leave some workgroups
an odd and others an even number of heads, so every path of its two-heads-per-trip loop and
its tail runs. Every head of every step is compared with the fp64 oracle."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("extra", [None, 0, 1, -1, "x2+1", "x3+1", "x4+3"])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_decode_head_counts(gpu, extra, ydt):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    G = _cus()
    if extra is None:
        heads = 3                                   # far fewer heads than workgroups
    elif isinstance(extra, int):
        heads = G + extra                           # G - 1, G, G + 1
    else:
        m, r = extra[1:].split("+")
        heads = int(m) * G + int(r)                 # some workgroups one head more than others
    N, H, S_ = heads, 1, 2
    _announce(f"decode heads={heads} (grid {min(heads, G)}) y={ydt}, {S_} steps")
    inp = gi.make_inputs(gi.DECODE, seed=heads, N=N, H=H, steps=S_)
    f32 = lambda a: C.dev(np.ascontiguousarray(a, dtype=np.float32))  # noqa: E731
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None,
                                          f32(inp["a_raw"].reshape(S_ * N, H)),
                                          f32(inp["b_raw"].reshape(S_ * N, H)),
                                          f32(inp["A_log"]), f32(inp["dt_bias"]), H=H)
    g = g.view(S_, N, H)
    beta = beta.view(S_, N, H)
    state = C.dev(inp["state"])
    ys = []
    for s in range(S_):
        ys.append(gdn.gdn_decode_step(C.dev(inp["q"][s], True), C.dev(inp["k"][s], True),
                                      C.dev(inp["v"][s], True), g[s].contiguous(),
                                      beta[s].contiguous(), state, y_dtype=ydt))
    torch.cuda.synchronize()
    perm = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape(N * S_, *a.shape[2:]))  # noqa
    q = perm(gi.as_f64(inp["q"], True))
    k = perm(gi.as_f64(inp["k"], True))
    v = perm(gi.as_f64(inp["v"], True))
    og, al, be = C.oracle.gates(perm(inp["a_raw"].astype(np.float64)),
                                perm(inp["b_raw"].astype(np.float64)),
                                inp["A_log"].astype(np.float64), inp["dt_bias"].astype(np.float64))
    cu = np.arange(0, N * S_ + 1, S_)
    y_ref, S_ref = C.oracle.recurrence(q, k, v, al, be, inp["state"].astype(np.float64), cu)
    y_gpu = np.stack([C.host(y) for y in ys], axis=1).reshape(N * S_, H, 128)
    ey = C.assert_close("y", y_gpu, y_ref, True, stored_bf16=(ydt == "bf16"), cu=cu, H=H)
    es = C.assert_close("S", C.host(state), S_ref, True, state=True)
    print(f"  max slice rel L2: y {ey:.2e}, S {es:.2e}", flush=True)
