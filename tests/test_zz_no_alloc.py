"""The allocation-free prefill entry point (gdn_chunk_prefill_noalloc, for callers that cannot
allocate device memory) against gdn_chunk_prefill with a caller-provided workspace: the same
kernels, so the same outputs bit for bit. Two calls in a row, the second on a smaller input,
since every call on the GPU shares the library's one scratch array and keeps the last call's
contents."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _pair(inp, y_dtype):
    """Returns ((y, ST) with a workspace, (y, ST) without) on the same device inputs."""
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    sh = inp["shape"]
    bf = sh.bf16
    cu = inp["cu_seqlens"]
    cu_d = None if sh.equal_lengths else C.dev(cu)
    cu_h = None if sh.equal_lengths else cu
    q, k, v = C.dev(inp["q"], bf), C.dev(inp["k"], bf), C.dev(inp["v"], bf)
    f32 = lambda a: C.dev(np.asarray(a, dtype=np.float32))  # noqa: E731
    _, _, _, g, beta = gdn.gdn_preprocess(None, None, None, None, None, None, f32(inp["a_raw"]),
                                          f32(inp["b_raw"]), f32(inp["A_log"]),
                                          f32(inp["dt_bias"]), H=sh.H)
    S0 = f32(inp["S0"]) if inp.get("S0") is not None else None
    ydt = torch.bfloat16 if y_dtype == "bf16" else torch.float32
    y_ws, ST_ws = gdn.gdn_chunk_prefill(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu_d,
                                        cu_seqlens_host=cu_h, num_seqs=sh.num_seqs, y_dtype=ydt)
    y_na = torch.empty_like(y_ws)
    ST_na = torch.empty_like(ST_ws)
    gdn.gdn_chunk_prefill_noalloc(q, k, v, g, beta, y=y_na, initial_state=S0, final_state=ST_na,
                                  cu_seqlens=cu_d, cu_seqlens_host=cu_h, num_seqs=sh.num_seqs)
    torch.cuda.synchronize()
    return (y_ws, ST_ws), (y_na, ST_na)


def test_noalloc_prefill_equals_workspace_prefill(gpu):
    import torch
    cases = [
        ("long-context bf16 B=1 H=8 T=8000 with S0", gi.make_inputs(gi.LONG_CONTEXT, seed=31,
                                                                     H=8, T=8000), "bf16"),
        ("varlen bf16 lengths 0,1,63,64,65,300,129 H=3 (smaller, second)",
         gi.make_inputs(gi.LONG_CONTEXT, seed=32, H=3, lengths=[0, 1, 63, 64, 65, 300, 129]),
         "f32"),
        ("tiny fp32 path B=2 H=2 T=130 d=64 (no scratch needed)",
         gi.make_inputs(gi.TINY_FP32, seed=33, B=2, T=130), "f32"),
    ]
    for name, inp, ydt in cases:
        _announce(f"no-alloc prefill vs workspace prefill: {name}")
        (ya, Sa), (yb, Sb) = _pair(inp, ydt)
        assert torch.equal(ya, yb), f"{name}: y differs"
        assert torch.equal(Sa, Sb), f"{name}: final state differs"
        print("  equal bit for bit", flush=True)
