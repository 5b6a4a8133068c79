"""Calls launched on a stream other than torch's current one. The binding allocates the
workspace and default outputs from torch's caching allocator on the current stream; it records
them on the launch stream, so memory the kernels still use is not handed to new work on the
current stream before they finish. The test allocates and overwrites memory on the current
stream while the side-stream kernels run, then checks the results against the same calls on
the current stream, bit for bit."""
import sys

import numpy as np
import pytest

from gated_deltanet_recurrence_chunked_amd import inputs as gi
import gdn_cases as C

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _scribble(nbytes, rounds=6):
    """New allocations on the current stream, overwritten at once (a freed block that is
    handed out again too early gets these bytes)."""
    import torch
    keep = []
    for _ in range(rounds):
        t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        t.fill_(0x7F)
        keep.append(t)
    return keep


@pytest.mark.parametrize("entry", ["prefill", "backward", "kda", "fused_prefill"])
def test_side_stream_results_equal_current_stream(gpu, entry):
    import torch
    import gated_deltanet_recurrence_chunked_amd as gdn
    _announce(f"side stream: {entry}, B=2 H=4 T=4096 d=128 bf16")
    inp = gi.make_inputs(gi.PREFILL, seed=21, B=2, H=4, T=4096)
    sh = inp["shape"]
    res = C.gpu_run(inp, y_dtype="bf16")
    q, k, v, g, beta = (res[x] for x in ("q", "k", "v", "g", "beta"))
    X = {x: C.dev(inp[x], True) for x in ("xq", "xk", "xv", "z")}
    W = {x: C.dev(np.ascontiguousarray(inp[x], dtype=np.float32))
         for x in ("wq", "wk", "wv", "a_raw", "b_raw", "A_log", "dt_bias", "norm_weight")}
    dy = torch.randn(v.shape, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
    dy = dy.to(torch.bfloat16)
    gk = -torch.rand((sh.ntok, sh.H, sh.dk), device="cuda",
                     generator=torch.Generator("cuda").manual_seed(4)) * 0.5

    def call(stream):
        if entry == "prefill":
            y, ST = gdn.gdn_chunk_prefill(q, k, v, g, beta, num_seqs=sh.num_seqs, stream=stream)
            return [y, ST]
        if entry == "backward":
            out = gdn.gdn_chunk_backward(q, k, v, g, beta, dy, num_seqs=sh.num_seqs,
                                         stream=stream)
            return [out[x] for x in ("dq", "dk", "dv", "dg", "dbeta", "dinitial_state")]
        if entry == "kda":
            y, ST = gdn.gdn_kda_chunk_prefill(q, k, v, gk, beta, num_seqs=sh.num_seqs,
                                              stream=stream)
            return [y, ST]
        o, ST = gdn.gdn_fused_prefill(X["xq"], X["xk"], X["xv"], W["wq"], W["wk"], W["wv"],
                                      W["a_raw"], W["b_raw"], W["A_log"], W["dt_bias"], X["z"],
                                      W["norm_weight"], H=sh.H, num_seqs=sh.num_seqs,
                                      stream=stream)
        return [o, ST]

    ref = call(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = call(side)
    junk = _scribble(64 << 20)          # on the current stream, while the side stream runs
    torch.cuda.synchronize()
    del junk
    for a, b in zip(ref, got):
        assert torch.equal(a, b), f"{entry}: the side-stream result differs"
    print(f"  {entry}: side-stream results equal the current-stream ones bit for bit")
