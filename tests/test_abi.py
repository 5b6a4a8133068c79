"""The C ABI without a GPU: libgdn.so loads, exports every function include/gdn.h declares,
and rejects invalid arguments on the host before any HIP call (no kernel is launched)."""
import ctypes
import os
import re

import pytest

import gated_deltanet_recurrence_chunked_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.skip("libgdn.so not built")
    return gdn.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"gdn_preprocess", "gdn_chunk_prefill", "gdn_decode_step", "gdn_output_gate"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    declared = int(re.search(r"#define GDN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.gdn_abi_version() == declared


def test_status_strings(L):
    assert L.gdn_status_string(0) == b"GDN_OK"
    assert L.gdn_status_string(7) == b"GDN_ERR_HIP"


FAKE = 0x10000      # 16-byte aligned non-null address; never dereferenced (validation fails first)
MIS = 0x10004       # misaligned


def _prefill(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, g=FAKE, beta=FAKE, s0=None, st=None, cu=None,
             cu_host=None, num_seqs=1, ntok=128, H=2, dk=128, dv=128, y=FAKE, y_dtype=1, ws=None,
             wsb=0)
    a.update(kw)
    return L.gdn_chunk_prefill(a["q"], a["k"], a["v"], a["in_dtype"], a["g"], a["beta"], a["s0"],
                               a["st"], a["cu"], a["cu_host"], a["num_seqs"], a["ntok"], a["H"],
                               a["dk"], a["dv"], a["y"], a["y_dtype"], a["ws"], a["wsb"], None)


def test_prefill_validation(L):
    assert _prefill(L, q=None) == 1
    assert L.gdn_last_error().startswith(b"q must not be NULL")
    assert _prefill(L, dk=96) == 2
    assert _prefill(L, in_dtype=5) == 3
    assert _prefill(L, k=MIS) == 5
    assert _prefill(L, num_seqs=3, ntok=128) == 2          # 128 not a multiple of 3
    bad = (ctypes.c_int32 * 3)(0, 100, 120)                # last offset != ntok
    assert _prefill(L, num_seqs=2, cu=FAKE, cu_host=ctypes.cast(bad, ctypes.c_void_p)) == 4
    dec = (ctypes.c_int32 * 3)(0, 100, 90)
    dec2 = (ctypes.c_int32 * 3)(0, 100, 128)
    assert _prefill(L, num_seqs=2, cu=FAKE, cu_host=ctypes.cast(dec, ctypes.c_void_p)) == 4
    assert _prefill(L, num_seqs=2, cu=None, cu_host=ctypes.cast(dec2, ctypes.c_void_p)) == 1
    # with no tokens the token-indexed arrays may be NULL; alignment is still checked, and the
    # matrix path still needs its workspace (both fail before anything is enqueued)
    assert _prefill(L, ntok=0, q=None, k=None, v=None, g=None, beta=None, y=MIS) == 5
    assert _prefill(L, ntok=0, q=None, k=None, v=None, g=None, beta=None, y=None) == 6
    assert _prefill(L, ntok=1, num_seqs=1, q=None) == 1
    # arrays beyond 2^31 - 1 elements are refused (2^24 tokens x 1024 heads x 128)
    assert _prefill(L, ntok=1 << 24, H=1024) == 2
    assert L.gdn_last_error().startswith(b"token arrays of 16777216 rows")
    assert _prefill(L, ntok=1 << 17, num_seqs=1 << 17, H=2) == 2      # 2^17 states of 2^15
    assert L.gdn_last_error().startswith(b"state arrays of 131072 x 32768")


def test_decode_and_gate_validation(L):
    assert L.gdn_decode_step(FAKE, FAKE, None, 1, FAKE, FAKE, FAKE, 4, 2, 128, 128, FAKE, 1, None) == 1
    assert L.gdn_decode_step(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 4, 0, 128, 128, FAKE, 1, None) == 2
    assert L.gdn_output_gate(FAKE, 1, FAKE, 1, FAKE, 10, 2, 32, 1e-6, FAKE, 1, None) == 2
    assert L.gdn_output_gate(FAKE, 1, FAKE, 1, FAKE, 10, 2, 128, -1.0, FAKE, 1, None) == 2
    assert L.gdn_output_gate(FAKE, 2, FAKE, 1, FAKE, 10, 2, 128, 1e-6, FAKE, 1, None) == 3


def test_preprocess_validation(L):
    n = None
    # nothing to do
    assert L.gdn_preprocess(n, n, n, 1, n, n, n, 4, n, n, n, n, n, 1, 8, 2, 128, 128, 1e-6,
                            n, n, n, 1, n, n, None) == 1
    # conv width other than 4
    assert L.gdn_preprocess(FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 3, n, n, n, n, n, 1, 8, 2, 128,
                            128, 1e-6, FAKE, FAKE, FAKE, 1, n, n, None) == 2
    # half of the gate pointers
    assert L.gdn_preprocess(n, n, n, 1, n, n, n, 4, FAKE, FAKE, n, n, n, 1, 8, 2, 128, 128, 1e-6,
                            n, n, n, 1, n, n, None) == 1


def test_stateful_preprocess_and_multi_decode_validation(L):
    n = None
    F = FAKE
    # conv state without the conv inputs
    assert L.gdn_preprocess_stateful(n, n, n, 1, n, n, n, 4, F, F, F, F, n, 1, 8, 2, 128, 128,
                                     1e-6, n, n, n, 1, F, F, F, n, None) == 1
    # overlapping states (double-buffer them)
    st = L.gdn_preprocess_stateful(F, F, F, 1, F, F, F, 4, n, n, n, n, n, 1, 8, 2, 128, 128, 1e-6,
                                   F, F, F, 1, n, n, F, F + 16, None)
    assert st == 2 and b"overlap" in L.gdn_last_error()
    assert L.gdn_preprocess_stateful(F, F, F, 1, F, F, F, 4, n, n, n, n, n, 1, 8, 2, 128, 128,
                                     1e-6, F, F, F, 1, n, n, MIS, n, None) == 5
    for T in (0, 9):   # 1 <= T <= GDN_DECODE_MAX_TOKENS
        st = L.gdn_decode_multi(F, F, F, 1, F, F, F, 1, T, 1, 128, 128, F, 1, n, None)
        assert st == 2 and b"T must be" in L.gdn_last_error()
    st = L.gdn_decode_multi(F, F, F, 1, F, F, F, 2, 4, 1, 128, 128, F, 1, F + 64, None)
    assert st == 2 and b"overlap" in L.gdn_last_error()


def test_backward_validation(L):
    n = None
    F = FAKE
    need = L.gdn_chunk_backward_workspace_size(128, 1, 2, 128, 128)
    assert need > 0
    assert L.gdn_chunk_backward_workspace_size(128, 1, 2, 96, 128) == 0

    def call(**kw):
        a = dict(q=F, k=F, v=F, it=1, g=F, b=F, s0=n, dy=F, dyt=1, dst=n, cu=n, cuh=n, ns=1,
                 nt=128, H=2, dk=128, dv=128, dq=F, dkk=F, dvv=F, dg=F, db=F, ds0=n, ws=F,
                 wsb=need)
        a.update(kw)
        return L.gdn_chunk_backward(a["q"], a["k"], a["v"], a["it"], a["g"], a["b"], a["s0"],
                                    a["dy"], a["dyt"], a["dst"], a["cu"], a["cuh"], a["ns"],
                                    a["nt"], a["H"], a["dk"], a["dv"], a["dq"], a["dkk"], a["dvv"],
                                    a["dg"], a["db"], a["ds0"], a["ws"], a["wsb"], None)
    assert call(dy=None) == 1
    assert call(dyt=3) == 3
    assert call(dv=32) == 2
    assert call(wsb=need - 1) == 6
    assert call(dq=MIS) == 5
    assert call(ns=3) == 2


def test_kda_validation(L):
    n = None
    F = FAKE
    need = L.gdn_kda_chunk_prefill_workspace_size(128, 1, 2, 128)
    assert need > 0

    def call(**kw):
        a = dict(q=F, k=F, v=F, it=1, g=F, b=F, s0=n, st=n, cu=n, cuh=n, ns=1, nt=128, H=2,
                 dk=128, dv=128, y=F, yt=1, ws=F, wsb=need)
        a.update(kw)
        return L.gdn_kda_chunk_prefill(a["q"], a["k"], a["v"], a["it"], a["g"], a["b"], a["s0"],
                                       a["st"], a["cu"], a["cuh"], a["ns"], a["nt"], a["H"],
                                       a["dk"], a["dv"], a["y"], a["yt"], a["ws"], a["wsb"], None)
    assert call(g=None) == 1
    assert call(dk=32) == 2
    assert call(wsb=need - 1) == 6
    assert call(yt=9) == 3


def test_fused_validation(L):
    n = None
    F = FAKE
    need = L.gdn_fused_prefill_workspace_size(128, 1, 2, 128, 128)
    assert need > 0
    assert L.gdn_fused_prefill_workspace_size(128, 1, 2, 64, 128) == 0   # dk must be 128

    def prefill(**kw):
        a = dict(xq=F, xk=F, xv=F, xt=1, wq=F, wk=F, wv=F, ck=4, ar=F, br=F, al=F, dt=F, l2=1e-6,
                 z=F, zt=1, nw=F, re=1e-6, s0=n, st=n, cu=n, cuh=n, ns=1, nt=128, H=2, dk=128,
                 dv=128, o=F, ot=1, q=n, k=n, v=n, g=n, b=n, y=n, ws=F, wsb=need)
        a.update(kw)
        return L.gdn_fused_prefill(*a.values(), None)
    assert prefill(xq=None) == 1
    assert prefill(dk=64) == 2
    assert prefill(ck=3) == 2
    assert prefill(zt=4) == 3
    assert prefill(wsb=need - 1) == 6
    assert prefill(ws=None) == 6
    assert prefill(g=F) == 1                  # g without beta
    assert prefill(q=MIS) == 5
    assert prefill(ns=3) == 2                 # 128 tokens do not split into 3 equal sequences

    def decode(**kw):
        a = dict(xq=F, xk=F, xv=F, xt=1, wq=F, wk=F, wv=F, ck=4, cs=F, ar=F, br=F, al=F, dt=F,
                 l2=1e-6, state=F, z=F, nw=F, re=1e-6, N=4, H=2, dk=128, dv=128, o=F, ot=1, y=n)
        a.update(kw)
        return L.gdn_fused_decode(*a.values(), None)
    assert decode(cs=None) == 1
    assert decode(dv=96) == 2
    assert decode(ck=2) == 2
    assert decode(ot=2) == 3
    assert decode(y=MIS) == 5
    assert decode(re=-1.0) == 2


def test_fused_decode_multi_validation(L):
    n = None
    F = FAKE

    def call(**kw):
        a = dict(xq=F, xk=F, xv=F, xt=1, wq=F, wk=F, wv=F, ck=4, hin=F, hout=F, ar=F, br=F, al=F,
                 dt=F, l2=1e-6, state=F, z=F, nw=F, re=1e-6, N=4, T=4, H=2, dk=128, dv=128, o=F,
                 ot=1, y=n, st=n)
        a.update(kw)
        return L.gdn_fused_decode_multi(*a.values(), None)
    for T in (0, 9):
        assert call(T=T) == 2 and b"T must be" in L.gdn_last_error()
    assert call(hin=n) == 1
    st = call(hout=F + 64)                   # partial overlap of the conv histories
    assert st == 2 and b"conv_state_in" in L.gdn_last_error()
    st = call(st=F + 64)                      # step states over the state
    assert st == 2 and b"step_states" in L.gdn_last_error()
    assert call(xt=3) == 3


def test_noalloc_prefill_refuses_sizes_beyond_its_scratch(L):
    """gdn_chunk_prefill_noalloc checks the workspace these sizes need against the library's
    scratch array on the host, before anything touches the device."""
    import gated_deltanet_recurrence_chunked_amd as g
    need = L.gdn_chunk_prefill_workspace_size(65536, 1, 32, 128, 128, 1)
    assert need > g.NOALLOC_SCRATCH_BYTES
    st = L.gdn_chunk_prefill_noalloc(FAKE, FAKE, FAKE, 1, FAKE, FAKE, None, None, None, None, 1,
                                     65536, 32, 128, 128, FAKE, 1, None)
    assert st == 6
    assert b"scratch array" in L.gdn_last_error()
    header = open(HEADER).read()
    assert f"#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in header
    assert g.NOALLOC_SCRATCH_BYTES == 128 << 20
    # the same validation as gdn_chunk_prefill comes first
    st = L.gdn_chunk_prefill_noalloc(None, FAKE, FAKE, 1, FAKE, FAKE, None, None, None, None, 1,
                                     128, 2, 128, 128, FAKE, 1, None)
    assert st == 1


def test_measurement_aid_validation(L):
    assert L.gdn_mb_stream(FAKE, FAKE + 4096, 17, None) == 2          # not a multiple of 16
    assert L.gdn_mb_stream(None, FAKE, 16, None) == 1
    assert L.gdn_mb_stream(MIS, FAKE + 4096, 16, None) == 5
    assert L.gdn_mb_stream(FAKE, FAKE + 16, 64, None) == 2           # partial overlap
    assert L.gdn_last_error().startswith(b"src and dst must be the same buffer")
    assert L.gdn_mb_mfma_bf16(FAKE, -1, 1, None) == 2
    assert L.gdn_mb_mfma_bf16(FAKE, 1, 0, None) == 2
    assert L.gdn_mb_mfma_bf16(None, 1, 1, None) == 1
