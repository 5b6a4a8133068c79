"""Gated DeltaNet token mixer for MI355X (gfx950): Python binding of libgdn.so.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI of
include/gdn.h. torch supplies device memory and the current stream. There is no
CPU or PyTorch fallback: if libgdn.so is missing these functions raise.

The functions keep the C names:
  gdn_preprocess     eqs. (6)-(10)  ShortConv -> SiLU -> L2Norm (q, k), SiLU (v), gates
  gdn_chunk_prefill  eqs. (1)-(4)   chunkwise (C = 64) gated delta rule over packed sequences
  gdn_preprocess_stateful           the same for sequences that continue earlier input
                                    (carried conv history in and out)
  gdn_chunk_backward eqs. (1)-(4)   gradients of the chunked prefill (dq, dk, dv, dg, dbeta, dS0)
  gdn_kda_chunk_prefill             the same recurrence with a per-channel decay (KDA-style)
  gdn_decode_step    eqs. (1)-(4)   one token per sequence, state updated in place
  gdn_decode_multi   eqs. (1)-(4)   T <= 8 tokens per sequence (multi-token prediction
                                    verify) in one pass over each state
  gdn_output_gate    eq. (11)       sigmoid(z) * zero-centred RMSNorm(y) (without W_o)
(equation numbers of section 2.1.1 of the reading notes of "On the Design of
Qwen3.8-Next Architecture").
"""
from __future__ import annotations

import ctypes
import os

import torch

GDN_F32 = 0
GDN_BF16 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int


class GdnError(RuntimeError):
    pass


def lib():
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GdnError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python -m gated_deltanet_recurrence_chunked_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_abi_version.restype = _i
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [_i]
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_preprocess.restype = _i
        L.gdn_preprocess.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp,
                                     _i, _i, _i, _i, _i, ctypes.c_float, _vp, _vp, _vp, _i, _vp,
                                     _vp, _vp]
        L.gdn_preprocess_stateful.restype = _i
        L.gdn_preprocess_stateful.argtypes = L.gdn_preprocess.argtypes[:-1] + [_vp, _vp, _vp]
        L.gdn_chunk_prefill_workspace_size.restype = ctypes.c_size_t
        L.gdn_chunk_prefill_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
        L.gdn_chunk_prefill.restype = _i
        L.gdn_chunk_prefill.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                        _i, _i, _i, _vp, _i, _vp, ctypes.c_size_t, _vp]
        L.gdn_chunk_prefill_noalloc.restype = _i
        L.gdn_chunk_prefill_noalloc.argtypes = L.gdn_chunk_prefill.argtypes[:17] + [_vp]
        L.gdn_chunk_backward_workspace_size.restype = ctypes.c_size_t
        L.gdn_chunk_backward_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        L.gdn_chunk_backward.restype = _i
        L.gdn_chunk_backward.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _vp, _vp, _vp,
                                         _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         ctypes.c_size_t, _vp]
        L.gdn_kda_chunk_prefill_workspace_size.restype = ctypes.c_size_t
        L.gdn_kda_chunk_prefill_workspace_size.argtypes = [_i, _i, _i, _i]
        L.gdn_kda_chunk_prefill.restype = _i
        L.gdn_kda_chunk_prefill.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i,
                                            _i, _i, _i, _i, _vp, _i, _vp, ctypes.c_size_t, _vp]
        L.gdn_decode_step.restype = _i
        L.gdn_decode_step.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i,
                                      _vp]
        L.gdn_decode_multi.restype = _i
        L.gdn_decode_multi.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp,
                                       _i, _vp, _vp]
        L.gdn_output_gate.restype = _i
        L.gdn_output_gate.argtypes = [_vp, _i, _vp, _i, _vp, _i, _i, _i, ctypes.c_float, _vp, _i,
                                      _vp]
        L.gdn_fused_prefill_workspace_size.restype = ctypes.c_size_t
        L.gdn_fused_prefill_workspace_size.argtypes = [_i, _i, _i, _i, _i]
        L.gdn_fused_prefill.restype = _i
        L.gdn_fused_prefill.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                                        ctypes.c_float, _vp, _i, _vp, ctypes.c_float, _vp, _vp,
                                        _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.gdn_fused_decode.restype = _i
        L.gdn_fused_decode.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp, _vp,
                                       _vp, ctypes.c_float, _vp, _vp, _vp, ctypes.c_float, _i, _i,
                                       _i, _i, _vp, _i, _vp, _vp]
        L.gdn_fused_decode_multi.restype = _i
        L.gdn_fused_decode_multi.argtypes = [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _vp, _vp, _vp,
                                             _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                             ctypes.c_float, _i, _i, _i, _i, _i, _vp, _i, _vp,
                                             _vp, _vp]
        L.gdn_kda_chunk_prefill_bounded_workspace_size.restype = ctypes.c_size_t
        L.gdn_kda_chunk_prefill_bounded_workspace_size.argtypes = [_i, _i, _i]
        L.gdn_kda_chunk_prefill_bounded.argtypes = L.gdn_kda_chunk_prefill.argtypes
        L.gdn_mb_stream.argtypes = [_vp, _vp, ctypes.c_size_t, _vp]
        L.gdn_mb_mfma_bf16.argtypes = [_vp, _i, _i, _vp]
        _lib = L
    return _lib


# ----------------------------------------------------------------------------- marshalling
def _dtype_tag(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise GdnError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _tag_dtype(tag: int) -> torch.dtype:
    return torch.bfloat16 if tag == GDN_BF16 else torch.float32


def _ptr(t, name, dtype=None, device=True):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise GdnError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise GdnError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise GdnError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise GdnError(f"{name} must be a device tensor")
    return t.data_ptr() or None


def _shape(name, t, *shape):
    """The kernels see bare pointers, so every tensor's extent is checked here, on the host:
    raise unless t (when given) has exactly this shape."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise GdnError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype(name, t, dtype):
    """An output tensor given by the caller must have the dtype the call writes: the kernels
    see bare pointers, and a mismatch would write past a smaller-element buffer."""
    if t is not None and t.dtype != dtype:
        raise GdnError(f"{name} must be {dtype} to match the requested output dtype "
                       f"(got {t.dtype})")


def _same_dtype(ref_name, ref, **others):
    for name, t in others.items():
        if t is not None and t.dtype != ref.dtype:
            raise GdnError(f"{name} must have the dtype of {ref_name} ({ref.dtype}, got {t.dtype})")


def _packing(cu_seqlens, cu_seqlens_host, num_seqs):
    _shape("cu_seqlens", cu_seqlens, num_seqs + 1)
    if cu_seqlens_host is not None and len(cu_seqlens_host) != num_seqs + 1:
        raise GdnError(f"cu_seqlens_host has {len(cu_seqlens_host)} entries, expected {num_seqs + 1}")


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class _Alloc:
    """Tensors a call allocates on the caller's behalf (see _keep)."""

    def __init__(self, device):
        self.device = device
        self.made = []

    def __call__(self, shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=self.device)
        self.made.append(t)
        return t

    def get(self, outs, name, shape, dtype):
        return outs[name] if outs.get(name) is not None else self(shape, dtype)


def _keep(stream, *tensors):
    """Tensors a call allocates (workspaces, default outputs) come from torch's caching
    allocator on torch's current stream, while the kernels run on `stream`. When the two
    differ, record the tensors on `stream`, so their memory is not handed to other work
    before the kernels that use it have finished."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if s == torch.cuda.current_stream(s.device):
        return
    for t in tensors:
        if t is not None and t.numel() > 0:
            t.record_stream(s)


def _check(status: int, fn: str):
    if status != 0:
        L = lib()
        raise GdnError(f"{fn}: {L.gdn_status_string(status).decode()}: "
                       f"{L.gdn_last_error().decode()}")


def _tag(dtype) -> int:
    if dtype in (torch.bfloat16, "bf16", GDN_BF16):
        return GDN_BF16
    if dtype in (torch.float32, "f32", GDN_F32):
        return GDN_F32
    raise GdnError(f"unsupported dtype {dtype}")


# ----------------------------------------------------------------------------- entry points
def gdn_preprocess(xq, xk, xv, wq, wk, wv, a_raw, b_raw, A_log, dt_bias, *, H, cu_seqlens=None,
                   num_seqs=1, l2_eps=1e-6, out_dtype=torch.bfloat16, ntok=None, outs=None,
                   stream=None):
    """eqs. 6-10. x*: [ntok,H,d] (bf16/fp32) or all None (gates only); w*: [H*d,4] fp32;
    a_raw, b_raw: [ntok,H] fp32 or None (no gates); A_log, dt_bias: [H] fp32.
    Returns (q, k, v, g, beta) with None for the parts not computed."""
    conv = xq is not None
    gates = a_raw is not None
    ref = xq if conv else a_raw
    if ntok is None:
        ntok = ref.shape[0]
    dk = xq.shape[-1] if conv else 128
    dv = xv.shape[-1] if conv else 128
    dev = ref.device
    x_tag = _dtype_tag(xq) if conv else GDN_F32
    o_tag = _tag(out_dtype)
    if outs is None:
        outs = {}
    if conv:
        _shape("xq", xq, ntok, H, dk)
        _shape("xk", xk, ntok, H, dk)
        _shape("xv", xv, ntok, H, dv)
        _same_dtype("xq", xq, xk=xk, xv=xv)
        _shape("wq", wq, H * dk, 4)
        _shape("wk", wk, H * dk, 4)
        _shape("wv", wv, H * dv, 4)
    if gates:
        _shape("a_raw", a_raw, ntok, H)
        _shape("b_raw", b_raw, ntok, H)
        _shape("A_log", A_log, H)
        _shape("dt_bias", dt_bias, H)
    _packing(cu_seqlens, None, num_seqs)
    for name, shp in (("q", (ntok, H, dk)), ("k", (ntok, H, dk)), ("v", (ntok, H, dv)),
                      ("g", (ntok, H)), ("beta", (ntok, H))):
        _shape(name, outs.get(name), *shp)
    q = k = v = g = beta = None
    od, f32 = _tag_dtype(o_tag), torch.float32
    for name, dt in (("q", od), ("k", od), ("v", od), ("g", f32), ("beta", f32)):
        _dtype(name, outs.get(name), dt)
    new = _Alloc(dev)
    if conv:
        q = new.get(outs, "q", (ntok, H, dk), od)
        k = new.get(outs, "k", (ntok, H, dk), od)
        v = new.get(outs, "v", (ntok, H, dv), od)
    if gates:
        g = new.get(outs, "g", (ntok, H), f32)
        beta = new.get(outs, "beta", (ntok, H), f32)
    st = lib().gdn_preprocess(
        _ptr(xq, "xq"), _ptr(xk, "xk"), _ptr(xv, "xv"), x_tag,
        _ptr(wq, "wq", f32), _ptr(wk, "wk", f32), _ptr(wv, "wv", f32), 4,
        _ptr(a_raw, "a_raw", f32), _ptr(b_raw, "b_raw", f32), _ptr(A_log, "A_log", f32),
        _ptr(dt_bias, "dt_bias", f32), _ptr(cu_seqlens, "cu_seqlens", torch.int32), num_seqs, ntok,
        H, dk, dv, l2_eps, _ptr(q, "q", od), _ptr(k, "k", od), _ptr(v, "v", od), o_tag,
        _ptr(g, "g", f32), _ptr(beta, "beta", f32), _stream(stream))
    _check(st, "gdn_preprocess")
    _keep(stream, *new.made)
    return q, k, v, g, beta


def gdn_preprocess_stateful(xq, xk, xv, wq, wk, wv, a_raw, b_raw, A_log, dt_bias, *, H,
                            conv_state_in=None, conv_state_out=None, cu_seqlens=None,
                            num_seqs=1, l2_eps=1e-6, out_dtype=torch.bfloat16, outs=None,
                            stream=None):
    """gdn_preprocess for sequences that continue earlier input. conv_state_in/out:
    [num_seqs, 3, H*(2*dk+dv)] in the dtype of x* (channels q | k | v), conv_state_in None =
    zero history; pass conv_state_out=True to have it allocated. The two must not overlap.
    Returns (q, k, v, g, beta, conv_state_out)."""
    ntok, _, dk = xq.shape
    dv = xv.shape[-1]
    dev = xq.device
    o_tag = _tag(out_dtype)
    new = _Alloc(dev)
    if conv_state_out is True:
        conv_state_out = new((num_seqs, 3, H * (2 * dk + dv)), xq.dtype)
    outs = {} if outs is None else outs
    _shape("xq", xq, ntok, H, dk)
    _shape("xk", xk, ntok, H, dk)
    _shape("xv", xv, ntok, H, dv)
    _same_dtype("xq", xq, xk=xk, xv=xv)
    _shape("wq", wq, H * dk, 4)
    _shape("wk", wk, H * dk, 4)
    _shape("wv", wv, H * dv, 4)
    if a_raw is not None:
        _shape("a_raw", a_raw, ntok, H)
        _shape("b_raw", b_raw, ntok, H)
        _shape("A_log", A_log, H)
        _shape("dt_bias", dt_bias, H)
    _shape("conv_state_in", conv_state_in, num_seqs, 3, H * (2 * dk + dv))
    _shape("conv_state_out", conv_state_out, num_seqs, 3, H * (2 * dk + dv))
    _packing(cu_seqlens, None, num_seqs)
    for name, shp in (("q", (ntok, H, dk)), ("k", (ntok, H, dk)), ("v", (ntok, H, dv)),
                      ("g", (ntok, H)), ("beta", (ntok, H))):
        _shape(name, outs.get(name), *shp)
    od, f32 = _tag_dtype(o_tag), torch.float32
    for name, dt in (("q", od), ("k", od), ("v", od), ("g", f32), ("beta", f32)):
        _dtype(name, outs.get(name), dt)
    q = new.get(outs, "q", (ntok, H, dk), od)
    k = new.get(outs, "k", (ntok, H, dk), od)
    v = new.get(outs, "v", (ntok, H, dv), od)
    g = beta = None
    if a_raw is not None:
        g = new.get(outs, "g", (ntok, H), f32)
        beta = new.get(outs, "beta", (ntok, H), f32)
    st = lib().gdn_preprocess_stateful(
        _ptr(xq, "xq"), _ptr(xk, "xk"), _ptr(xv, "xv"), _dtype_tag(xq),
        _ptr(wq, "wq", f32), _ptr(wk, "wk", f32), _ptr(wv, "wv", f32), 4,
        _ptr(a_raw, "a_raw", f32), _ptr(b_raw, "b_raw", f32), _ptr(A_log, "A_log", f32),
        _ptr(dt_bias, "dt_bias", f32), _ptr(cu_seqlens, "cu_seqlens", torch.int32), num_seqs, ntok,
        H, dk, dv, l2_eps, _ptr(q, "q", od), _ptr(k, "k", od), _ptr(v, "v", od), o_tag,
        _ptr(g, "g", f32), _ptr(beta, "beta", f32),
        _ptr(conv_state_in, "conv_state_in", xq.dtype),
        _ptr(conv_state_out, "conv_state_out", xq.dtype), _stream(stream))
    _check(st, "gdn_preprocess_stateful")
    _keep(stream, *new.made)
    return q, k, v, g, beta, conv_state_out


def gdn_chunk_prefill_workspace_size(ntok, num_seqs, H, dk, dv, in_dtype=torch.bfloat16) -> int:
    return int(lib().gdn_chunk_prefill_workspace_size(ntok, num_seqs, H, dk, dv, _tag(in_dtype)))


def gdn_chunk_prefill(q, k, v, g, beta, *, initial_state=None, final_state=None, cu_seqlens=None,
                      cu_seqlens_host=None, num_seqs=1, y=None, y_dtype=None, workspace=None,
                      output_final_state=True, stream=None):
    """eqs. 1-4 chunkwise. q,k: [ntok,H,dk], v: [ntok,H,dv] (bf16/fp32); g, beta: [ntok,H] fp32;
    states [num_seqs,H,dk,dv] fp32. Returns (y, final_state)."""
    ntok, H, dk = q.shape
    dv = v.shape[-1]
    in_tag = _dtype_tag(q)
    y_tag = _tag(y_dtype) if y_dtype is not None else (_dtype_tag(y) if y is not None else in_tag)
    dev = q.device
    _shape("k", k, ntok, H, dk)
    _shape("v", v, ntok, H, dv)
    _same_dtype("q", q, k=k, v=v)
    _shape("g", g, ntok, H)
    _shape("beta", beta, ntok, H)
    _shape("initial_state", initial_state, num_seqs, H, dk, dv)
    _shape("final_state", final_state, num_seqs, H, dk, dv)
    _shape("y", y, ntok, H, dv)
    _packing(cu_seqlens, cu_seqlens_host, num_seqs)
    yd = _tag_dtype(y_tag)
    _dtype("y", y, yd)
    _dtype("final_state", final_state, torch.float32)
    new = _Alloc(dev)
    if y is None:
        y = new((ntok, H, dv), yd)
    if final_state is None and output_final_state:
        final_state = new((num_seqs, H, dk, dv), torch.float32)
    need = gdn_chunk_prefill_workspace_size(ntok, num_seqs, H, dk, dv, in_tag)
    if need and workspace is None:
        workspace = new(need, torch.uint8)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    f32 = torch.float32
    st = lib().gdn_chunk_prefill(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), in_tag, _ptr(g, "g", f32), _ptr(beta, "beta", f32),
        _ptr(initial_state, "initial_state", f32), _ptr(final_state, "final_state", f32),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32),
        ctypes.cast(host_cu, _vp) if host_cu is not None else None, num_seqs, ntok, H, dk, dv,
        _ptr(y, "y", yd), y_tag, _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gdn_chunk_prefill")
    _keep(stream, *new.made)
    return y, final_state


NOALLOC_SCRATCH_BYTES = 128 << 20      # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


def gdn_chunk_prefill_noalloc(q, k, v, g, beta, *, y, initial_state=None, final_state=None,
                              cu_seqlens=None, cu_seqlens_host=None, num_seqs=1, stream=None):
    """gdn_chunk_prefill without a workspace: the library uses its own scratch array (one per
    GPU, NOALLOC_SCRATCH_BYTES). Allocates nothing, here or in the library, so the caller
    passes y [ntok,H,dv] (bf16 or fp32: its dtype is y_dtype) and final_state (or None: not
    written). Calls that overlap in time on one GPU share the array and race.
    Returns (y, final_state)."""
    ntok, H, dk = q.shape
    dv = v.shape[-1]
    _shape("k", k, ntok, H, dk)
    _shape("v", v, ntok, H, dv)
    _same_dtype("q", q, k=k, v=v)
    _shape("g", g, ntok, H)
    _shape("beta", beta, ntok, H)
    _shape("initial_state", initial_state, num_seqs, H, dk, dv)
    _shape("final_state", final_state, num_seqs, H, dk, dv)
    _shape("y", y, ntok, H, dv)
    _dtype("final_state", final_state, torch.float32)
    _packing(cu_seqlens, cu_seqlens_host, num_seqs)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    f32 = torch.float32
    st = lib().gdn_chunk_prefill_noalloc(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _dtype_tag(q), _ptr(g, "g", f32),
        _ptr(beta, "beta", f32), _ptr(initial_state, "initial_state", f32),
        _ptr(final_state, "final_state", f32), _ptr(cu_seqlens, "cu_seqlens", torch.int32),
        ctypes.cast(host_cu, _vp) if host_cu is not None else None, num_seqs, ntok, H, dk, dv,
        _ptr(y, "y"), _dtype_tag(y), _stream(stream))
    _check(st, "gdn_chunk_prefill_noalloc")
    return y, final_state


def gdn_chunk_backward_workspace_size(ntok, num_seqs, H, dk, dv) -> int:
    return int(lib().gdn_chunk_backward_workspace_size(ntok, num_seqs, H, dk, dv))


def gdn_chunk_backward(q, k, v, g, beta, dy, *, initial_state=None, dfinal_state=None,
                       cu_seqlens=None, cu_seqlens_host=None, num_seqs=1, workspace=None,
                       want_dinitial_state=True, stream=None):
    """Gradients of gdn_chunk_prefill. Inputs as its forward (q,k,v bf16/fp32; g, beta fp32),
    dy [ntok,H,dv] (bf16/fp32), dfinal_state [num_seqs,H,dk,dv] fp32 or None.
    Returns dict(dq, dk, dv, dg, dbeta, dinitial_state) of fp32 tensors."""
    ntok, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    _shape("k", k, ntok, H, dk)
    _shape("v", v, ntok, H, dv)
    _same_dtype("q", q, k=k, v=v)
    _shape("g", g, ntok, H)
    _shape("beta", beta, ntok, H)
    _shape("dy", dy, ntok, H, dv)
    _shape("initial_state", initial_state, num_seqs, H, dk, dv)
    _shape("dfinal_state", dfinal_state, num_seqs, H, dk, dv)
    _packing(cu_seqlens, cu_seqlens_host, num_seqs)
    f32 = torch.float32
    new = _Alloc(dev)
    out = dict(dq=new((ntok, H, dk), f32), dk=new((ntok, H, dk), f32), dv=new((ntok, H, dv), f32),
               dg=new((ntok, H), f32), dbeta=new((ntok, H), f32),
               dinitial_state=new((num_seqs, H, dk, dv), f32) if want_dinitial_state else None)
    need = gdn_chunk_backward_workspace_size(ntok, num_seqs, H, dk, dv)
    if workspace is None:
        workspace = new(max(need, 1), torch.uint8)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    st = lib().gdn_chunk_backward(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), _dtype_tag(q), _ptr(g, "g", f32),
        _ptr(beta, "beta", f32), _ptr(initial_state, "initial_state", f32), _ptr(dy, "dy"),
        _dtype_tag(dy), _ptr(dfinal_state, "dfinal_state", f32),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32),
        ctypes.cast(host_cu, _vp) if host_cu is not None else None, num_seqs, ntok, H, dk, dv,
        _ptr(out["dq"], "dq"), _ptr(out["dk"], "dk"), _ptr(out["dv"], "dv"), _ptr(out["dg"], "dg"),
        _ptr(out["dbeta"], "dbeta"), _ptr(out["dinitial_state"], "dinitial_state"),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "gdn_chunk_backward")
    _keep(stream, *new.made)
    return out


def _kda(bounded, q, k, v, g, beta, initial_state, final_state, cu_seqlens, cu_seqlens_host,
         num_seqs, y, y_dtype, workspace, output_final_state, stream):
    ntok, H, dk = q.shape
    dv = v.shape[-1]
    in_tag = _dtype_tag(q)
    y_tag = _tag(y_dtype) if y_dtype is not None else (_dtype_tag(y) if y is not None else in_tag)
    dev = q.device
    _shape("k", k, ntok, H, dk)
    _shape("v", v, ntok, H, dv)
    _same_dtype("q", q, k=k, v=v)
    _shape("g", g, ntok, H, dk)
    _shape("beta", beta, ntok, H)
    _shape("initial_state", initial_state, num_seqs, H, dk, dv)
    _shape("final_state", final_state, num_seqs, H, dk, dv)
    _shape("y", y, ntok, H, dv)
    _packing(cu_seqlens, cu_seqlens_host, num_seqs)
    yd = _tag_dtype(y_tag)
    _dtype("y", y, yd)
    _dtype("final_state", final_state, torch.float32)
    new = _Alloc(dev)
    if y is None:
        y = new((ntok, H, dv), yd)
    if final_state is None and output_final_state:
        final_state = new((num_seqs, H, dk, dv), torch.float32)
    name = "gdn_kda_chunk_prefill_bounded" if bounded else "gdn_kda_chunk_prefill"
    if bounded:
        need = int(lib().gdn_kda_chunk_prefill_bounded_workspace_size(ntok, num_seqs, H))
    else:
        need = int(lib().gdn_kda_chunk_prefill_workspace_size(ntok, num_seqs, H, dk))
    if workspace is None:
        workspace = new(max(need, 1), torch.uint8)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    f32 = torch.float32
    st = getattr(lib(), name)(
        _ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), in_tag, _ptr(g, "g", f32), _ptr(beta, "beta", f32),
        _ptr(initial_state, "initial_state", f32), _ptr(final_state, "final_state", f32),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32),
        ctypes.cast(host_cu, _vp) if host_cu is not None else None, num_seqs, ntok, H, dk, dv,
        _ptr(y, "y", yd), y_tag, _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, name)
    _keep(stream, *new.made)
    return y, final_state


def gdn_kda_chunk_prefill(q, k, v, g, beta, *, initial_state=None, final_state=None,
                          cu_seqlens=None, cu_seqlens_host=None, num_seqs=1, y=None, y_dtype=None,
                          workspace=None, output_final_state=True, stream=None):
    """Per-channel-decay delta rule. q,k: [ntok,H,dk], v: [ntok,H,dv] (bf16/fp32);
    g: [ntok,H,dk] fp32 log-decays; beta: [ntok,H] fp32; final_state: None (allocated when
    output_final_state) or [num_seqs,H,dk,dv] fp32, which may be initial_state (updated in
    place). Returns (y, final_state)."""
    return _kda(False, q, k, v, g, beta, initial_state, final_state, cu_seqlens, cu_seqlens_host,
                num_seqs, y, y_dtype, workspace, output_final_state, stream)


def gdn_kda_chunk_prefill_bounded(q, k, v, g, beta, *, initial_state=None, final_state=None,
                                  cu_seqlens=None, cu_seqlens_host=None, num_seqs=1, y=None,
                                  y_dtype=None, workspace=None, output_final_state=True,
                                  stream=None):
    """gdn_kda_chunk_prefill for log-decays -5 <= g <= 0 on the bf16 matrix cores: q, k, v bf16,
    dk = dv = 128. Returns (y, final_state)."""
    return _kda(True, q, k, v, g, beta, initial_state, final_state, cu_seqlens, cu_seqlens_host,
                num_seqs, y, y_dtype, workspace, output_final_state, stream)


def gdn_decode_step(q, k, v, g, beta, state, *, y=None, y_dtype=None, stream=None):
    """One token per sequence. q,k: [N,H,dk], v: [N,H,dv]; g,beta: [N,H] fp32;
    state: [N,H,dk,dv] fp32 updated in place. Returns y [N,H,dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    _shape("k", k, N, H, dk)
    _shape("v", v, N, H, dv)
    _same_dtype("q", q, k=k, v=v)
    _shape("g", g, N, H)
    _shape("beta", beta, N, H)
    _shape("state", state, N, H, dk, dv)
    _shape("y", y, N, H, dv)
    in_tag = _dtype_tag(q)
    y_tag = _tag(y_dtype) if y_dtype is not None else (_dtype_tag(y) if y is not None else in_tag)
    yd = _tag_dtype(y_tag)
    _dtype("y", y, yd)
    new = _Alloc(q.device)
    if y is None:
        y = new((N, H, dv), yd)
    f32 = torch.float32
    st = lib().gdn_decode_step(_ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), in_tag, _ptr(g, "g", f32),
                               _ptr(beta, "beta", f32), _ptr(state, "state", f32), N, H, dk, dv,
                               _ptr(y, "y", yd), y_tag, _stream(stream))
    _check(st, "gdn_decode_step")
    _keep(stream, *new.made)
    return y


def gdn_decode_multi(q, k, v, g, beta, state, *, y=None, y_dtype=None, step_states=None,
                     stream=None):
    """T tokens per sequence in one pass over each state. q,k: [N,T,H,dk], v: [N,T,H,dv];
    g,beta: [N,T,H] fp32; state: [N,H,dk,dv] fp32 updated in place; step_states: None, True
    (allocate) or [N,T,H,dk,dv] fp32 receiving the state after each token.
    Returns (y [N,T,H,dv], step_states)."""
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    _shape("k", k, N, T, H, dk)
    _shape("v", v, N, T, H, dv)
    _same_dtype("q", q, k=k, v=v)
    _shape("g", g, N, T, H)
    _shape("beta", beta, N, T, H)
    _shape("state", state, N, H, dk, dv)
    _shape("y", y, N, T, H, dv)
    if step_states is not True:
        _shape("step_states", step_states, N, T, H, dk, dv)
    in_tag = _dtype_tag(q)
    y_tag = _tag(y_dtype) if y_dtype is not None else (_dtype_tag(y) if y is not None else in_tag)
    yd = _tag_dtype(y_tag)
    _dtype("y", y, yd)
    new = _Alloc(q.device)
    if y is None:
        y = new((N, T, H, dv), yd)
    if step_states is True:
        step_states = new((N, T, H, dk, dv), torch.float32)
    f32 = torch.float32
    st = lib().gdn_decode_multi(_ptr(q, "q"), _ptr(k, "k"), _ptr(v, "v"), in_tag,
                                _ptr(g, "g", f32), _ptr(beta, "beta", f32),
                                _ptr(state, "state", f32), N, T, H, dk, dv, _ptr(y, "y", yd), y_tag,
                                _ptr(step_states, "step_states", f32), _stream(stream))
    _check(st, "gdn_decode_multi")
    _keep(stream, *new.made)
    return y, step_states


def gdn_output_gate(y, z, norm_weight, *, eps=1e-6, o=None, o_dtype=None, stream=None):
    """eq. 11 without W_o. y, z: [ntok,H,dv]; norm_weight: [dv] fp32. Returns o."""
    ntok, H, dv = y.shape
    _shape("z", z, ntok, H, dv)
    _shape("norm_weight", norm_weight, dv)
    _shape("o", o, ntok, H, dv)
    o_tag = _tag(o_dtype) if o_dtype is not None else (_dtype_tag(o) if o is not None else _dtype_tag(y))
    od = _tag_dtype(o_tag)
    _dtype("o", o, od)
    new = _Alloc(y.device)
    if o is None:
        o = new((ntok, H, dv), od)
    st = lib().gdn_output_gate(_ptr(y, "y"), _dtype_tag(y), _ptr(z, "z"), _dtype_tag(z),
                               _ptr(norm_weight, "norm_weight", torch.float32), ntok, H, dv, eps,
                               _ptr(o, "o", od), o_tag, _stream(stream))
    _check(st, "gdn_output_gate")
    _keep(stream, *new.made)
    return o


def gdn_mb_stream(src, dst, *, stream=None):
    """Measurement aid: copies src into dst (the same tensor for the in-place stream) with
    16-byte nontemporal loads and stores. Both are contiguous device tensors of equal byte
    size, a multiple of 16."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise GdnError("src and dst must have the same size in bytes")
    st = lib().gdn_mb_stream(_ptr(src, "src"), _ptr(dst, "dst"), nbytes, _stream(stream))
    _check(st, "gdn_mb_stream")


def gdn_mb_mfma_bf16(sink, iters, *, stream=None):
    """Measurement aid: sink.numel() workgroups of 4 waves, each wave issuing iters rounds of
    four independent 32x32x16 bf16 matrix-core products. Returns the flops of the call."""
    _dtype("sink", sink, torch.float32)
    wg = sink.numel()
    st = lib().gdn_mb_mfma_bf16(_ptr(sink, "sink"), wg, int(iters), _stream(stream))
    _check(st, "gdn_mb_mfma_bf16")
    return wg * 4 * int(iters) * 4 * 32768


def gdn_fused_prefill_workspace_size(ntok, num_seqs, H, dk, dv) -> int:
    return int(lib().gdn_fused_prefill_workspace_size(ntok, num_seqs, H, dk, dv))


def gdn_fused_prefill(xq, xk, xv, wq, wk, wv, a_raw, b_raw, A_log, dt_bias, z, norm_weight, *,
                      H, initial_state=None, output_final_state=True, cu_seqlens=None,
                      cu_seqlens_host=None, num_seqs=1, l2_eps=1e-6, rms_eps=1e-6, o=None,
                      o_dtype=None, export=False, workspace=None, stream=None):
    """eqs. 6-11 in one call. xq, xk: [ntok,H,128], xv, z: [ntok,H,dv] (bf16/fp32); conv taps
    [H*d,4] fp32; a_raw, b_raw: [ntok,H] fp32; A_log, dt_bias: [H]; norm_weight: [dv].
    o_dtype: the dtype of o (default: that of a given o, else bf16).
    Returns (o, final_state) or, with export=True, (o, final_state, dict(q, k, v, g, beta, y))."""
    ntok = xq.shape[0]
    dk, dv = xq.shape[-1], xv.shape[-1]
    dev = xq.device
    _shape("xq", xq, ntok, H, dk)
    _shape("xk", xk, ntok, H, dk)
    _shape("xv", xv, ntok, H, dv)
    _same_dtype("xq", xq, xk=xk, xv=xv)
    _shape("wq", wq, H * dk, 4)
    _shape("wk", wk, H * dk, 4)
    _shape("wv", wv, H * dv, 4)
    _shape("a_raw", a_raw, ntok, H)
    _shape("b_raw", b_raw, ntok, H)
    _shape("A_log", A_log, H)
    _shape("dt_bias", dt_bias, H)
    _shape("z", z, ntok, H, dv)
    _shape("norm_weight", norm_weight, dv)
    _shape("initial_state", initial_state, num_seqs, H, dk, dv)
    _shape("o", o, ntok, H, dv)
    _packing(cu_seqlens, cu_seqlens_host, num_seqs)
    o_tag = _tag(o_dtype) if o_dtype is not None else (_dtype_tag(o) if o is not None else GDN_BF16)
    od = _tag_dtype(o_tag)
    _dtype("o", o, od)
    new = _Alloc(dev)
    if o is None:
        o = new((ntok, H, dv), od)
    final_state = new((num_seqs, H, dk, dv), torch.float32) if output_final_state else None
    ex = {}
    if export:
        bf = torch.bfloat16
        ex = dict(q=new((ntok, H, dk), bf), k=new((ntok, H, dk), bf), v=new((ntok, H, dv), bf),
                  g=new((ntok, H), torch.float32), beta=new((ntok, H), torch.float32),
                  y=new((ntok, H, dv), bf))
    need = gdn_fused_prefill_workspace_size(ntok, num_seqs, H, dk, dv)
    if workspace is None:
        workspace = new(max(need, 1), torch.uint8)
    host_cu = None
    if cu_seqlens_host is not None:
        host_cu = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    f32 = torch.float32
    st = lib().gdn_fused_prefill(
        _ptr(xq, "xq"), _ptr(xk, "xk"), _ptr(xv, "xv"), _dtype_tag(xq), _ptr(wq, "wq", f32),
        _ptr(wk, "wk", f32), _ptr(wv, "wv", f32), 4, _ptr(a_raw, "a_raw", f32),
        _ptr(b_raw, "b_raw", f32), _ptr(A_log, "A_log", f32), _ptr(dt_bias, "dt_bias", f32),
        l2_eps, _ptr(z, "z"), _dtype_tag(z), _ptr(norm_weight, "norm_weight", f32), rms_eps,
        _ptr(initial_state, "initial_state", f32), _ptr(final_state, "final_state", f32),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32),
        ctypes.cast(host_cu, _vp) if host_cu is not None else None, num_seqs, ntok, H, dk, dv,
        _ptr(o, "o", od), o_tag, _ptr(ex.get("q"), "q"), _ptr(ex.get("k"), "k"),
        _ptr(ex.get("v"), "v"), _ptr(ex.get("g"), "g"), _ptr(ex.get("beta"), "beta"),
        _ptr(ex.get("y"), "y"), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gdn_fused_prefill")
    _keep(stream, *new.made)
    return (o, final_state, ex) if export else (o, final_state)


def gdn_fused_decode(xq, xk, xv, wq, wk, wv, conv_state, a_raw, b_raw, A_log, dt_bias, state, z,
                     norm_weight, *, l2_eps=1e-6, rms_eps=1e-6, o=None, o_dtype=None,
                     want_y=False, stream=None):
    """One decode step from the projected streams. xq, xk: [N,H,dk], xv, z: [N,H,dv] (bf16/fp32,
    z in the dtype of x); conv_state: [N,3,H*(2dk+dv)] (x dtype) and state: [N,H,dk,dv] fp32,
    both updated in place. Returns o, or (o, y) with want_y=True."""
    N, H, dk = xq.shape
    dv = xv.shape[-1]
    x_tag = _dtype_tag(xq)
    _shape("xk", xk, N, H, dk)
    _shape("xv", xv, N, H, dv)
    _same_dtype("xq", xq, xk=xk, xv=xv, z=z, conv_state=conv_state)
    _shape("wq", wq, H * dk, 4)
    _shape("wk", wk, H * dk, 4)
    _shape("wv", wv, H * dv, 4)
    _shape("conv_state", conv_state, N, 3, H * (2 * dk + dv))
    _shape("a_raw", a_raw, N, H)
    _shape("b_raw", b_raw, N, H)
    _shape("A_log", A_log, H)
    _shape("dt_bias", dt_bias, H)
    _shape("state", state, N, H, dk, dv)
    _shape("z", z, N, H, dv)
    _shape("norm_weight", norm_weight, dv)
    _shape("o", o, N, H, dv)
    o_tag = _tag(o_dtype) if o_dtype is not None else (_dtype_tag(o) if o is not None else x_tag)
    od = _tag_dtype(o_tag)
    _dtype("o", o, od)
    new = _Alloc(xq.device)
    if o is None:
        o = new((N, H, dv), od)
    y = new((N, H, dv), od) if want_y else None
    f32 = torch.float32
    st = lib().gdn_fused_decode(
        _ptr(xq, "xq"), _ptr(xk, "xk"), _ptr(xv, "xv"), x_tag, _ptr(wq, "wq", f32),
        _ptr(wk, "wk", f32), _ptr(wv, "wv", f32), 4, _ptr(conv_state, "conv_state", xq.dtype),
        _ptr(a_raw, "a_raw", f32), _ptr(b_raw, "b_raw", f32), _ptr(A_log, "A_log", f32),
        _ptr(dt_bias, "dt_bias", f32), l2_eps, _ptr(state, "state", f32), _ptr(z, "z"),
        _ptr(norm_weight, "norm_weight", f32), rms_eps, N, H, dk, dv, _ptr(o, "o", od), o_tag,
        _ptr(y, "y", od), _stream(stream))
    _check(st, "gdn_fused_decode")
    _keep(stream, *new.made)
    return (o, y) if want_y else o


def gdn_fused_decode_multi(xq, xk, xv, wq, wk, wv, conv_state_in, a_raw, b_raw, A_log, dt_bias,
                           state, z, norm_weight, *, conv_state_out=None, l2_eps=1e-6,
                           rms_eps=1e-6, o=None, o_dtype=None, want_y=False, step_states=None,
                           stream=None):
    """T tokens per sequence through the fused step. xq, xk: [N,T,H,dk], xv, z: [N,T,H,dv]
    (x dtype); a_raw, b_raw: [N,T,H] fp32; conv_state_in: [N,3,H*(2dk+dv)]; conv_state_out:
    None (update conv_state_in in place) or a separate buffer of that shape; state updated in
    place; step_states: None, True (allocate) or [N,T,H,dk,dv] fp32.
    Returns (o, y or None, step_states)."""
    N, T, H, dk = xq.shape
    dv = xv.shape[-1]
    x_tag = _dtype_tag(xq)
    _shape("xk", xk, N, T, H, dk)
    _shape("xv", xv, N, T, H, dv)
    _same_dtype("xq", xq, xk=xk, xv=xv, z=z, conv_state_in=conv_state_in,
                conv_state_out=conv_state_out)
    _shape("wq", wq, H * dk, 4)
    _shape("wk", wk, H * dk, 4)
    _shape("wv", wv, H * dv, 4)
    _shape("conv_state_in", conv_state_in, N, 3, H * (2 * dk + dv))
    _shape("conv_state_out", conv_state_out, N, 3, H * (2 * dk + dv))
    _shape("a_raw", a_raw, N, T, H)
    _shape("b_raw", b_raw, N, T, H)
    _shape("A_log", A_log, H)
    _shape("dt_bias", dt_bias, H)
    _shape("state", state, N, H, dk, dv)
    _shape("z", z, N, T, H, dv)
    _shape("norm_weight", norm_weight, dv)
    _shape("o", o, N, T, H, dv)
    if step_states is not True:
        _shape("step_states", step_states, N, T, H, dk, dv)
    o_tag = _tag(o_dtype) if o_dtype is not None else (_dtype_tag(o) if o is not None else x_tag)
    od = _tag_dtype(o_tag)
    _dtype("o", o, od)
    new = _Alloc(xq.device)
    if o is None:
        o = new((N, T, H, dv), od)
    y = new((N, T, H, dv), od) if want_y else None
    if conv_state_out is None:
        conv_state_out = conv_state_in
    if step_states is True:
        step_states = new((N, T, H, dk, dv), torch.float32)
    f32 = torch.float32
    st = lib().gdn_fused_decode_multi(
        _ptr(xq, "xq"), _ptr(xk, "xk"), _ptr(xv, "xv"), x_tag, _ptr(wq, "wq", f32),
        _ptr(wk, "wk", f32), _ptr(wv, "wv", f32), 4, _ptr(conv_state_in, "conv_state_in", xq.dtype),
        _ptr(conv_state_out, "conv_state_out", xq.dtype), _ptr(a_raw, "a_raw", f32),
        _ptr(b_raw, "b_raw", f32), _ptr(A_log, "A_log", f32), _ptr(dt_bias, "dt_bias", f32),
        l2_eps, _ptr(state, "state", f32), _ptr(z, "z"), _ptr(norm_weight, "norm_weight", f32),
        rms_eps, N, T, H, dk, dv, _ptr(o, "o", od), o_tag, _ptr(y, "y", od),
        _ptr(step_states, "step_states", f32), _stream(stream))
    _check(st, "gdn_fused_decode_multi")
    _keep(stream, *new.made)
    return o, y, step_states


__all__ = ["GDN_F32", "GDN_BF16", "GdnError", "lib", "gdn_preprocess", "gdn_preprocess_stateful",
           "gdn_chunk_prefill", "gdn_chunk_prefill_workspace_size", "gdn_chunk_prefill_noalloc",
           "NOALLOC_SCRATCH_BYTES", "gdn_chunk_backward",
           "gdn_chunk_backward_workspace_size", "gdn_kda_chunk_prefill", "gdn_decode_step",
           "gdn_decode_multi", "gdn_output_gate", "gdn_fused_prefill",
           "gdn_fused_prefill_workspace_size", "gdn_fused_decode", "gdn_fused_decode_multi",
           "gdn_mb_stream", "gdn_mb_mfma_bf16", "gdn_kda_chunk_prefill_bounded"]
