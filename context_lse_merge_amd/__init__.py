"""Python binding of libdcp.so, the MI355X DCP LSE merge (C ABI in include/dcp.h).

Argument marshalling only: every function here has the name of the C entry
point it calls, turns torch tensors into device pointers, element strides and
the current HIP stream, and raises ``DcpError`` on a nonzero status.  Every
step of the computation runs in the library's HIP kernels; there is no other
path.  If the library has not been built, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcp.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dcp.h")


def _header_constants(path):
    consts = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"#define\s+(DCP_[A-Z0-9_]+)\s+(-?\d+)\b", line)
            if m:
                consts[m.group(1)] = int(m.group(2))
    return consts


_C = _header_constants(HEADER_PATH)
DCP_OK = _C["DCP_OK"]
DCP_ERR_INVALID_ARG = _C["DCP_ERR_INVALID_ARG"]
DCP_ERR_LAYOUT = _C["DCP_ERR_LAYOUT"]
DCP_ERR_ALIGN = _C["DCP_ERR_ALIGN"]
DCP_ERR_STREAM = _C["DCP_ERR_STREAM"]
DCP_ERR_WORKSPACE = _C["DCP_ERR_WORKSPACE"]
DCP_ERR_HIP = _C["DCP_ERR_HIP"]
DCP_LSE_BASE_E = _C["DCP_LSE_BASE_E"]
DCP_LSE_BASE_2 = _C["DCP_LSE_BASE_2"]
DCP_LSE_BHC = _C["DCP_LSE_BHC"]
DCP_LSE_BH1 = _C["DCP_LSE_BH1"]
DCP_DTYPE_BF16 = _C["DCP_DTYPE_BF16"]
DCP_DTYPE_FP16 = _C["DCP_DTYPE_FP16"]
DCP_HEAD_DIM = _C["DCP_HEAD_DIM"]
DCP_QK_DIM = _C["DCP_QK_DIM"]
DCP_MAX_CP = _C["DCP_MAX_CP"]
DCP_LOAD_STREAMING = _C["DCP_LOAD_STREAMING"]
DCP_LOAD_CACHED = _C["DCP_LOAD_CACHED"]
DCP_KV_CONTIGUOUS = _C["DCP_KV_CONTIGUOUS"]
DCP_KV_INTERLEAVED = _C["DCP_KV_INTERLEAVED"]
DCP_NOALLOC_SCRATCH_BYTES = _C["DCP_NOALLOC_SCRATCH_BYTES"]
DCP_FUSE_NONE = _C["DCP_FUSE_NONE"]
DCP_FUSE_EPILOGUE = _C["DCP_FUSE_EPILOGUE"]
DCP_FUSE_AUTO = _C["DCP_FUSE_AUTO"]
DCP_FUSE_REDUCTIONS = _C["DCP_FUSE_REDUCTIONS"]

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "context_lse_merge_amd: %s is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "(or python context_lse_merge_amd/_build.py) first" % LIB_PATH)

# torch ships its own HIP runtime.  Loading it first makes libdcp.so bind to
# that same runtime (the sonames match); loaded the other way round, the
# process would hold two HIP runtimes and kernels launched through one would
# not see the device state of the other.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_lib.dcp_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]
_lib.dcp_workspace_create.argtypes = [_vp, _sz, _i64, _i32, _i32, _i32, _i32, _vp, ctypes.POINTER(_vp)]
_lib.dcp_workspace_recv.argtypes = [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.POINTER(_i64),
                                    ctypes.POINTER(_vp), ctypes.POINTER(_i64)]
_lib.dcp_workspace_destroy.argtypes = [_vp]
_lib.dcp_workspace_set_load_policy.argtypes = [_vp, _i32]
_lib.dcp_lse_combine.argtypes = [_vp, _vp, _i64, _i32, _i64, _i64, _vp, _i32, _i64, _i64, _i64, _i32, _vp, _i64,
                                 _i64, _vp, _i64, _vp]
_lib.dcp_mla_partial_decode_scratch_size.argtypes = [_i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
_lib.dcp_mla_partial_decode.argtypes = [_vp, _i64, _i32, _i64, _i64, _vp, _i64, _i64, _i32, _i32, ctypes.c_float,
                                        _i32, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp]
_lib.dcp_mla_partial_decode_noalloc.argtypes = [_vp, _i64, _i32, _i64, _i64, _vp, _i64, _i64, _i32, _i32,
                                                ctypes.c_float, _i32, _vp, _i64, _i64, _vp, _i64, _vp]
_lib.dcp_mla_decode_merged_scratch_size.argtypes = [_i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
_lib.dcp_mla_decode_merged.argtypes = [_vp, _i64, _i32, _i64, _i64, _vp, _i64, _i64, _i32, _i32, ctypes.c_float, _i32,
                                       _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i32, _vp, _sz, _vp]
_lib.dcp_mla_partial_decode_varlen_scratch_size.argtypes = [_i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
_lib.dcp_mla_partial_decode_varlen.argtypes = [_vp, _i64, _i32, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i32, _i32,
                                               _i32, ctypes.c_float, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _sz, _vp]
_lib.dcp_last_error.restype = ctypes.c_char_p
_lib.dcp_status_string.argtypes = [_i32]
_lib.dcp_status_string.restype = ctypes.c_char_p
for _f in ("dcp_workspace_size", "dcp_workspace_create", "dcp_workspace_recv", "dcp_workspace_destroy", "dcp_workspace_set_load_policy", "dcp_lse_combine",
           "dcp_mla_partial_decode_scratch_size", "dcp_mla_partial_decode", "dcp_mla_partial_decode_noalloc",
           "dcp_mla_decode_merged_scratch_size", "dcp_mla_decode_merged",
           "dcp_mla_partial_decode_varlen_scratch_size", "dcp_mla_partial_decode_varlen"):
    getattr(_lib, _f).restype = _i32


class DcpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (dcp_status_string(status), message))
        self.status = status


def dcp_last_error() -> str:
    return _lib.dcp_last_error().decode()


def dcp_status_string(status: int) -> str:
    return _lib.dcp_status_string(status).decode()


def _check(rc: int):
    if rc != DCP_OK:
        raise DcpError(rc, dcp_last_error())


def _stream_handle(stream):
    """A hipStream_t as an integer: None -> torch's current stream on the current device."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (got device %s)" % (name, t.device))
    return t.data_ptr()


class Workspace:
    """Owns a dcp_workspace handle; ``handle`` is what the C calls take.  ``buf``
    is the device buffer it was created over (kept alive with it)."""

    def __init__(self, handle: int, capacity: int, h_local: int, cp: int, stream: int, dtype: int, buf=None):
        self.handle = handle
        self.capacity = capacity
        self.h_local = h_local
        self.cp = cp
        self.stream = stream
        self.dtype = dtype
        self.buf = buf

    def close(self):
        if self.handle:
            _check(_lib.dcp_workspace_destroy(self.handle))
            self.handle = None
        self.buf = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def dcp_workspace_size(capacity_tokens: int, h_local: int, cp: int, d: int = DCP_HEAD_DIM,
                       dtype: int = DCP_DTYPE_BF16) -> int:
    """Bytes of device memory a workspace of this geometry needs."""
    n = _sz()
    _check(_lib.dcp_workspace_size(capacity_tokens, h_local, cp, d, dtype, ctypes.byref(n)))
    return n.value


def dcp_workspace_create(capacity_tokens: int, h_local: int, cp: int, d: int = DCP_HEAD_DIM,
                         dtype: int = DCP_DTYPE_BF16, stream=None, buf=None, buf_bytes=None) -> Workspace:
    """Create a workspace bound to ``stream`` (default: torch's current stream).
    ``dtype`` is DCP_DTYPE_BF16 or DCP_DTYPE_FP16, the payload type of every call.
    ``buf`` is its device buffer: a GPU tensor, a raw device address (with
    ``buf_bytes``), or None to allocate dcp_workspace_size() bytes with torch on
    the current device."""
    s = _stream_handle(stream)
    if buf is None:
        import torch
        n = dcp_workspace_size(capacity_tokens, h_local, cp, d, dtype)
        buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    if isinstance(buf, int):
        ptr, nbytes = buf, int(buf_bytes or 0)
    else:
        ptr, nbytes = _dev_ptr(buf, "buf"), buf.numel() * buf.element_size()
    h = _vp()
    _check(_lib.dcp_workspace_create(ptr, nbytes, capacity_tokens, h_local, cp, d, dtype, s, ctypes.byref(h)))
    return Workspace(h.value, capacity_tokens, h_local, cp, s, dtype, buf)


def dcp_workspace_recv(ws: Workspace):
    """The workspace's landing zone as torch views of its buffer: ``attn``
    [capacity, cp*h_local, D] in the workspace's dtype (head s*h_local + j holds
    shard s of local head j) and ``lse`` [capacity, cp*h_local] fp32 (FlashMLA
    layout: merge with DCP_LSE_BH1)."""
    import torch
    a, lp = _vp(), _vp()
    sb, sh, lsb = _i64(), _i64(), _i64()
    _check(_lib.dcp_workspace_recv(ws.handle, ctypes.byref(a), ctypes.byref(sb), ctypes.byref(sh), ctypes.byref(lp),
                                   ctypes.byref(lsb)))
    if not isinstance(ws.buf, torch.Tensor):
        raise ValueError("dcp_workspace_recv: the workspace was created over a raw address, not a tensor")
    base = ws.buf.data_ptr()
    H = ws.cp * ws.h_local
    dt = torch.float16 if ws.dtype == DCP_DTYPE_FP16 else torch.bfloat16
    n_attn = ws.capacity * sb.value
    attn = ws.buf[a.value - base:a.value - base + 2 * n_attn].view(dt).view(ws.capacity, H, DCP_HEAD_DIM)
    lse = ws.buf[lp.value - base:lp.value - base + 4 * ws.capacity * lsb.value].view(torch.float32)
    assert sh.value == DCP_HEAD_DIM and sb.value == H * DCP_HEAD_DIM and lsb.value == H
    return attn, lse.view(ws.capacity, H)


def dcp_workspace_destroy(ws: Workspace):
    ws.close()


def dcp_workspace_set_load_policy(ws: Workspace, policy: int):
    """DCP_LOAD_STREAMING (non-temporal loads, the default) or DCP_LOAD_CACHED
    (plain loads, for partials that are still cache-resident); the output is
    written with non-temporal stores under both."""
    _check(_lib.dcp_workspace_set_load_policy(ws.handle, policy))


def dcp_lse_combine(ws: Workspace, attn, lse, lse_layout: int, lse_mode: int, out, out_lse=None, stream=None):
    """Merge the cp shard partials of ``attn`` [B, H, D] (the workspace's bf16 or fp16, any token/head strides)
    into ``out`` [B, H/cp, D] and optionally ``out_lse`` [B, H/cp].

    ``lse`` is [B, H/cp, cp] for ``DCP_LSE_BHC`` or [B, H, 1] / [B, H] for
    ``DCP_LSE_BH1``; strides are taken from the tensors.  ``stream`` defaults
    to torch's current stream."""
    import torch
    if attn.dim() != 3 or out.dim() != 3:
        raise ValueError("attn and out must be 3-D [B, H, D] / [B, H/cp, D]")
    want = torch.float16 if ws.dtype == DCP_DTYPE_FP16 else torch.bfloat16
    if attn.dtype != want or out.dtype != want:
        raise ValueError("attn and out must be %s (the workspace's dtype)" % want)
    if lse.dtype != torch.float32 or (out_lse is not None and out_lse.dtype != torch.float32):
        raise ValueError("lse and out_lse must be float32")
    B, H, D = attn.shape
    if out.shape[0] != B or out.shape[2] != D or (out_lse is not None and out_lse.shape[0] != B):
        raise ValueError("out / out_lse shapes do not match attn")
    if attn.stride(2) != 1 or out.stride(2) != 1:
        raise ValueError("the innermost (D) stride of attn and out must be 1")
    if out.shape[1] * ws.cp != H or (out_lse is not None and out_lse.shape[1] * ws.cp != H):
        raise ValueError("out has %d heads; expected H / cp = %d" % (out.shape[1], H // ws.cp))
    if lse_layout == DCP_LSE_BHC:
        if lse.dim() != 3 or tuple(lse.shape) != (B, H // ws.cp, ws.cp):
            raise ValueError("DCP_LSE_BHC lse must be [B, H/cp, cp] = %s" % ((B, H // ws.cp, ws.cp),))
        l0, l1, l2 = lse.stride()
    else:
        if lse.dim() not in (2, 3) or lse.shape[0] != B or lse.shape[1] != H or (lse.dim() == 3 and lse.shape[2] != 1):
            raise ValueError("DCP_LSE_BH1 lse must be [B, H, 1] or [B, H]")
        l0, l1, l2 = lse.stride(0), lse.stride(1), 0
    if out_lse is not None and out_lse.dim() != 2:
        raise ValueError("out_lse must be [B, H/cp]")
    if out_lse is not None and out_lse.stride(1) != 1:
        raise ValueError("out_lse must have unit head stride")
    s = _stream_handle(stream)
    _check(_lib.dcp_lse_combine(
        ws.handle, _dev_ptr(attn, "attn"), B, H, attn.stride(0), attn.stride(1),
        _dev_ptr(lse, "lse"), lse_layout, l0, l1, l2, lse_mode,
        _dev_ptr(out, "out"), out.stride(0), out.stride(1),
        _dev_ptr(out_lse, "out_lse"), out_lse.stride(0) if out_lse is not None else 0, s))
    return out, out_lse


def dcp_mla_partial_decode_scratch_size(B: int, hq: int, kv_tokens: int, cp: int) -> int:
    """Bytes of scratch dcp_mla_partial_decode needs for this shape (0: none)."""
    n = _sz()
    _check(_lib.dcp_mla_partial_decode_scratch_size(B, hq, kv_tokens, cp, ctypes.byref(n)))
    return n.value


def dcp_mla_partial_decode(q, kv, cp: int, softmax_scale: float, lse_mode: int, o_part, lse_part, scratch=None,
                           stream=None):
    """Per-shard MLA decode partials.  ``q`` [B, hq, 576], ``kv`` [T, 576] and
    ``o_part`` [B, cp*hq, 512] all bf16 or all fp16 (the element type passed on),
    ``lse_part`` [B, cp*hq] fp32, ``scratch`` a GPU tensor of at least
    dcp_mla_partial_decode_scratch_size() bytes (or None when 0)."""
    B, hq, T, dtype = _producer_args(q, kv, cp, o_part, lse_part)
    nbytes = 0
    if scratch is not None:
        nbytes = scratch.numel() * scratch.element_size()
    s = _stream_handle(stream)
    _check(_lib.dcp_mla_partial_decode(
        _dev_ptr(q, "q"), B, hq, q.stride(0), q.stride(1), _dev_ptr(kv, "kv") if T > 0 else None, T, kv.stride(0),
        dtype, cp, float(softmax_scale), lse_mode, _dev_ptr(o_part, "o_part"), o_part.stride(0), o_part.stride(1),
        _dev_ptr(lse_part, "lse_part"), lse_part.stride(0), _dev_ptr(scratch, "scratch"), nbytes, s))
    return o_part, lse_part


def _producer_args(q, kv, cp, o_part, lse_part):
    """Shape and dtype checks shared by the fixed-length producer entry points;
    returns (B, hq, T, dtype code)."""
    import torch
    if q.dim() != 3 or kv.dim() != 2 or o_part.dim() != 3 or lse_part.dim() != 2:
        raise ValueError("q [B,hq,576], kv [T,576], o_part [B,cp*hq,512], lse_part [B,cp*hq] expected")
    if q.dtype not in (torch.bfloat16, torch.float16) or kv.dtype != q.dtype or o_part.dtype != q.dtype:
        raise ValueError("q, kv and o_part must all be bfloat16 or all float16")
    if lse_part.dtype != torch.float32:
        raise ValueError("lse_part must be float32")
    B, hq, dqk = q.shape
    if dqk != DCP_QK_DIM or kv.shape[1] != DCP_QK_DIM:
        raise ValueError("q and kv rows must have %d columns" % DCP_QK_DIM)
    if tuple(o_part.shape) != (B, cp * hq, DCP_HEAD_DIM) or tuple(lse_part.shape) != (B, cp * hq):
        raise ValueError("o_part must be [B, cp*hq, %d] and lse_part [B, cp*hq]" % DCP_HEAD_DIM)
    if q.stride(2) != 1 or kv.stride(1) != 1 or o_part.stride(2) != 1 or lse_part.stride(1) != 1:
        raise ValueError("innermost strides must be 1")
    return B, hq, kv.shape[0], (DCP_DTYPE_FP16 if q.dtype == torch.float16 else DCP_DTYPE_BF16)


def dcp_mla_partial_decode_noalloc(q, kv, cp: int, softmax_scale: float, lse_mode: int, o_part, lse_part,
                                   stream=None):
    """dcp_mla_partial_decode with the split partials in the library's static
    device array (no scratch argument; the C entry point allocates nothing)."""
    B, hq, T, dtype = _producer_args(q, kv, cp, o_part, lse_part)
    s = _stream_handle(stream)
    _check(_lib.dcp_mla_partial_decode_noalloc(
        _dev_ptr(q, "q"), B, hq, q.stride(0), q.stride(1), _dev_ptr(kv, "kv") if T > 0 else None, T, kv.stride(0),
        dtype, cp, float(softmax_scale), lse_mode, _dev_ptr(o_part, "o_part"), o_part.stride(0), o_part.stride(1),
        _dev_ptr(lse_part, "lse_part"), lse_part.stride(0), s))
    return o_part, lse_part


def dcp_mla_decode_merged_scratch_size(B: int, hq: int, kv_tokens: int, cp: int) -> int:
    """Bytes of zero-filled scratch dcp_mla_decode_merged needs for this shape."""
    n = _sz()
    _check(_lib.dcp_mla_decode_merged_scratch_size(B, hq, kv_tokens, cp, ctypes.byref(n)))
    return n.value


def dcp_mla_decode_merged(q, kv, cp: int, softmax_scale: float, lse_mode: int, o_part, lse_part, out, out_lse=None,
                          fuse: int = DCP_FUSE_AUTO, scratch=None, stream=None):
    """The producer's per-shard partials and their LSE merge in one call.  ``out`` [B, hq, 512] in the
    element type of q, ``out_lse`` [B, hq] fp32 or None; ``fuse`` DCP_FUSE_NONE / _EPILOGUE / _REDUCTIONS / _AUTO.
    ``scratch``: a GPU tensor of dcp_mla_decode_merged_scratch_size() bytes that was zero-filled before its
    first use (every call leaves its counters at zero); None allocates a zeroed one for this call."""
    import torch
    B, hq, T, dtype = _producer_args(q, kv, cp, o_part, lse_part)
    if out.dim() != 3 or tuple(out.shape) != (B, hq, DCP_HEAD_DIM) or out.dtype != q.dtype or out.stride(2) != 1:
        raise ValueError("out must be [B, hq, %d] of q's dtype with unit innermost stride" % DCP_HEAD_DIM)
    if out_lse is not None and (tuple(out_lse.shape) != (B, hq) or out_lse.dtype != torch.float32
                                or out_lse.stride(1) != 1):
        raise ValueError("out_lse must be [B, hq] float32 with unit head stride")
    if scratch is None:
        n = dcp_mla_decode_merged_scratch_size(B, hq, T, cp)
        scratch = torch.zeros(max(n, 16), dtype=torch.uint8, device=q.device)
    nbytes = scratch.numel() * scratch.element_size()
    s = _stream_handle(stream)
    _check(_lib.dcp_mla_decode_merged(
        _dev_ptr(q, "q"), B, hq, q.stride(0), q.stride(1), _dev_ptr(kv, "kv") if T > 0 else None, T, kv.stride(0),
        dtype, cp, float(softmax_scale), lse_mode, _dev_ptr(o_part, "o_part"), o_part.stride(0), o_part.stride(1),
        _dev_ptr(lse_part, "lse_part"), lse_part.stride(0), _dev_ptr(out, "out"), out.stride(0), out.stride(1),
        _dev_ptr(out_lse, "out_lse"), out_lse.stride(0) if out_lse is not None else 0, fuse,
        _dev_ptr(scratch, "scratch"), nbytes, s))
    return out, out_lse


def dcp_mla_partial_decode_varlen_scratch_size(B: int, hq: int, max_seq_len: int, cp: int) -> int:
    """Bytes of scratch dcp_mla_partial_decode_varlen needs for this shape (0 only when B == 0)."""
    n = _sz()
    _check(_lib.dcp_mla_partial_decode_varlen_scratch_size(B, hq, max_seq_len, cp, ctypes.byref(n)))
    return n.value


def dcp_mla_partial_decode_varlen(q, kv, seq_lens, max_seq_len: int, kv_layout: int, cp: int, softmax_scale: float,
                                  lse_mode: int, o_part, lse_part, scratch=None, stream=None):
    """Per-token-length MLA decode partials.  ``q`` [B, hq, 576]; ``kv`` [B, Tmax, 576]
    (token b's cache) or [Tmax, 576] (one cache shared by every token, kv_sb = 0);
    ``seq_lens`` int32 [B] on the GPU; ``kv_layout`` DCP_KV_CONTIGUOUS or
    DCP_KV_INTERLEAVED.  q, kv and o_part all bf16 or all fp16."""
    import torch
    if q.dim() != 3 or kv.dim() not in (2, 3) or o_part.dim() != 3 or lse_part.dim() != 2:
        raise ValueError("q [B,hq,576], kv [B,T,576] or [T,576], o_part [B,cp*hq,512], lse_part [B,cp*hq] expected")
    if q.dtype not in (torch.bfloat16, torch.float16) or kv.dtype != q.dtype or o_part.dtype != q.dtype:
        raise ValueError("q, kv and o_part must all be bfloat16 or all float16")
    if lse_part.dtype != torch.float32 or seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("lse_part must be float32 and seq_lens a 1-D int32 tensor")
    dtype = DCP_DTYPE_FP16 if q.dtype == torch.float16 else DCP_DTYPE_BF16
    B, hq, dqk = q.shape
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens must have B = %d entries" % B)
    if kv.dim() == 3:
        if kv.shape[0] != B:
            raise ValueError("kv [B, T, 576] must have B = %d caches" % B)
        kv_sb, T = kv.stride(0), kv.shape[1]
    else:
        kv_sb, T = 0, kv.shape[0]
    if max_seq_len > T:
        raise ValueError("max_seq_len = %d exceeds the %d cache rows" % (max_seq_len, T))
    if dqk != DCP_QK_DIM or kv.shape[-1] != DCP_QK_DIM:
        raise ValueError("q and kv rows must have %d columns" % DCP_QK_DIM)
    if tuple(o_part.shape) != (B, cp * hq, DCP_HEAD_DIM) or tuple(lse_part.shape) != (B, cp * hq):
        raise ValueError("o_part must be [B, cp*hq, %d] and lse_part [B, cp*hq]" % DCP_HEAD_DIM)
    if q.stride(2) != 1 or kv.stride(-1) != 1 or o_part.stride(2) != 1 or lse_part.stride(1) != 1:
        raise ValueError("innermost strides must be 1")
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    s = _stream_handle(stream)
    _check(_lib.dcp_mla_partial_decode_varlen(
        _dev_ptr(q, "q"), B, hq, q.stride(0), q.stride(1), _dev_ptr(kv, "kv") if max_seq_len > 0 else None, kv_sb,
        kv.stride(-2), max_seq_len, _dev_ptr(seq_lens, "seq_lens"), kv_layout, dtype, cp, float(softmax_scale),
        lse_mode, _dev_ptr(o_part, "o_part"), o_part.stride(0), o_part.stride(1), _dev_ptr(lse_part, "lse_part"),
        lse_part.stride(0), _dev_ptr(scratch, "scratch"), nbytes, s))
    return o_part, lse_part
