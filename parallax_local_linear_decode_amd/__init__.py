"""Python binding of libparallax (Parallax attention on MI355X / gfx950).

The functions here carry the names of the C entry points in
``include/parallax.h`` and do argument marshalling only: torch tensors become
device pointers, element strides and the current HIP stream, and non-OK
statuses become exceptions.  Every step of the computation runs in the HIP
kernels of ``libparallax.so``; there is no fallback.  If the library is not
built, every call raises.

Operation (page "Parallax: Parameterized Local Linear Attention Gives
Transformers a 'Second Eye'", section 1.3): o = o_SA - S_KV rho, softmax
attention minus the softmax-weighted key/value covariance applied to the
per-query probe rho.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libparallax.so")

PARALLAX_OK = 0
PARALLAX_ERR_INVALID_ARG = 1
PARALLAX_ERR_UNSUPPORTED = 2
PARALLAX_ERR_WORKSPACE = 3
PARALLAX_ERR_HIP = 4
PARALLAX_F32 = 0
PARALLAX_BF16 = 1
ABI_VERSION = 5
# bytes of the library-owned scratch parallax_decode_no_alloc uses per device
NO_ALLOC_SCRATCH_BYTES = 64 << 20

_i32, _i64, _u32, _f32, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float,
                               ctypes.c_void_p)


class DecodeArgs(ctypes.Structure):
    """Mirror of parallax_decode_args_t."""
    _fields_ = [
        ("struct_size", _u32), ("batch", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
        ("head_dim", _i32), ("scale", _f32),
        ("q", _vp), ("q_stride_b", _i64), ("q_stride_h", _i64),
        ("rho", _vp), ("rho_stride_b", _i64), ("rho_stride_h", _i64),
        ("out", _vp), ("out_stride_b", _i64), ("out_stride_h", _i64),
        ("kv_dtype", _i32),
        ("k", _vp), ("k_stride_0", _i64), ("k_stride_h", _i64), ("k_stride_t", _i64),
        ("v", _vp), ("v_stride_0", _i64), ("v_stride_h", _i64), ("v_stride_t", _i64),
        ("seq_lens", _vp), ("max_seq_len", _i32),
        ("block_table", _vp), ("block_size", _i32), ("max_blocks_per_seq", _i32),
        ("split_tokens", _i32),
        ("window", _i32),
    ]


class PrefillArgs(ctypes.Structure):
    """Mirror of parallax_prefill_args_t."""
    _fields_ = [
        ("struct_size", _u32), ("batch", _i32), ("seq_len", _i32), ("num_q_heads", _i32),
        ("num_kv_heads", _i32), ("head_dim", _i32), ("scale", _f32), ("causal", _i32),
        ("q", _vp), ("q_stride_b", _i64), ("q_stride_s", _i64), ("q_stride_h", _i64),
        ("rho", _vp), ("rho_stride_b", _i64), ("rho_stride_s", _i64), ("rho_stride_h", _i64),
        ("k", _vp), ("k_stride_b", _i64), ("k_stride_s", _i64), ("k_stride_h", _i64),
        ("v", _vp), ("v_stride_b", _i64), ("v_stride_s", _i64), ("v_stride_h", _i64),
        ("out", _vp), ("out_stride_b", _i64), ("out_stride_s", _i64), ("out_stride_h", _i64),
        ("window", _i32),
        ("lse", _vp), ("rmean", _vp), ("o_sa", _vp),
        ("workgroups", _i32),
    ]


class LlaArgs(ctypes.Structure):
    """Mirror of parallax_lla_args_t."""
    _fields_ = [("struct_size", _u32), ("lam", _f32), ("iterations", _i32), ("rho_out", _vp),
                ("resid", _vp)]


class ProjectionArgs(ctypes.Structure):
    """Mirror of parallax_qr_projection_args_t."""
    _fields_ = [
        ("struct_size", _u32), ("tokens", _i32), ("model_dim", _i32), ("num_q_heads", _i32),
        ("head_dim", _i32), ("out_dtype", _i32),
        ("x", _vp), ("x_stride_t", _i64), ("w_q", _vp), ("w_r", _vp), ("w_stride_n", _i64),
        ("q", _vp), ("q_stride_t", _i64), ("q_stride_h", _i64),
        ("rho", _vp), ("rho_stride_t", _i64), ("rho_stride_h", _i64),
    ]


class PrefillBackwardArgs(ctypes.Structure):
    """Mirror of parallax_prefill_backward_args_t."""
    _fields_ = [
        ("struct_size", _u32), ("batch", _i32), ("seq_len", _i32), ("num_q_heads", _i32),
        ("num_kv_heads", _i32), ("head_dim", _i32), ("scale", _f32), ("causal", _i32),
        ("window", _i32),
        ("q", _vp), ("q_stride_b", _i64), ("q_stride_s", _i64), ("q_stride_h", _i64),
        ("rho", _vp), ("rho_stride_b", _i64), ("rho_stride_s", _i64), ("rho_stride_h", _i64),
        ("k", _vp), ("k_stride_b", _i64), ("k_stride_s", _i64), ("k_stride_h", _i64),
        ("v", _vp), ("v_stride_b", _i64), ("v_stride_s", _i64), ("v_stride_h", _i64),
        ("dout", _vp), ("dout_stride_b", _i64), ("dout_stride_s", _i64), ("dout_stride_h", _i64),
        ("out", _vp), ("o_sa", _vp),
        ("out_stride_b", _i64), ("out_stride_s", _i64), ("out_stride_h", _i64),
        ("lse", _vp), ("rmean", _vp),
        ("dq", _vp), ("drho", _vp), ("dq_stride_b", _i64), ("dq_stride_s", _i64),
        ("dq_stride_h", _i64),
        ("dk", _vp), ("dv", _vp), ("dk_stride_b", _i64), ("dk_stride_s", _i64),
        ("dk_stride_h", _i64),
    ]


_lib = None


def load_library():
    """Load libparallax.so (built by ``python -m parallax_local_linear_decode_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libparallax.so is not built ({LIB_PATH}); run "
                           "`python -m parallax_local_linear_decode_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.parallax_abi_version.restype = ctypes.c_int
    lib.parallax_status_string.restype = ctypes.c_char_p
    lib.parallax_status_string.argtypes = [ctypes.c_int]
    lib.parallax_last_error.restype = ctypes.c_char_p
    lib.parallax_decode_workspace_size.restype = ctypes.c_int
    lib.parallax_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs),
                                                   ctypes.POINTER(ctypes.c_size_t)]
    lib.parallax_decode.restype = ctypes.c_int
    lib.parallax_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp, ctypes.c_size_t, _vp]
    lib.parallax_decode_no_alloc.restype = ctypes.c_int
    lib.parallax_decode_no_alloc.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
    lib.parallax_prefill.restype = ctypes.c_int
    lib.parallax_prefill.argtypes = [ctypes.POINTER(PrefillArgs), _vp]
    lib.parallax_decode_lla_workspace_size.restype = ctypes.c_int
    lib.parallax_decode_lla_workspace_size.argtypes = [
        ctypes.POINTER(DecodeArgs), ctypes.POINTER(LlaArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.parallax_decode_lla.restype = ctypes.c_int
    lib.parallax_decode_lla.argtypes = [ctypes.POINTER(DecodeArgs), ctypes.POINTER(LlaArgs), _vp,
                                        ctypes.c_size_t, _vp]
    lib.parallax_qr_projection.restype = ctypes.c_int
    lib.parallax_qr_projection.argtypes = [ctypes.POINTER(ProjectionArgs), _vp]
    lib.parallax_prefill_backward_workspace_size.restype = ctypes.c_int
    lib.parallax_prefill_backward_workspace_size.argtypes = [
        ctypes.POINTER(PrefillBackwardArgs), ctypes.POINTER(ctypes.c_size_t)]
    lib.parallax_prefill_backward.restype = ctypes.c_int
    lib.parallax_prefill_backward.argtypes = [ctypes.POINTER(PrefillBackwardArgs), _vp,
                                              ctypes.c_size_t, _vp]
    if lib.parallax_abi_version() != ABI_VERSION:
        raise RuntimeError("libparallax ABI version mismatch")
    _lib = lib
    return lib


class ParallaxError(RuntimeError):
    pass


def _raise(status: int, lib) -> None:
    msg = f"{lib.parallax_status_string(status).decode()}: {lib.parallax_last_error().decode()}"
    if status == PARALLAX_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == PARALLAX_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise ParallaxError(msg)


def parallax_abi_version() -> int:
    return load_library().parallax_abi_version()


def parallax_status_string(status: int) -> str:
    return load_library().parallax_status_string(status).decode()


def parallax_last_error() -> str:
    return load_library().parallax_last_error().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _decode_args(q, rho, k, v, out, scale, seq_lens, block_table, max_seq_len, split_tokens,
                 window=0):
    if q.dim() != 3 or rho.shape != q.shape:
        raise ValueError("q and rho must be [B, Hq, d] of the same shape")
    if q.dtype != torch.float32 or rho.dtype != torch.float32 or out.dtype != torch.float32:
        raise TypeError("q, rho and out must be float32")
    if k.dtype != v.dtype or k.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("k and v must both be float32 or both bfloat16")
    if k.dim() != 4 or v.dim() != 4:
        raise ValueError("k and v must be 4-d ([B, Hkv, L, d] or [pages, Hkv, 16, d])")
    for name, t in (("q", q), ("rho", rho), ("out", out), ("k", k), ("v", v)):
        if t.stride(-1) != 1:
            raise ValueError(f"{name}: the head-dim axis must be contiguous")
    B, Hq, d = q.shape
    paged = block_table is not None
    if max_seq_len is None:
        if paged:
            max_seq_len = block_table.shape[1] * k.shape[2]
        else:
            max_seq_len = k.shape[2]
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    a.batch, a.num_q_heads, a.num_kv_heads, a.head_dim = B, Hq, k.shape[1], d
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d))
    a.q, a.q_stride_b, a.q_stride_h = _ptr(q), q.stride(0), q.stride(1)
    a.rho, a.rho_stride_b, a.rho_stride_h = _ptr(rho), rho.stride(0), rho.stride(1)
    a.out, a.out_stride_b, a.out_stride_h = _ptr(out), out.stride(0), out.stride(1)
    a.kv_dtype = PARALLAX_BF16 if k.dtype == torch.bfloat16 else PARALLAX_F32
    a.k, a.k_stride_0, a.k_stride_h, a.k_stride_t = _ptr(k), k.stride(0), k.stride(1), k.stride(2)
    a.v, a.v_stride_0, a.v_stride_h, a.v_stride_t = _ptr(v), v.stride(0), v.stride(1), v.stride(2)
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,) or not seq_lens.is_contiguous():
            raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    a.seq_lens = _ptr(seq_lens)
    a.max_seq_len = int(max_seq_len)
    if paged:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                block_table.shape[0] != B or not block_table.is_contiguous():
            raise ValueError("block_table must be a contiguous int32 [B, max_blocks] tensor")
        a.block_table = _ptr(block_table)
        a.block_size = k.shape[2]
        a.max_blocks_per_seq = block_table.shape[1]
    a.split_tokens = int(split_tokens)
    a.window = int(window)
    return a


_workspaces: dict = {}


def _workspace(device, stream, nbytes):
    """A workspace per (device, stream), grown on demand and reused across
    calls (its contents need no initialisation).  Not under graph capture:
    growing it would synchronise, and graphs captured on one stream would
    share it, so a captured call must bring its own workspace."""
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("under HIP graph capture, pass workspace= (a buffer the graph owns) "
                           "or use parallax_decode_no_alloc")
    key = (str(device), stream.value)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            # the old buffer goes back to torch's allocator, which only orders
            # its reuse after torch's own stream: let work queued on `stream`
            # finish with it first (growth happens a few times per process)
            torch.cuda.synchronize(device)
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def parallax_decode_workspace_size(q, rho, k, v, *, scale=None, seq_lens=None, block_table=None,
                                   max_seq_len=None, split_tokens=0, window=0) -> int:
    """Bytes of workspace parallax_decode needs for these tensors."""
    lib = load_library()
    # The size depends on shapes only; q stands in for the output tensor.
    a = _decode_args(q, rho, k, v, q, scale, seq_lens, block_table, max_seq_len, split_tokens,
                     window)
    nbytes = ctypes.c_size_t(0)
    st = lib.parallax_decode_workspace_size(ctypes.byref(a), ctypes.byref(nbytes))
    if st != PARALLAX_OK:
        _raise(st, lib)
    return nbytes.value


def parallax_decode(q, rho, k, v, *, scale=None, seq_lens=None, block_table=None,
                    max_seq_len=None, out=None, workspace=None, split_tokens=0, window=0,
                    stream=None):
    """Parallax decode over a contiguous ([B, Hkv, L, d]) or paged
    ([pages, Hkv, 16, d] + block_table [B, max_blocks]) KV cache.

    q, rho: float32 [B, Hq, d]; k, v: bfloat16 or float32; seq_lens int32 [B]
    (required when paged).  window: 0 for every cached token, W >= 1 for each
    row's last W tokens.  Returns out float32 [B, Hq, d].  `workspace`, if
    given, is a uint8 device tensor of at least
    parallax_decode_workspace_size(...) bytes (any contents).
    """
    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    a = _decode_args(q, rho, k, v, out, scale, seq_lens, block_table, max_seq_len, split_tokens,
                     window)
    nbytes = ctypes.c_size_t(0)
    st = lib.parallax_decode_workspace_size(ctypes.byref(a), ctypes.byref(nbytes))
    if st != PARALLAX_OK:
        _raise(st, lib)
    s = _stream_handle(q, stream)
    if workspace is None and nbytes.value > 0:
        workspace = _workspace(q.device, s, nbytes.value)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.parallax_decode(ctypes.byref(a), ws_ptr, ws_bytes, s)
    if st != PARALLAX_OK:
        _raise(st, lib)
    return out


def parallax_decode_no_alloc(q, rho, k, v, out, *, scale=None, seq_lens=None, block_table=None,
                             max_seq_len=None, split_tokens=0, window=0, stream=None):
    """parallax_decode without a workspace: the split partials live in the
    library's per-device scratch (NO_ALLOC_SCRATCH_BYTES), so neither this
    call nor the library allocates; `out` (float32 [B, Hq, d]) must be given.
    Calls that may overlap on one device race on that scratch.  Same
    arguments as parallax_decode otherwise; returns out."""
    lib = load_library()
    a = _decode_args(q, rho, k, v, out, scale, seq_lens, block_table, max_seq_len, split_tokens,
                     window)
    st = lib.parallax_decode_no_alloc(ctypes.byref(a), _stream_handle(q, stream))
    if st != PARALLAX_OK:
        _raise(st, lib)
    return out


def parallax_decode_lla(q, k, v, *, lam, iterations, scale=None, seq_lens=None,
                        block_table=None, max_seq_len=None, out=None, rho_out=None, resid=None,
                        workspace=None, split_tokens=0, window=0, stream=None):
    """Decode with local linear attention's solved probe
    rho* = (S_KK + lam I)^{-1} (kbar - q), by `iterations` conjugate-gradient
    steps, each one decode sweep with the keys as values.  Cache arguments as
    parallax_decode.  Returns (out, rho_out, resid): out float32 [B, Hq, d]
    (the Parallax output with rho*), rho_out float32 [B, Hq, d], resid float32
    [B, Hq] (|residual| / |kbar - q| after the last step)."""
    lib = load_library()
    B, Hq, d = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if rho_out is None:
        rho_out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if resid is None:
        resid = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if not (rho_out.is_contiguous() and resid.is_contiguous()):
        raise ValueError("rho_out and resid must be contiguous")
    a = _decode_args(q, q, k, v, out, scale, seq_lens, block_table, max_seq_len, split_tokens,
                     window)
    a.rho = None
    la = LlaArgs()
    la.struct_size = ctypes.sizeof(LlaArgs)
    la.lam, la.iterations = float(lam), int(iterations)
    la.rho_out, la.resid = _ptr(rho_out), _ptr(resid)
    nbytes = ctypes.c_size_t(0)
    st = lib.parallax_decode_lla_workspace_size(ctypes.byref(a), ctypes.byref(la),
                                                ctypes.byref(nbytes))
    if st != PARALLAX_OK:
        _raise(st, lib)
    s = _stream_handle(q, stream)
    if workspace is None:
        workspace = _workspace(q.device, s, nbytes.value)
    st = lib.parallax_decode_lla(ctypes.byref(a), ctypes.byref(la), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), s)
    if st != PARALLAX_OK:
        _raise(st, lib)
    return out, rho_out, resid


def parallax_qr_projection(x, w_q, w_r, *, num_q_heads, out_dtype=torch.float32, q=None,
                           rho=None, stream=None):
    """q = W_Q x and rho = W_R x for every token row, in one launch.

    x bf16 [T, D]; w_q, w_r bf16 [Hq * d, D].  Returns (q, rho) of out_dtype
    (float32 for parallax_decode, bfloat16 for parallax_prefill), each
    [T, Hq, d] -- or written into the given tensors (any strides with a
    contiguous head dim)."""
    lib = load_library()
    for name, t in (("x", x), ("w_q", w_q), ("w_r", w_r)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a 2-d bfloat16 tensor with contiguous rows")
    if w_q.shape != w_r.shape or w_q.stride() != w_r.stride() or w_q.shape[1] != x.shape[1]:
        raise ValueError("w_q and w_r must be [Hq * d, D] with the same strides")
    T, D = x.shape
    N = w_q.shape[0]
    if N % num_q_heads:
        raise ValueError("w_q rows must be num_q_heads * head_dim")
    d = N // num_q_heads
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    q = torch.empty((T, num_q_heads, d), dtype=out_dtype, device=x.device) if q is None else q
    rho = torch.empty_like(q) if rho is None else rho
    for name, t in (("q", q), ("rho", rho)):
        if t.dtype != out_dtype or tuple(t.shape) != (T, num_q_heads, d) or t.stride(-1) != 1:
            raise ValueError(f"{name} must be {out_dtype} [T, Hq, d] with a contiguous head dim")
    a = ProjectionArgs()
    a.struct_size = ctypes.sizeof(ProjectionArgs)
    a.tokens, a.model_dim, a.num_q_heads, a.head_dim = T, D, num_q_heads, d
    a.out_dtype = PARALLAX_F32 if out_dtype == torch.float32 else PARALLAX_BF16
    a.x, a.x_stride_t = _ptr(x), x.stride(0)
    a.w_q, a.w_r, a.w_stride_n = _ptr(w_q), _ptr(w_r), w_q.stride(0)
    a.q, a.q_stride_t, a.q_stride_h = _ptr(q), q.stride(0), q.stride(1)
    a.rho, a.rho_stride_t, a.rho_stride_h = _ptr(rho), rho.stride(0), rho.stride(1)
    st = lib.parallax_qr_projection(ctypes.byref(a), _stream_handle(x, stream))
    if st != PARALLAX_OK:
        _raise(st, lib)
    return q, rho


def parallax_prefill(q, rho, k, v, *, scale=None, out=None, causal=True, window=0,
                     stream=None, return_stats=False, workgroups=0):
    """Causal Parallax prefill.  q, rho bf16 [B, S, Hq, d]; k, v bf16
    [B, S, Hkv, d].  window: 0 for keys 0..i, W >= 1 for keys i-W+1..i.
    Returns out float32 [B, S, Hq, d]; with return_stats, (out, lse, rmean,
    o_sa): what parallax_prefill_backward needs (lse, rmean float32
    [B, Hq, S]; o_sa float32 like out).  workgroups: head dim 128's
    persistent workgroups, 0 for one per compute unit, n >= 1 for at most n."""
    lib = load_library()
    for name, t in (("q", q), ("rho", rho), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a 4-d bfloat16 tensor with contiguous head dim")
    B, S, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, S, Hq, d), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or out.stride(-1) != 1:
        raise ValueError("out must be float32 with a contiguous head dim")
    a = PrefillArgs()
    a.struct_size = ctypes.sizeof(PrefillArgs)
    a.batch, a.seq_len, a.num_q_heads, a.num_kv_heads, a.head_dim = B, S, Hq, k.shape[2], d
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d))
    a.causal = 1 if causal else 0
    a.q, a.q_stride_b, a.q_stride_s, a.q_stride_h = _ptr(q), *q.stride()[:3]
    a.rho, a.rho_stride_b, a.rho_stride_s, a.rho_stride_h = _ptr(rho), *rho.stride()[:3]
    a.k, a.k_stride_b, a.k_stride_s, a.k_stride_h = _ptr(k), *k.stride()[:3]
    a.v, a.v_stride_b, a.v_stride_s, a.v_stride_h = _ptr(v), *v.stride()[:3]
    a.out, a.out_stride_b, a.out_stride_s, a.out_stride_h = _ptr(out), *out.stride()[:3]
    a.window = int(window)
    a.workgroups = int(workgroups)
    if return_stats:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
        rmean = torch.empty_like(lse)
        o_sa = torch.empty_like(out)
        a.lse, a.rmean, a.o_sa = _ptr(lse), _ptr(rmean), _ptr(o_sa)
    st = lib.parallax_prefill(ctypes.byref(a), _stream_handle(q, stream))
    if st != PARALLAX_OK:
        _raise(st, lib)
    return (out, lse, rmean, o_sa) if return_stats else out


def _backward_args(q, rho, k, v, dout, out, o_sa, lse, rmean, dq, drho, dk, dv, scale, causal,
                   window):
    a = PrefillBackwardArgs()
    a.struct_size = ctypes.sizeof(PrefillBackwardArgs)
    B, S, Hq, d = q.shape
    a.batch, a.seq_len, a.num_q_heads, a.num_kv_heads, a.head_dim = B, S, Hq, k.shape[2], d
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d))
    a.causal = 1 if causal else 0
    a.window = int(window)
    a.q, a.q_stride_b, a.q_stride_s, a.q_stride_h = _ptr(q), *q.stride()[:3]
    a.rho, a.rho_stride_b, a.rho_stride_s, a.rho_stride_h = _ptr(rho), *rho.stride()[:3]
    a.k, a.k_stride_b, a.k_stride_s, a.k_stride_h = _ptr(k), *k.stride()[:3]
    a.v, a.v_stride_b, a.v_stride_s, a.v_stride_h = _ptr(v), *v.stride()[:3]
    a.dout, a.dout_stride_b, a.dout_stride_s, a.dout_stride_h = _ptr(dout), *dout.stride()[:3]
    a.out, a.o_sa = _ptr(out), _ptr(o_sa)
    a.out_stride_b, a.out_stride_s, a.out_stride_h = out.stride()[:3]
    a.lse, a.rmean = _ptr(lse), _ptr(rmean)
    a.dq, a.drho = _ptr(dq), _ptr(drho)
    a.dq_stride_b, a.dq_stride_s, a.dq_stride_h = dq.stride()[:3]
    a.dk, a.dv = _ptr(dk), _ptr(dv)
    a.dk_stride_b, a.dk_stride_s, a.dk_stride_h = dk.stride()[:3]
    return a


def parallax_prefill_backward(q, rho, k, v, dout, out, o_sa, lse, rmean, *, scale=None,
                              causal=True, window=0, dq=None, drho=None, dk=None, dv=None,
                              workspace=None, stream=None):
    """Gradients of sum(dout * out) of a causal Parallax prefill.

    q, rho, k, v as parallax_prefill; dout bf16 [B, S, Hq, d]; out, o_sa,
    lse, rmean from ``parallax_prefill(..., return_stats=True)``.  Returns
    (dq, drho, dk, dv), float32, dq/drho [B, S, Hq, d] and dk/dv
    [B, S, Hkv, d] (allocated when not given; overwritten when given).
    """
    lib = load_library()
    for name, t in (("q", q), ("rho", rho), ("k", k), ("v", v), ("dout", dout)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a 4-d bfloat16 tensor with contiguous head dim")
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if o_sa.stride() != out.stride():
        raise ValueError("o_sa must share out's strides")
    for name, t, shape in (("out", out, (B, S, Hq, d)), ("o_sa", o_sa, (B, S, Hq, d)),
                           ("lse", lse, (B, Hq, S)), ("rmean", rmean, (B, Hq, S))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be float32 of shape {shape}")
    if not (lse.is_contiguous() and rmean.is_contiguous()):
        raise ValueError("lse and rmean must be contiguous")
    dq = torch.empty((B, S, Hq, d), dtype=torch.float32, device=q.device) if dq is None else dq
    drho = torch.empty_like(dq) if drho is None else drho
    dk = torch.empty((B, S, Hkv, d), dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty_like(dk) if dv is None else dv
    if drho.stride() != dq.stride() or dv.stride() != dk.stride():
        raise ValueError("drho must share dq's strides and dv dk's")
    a = _backward_args(q, rho, k, v, dout, out, o_sa, lse, rmean, dq, drho, dk, dv, scale,
                       causal, window)
    need = ctypes.c_size_t(0)
    st = lib.parallax_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(need))
    if st != PARALLAX_OK:
        _raise(st, lib)
    s = _stream_handle(q, stream)
    if workspace is None:  # the per-stream buffer: no temporary freed while the launch runs
        workspace = _workspace(q.device, s, max(int(need.value), 16))
    st = lib.parallax_prefill_backward(ctypes.byref(a), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), s)
    if st != PARALLAX_OK:
        _raise(st, lib)
    return dq, drho, dk, dv


class _PrefillFunction(torch.autograd.Function):
    """parallax_prefill forward (keeping the per-row statistics) with
    parallax_prefill_backward as its gradient, for torch autograd."""

    @staticmethod
    def forward(ctx, q, rho, k, v, scale, window):
        out, lse, rmean, o_sa = parallax_prefill(q, rho, k, v, scale=scale, window=window,
                                                 return_stats=True)
        ctx.save_for_backward(q, rho, k, v, out, o_sa, lse, rmean)
        ctx.scale, ctx.window = scale, window
        return out

    @staticmethod
    def backward(ctx, dout):
        q, rho, k, v, out, o_sa, lse, rmean = ctx.saved_tensors
        # the kernels take dout in bf16, like the other inputs
        dq, drho, dk, dv = parallax_prefill_backward(
            q, rho, k, v, dout.to(torch.bfloat16), out, o_sa, lse, rmean, scale=ctx.scale,
            window=ctx.window)
        return (dq.to(q.dtype), drho.to(rho.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None)


def parallax_prefill_attention(q, rho, k, v, *, scale=None, window=0):
    """Differentiable causal Parallax prefill: parallax_prefill in the
    forward, parallax_prefill_backward in the backward (upstream gradients
    are rounded to bf16 for it, and the input gradients come back in the
    inputs' dtype).  Same tensors and layouts as parallax_prefill."""
    return _PrefillFunction.apply(q, rho, k, v, scale, window)


__all__ = [
    "parallax_decode", "parallax_decode_workspace_size", "parallax_decode_no_alloc",
    "parallax_prefill",
    "parallax_prefill_backward", "parallax_prefill_attention", "PrefillBackwardArgs",
    "parallax_decode_lla", "LlaArgs",
    "parallax_qr_projection", "ProjectionArgs",
    "parallax_status_string", "parallax_last_error", "parallax_abi_version", "load_library",
    "DecodeArgs", "PrefillArgs", "ParallaxError",
]
