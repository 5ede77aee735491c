"""Plain fp64 CPU reference for Parallax attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The library path never does, and the
oracle shares no code with it.

The arithmetic lives in ``oracle.c`` (fp64, libm ``exp``); this module only
builds it with gcc, marshals numpy arrays into it and returns fp64 results.
What it computes (page "Parallax: Parameterized Local Linear Attention Gives
Transformers a 'Second Eye'", section 1.3): for each query row,
``o = o_SA - S_KV @ rho`` with ``o_SA`` the softmax attention output and
``S_KV`` the softmax-weighted, centred covariance of values against keys.

The training side (same page, section 2.2 trains the layer end to end):
``prefill_stats`` gives the per-row quantities a forward pass keeps (log of
the softmax denominator, ``r``, ``o_SA``) and ``prefill_backward`` the
gradients of ``sum(dout * out)`` with respect to q, rho, k and v, by the chain
rule through the forward steps.

Local linear attention's solved probe (same page, sections 1.2-1.3 and the
taxonomy of section 2.1): ``solved_probe`` gives, per decode row,
rho* = (S_KK + lam I)^{-1} (kbar - q) by a direct fp64 solve, and
``lla_decode`` the Parallax output with that probe, which is the intercept of
the softmax-weighted, ridge-regularised local linear fit v ~ b + W (k - q).

The probe projection (same page, section 1.3: rho = W_R x, a learned linear
map of the layer input, computed beside the query projection q = W_Q x):
``qr_projection`` gives both for a batch of token rows, as fp64 matrix
products.

Array conventions (numpy):
  * float64 / float32 arrays are read as such;
  * uint16 arrays are raw bfloat16 bit patterns (widened exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2
EXPLICIT, STREAMING = 0, 1
_FORMS = {"explicit": EXPLICIT, "streaming": STREAMING}

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c99", "-fPIC",
           "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, dbl, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.orc_decode.restype = i32
    lib.orc_decode.argtypes = [i32, i32, i32, i32, i32, i32, dbl,
                               vp, i32, vp, i32, vp, vp, i32,
                               i64, i64, i64, i64, i64, i64,
                               vp, i32, vp, i32, i32, i32, vp, i32]
    lib.orc_prefill.restype = i32
    lib.orc_prefill.argtypes = [i32, i32, i32, i32, i32, i32, i32, dbl,
                                vp, i32, vp, i32, vp, vp, i32,
                                vp, i32, i32, vp, i32]
    lib.orc_prefill_stats.restype = i32
    lib.orc_prefill_stats.argtypes = [i32, i32, i32, i32, i32, i32, dbl,
                                      vp, i32, vp, i32, vp, vp, i32,
                                      vp, i32, i32, vp, vp, vp, i32]
    lib.orc_prefill_backward.restype = i32
    lib.orc_prefill_backward.argtypes = [i32, i32, i32, i32, i32, i32, dbl,
                                         vp, i32, vp, i32, vp, vp, i32, vp, i32,
                                         vp, i32, i32, vp, vp, vp, vp, i32]
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle: unsupported array dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def decode(q, rho, k, v, scale, *, seq_lens=None, block_table=None, form="streaming",
           window=0, threads=None):
    """Decode attention rows, one per (batch, query head).

    q, rho : [B, Hq, dk]
    contiguous cache (block_table is None):
        k [B, Hkv, Lcap, dk], v [B, Hkv, Lcap, dv]; row b sees seq_lens[b]
        tokens (all Lcap when seq_lens is None)
    paged cache:
        k [NB, Hkv, P, dk], v [NB, Hkv, P, dv] (P tokens per page),
        block_table [B, max_blocks] int32 of page ids, seq_lens [B] int32
    window : 0 (every cached token) or W >= 1 (each row's last W tokens)
    Returns out [B, Hq, dv] float64.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    rho = np.ascontiguousarray(rho)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, Hq, dk = q.shape
    if rho.shape != q.shape:
        raise ValueError("rho must have q's shape")
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    Hkv = k.shape[1]
    dv = v.shape[3]
    if k.shape[3] != dk or v.shape[:3] != k.shape[:3]:
        raise ValueError("inconsistent k/v shapes")
    _, _, P, _ = k.shape
    k_str = (Hkv * P * dk, P * dk, dk)
    v_str = (Hkv * P * dv, P * dv, dv)
    if seq_lens is not None:
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if seq_lens.shape != (B,):
            raise ValueError("seq_lens must be [B]")
    if block_table is not None:
        if seq_lens is None:
            raise ValueError("paged decode needs seq_lens")
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        if block_table.ndim != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_blocks]")
        max_blocks = block_table.shape[1]
        if np.any(seq_lens > max_blocks * P):
            raise ValueError("seq_lens exceed the block table")
        L_all = 0
    else:
        max_blocks = 0
        if k.shape[0] != B:
            raise ValueError("contiguous k must be [B, Hkv, Lcap, dk]")
        if seq_lens is not None and np.any(seq_lens > P):
            raise ValueError("seq_lens exceed the cache capacity")
        L_all = P
    if seq_lens is not None and np.any(seq_lens < 0):
        raise ValueError("negative seq_lens")
    out = np.empty((B, Hq, dv), dtype=np.float64)
    rc = lib.orc_decode(_FORMS[form], B, Hq, Hkv, dk, dv, float(scale),
                        _ptr(q), _dtype_code(q), _ptr(rho), _dtype_code(rho),
                        _ptr(k), _ptr(v), _dtype_code(k),
                        *k_str, *v_str,
                        _ptr(seq_lens), L_all,
                        _ptr(block_table), P if block_table is not None else 0, max_blocks,
                        int(window), _ptr(out), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: orc_decode rejected its arguments")
    return out


def prefill(q, rho, k, v, scale, *, rows=None, form="streaming", window=0, threads=None):
    """Causal prefill rows: row i of (b, h) attends to keys 0..i (with window
    W >= 1: keys max(0, i-W+1)..i).

    q, rho : [B, S, Hq, dk];  k : [B, S, Hkv, dk];  v : [B, S, Hkv, dv]
    rows   : query positions to evaluate (default: all S)
    Returns out [B, len(rows), Hq, dv] float64.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    rho = np.ascontiguousarray(rho)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, S, Hq, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[3]
    if rho.shape != q.shape or k.shape != (B, S, Hkv, dk) or v.shape[:3] != (B, S, Hkv):
        raise ValueError("inconsistent prefill shapes")
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    if rows is None:
        rows = np.arange(S, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((B, rows.size, Hq, dv), dtype=np.float64)
    rc = lib.orc_prefill(_FORMS[form], B, S, Hq, Hkv, dk, dv, float(scale),
                         _ptr(q), _dtype_code(q), _ptr(rho), _dtype_code(rho),
                         _ptr(k), _ptr(v), _dtype_code(k),
                         _ptr(rows), int(rows.size), int(window), _ptr(out),
                         int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: orc_prefill rejected its arguments")
    return out


def _prefill_common(q, rho, k, v):
    q = np.ascontiguousarray(q)
    rho = np.ascontiguousarray(rho)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, S, Hq, dk = q.shape
    Hkv = k.shape[2]
    dv = v.shape[3]
    if rho.shape != q.shape or k.shape != (B, S, Hkv, dk) or v.shape[:3] != (B, S, Hkv):
        raise ValueError("inconsistent prefill shapes")
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    return q, rho, k, v, (B, S, Hq, Hkv, dk, dv)


def _rows(rows, S):
    if rows is None:
        rows = np.arange(S, dtype=np.int32)
    return np.ascontiguousarray(rows, dtype=np.int32)


def prefill_stats(q, rho, k, v, scale, *, rows=None, window=0, threads=None):
    """What a causal prefill forward pass keeps for its backward pass, per
    (batch, row, query head): ``lse`` = natural log of sum_j exp(scale q.k_j)
    over the row's keys, ``r`` = sum_j p_j (rho . k_j), ``a`` = o_SA.

    Shapes as ``prefill``.  Returns lse [B, R, Hq], r [B, R, Hq],
    a [B, R, Hq, dv] (float64; R = len(rows)).
    """
    lib = _load()
    q, rho, k, v, (B, S, Hq, Hkv, dk, dv) = _prefill_common(q, rho, k, v)
    rows = _rows(rows, S)
    lse = np.empty((B, rows.size, Hq), dtype=np.float64)
    r = np.empty((B, rows.size, Hq), dtype=np.float64)
    a = np.empty((B, rows.size, Hq, dv), dtype=np.float64)
    rc = lib.orc_prefill_stats(B, S, Hq, Hkv, dk, dv, float(scale),
                               _ptr(q), _dtype_code(q), _ptr(rho), _dtype_code(rho),
                               _ptr(k), _ptr(v), _dtype_code(k),
                               _ptr(rows), int(rows.size), int(window),
                               _ptr(lse), _ptr(r), _ptr(a), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: orc_prefill_stats rejected its arguments")
    return lse, r, a


def prefill_backward(q, rho, k, v, dout, scale, *, rows=None, window=0, threads=None):
    """Gradients of sum(dout * prefill(q, rho, k, v)) (causal, optional window).

    dout : [B, S, Hq, dv]
    rows : query rows whose terms are included (default all).  dq and drho are
           returned for these rows; dk and dv sum these rows' contributions
           only, so they are exact for key j when every row that sees key j
           is included.
    Returns dq [B, R, Hq, dk], drho [B, R, Hq, dk], dk [B, S, Hkv, dk],
    dv [B, S, Hkv, dv] (float64).
    """
    lib = _load()
    q, rho, k, v, (B, S, Hq, Hkv, dk, dv) = _prefill_common(q, rho, k, v)
    dout = np.ascontiguousarray(dout)
    if dout.shape != (B, S, Hq, dv):
        raise ValueError("dout must be [B, S, Hq, dv]")
    rows = _rows(rows, S)
    dq = np.empty((B, rows.size, Hq, dk), dtype=np.float64)
    drho = np.empty_like(dq)
    dkk = np.empty((B, S, Hkv, dk), dtype=np.float64)
    dvv = np.empty((B, S, Hkv, dv), dtype=np.float64)
    rc = lib.orc_prefill_backward(B, S, Hq, Hkv, dk, dv, float(scale),
                                  _ptr(q), _dtype_code(q), _ptr(rho), _dtype_code(rho),
                                  _ptr(k), _ptr(v), _dtype_code(k), _ptr(dout), _dtype_code(dout),
                                  _ptr(rows), int(rows.size), int(window),
                                  _ptr(dq), _ptr(drho), _ptr(dkk), _ptr(dvv),
                                  int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: orc_prefill_backward rejected its arguments")
    return dq, drho, dkk, dvv


def _row_keys(k, b, hk, L, block_table, window):
    """Keys [n, dk] (float64) of decode row (b, kv head hk) over its L cached
    tokens, restricted to the last `window` of them when window >= 1."""
    j0 = max(0, L - window) if window > 0 else 0
    js = np.arange(j0, L)
    if block_table is None:
        rows = k[b, hk, js]
    else:
        P = k.shape[2]
        rows = k[block_table[b, js // P], hk, js % P]
    return _as_f64(rows)


def _as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:  # raw bf16 bits
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def solved_probe(q, k, scale, lam, *, seq_lens=None, block_table=None, window=0):
    """LLA's solved probe for every decode row (b, h):
    rho* = (S_KK + lam I)^{-1} (kbar - q), where p = softmax(scale K q) over
    the row's keys, kbar = sum p_j k_j and S_KK = sum p_j (k_j - kbar)(k_j -
    kbar)^T.  A row with no keys gets rho* = 0.

    The pages state the per-token system S x = mu with a regulariser lam
    (page "Parallax: Parameterized Local Linear Attention ...", section 1.2)
    and the optimal probe rho* = S^{-1} mu (section 1.3) without defining mu;
    mu = kbar - q and S = S_KK + lam I is the reading under which the
    softmax-weighted fit v ~ b + W (k - q) with ridge penalty lam ||W||^2 has
    intercept o_SA - S_KV rho*.  Solved directly (numpy.linalg.solve) in fp64.

    q [B, Hq, dk]; k contiguous [B, Hkv, Lcap, dk] or paged [NB, Hkv, P, dk]
    with block_table [B, max_blocks]; seq_lens [B] (default: all Lcap).
    Returns rho* [B, Hq, dk] float64.
    """
    qd = _as_f64(q)
    B, Hq, dk = qd.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if seq_lens is None:
        if block_table is not None:
            raise ValueError("paged keys need seq_lens")
        seq_lens = np.full(B, k.shape[2], dtype=np.int64)
    out = np.zeros((B, Hq, dk), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        for hk in range(Hkv):
            K = _row_keys(k, b, hk, L, block_table, window)
            if K.shape[0] == 0:
                continue
            for h in range(hk * G, (hk + 1) * G):
                s = scale * (K @ qd[b, h])
                p = np.exp(s - s.max())
                p /= p.sum()
                kbar = p @ K
                Kc = K - kbar
                S_KK = (Kc * p[:, None]).T @ Kc
                out[b, h] = np.linalg.solve(S_KK + lam * np.eye(dk), kbar - qd[b, h])
    return out


def lla_decode(q, k, v, scale, lam, *, seq_lens=None, block_table=None, window=0,
               threads=None):
    """Decode with LLA's solved probe: (out, rho*), out = o_SA - S_KV rho*
    (the Parallax output with the solved probe), both float64."""
    rho = solved_probe(q, k, scale, lam, seq_lens=seq_lens, block_table=block_table,
                       window=window)
    out = decode(q, rho, k, v, scale, seq_lens=seq_lens, block_table=block_table,
                 window=window, threads=threads)
    return out, rho


def qr_projection(x, w_q, w_r):
    """q = W_Q x and rho = W_R x for every token row of x.

    x [T, D]; w_q, w_r [N, D] (N = heads * head_dim).  Returns q, rho [T, N]
    float64: plain fp64 matrix products of the exactly widened inputs.
    """
    xd, wq, wr = _as_f64(x), _as_f64(w_q), _as_f64(w_r)
    if xd.ndim != 2 or wq.shape != wr.shape or wq.shape[1] != xd.shape[1]:
        raise ValueError("x must be [T, D] and w_q, w_r [N, D]")
    return xd @ wq.T, xd @ wr.T
