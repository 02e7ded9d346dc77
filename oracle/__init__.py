"""CPU oracle for the batch-invariant bf16 GEMM -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and shares no code with it.

Contents:

* ``gemm_f64``      fp64 reference y = x W^T over bf16 inputs, plus the
                    per-element scale a = sum_k |x_k w_k| (``oracle.c``);
* ``gemm_i64``      exact int64 result for integer-valued inputs;
* ``grouped_f64``   the MoE expert-grouped variant;
* ``fold_f32``      the in-order fp32 combine of split partial sums;
* ``moe_topk``, ``moe_permute``, ``swiglu_f64``, ``moe_combine_f64``
                    the MoE layer's steps around the grouped GEMM: routing,
                    grouping by expert, SwiGLU and the weighted combine;
* ``rmsnorm_f64``   RMSNorm over the hidden dimension (the step before the
                    gate+up projection);
* ``decode_attn_f64`` decode attention of one query token per sequence against
                    its KV cache (grouped-query heads), by the definition;
* ``exact``         exact-rational brute force (``oracle/exact.py``).

Each function cites the passage it follows in ``oracle.c``.  Every function is
pinned by tests that do not re-use it (exact rationals, integer closed forms,
numpy's fp64 matmul, identity and one-hot special cases).  The specific fp32
bits the GPU returns are not fixed by the pages (any fixed reduction tree is a
correct answer); the oracle judges them through the accuracy bound
``|y - y_ref| <= 1e-4 * a``, and bit-level batch invariance is checked GPU
against GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source into a shared library with gcc."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def open_library(path: str):
    """Load an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    lib.oracle_gemm_f64.argtypes = [P, P, L, L, L, P, L, P, P, I]
    lib.oracle_gemm_i64.argtypes = [P, P, L, L, L, P, L, P, I]
    lib.oracle_grouped_f64.argtypes = [P, P, L, L, L, P, L, P, L, P, P, I]
    lib.oracle_fold_f32.argtypes = [P, L, L, P]
    lib.oracle_max_threads.argtypes = []
    lib.oracle_moe_topk.argtypes = [P, L, L, L, P, P]
    lib.oracle_moe_permute.argtypes = [P, L, L, L, P, P, P]
    lib.oracle_swiglu_f64.argtypes = [P, L, L, P]
    lib.oracle_moe_combine_f64.argtypes = [P, L, P, P, L, L, L, P, P]
    lib.oracle_rmsnorm_f64.argtypes = [P, P, L, L, ctypes.c_double, P, P]
    lib.oracle_decode_attn_f64.argtypes = [P, P, P, P, L, L, L, L, L, ctypes.c_double, P, P, P]
    for f in (lib.oracle_gemm_f64, lib.oracle_gemm_i64, lib.oracle_grouped_f64,
              lib.oracle_fold_f32, lib.oracle_max_threads, lib.oracle_moe_topk,
              lib.oracle_moe_permute, lib.oracle_swiglu_f64, lib.oracle_moe_combine_f64,
              lib.oracle_rmsnorm_f64, lib.oracle_decode_attn_f64):
        f.restype = ctypes.c_int
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            _lib = open_library(build())
    return _lib


def _u16(a, ndim):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16 or a.ndim != ndim:
        raise TypeError("expected a uint16 (bf16 bits) array of rank %d, got %s %s" % (ndim, a.dtype, a.shape))
    return a


def _rows(rows, m):
    if rows is None:
        return None, m
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


def max_threads(lib=None) -> int:
    """Threads an OpenMP region of the oracle uses by default."""
    return int(_load(lib).oracle_max_threads())


def gemm_f64(x_bits, w_bits, rows=None, threads: int = 0, lib=None):
    """fp64 ``y[r] = x[rows[r]] @ w.T`` and ``a[r] = |x[rows[r]]| @ |w|.T``.

    ``x_bits`` [M,K] and ``w_bits`` [N,K] are bf16 bit patterns (uint16).
    ``rows`` selects rows of x (default: all).  Returns ``(y, a)`` float64
    arrays of shape [len(rows), N].
    """
    x = _u16(x_bits, 2)
    w = _u16(w_bits, 2)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    m, k = x.shape
    n = w.shape[0]
    r, nr = _rows(rows, m)
    y = np.empty((nr, n), np.float64)
    a = np.empty((nr, n), np.float64)
    rc = _load(lib).oracle_gemm_f64(x.ctypes.data, w.ctypes.data, m, n, k,
                                 None if r is None else r.ctypes.data, nr,
                                 y.ctypes.data, a.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError("oracle_gemm_f64 rejected its arguments (%d)" % rc)
    return y, a


def gemm_i64(x_bits, w_bits, rows=None, threads: int = 0, lib=None):
    """Exact int64 ``x @ w.T`` for integer-valued bf16 inputs (|v| <= 256)."""
    x = _u16(x_bits, 2)
    w = _u16(w_bits, 2)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    m, k = x.shape
    n = w.shape[0]
    r, nr = _rows(rows, m)
    y = np.empty((nr, n), np.int64)
    rc = _load(lib).oracle_gemm_i64(x.ctypes.data, w.ctypes.data, m, n, k,
                                 None if r is None else r.ctypes.data, nr,
                                 y.ctypes.data, int(threads))
    if rc == -2:
        raise ValueError("gemm_i64 needs integer-valued inputs with |v| <= 256")
    if rc != 0:
        raise ValueError("oracle_gemm_i64 rejected its arguments (%d)" % rc)
    return y


def grouped_f64(x_bits, w_bits, offsets, rows=None, threads: int = 0, lib=None):
    """Expert-grouped GEMM: row i of x uses expert e with offsets[e] <= i < offsets[e+1].

    ``w_bits`` is [E,N,K]; ``offsets`` is [E+1] int32, 0 .. R, nondecreasing.
    Returns ``(y, a)`` of shape [len(rows), N].
    """
    x = _u16(x_bits, 2)
    w = _u16(w_bits, 3)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    e, n, k = w.shape
    if x.shape[1] != k or off.shape != (e + 1,):
        raise ValueError("shape mismatch")
    rr = x.shape[0]
    r, nr = _rows(rows, rr)
    y = np.empty((nr, n), np.float64)
    a = np.empty((nr, n), np.float64)
    rc = _load(lib).oracle_grouped_f64(x.ctypes.data, w.ctypes.data, e, n, k, off.ctypes.data, rr,
                                    None if r is None else r.ctypes.data, nr,
                                    y.ctypes.data, a.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError("oracle_grouped_f64 rejected its arguments (%d)" % rc)
    return y, a


def fold_f32(parts, lib=None):
    """In-order fp32 fold ``((p[0] + p[1]) + p[2]) + ...`` over axis 0."""
    p = np.ascontiguousarray(parts, dtype=np.float32)
    s = p.shape[0]
    flat = p.reshape(s, -1)
    out = np.empty(flat.shape[1], np.float32)
    rc = _load(lib).oracle_fold_f32(flat.ctypes.data, s, flat.shape[1], out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_fold_f32 rejected its arguments (%d)" % rc)
    return out.reshape(p.shape[1:])


def moe_topk(logits, k: int, lib=None):
    """Top-k routing: ``(ids [T,k] int32, w [T,k] float64)``, best first, ties to
    the lower expert id; ``w`` is the softmax over the chosen logits."""
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    if lg.ndim != 2:
        raise ValueError("logits must be [T, E]")
    t, e = lg.shape
    ids = np.empty((t, k), np.int32)
    w = np.empty((t, k), np.float64)
    rc = _load(lib).oracle_moe_topk(lg.ctypes.data, t, e, int(k), ids.ctypes.data, w.ctypes.data)
    if rc == -3:
        raise ValueError("moe_topk needs finite logits")
    if rc != 0:
        raise ValueError("oracle_moe_topk rejected its arguments (%d)" % rc)
    return ids, w


def moe_permute(ids, experts: int, lib=None):
    """Stable grouping of the (token, slot) pairs by expert:
    ``(offsets [E+1], token_of_row [R], row_of [T,k])``, all int32."""
    a = np.ascontiguousarray(ids, dtype=np.int32)
    if a.ndim != 2:
        raise ValueError("ids must be [T, k]")
    t, k = a.shape
    off = np.empty(experts + 1, np.int32)
    tok = np.empty(t * k, np.int32)
    row_of = np.empty((t, k), np.int32)
    rc = _load(lib).oracle_moe_permute(a.ctypes.data, t, int(experts), k, off.ctypes.data,
                                    tok.ctypes.data, row_of.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_moe_permute rejected its arguments (%d)" % rc)
    return off, tok, row_of


def swiglu_f64(h, lib=None):
    """``silu(h[:, :I]) * h[:, I:]`` in fp64 for h float32 [R, 2I]."""
    hh = np.ascontiguousarray(h, dtype=np.float32)
    if hh.ndim != 2 or hh.shape[1] % 2:
        raise ValueError("h must be [R, 2I]")
    r, i2 = hh.shape
    out = np.empty((r, i2 // 2), np.float64)
    rc = _load(lib).oracle_swiglu_f64(hh.ctypes.data, r, i2 // 2, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_swiglu_f64 rejected its arguments (%d)" % rc)
    return out


def moe_combine_f64(o, w, row_of, lib=None):
    """``y[t] = sum_j w[t,j] * o[row_of[t,j]]`` in fp64 and its magnitude
    ``s[t] = sum_j |w[t,j] * o[row_of[t,j]]|``."""
    oo = np.ascontiguousarray(o, dtype=np.float32)
    ww = np.ascontiguousarray(w, dtype=np.float32)
    ro = np.ascontiguousarray(row_of, dtype=np.int32)
    if oo.ndim != 2 or ww.shape != ro.shape or ww.ndim != 2:
        raise ValueError("shape mismatch")
    r, h = oo.shape
    t, k = ww.shape
    y = np.empty((t, h), np.float64)
    s = np.empty((t, h), np.float64)
    rc = _load(lib).oracle_moe_combine_f64(oo.ctypes.data, r, ww.ctypes.data, ro.ctypes.data, t, k, h,
                                     y.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_moe_combine_f64 rejected its arguments (%d)" % rc)
    return y, s


def rmsnorm_f64(x_bits, g_bits, eps: float, lib=None):
    """``x * g / sqrt(mean(x^2) + eps)`` per row in fp64, and the rows' mean
    squares: ``(y [T,H] float64, ms [T] float64)``."""
    x = _u16(x_bits, 2)
    g = _u16(g_bits, 1)
    t, h = x.shape
    if g.shape != (h,):
        raise ValueError("gain must be [H]")
    y = np.empty((t, h), np.float64)
    ms = np.empty(t, np.float64)
    rc = _load(lib).oracle_rmsnorm_f64(x.ctypes.data, g.ctypes.data, t, h, float(eps), y.ctypes.data,
                                    ms.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_rmsnorm_f64 rejected its arguments (%d)" % rc)
    return y, ms


def decode_attn_f64(q_bits, k_bits, v_bits, seq_start, scale: float, lib=None):
    """Decode attention by the definition in fp64.  ``q_bits`` [B, Hq, D],
    ``k_bits`` and ``v_bits`` [Ntok, Hkv, D] (bf16 bits), ``seq_start``
    [B+1] int32.  Returns ``(out [B,Hq,D], mag [B,Hq,D], qk [B,Hq])``: the
    output, sum_t p_t |v_t| and the largest scale * sum |q k| over the keys."""
    q = _u16(q_bits, 3)
    k = _u16(k_bits, 3)
    v = _u16(v_bits, 3)
    st = np.ascontiguousarray(seq_start, dtype=np.int32)
    b, hq, d = q.shape
    ntok, hkv, d2 = k.shape
    if v.shape != k.shape or d2 != d or st.shape != (b + 1,):
        raise ValueError("shape mismatch")
    out = np.empty((b, hq, d), np.float64)
    mag = np.empty((b, hq, d), np.float64)
    qk = np.empty((b, hq), np.float64)
    rc = _load(lib).oracle_decode_attn_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, st.ctypes.data, b, hq,
                                        hkv, d, ntok, float(scale), out.ctypes.data, mag.ctypes.data,
                                        qk.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_decode_attn_f64 rejected its arguments (%d)" % rc)
    return out, mag, qk


def within_bound(y_gpu, y_ref, a, rel: float = 1e-4):
    """Boolean mask of ``|y_gpu - y_ref| <= rel * a``, evaluated in fp64.

    Where ``a == 0`` every product is zero and ``y_gpu`` must be exactly zero.
    """
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    return np.abs(y_gpu - y_ref) <= rel * a
