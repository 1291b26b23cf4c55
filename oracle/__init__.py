"""fp64 CPU oracle for exact (causal) softmax attention and its gradients.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library.  The arithmetic lives in ``attn_oracle.c`` (the
textbook definition, one materialised row of P at a time; see that file's
header for the equations it follows: CS336 A2 handout, section 4.2, Eq. 4-19).
This module only marshals numpy arrays to it.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB selects another build of the same source (the sanitizer build of
# oracle/build.py --sanitize, run with the sanitizer runtimes preloaded)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_long)
_L = ctypes.c_long
_D = ctypes.c_double
_I = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L, _D, _I, _I]
    lib.oracle_bwd.argtypes = [_dp] * 11 + [_L, _L, _L, _L, _D, _I, _I]
    lib.oracle_probs.argtypes = [_dp, _dp, _dp, _L, _L, _L, _D, _I]
    lib.oracle_head_stats.argtypes = [_dp] * 6 + [_L, _L, _D, _I, _I]
    lib.oracle_rows.argtypes = [_dp, _dp, _dp, _dp, _lp, _L, _dp, _dp, _dp, _L, _L, _D, _I, _I]
    lib.oracle_cols.argtypes = [_dp] * 6 + [_lp, _L, _dp, _dp, _L, _L, _D, _I, _I]
    lib.oracle_fwd_offset.argtypes = [_dp, _dp, _dp, _dp, _dp, _L, _L, _L, _L, _D, _I, _L, _I]
    lib.oracle_merge.argtypes = [_dp, _dp, _L, _dp, _dp, _L, _L]
    lib.oracle_bwd_partial.argtypes = [_dp] * 9 + [_L, _L, _L, _L, _D, _I, _L, _I]
    for f in (lib.oracle_fwd, lib.oracle_bwd, lib.oracle_probs, lib.oracle_head_stats,
              lib.oracle_rows, lib.oracle_cols, lib.oracle_fwd_offset, lib.oracle_merge,
              lib.oracle_bwd_partial):
        f.restype = None
    _lib = lib
    return lib


def _f64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a


def _ptr(a):
    return a.ctypes.data_as(_dp)


def _heads(x):
    """View [..., S, D] as [BH, S, D]."""
    x = _f64(x)
    return x.reshape(-1, x.shape[-2], x.shape[-1]), x.shape


def forward(q, k, v, scale=None, causal=True, nthreads=0):
    """O, L of softmax(scale * Q K^T) V for [..., S, D] arrays (fp64)."""
    lib = _load()
    qh, qshape = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    BH, Sq, D = qh.shape
    Sk = kh.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty_like(qh)
    lse = np.empty((BH, Sq), dtype=np.float64)
    lib.oracle_fwd(_ptr(qh), _ptr(kh), _ptr(vh), _ptr(o), _ptr(lse), BH, Sq, Sk, D,
                   float(scale), int(bool(causal)), int(nthreads))
    return o.reshape(qshape), lse.reshape(qshape[:-1])


def forward_offset(q, k, v, q_offset=0, scale=None, causal=True, nthreads=0):
    """O, L for [..., Sq, D] queries against [..., Sk, D] keys, query i placed
    q_offset positions after key 0 (causal: key j allowed iff j <= i + q_offset).
    Rows with no allowed key give O = 0, L = -inf."""
    lib = _load()
    qh, qshape = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    BH, Sq, D = qh.shape
    Sk = kh.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.empty_like(qh)
    lse = np.empty((BH, Sq), dtype=np.float64)
    lib.oracle_fwd_offset(_ptr(qh), _ptr(kh), _ptr(vh), _ptr(o), _ptr(lse), BH, Sq, Sk, D,
                          float(scale), int(bool(causal)), int(q_offset), int(nthreads))
    return o.reshape(qshape), lse.reshape(qshape[:-1])


def merge(o_parts, lse_parts):
    """Merge results over disjoint key sets: o_parts [n, ..., S, D], lse_parts [n, ..., S]."""
    lib = _load()
    op = _f64(o_parts)
    lp = _f64(lse_parts)
    n = op.shape[0]
    D = op.shape[-1]
    rows = int(np.prod(op.shape[1:-1])) if op.ndim > 2 else 1
    assert lp.shape == op.shape[:-1]
    o = np.empty(op.shape[1:])
    lse = np.empty(lp.shape[1:])
    lib.oracle_merge(_ptr(op), _ptr(lp), n, _ptr(o), _ptr(lse), rows, D)
    return o, lse


def backward_partial(q, k, v, dout, lse, delta, q_offset=0, scale=None, causal=True, nthreads=0):
    """dQ, dK, dV contributions of the keys k, v ([..., Sk, D]) for queries q ([..., Sq, D])
    placed q_offset positions after key 0, given the full attention's L and Delta ([..., Sq])."""
    lib = _load()
    qh, qshape = _heads(q)
    kh, kshape = _heads(k)
    vh, _ = _heads(v)
    doh, _ = _heads(dout)
    BH, Sq, D = qh.shape
    Sk = kh.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    lse = _f64(lse).reshape(BH, Sq)
    delta = _f64(delta).reshape(BH, Sq)
    dq = np.empty_like(qh)
    dk = np.empty_like(kh)
    dv = np.empty_like(kh)
    lib.oracle_bwd_partial(_ptr(qh), _ptr(kh), _ptr(vh), _ptr(doh), _ptr(lse), _ptr(delta),
                           _ptr(dq), _ptr(dk), _ptr(dv), BH, Sq, Sk, D, float(scale),
                           int(bool(causal)), int(q_offset), int(nthreads))
    return dq.reshape(qshape), dk.reshape(kshape), dv.reshape(kshape)


def backward(q, k, v, dout, scale=None, causal=True, nthreads=0):
    """Full materialised backward (self-attention shapes, Sq == Sk allowed to differ).

    Returns dict with dq, dk, dv, o, lse, delta_p (sum_j P dP) and delta_o (<dO, O>).
    """
    lib = _load()
    qh, qshape = _heads(q)
    kh, kshape = _heads(k)
    vh, _ = _heads(v)
    doh, _ = _heads(dout)
    BH, Sq, D = qh.shape
    Sk = kh.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.empty_like(qh)
    dk = np.empty_like(kh)
    dv = np.empty_like(kh)
    o = np.empty_like(qh)
    lse = np.empty((BH, Sq))
    dlp = np.empty((BH, Sq))
    dlo = np.empty((BH, Sq))
    lib.oracle_bwd(_ptr(qh), _ptr(kh), _ptr(vh), _ptr(doh), _ptr(dq), _ptr(dk), _ptr(dv),
                   _ptr(o), _ptr(lse), _ptr(dlp), _ptr(dlo), BH, Sq, Sk, D, float(scale),
                   int(bool(causal)), int(nthreads))
    return {
        "dq": dq.reshape(qshape), "dk": dk.reshape(kshape), "dv": dv.reshape(kshape),
        "o": o.reshape(qshape), "lse": lse.reshape(qshape[:-1]),
        "delta_p": dlp.reshape(qshape[:-1]), "delta_o": dlo.reshape(qshape[:-1]),
    }


def probs(q, k, scale=None, causal=True):
    """Materialised P [Sq, Sk] of one head (small shapes)."""
    lib = _load()
    q = _f64(q)
    k = _f64(k)
    Sq, D = q.shape
    Sk = k.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    P = np.empty((Sq, Sk))
    lib.oracle_probs(_ptr(q), _ptr(k), _ptr(P), Sq, Sk, D, float(scale), int(bool(causal)))
    return P


def head_stats(q, k, v, dout, scale=None, causal=True, nthreads=0):
    """L_i and Delta_i = <dO_i, O_i> for every row of one head [S, D]."""
    lib = _load()
    q, k, v, dout = (_f64(x) for x in (q, k, v, dout))
    S, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    lse = np.empty(S)
    delta = np.empty(S)
    lib.oracle_head_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                          S, D, float(scale), int(bool(causal)), int(nthreads))
    return lse, delta


def rows(q, k, v, dout, row_idx, scale=None, causal=True, nthreads=0):
    """O_i, L_i, dQ_i for the listed query rows of one head [S, D]."""
    lib = _load()
    q, k, v, dout = (_f64(x) for x in (q, k, v, dout))
    S, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    ridx = np.ascontiguousarray(np.asarray(row_idx, dtype=np.int64))
    assert ridx.size == 0 or (ridx.min() >= 0 and ridx.max() < S)
    n = ridx.size
    o = np.empty((n, D))
    lse = np.empty(n)
    dq = np.empty((n, D))
    lib.oracle_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), ridx.ctypes.data_as(_lp), n,
                    _ptr(o), _ptr(lse), _ptr(dq), S, D, float(scale), int(bool(causal)),
                    int(nthreads))
    return o, lse, dq


def cols(q, k, v, dout, lse, delta, col_idx, scale=None, causal=True, nthreads=0):
    """dK_j, dV_j for the listed keys of one head, given that head's full L and Delta."""
    lib = _load()
    q, k, v, dout, lse, delta = (_f64(x) for x in (q, k, v, dout, lse, delta))
    S, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    cidx = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int64))
    assert cidx.size == 0 or (cidx.min() >= 0 and cidx.max() < S)
    n = cidx.size
    dk = np.empty((n, D))
    dv = np.empty((n, D))
    lib.oracle_cols(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(delta),
                    cidx.ctypes.data_as(_lp), n, _ptr(dk), _ptr(dv), S, D, float(scale),
                    int(bool(causal)), int(nthreads))
    return dk, dv
