"""CPU oracle for CSA / HCA -- TEST INFRASTRUCTURE ONLY.

A plain, single-threaded fp64 implementation of every step of the attention
hot path (compression, RMSNorm, lightning-indexer scores, causal top-k, sparse
and dense multi-query attention, MXFP4 quantisation).  The arithmetic lives in
``oracle.c`` (plain C, doubles); this module builds it with gcc and marshals
numpy arrays.  Only the test-suite, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it; the GPU library never does, and
the two share no source.

Each wrapper names the web-page passage its C function follows; see the header
of ``oracle.c`` for the list of pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_U8 = ctypes.POINTER(ctypes.c_uint8)


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (strict IEEE: no fast-math) into liboracle.so."""
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _get():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
        lib.oracle_compress.argtypes = [_D, _D, _D, _D, _D, _D, L, L, I, I, I, L, L, _D]
        lib.oracle_compress.restype = I
        lib.oracle_rmsnorm.argtypes = [_D, L, I, _D, D, _D]
        lib.oracle_rmsnorm.restype = None
        lib.oracle_visible.argtypes = [L, L, I]
        lib.oracle_visible.restype = L
        lib.oracle_index_scores.argtypes = [_D, _D, _D, I, I, L, _D]
        lib.oracle_index_scores.restype = None
        lib.oracle_topk.argtypes = [_D, L, I, _I32]
        lib.oracle_topk.restype = None
        lib.oracle_sparse_mqa.argtypes = [_D, _D, L, _I32, I, _D, L, L, L, I, I, I, D, D, _D, _D, _D, _D]
        lib.oracle_sparse_mqa.restype = I
        lib.oracle_dense_mqa.argtypes = [_D, _D, L, I, _D, L, L, L, I, I, I, D, D, _D, _D, _D, _D]
        lib.oracle_dense_mqa.restype = I
        lib.oracle_mxfp4_quantize.argtypes = [_D, L, _U8, _U8]
        lib.oracle_mxfp4_quantize.restype = None
        lib.oracle_mxfp4_dequantize.argtypes = [_U8, _U8, L, _D]
        lib.oracle_mxfp4_dequantize.restype = None
        lib.oracle_fp8_quantize.argtypes = [_D, L, _U8]
        lib.oracle_fp8_quantize.restype = None
        lib.oracle_fp8_dequantize.argtypes = [_U8, L, _D]
        lib.oracle_fp8_dequantize.restype = None
        lib.oracle_rope_conjugate.argtypes = [_D, I, I, _D]
        lib.oracle_rope_conjugate.restype = None
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a, t=_D):
    return None if a is None else a.ctypes.data_as(t)


def compress(A, Bv, za, zb, m, bias_a=None, bias_b=None, tok_base=0, entry_begin=0, entry_end=None):
    """Overlapping two-stream softmax pooling ("DeepSeek v4" summary page, section
    "Compressed Sparse Attention", compressed KV entries; anthology record
    ARXIV-2606.19348, Key takeaways).  A, Bv: [rows, c]; za, zb: [rows] or [rows, c].
    Returns [entry_end - entry_begin, c] float64."""
    A, Bv = _f64(A), _f64(Bv)
    rows, c = A.shape
    za, zb = _f64(za).reshape(rows, -1), _f64(zb).reshape(rows, -1)
    zc = za.shape[1]
    if entry_end is None:
        entry_end = (tok_base + rows) // m
    ba = None if bias_a is None else _f64(bias_a).reshape(m, zc)
    bb = None if bias_b is None else _f64(bias_b).reshape(m, zc)
    out = np.zeros((entry_end - entry_begin, c), dtype=np.float64)
    rc = _get().oracle_compress(_p(A), _p(Bv), _p(za), _p(zb), _p(ba), _p(bb), tok_base, rows, c, m, zc,
                                entry_begin, entry_end, _p(out))
    if rc != 0:
        raise ValueError("oracle_compress: rows do not cover the requested entries")
    return out


def rmsnorm(x, eps, gamma=None):
    """RMSNorm (anthology record, Key takeaways; techniques map, "QK normalization")."""
    x = _f64(x)
    d = x.shape[-1]
    out = np.empty_like(x)
    g = None if gamma is None else _f64(gamma)
    _get().oracle_rmsnorm(_p(x), x.size // d, d, _p(g), float(eps), _p(out))
    return out


def visible(t, n_entries, m):
    """V(t) = min(N, floor((t+1)/m)): complete, preceding blocks only."""
    return int(_get().oracle_visible(int(t), int(n_entries), int(m)))


def index_scores(q, w, K):
    """Lightning-indexer score sum_h w_h * ReLU(q_h . K_s) ("DeepSeek v4" summary,
    lightning indexer).  q [H_I, d_I], w [H_I], K [n, d_I] -> [n] float64."""
    q, w, K = _f64(q), _f64(w), _f64(K)
    H, dI = q.shape
    n = K.shape[0]
    out = np.empty(n, dtype=np.float64)
    _get().oracle_index_scores(_p(q), _p(w), _p(K), H, dI, n, _p(out))
    return out


def topk(scores, n_visible, k):
    """Top-k by (score desc, index asc) over the first n_visible scores, -1 padded."""
    s = _f64(scores)
    out = np.empty(k, dtype=np.int32)
    _get().oracle_topk(_p(s), int(n_visible), int(k), _p(out, _I32))
    return out


def index_topk_rescored(q4, w, k4, q16, k16, n_visible, cand, k):
    """MXFP4 prefilter + bf16 rescoring, a labelled variant of the FP4 QK selector
    (forum post on the DeepSeek V4 paper; techniques map, "FP4 precision for the
    attention indexer"; the pages give no rescoring step).  Over the first n_visible
    entries: the `cand` best by the indexer score of the dequantised MXFP4 values
    (q4 [H_I, d_I], k4 [n, d_I]); those candidates rescored with the bf16 values
    (q16, k16); the k best rescored candidates, score descending then entry index
    ascending.  Returns (idx [k] ascending, -1 padded; candidates ascending; their
    rescored scores)."""
    V = int(n_visible)
    s4 = index_scores(q4, w, np.asarray(k4)[:V]) if V > 0 else np.zeros(0)
    c = np.sort(topk(s4, V, cand))
    c = c[c >= 0]
    s16 = index_scores(q16, w, np.asarray(k16)[c]) if len(c) else np.zeros(0)
    p = topk(s16, len(c), k)          # positions in c: a lower position is a lower entry
    sel = np.sort(c[p[p >= 0]])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(sel)] = sel
    return out, c, s16


def sparse_mqa(q, kv, idx, kv_raw, raw_base, t, window, scale, eps, gamma=None, sink=None):
    """MQA of one query over kv[idx] (-1 skipped) plus the sliding window, one softmax
    (with the per-head sink logits in its denominator when sink [H] is given).
    q [H, d]; kv [N, d]; kv_raw [W, d].  Returns (out [H, d], lse [H])."""
    q, kv, kv_raw = _f64(q), _f64(kv), _f64(kv_raw)
    H, d = q.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    g = None if gamma is None else _f64(gamma)
    sk = None if sink is None else _f64(sink)
    rc = _get().oracle_sparse_mqa(_p(q), _p(kv), kv.shape[0], _p(idx, _I32), idx.size, _p(kv_raw),
                                  kv_raw.shape[0], int(raw_base), int(t), int(window), H, d, float(scale),
                                  float(eps), _p(g), _p(sk), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_sparse_mqa: index or window row out of range")
    return out, lse


def dense_mqa(q, kv, n_entries, m, kv_raw, raw_base, t, window, scale, eps, gamma=None, sink=None):
    """HCA: MQA over every visible compressed entry plus the window, one softmax
    (with the per-head sink logits in its denominator when sink [H] is given)."""
    q, kv, kv_raw = _f64(q), _f64(kv), _f64(kv_raw)
    H, d = q.shape
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    g = None if gamma is None else _f64(gamma)
    sk = None if sink is None else _f64(sink)
    rc = _get().oracle_dense_mqa(_p(q), _p(kv), int(n_entries), int(m), _p(kv_raw), kv_raw.shape[0],
                                 int(raw_base), int(t), int(window), H, d, float(scale), float(eps),
                                 _p(g), _p(sk), _p(out), _p(lse))
    if rc != 0:
        raise ValueError("oracle_dense_mqa: window row out of range")
    return out, lse


def mxfp4_quantize(x):
    """OCP MX v1.0 MXFP4 along the last axis (multiple of 32).
    Returns (codes uint8 [..., n/2], scales uint8 [..., n/32])."""
    x = _f64(x)
    n = x.shape[-1]
    assert n % 32 == 0
    nb = x.size // 32
    codes = np.empty(x.shape[:-1] + (n // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (n // 32,), dtype=np.uint8)
    _get().oracle_mxfp4_quantize(_p(x), nb, _p(codes, _U8), _p(scales, _U8))
    return codes, scales


def mxfp4_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    nb = scales.size
    out = np.empty(scales.shape[:-1] + (scales.shape[-1] * 32,), dtype=np.float64)
    _get().oracle_mxfp4_dequantize(_p(codes, _U8), _p(scales, _U8), nb, _p(out))
    return out


def csa_decode_query(q, kv, n_entries, m, qI, w, kI, k, kv_raw, raw_base, t, window, scale, eps,
                     gamma=None):
    """One CSA decode query end to end: visible set -> indexer scores -> top-k ->
    sparse MQA.  Returns dict(scores, idx, out, lse)."""
    V = visible(t, n_entries, m)
    scores = index_scores(qI, w, np.asarray(kI)[:V]) if V > 0 else np.zeros(0)
    idx = topk(scores, V, k)
    out, lse = sparse_mqa(q, kv, idx, kv_raw, raw_base, t, window, scale, eps, gamma)
    return {"scores": scores, "idx": idx, "out": out, "lse": lse, "visible": V}


def fp8_quantize(x):
    """FP8 E4M3 codes (uint8, same shape) of x: clamp to +-448, nearest finite value,
    ties to the even code, sign kept (OCP 8-bit floating point; techniques map,
    "FP8 KV-cache quantization")."""
    x = _f64(x)
    codes = np.empty(x.shape, dtype=np.uint8)
    _get().oracle_fp8_quantize(_p(x), x.size, _p(codes, _U8))
    return codes


def fp8_dequantize(codes):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    x = np.empty(codes.shape, dtype=np.float64)
    _get().oracle_fp8_dequantize(_p(codes, _U8), codes.size, _p(x))
    return x


def rope_conjugate(out, cs):
    """Rope-conjugate rotation of an attention output (techniques map, "Gated attention
    output" and "Partial RoPE"): the trailing 64 dims of each head, rotated by the
    query's cos and the negated sin.  out [H, d]; cs [128] = cos[64], sin[64].
    Returns a new array."""
    y = np.array(out, dtype=np.float64, order="C")
    H, d = y.shape
    c = _f64(cs).reshape(128)
    _get().oracle_rope_conjugate(_p(y), H, d, _p(c))
    return y
