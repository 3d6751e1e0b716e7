"""Thin ctypes binding of libcsa.so (declared in include/csa.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of libcsa.so.  Tensors must be CUDA (HIP) tensors on one device,
contiguous, with the dtypes documented per function; torch provides device
memory and the current stream, nothing else.  There is no CPU fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
_lib = None

F32, BF16, MXFP4, FP8 = 0, 1, 2, 3


class CsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("libcsa status %d: %s" % (status, msg))
        self.status = status


class CompressDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "channels", "m", "zc", "n_rows", "tok_base", "entry_begin", "entry_end", "out_cap",
        "in_dtype", "out_dtype", "norm")] + [("norm_eps", ctypes.c_float)]


class IndexDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q", "idx_heads", "idx_dim", "m", "topk", "n_max", "k_cap", "dtype", "q_quantize")]


class MqaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q", "heads", "head_dim", "topk", "m", "n_max", "window", "kv_cap", "raw_cap")] + [
        ("scale", ctypes.c_float), ("eps", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("split_items", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


_P = ctypes.c_void_p


class CompressJob(ctypes.Structure):
    _fields_ = [("desc", CompressDesc), ("a", _P), ("b", _P), ("za", _P), ("zb", _P), ("bias_a", _P),
                ("bias_b", _P), ("norm_weight", _P), ("out", _P)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("index", IndexDesc), ("attn", MqaDesc), ("kv_job", ctypes.POINTER(CompressJob)),
                ("key_job", ctypes.POINTER(CompressJob))] + [(n, _P) for n in (
                    "q", "kv", "kv_raw", "raw_base", "q_pos", "rms_weight", "sink", "rope", "q_idx", "q_idx_scale", "w", "k_idx",
                    "k_idx_scale", "n_entries", "out_idx", "out_score", "out", "lse")]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 40), ("launches", ctypes.c_int32), ("total_us", ctypes.c_double),
                ("min_us", ctypes.c_double), ("max_us", ctypes.c_double)]


def lib():
    """Load libcsa.so (built in-tree by build_lib / __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libcsa.so is not built (run python -m long_context_compressed_04_amd.build_lib)")
        L = ctypes.CDLL(_LIB_PATH)
        S, V, Z = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.csa_abi_version.restype = ctypes.c_int
        L.csa_status_string.restype = ctypes.c_char_p
        L.csa_status_string.argtypes = [ctypes.c_int]
        L.csa_last_error.restype = ctypes.c_char_p
        L.csa_compress.argtypes = [ctypes.POINTER(CompressDesc)] + [V] * 9
        L.csa_compress.restype = S
        L.csa_mxfp4_quantize.argtypes = [ctypes.c_int32, V, ctypes.c_int64, V, V, V]
        L.csa_mxfp4_quantize.restype = S
        L.csa_fp8_quantize.argtypes = [ctypes.c_int32, V, ctypes.c_int64, V, V]
        L.csa_fp8_quantize.restype = S
        L.csa_index_workspace_size.argtypes = [ctypes.POINTER(IndexDesc)]
        L.csa_index_workspace_size.restype = Z
        L.csa_index_scores.argtypes = [ctypes.POINTER(IndexDesc)] + [V] * 9
        L.csa_index_scores.restype = S
        L.csa_index_topk.argtypes = [ctypes.POINTER(IndexDesc)] + [V] * 9 + [V, Z, V]
        L.csa_index_topk.restype = S
        L.csa_index_rescored_workspace_size.argtypes = [ctypes.POINTER(IndexDesc), ctypes.c_int32]
        L.csa_index_rescored_workspace_size.restype = Z
        L.csa_index_topk_rescored.argtypes = [ctypes.POINTER(IndexDesc), ctypes.c_int32] + [V] * 11 + [V, Z, V]
        L.csa_index_topk_rescored.restype = S
        L.csa_mqa_workspace_size.argtypes = [ctypes.POINTER(MqaDesc), ctypes.c_int32]
        L.csa_mqa_workspace_size.restype = Z
        L.csa_sparse_mqa.argtypes = [ctypes.POINTER(MqaDesc)] + [V] * 11 + [V, Z, V]
        L.csa_sparse_mqa.restype = S
        L.hca_dense_mqa.argtypes = [ctypes.POINTER(MqaDesc)] + [V] * 11 + [V, Z, V]
        L.hca_dense_mqa.restype = S
        L.csa_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeArgs)]
        L.csa_decode_workspace_size.restype = Z
        L.csa_decode.argtypes = [ctypes.POINTER(DecodeArgs), V, Z, V]
        L.csa_decode.restype = S
        L.csa_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), V]
        L.csa_decode_noalloc.restype = S
        L.csa_timing_enable.argtypes = [ctypes.c_int32]
        L.csa_timing_enable.restype = S
        L.csa_timing_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32]
        L.csa_timing_collect.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise CsaError(status, lib().csa_last_error().decode())


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libcsa takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libcsa takes contiguous tensors")
    return t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        return MXFP4
    raise ValueError("unsupported dtype %s" % t.dtype)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() < nbytes:
        raise ValueError("workspace of %d bytes needed" % nbytes)
    return ws, ws.numel()


# ----------------------------------------------------------------------------------
def _compress_desc(a, za, m, out, tok_base, entry_begin, entry_end, norm_eps):
    B, rows, c = a.shape
    zc = 1 if za.dim() == 2 else za.shape[-1]
    if entry_end is None:
        entry_end = (tok_base + rows) // m
    norm = 0 if norm_eps is None else 1
    return CompressDesc(B, c, m, zc, rows, tok_base, entry_begin, entry_end, out.shape[1], _dtype_code(a),
                        _dtype_code(out), norm, 0.0 if norm_eps is None else float(norm_eps))


def compress(a, b, za, zb, m, out, *, tok_base=0, entry_begin=0, entry_end=None, bias_a=None, bias_b=None,
             norm_eps=None, norm_weight=None):
    """Pool token rows into compressed entries (csa_compress).  a, b: [B, rows, c]
    fp32/bf16; za, zb: [B, rows] or [B, rows, c] fp32; out: [B, cap, c] fp32/bf16,
    entry j written to row j.  norm_eps given: each entry RMS-normalised (times
    norm_weight [c] fp32, or ones) before it is stored."""
    d = _compress_desc(a, za, m, out, tok_base, entry_begin, entry_end, norm_eps)
    _check(lib().csa_compress(ctypes.byref(d), _p(a), _p(b), _p(za), _p(zb), _p(bias_a), _p(bias_b),
                              _p(norm_weight), _p(out), _stream(a)))
    return out


def compress_job(a, b, za, zb, m, out, *, tok_base=0, entry_begin=0, entry_end=None, bias_a=None, bias_b=None,
                 norm_eps=None, norm_weight=None):
    """A compression for Decoder's kv_job / key_job: the same arguments as compress(),
    run inside each decode call before the indexer."""
    d = _compress_desc(a, za, m, out, tok_base, entry_begin, entry_end, norm_eps)
    job = CompressJob(d, _p(a), _p(b), _p(za), _p(zb), _p(bias_a), _p(bias_b), _p(norm_weight), _p(out))
    job._keep = [a, b, za, zb, out, bias_a, bias_b, norm_weight]
    return job


def mxfp4_quantize(x, codes=None, scales=None):
    """MXFP4 along the last axis (multiple of 32): returns (codes uint8 [..., n/2],
    scales uint8 [..., n/32]), written into `codes` / `scales` when given."""
    n = x.shape[-1]
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (n // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (n // 32,), dtype=torch.uint8, device=x.device)
    if codes.numel() * 2 != x.numel() or scales.numel() * 32 != x.numel():
        raise ValueError("codes / scales do not match x")
    _check(lib().csa_mxfp4_quantize(_dtype_code(x), _p(x), x.numel() // 32, _p(codes), _p(scales), _stream(x)))
    return codes, scales


def fp8_quantize(x, codes=None):
    """FP8 E4M3 codes (uint8, same shape as x): clamp to +-448, nearest value, ties to
    the even code.  x float32 or bfloat16 with a multiple of 8 elements."""
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if codes.numel() != x.numel():
        raise ValueError("codes do not match x")
    _check(lib().csa_fp8_quantize(_dtype_code(x), _p(x), x.numel(), _p(codes), _stream(x)))
    return codes


def _index_dtype(q_idx, k_idx):
    """(dtype, q_quantize): MXFP4 keys with fp32 queries quantise the queries inside
    the call; otherwise q_idx and k_idx share one dtype."""
    if _dtype_code(k_idx) == MXFP4 and q_idx.dtype != torch.uint8:
        if q_idx.dtype != torch.float32:
            raise ValueError("queries quantised inside the call must be float32")
        return MXFP4, 1
    return _dtype_code(q_idx), 0


def _index_desc(q_idx, k_idx, m, topk, n_max, dtype, q_quantize=0):
    B, n_q, HI = q_idx.shape[:3]
    dI = q_idx.shape[3] * (2 if dtype == MXFP4 and not q_quantize else 1)
    k_cap = k_idx.shape[1]
    return IndexDesc(B, n_q, HI, dI, m, topk, k_cap if n_max is None else n_max, k_cap, dtype, q_quantize)


def index_scores(q_idx, w, k_idx, n_entries, q_pos, *, m, n_max=None, q_scale=None, k_scale=None):
    """Indexer score rows [B, n_q, n_max] fp32 (-inf where not visible)."""
    d = _index_desc(q_idx, k_idx, m, 1, n_max, *_index_dtype(q_idx, k_idx))
    scores = torch.empty((d.batch, d.n_q, d.n_max), dtype=torch.float32, device=q_idx.device)
    _check(lib().csa_index_scores(ctypes.byref(d), _p(q_idx), _p(q_scale), _p(w), _p(k_idx), _p(k_scale),
                                  _p(n_entries), _p(q_pos), _p(scores), _stream(q_idx)))
    return scores


def index_topk(q_idx, w, k_idx, n_entries, q_pos, *, m, topk, n_max=None, q_scale=None, k_scale=None,
               workspace=None, out_idx=None, out_score=None):
    """Indexer + causal top-k: returns (idx int32 [B, n_q, topk], score fp32 [B, n_q, topk])."""
    d = _index_desc(q_idx, k_idx, m, topk, n_max, *_index_dtype(q_idx, k_idx))
    dev = q_idx.device
    if out_idx is None:
        out_idx = torch.empty((d.batch, d.n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None:
        out_score = torch.empty((d.batch, d.n_q, topk), dtype=torch.float32, device=dev)
    ws, nb = _workspace(lib().csa_index_workspace_size(ctypes.byref(d)), dev, workspace)
    _check(lib().csa_index_topk(ctypes.byref(d), _p(q_idx), _p(q_scale), _p(w), _p(k_idx), _p(k_scale),
                                _p(n_entries), _p(q_pos), _p(out_idx), _p(out_score), _p(ws), nb, _stream(q_idx)))
    return out_idx, out_score


def index_topk_rescored(q_idx, q_scale, q_bf16, w, k_idx, k_scale, k_bf16, n_entries, q_pos, *, m, topk, cand,
                        n_max=None, workspace=None, out_idx=None, out_score=None):
    """MXFP4 prefilter of `cand` entries, bf16 rescoring, top-k of the rescored
    candidates: returns (idx int32 [B, n_q, topk], rescored score fp32 [B, n_q, topk])."""
    d = _index_desc(q_idx, k_idx, m, topk, n_max, *_index_dtype(q_idx, k_idx))
    dev = q_idx.device
    if out_idx is None:
        out_idx = torch.empty((d.batch, d.n_q, topk), dtype=torch.int32, device=dev)
    if out_score is None:
        out_score = torch.empty((d.batch, d.n_q, topk), dtype=torch.float32, device=dev)
    ws, nb = _workspace(lib().csa_index_rescored_workspace_size(ctypes.byref(d), cand), dev, workspace)
    _check(lib().csa_index_topk_rescored(ctypes.byref(d), cand, _p(q_idx), _p(q_scale), _p(q_bf16), _p(w),
                                         _p(k_idx), _p(k_scale), _p(k_bf16), _p(n_entries), _p(q_pos),
                                         _p(out_idx), _p(out_score), _p(ws), nb, _stream(q_idx)))
    return out_idx, out_score


def _mqa_desc(q, kv, kv_raw, *, topk=0, m=1, n_max=0, window=128, scale=0.0, eps=1e-6, split_items=0):
    B, n_q, H, D = q.shape
    # uint8 caches hold FP8 E4M3 rows (fp8_quantize)
    kv_dtype = FP8 if kv.dtype == torch.uint8 else 0
    if (kv_raw.dtype == torch.uint8) != (kv_dtype == FP8):
        raise ValueError("kv and kv_raw must both be FP8 (uint8) or both of q's dtype")
    return MqaDesc(B, n_q, H, D, topk, m, n_max, window, kv.shape[1], kv_raw.shape[1], float(scale), float(eps),
                   _dtype_code(q), split_items, kv_dtype)


def sparse_mqa(q, kv, idx, kv_raw, raw_base, q_pos, *, window, scale=0.0, eps=1e-6, rms_weight=None, sink=None,
               rope=None, split_items=0, workspace=None, out=None, lse=None):
    """CSA attention over idx (-1 skipped) plus the sliding window.  Returns (out, lse).
    sink: per-head sink logits [heads] fp32 or None; split_items > 0 selects
    batch-invariant splitting (see csa_mqa_desc).  kv and kv_raw as uint8: FP8 E4M3
    rows (bf16 q, no rms_weight).  rope: [B, n_q, 128] fp32 cos and sin of each query
    (rope-conjugate rotation of the output's trailing 64 dims), or None."""
    d = _mqa_desc(q, kv, kv_raw, topk=idx.shape[-1], window=window, scale=scale, eps=eps, split_items=split_items)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    ws, nb = _workspace(lib().csa_mqa_workspace_size(ctypes.byref(d), 0), q.device, workspace)
    _check(lib().csa_sparse_mqa(ctypes.byref(d), _p(q), _p(kv), _p(idx), _p(kv_raw), _p(raw_base), _p(q_pos),
                                _p(rms_weight), _p(sink), _p(rope), _p(out), _p(lse), _p(ws), nb, _stream(q)))
    return out, lse


def hca_dense_mqa(q, kv, n_entries, kv_raw, raw_base, q_pos, *, m, window, n_max=None, scale=0.0, eps=1e-6,
                  rms_weight=None, sink=None, rope=None, split_items=0, workspace=None, out=None, lse=None):
    """HCA attention over every visible compressed entry plus the window.  Returns (out, lse).
    sink: per-head sink logits [heads] fp32 or None; split_items > 0 selects
    batch-invariant splitting (see csa_mqa_desc).  kv and kv_raw as uint8: FP8 E4M3
    rows (bf16 q, no rms_weight).  rope: as sparse_mqa."""
    d = _mqa_desc(q, kv, kv_raw, m=m, n_max=kv.shape[1] if n_max is None else n_max, window=window, scale=scale,
                  eps=eps, split_items=split_items)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    ws, nb = _workspace(lib().csa_mqa_workspace_size(ctypes.byref(d), 1), q.device, workspace)
    _check(lib().hca_dense_mqa(ctypes.byref(d), _p(q), _p(kv), _p(n_entries), _p(kv_raw), _p(raw_base), _p(q_pos),
                               _p(rms_weight), _p(sink), _p(rope), _p(out), _p(lse), _p(ws), nb, _stream(q)))
    return out, lse


class Decoder:
    """Fused CSA step (csa_decode) with its argument block and workspace built once,
    so that repeated calls only re-enqueue the kernels."""

    def __init__(self, q, kv, kv_raw, raw_base, q_pos, q_idx, w, k_idx, n_entries, *, m, topk, window,
                 n_max=None, q_scale=None, k_scale=None, scale=0.0, eps=1e-6, rms_weight=None, sink=None,
                 rope=None, split_items=0, out=None, out_idx=None, out_score=None, lse=None, kv_job=None,
                 key_job=None):
        """kv_job / key_job: compress_job() results, run at the start of every call (the
        entries a step's completed block adds to the KV cache and to the index keys)."""
        self.tensors = [q, kv, kv_raw, raw_base, q_pos, q_idx, w, k_idx, n_entries, q_scale, k_scale, rms_weight,
                        sink, rope]
        self.jobs = (kv_job, key_job)
        a = DecodeArgs()
        a.kv_job = ctypes.pointer(kv_job) if kv_job is not None else None
        a.key_job = ctypes.pointer(key_job) if key_job is not None else None
        a.index = _index_desc(q_idx, k_idx, m, topk, n_max, *_index_dtype(q_idx, k_idx))
        a.attn = _mqa_desc(q, kv, kv_raw, topk=topk, window=window, scale=scale, eps=eps, split_items=split_items)
        dev = q.device
        self.out = torch.empty_like(q) if out is None else out
        self.out_idx = torch.empty((q.shape[0], q.shape[1], topk), dtype=torch.int32, device=dev) \
            if out_idx is None else out_idx
        self.out_score = out_score
        self.lse = lse
        for name, t in (("q", q), ("kv", kv), ("kv_raw", kv_raw), ("raw_base", raw_base), ("q_pos", q_pos),
                        ("rms_weight", rms_weight), ("sink", sink), ("rope", rope), ("q_idx", q_idx), ("q_idx_scale", q_scale),
                        ("w", w),
                        ("k_idx", k_idx), ("k_idx_scale", k_scale), ("n_entries", n_entries),
                        ("out_idx", self.out_idx), ("out_score", out_score), ("out", self.out), ("lse", lse)):
            setattr(a, name, _p(t))
        self.args = a
        self.ws, self.nb = _workspace(lib().csa_decode_workspace_size(ctypes.byref(a)), dev, None)
        self.stream_of = q

    def __call__(self):
        _check(lib().csa_decode(ctypes.byref(self.args), _p(self.ws), self.nb, _stream(self.stream_of)))
        return self.out, self.out_idx

    def call_noalloc(self):
        """The same step through csa_decode_noalloc: the library's own scratch array as
        the workspace (this object's workspace is not used)."""
        _check(lib().csa_decode_noalloc(ctypes.byref(self.args), _stream(self.stream_of)))
        return self.out, self.out_idx


def timing_enable(on=True):
    """Bracket every later library launch (outside graph capture) with HIP events."""
    _check(lib().csa_timing_enable(1 if on else 0))


def timing_collect():
    """Wait for the timed launches; return {kernel: {launches, avg_us, min_us, max_us}}."""
    L = lib()
    buf = (KernelTime * 64)()
    n = L.csa_timing_collect(buf, 64)
    res = {}
    for t in buf[:n]:
        res[t.name.decode()] = {"launches": t.launches, "avg_us": t.total_us / max(1, t.launches),
                                "min_us": t.min_us, "max_us": t.max_us}
    return res
