"""Seeded synthetic inputs with the shapes of the CSA / HCA workloads.

This module draws random numbers and nothing else: it holds none of the
attention method's arithmetic (no pooling, normalisation, scoring, selection,
attention or quantisation).  Its only transformation is rounding fp32 masters
to bf16 storage (round-to-nearest-even), because the bf16 workloads store
bf16.  Both the GPU path and the CPU oracle consume exactly these arrays.

Recipe: a fresh ``numpy.random.Generator(PCG64(seed))`` per workload, fp32
masters from ``standard_normal`` (N(0,1)) or ``random`` (U[0,1)), tensors drawn
in the order they are listed in each function.  bf16 arrays are returned as
uint16 bit patterns.

The five named workloads follow the method's published shapes (DeepSeek-V4:
128 query heads sharing one 512-wide KV head, a 128-token sliding window,
compression ratios 4 and 128, a 64-head x 128 indexer keeping the top 1024).
"""
from __future__ import annotations

import numpy as np

CHUNK = 1 << 24


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(rng, shape) -> np.ndarray:
    """fp32 N(0,1) master, drawn in chunks to bound memory for large tensors."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def uniform(rng, shape) -> np.ndarray:
    return rng.random(shape, dtype=np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for s in range(0, flat_u.size, CHUNK):
        v = flat_u[s:s + CHUNK].astype(np.uint64)
        flat_o[s:s + CHUNK] = ((v + 0x7FFF + ((v >> 16) & 1)) >> 16).astype(np.uint16)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp8_cache_codes(rng, shape) -> np.ndarray:
    """FP8 E4M3 cache rows drawn directly as codes (uint8), no rounding: a uniform sign,
    an exponent field whose weights follow where |N(0,1)| values fall (field e covers
    [2^(e-7), 2^(e-6)), e = 7 is [1, 2)), and a uniform 3-bit mantissa.  Unit-scale data
    like the bf16 caches; every code is finite."""
    w = np.array([0.012, 0.024, 0.048, 0.095, 0.18, 0.30, 0.27, 0.045, 0.0001])   # fields 1 .. 9
    n = int(np.prod(shape))
    sign = rng.integers(0, 2, n, dtype=np.uint8)
    field = (rng.choice(len(w), size=n, p=w / w.sum()) + 1).astype(np.uint8)
    mant = rng.integers(0, 8, n, dtype=np.uint8)
    return ((sign << 7) | (field << 3) | mant).astype(np.uint8).reshape(shape)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 master -> storage array ('f32': float32, 'bf16': uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(dtype)


def value(x: np.ndarray) -> np.ndarray:
    """Storage array -> exact float64 values (uint16 arrays are bf16 bits)."""
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Decode workloads (one query per sequence, at position t = T - 1).
# --------------------------------------------------------------------------

def csa_decode(seed=0, B=8, T=65536, m=4, H=128, d=512, HI=64, dI=128, k=1024, window=128,
               dtype="bf16", idx_dtype="bf16", n_entries=None, t=None):
    """CSA decode with given caches.  Draw order: kv [B,N,d], kI [B,N,dI], q [B,H,d],
    qI [B,HI,dI], w [B,HI] U[0,1), kv_raw [B,window,d].  idx_dtype 'mxfp4' returns
    fp32 masters for qI and kI (the quantisation is a method step)."""
    rng = rng_for(seed)
    N = T // m if n_entries is None else n_entries
    t = T - 1 if t is None else t
    W = max(window, 1)
    kv = store(normal(rng, (B, N, d)), dtype)
    kI = normal(rng, (B, N, dI))
    q = store(normal(rng, (B, H, d)), dtype)
    qI = normal(rng, (B, HI, dI))
    w = uniform(rng, (B, HI))
    kv_raw = store(normal(rng, (B, W, d)), dtype)
    if idx_dtype in ("f32", "bf16"):
        kI, qI = store(kI, idx_dtype), store(qI, idx_dtype)
    return dict(kind="csa", B=B, T=T, m=m, H=H, d=d, HI=HI, dI=dI, k=k, window=window, N=N,
                dtype=dtype, idx_dtype=idx_dtype, eps=1e-6, scale=1.0 / np.sqrt(d),
                kv=kv, kI=kI, q=q, qI=qI, w=w, kv_raw=kv_raw,
                q_pos=np.full((B,), t, dtype=np.int32),
                raw_base=np.full((B,), max(0, t - window + 1), dtype=np.int32),
                n_entries=np.full((B,), N, dtype=np.int32))


def hca_decode(seed=0, B=4, T=1 << 20, m=128, H=128, d=512, window=128, dtype="bf16",
               n_entries=None, t=None):
    """HCA dense decode with a given cache.  Draw order: kv [B,N,d], q [B,H,d],
    kv_raw [B,window,d]."""
    rng = rng_for(seed)
    N = T // m if n_entries is None else n_entries
    t = T - 1 if t is None else t
    W = max(window, 1)
    kv = store(normal(rng, (B, N, d)), dtype)
    q = store(normal(rng, (B, H, d)), dtype)
    kv_raw = store(normal(rng, (B, W, d)), dtype)
    return dict(kind="hca", B=B, T=T, m=m, H=H, d=d, window=window, N=N, dtype=dtype, eps=1e-6,
                scale=1.0 / np.sqrt(d), kv=kv, q=q, kv_raw=kv_raw,
                q_pos=np.full((B,), t, dtype=np.int32),
                raw_base=np.full((B,), max(0, t - window + 1), dtype=np.int32),
                n_entries=np.full((B,), N, dtype=np.int32))


def csa_decode_small_fp32(seed=0, T=2048, m=4, H=8, d=64, HI=4, dI=32, k=64, window=128):
    """The fp32 single-layer CSA decode (T=2048, m=4 -> 512 entries).  Draw order:
    A [T,d], B [T,d], z [T] (pooling logits, shared by both streams), q [H,d],
    qI [HI,dI], kI [T/m,dI], w [HI] U[0,1).  The sliding window reads the last
    `window` rows of stream A (the only token-level KV this workload defines)."""
    rng = rng_for(seed)
    A = normal(rng, (T, d))
    Bs = normal(rng, (T, d))
    z = normal(rng, (T,))
    q = normal(rng, (H, d))
    qI = normal(rng, (HI, dI))
    kI = normal(rng, (T // m, dI))
    w = uniform(rng, (HI,))
    t = T - 1
    return dict(kind="csa_tokens", B=1, T=T, m=m, H=H, d=d, HI=HI, dI=dI, k=k, window=window,
                N=T // m, dtype="f32", idx_dtype="f32", eps=1e-6, scale=1.0 / np.sqrt(d),
                A=A[None], Bs=Bs[None], z=z[None], q=q[None], qI=qI[None], kI=kI[None], w=w[None],
                kv_raw=np.ascontiguousarray(A[None, T - window:T]),
                q_pos=np.full((1,), t, dtype=np.int32),
                raw_base=np.full((1,), T - window, dtype=np.int32),
                n_entries=np.full((1,), T // m, dtype=np.int32))


def csa_decode_fp4(seed=0, T=1 << 20, m=4, H=128, d=512, HI=64, dI=128, k=1024, window=128, B=1):
    """CSA decode at long context with an MXFP4 indexer: bf16 KV, fp32 indexer masters.
    Draw order as csa_decode."""
    return csa_decode(seed=seed, B=B, T=T, m=m, H=H, d=d, HI=HI, dI=dI, k=k, window=window,
                      dtype="bf16", idx_dtype="mxfp4")


def csa_prefill(seed=0, T_prior=61440, n_new=4096, m=4, H=128, d=512, HI=64, dI=128, k=1024,
                window=128, dtype="bf16"):
    """CSA prefill chunk: n_new query tokens appended to T_prior tokens.  Entries
    covering only prior tokens are given; entries of the new blocks are compressed
    from token streams (B stream lags one block, so the streams start m rows early).
    Draw order: kv_prior [P,d], kI_prior [P,dI], A [R,d], B [R,d], z [R],
    AI [R,dI], BI [R,dI], zI [R], q [Q,H,d], qI [Q,HI,dI], w [Q,HI] U,
    kv_raw [Q+window-1, d]  (P = T_prior/m, R = n_new + m, Q = n_new)."""
    rng = rng_for(seed)
    P = T_prior // m
    R = n_new + m
    Q = n_new
    kv_prior = store(normal(rng, (P, d)), dtype)
    kI_prior = store(normal(rng, (P, dI)), dtype)
    A = store(normal(rng, (R, d)), dtype)
    Bs = store(normal(rng, (R, d)), dtype)
    z = normal(rng, (R,))
    AI = store(normal(rng, (R, dI)), dtype)
    BI = store(normal(rng, (R, dI)), dtype)
    zI = normal(rng, (R,))
    q = store(normal(rng, (Q, H, d)), dtype)
    qI = store(normal(rng, (Q, HI, dI)), dtype)
    w = uniform(rng, (Q, HI))
    n_raw = Q + window - 1
    kv_raw = store(normal(rng, (n_raw, d)), dtype)
    T = T_prior + n_new
    return dict(kind="prefill", B=1, T=T, T_prior=T_prior, n_new=Q, m=m, H=H, d=d, HI=HI, dI=dI, k=k,
                window=window, N=T // m, P=P, dtype=dtype, idx_dtype=dtype, eps=1e-6,
                scale=1.0 / np.sqrt(d), kv_prior=kv_prior, kI_prior=kI_prior, A=A, Bs=Bs, z=z,
                AI=AI, BI=BI, zI=zI, tok_base=T_prior - m, q=q, qI=qI, w=w, kv_raw=kv_raw,
                raw_base=T_prior - window + 1,
                q_pos=np.arange(T_prior, T, dtype=np.int32))


# Named workloads (the five single-GPU configurations).
def cfg1(seed=0):
    return csa_decode_small_fp32(seed)


def cfg2(seed=0):
    return csa_decode(seed, B=8, T=65536)


def cfg3(seed=0):
    return hca_decode(seed, B=4, T=1 << 20)


def cfg4(seed=0):
    return csa_decode_fp4(seed, T=1 << 20)


def cfg5(seed=0):
    return csa_prefill(seed)
