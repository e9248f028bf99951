"""fp64 CPU oracle for causal multi-head attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never loads it and
shares no code with it.

The arithmetic lives in ``attn_oracle.c`` (plain loops, fp64, the full score
matrix of each head materialised); this module compiles it with gcc, loads
it with ctypes and widens inputs to fp64 exactly. Passages followed: the
"Hand-written Masked Multi-Head Attention CUDA kernel" page, sections 2,
2.1 and 2.2 (definition, [B,S,H,D] layout, j <= i), and the "Week-4 CUDA
notes" page, section 2.2 (unfused softmax(QK^T/sqrt(d))V, -inf mask, max
subtraction; the running sum whose log is the log-sum-exp output; a padded
key's score set to -inf so that its weight is exactly 0).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

BUILD_CMD = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` next to its source (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = BUILD_CMD[:-3] + ["-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            dp = ctypes.POINTER(ctypes.c_double)
            ip = ctypes.POINTER(ctypes.c_int32)
            lib.oracle_attn_fwd_f64.argtypes = [dp, dp, dp, dp, dp] + [ctypes.c_int] * 6
            lib.oracle_attn_fwd_f64.restype = ctypes.c_int
            lib.oracle_attn_decode_f64.argtypes = [dp, dp, dp, ip, dp] + [ctypes.c_int] * 4
            lib.oracle_attn_decode_f64.restype = ctypes.c_int
            lib.oracle_attn_fwd_kvcache_f64.argtypes = [dp, dp, dp, ip, dp, dp] + [ctypes.c_int] * 6
            lib.oracle_attn_fwd_kvcache_f64.restype = ctypes.c_int
            u8p = ctypes.POINTER(ctypes.c_uint8)
            lib.oracle_attn_fwd_mask_f64.argtypes = [dp, dp, dp, u8p, dp, dp] + [ctypes.c_int] * 6
            lib.oracle_attn_fwd_mask_f64.restype = ctypes.c_int
            lib.oracle_qkv_proj_f64.argtypes = [dp, dp, dp, dp, dp] + [ctypes.c_int] * 3
            lib.oracle_qkv_proj_f64.restype = ctypes.c_int
            lib.oracle_sinusoidal_pe_f64.argtypes = [dp] + [ctypes.c_int] * 3
            lib.oracle_sinusoidal_pe_f64.restype = ctypes.c_int
            lib.oracle_masked_softmax_f64.argtypes = [dp, dp] + [ctypes.c_int] * 4 + [ctypes.c_double, ctypes.c_int]
            lib.oracle_masked_softmax_f64.restype = ctypes.c_int
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact widening to a C-contiguous float64 array (bf16/fp32 -> fp64 is exact)."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attn_fwd(q, k, v, causal: bool = True, return_p: bool = False):
    """O = softmax(Q K^T / sqrt(D) + M) V in fp64.

    q: [B, S_q, H, D]; k, v: [B, S_kv, H, D]. Returns O [B, S_q, H, D] (fp64
    numpy) and, with ``return_p``, P [B, H, S_q, S_kv].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    if k.shape != (B, S_kv, H, D) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    o = np.zeros((B, S_q, H, D), dtype=np.float64)
    p = np.zeros((B, H, S_q, S_kv), dtype=np.float64) if return_p else None
    rc = _load().oracle_attn_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(p) if p is not None else None,
                                     B, H, S_q, S_kv, D, int(bool(causal)))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd_f64 rejected the arguments (code {rc})")
    return (o, p) if return_p else o


def attn_decode(q, kcache, vcache, seqlens):
    """Single-query decode: q [B,1,H,D], caches [B,S_cap,H,D], seqlens int32[B]."""
    q, kc, vc = _f64(q), _f64(kcache), _f64(vcache)
    B, _, H, D = q.shape
    S_cap = kc.shape[1]
    if hasattr(seqlens, "numpy"):
        seqlens = seqlens.cpu().numpy()
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    if sl.shape != (B,):
        raise ValueError("seqlens must be int32[B]")
    o = np.zeros((B, 1, H, D), dtype=np.float64)
    rc = _load().oracle_attn_decode_f64(_ptr(q), _ptr(kc), _ptr(vc),
                                        sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                        _ptr(o), B, H, S_cap, D)
    if rc != 0:
        raise ValueError(f"oracle_attn_decode_f64 rejected the arguments (code {rc})")
    return o


def attn_fwd_kvcache(q, kcache, vcache, seqlens=None, causal: bool = True):
    """Chunk of queries against a KV cache with per-entry lengths, plus log-sum-exp.

    q [B,S_q,H,D]; caches [B,S_cap,H,D]; seqlens int32[B] or None (all S_cap rows).
    Returns (O [B,S_q,H,D], LSE [B,H,S_q]) as fp64 numpy arrays; rows that see no
    key are 0 with LSE -inf.
    """
    q, kc, vc = _f64(q), _f64(kcache), _f64(vcache)
    B, S_q, H, D = q.shape
    S_cap = kc.shape[1]
    if kc.shape != (B, S_cap, H, D) or vc.shape != kc.shape:
        raise ValueError("shape mismatch")
    sl = None
    if seqlens is not None:
        if hasattr(seqlens, "numpy"):
            seqlens = seqlens.cpu().numpy()
        sl = np.ascontiguousarray(seqlens, dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seqlens must be int32[B]")
    o = np.zeros((B, S_q, H, D), dtype=np.float64)
    lse = np.zeros((B, H, S_q), dtype=np.float64)
    rc = _load().oracle_attn_fwd_kvcache_f64(
        _ptr(q), _ptr(kc), _ptr(vc), sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if sl is not None else None,
        _ptr(o), _ptr(lse), B, H, S_q, S_cap, D, int(bool(causal)))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd_kvcache_f64 rejected the arguments (code {rc})")
    return o, lse


def attn_fwd_mask(q, k, v, key_mask=None, causal: bool = True):
    """Forward with a key-padding mask, plus log-sum-exp.

    q [B,S_q,H,D]; k, v [B,S_kv,H,D]; key_mask [B,S_kv] (nonzero = visible) or
    None. Returns (O [B,S_q,H,D], LSE [B,H,S_q]) as fp64 numpy arrays; rows with
    no visible key are 0 with LSE -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    if k.shape != (B, S_kv, H, D) or v.shape != k.shape:
        raise ValueError("shape mismatch")
    km = None
    if key_mask is not None:
        if hasattr(key_mask, "numpy"):
            key_mask = key_mask.cpu().numpy()
        km = np.ascontiguousarray(np.asarray(key_mask) != 0, dtype=np.uint8)
        if km.shape != (B, S_kv):
            raise ValueError("key_mask must be [B, S_kv]")
    o = np.zeros((B, S_q, H, D), dtype=np.float64)
    lse = np.zeros((B, H, S_q), dtype=np.float64)
    rc = _load().oracle_attn_fwd_mask_f64(
        _ptr(q), _ptr(k), _ptr(v), km.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)) if km is not None else None,
        _ptr(o), _ptr(lse), B, H, S_q, S_kv, D, int(bool(causal)))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd_mask_f64 rejected the arguments (code {rc})")
    return o, lse


def qkv_proj(x, w, H: int, D: int):
    """Q, K, V projections as one stacked GEMM.

    x [B,S,E] (or [M,E]); w [3*H*D, E] output-major (rows 0..HD-1 give Q's
    columns, then K's, then V's). Returns (q, k, v), each [B,S,H,D] (or
    [M,H,D]) fp64 numpy arrays.
    """
    x, w = _f64(x), _f64(w)
    lead = x.shape[:-1]
    E = x.shape[-1]
    M = int(np.prod(lead))
    N = H * D
    if w.shape != (3 * N, E):
        raise ValueError(f"w must be [3*H*D, E] = {(3 * N, E)}, got {w.shape}")
    x2 = np.ascontiguousarray(x.reshape(M, E))
    outs = [np.zeros((M, N), dtype=np.float64) for _ in range(3)]
    rc = _load().oracle_qkv_proj_f64(_ptr(x2), _ptr(w), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), M, E, N)
    if rc != 0:
        raise ValueError(f"oracle_qkv_proj_f64 rejected the arguments (code {rc})")
    return tuple(o.reshape(*lead, H, D) for o in outs)


def sinusoidal_pe(S: int, d_model: int, pos0: int = 0):
    """[S, d_model] fp64 position encoding for positions pos0 .. pos0+S-1."""
    pe = np.zeros((S, d_model), dtype=np.float64)
    rc = _load().oracle_sinusoidal_pe_f64(_ptr(pe), S, d_model, pos0)
    if rc != 0:
        raise ValueError(f"oracle_sinusoidal_pe_f64 rejected the arguments (code {rc})")
    return pe


def masked_softmax(s, scale: float = 1.0, causal: bool = True):
    """Row softmax of scale * s [B, H, S_q, S_kv] under the causal rule (bottom-right);
    masked entries 0, rows with no visible key 0. fp64 numpy."""
    s = _f64(s)
    B, H, S_q, S_kv = s.shape
    p = np.zeros_like(s)
    rc = _load().oracle_masked_softmax_f64(_ptr(s), _ptr(p), B, H, S_q, S_kv, float(scale), int(bool(causal)))
    if rc != 0:
        raise ValueError(f"oracle_masked_softmax_f64 rejected the arguments (code {rc})")
    return p


def num_threads() -> int:
    return int(_load().oracle_num_threads())
