"""Causal multi-head attention for MI355X (gfx950): Python binding of libattn.so.

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/attn.h``; this module checks
tensors (device, dtype, layout), passes their device pointers and the current
torch stream, and turns status codes into exceptions. There is no CPU or
PyTorch fallback: if ``libattn.so`` is missing the import fails.

    o = attn_fwd(q, k, v, causal=True)                      # [B, S, H, D]
    o = attn_decode(q, kcache, vcache, seqlens)             # q [B, 1, H, D]
    o, lse = attn_fwd_kvcache(q, kcache, vcache, seqlens_kv, return_lse=True)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_F16 = 0, 1, 2
ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = 0, 1, 2, 3, 4

_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class FwdPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("kernel", "block_m", "block_n", "paired", "grid", "threads",
                                           "lds_bytes", "max_tiles", "min_tiles")]


class DecodePlan(ctypes.Structure):
    _fields_ = [("split_workgroups", ctypes.c_int), ("records", ctypes.c_int), ("threads", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m causal_head_attention_amd.build` "
                          "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i]
    lib.attn_fwd.restype = i
    lib.attn_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i]
    lib.attn_fwd_kvcache.restype = i
    lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz]
    lib.attn_decode.restype = i
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i]
    lib.attn_decode_noalloc.restype = i
    lib.attn_fwd_mask.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i]
    lib.attn_fwd_mask.restype = i
    lib.attn_qkv_proj.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i]
    lib.attn_qkv_proj.restype = i
    lib.attn_sinusoidal_pe.argtypes = [vp, i, i, i]
    lib.attn_masked_softmax.argtypes = [vp, vp, i, i, i, i, ctypes.c_float, i, i]
    lib.attn_masked_softmax.restype = i
    lib.attn_sinusoidal_pe.restype = i
    lib.attn_set_stream.argtypes = [vp]
    lib.attn_set_stream.restype = i
    lib.attn_set_timing_events.argtypes = [vp, vp]
    lib.attn_set_timing_events.restype = i
    lib.attn_set_clock_probe.argtypes = [vp]
    lib.attn_set_clock_probe.restype = i
    lib.attn_get_stream.argtypes = []
    lib.attn_get_stream.restype = vp
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_fwd_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(FwdPlan)]
    lib.attn_fwd_plan.restype = i
    lib.attn_decode_plan.argtypes = [i, i, i, i, i, ctypes.POINTER(DecodePlan)]
    lib.attn_decode_plan.restype = i
    lib.attn_xcd_remap.argtypes = [i, i]
    lib.attn_xcd_remap.restype = i
    lib.attn_decode_range_start.argtypes = [i, i]
    lib.attn_decode_range_start.restype = i
    lib.attn_decode_range_of.argtypes = [i, i]
    lib.attn_decode_range_of.restype = i
    return lib


def load() -> ctypes.CDLL:
    """Load libattn.so (once). Raises ImportError if it is not built: no fallback exists."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):  # module attribute `lib` loads the library on first use
    if name == "lib":
        return load()
    raise AttributeError(name)


def _status_name(status: int) -> str:
    return load().attn_status_string(status).decode()


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, load().attn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}: float32, bfloat16 or float16")
    return _DTYPES[t.dtype]


def _dev_tensor(name: str, t: torch.Tensor, dim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous ([B, S, H, D] row-major)")


def _set_stream(device: torch.device) -> None:
    _check(load().attn_set_stream(ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)))


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None,
             causal: bool = True) -> torch.Tensor:
    """Fused masked attention forward. q [B,S_q,H,D]; k, v [B,S_kv,H,D]; returns o [B,S_q,H,D]."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, 4)
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    if tuple(k.shape) != (B, S_kv, H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if o is None:
        o = torch.empty_like(q)
    else:
        _dev_tensor("o", o, 4)
        if tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype:
            raise ValueError("o must match q in shape and dtype")
    _set_stream(q.device)
    _check(load().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, S_q, S_kv, D,
                        int(bool(causal)), _dtype_code(q)))
    return o


def attn_fwd_kvcache(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
                     seqlens_kv: torch.Tensor | None = None, o: torch.Tensor | None = None,
                     causal: bool = True, return_lse: bool = False):
    """Chunk of queries against a KV cache with per-sequence lengths.

    q [B,S_q,H,D]; caches [B,S_cap,H,D]; seqlens_kv int32[B] on the GPU or None (all S_cap rows valid).
    Returns o [B,S_q,H,D], or (o, lse) with lse float32 [B,H,S_q] when return_lse is set."""
    for n, t in (("q", q), ("kcache", kcache), ("vcache", vcache)):
        _dev_tensor(n, t, 4)
    B, S_q, H, D = q.shape
    S_cap = kcache.shape[1]
    if tuple(kcache.shape) != (B, S_cap, H, D) or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kcache {tuple(kcache.shape)}, "
                         f"vcache {tuple(vcache.shape)}")
    if not (q.dtype == kcache.dtype == vcache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if seqlens_kv is not None:
        _dev_tensor("seqlens_kv", seqlens_kv, 1)
        if seqlens_kv.dtype != torch.int32 or seqlens_kv.shape[0] != B:
            raise ValueError("seqlens_kv must be int32[B]")
    if o is None:
        o = torch.empty_like(q)
    else:
        _dev_tensor("o", o, 4)
        if tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype:
            raise ValueError("o must match q in shape and dtype")
    lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device) if return_lse else None
    _set_stream(q.device)
    _check(load().attn_fwd_kvcache(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                                   seqlens_kv.data_ptr() if seqlens_kv is not None else None, o.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, B, H, S_q, S_cap, D,
                                   int(bool(causal)), _dtype_code(q)))
    return (o, lse) if return_lse else o


def attn_fwd_mask(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, key_mask: torch.Tensor | None = None,
                  o: torch.Tensor | None = None, causal: bool = True, return_lse: bool = False):
    """Forward with a key-padding mask. q [B,S_q,H,D]; k, v [B,S_kv,H,D]; key_mask [B,S_kv] on the GPU
    (bool or uint8; False / 0 hides the key from every query of its entry) or None.
    Returns o, or (o, lse) with lse float32 [B,H,S_q] when return_lse is set."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dev_tensor(n, t, 4)
    B, S_q, H, D = q.shape
    S_kv = k.shape[1]
    if tuple(k.shape) != (B, S_kv, H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if key_mask is not None:
        _dev_tensor("key_mask", key_mask, 2)
        if tuple(key_mask.shape) != (B, S_kv):
            raise ValueError(f"key_mask must be [B, S_kv] = {(B, S_kv)}, got {tuple(key_mask.shape)}")
        if key_mask.dtype == torch.bool:
            key_mask = key_mask.view(torch.uint8)
        elif key_mask.dtype != torch.uint8:
            raise TypeError("key_mask must be bool or uint8")
    if o is None:
        o = torch.empty_like(q)
    else:
        _dev_tensor("o", o, 4)
        if tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype:
            raise ValueError("o must match q in shape and dtype")
    lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device) if return_lse else None
    _set_stream(q.device)
    _check(load().attn_fwd_mask(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                key_mask.data_ptr() if key_mask is not None else None, o.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, H, S_q, S_kv, D,
                                int(bool(causal)), _dtype_code(q)))
    return (o, lse) if return_lse else o


def qkv_proj(x: torch.Tensor, w: torch.Tensor, H: int, D: int, q: torch.Tensor | None = None,
             k: torch.Tensor | None = None, v: torch.Tensor | None = None):
    """Q, K, V projections as one GEMM. x [B,S,E] (or [M,E]); w [3*H*D, E] output-major.
    Returns (q, k, v), each [B,S,H,D] (or [M,H,D]) in x's dtype (bfloat16 or float16)."""
    if not isinstance(x, torch.Tensor) or not isinstance(w, torch.Tensor):
        raise TypeError("x and w must be torch.Tensors")
    for n, t in (("x", x), ("w", w)):
        if not t.is_cuda:
            raise ValueError(f"{n} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if x.dim() < 2 or w.dim() != 2:
        raise ValueError("x must be [..., E] and w [3*H*D, E]")
    if x.dtype != w.dtype:
        raise TypeError("x and w must share one dtype")
    E = x.shape[-1]
    lead = tuple(x.shape[:-1])
    M = 1
    for s in lead:
        M *= s
    if tuple(w.shape) != (3 * H * D, E):
        raise ValueError(f"w must be [3*H*D, E] = {(3 * H * D, E)}, got {tuple(w.shape)}")
    outs = []
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            t = torch.empty(lead + (H, D), dtype=x.dtype, device=x.device)
        else:
            _dev_tensor(n, t, len(lead) + 2)
            if tuple(t.shape) != lead + (H, D) or t.dtype != x.dtype:
                raise ValueError(f"{n} must be {lead + (H, D)} of dtype {x.dtype}")
        outs.append(t)
    _set_stream(x.device)
    _check(load().attn_qkv_proj(x.data_ptr(), w.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                                outs[2].data_ptr(), M, E, H, D, _dtype_code(x)))
    return tuple(outs)


def sinusoidal_pe(S: int, d_model: int, pos0: int = 0, out: torch.Tensor | None = None,
                  device: torch.device | str = "cuda") -> torch.Tensor:
    """[S, d_model] float32 position encoding for positions pos0 .. pos0+S-1, on the GPU."""
    if out is None:
        out = torch.empty(S, d_model, dtype=torch.float32, device=device)
    else:
        _dev_tensor("out", out, 2)
        if tuple(out.shape) != (S, d_model) or out.dtype != torch.float32:
            raise ValueError(f"out must be float32 [{S}, {d_model}]")
    _set_stream(out.device)
    _check(load().attn_sinusoidal_pe(out.data_ptr(), S, d_model, pos0))
    return out


def masked_softmax(s: torch.Tensor, scale: float = 1.0, causal: bool = True,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Row softmax of scale * s [B,H,S_q,S_kv] under the causal rule (bottom-right); masked
    entries 0. out may be s itself (in place). float32, bfloat16 or float16."""
    _dev_tensor("s", s, 4)
    if out is None:
        out = torch.empty_like(s)
    else:
        _dev_tensor("out", out, 4)
        if tuple(out.shape) != tuple(s.shape) or out.dtype != s.dtype:
            raise ValueError(f"out must be {tuple(s.shape)} of dtype {s.dtype}")
    B, H, S_q, S_kv = s.shape
    _set_stream(s.device)
    _check(load().attn_masked_softmax(s.data_ptr(), out.data_ptr(), B, H, S_q, S_kv, float(scale), int(bool(causal)),
                                      _dtype_code(s)))
    return out


def attn_decode_workspace_bytes(B: int, H: int, S_cap: int, D: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, H, S_cap, D))


def attn_decode(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, seqlens: torch.Tensor,
                o: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Single-query decode. q [B,1,H,D]; caches [B,S_cap,H,D]; seqlens int32[B] on the GPU."""
    for n, t in (("q", q), ("kcache", kcache), ("vcache", vcache)):
        _dev_tensor(n, t, 4)
    _dev_tensor("seqlens", seqlens, 1)
    B, one, H, D = q.shape
    S_cap = kcache.shape[1]
    if one != 1 or tuple(kcache.shape) != (B, S_cap, H, D) or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kcache {tuple(kcache.shape)}, "
                         f"vcache {tuple(vcache.shape)}")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32[B]")
    if not (q.dtype == kcache.dtype == vcache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if o is None:
        o = torch.empty_like(q)
    else:
        _dev_tensor("o", o, 4)
        if tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype or o.device != q.device:
            raise ValueError("o must match q in shape, dtype and device")
    need = attn_decode_workspace_bytes(B, H, S_cap, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        if not isinstance(workspace, torch.Tensor):
            raise TypeError("workspace must be a torch.Tensor")
        if not workspace.is_cuda or workspace.device != q.device:
            raise ValueError("workspace must be a GPU tensor on q's device")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        # its size is checked by the library (ATTN_ERR_WORKSPACE)
    _set_stream(q.device)
    _check(load().attn_decode(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), seqlens.data_ptr(),
                           o.data_ptr(), B, H, S_cap, D, _dtype_code(q), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size()))
    return o


def attn_decode_noalloc(q: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor, seqlens: torch.Tensor,
                        o: torch.Tensor) -> torch.Tensor:
    """attn_decode without a workspace argument: the library's fixed per-GPU
    scratch serves instead, and nothing is allocated (o must be given)."""
    for n, t in (("q", q), ("kcache", kcache), ("vcache", vcache), ("o", o)):
        _dev_tensor(n, t, 4)
    _dev_tensor("seqlens", seqlens, 1)
    B, one, H, D = q.shape
    S_cap = kcache.shape[1]
    if one != 1 or tuple(kcache.shape) != (B, S_cap, H, D) or tuple(vcache.shape) != tuple(kcache.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, kcache {tuple(kcache.shape)}, "
                         f"vcache {tuple(vcache.shape)}")
    if seqlens.dtype != torch.int32 or seqlens.shape[0] != B:
        raise ValueError("seqlens must be int32[B]")
    if not (q.dtype == kcache.dtype == vcache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if tuple(o.shape) != tuple(q.shape) or o.dtype != q.dtype or o.device != q.device:
        raise ValueError("o must match q in shape, dtype and device")
    _set_stream(q.device)
    _check(load().attn_decode_noalloc(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), seqlens.data_ptr(),
                                      o.data_ptr(), B, H, S_cap, D, _dtype_code(q)))
    return o


def attn_set_timing_events(start: int | None, stop: int | None) -> None:
    """Arm two hipEvent_t handles for the next attn_fwd / attn_decode call on this thread."""
    _check(load().attn_set_timing_events(ctypes.c_void_p(start or 0), ctypes.c_void_p(stop or 0)))


def attn_set_clock_probe(buf: torch.Tensor | None) -> None:
    """Arm a device int64[4] buffer for the next attn_fwd call on this thread:
    the prefill kernel's workgroup 0 writes (shader clock, 100 MHz real time)
    at its start and at its end. None disarms."""
    if buf is None:
        _check(load().attn_set_clock_probe(ctypes.c_void_p(0)))
        return
    _dev_tensor("clock probe", buf, 1)
    if buf.dtype != torch.int64 or buf.numel() < 4:
        raise ValueError("clock probe must be an int64 GPU tensor of at least 4 elements")
    _check(load().attn_set_clock_probe(ctypes.c_void_p(buf.data_ptr())))


def attn_fwd_plan(B: int, H: int, S_q: int, S_kv: int, D: int, causal: bool, dtype: int) -> FwdPlan:
    plan = FwdPlan()
    _check(load().attn_fwd_plan(B, H, S_q, S_kv, D, int(bool(causal)), dtype, ctypes.byref(plan)))
    return plan


def attn_decode_plan(B: int, H: int, S_cap: int, D: int, dtype: int) -> DecodePlan:
    plan = DecodePlan()
    _check(load().attn_decode_plan(B, H, S_cap, D, dtype, ctypes.byref(plan)))
    return plan


__all__ = ["attn_fwd", "attn_fwd_kvcache", "attn_fwd_mask", "attn_decode", "attn_decode_noalloc", "qkv_proj", "sinusoidal_pe", "masked_softmax", "attn_decode_workspace_bytes", "attn_fwd_plan", "attn_decode_plan",
           "attn_set_timing_events", "attn_set_clock_probe",
           "AttnError", "ATTN_F32", "ATTN_BF16", "ATTN_F16", "lib", "LIB_PATH"]
