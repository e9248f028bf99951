"""Seeded synthetic inputs for causal multi-head attention.

This module is shared by the tests, the benchmark and the oracle checks. It
holds shapes, seeds and random draws only: none of the attention arithmetic
lives here, so neither the GPU path nor the oracle depends on the other
through it.

Layout of every tensor is ``[B, S, H, D]`` row-major, the (batch, sequence,
heads, head_dim) layout the Masked Multi-Head Attention page fixes in its
section 2.1 (tensors flattened to ``(B*S, H*D)`` rows).

The five workloads:

* ``fp32_tiny``     fp32, B=1, H=2,  S=64,   D=32,  causal, N(0,1)
* ``fp32_small``    fp32, B=2, H=8,  S=512,  D=64,  causal, N(0,1)
* ``bf16_s2048``    bf16, B=1, H=32, S=2048, D=128, causal, N(0,1)
                    (hidden 4096: the LLaMA-7B layer shape of the MMHA page, section 1)
* ``bf16_s4096``    bf16, B=1, H=32, S=4096, D=128, causal, Q,K ~ N(0, 4^2),
                    V ~ N(0,1) (logits reach about +-100: stability stress)
* ``bf16_decode``   bf16 decode, B=16 sequences, one query each, H=32, D=128,
                    KV-cache capacity 4096, lengths uniform in [1, 4096]
* ``bf16_kvcache``  bf16 chunked prefill into a KV cache: B=8 sequences, a chunk
                    of 512 new queries each, H=32, D=128, cache capacity 4096,
                    lengths (cached tokens including the chunk) uniform in
                    [512, 4096], causal
* ``fp16_s2048``    the bf16_s2048 shape in fp16 (the pages' half-precision
                    storage), N(0,1)
* ``bf16_keypad``   bf16 key-padding forward: B=8 sequences padded to S=1024,
                    H=32, D=128, no causal rule, key j of entry b visible iff
                    j < len_b with len_b uniform in [256, 1024] (right padding)
* ``bf16_qkv``      bf16 Q/K/V projection of the bf16_s2048 layer: X [1, 2048,
                    4096] ~ N(0,1), stacked weights [3*32*128, 4096] ~ N(0,
                    1/4096) (unit-variance outputs), drawn x then w
* ``bf16_softmax``  bf16 score matrix of the bf16_s2048 layer, [1, 32, 2048,
                    2048], entries ~ N(0, 128) (the spread of q.k for unit
                    q, k of length 128), scale 1/sqrt(128), causal

Generator: a torch CPU ``Generator`` seeded with ``1000 + index`` (1001..1010).
Prefill draws q, k, v in that order as ``randn(B,S,H,D) * std``; decode,
the KV-cache prefill and the key-padding forward draw the lengths first,
then q, K and V. bf16 tensors are the
round-to-nearest-even cast of the fp32 draw (``Tensor.to(torch.bfloat16)``).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Prefill:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    S_q: int
    S_kv: int
    D: int
    causal: bool
    seed: int
    qk_std: float = 1.0
    v_std: float = 1.0

    def flops(self) -> int:
        """Algorithmic FLOP: 4*B*H*D per visible (query, key) pair.

        Two multiply-adds (QK^T and P.V) per visible pair; masked pairs and the
        softmax exponentials are not counted.
        """
        return 4 * self.B * self.H * self.D * visible_pairs(self.S_q, self.S_kv, self.causal)


@dataclass(frozen=True)
class Decode:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    S_cap: int
    D: int
    seed: int
    len_lo: int = 1
    len_hi: int = 4096


@dataclass(frozen=True)
class KVCachePrefill:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    S_q: int
    S_cap: int
    D: int
    seed: int
    len_lo: int
    len_hi: int
    causal: bool = True

    def flops(self, seqlens) -> int:
        """Algorithmic FLOP: 4*H*D per visible (query, key) pair, summed over entries."""
        pairs = 0
        for n in seqlens:
            n = max(0, min(int(n), self.S_cap))
            pairs += visible_pairs_kv(self.S_q, n, self.causal)
        return 4 * self.H * self.D * pairs


def visible_pairs_kv(S_q: int, n: int, causal: bool) -> int:
    """Visible pairs of S_q queries at positions n-S_q .. n-1 over n keys (none for a
    query at a negative position)."""
    if not causal:
        return S_q * n
    return sum(max(0, min(n, n - S_q + i + 1)) for i in range(S_q))


def visible_pairs(S_q: int, S_kv: int, causal: bool) -> int:
    """Number of (i, j) pairs a query sees (bottom-right causal alignment)."""
    if not causal:
        return S_q * S_kv
    off = S_kv - S_q
    return sum(min(S_kv, i + 1 + off) for i in range(S_q))


FP32_TINY = Prefill("fp32_tiny", torch.float32, 1, 2, 64, 64, 32, True, 1001)
FP32_SMALL = Prefill("fp32_small", torch.float32, 2, 8, 512, 512, 64, True, 1002)
BF16_S2048 = Prefill("bf16_s2048", torch.bfloat16, 1, 32, 2048, 2048, 128, True, 1003)
BF16_S4096 = Prefill("bf16_s4096", torch.bfloat16, 1, 32, 4096, 4096, 128, True, 1004,
                     qk_std=4.0, v_std=1.0)
BF16_DECODE = Decode("bf16_decode", torch.bfloat16, 16, 32, 4096, 128, 1005)
BF16_KVCACHE = KVCachePrefill("bf16_kvcache", torch.bfloat16, 8, 32, 512, 4096, 128, 1006, 512, 4096)
FP16_S2048 = Prefill("fp16_s2048", torch.float16, 1, 32, 2048, 2048, 128, True, 1007)


@dataclass(frozen=True)
class KeyPadPrefill:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    S: int
    D: int
    seed: int
    len_lo: int
    len_hi: int

    def flops(self, lens) -> int:
        """Algorithmic FLOP: 4*H*D per visible pair; every one of the S queries of
        entry b sees its len_b unpadded keys."""
        return 4 * self.H * self.D * self.S * sum(max(0, min(int(n), self.S)) for n in lens)


BF16_KEYPAD = KeyPadPrefill("bf16_keypad", torch.bfloat16, 8, 32, 1024, 128, 1008, 256, 1024)


@dataclass(frozen=True)
class QkvProj:
    name: str
    dtype: torch.dtype
    B: int
    S: int
    E: int
    H: int
    D: int
    seed: int

    def flops(self) -> int:
        """2 * M * E * 3HD: one multiply-add per (row, input, output) triple."""
        return 2 * self.B * self.S * self.E * 3 * self.H * self.D


BF16_QKV = QkvProj("bf16_qkv", torch.bfloat16, 1, 2048, 4096, 32, 128, 1009)

@dataclass(frozen=True)
class Scores:
    """A materialised score matrix [B, H, S_q, S_kv] for the standalone softmax."""
    name: str
    dtype: torch.dtype
    B: int
    H: int
    S_q: int
    S_kv: int
    causal: bool
    seed: int
    std: float
    scale: float

    def algorithmic_bytes(self) -> int:
        """Visible scores read once, every probability (zeros included) written once."""
        es = torch.empty(0, dtype=self.dtype).element_size()
        rows = self.B * self.H
        return es * rows * (visible_pairs(self.S_q, self.S_kv, self.causal) + self.S_q * self.S_kv)


BF16_SOFTMAX = Scores("bf16_softmax", torch.bfloat16, 1, 32, 2048, 2048, True, 1010,
                      std=128 ** 0.5, scale=128 ** -0.5)


def make_scores(cfg: Scores) -> torch.Tensor:
    """Draw s = randn(B, H, S_q, S_kv) * std on the CPU, cast to cfg.dtype."""
    g = torch.Generator().manual_seed(cfg.seed)
    s = torch.randn(cfg.B, cfg.H, cfg.S_q, cfg.S_kv, generator=g) * cfg.std
    return s.to(cfg.dtype).contiguous()


# Position-encoding table of the bf16_s2048 layer's width, for 4096 positions
# (no random draw: the table is a function of its sizes).
PE_S, PE_D = 4096, 4096

PREFILL_CONFIGS = (FP32_TINY, FP32_SMALL, BF16_S2048, BF16_S4096)


def make_prefill(cfg: Prefill, device: str | torch.device = "cpu"):
    """Draw (q, k, v) for a prefill workload; CPU draw, then optional copy."""
    g = torch.Generator().manual_seed(cfg.seed)
    q = torch.randn(cfg.B, cfg.S_q, cfg.H, cfg.D, generator=g) * cfg.qk_std
    k = torch.randn(cfg.B, cfg.S_kv, cfg.H, cfg.D, generator=g) * cfg.qk_std
    v = torch.randn(cfg.B, cfg.S_kv, cfg.H, cfg.D, generator=g) * cfg.v_std
    out = tuple(t.to(cfg.dtype).contiguous() for t in (q, k, v))
    if str(device) != "cpu":
        out = tuple(t.to(device) for t in out)
    return out


def make_prefill_shape(seed: int, dtype: torch.dtype, B: int, H: int, S_q: int, S_kv: int,
                       D: int, qk_std: float = 1.0, v_std: float = 1.0):
    """Same recipe as :func:`make_prefill` for an arbitrary (edge-case) shape."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S_q, H, D, generator=g) * qk_std
    k = torch.randn(B, S_kv, H, D, generator=g) * qk_std
    v = torch.randn(B, S_kv, H, D, generator=g) * v_std
    return tuple(t.to(dtype).contiguous() for t in (q, k, v))


def make_decode(cfg: Decode, nan_fill: bool = False, seqlens=None, S_cap: int | None = None,
                B: int | None = None):
    """Draw (seqlens, q, kcache, vcache) on the CPU.

    ``seqlens`` is int32[B] drawn uniform in [len_lo, len_hi] unless given.
    With ``nan_fill`` every cache slot at or beyond a sequence's length holds
    NaN, so any read past the valid prefix shows up in the output.
    """
    B = cfg.B if B is None else B
    S_cap = cfg.S_cap if S_cap is None else S_cap
    g = torch.Generator().manual_seed(cfg.seed)
    drawn = torch.randint(cfg.len_lo, cfg.len_hi + 1, (B,), generator=g, dtype=torch.int32)
    if seqlens is None:
        seqlens = drawn
    else:
        seqlens = torch.as_tensor(seqlens, dtype=torch.int32)
    q = torch.randn(B, 1, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    kc = torch.randn(B, S_cap, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    vc = torch.randn(B, S_cap, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    if nan_fill:
        for b in range(B):
            n = max(0, min(int(seqlens[b]), S_cap))
            kc[b, n:] = float("nan")
            vc[b, n:] = float("nan")
    return seqlens, q.contiguous(), kc.contiguous(), vc.contiguous()


def decode_kv_bytes(seqlens, H: int, D: int, elem_bytes: int, S_cap: int) -> int:
    """Algorithmic decode traffic: K and V rows of every valid token, plus q and o."""
    total = 0
    for n in seqlens:
        total += max(0, min(int(n), S_cap))
    B = len(seqlens)
    return total * H * D * 2 * elem_bytes + 2 * B * H * D * elem_bytes


def make_keypad_prefill(cfg: KeyPadPrefill):
    """Draw (lens, key_mask, q, k, v) on the CPU: right-padded entries, key j of
    entry b visible iff j < lens[b] (key_mask is bool [B, S])."""
    g = torch.Generator().manual_seed(cfg.seed)
    lens = torch.randint(cfg.len_lo, cfg.len_hi + 1, (cfg.B,), generator=g, dtype=torch.int32)
    q = torch.randn(cfg.B, cfg.S, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    k = torch.randn(cfg.B, cfg.S, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    v = torch.randn(cfg.B, cfg.S, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    mask = torch.arange(cfg.S)[None, :] < lens[:, None]
    return lens, mask, q.contiguous(), k.contiguous(), v.contiguous()


def make_qkv_proj(cfg: QkvProj, B: int | None = None, S: int | None = None, E: int | None = None,
                  H: int | None = None, D: int | None = None):
    """Draw (x [B,S,E], w [3*H*D, E]) on the CPU; w ~ N(0, 1/E) so the outputs
    have unit variance."""
    B = cfg.B if B is None else B
    S = cfg.S if S is None else S
    E = cfg.E if E is None else E
    H = cfg.H if H is None else H
    D = cfg.D if D is None else D
    g = torch.Generator().manual_seed(cfg.seed)
    x = torch.randn(B, S, E, generator=g).to(cfg.dtype)
    w = (torch.randn(3 * H * D, E, generator=g) / E ** 0.5).to(cfg.dtype)
    return x.contiguous(), w.contiguous()


def make_kvcache_prefill(cfg: KVCachePrefill, nan_fill: bool = False, seqlens=None, S_cap: int | None = None,
                         B: int | None = None, S_q: int | None = None):
    """Draw (seqlens, q, kcache, vcache) for a KV-cache prefill on the CPU.

    ``seqlens`` is int32[B] uniform in [len_lo, len_hi] unless given; with
    ``nan_fill`` the cache rows at or past each length hold NaN.
    """
    B = cfg.B if B is None else B
    S_cap = cfg.S_cap if S_cap is None else S_cap
    S_q = cfg.S_q if S_q is None else S_q
    g = torch.Generator().manual_seed(cfg.seed)
    drawn = torch.randint(cfg.len_lo, cfg.len_hi + 1, (B,), generator=g, dtype=torch.int32)
    seqlens = drawn if seqlens is None else torch.as_tensor(seqlens, dtype=torch.int32)
    q = torch.randn(B, S_q, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    kc = torch.randn(B, S_cap, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    vc = torch.randn(B, S_cap, cfg.H, cfg.D, generator=g).to(cfg.dtype)
    if nan_fill:
        for b in range(B):
            n = max(0, min(int(seqlens[b]), S_cap))
            kc[b, n:] = float("nan")
            vc[b, n:] = float("nan")
    return seqlens, q.contiguous(), kc.contiguous(), vc.contiguous()
