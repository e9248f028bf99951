"""The allocation-free decode entry point (attn_decode_noalloc) against
attn_decode through the C ABI, on the GPU.

Two calls in a row share the one fixed scratch array of the GPU; the second
is smaller, so it runs over what the first left there. Each must equal
attn_decode on the same inputs bit for bit (same kernel, same merge order) and
meet the oracle bar of the parity tests.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

BARS = {torch.bfloat16: (2e-2, 1e-2), torch.float16: (5e-3, 3e-3), torch.float32: (1e-4, None)}


def _case(seed, B, H, S_cap, D, dtype):
    g = torch.Generator().manual_seed(seed)
    sl = torch.randint(-2, S_cap + 3, (B,), generator=g, dtype=torch.int32)
    q = torch.randn(B, 1, H, D, generator=g).to(dtype)
    kc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    vc = torch.randn(B, S_cap, H, D, generator=g).to(dtype)
    for b in range(B):   # slots past each length hold NaN: never read
        n = max(0, min(int(sl[b]), S_cap))
        kc[b, n:] = float("nan")
        vc[b, n:] = float("nan")
    return sl, q, kc, vc


def test_noalloc_matches_attn_decode_on_two_calls_second_smaller():
    import causal_head_attention_amd as attn
    cases = [  # seed, B, H, S_cap, D, dtype: the second smaller than the first
        (1701, 16, 32, 4096, 128, torch.bfloat16),
        (1702, 5, 8, 600, 64, torch.float16),
    ]
    for seed, B, H, S_cap, D, dtype in cases:
        print(f"[no-alloc] seed={seed} B={B} H={H} S_cap={S_cap} D={D} {dtype}", flush=True)
        sl, q, kc, vc = _case(seed, B, H, S_cap, D, dtype)
        qd, kd, vd, sd = q.cuda(), kc.cuda(), vc.cuda(), sl.cuda()
        ref = attn.attn_decode(qd, kd, vd, sd)
        o = torch.full_like(qd, float("nan"))
        attn.attn_decode_noalloc(qd, kd, vd, sd, o)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"seed {seed}: differs from attn_decode"
        exact = oracle.attn_decode(q, kc, vc, sl.numpy())
        got = o.float().cpu().double().numpy()
        atol, rell2 = BARS[dtype]
        assert np.abs(got - exact).max() <= atol
        if rell2 is not None:
            assert np.linalg.norm(got - exact) / np.linalg.norm(exact) <= rell2
        assert torch.all(o.cpu()[sl <= 0] == 0)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import causal_head_attention_amd as attn
    B, H, S_cap, D = 1000, 64, 16, 128   # (256 + 999) * 64 records of 536 bytes: 43 MB > 16 MiB
    q = torch.zeros(B, 1, H, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, S_cap, H, D, dtype=torch.bfloat16, device="cuda")
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    with pytest.raises(attn.AttnError) as e:
        attn.attn_decode_noalloc(q, kc, kc, sl, o)
    assert e.value.status == attn.ATTN_ERR_WORKSPACE
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)   # rejected before any launch
