"""Chunked prefill on the GPU (the forward kernels with a query position offset) against the
fp64 oracle.  Bars as for the forward: fp32 max |o - o_ref|, max |lse - lse_ref| <= 2e-5;
bf16 normwise <= 2e-2."""
import numpy as np
import pytest

import oracle
from helpers import BF16_ABS_LSE, BF16_REL, F32_ABS_O, normwise

pytestmark = pytest.mark.gpu


def make(B, Hq, Hkv, Tq, Tk, D, seed, bf16):
    import torch
    r = np.random.default_rng(seed)
    x = [r.standard_normal((B, Hq, Tq, D)).astype(np.float32),
         r.standard_normal((B, Hkv, Tk, D)).astype(np.float32),
         r.standard_normal((B, Hkv, Tk, D)).astype(np.float32)]
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = [torch.from_numpy(a).to(dt).cuda() for a in x]
    return dev, [t.float().cpu().numpy().astype(np.float64) for t in dev]


CASES = [
    # B, Hq, Hkv, Tq, Tk, D
    (2, 4, 2, 37, 100, 64),
    (1, 12, 4, 128, 512, 64),      # gpu-model heads, a 128-token chunk after 384
    (2, 8, 2, 1, 300, 32),         # one query: a decode step
    (1, 6, 3, 64, 64, 64),         # an empty cache: the causal forward
    (1, 8, 1, 77, 333, 32),
    (2, 16, 4, 200, 1000, 64),
    (1, 8, 2, 96, 400, 128),       # head size 128
    (1, 8, 2, 64, 16384, 128),     # a 64-token chunk after 16,320 cached (head size 128)
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_prefill_parity(ne, case, bf16):
    import torch
    B, Hq, Hkv, Tq, Tk, D = case
    print(f"\n[case] prefill B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tk{Tk} D{D} bf16={bf16}", flush=True)
    (q, k, v), (qh, kh, vh) = make(B, Hq, Hkv, Tq, Tk, D, 4, bf16)
    o, lse = ne.prefill(q, k, v)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_prefill(qh, kh, vh)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    if bf16:
        assert normwise(o, o_ref) <= BF16_REL and normwise(lse, lse_ref) <= BF16_REL
        assert np.abs(lse - lse_ref).max() <= BF16_ABS_LSE
    else:
        assert np.abs(o - o_ref).max() <= F32_ABS_O and np.abs(lse - lse_ref).max() <= F32_ABS_O


@pytest.mark.parametrize("bf16", [False, True])
def test_prefill_without_history_is_the_forward(ne, bf16):
    """Tq = Tk runs the forward's own kernel with offset 0: bitwise the causal forward."""
    import torch
    (q, k, v), _ = make(2, 8, 2, 150, 150, 64, 5, bf16)
    o1, l1 = ne.prefill(q, k, v)
    o2, l2 = ne.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
