"""Decode step on the GPU (split-KV + log-sum-exp merge) against the fp64 oracle.

Cache rows past each length are NaN on the device, so reading one would show in the result.
Bars as for the forward: fp32 max |o - o_ref| and max |lse - lse_ref| <= 2e-5; bf16 normwise
relative error <= 2e-2 on o and lse.
"""
import numpy as np
import pytest

import oracle
from helpers import BF16_ABS_LSE, BF16_REL, F32_ABS_O, normwise

pytestmark = pytest.mark.gpu


def make(B, Hq, Hkv, Tc, D, lens, seed, bf16):
    import torch
    r = np.random.default_rng(seed)
    x = [r.standard_normal((B, Hq, D)).astype(np.float32),
         r.standard_normal((B, Hkv, Tc, D)).astype(np.float32),
         r.standard_normal((B, Hkv, Tc, D)).astype(np.float32)]
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = [torch.from_numpy(a).to(dt).cuda() for a in x]
    host = [t.float().cpu().numpy().astype(np.float64) for t in dev]  # exactly what the GPU sees
    for b, n in enumerate(lens):
        dev[1][b, :, n:] = float("nan")
        dev[2][b, :, n:] = float("nan")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return dev, host, ln


def run_case(ne, B, Hq, Hkv, Tc, D, lens, bf16, seed=0):
    import torch
    print(f"\n[case] decode B{B} Hq{Hq} Hkv{Hkv} Tc{Tc} D{D} lens={lens} bf16={bf16}", flush=True)
    (q, k, v), (qh, kh, vh), ln = make(B, Hq, Hkv, Tc, D, lens, seed, bf16)
    o, lse = ne.decode(q, k, v, ln)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(qh, kh, vh, lens)
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    empty = np.array(lens) == 0
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0.0)
    full = ~empty
    assert np.isfinite(o[full]).all() and np.isfinite(lse[full]).all()
    if bf16:
        assert normwise(o[full], o_ref[full]) <= BF16_REL
        assert normwise(lse[full], lse_ref[full]) <= BF16_REL
        assert np.abs(lse[full] - lse_ref[full]).max() <= BF16_ABS_LSE
    else:
        assert np.abs(o[full] - o_ref[full]).max() <= F32_ABS_O
        assert np.abs(lse[full] - lse_ref[full]).max() <= F32_ABS_O
    return o, lse


CASES = [
    # B, Hq, Hkv, Tc, D, lens
    (2, 4, 2, 300, 64, [300, 57]),
    (3, 12, 4, 1000, 64, [1, 256, 999]),      # a split boundary, one key
    (2, 8, 1, 513, 32, [513, 255]),           # group of 8
    (2, 6, 2, 700, 32, [0, 700]),             # an empty cache row
    (1, 10, 1, 300, 64, [300]),               # group of 10: chunks of 8 and 2 heads
    (2, 3, 3, 64, 64, [64, 63]),              # no grouping
    (1, 24, 3, 4097, 64, [4097]),             # group of 8, ragged last split
    (2, 8, 2, 600, 128, [600, 300]),          # head size 128 (fp32: 32 lanes per row)
    (1, 16, 2, 1030, 128, [1030]),            # head size 128, group of 8
    # caches of at most 512 keys: one launch, no merge
    (2, 12, 4, 512, 64, [512, 200]),          # 16 waves of 32 keys, groups of 3 (as 4)
    (2, 16, 2, 480, 32, [480, 17]),           # group of 8 at D 32: 16 waves (fp32) or 8 of 64
    (1, 8, 1, 400, 64, [400]),                # group of 8: 8 waves of 64 keys
    (2, 4, 2, 500, 128, [500, 260]),          # head size 128, 16 waves
    (2, 16, 2, 200, 128, [200, 33]),          # head size 128, group of 8, 8 waves of 32 keys
]


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_decode_parity(ne, case, bf16):
    B, Hq, Hkv, Tc, D, lens = case
    run_case(ne, B, Hq, Hkv, Tc, D, lens, bf16)


def test_decode_long_cache(ne):
    """A 32K-token cache, one full row and one at 20,000 keys."""
    run_case(ne, 2, 8, 2, 32768, 64, [32768, 20000], True, seed=1)


def test_decode_is_deterministic(ne):
    import torch
    (q, k, v), _, ln = make(2, 8, 2, 2000, 64, [2000, 1500], 2, True)
    o1, l1 = ne.decode(q, k, v, ln)
    o2, l2 = ne.decode(q, k, v, ln)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
