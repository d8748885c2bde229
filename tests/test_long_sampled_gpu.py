"""The forward at T = 65536, in the launch configuration of the library, checked on sampled rows.

The whole causal forward at this length is out of the oracle's reach, but each output row is a
plain function of one query and the keys up to it: row i equals the oracle's prefill of that one
query (at position i) against keys 0..i.  Sampled rows include the first, the last and both sides
of tile boundaries.  With RoPE the oracle rotates q and k itself (fp64) before attending.
"""
import numpy as np
import pytest

from helpers import BF16_REL, F32_ABS_O, normwise

pytestmark = pytest.mark.gpu

T = 65536
ROWS = [0, 1, 31, 32, 63, 64, 1000, 4095, 4096, 32767, 40000, 65535]


def _inputs(B, Hq, Hkv, D, seed, bf16):
    import torch
    r = np.random.default_rng(seed)
    x = [r.standard_normal((B, Hq, T, D)).astype(np.float32),
         r.standard_normal((B, Hkv, T, D)).astype(np.float32),
         r.standard_normal((B, Hkv, T, D)).astype(np.float32)]
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = [torch.from_numpy(a).cuda().to(dt).contiguous() for a in x]
    return dev, [t.float().cpu().numpy().astype(np.float64) for t in dev]


@pytest.mark.parametrize("bf16,D,rope", [(False, 64, 0.0), (True, 128, 10000.0)])
def test_forward_at_65536_sampled_rows(ne, oracle_mod, bf16, D, rope):
    import torch
    B, Hq, Hkv = 1, 2, 1
    print(f"\n[case] T{T} D{D} bf16={bf16} rope={rope} sampled rows", flush=True)
    (q, k, v), (qh, kh, vh) = _inputs(B, Hq, Hkv, D, 21, bf16)
    o, lse = ne.forward(q, k, v, causal=True, rope_base=rope)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    if rope:
        qh, kh = oracle_mod.rope(qh, rope), oracle_mod.rope(kh, rope)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for i in ROWS:
        ro, rl = oracle_mod.attn_prefill(qh[:, :, i:i + 1], kh[:, :, :i + 1], vh[:, :, :i + 1])
        got_o.append(o[:, :, i])
        got_l.append(lse[:, :, i])
        ref_o.append(ro[:, :, 0])
        ref_l.append(rl[:, :, 0])
    go, gl, ro_, rl_ = (np.stack(a) for a in (got_o, got_l, ref_o, ref_l))
    if bf16:
        assert normwise(go, ro_) <= BF16_REL and normwise(gl, rl_) <= BF16_REL
    else:
        assert np.abs(go - ro_).max() <= F32_ABS_O and np.abs(gl - rl_).max() <= F32_ABS_O
