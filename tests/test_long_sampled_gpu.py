"""The forward at T = 65536, in the launch configuration of the library, checked on sampled rows.

The whole causal forward at this length is out of the oracle's reach, but each output row is a
plain function of one query and the keys up to it: row i equals the oracle's prefill of that one
query (at position i) against keys 0..i.  Sampled rows include the first, the last and both sides
of tile boundaries.  With RoPE the oracle rotates q and k itself (fp64) before attending.
"""
import numpy as np
import pytest

from helpers import BF16_ABS_LSE, BF16_REL, F32_ABS_O, normwise

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
        assert np.abs(gl - rl_).max() <= BF16_ABS_LSE
    else:
        assert np.abs(go - ro_).max() <= F32_ABS_O and np.abs(gl - rl_).max() <= F32_ABS_O


# bf16 + RoPE at a million positions.  RoPE angles grow with the position, so an angle formed
# or reduced in float32 would be off by a sizeable fraction of a radian here.
TL = 1 << 20
ROWS_L = [0, 1, 31, 32, 63, 64, 4095, 65536, 333333, (1 << 19) + 17, TL - 33, TL - 1]


def test_bf16_rope_forward_at_a_million_positions(ne, oracle_mod):
    """Sampled rows of the forward at T = 2^20 against the oracle's prefill of each query on
    keys 0..i, with q and k rotated by the oracle in fp64."""
    import torch
    B, Hq, Hkv, D, base = 1, 1, 1, 64, 10000.0
    print(f"\n[case] T{TL} D{D} bf16 rope={base} sampled rows", flush=True)
    r = np.random.default_rng(23)
    dev = [torch.from_numpy(r.standard_normal((B, H, TL, D), dtype=np.float32)).cuda()
           .to(torch.bfloat16) for H in (Hq, Hkv, Hkv)]
    q, k, v = dev
    o, lse = ne.forward(q, k, v, causal=True, rope_base=base)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    qh, kh, vh = (t.float().cpu().numpy().astype(np.float64) for t in dev)
    qh, kh = oracle_mod.rope(qh, base), oracle_mod.rope(kh, base)
    go, gl, ro_, rl_ = [], [], [], []
    for i in ROWS_L:
        ro, rl = oracle_mod.attn_prefill(qh[:, :, i:i + 1], kh[:, :, :i + 1], vh[:, :, :i + 1])
        go.append(o[:, :, i])
        gl.append(lse[:, :, i])
        ro_.append(ro[:, :, 0])
        rl_.append(rl[:, :, 0])
    go, gl, ro_, rl_ = (np.stack(a) for a in (go, gl, ro_, rl_))
    eo, el = normwise(go, ro_), float(np.abs(gl - rl_).max())
    print(f"  o_rel={eo:.2e} lse_abs={el:.2e}")
    assert eo <= BF16_REL and el <= BF16_ABS_LSE


def test_bf16_rope_backward_at_a_million_positions(ne, oracle_mod):
    """Every row of the forward and backward at T = 2^20 with RoPE in the kernel, against the
    same kernels without RoPE applied to q and k rotated by the oracle (fp64), whose dq and dk
    the oracle then rotates back: both sides share every product and differ only in where the
    rotation happens, so a wrong angle or a wrong inverse at large positions shows at once."""
    import torch
    B, Hq, Hkv, D, base = 1, 2, 1, 64, 10000.0
    print(f"\n[case] T{TL} D{D} bf16 rope={base} fwd+bwd vs pre-rotated inputs", flush=True)
    r = np.random.default_rng(24)
    shapes = ((B, Hq, TL, D), (B, Hkv, TL, D), (B, Hkv, TL, D), (B, Hq, TL, D))
    dev = [torch.from_numpy(r.standard_normal(s, dtype=np.float32)).cuda().to(torch.bfloat16)
           for s in shapes]
    q, k, v, dO = dev
    o, lse = ne.forward(q, k, v, causal=True, rope_base=base)
    dq, dk, dv = ne.backward(q, k, v, o, lse, dO, causal=True, rope_base=base)
    torch.cuda.synchronize()
    qh, kh = (t.float().cpu().numpy().astype(np.float64) for t in (q, k))
    qr = torch.from_numpy(oracle_mod.rope(qh, base)).to(torch.bfloat16).cuda()
    kr = torch.from_numpy(oracle_mod.rope(kh, base)).to(torch.bfloat16).cuda()
    o2, lse2 = ne.forward(qr, kr, v, causal=True)
    dq2, dk2, dv2 = ne.backward(qr, kr, v, o2, lse2, dO, causal=True)
    torch.cuda.synchronize()
    h = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    ref = {"o": h(o2), "lse": h(lse2), "dv": h(dv2),
           "dq": oracle_mod.rope(h(dq2), base, inverse=True),
           "dk": oracle_mod.rope(h(dk2), base, inverse=True)}
    got = {"o": h(o), "lse": h(lse), "dq": h(dq), "dk": h(dk), "dv": h(dv)}
    errs = {n: normwise(got[n], ref[n]) for n in got}
    el = float(np.abs(got["lse"] - ref["lse"]).max())
    print("  " + " ".join(f"{n}_rel={e:.2e}" for n, e in errs.items()) + f" lse_abs={el:.2e}")
    assert all(e <= BF16_REL for e in errs.values()) and el <= BF16_ABS_LSE
