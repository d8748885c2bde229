"""Seeded random configurations against the fp64 oracle: dtype, head size (32, 64, 128), group
size (1..8), batch, ragged T (1..599), causal or not, RoPE or not, and for fp32 the two-pass or
the single-pass backward.  Same bars as the other parity tests: fp32 max |o - o_ref| and
max |lse - lse_ref| <= 2e-5, normwise <= 1e-4 on the gradients; bf16 normwise <= 2e-2."""
import numpy as np
import pytest

from helpers import BF16_REL, F32_ABS_O, F32_REL_GRAD, normwise, oracle_fwd_bwd
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

N_CASES = 100


def _config(c):
    r = np.random.default_rng(1000 + c)
    D = int(r.choice([32, 64, 128]))
    Hkv = int(r.integers(1, 5))
    G = int(r.choice([1, 2, 3, 4, 5, 6, 8]))
    B = int(r.integers(1, 3))
    T = int(r.integers(1, 600))
    bf16 = bool(r.random() < 0.5)
    causal = bool(r.random() < 0.75)
    rope = 10000.0 if r.random() < 0.4 else 0.0
    fused = (not bf16) and bool(r.random() < 0.4)
    return B, G * Hkv, Hkv, T, D, bf16, causal, rope, fused


@pytest.mark.parametrize("c", range(N_CASES))
def test_random_configuration(ne, oracle_mod, c):
    import torch
    B, Hq, Hkv, T, D, bf16, causal, rope, fused = _config(c)
    print(f"\n[case {c}] B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} bf16={bf16} causal={causal} rope={rope} "
          f"fused={fused}", flush=True)
    w = Workload("random", B, Hq, Hkv, T, D, dtype="bf16" if bf16 else "f32", rope_base=rope)
    x = make_inputs(w, 100 + c)
    dt = torch.bfloat16 if bf16 else torch.float32
    q, k, v, dO = (torch.from_numpy(x[m]).cuda().to(dt).contiguous() for m in ("q", "k", "v", "dO"))
    o, lse = ne.forward(q, k, v, causal=causal, rope_base=rope)
    bwd = ne.backward_fused if fused else ne.backward
    dq, dk, dv = bwd(q, k, v, o, lse, dO, causal=causal, rope_base=rope)
    torch.cuda.synchronize()
    ref = oracle_fwd_bwd(oracle_mod, x, causal=causal, rope_base=rope)
    got = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
    for m, t in got.items():
        a = t.float().cpu().numpy().astype(np.float64)
        if bf16:
            assert normwise(a, ref[m]) <= BF16_REL, (c, m)
        elif m in ("o", "lse"):
            assert np.abs(a - ref[m]).max() <= F32_ABS_O, (c, m)
        else:
            assert normwise(a, ref[m]) <= F32_REL_GRAD, (c, m)
