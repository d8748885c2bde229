"""Single-pass backward (ne_attn_bwd_fused: dq added with fp32 atomics) against the fp64 oracle,
with and without RoPE.

Same bar as the two-pass backward: normwise relative error max |g - g_ref| / max |g_ref| <= 1e-4
on dq, dk, dv.  dk and dv are bitwise reproducible; dq is not (atomic order) and is compared
run to run within the same tolerance.
"""
import numpy as np
import pytest

from helpers import F32_REL_GRAD, normwise, oracle_fwd_bwd
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def run_fused(ne, oracle_mod, w, seed=0, causal=True):
    import torch
    x = make_inputs(w, seed)
    rb = w.rope_base
    print(f"\n[case] fused bwd {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} T{w.T} D{w.D} "
          f"causal={causal} rope={rb} seed={seed}", flush=True)
    q, k, v, dO = (torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v", "dO"))
    o, lse = ne.forward(q, k, v, causal=causal, rope_base=rb)
    dq, dk, dv = ne.backward_fused(q, k, v, o, lse, dO, causal=causal, rope_base=rb)
    torch.cuda.synchronize()
    ref = oracle_fwd_bwd(oracle_mod, x, causal=causal, rope_base=rb)
    got = {"dq": dq, "dk": dk, "dv": dv}
    for n in ("dq", "dk", "dv"):
        e = normwise(got[n].cpu().double().numpy(), ref[n])
        print(f"  {n}_rel={e:.2e}")
        assert e <= F32_REL_GRAD, (w.name, n, e)
    return q, k, v, o, lse, dO, got


@pytest.mark.parametrize("name", ["tiny", "cpu_model", "gpu_model"])
def test_fused_workloads(ne, oracle_mod, name):
    run_fused(ne, oracle_mod, WORKLOADS[name])


SHAPES = [
    (1, 4, 2, 1, 32), (1, 3, 1, 17, 64), (2, 4, 4, 37, 32), (1, 6, 2, 65, 64),
    (2, 12, 4, 255, 64), (1, 16, 2, 33, 64), (1, 5, 5, 96, 32), (1, 8, 1, 200, 64),
    (1, 10, 2, 77, 64), (3, 2, 2, 7, 64),
    # head size 128: one work-group (four waves, one per SIMD) per compute unit
    (1, 4, 2, 64, 128), (2, 12, 4, 130, 128), (1, 8, 1, 257, 128),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda c: "B{}_Hq{}_Hkv{}_T{}_D{}".format(*c))
def test_fused_shapes(ne, oracle_mod, shape, causal):
    B, Hq, Hkv, T, D = shape
    run_fused(ne, oracle_mod, Workload("fused", B, Hq, Hkv, T, D), seed=7, causal=causal)


ROPE_SHAPES = [(1, 4, 2, 64, 32), (2, 12, 4, 130, 64), (1, 6, 3, 517, 64), (1, 8, 1, 1024, 64),
               (1, 8, 2, 200, 128)]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", ROPE_SHAPES, ids=lambda c: "B{}_Hq{}_Hkv{}_T{}_D{}".format(*c))
def test_fused_rope(ne, oracle_mod, shape, causal):
    """RoPE (base 10000): dq summed in the rotated frame, then rotated back."""
    B, Hq, Hkv, T, D = shape
    run_fused(ne, oracle_mod, Workload("fused_rope", B, Hq, Hkv, T, D, rope_base=10000.0),
              seed=11, causal=causal)


def test_fused_head_size_128_workload(ne, oracle_mod):
    """The head-size-128 workload at a reduced batch (the oracle's cost)."""
    run_fused(ne, oracle_mod, WORKLOADS["d128_f32"].with_(B=1))


def test_fused_matches_two_pass_and_dkdv_is_reproducible(ne, oracle_mod):
    import torch
    q, k, v, o, lse, dO, a = run_fused(ne, oracle_mod, Workload("fused", 2, 8, 2, 300, 64), seed=9)
    dq2, dk2, dv2 = ne.backward_fused(q, k, v, o, lse, dO)
    dq3, dk3, dv3 = ne.backward(q, k, v, o, lse, dO)
    torch.cuda.synchronize()
    assert torch.equal(a["dk"], dk2) and torch.equal(a["dv"], dv2)
    for x, y in ((a["dq"], dq2), (a["dq"], dq3), (a["dk"], dk3), (a["dv"], dv3)):
        assert normwise(x.cpu().double().numpy(), y.cpu().double().numpy()) <= 1e-5
