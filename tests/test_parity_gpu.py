"""HIP path against the fp64 oracle, element by element, through the C ABI.

fp32: max |o - o_ref| <= 2e-5 and max |lse - lse_ref| <= 2e-5; normwise relative error
(max |g - g_ref| / max |g_ref|) <= 1e-4 on dq, dk, dv.
"""
import numpy as np
import pytest

from helpers import assert_f32, errors, gpu_fwd_bwd, oracle_fwd_bwd
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def run_case(ne, oracle_mod, w: Workload, seed=0, causal=None):
    causal = w.causal if causal is None else causal
    x = make_inputs(w, seed)
    print(f"\n[case] {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} T{w.T} D{w.D} causal={causal} seed={seed}",
          flush=True)
    res = gpu_fwd_bwd(ne, x, causal=causal)
    ref = oracle_fwd_bwd(oracle_mod, x, causal=causal)
    e = assert_f32(res, ref, w.name)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in e.items() if k.endswith(("_abs", "_rel"))))
    return res


@pytest.mark.parametrize("name", ["tiny", "cpu_model", "gpu_model", "long_ctx"])
def test_workload_parity(ne, oracle_mod, name):
    run_case(ne, oracle_mod, WORKLOADS[name])


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", ["tiny", "cpu_model", "gpu_model", "long_ctx"])
def test_workload_parity_other_seeds(ne, oracle_mod, name, seed):
    run_case(ne, oracle_mod, WORKLOADS[name], seed=seed)


RAGGED = [
    (1, 4, 2, 1, 32), (1, 3, 1, 17, 64), (2, 4, 4, 37, 32), (1, 6, 2, 65, 64),
    (1, 2, 1, 100, 64), (1, 8, 2, 130, 32), (2, 12, 4, 255, 64), (1, 16, 2, 33, 64),
    (1, 5, 5, 96, 32), (1, 1, 1, 31, 64), (3, 2, 2, 7, 64),
    # group sizes 5..8: work-groups of 5..8 waves
    (1, 10, 2, 77, 64), (1, 6, 1, 100, 64), (1, 7, 1, 90, 32), (1, 8, 1, 200, 64),
    # 256 (batch, kv head) pairs: single-wave fp32 launches with the per-XCD pair sets
    (64, 4, 4, 128, 32),
    # 256 work-groups per tile index: the forward's mirrored tile order with a stride of one row
    (64, 16, 4, 128, 32),
    # head size 128 (work-groups of at most 4 waves, one wave per SIMD)
    (1, 4, 2, 64, 128), (1, 3, 1, 77, 128), (2, 12, 4, 130, 128), (1, 8, 1, 100, 128),
    (1, 2, 2, 33, 128), (1, 16, 2, 257, 128),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda c: "B{}_Hq{}_Hkv{}_T{}_D{}".format(*c))
def test_ragged_and_odd_shapes(ne, oracle_mod, shape, causal):
    B, Hq, Hkv, T, D = shape
    run_case(ne, oracle_mod, Workload("ragged", B, Hq, Hkv, T, D), seed=7, causal=causal)


@pytest.mark.parametrize("name", ["tiny", "cpu_model"])
def test_non_causal_workloads(ne, oracle_mod, name):
    run_case(ne, oracle_mod, WORKLOADS[name], causal=False)


ROPE_CASES = [
    (1, 4, 2, 64, 32, 10000.0), (2, 12, 4, 130, 64, 10000.0), (1, 6, 3, 517, 64, 10000.0),
    (1, 16, 4, 1024, 64, 10000.0), (1, 4, 4, 33, 32, 500.0), (1, 8, 2, 200, 128, 10000.0),
]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", ROPE_CASES)
def test_fp32_fused_rope(ne, oracle_mod, case, causal):
    """fp32 with RoPE applied in-kernel against the oracle's fp64 rotation; dq, dk are gradients
    with respect to the un-rotated q, k."""
    B, Hq, Hkv, T, D, base = case
    w = Workload("rope_f32", B, Hq, Hkv, T, D, rope_base=base)
    x = make_inputs(w, 11)
    print(f"\n[case] rope fp32 {case} causal={causal}", flush=True)
    res = gpu_fwd_bwd(ne, x, causal=causal, rope_base=base)
    ref = oracle_fwd_bwd(oracle_mod, x, causal=causal, rope_base=base)
    assert_f32(res, ref, f"rope {case}")


def test_head_size_128_workload(ne, oracle_mod):
    """The head-size-128 workload at the batch it is timed at (B = 8)."""
    run_case(ne, oracle_mod, WORKLOADS["d128_f32"])


def test_long_sequence_head_size_128(ne, oracle_mod):
    """T = 8192 at D = 128: 256 key tiles streamed per query tile, causal skipping at length."""
    run_case(ne, oracle_mod, Workload("long_d128", 1, 2, 1, 8192, 128), seed=3)


def test_fp32_rope_long_positions(ne, oracle_mod):
    """Positions up to 4095: the angle must be reduced accurately at large t."""
    w = Workload("rope_long", 1, 4, 1, 4096, 64, rope_base=10000.0)
    x = make_inputs(w, 12)
    print("\n[case] rope fp32 T4096", flush=True)
    res = gpu_fwd_bwd(ne, x, causal=True, rope_base=w.rope_base)
    ref = oracle_fwd_bwd(oracle_mod, x, causal=True, rope_base=w.rope_base)
    assert_f32(res, ref, "rope long")
