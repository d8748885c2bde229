"""bf16 path (optional fused RoPE) against the fp64 oracle on the same bf16-rounded inputs.

Bar: normwise relative error max |x - x_ref| / max |x_ref| <= 2e-2 on o, lse, dq, dk, dv.
"""
import numpy as np
import pytest

from helpers import assert_bf16, gpu_fwd_bwd, oracle_fwd_bwd
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def run_bf16(ne, oracle_mod, w, seed=0, causal=True, rope_base=None):
    import torch
    rope_base = w.rope_base if rope_base is None else rope_base
    x = make_inputs(w.with_(dtype="bf16"), seed)
    print(f"\n[case] bf16 {w.name} B{w.B} Hq{w.Hq} Hkv{w.Hkv} T{w.T} D{w.D} causal={causal} "
          f"rope={rope_base} seed={seed}", flush=True)
    res = gpu_fwd_bwd(ne, x, causal=causal, rope_base=rope_base, dtype=torch.bfloat16)
    ref = oracle_fwd_bwd(oracle_mod, x, causal=causal, rope_base=rope_base)
    e = assert_bf16(res, ref, w.name)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in e.items()
                          if k.endswith("_rel") or k == "lse_abs"))
    return res, ref


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bf16_rope_workload(ne, oracle_mod, seed):
    """The full bf16 + RoPE workload (B16 Hq16 Hkv4 T1024 D64, base 10000), three seeds."""
    run_bf16(ne, oracle_mod, WORKLOADS["bf16_rope"], seed=seed)


BF16_CASES = [
    (1, 4, 2, 64, 32), (2, 12, 4, 130, 64), (1, 6, 3, 517, 64), (1, 16, 4, 256, 64),
    (1, 2, 1, 100, 64), (1, 8, 2, 33, 32), (2, 5, 5, 1, 64),
    # group sizes 5..8: 5..8 waves share each staged K/V tile, some copying a piece twice
    (1, 10, 2, 77, 64), (1, 6, 1, 100, 64), (1, 7, 1, 90, 32), (1, 8, 1, 200, 64),
    (1, 7, 1, 130, 64),
    # head size 128: 256-byte rows (their own swizzle), work-groups of at most 4 waves; groups
    # of 4 (four pieces per wave and tile), 2 (eight), 3 (the general copy path) and 1
    (1, 4, 1, 64, 128), (2, 8, 2, 130, 128), (1, 6, 3, 200, 128), (1, 3, 1, 150, 128),
    (1, 2, 2, 77, 128), (1, 8, 1, 257, 128), (1, 4, 4, 1, 128),
]


@pytest.mark.parametrize("rope", [0.0, 10000.0])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", BF16_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_T{}_D{}".format(*c))
def test_bf16_shapes(ne, oracle_mod, shape, causal, rope):
    B, Hq, Hkv, T, D = shape
    run_bf16(ne, oracle_mod, Workload("bf16", B, Hq, Hkv, T, D, dtype="bf16"), seed=5,
             causal=causal, rope_base=rope)


def test_bf16_head_size_128_workload(ne, oracle_mod):
    """The head-size-128 bf16 + RoPE workload at the batch it is timed at (B = 8)."""
    run_bf16(ne, oracle_mod, WORKLOADS["d128_bf16_rope"])


def test_bf16_long_sequence_head_size_128(ne, oracle_mod):
    """T = 8192 at D = 128 with RoPE (positions up to 8191)."""
    run_bf16(ne, oracle_mod, Workload("long_d128", 1, 2, 1, 8192, 128, dtype="bf16",
                                      rope_base=10000.0), seed=3)


def test_bf16_gpu_model_shape(ne, oracle_mod):
    """The GPU-model layer shape (boosted query rows) in bf16 without RoPE."""
    run_bf16(ne, oracle_mod, WORKLOADS["gpu_model"].with_(dtype="bf16"))


def test_bf16_determinism_and_causality(ne):
    import torch
    w = Workload("bf16", 2, 8, 2, 300, 64, dtype="bf16", rope_base=10000.0)
    x = make_inputs(w, 9)
    a = gpu_fwd_bwd(ne, x, rope_base=w.rope_base, dtype=torch.bfloat16)
    b = gpu_fwd_bwd(ne, x, rope_base=w.rope_base, dtype=torch.bfloat16)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
    t = 150
    y = {n: v.copy() for n, v in x.items()}
    r = np.random.default_rng(3)
    for n in y:
        y[n][:, :, t + 1:] = r.standard_normal(y[n][:, :, t + 1:].shape).astype(np.float32)
    c = gpu_fwd_bwd(ne, y, rope_base=w.rope_base, dtype=torch.bfloat16, with_bwd=False)
    assert np.array_equal(a["o"][:, :, :t + 1], c["o"][:, :, :t + 1])
    assert np.array_equal(a["lse"][:, :, :t + 1], c["lse"][:, :, :t + 1])


def _ramp_inputs(B, Hq, Hkv, T, D, peak, seed):
    """Scores that rise (peak > 0) or fall (peak < 0) along the key axis: the keys carry a
    common direction u with weight peak * sqrt(D) * ramp(t), every query has unit weight on u,
    so the score of key t is about peak * ramp(t) plus noise of order one."""
    import torch
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    ramp = np.linspace(0.0, 1.0, T) ** 2
    if peak < 0:
        ramp = ramp[::-1].copy()
    q = 0.3 * rng.standard_normal((B, Hq, T, D)) + u
    k = 0.3 * rng.standard_normal((B, Hkv, T, D)) + abs(peak) * np.sqrt(D) * ramp[None, None, :, None] * u
    v = rng.standard_normal((B, Hkv, T, D))
    dO = rng.standard_normal((B, Hq, T, D))
    rnd = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    return {"q": rnd(q), "k": rnd(k), "v": rnd(v), "dO": rnd(dO)}


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("peak", [20.0, 200.0, 4000.0, -200.0])
def test_bf16_scores_growing_along_keys(ne, oracle_mod, peak, causal):
    """Row maxima that jump far above those of the first key tile (by 2^5 to past the fp32
    exponent range in base-2 units) or only fall: the forward's reference maximum has to move,
    or never does.  Forward only: with keys this large, dq = sum dS k cancels terms far larger
    than itself, which a bf16 dS cannot resolve to the bar whatever the forward does."""
    import torch
    x = _ramp_inputs(1, 4, 2, 300, 64, peak, seed=11)
    print(f"\n[case] bf16 ramp peak={peak} causal={causal} B1 Hq4 Hkv2 T300 D64", flush=True)
    res = gpu_fwd_bwd(ne, x, causal=causal, dtype=torch.bfloat16, with_bwd=False)
    ref = oracle_fwd_bwd(oracle_mod, x, causal=causal, with_bwd=False)
    e = assert_bf16(res, ref, f"ramp {peak}")
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in e.items() if k.endswith("_rel")))
