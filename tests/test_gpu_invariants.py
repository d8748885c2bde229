"""Properties of the HIP path that hold at any size, checked without the oracle."""
import math

import numpy as np
import pytest

from helpers import gpu_fwd_bwd, normwise
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def qkvd(B, Hq, Hkv, T, D, seed):
    return {"q": rnd((B, Hq, T, D), seed), "k": rnd((B, Hkv, T, D), seed + 1),
            "v": rnd((B, Hkv, T, D), seed + 2), "dO": rnd((B, Hq, T, D), seed + 3)}


@pytest.mark.parametrize("name", ["gpu_model", "cpu_model"])
def test_bitwise_determinism(ne, name):
    """No atomics anywhere: two runs give identical bits."""
    x = make_inputs(WORKLOADS[name], 0)
    print(f"\n[case] determinism {name}", flush=True)
    a = gpu_fwd_bwd(ne, x)
    b = gpu_fwd_bwd(ne, x)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("t", [63, 200, 255])
def test_causality_is_bitwise(ne, t, bf16):
    """Changing q, k, v, dO at positions > t leaves o and lse at positions <= t bit-identical
    (masked probabilities are exactly 0, and a row's running maximum depends on its own scores
    only); changing queries and dO at positions < 32*floor(t/32) leaves dk, dv at keys
    >= 32*floor(t/32) bit-identical."""
    import torch
    dt = torch.bfloat16 if bf16 else torch.float32
    B, Hq, Hkv, T, D = 2, 6, 2, 300, 64
    x = qkvd(B, Hq, Hkv, T, D, 40)
    y = {n: a.copy() for n, a in x.items()}
    r = np.random.default_rng(41)
    for n in y:
        y[n][:, :, t + 1:] = r.standard_normal(y[n][:, :, t + 1:].shape)
    # rows that make the running maximum move late: boosted queries after row t
    y["q"][:, :, t + 1::7] *= 6.0
    print(f"\n[case] causality t={t} bf16={bf16}", flush=True)
    a = gpu_fwd_bwd(ne, x, with_bwd=False, dtype=dt)
    b = gpu_fwd_bwd(ne, y, with_bwd=False, dtype=dt)
    assert np.array_equal(a["o"][:, :, :t + 1], b["o"][:, :, :t + 1])
    assert np.array_equal(a["lse"][:, :, :t + 1], b["lse"][:, :, :t + 1])
    assert not np.array_equal(a["o"][:, :, t + 1:], b["o"][:, :, t + 1:])
    tb = 32 * (t // 32)
    z = {n: a_.copy() for n, a_ in x.items()}
    z["q"][:, :, :tb] = r.standard_normal(z["q"][:, :, :tb].shape)
    z["dO"][:, :, :tb] = r.standard_normal(z["dO"][:, :, :tb].shape)
    ga = gpu_fwd_bwd(ne, x, dtype=dt)
    gz = gpu_fwd_bwd(ne, z, dtype=dt)
    assert np.array_equal(ga["dk"][:, :, tb:], gz["dk"][:, :, tb:])
    assert np.array_equal(ga["dv"][:, :, tb:], gz["dv"][:, :, tb:])


def test_zero_queries_give_prefix_means(ne):
    B, Hq, Hkv, T, D = 1, 8, 2, 257, 64
    x = qkvd(B, Hq, Hkv, T, D, 50)
    x["q"][:] = 0
    print("\n[case] q=0", flush=True)
    res = gpu_fwd_bwd(ne, x, with_bwd=False)
    G = Hq // Hkv
    n = np.arange(1, T + 1)
    for h in range(Hq):
        pm = np.cumsum(x["v"][:, h // G].astype(np.float64), axis=1) / n[None, :, None]
        assert np.abs(res["o"][:, h] - pm).max() < 2e-5
        assert np.abs(res["lse"][:, h] - np.log(n)[None]).max() < 2e-5


@pytest.mark.parametrize("causal", [True, False])
def test_single_position(ne, causal):
    """T = 1: o = v_0 exactly, lse = q.k/sqrt(D), dq = dk = 0, dv = sum of dO over the group."""
    B, Hq, Hkv, D = 3, 12, 4, 64
    x = qkvd(B, Hq, Hkv, 1, D, 60)
    print("\n[case] T=1", flush=True)
    res = gpu_fwd_bwd(ne, x, causal=causal)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        assert np.array_equal(res["o"][:, h, 0], x["v"][:, g, 0].astype(np.float64))
        s = (x["q"][:, h, 0].astype(np.float64) * x["k"][:, g, 0]).sum(-1) / math.sqrt(D)
        assert np.abs(res["lse"][:, h, 0] - s).max() < 2e-5
    assert np.abs(res["dq"]).max() < 1e-5 and np.abs(res["dk"]).max() < 1e-5
    ref = x["dO"].astype(np.float64).reshape(B, Hkv, G, 1, D).sum(2)
    assert np.abs(res["dv"] - ref).max() < 1e-5


def test_constant_values(ne):
    """v_j = c: o_i = c and dq = dk = 0 up to rounding."""
    B, Hq, Hkv, T, D = 2, 6, 3, 190, 64
    x = qkvd(B, Hq, Hkv, T, D, 70)
    c = rnd((D,), 71)
    x["v"][:] = c
    print("\n[case] constant v", flush=True)
    res = gpu_fwd_bwd(ne, x)
    assert np.abs(res["o"] - c).max() < 1e-5
    scale = np.abs(x["dO"]).max() * np.abs(x["k"]).max()
    assert np.abs(res["dq"]).max() < 1e-5 * scale
    assert np.abs(res["dk"]).max() < 1e-5 * scale * T


@pytest.mark.parametrize("causal", [True, False])
def test_gradient_sum_identities(ne, causal):
    """Without RoPE: sum_j dk_j = 0 and sum_j dv_j = sum over the group and all i of dO_i."""
    B, Hq, Hkv, T, D = 2, 12, 4, 200, 64
    x = qkvd(B, Hq, Hkv, T, D, 80)
    print(f"\n[case] gradient sums causal={causal}", flush=True)
    res = gpu_fwd_bwd(ne, x, causal=causal)
    G = Hq // Hkv
    dk_scale = np.abs(res["dk"]).max()
    assert np.abs(res["dk"].sum(2)).max() < 1e-4 * dk_scale * math.sqrt(T)
    ref = x["dO"].astype(np.float64).reshape(B, Hkv, G, T, D).sum((2, 3))
    assert normwise(res["dv"].sum(2), ref) < 1e-5


def test_gqa_matches_mha_on_repeated_kv(ne):
    B, Hq, Hkv, T, D = 2, 12, 4, 160, 64
    x = qkvd(B, Hq, Hkv, T, D, 90)
    G = Hq // Hkv
    y = dict(x, k=np.repeat(x["k"], G, axis=1), v=np.repeat(x["v"], G, axis=1))
    print("\n[case] gqa vs mha", flush=True)
    a = gpu_fwd_bwd(ne, x)
    b = gpu_fwd_bwd(ne, y)
    assert np.abs(a["o"] - b["o"]).max() < 1e-5
    assert np.abs(a["lse"] - b["lse"]).max() < 1e-5
    assert normwise(a["dq"], b["dq"]) < 1e-5
    assert normwise(a["dk"], b["dk"].reshape(B, Hkv, G, T, D).sum(2)) < 1e-5
    assert normwise(a["dv"], b["dv"].reshape(B, Hkv, G, T, D).sum(2)) < 1e-5


def test_key_shift_invariance(ne):
    """k_j -> k_j + u: o unchanged, lse_i increases by q_i.u/sqrt(D); large u stresses the
    running maximum."""
    B, Hq, Hkv, T, D = 1, 8, 2, 300, 64
    x = qkvd(B, Hq, Hkv, T, D, 100)
    u = 3.0 * rnd((D,), 101)
    y = dict(x, k=(x["k"] + u).astype(np.float32))
    print("\n[case] key shift", flush=True)
    a = gpu_fwd_bwd(ne, x, with_bwd=False)
    b = gpu_fwd_bwd(ne, y, with_bwd=False)
    assert np.abs(a["o"] - b["o"]).max() < 1e-4
    shift = (x["q"].astype(np.float64) @ u.astype(np.float64)) / math.sqrt(D)
    assert np.abs(b["lse"] - a["lse"] - shift).max() < 1e-3


def test_rope_single_position_is_identity(ne):
    """Position 0 is not rotated, so with T = 1 RoPE changes nothing."""
    x = qkvd(2, 8, 2, 1, 64, 110)
    print("\n[case] rope T=1", flush=True)
    a = gpu_fwd_bwd(ne, x, rope_base=10000.0)
    b = gpu_fwd_bwd(ne, x)
    for n in a:
        assert np.abs(a[n] - b[n]).max() < 1e-6, n


@pytest.mark.parametrize("dtype_name,rope", [("float32", 0.0), ("float32", 10000.0),
                                             ("bfloat16", 0.0), ("bfloat16", 10000.0)])
def test_split_backward_passes_match_combined(ne, dtype_name, rope):
    """ne_attn_bwd_dq_ex then ne_attn_bwd_dkdv_ex on one workspace (what the benchmark times)
    give the same bits as ne_attn_bwd_ex; the forward with an explicit workspace matches the
    convenience wrapper."""
    import torch
    dt = getattr(torch, dtype_name)
    x = qkvd(2, 8, 2, 300, 64, 120)
    q, k, v, dO = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v", "dO"))
    print(f"\n[case] split passes {dtype_name} rope={rope}", flush=True)
    ws = ne.workspace(q, k, rope)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ne.ne_attn_fwd_ex(q, k, v, o, lse, ws, rope_base=rope)
    o2, lse2 = ne.forward(q, k, v, rope_base=rope)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ne.ne_attn_bwd_dq_ex(q, k, v, o, lse, dO, dq, ws, rope_base=rope)
    ne.ne_attn_bwd_dkdv_ex(q, k, v, lse, dO, ws, dk, dv, rope_base=rope)
    dq2, dk2, dv2 = ne.backward(q, k, v, o, lse, dO, rope_base=rope)
    torch.cuda.synchronize()
    for a_, b_ in ((o, o2), (lse, lse2), (dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a_, b_)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conveniences_allocate_on_the_kernel_stream(ne, dtype):
    """backward(..., stream=s) with s not made current: its workspace (dropped when the call
    returns) and its outputs come from s's memory, so the default stream can take and overwrite
    memory while the kernels on s still run without touching what they read or write."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, Hq, Hkv, T, D, base = 2, 8, 2, 2048, 64, 10000.0
    x = qkvd(B, Hq, Hkv, T, D, 60)
    q, k, v, dO = (torch.from_numpy(x[n]).cuda().to(tdt) for n in ("q", "k", "v", "dO"))
    print(f"\n[case] conveniences on a side stream {dtype}", flush=True)
    o, lse = ne.forward(q, k, v, rope_base=base)
    ref = ne.backward(q, k, v, o, lse, dO, rope_base=base)
    torch.cuda.synchronize()
    nws = ne.ne_attn_workspace_bytes(B, Hq, Hkv, T, D, ne.NE_BF16 if dtype == "bf16" else ne.NE_F32,
                                     base)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        got = ne.backward(q, k, v, o, lse, dO, rope_base=base, stream=s)
        # the default stream takes blocks of the workspace's and the outputs' sizes and fills
        # them with NaN while the backward may still be running on s
        junk = [torch.full((nws,), 255, dtype=torch.uint8, device="cuda")]
        junk += [torch.full_like(t, float("nan")) for t in got]
        s.synchronize()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
        del junk
