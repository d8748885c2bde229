"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test fixes the oracle to something other than itself: a pure-Python brute force, the
library's fp64 scaled-dot-product attention with autograd, central finite differences in
double precision (the check the NanoEuler pages apply to every hand-written backward pass:
README translations, section "Verifying the backward pass"), closed forms and invariants.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, round_to_bf16

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def qkv(B, Hq, Hkv, T, D, seed=0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, T, D)), r.standard_normal((B, Hkv, T, D)),
            r.standard_normal((B, Hkv, T, D)), r.standard_normal((B, Hq, T, D)))


# ---------------------------------------------------------------- brute force (pure Python)

def brute_fwd(q, k, v, causal):
    """Triple loop over plain Python floats, written from the definition of softmax attention."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = [[[[0.0] * D for _ in range(T)] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(T):
                keys = range(i + 1) if causal else range(T)
                sc = []
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, h, i, d]) * float(k[b, g, j, d])
                    sc.append(acc / math.sqrt(D))
                z = sum(math.exp(x) for x in sc)
                lse[b][h][i] = math.log(z)
                for d in range(D):
                    o[b][h][i][d] = sum(math.exp(x) / z * float(v[b, g, j, d])
                                        for x, j in zip(sc, keys))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(1, 4, 2, 7, 4), (2, 3, 1, 5, 2), (1, 2, 2, 1, 3)])
def test_brute_force_fwd(shape, causal):
    q, k, v, _ = qkv(*shape, seed=11)
    o, lse = oracle.attn_fwd(q, k, v, causal=causal)
    ob, lb = brute_fwd(q, k, v, causal)
    assert np.abs(o - ob).max() < 1e-13
    assert np.abs(lse - lb).max() < 1e-13


# ---------------------------------------------------------------- library routine (torch fp64)

def torch_reference(q, k, v, dO, causal):
    G = q.shape[1] // k.shape[1]
    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kr = kt.repeat_interleave(G, dim=1)
    vr = vt.repeat_interleave(G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, is_causal=causal)
    o.backward(torch.tensor(dO, dtype=torch.float64))
    T, D = q.shape[2], q.shape[3]
    s = (qt.detach() @ kr.detach().transpose(-1, -2)) / math.sqrt(D)
    if causal:
        mask = torch.ones(T, T, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return (o.detach().numpy(), lse.numpy(), qt.grad.numpy(), kt.grad.numpy(),
            vt.grad.numpy())


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(2, 4, 2, 33, 16), (1, 12, 4, 70, 64), (1, 4, 2, 40, 128),
                                   (1, 3, 3, 9, 8),
                                   (1, 8, 1, 17, 32)])
def test_against_torch_sdpa_fp64(shape, causal):
    q, k, v, dO = qkv(*shape, seed=3)
    ro, rl, rdq, rdk, rdv = torch_reference(q, k, v, dO, causal)
    o, lse = oracle.attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dO, causal=causal)
    for a, r in ((o, ro), (lse, rl), (dq, rdq), (dk, rdk), (dv, rdv)):
        assert np.abs(a - r).max() <= 1e-12 * max(1.0, np.abs(r).max())


# ---------------------------------------------------------------- finite differences in fp64

def fd_check(q, k, v, dO, causal, rope_base, elems=None, h=1e-6):
    """Central differences of L = sum(dO * o) against the oracle's analytic gradient.

    Returns the normwise relative error max|fd - an| / max|an| over the checked elements."""
    dq, dk, dv = oracle.attn_bwd(q, k, v, dO, causal=causal, rope_base=rope_base)
    ins = {"q": q, "k": k, "v": v}
    ans = {"q": dq, "k": dk, "v": dv}
    worst = 0.0
    for name in ("q", "k", "v"):
        x = ins[name]
        idx = range(x.size) if elems is None else elems(x.size)
        fd = []
        an = []
        for flat in idx:
            pos = np.unravel_index(flat, x.shape)
            xp = x.copy()
            xm = x.copy()
            xp[pos] += h
            xm[pos] -= h
            args_p = dict(ins, **{name: xp})
            args_m = dict(ins, **{name: xm})
            op, _ = oracle.attn_fwd(args_p["q"], args_p["k"], args_p["v"], causal=causal,
                                    rope_base=rope_base)
            om, _ = oracle.attn_fwd(args_m["q"], args_m["k"], args_m["v"], causal=causal,
                                    rope_base=rope_base)
            fd.append(((op - om) * dO).sum() / (2 * h))
            an.append(ans[name][pos])
        fd = np.array(fd)
        an = np.array(an)
        worst = max(worst, np.abs(fd - an).max() / np.abs(an).max())
    return worst


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("rope_base", [0.0, 10000.0, 7.0])
def test_finite_differences_all_elements(causal, rope_base):
    q, k, v, dO = qkv(1, 4, 2, 6, 4, seed=5)
    assert fd_check(q, k, v, dO, causal, rope_base) < 1e-7


def test_finite_differences_sampled_tiny_workload():
    w = WORKLOADS["tiny"]
    x = make_inputs(w, seed=0)
    rng = np.random.default_rng(9)
    err = fd_check(x["q"].astype(np.float64), x["k"].astype(np.float64),
                   x["v"].astype(np.float64), x["dO"].astype(np.float64), True, 0.0,
                   elems=lambda n: rng.choice(n, 12, replace=False), h=1e-5)
    assert err < 1e-6


def test_finite_differences_rope_sampled():
    q, k, v, dO = qkv(1, 4, 1, 24, 8, seed=6)
    rng = np.random.default_rng(1)
    err = fd_check(q, k, v, dO, True, 10000.0,
                   elems=lambda n: rng.choice(n, 16, replace=False), h=1e-5)
    assert err < 1e-6


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [True, False])
def test_single_position(causal):
    """T = 1: o = v_0, lse = q.k/sqrt(D), dq = dk = 0, dv = sum of dO over the group."""
    B, Hq, Hkv, D = 2, 6, 2, 8
    q, k, v, dO = qkv(B, Hq, Hkv, 1, D, seed=2)
    o, lse = oracle.attn_fwd(q, k, v, causal=causal)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dO, causal=causal)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        assert np.array_equal(o[:, h, 0], v[:, g, 0] * 1.0) or \
            np.abs(o[:, h, 0] - v[:, g, 0]).max() < 1e-15
        ref = (q[:, h, 0] * k[:, g, 0]).sum(-1) / math.sqrt(D)
        assert np.abs(lse[:, h, 0] - ref).max() < 1e-14
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    for g in range(Hkv):
        ref = dO[:, g * G:(g + 1) * G, 0].sum(1)
        assert np.abs(dv[:, g, 0] - ref).max() < 1e-14


def test_zero_queries_give_prefix_means():
    """q = 0 makes every allowed score 0: P_ij = 1/(i+1), o_i = mean(v_0..v_i),
    lse_i = ln(i+1).  Fixes the diagonal as visible and the natural log of the statistic."""
    B, Hq, Hkv, T, D = 1, 4, 2, 40, 16
    _, k, v, _ = qkv(B, Hq, Hkv, T, D, seed=4)
    q = np.zeros((B, Hq, T, D))
    o, lse = oracle.attn_fwd(q, k, v, causal=True)
    G = Hq // Hkv
    for h in range(Hq):
        pm = np.cumsum(v[:, h // G], axis=1) / np.arange(1, T + 1)[None, :, None]
        assert np.abs(o[:, h] - pm).max() < 1e-13
        assert np.abs(lse[:, h] - np.log(np.arange(1, T + 1))[None]).max() < 1e-13
    o_nc, lse_nc = oracle.attn_fwd(q, k, v, causal=False)
    assert np.abs(lse_nc - math.log(T)).max() < 1e-13
    assert np.abs(o_nc[:, 0] - v[:, 0].mean(axis=1, keepdims=True)).max() < 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_rows_sum_to_one(causal):
    B, Hq, Hkv, T, D = 2, 6, 3, 29, 8
    q, k, v, _ = qkv(B, Hq, Hkv, T, D, seed=8)
    _, lse = oracle.attn_fwd(q, k, v, causal=causal)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            s = q[b, h] @ k[b, h // G].T / math.sqrt(D)
            if causal:
                s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
            tot = np.exp(s - lse[b, h][:, None]).sum(-1)
            assert np.abs(tot - 1).max() < 1e-13


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
def test_causality(rope_base):
    """Changing q, k, v, dO at positions > t leaves o, lse at positions <= t unchanged, and
    dk, dv at position j depend only on queries at positions >= j."""
    B, Hq, Hkv, T, D = 1, 4, 2, 24, 8
    q, k, v, dO = qkv(B, Hq, Hkv, T, D, seed=12)
    t = 9
    q2, k2, v2, dO2 = (x.copy() for x in (q, k, v, dO))
    r = np.random.default_rng(13)
    for x in (q2, k2, v2, dO2):
        x[:, :, t + 1:] = r.standard_normal(x[:, :, t + 1:].shape)
    o, lse = oracle.attn_fwd(q, k, v, causal=True, rope_base=rope_base)
    o2, lse2 = oracle.attn_fwd(q2, k2, v2, causal=True, rope_base=rope_base)
    assert np.array_equal(o[:, :, :t + 1], o2[:, :, :t + 1])
    assert np.array_equal(lse[:, :, :t + 1], lse2[:, :, :t + 1])
    assert not np.array_equal(o[:, :, t + 1:], o2[:, :, t + 1:])
    # dk/dv at key j only gathers queries i >= j: changing queries/dO before j leaves them.
    q3, dO3 = q.copy(), dO.copy()
    q3[:, :, :t] = r.standard_normal(q3[:, :, :t].shape)
    dO3[:, :, :t] = r.standard_normal(dO3[:, :, :t].shape)
    _, dk, dv = oracle.attn_bwd(q, k, v, dO, causal=True, rope_base=rope_base)
    _, dk3, dv3 = oracle.attn_bwd(q3, k, v, dO3, causal=True, rope_base=rope_base)
    assert np.abs(dk[:, :, t:] - dk3[:, :, t:]).max() < 1e-13
    assert np.abs(dv[:, :, t:] - dv3[:, :, t:]).max() < 1e-13
    assert np.abs(dv[:, :, :t] - dv3[:, :, :t]).max() > 1e-3


@pytest.mark.parametrize("causal", [True, False])
def test_constant_values(causal):
    """v_j = c for all j: o_i = c; and then dP_ij = dO_i.c does not depend on j, so dS = 0 and
    dq = dk = 0."""
    B, Hq, Hkv, T, D = 1, 4, 2, 20, 8
    q, k, _, dO = qkv(B, Hq, Hkv, T, D, seed=14)
    c = np.random.default_rng(15).standard_normal(D)
    v = np.broadcast_to(c, (B, Hkv, T, D)).copy()
    o, _ = oracle.attn_fwd(q, k, v, causal=causal)
    assert np.abs(o - c).max() < 1e-13
    dq, dk, _ = oracle.attn_bwd(q, k, v, dO, causal=causal)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13


@pytest.mark.parametrize("causal", [True, False])
def test_gradient_sum_identities(causal):
    """Without RoPE: sum_j dk_j = 0 (softmax rows are shift invariant) and
    sum_j dv_j = sum over the group's heads and all i of dO_i (rows of P sum to one)."""
    B, Hq, Hkv, T, D = 2, 6, 2, 31, 8
    q, k, v, dO = qkv(B, Hq, Hkv, T, D, seed=16)
    _, dk, dv = oracle.attn_bwd(q, k, v, dO, causal=causal)
    G = Hq // Hkv
    assert np.abs(dk.sum(2)).max() < 1e-12
    ref = dO.reshape(B, Hkv, G, T, D).sum((2, 3))
    assert np.abs(dv.sum(2) - ref).max() < 1e-12


def test_gqa_equals_mha_on_repeated_kv():
    B, Hq, Hkv, T, D = 2, 6, 2, 19, 8
    q, k, v, dO = qkv(B, Hq, Hkv, T, D, seed=17)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o, lse = oracle.attn_fwd(q, k, v)
    om, lsem = oracle.attn_fwd(q, kr, vr)
    assert np.abs(o - om).max() < 1e-14 and np.abs(lse - lsem).max() < 1e-14
    dq, dk, dv = oracle.attn_bwd(q, k, v, dO)
    dqm, dkm, dvm = oracle.attn_bwd(q, kr, vr, dO)
    assert np.abs(dq - dqm).max() < 1e-13
    assert np.abs(dk - dkm.reshape(B, Hkv, G, T, D).sum(2)).max() < 1e-13
    assert np.abs(dv - dvm.reshape(B, Hkv, G, T, D).sum(2)).max() < 1e-13


def test_key_shift_invariance():
    """k_j -> k_j + u for all j leaves o unchanged and adds q_i.u/sqrt(D) to lse_i; with
    large shifts this exercises the running maximum."""
    B, Hq, Hkv, T, D = 1, 4, 2, 33, 8
    q, k, v, _ = qkv(B, Hq, Hkv, T, D, seed=18)
    u = 5.0 * np.random.default_rng(19).standard_normal(D)
    o, lse = oracle.attn_fwd(q, k, v)
    o2, lse2 = oracle.attn_fwd(q, k + u, v)
    assert np.abs(o - o2).max() < 1e-11
    assert np.abs(lse2 - lse - (q @ u) / math.sqrt(D)).max() < 1e-11


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity_and_norm_preserving():
    x = rand((2, 3, 17, 8), 20)
    for pairing in (0, 1):
        y = oracle.rope(x, 10000.0, pairing)
        assert np.array_equal(y[:, :, 0], x[:, :, 0])
        assert np.abs(np.linalg.norm(y, axis=-1) - np.linalg.norm(x, axis=-1)).max() < 1e-13
        back = oracle.rope(y, 10000.0, pairing, inverse=True)
        assert np.abs(back - x).max() < 1e-14


def test_rope_closed_form_angles():
    """One unit vector in the first slot of every pair for q, in the second slot for k:
    q'_i . k'_j = sum_p sin((i - j) theta_p), theta_p = base^(-2p/D).  Interleaved pairs
    (2p, 2p+1); with D = 4 and base 10000 the frequencies are 1 and 1/100."""
    T, D, base = 12, 4, 10000.0
    q = np.zeros((1, 1, T, D))
    k = np.zeros((1, 1, T, D))
    q[..., 0::2] = 1.0
    k[..., 1::2] = 1.0
    qr = oracle.rope(q, base)[0, 0]
    kr = oracle.rope(k, base)[0, 0]
    s = qr @ kr.T
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    ref = np.sin(i - j) + np.sin((i - j) / 100.0)
    assert np.abs(s - ref).max() < 1e-13


def test_rope_half_split_pairing_closed_form():
    T, D, base = 10, 4, 10000.0
    q = np.zeros((1, 1, T, D))
    k = np.zeros((1, 1, T, D))
    q[..., 0] = 1.0   # pair (0, 2), first slot
    k[..., 2] = 1.0   # pair (0, 2), second slot
    s = oracle.rope(q, base, 1)[0, 0] @ oracle.rope(k, base, 1)[0, 0].T
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    assert np.abs(s - np.sin(i - j)).max() < 1e-13


def test_rope_single_position_matches_no_rope():
    q, k, v, dO = qkv(2, 4, 2, 1, 8, seed=21)
    a = oracle.attn_fwd(q, k, v, rope_base=10000.0)
    b = oracle.attn_fwd(q, k, v)
    assert np.abs(a[0] - b[0]).max() < 1e-15 and np.abs(a[1] - b[1]).max() < 1e-15


def test_rope_attention_is_relative():
    """With the same q vector at every position and the same k vector at every position,
    rotated scores depend on i - j only: every diagonal of the score matrix is constant."""
    T, D, base = 16, 8, 10000.0
    r = np.random.default_rng(22)
    q = np.broadcast_to(r.standard_normal(D), (1, 1, T, D)).copy()
    k = np.broadcast_to(r.standard_normal(D), (1, 1, T, D)).copy()
    qr = oracle.rope(q, base)[0, 0]
    kr = oracle.rope(k, base)[0, 0]
    s = qr @ kr.T
    for dlt in range(-T + 1, T):
        diag = np.diagonal(s, offset=-dlt)
        assert np.ptp(diag) < 1e-12


# ---------------------------------------------------------------- input generator

def test_bf16_rounding_is_exact_and_ties_to_even():
    x = np.array([1.0, 1.00390625, 1.01171875, 3.0e-39, -2.5, 65504.0], dtype=np.float32)
    y = round_to_bf16(x)
    assert np.array_equal(y, torch.tensor(x).to(torch.bfloat16).float().numpy())
    z = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    assert np.array_equal(round_to_bf16(z), torch.tensor(z).to(torch.bfloat16).float().numpy())


def test_boosted_rows_count():
    w = WORKLOADS["gpu_model"].with_(B=1, T=64)
    x = make_inputs(w, seed=0)
    base = make_inputs(w.with_(boost_frac=0.0), seed=0)
    rows = np.abs(x["q"] - base["q"]).reshape(-1, w.D).max(-1) > 0
    assert rows.sum() == round(0.1 * w.B * w.Hq * w.T)
