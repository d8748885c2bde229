"""Pins for the oracle's decode step and chunked prefill against a key/value cache.

Decode is the last row of causal attention over a sequence that ends with the new query, and a
prefill chunk its last rows, so both are pinned to the causal oracle (itself pinned by brute
force, the library's fp64 attention and finite differences) and to closed forms.
"""
import math

import numpy as np
import pytest

import oracle


def cache(B, Hq, Hkv, Tc, D, lens, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, D))
    k = r.standard_normal((B, Hkv, Tc, D))
    v = r.standard_normal((B, Hkv, Tc, D))
    for b, n in enumerate(lens):  # entries past the length must not matter
        k[b, :, n:] = 1e6
        v[b, :, n:] = -1e6
    return q, k, v


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (4, 4), (8, 1)])
def test_decode_is_last_row_of_causal_attention(Hq, Hkv):
    B, Tc, D = 3, 40, 16
    lens = [40, 17, 1]
    q, k, v = cache(B, Hq, Hkv, Tc, D, lens, seed=1)
    o, lse = oracle.attn_decode(q, k, v, lens)
    r = np.random.default_rng(2)
    for b, n in enumerate(lens):
        qf = r.standard_normal((1, Hq, n, D))
        qf[0, :, n - 1] = q[b]
        of, lf = oracle.attn_fwd(qf, k[b:b + 1, :, :n], v[b:b + 1, :, :n], causal=True)
        np.testing.assert_allclose(o[b], of[0, :, n - 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], lf[0, :, n - 1], rtol=0, atol=1e-12)


def test_decode_zero_query_gives_mean_of_values():
    B, Hq, Hkv, Tc, D = 2, 4, 2, 33, 8
    lens = [33, 5]
    _, k, v = cache(B, Hq, Hkv, Tc, D, lens, seed=3)
    o, lse = oracle.attn_decode(np.zeros((B, Hq, D)), k, v, lens)
    for b, n in enumerate(lens):
        for h in range(Hq):
            np.testing.assert_allclose(o[b, h], v[b, h // 2, :n].mean(axis=0), atol=1e-12)
            assert abs(lse[b, h] - math.log(n)) < 1e-12


def test_decode_single_key_and_empty_cache():
    B, Hq, Hkv, Tc, D = 2, 2, 1, 4, 8
    q, k, v = cache(B, Hq, Hkv, Tc, D, [1, 0], seed=4)
    o, lse = oracle.attn_decode(q, k, v, [1, 0])
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], v[0, 0, 0], atol=1e-12)
        assert abs(lse[0, h] - q[0, h] @ k[0, 0, 0] / math.sqrt(D)) < 1e-12
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))


def test_decode_rejects_lengths_past_the_cache():
    q, k, v = cache(1, 2, 1, 4, 8, [4], seed=5)
    with pytest.raises(ValueError):
        oracle.attn_decode(q, k, v, [5])


# ---------------------------------------------------------------- chunked prefill

@pytest.mark.parametrize("Tq,Tk", [(5, 23), (1, 9), (16, 16), (7, 8)])
def test_prefill_is_last_rows_of_causal_attention(Tq, Tk):
    """A chunk of Tq queries at positions Tk-Tq .. Tk-1 is the last Tq rows of causal
    attention over Tk positions (earlier query rows arbitrary)."""
    B, Hq, Hkv, D = 2, 6, 2, 16
    r = np.random.default_rng(6)
    q = r.standard_normal((B, Hq, Tq, D))
    k = r.standard_normal((B, Hkv, Tk, D))
    v = r.standard_normal((B, Hkv, Tk, D))
    o, lse = oracle.attn_prefill(q, k, v)
    qf = np.concatenate([r.standard_normal((B, Hq, Tk - Tq, D)), q], axis=2)
    of, lf = oracle.attn_fwd(qf, k, v, causal=True)
    np.testing.assert_allclose(o, of[:, :, Tk - Tq:], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lf[:, :, Tk - Tq:], rtol=0, atol=1e-12)


def test_prefill_of_one_query_is_a_decode_step():
    B, Hq, Hkv, Tk, D = 3, 4, 2, 19, 8
    r = np.random.default_rng(8)
    q = r.standard_normal((B, Hq, 1, D))
    k = r.standard_normal((B, Hkv, Tk, D))
    v = r.standard_normal((B, Hkv, Tk, D))
    o, lse = oracle.attn_prefill(q, k, v)
    od, ld = oracle.attn_decode(q[:, :, 0], k, v, [Tk] * B)
    np.testing.assert_allclose(o[:, :, 0], od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, 0], ld, rtol=0, atol=1e-12)
