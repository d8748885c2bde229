"""Pins of the sub-block oracle (oracle/block.py) against what does not depend on it:
central finite differences in float64 on every input, closed forms (w_o = 0 gives y = x and
dx = dy; the RMSNorm of a row is scale invariant), and the attention oracle it is built on."""
import numpy as np
import pytest

from oracle.block import block_bwd, block_fwd

B, T, Hq, Hkv, D = 1, 5, 2, 1, 4
C = Hq * D
W = (Hq + 2 * Hkv) * D


def _inputs(seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, T, C)), 1.0 + 0.3 * r.standard_normal(C),
            0.4 * r.standard_normal((C, W)), 0.4 * r.standard_normal((Hq * D, C)),
            r.standard_normal((B, T, C)))


@pytest.mark.parametrize("rope", [0.0, 10000.0])
def test_block_finite_differences(rope):
    x, g, wq, wo, dy = _inputs(1)
    dx, dg, dwq, dwo = block_bwd(x, g, wq, wo, dy, Hq, Hkv, D, rope_base=rope)
    args = [x, g, wq, wo]
    grads = [dx, dg, dwq, dwo]

    def loss(a):
        y, _ = block_fwd(*a, Hq, Hkv, D, rope_base=rope)
        return float(np.sum(y * dy))

    for n, (a, ga) in enumerate(zip(args, grads)):
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            h = 1e-5 * max(1.0, abs(a[idx]))
            plus = [t.copy() for t in args]
            minus = [t.copy() for t in args]
            plus[n][idx] += h
            minus[n][idx] -= h
            fd[idx] = (loss(plus) - loss(minus)) / (2 * h)
        err = np.abs(fd - ga).max() / np.abs(fd).max()
        assert err <= 1e-6, (n, err)


def test_zero_output_projection_is_the_identity():
    x, g, wq, wo, dy = _inputs(2)
    y, _ = block_fwd(x, g, wq, 0 * wo, Hq, Hkv, D)
    assert np.array_equal(y, x)
    dx, dg, dwq, _ = block_bwd(x, g, wq, 0 * wo, dy, Hq, Hkv, D)
    assert np.array_equal(dx, dy) and not dg.any() and not dwq.any()


def test_rmsnorm_is_scale_invariant():
    """The branch depends on x only through x / rms(x) (eps aside): scaling x by 3 scales
    the residual part of y only through the residual itself."""
    x, g, wq, wo, _ = _inputs(3)
    y1, _ = block_fwd(x, g, wq, wo, Hq, Hkv, D, eps=0.0)
    y3, _ = block_fwd(3 * x, g, wq, wo, Hq, Hkv, D, eps=0.0)
    assert np.allclose(y3 - 3 * x, y1 - x, rtol=1e-12, atol=1e-12)


def test_identity_projections_reduce_to_attention():
    """With gamma = 1, w_qkv selecting the same features for q, k and v, and w_o = I, the
    branch is attention of the normalised rows with itself."""
    import oracle
    x, _, _, _, _ = _inputs(4)
    Hq1, Hkv1 = 2, 2
    eye = np.eye(C)
    wq = np.concatenate([eye, eye, eye], axis=1)
    y, st = block_fwd(x, np.ones(C), wq, np.eye(C), Hq1, Hkv1, D)
    xn = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + 1e-5)
    h = np.ascontiguousarray(xn.reshape(B, T, Hq1, D).transpose(0, 2, 1, 3))
    o, _ = oracle.attn_fwd(h, h, h, causal=True)
    assert np.allclose(y - x, o.transpose(0, 2, 1, 3).reshape(B, T, C), rtol=1e-12, atol=1e-12)
