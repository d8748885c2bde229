"""A NaN in the inputs reaches exactly the outputs that depend on it, and the kernels complete.

Causal attention row t of head h reads query t of h and keys/values 0..t of its key/value head
g = h // G.  So a NaN in q[b, h, t] makes o[b, h, t] and lse[b, h, t] NaN and leaves every other
forward output bitwise as it was without it.  A NaN in v[b, g, j] makes o[b, h, i] NaN for every
head of the group and every i >= j, and leaves lse untouched (lse does not read v); rows i < j
that share j's 64-key tile multiply the NaN by their exact-zero masked probabilities (0 * NaN is
NaN), so only rows before that tile, other heads and other batch elements are asserted
unchanged.

Backward with the NaN in q[b, h, t]: dq row t is NaN and every other dq row is unchanged; dk and
dv rows 0..t of key/value head g are NaN (query t's probabilities reach them).  Rows of dk, dv in
key blocks past t's 32-row block, other key/value heads and other batch elements are unchanged.
(Inside t's own key block the masked probabilities are exact zeros, but dS = P (dP - delta) with
delta_t = NaN makes 0 * NaN; those rows are not asserted either way.)
"""
import numpy as np
import pytest

from helpers import gpu_fwd_bwd
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _same_or_both_nan(a, b):
    return np.array_equal(a, b, equal_nan=True)


CASES = [("f32", 0.0), ("bf16", 0.0), ("bf16", 10000.0), ("f32", 10000.0)]


@pytest.mark.parametrize("dtype,rope", CASES)
def test_nan_in_query_row(ne, dtype, rope):
    import torch
    w = Workload("nan", 2, 8, 2, 200, 64, dtype=dtype, rope_base=rope)
    x = make_inputs(w, 31)
    b, h, t = 1, 5, 77
    g = h // w.G
    y = {n: v.copy() for n, v in x.items()}
    y["q"][b, h, t, 3] = np.nan
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"\n[case] NaN in q[{b},{h},{t}] {dtype} rope={rope}", flush=True)
    ref = gpu_fwd_bwd(ne, x, rope_base=rope, dtype=tdt)
    got = gpu_fwd_bwd(ne, y, rope_base=rope, dtype=tdt)

    # forward: exactly row (b, h, t) is NaN
    assert np.isnan(got["o"][b, h, t]).all() and np.isnan(got["lse"][b, h, t])
    for n in ("o", "lse"):
        mask = np.ones(got[n].shape[:3], bool)
        mask[b, h, t] = False
        assert not np.isnan(got[n][mask]).any(), n
        assert np.array_equal(got[n][mask], ref[n][mask]), n

    # dq: row t NaN, every other row unchanged
    assert np.isnan(got["dq"][b, h, t]).all()
    mask = np.ones(got["dq"].shape[:3], bool)
    mask[b, h, t] = False
    assert np.array_equal(got["dq"][mask], ref["dq"][mask])

    # dk, dv: rows 0..t of (b, g) NaN; later key blocks, other heads, other batches unchanged
    nxt = (t // 32 + 1) * 32
    for n in ("dk", "dv"):
        assert np.isnan(got[n][b, g, :t + 1]).any(axis=-1).all(), n
        assert np.array_equal(got[n][b, g, nxt:], ref[n][b, g, nxt:]), n
        other = np.ones(got[n].shape[:2], bool)
        other[b, g] = False
        assert np.array_equal(got[n][other], ref[n][other]), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_in_value_row(ne, dtype):
    import torch
    w = Workload("nan", 2, 8, 2, 200, 64, dtype=dtype)
    x = make_inputs(w, 32)
    b, g, j = 0, 1, 130
    y = {n: v.copy() for n, v in x.items()}
    y["v"][b, g, j, 10] = np.nan
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"\n[case] NaN in v[{b},{g},{j}] {dtype}", flush=True)
    ref = gpu_fwd_bwd(ne, x, dtype=tdt, with_bwd=False)
    got = gpu_fwd_bwd(ne, y, dtype=tdt, with_bwd=False)
    heads = slice(g * w.G, (g + 1) * w.G)
    assert np.isnan(got["o"][b, heads, j:]).any(axis=-1).all()
    mask = np.ones(got["o"].shape[:3], bool)
    mask[b, heads, (j // 64) * 64:] = False
    assert np.array_equal(got["o"][mask], ref["o"][mask])
    assert np.array_equal(got["lse"], ref["lse"])  # lse does not read v
