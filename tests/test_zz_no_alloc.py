"""ne_attn_bwd_noalloc (static scratch, no workspace argument) against ne_attn_bwd_ex through
the C ABI: two calls in a row, the second on a smaller input, each bitwise equal to the backward
that takes a caller workspace (same kernels, same order of operations)."""
import ctypes

import numpy as np
import pytest

from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _tensors(w, seed):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = make_inputs(w, seed)
    return [torch.from_numpy(x[n]).cuda().to(dt).contiguous() for n in ("q", "k", "v", "dO")]


def _both(ne, w, seed):
    import torch
    q, k, v, dO = _tensors(w, seed)
    code = ne.NE_BF16 if w.dtype == "bf16" else ne.NE_F32
    o, lse = ne.forward(q, k, v, causal=w.causal, rope_base=w.rope_base)
    ref = ne.backward(q, k, v, o, lse, dO, causal=w.causal, rope_base=w.rope_base)
    got = [torch.full_like(t, float("nan")) for t in ref]
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = ne.lib().ne_attn_bwd_noalloc(P(q), P(k), P(v), P(o), P(lse), P(dO), *(P(t) for t in got),
                                      w.B, w.Hq, w.Hkv, w.T, w.D, int(w.causal), code,
                                      ctypes.c_float(w.rope_base), st)
    assert rc == ne.NE_OK, ne.ne_attn_strerror(rc)
    torch.cuda.synchronize()
    return got, ref


SEQS = [
    [Workload("big", 16, 16, 4, 1024, 64, dtype="bf16", rope_base=10000.0),
     Workload("small", 1, 4, 2, 300, 64, dtype="bf16", rope_base=10000.0)],
    [Workload("big", 16, 12, 4, 512, 64), Workload("small", 2, 6, 2, 77, 32, causal=False)],
    [Workload("big", 2, 8, 2, 1000, 128, rope_base=500.0), Workload("small", 1, 3, 1, 65, 128)],
]


@pytest.mark.parametrize("seq", SEQS, ids=["bf16_rope", "f32", "f32_d128"])
def test_noalloc_backward_matches_workspace_backward(ne, seq):
    for i, w in enumerate(seq):
        print(f"\n[case] noalloc call {i}: {w}", flush=True)
        got, ref = _both(ne, w, 50 + i)
        for n, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert not a.isnan().any(), n
            assert np.array_equal(a.float().cpu().numpy(), b.float().cpu().numpy()), (i, n)
