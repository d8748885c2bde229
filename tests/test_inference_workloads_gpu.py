"""The decode and prefill workloads that bench.py times, at their full sizes, with the inputs it
draws (workloads.make_decode_inputs / make_prefill_inputs, seed 0) and through the same entry
points, against the fp64 oracle.

Decode: every output.  Prefill: the rows of the GPU-model chunk all, those of the long chunk
sampled; each row i is checked against the oracle's decode step of its query over keys
0 .. Tk - Tq + i, which is the oracle's prefill row i (tests/test_oracle_decode.py pins the two
together).  Bars as for the forward: fp32 max |o - o_ref| and max |lse - lse_ref| <= 2e-5;
bf16 normwise relative error <= 2e-2 on o and lse.
"""
import numpy as np
import pytest

import oracle
from helpers import BF16_ABS_LSE, BF16_REL, F32_ABS_O, normwise
from workloads import (DECODE_WORKLOADS, PREFILL_WORKLOADS, make_decode_inputs,
                       make_prefill_inputs)

pytestmark = pytest.mark.gpu


def check(o, lse, o_ref, lse_ref, bf16, label):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), label
    if bf16:
        assert normwise(o, o_ref) <= BF16_REL, label
        assert normwise(lse, lse_ref) <= BF16_REL, label
        assert np.abs(lse - lse_ref).max() <= BF16_ABS_LSE, label
    else:
        assert np.abs(o - o_ref).max() <= F32_ABS_O, label
        assert np.abs(lse - lse_ref).max() <= F32_ABS_O, label


def to_dev(a, bf16):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if bf16 else t  # bf16 inputs are already bf16 values: exact


@pytest.mark.parametrize("name", sorted(DECODE_WORKLOADS))
def test_decode_workload_full(ne, name):
    import torch
    w = DECODE_WORKLOADS[name]
    bf16 = w.dtype == "bf16"
    print(f"\n[case] decode workload {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Tc{w.Tc} D{w.D} {w.dtype}",
          flush=True)
    x = make_decode_inputs(w, 0)
    q, k, v = (to_dev(x[n], bf16) for n in ("q", "k", "v"))
    o, lse = ne.decode(q, k, v, torch.from_numpy(x["lens"]).cuda())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_decode(x["q"], x["k"], x["v"], x["lens"])
    check(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, bf16, name)


@pytest.mark.parametrize("name", sorted(PREFILL_WORKLOADS))
def test_prefill_workload_rows(ne, name):
    import torch
    w = PREFILL_WORKLOADS[name]
    bf16 = w.dtype == "bf16"
    print(f"\n[case] prefill workload {name}: B{w.B} Hq{w.Hq} Hkv{w.Hkv} Tq{w.Tq} Tk{w.Tk} D{w.D} "
          f"{w.dtype}", flush=True)
    x = make_prefill_inputs(w, 0)
    q, k, v = (to_dev(x[n], bf16) for n in ("q", "k", "v"))
    o, lse = ne.prefill(q, k, v)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    if w.Tq <= 128:
        rows = np.arange(w.Tq)
    else:  # both ends, the middle and random rows
        extra = np.random.default_rng(7).integers(0, w.Tq, 44)
        rows = np.unique(np.concatenate([[0, 1, w.Tq // 2, w.Tq - 1], extra]))
    for i in rows:
        lens = np.full(w.B, w.Tk - w.Tq + i + 1, dtype=np.int32)
        o_ref, lse_ref = oracle.attn_decode(x["q"][:, :, i, :], x["k"], x["v"], lens)
        check(o[:, :, i, :], lse[:, :, i], o_ref, lse_ref, bf16, f"{name} row {i}")
