"""Shared test helpers: run the HIP path through the binding and compare with the oracle."""
from __future__ import annotations

import numpy as np

# Tolerances against the fp64 oracle.
F32_ABS_O = 2e-5        # max |o - o_ref| and max |lse - lse_ref|
F32_REL_GRAD = 1e-4     # max |g - g_ref| / max |g_ref| for dq, dk, dv
BF16_REL = 2e-2         # normwise relative error on every output in bf16
# bf16: max |lse - lse_ref|.  lse is formed from fp32 scores of the bf16 inputs and the sum of
# the probabilities as rounded to bf16 (relative error at most 2^-9, so at most 2e-3 in lse);
# with RoPE the rotated q and k are rounded to bf16 too, which moves a score by about 2e-3 (one
# standard deviation) -- the bar leaves room for the largest of about 10^6 rows.
BF16_ABS_LSE = 1e-2


def normwise(a, r) -> float:
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.abs(r).max()
    return float(np.abs(a - r).max() / (den if den > 0 else 1.0))


def to_dev(x: np.ndarray, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def gpu_fwd_bwd(ne, inputs, causal=True, rope_base=0.0, dtype=None, with_bwd=True):
    """Runs forward (and backward) on cuda:0; returns float64 numpy arrays."""
    import torch
    dtype = dtype or torch.float32
    q, k, v, dO = (to_dev(inputs[n], dtype) for n in ("q", "k", "v", "dO"))
    o, lse = ne.forward(q, k, v, causal=causal, rope_base=rope_base)
    out = {"o": o, "lse": lse}
    if with_bwd:
        dq, dk, dv = ne.backward(q, k, v, o, lse, dO, causal=causal, rope_base=rope_base)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()}


def oracle_fwd_bwd(oracle, inputs, causal=True, rope_base=0.0, with_bwd=True):
    q, k, v, dO = (inputs[n].astype(np.float64) for n in ("q", "k", "v", "dO"))
    o, lse = oracle.attn_fwd(q, k, v, causal=causal, rope_base=rope_base)
    ref = {"o": o, "lse": lse}
    if with_bwd:
        dq, dk, dv = oracle.attn_bwd(q, k, v, dO, causal=causal, rope_base=rope_base)
        ref.update(dq=dq, dk=dk, dv=dv)
    return ref


def errors(res, ref) -> dict:
    e = {}
    for n in res:
        e[n + "_abs"] = float(np.abs(res[n] - ref[n]).max())
        e[n + "_rel"] = normwise(res[n], ref[n])
    return e


def assert_f32(res, ref, label=""):
    e = errors(res, ref)
    assert np.isfinite(list(e.values())).all(), (label, e)
    assert e["o_abs"] <= F32_ABS_O, (label, e)
    assert e["lse_abs"] <= F32_ABS_O, (label, e)
    for n in ("dq", "dk", "dv"):
        if n in res:
            assert e[n + "_rel"] <= F32_REL_GRAD, (label, n, e)
    return e


def assert_bf16(res, ref, label=""):
    e = errors(res, ref)
    assert np.isfinite(list(e.values())).all(), (label, e)
    for n in res:
        assert e[n + "_rel"] <= BF16_REL, (label, n, e)
    if "lse" in res:
        assert e["lse_abs"] <= BF16_ABS_LSE, (label, "lse", e)
    return e
