"""The attention sub-block x + attn(rmsnorm(x)) (ne_attn_block_fwd / _bwd) against its fp64
oracle (oracle/block.py): normwise relative error max |g - g_ref| / max |g_ref| <= 1e-4 on y, dx,
dgamma, dw_qkv and dw_o (float32 products over up to 8192 rows)."""
import numpy as np
import pytest

from helpers import normwise
from workloads import BLOCK_WORKLOADS, BlockWorkload, make_block_inputs

pytestmark = pytest.mark.gpu
BAR = 1e-4


def run_block(ne, w, seed=0):
    import torch
    from oracle.block import block_bwd, block_fwd
    print(f"\n[case] block B{w.B} T{w.T} Hq{w.Hq} Hkv{w.Hkv} D{w.D} rope={w.rope_base}", flush=True)
    x = make_block_inputs(w, seed)
    dev = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
    y, ws = ne.block_forward(dev["x"], dev["gamma"], dev["w_qkv"], dev["w_o"], w.Hq, w.Hkv, w.D,
                             w.eps, w.rope_base)
    grads = ne.block_backward(dev["x"], dev["gamma"], dev["w_qkv"], dev["w_o"], dev["dy"], ws,
                              w.Hq, w.Hkv, w.D, w.eps, w.rope_base)
    torch.cuda.synchronize()
    ry, _ = block_fwd(x["x"], x["gamma"], x["w_qkv"], x["w_o"], w.Hq, w.Hkv, w.D, w.eps,
                      w.rope_base)
    rg = block_bwd(x["x"], x["gamma"], x["w_qkv"], x["w_o"], x["dy"], w.Hq, w.Hkv, w.D, w.eps,
                   w.rope_base)
    for name, a, r in zip(("y", "dx", "dgamma", "dw_qkv", "dw_o"), (y,) + tuple(grads),
                          (ry,) + tuple(rg)):
        e = normwise(a.double().cpu().numpy(), r)
        print(f"  {name}_rel={e:.2e}")
        assert e <= BAR, (name, e)


@pytest.mark.parametrize("shape,rope", [((1, 37, 4, 2, 32), 0.0), ((1, 37, 4, 2, 32), 10000.0),
                                        ((2, 130, 12, 4, 64), 10000.0), ((1, 65, 8, 1, 128), 500.0),
                                        ((2, 100, 6, 6, 64), 0.0)],
                         ids=lambda v: str(v))
def test_block_shapes(ne, shape, rope):
    B, T, Hq, Hkv, D = shape
    run_block(ne, BlockWorkload("block", B, T, Hq, Hkv, D, rope_base=rope), seed=3)


def test_block_gpu_model_shape(ne):
    """The GPU model's sub-block (dim 768, 12/4 heads, T 512) at B = 2."""
    from dataclasses import replace
    run_block(ne, replace(BLOCK_WORKLOADS["block_gpu_model"], B=2))


def test_block_gpu_model_bench_batch(ne):
    """The sub-block at the batch it is timed at (B = 16, 8192 rows): the attention kernels then
    take their mirrored tile order and rocBLAS its kernels for that many rows."""
    run_block(ne, BLOCK_WORKLOADS["block_gpu_model"])


def test_block_widest_rows(ne):
    """The widest rows the entry points accept, C = Hq D = 8192 (64 query heads of 128): the
    RMSNorm backward then keeps four rows of C floats, 128 KB, in LDS.  T = 40 is ragged."""
    run_block(ne, BlockWorkload("block", 1, 40, 64, 8, 128, rope_base=10000.0), seed=5)


def test_block_two_host_threads(ne):
    """Two host threads, each on a stream of its own, run the sub-block forward at once: the
    products share the device's rocBLAS handle, whose stream and scratch (a region of the
    call's own workspace) each call binds under a lock, so every result is bitwise the one
    computed alone."""
    import threading
    import torch
    w = BlockWorkload("block", 2, 130, 12, 4, 64, rope_base=10000.0)
    print("\n[case] block forward from two host threads", flush=True)
    dev = [{n: torch.from_numpy(a).cuda() for n, a in make_block_inputs(w, s).items()}
           for s in (11, 12)]
    args = lambda d: (d["x"], d["gamma"], d["w_qkv"], d["w_o"], w.Hq, w.Hkv, w.D, w.eps,
                      w.rope_base)
    ref = [ne.block_forward(*args(d))[0] for d in dev]
    torch.cuda.synchronize()
    reps = 8
    out = [[None] * reps for _ in dev]
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(reps):
                    out[i][r] = ne.block_forward(*args(dev[i]), stream=s)[0]
            s.synchronize()
        except Exception as e:  # surfaced in the main thread below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(dev))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(dev)):
        for r in range(reps):
            assert torch.equal(out[i][r], ref[i]), (i, r)
