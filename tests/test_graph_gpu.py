"""The entry points captured into a HIP graph: every replay matches the eager result.

The graph records forward + backward (two passes, or the single-pass variant) on preallocated
tensors.  Between replays the test does eager work of its own (overwriting the outputs and
running other kernels) and synchronises, then checks each replay: bitwise for the two-pass
path (deterministic), within rounding for the single-pass dq (atomic order).
"""
import numpy as np
import pytest

from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _setup(ne, w, seed):
    import torch
    x = make_inputs(w, seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, dO = (torch.from_numpy(x[n]).cuda().to(dt).contiguous() for n in ("q", "k", "v", "dO"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = ne.workspace(q, k, w.rope_base)
    return q, k, v, dO, o, lse, dq, dk, dv, ws


def _graph_case(ne, w, fused, seed=3, replays=3):
    import torch
    q, k, v, dO, o, lse, dq, dk, dv, ws = _setup(ne, w, seed)
    rb = w.rope_base

    def step():
        ne.ne_attn_fwd_ex(q, k, v, o, lse, ws, causal=True, rope_base=rb)
        if fused:
            ne.ne_attn_bwd_fused(q, k, v, o, lse, dO, dq, dk, dv, ws, causal=True, rope_base=rb)
        else:
            ne.ne_attn_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, ws, causal=True, rope_base=rb)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, dq, dk, dv)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    scratch = torch.randn(1 << 20, device=q.device)
    for r in range(replays):
        for t in (o, lse, dq, dk, dv):  # the replay must rewrite every output
            t.fill_(float("nan"))
        scratch.mul_(1.0001).add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o, lse, dq, dk, dv)
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, eager):
            if fused and name == "dq":
                x, y = a.double().cpu().numpy(), b.double().cpu().numpy()
                assert np.abs(x - y).max() <= 1e-5 * np.abs(y).max(), (r, name)
            else:
                assert torch.equal(a, b), (r, name)


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_fp32(ne, fused):
    print(f"\n[case] graph fp32 fused={fused}", flush=True)
    _graph_case(ne, Workload("graph", 2, 12, 4, 300, 64), fused)


def test_graph_replays_fp32_rope_fused(ne):
    print("\n[case] graph fp32 RoPE fused", flush=True)
    _graph_case(ne, Workload("graph", 1, 8, 2, 257, 64, rope_base=10000.0), True)


@pytest.mark.parametrize("D", [64, 128])
def test_graph_replays_bf16_rope(ne, D):
    print(f"\n[case] graph bf16 RoPE D{D}", flush=True)
    _graph_case(ne, Workload("graph", 2, 8, 2, 300, D, dtype="bf16", rope_base=10000.0), False)


def test_graph_replays_decode(ne):
    import torch
    print("\n[case] graph decode", flush=True)
    r = np.random.default_rng(5)
    B, Hq, Hkv, Tc, D = 3, 8, 2, 700, 64
    q = torch.from_numpy(r.standard_normal((B, Hq, D)).astype(np.float32)).cuda()
    kc = torch.from_numpy(r.standard_normal((B, Hkv, Tc, D)).astype(np.float32)).cuda()
    vc = torch.from_numpy(r.standard_normal((B, Hkv, Tc, D)).astype(np.float32)).cuda()
    lens = torch.tensor([700, 300, 1], dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(ne.ne_attn_decode_workspace_bytes(B, Hq, Hkv, Tc, D, ne.NE_F32),
                     dtype=torch.uint8, device="cuda")
    ne.ne_attn_decode(q, kc, vc, lens, o, lse, ws)
    torch.cuda.synchronize()
    eo, el = o.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ne.ne_attn_decode(q, kc, vc, lens, o, lse, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ne.ne_attn_decode(q, kc, vc, lens, o, lse, ws)
    for _ in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el)


def test_graph_replays_block(ne):
    """The attention sub-block (its rocBLAS products included) captured forward + backward."""
    import torch
    from workloads import BlockWorkload, make_block_inputs
    print("\n[case] graph sub-block", flush=True)
    w = BlockWorkload("graph", 2, 96, 4, 2, 32)
    x = {n: torch.from_numpy(a).cuda() for n, a in make_block_inputs(w, 4).items()}
    y = torch.empty_like(x["x"])
    dx, dg = torch.empty_like(x["x"]), torch.empty_like(x["gamma"])
    dwq, dwo = torch.empty_like(x["w_qkv"]), torch.empty_like(x["w_o"])
    ws = torch.empty(ne.ne_attn_block_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D, w.rope_base),
                     dtype=torch.uint8, device="cuda")

    def step():
        ne.ne_attn_block_fwd(x["x"], x["gamma"], x["w_qkv"], x["w_o"], y, ws, w.Hq, w.Hkv, w.D,
                             w.eps, w.rope_base)
        ne.ne_attn_block_bwd(x["x"], x["gamma"], x["w_qkv"], x["w_o"], x["dy"], dx, dg, dwq, dwo,
                             ws, w.Hq, w.Hkv, w.D, w.eps, w.rope_base)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (y, dx, dg, dwq, dwo)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for t in (y, dx, dg, dwq, dwo):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((y, dx, dg, dwq, dwo), eager):
            assert torch.equal(a, b)
