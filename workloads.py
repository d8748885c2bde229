"""Seeded synthetic inputs for causal grouped-query attention.

This module holds the workload shapes and the random draws only; it contains none of the
attention arithmetic, and both the fp64 oracle side and the HIP side take their inputs from it.

Shapes follow the two models of the NanoEuler pages (README translations, configuration
table): the CPU model (dim 128, 4 query / 2 key-value heads, head size 32, context 512) and
the GPU model (dim 768, 12 query / 4 key-value heads, head size 64, context 512), plus a long
context, a planned wider model with RoPE applied in the kernel, and a tiny case.

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64, float32, in the order
q, k, v, dO, each i.i.d. N(0, 1)):

* ``boost_frac > 0``: after the dO draw, ``round(boost_frac * B * Hq * T)`` query rows, picked
  by ``rng.permutation``, are multiplied by ``boost``; this pushes scores far from zero and
  exercises the running-maximum bookkeeping of the online softmax.
* ``dtype == "bf16"``: every draw is rounded to the nearest bfloat16 (ties to even) so that
  the bf16 kernel inputs and the fp64 oracle inputs are the same numbers.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    dtype: str = "f32"          # "f32" or "bf16"
    causal: bool = True
    rope_base: float = 0.0      # 0 disables RoPE
    boost_frac: float = 0.0
    boost: float = 1.0
    note: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def flops_fwd(self) -> float:
        """Algorithmic forward FLOPs: QK^T and PV, causal counted as half of dense."""
        f = 4.0 * self.B * self.Hq * self.T * self.T * self.D
        return f / 2 if self.causal else f

    def flops_fwd_bwd(self) -> float:
        """Forward (2 GEMMs) plus backward (5 GEMMs): 3.5x the forward."""
        return 3.5 * self.flops_fwd()

    def bytes_fwd_bwd(self) -> int:
        """Algorithmic HBM bytes: fwd reads q,k,v and writes o,lse; bwd reads q,k,v,o,dO,lse
        and writes dq,dk,dv."""
        elt = 2 if self.dtype == "bf16" else 4
        nq = self.B * self.Hq * self.T * self.D
        nk = self.B * self.Hkv * self.T * self.D
        nl = self.B * self.Hq * self.T
        return elt * 6 * (nq + nk) + 8 * nl

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 2, 64, 32,
                     note="tiny causal GQA, oracle-checkable in seconds"),
    "cpu_model": Workload("cpu_model", 8, 4, 2, 512, 32,
                          note="CPU small-model attention layer shape"),
    "gpu_model": Workload("gpu_model", 16, 12, 4, 512, 64, boost_frac=0.1, boost=4.0,
                          note="GPU-model attention layer shape (dim 768)"),
    "long_ctx": Workload("long_ctx", 4, 12, 4, 4096, 64,
                         note="long context, tile streaming and causal skipping"),
    "bf16_rope": Workload("bf16_rope", 16, 16, 4, 1024, 64, dtype="bf16", rope_base=10000.0,
                          note="bf16 with RoPE applied in the kernel (dim 1024)"),
    "d128_f32": Workload("d128_f32", 8, 16, 4, 1024, 128,
                         note="head size 128 (dim 2048), a reading of the planned ~270M scale-up"),
    "d128_bf16_rope": Workload("d128_bf16_rope", 8, 16, 4, 1024, 128, dtype="bf16",
                               rope_base=10000.0,
                               note="head size 128 in bf16 with RoPE applied in the kernel"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Rounds float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32).reshape(x.shape)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Returns float32 numpy arrays q, k, v, dO for workload ``w``."""
    rng = np.random.default_rng(seed)
    qs = (w.B, w.Hq, w.T, w.D)
    ks = (w.B, w.Hkv, w.T, w.D)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    dO = rng.standard_normal(qs, dtype=np.float32)
    if w.boost_frac > 0:
        rows = w.B * w.Hq * w.T
        n = int(round(w.boost_frac * rows))
        idx = rng.permutation(rows)[:n]
        q.reshape(rows, w.D)[idx] *= np.float32(w.boost)
    if w.dtype == "bf16":
        q, k, v, dO = (round_to_bf16(a) for a in (q, k, v, dO))
    return {"q": q, "k": k, "v": v, "dO": dO}


# ---------------------------------------------------------------------------- decode steps

@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: a query per (batch, head) against a key/value cache of capacity Tc.
    Cached lengths are drawn uniformly from [min_len_frac * Tc, Tc] (a generation batch in
    which every sequence has its own length)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Tc: int
    D: int
    dtype: str = "f32"
    min_len_frac: float = 0.5
    note: str = ""

    def cache_bytes(self, lens) -> int:
        """Algorithmic HBM bytes of one step: the cached keys and values of every valid
        position, q read and o written, lse written."""
        elt = 2 if self.dtype == "bf16" else 4
        return (2 * elt * self.Hkv * self.D * int(np.sum(lens))
                + 2 * elt * self.B * self.Hq * self.D + 4 * self.B * self.Hq)


DECODE_WORKLOADS = {
    "decode_gpu_model": DecodeWorkload("decode_gpu_model", 16, 12, 4, 512, 64, min_len_frac=0.0,
                                       note="GPU-model heads, generation within its 512 context"),
    "decode_long": DecodeWorkload("decode_long", 32, 16, 4, 8192, 64, dtype="bf16",
                                  note="wider model, bf16 cache of 8192 positions"),
}


def make_decode_inputs(w: DecodeWorkload, seed: int = 0) -> dict:
    """float32 q [B,Hq,D], k, v [B,Hkv,Tc,D] (i.i.d. N(0,1), drawn in that order, bf16-rounded
    for bf16) and int32 lens [B] drawn last."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((w.B, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.Tc, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.Tc, w.D), dtype=np.float32)
    lo = max(1, int(round(w.min_len_frac * w.Tc)))
    lens = rng.integers(lo, w.Tc + 1, size=w.B).astype(np.int32)
    if w.dtype == "bf16":
        q, k, v = (round_to_bf16(a) for a in (q, k, v))
    return {"q": q, "k": k, "v": v, "lens": lens}


# ---------------------------------------------------------------------------- prefill chunks

@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    """A chunk of Tq new queries at positions Tk-Tq .. Tk-1 against Tk cached keys/values."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    D: int
    dtype: str = "f32"
    note: str = ""

    def flops(self) -> float:
        """QK^T and PV over the keys each query sees (position + 1 of them)."""
        off = self.Tk - self.Tq
        seen = self.Tq * off + self.Tq * (self.Tq + 1) / 2
        return 4.0 * self.B * self.Hq * self.D * seen


PREFILL_WORKLOADS = {
    "prefill_gpu_model": PrefillWorkload("prefill_gpu_model", 16, 12, 4, 128, 512, 64,
                                         note="GPU-model heads: the last 128 of 512 positions"),
    "prefill_long": PrefillWorkload("prefill_long", 4, 16, 4, 1024, 8192, 64, dtype="bf16",
                                    note="wider model, bf16: a 1024-token chunk after 7168"),
}


def make_prefill_inputs(w: PrefillWorkload, seed: int = 0) -> dict:
    """float32 q [B,Hq,Tq,D], k, v [B,Hkv,Tk,D], i.i.d. N(0,1) in that order (bf16-rounded for
    bf16)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((w.B, w.Hq, w.Tq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.Tk, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.Tk, w.D), dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = (round_to_bf16(a) for a in (q, k, v))
    return {"q": q, "k": k, "v": v}


# ----------------------------------------------------------------------- attention sub-block

@dataclasses.dataclass(frozen=True)
class BlockWorkload:
    """The attention sub-block x + attn(rmsnorm(x)) at one layer's shape: x [B, T, C],
    C = Hq D; gamma [C]; w_qkv [C, (Hq + 2 Hkv) D]; w_o [Hq D, C]."""
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    rope_base: float = 10000.0
    eps: float = 1e-5
    note: str = ""

    @property
    def C(self) -> int:
        return self.Hq * self.D

    def flops(self) -> float:
        """Forward + backward: the three projection GEMMs of each pass (forward 2 products,
        backward 4) plus the attention's 7 B Hq T^2 D (causal)."""
        n = self.B * self.T
        w = (self.Hq + 2 * self.Hkv) * self.D
        gemm_fwd = 2.0 * n * self.C * w + 2.0 * n * self.Hq * self.D * self.C
        return 3.0 * gemm_fwd + 3.5 * 2.0 * self.B * self.Hq * self.T * self.T * self.D


BLOCK_WORKLOADS = {
    "block_gpu_model": BlockWorkload("block_gpu_model", 16, 512, 12, 4, 64,
                                     note="the GPU model's attention sub-block (dim 768)"),
}


def make_block_inputs(w: BlockWorkload, seed: int = 0) -> dict:
    """Draws, in order, x ~ N(0, 1), gamma = 1 + 0.1 N(0, 1), w_qkv and w_o ~ N(0, 1 / C),
    dy ~ N(0, 1), float32."""
    rng = np.random.default_rng(seed)
    C, W = w.C, (w.Hq + 2 * w.Hkv) * w.D
    f = np.float32
    x = rng.standard_normal((w.B, w.T, C), dtype=f)
    gamma = (1.0 + 0.1 * rng.standard_normal(C, dtype=f)).astype(f)
    w_qkv = (rng.standard_normal((C, W), dtype=f) / np.sqrt(C)).astype(f)
    w_o = (rng.standard_normal((w.Hq * w.D, C), dtype=f) / np.sqrt(C)).astype(f)
    dy = rng.standard_normal((w.B, w.T, C), dtype=f)
    return {"x": x, "gamma": gamma, "w_qkv": w_qkv, "w_o": w_o, "dy": dy}
