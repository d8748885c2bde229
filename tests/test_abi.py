"""The C-ABI library loads, exports every entry point of include/ne_attn.h and rejects invalid
arguments before anything is launched.  No call here reaches a kernel, so these run without a
GPU (and are safe with one: every argument set below fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ne_attn.h")

VP = ctypes.c_void_p
A = 4096        # a 16-byte-aligned stand-in address; never dereferenced (validation fails first)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ne_attn_\w+)\s*\(", text)))


def test_header_declares_the_documented_entry_points(ne):
    assert header_functions() == sorted(ne.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(ne):
    L = ne.load()
    for name in header_functions():
        assert hasattr(L, name), name


C_CONSUMER = r"""
#include <stdio.h>
#include <string.h>
#include "ne_attn.h"
int main(void) {
    /* sizes: delta only without RoPE; 4 bytes per (batch, query head, position) */
    if (ne_attn_workspace_bytes(2, 4, 2, 64, 32, NE_F32, 0.0f) != 4u * 2 * 4 * 64) return 1;
    if (ne_attn_bwd_workspace_bytes(2, 4, 64) != 4u * 2 * 4 * 64) return 2;
    /* argument errors come back before any launch */
    if (ne_attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 4, 2, 64, 32, 1, NULL) != NE_ERR_NULL) return 3;
    if (strlen(ne_attn_strerror(NE_ERR_SHAPE)) == 0) return 4;
    printf("ok\n");
    return 0;
}
"""


def test_header_is_c99_and_the_library_links_from_c(ne, tmp_path):
    """A plain C99 program (no C++, no torch) includes the header under -pedantic -Werror, links
    the library and calls entry points that need no GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    lib_dir = os.path.dirname(ne.library_path())
    src = tmp_path / "consumer.c"
    exe = tmp_path / "consumer"
    src.write_text(C_CONSUMER)
    cmd = [gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I",
           os.path.join(ROOT, "include"), str(src), "-o", str(exe), "-L", lib_dir, "-lne_attn",
           "-Wl,-rpath," + lib_dir, "-Wl,-rpath-link,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


def test_strerror_covers_every_status(ne):
    seen = set()
    for st in range(7):
        s = ne.ne_attn_strerror(st)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 7
    assert ne.ne_attn_strerror(99) == "unknown status"
    assert ne.ne_attn_strerror(-1) == "unknown status"


def test_workspace_bytes(ne):
    assert ne.ne_attn_bwd_workspace_bytes(16, 12, 512) == 4 * 16 * 12 * 512
    assert ne.ne_attn_bwd_workspace_bytes(0, 12, 512) == 0
    assert ne.ne_attn_bwd_workspace_bytes(1, 1, 1) == 4


def up256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("dtype,es", [(0, 4), (1, 2)])
def test_ex_workspace_bytes(ne, dtype, es):
    """delta region, then (with RoPE) rotated k and rotated q, each on a 256-byte boundary."""
    B, Hq, Hkv, T, D = 3, 6, 2, 77, 64
    assert ne.ne_attn_workspace_bytes(B, Hq, Hkv, T, D, dtype, 0.0) == up256(4 * B * Hq * T)
    assert ne.ne_attn_workspace_bytes(B, Hq, Hkv, T, D, dtype, 10000.0) == (
        up256(4 * B * Hq * T) + up256(es * B * Hkv * T * D) + up256(es * B * Hq * T * D))
    assert ne.ne_attn_workspace_bytes(B, Hq, 4, T, D, dtype, 0.0) == 0    # Hq % Hkv != 0
    assert ne.ne_attn_workspace_bytes(B, Hq, Hkv, T, 48, dtype, 0.0) == 0  # unsupported D
    assert ne.ne_attn_workspace_bytes(B, Hq, Hkv, T, D, 7, 0.0) == 0       # unknown dtype
    assert ne.ne_attn_workspace_bytes(B, Hq, Hkv, T, D, dtype, -1.0) == 0


def fwd(ne, ptrs=None, B=1, Hq=4, Hkv=2, T=64, D=32, causal=1, dtype=None, rope=0.0, ws=A):
    L = ne.load()
    p = ptrs or [A] * 5
    if dtype is None:
        return L.ne_attn_fwd(*[VP(x) for x in p], B, Hq, Hkv, T, D, causal, VP(0))
    return L.ne_attn_fwd_ex(*[VP(x) for x in p], VP(ws), B, Hq, Hkv, T, D, causal, dtype, rope,
                            VP(0))


def bwd(ne, ptrs=None, B=1, Hq=4, Hkv=2, T=64, D=32, causal=1, dtype=None, rope=0.0):
    L = ne.load()
    p = ptrs or [A] * 10
    if dtype is None:
        return L.ne_attn_bwd(*[VP(x) for x in p], B, Hq, Hkv, T, D, causal, VP(0))
    return L.ne_attn_bwd_ex(*[VP(x) for x in p], B, Hq, Hkv, T, D, causal, dtype, rope, VP(0))


@pytest.mark.parametrize("which", range(5))
def test_fwd_null_pointer(ne, which):
    p = [A] * 5
    p[which] = 0
    assert fwd(ne, p) == ne.NE_ERR_NULL
    assert fwd(ne, p, dtype=0) == ne.NE_ERR_NULL
    assert fwd(ne, p, dtype=1, rope=10000.0) == ne.NE_ERR_NULL


@pytest.mark.parametrize("dtype", [0, 1])
def test_fwd_rope_needs_workspace(ne, dtype):
    """With RoPE the forward rotates the keys into the workspace: NULL or misaligned is refused
    before anything is enqueued."""
    assert fwd(ne, dtype=dtype, rope=10000.0, ws=0) == ne.NE_ERR_NULL
    assert fwd(ne, dtype=dtype, rope=10000.0, ws=A + 4) == ne.NE_ERR_ALIGN


@pytest.mark.parametrize("which", range(10))
def test_bwd_null_pointer(ne, which):
    p = [A] * 10
    p[which] = 0
    assert bwd(ne, p) == ne.NE_ERR_NULL
    assert bwd(ne, p, dtype=1, rope=10000.0) == ne.NE_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0), dict(Hkv=0), dict(T=0), dict(T=-5),
                                dict(Hq=4, Hkv=3), dict(Hq=2, Hkv=4),
                                dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, T=1 << 20),
                                dict(T=(1 << 24) + 1)])
def test_bad_shapes(ne, kw):
    assert fwd(ne, **kw) == ne.NE_ERR_SHAPE
    assert bwd(ne, **kw) == ne.NE_ERR_SHAPE
    assert fwd(ne, dtype=0, **kw) == ne.NE_ERR_SHAPE


def test_bf16_head_limit(ne):
    """The bf16 kernels address a head through 32-bit buffer offsets: a head of more than 2^31
    bytes is refused before any launch (T above 2^23 at D = 128), in every entry point."""
    T = (1 << 23) + 1
    assert fwd(ne, dtype=1, T=T, D=128) == ne.NE_ERR_SHAPE
    assert fwd(ne, dtype=1, T=T, D=128, rope=10000.0) == ne.NE_ERR_SHAPE
    assert bwd(ne, dtype=1, T=T, D=128) == ne.NE_ERR_SHAPE
    assert ne.ne_attn_workspace_bytes(1, 4, 2, T, 128, 1, 0.0) == 0
    assert ne.ne_attn_decode_workspace_bytes(1, 4, 2, T, 128, 1) == 0
    assert prefill_call(ne, Tq=16, Tk=T, D=128, dtype=1) == ne.NE_ERR_SHAPE
    # the same sizes are fine for shapes the bound does not reach (checked without launching)
    assert ne.ne_attn_workspace_bytes(1, 4, 2, T, 128, 0, 0.0) > 0
    assert ne.ne_attn_workspace_bytes(1, 4, 2, 1 << 24, 64, 1, 0.0) > 0


@pytest.mark.parametrize("kw", [dict(D=16), dict(D=256), dict(D=48), dict(dtype=2),
                                dict(dtype=-1), dict(dtype=0, rope=-1.0),
                                dict(dtype=0, rope=float("inf")), dict(dtype=0, rope=float("nan"))])
def test_unsupported(ne, kw):
    assert fwd(ne, **kw) == ne.NE_ERR_UNSUPPORTED
    assert bwd(ne, **kw) == ne.NE_ERR_UNSUPPORTED


def dq_pass(ne, ptrs=None, **kw):
    L = ne.load()
    p = ptrs or [A] * 8
    a = dict(B=1, Hq=4, Hkv=2, T=64, D=32, causal=1, dtype=0, rope=0.0)
    a.update(kw)
    return L.ne_attn_bwd_dq_ex(*[VP(x) for x in p], a["B"], a["Hq"], a["Hkv"], a["T"], a["D"],
                               a["causal"], a["dtype"], a["rope"], VP(0))


def dkdv_pass(ne, ptrs=None, **kw):
    L = ne.load()
    p = ptrs or [A] * 8
    a = dict(B=1, Hq=4, Hkv=2, T=64, D=32, causal=1, dtype=0, rope=0.0)
    a.update(kw)
    return L.ne_attn_bwd_dkdv_ex(*[VP(x) for x in p], a["B"], a["Hq"], a["Hkv"], a["T"],
                                 a["D"], a["causal"], a["dtype"], a["rope"], VP(0))


@pytest.mark.parametrize("which", range(8))
def test_backward_passes_validate(ne, which):
    p = [A] * 8
    p[which] = 0
    assert dq_pass(ne, p) == ne.NE_ERR_NULL
    assert dkdv_pass(ne, p) == ne.NE_ERR_NULL
    p[which] = A + 8
    assert dq_pass(ne, p) == ne.NE_ERR_ALIGN
    assert dkdv_pass(ne, p) == ne.NE_ERR_ALIGN
    assert dq_pass(ne, Hkv=3) == ne.NE_ERR_SHAPE
    assert dkdv_pass(ne, D=256) == ne.NE_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", range(10))
def test_misaligned(ne, which):
    p = [A] * 10
    p[which] = A + 4
    assert bwd(ne, p) == ne.NE_ERR_ALIGN
    if which < 5:
        assert fwd(ne, p[:5]) == ne.NE_ERR_ALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import causal_gqa_flashattention_attn_amd as m
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        m.load()


def test_single_hip_runtime_in_process():
    """The library must share the HIP runtime torch loaded, not bring a second one."""
    import subprocess
    import sys
    code = ("import re, causal_gqa_flashattention_attn_amd as ne; ne.load(); import torch; "
            "m = open('/proc/self/maps').read(); "
            "print(len(set(re.findall(r'/\\S*libamdhip64\\S*', m))))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.strip().splitlines()[-1]
    assert out == "1"


def decode_call(ne, ptrs=None, B=2, Hq=4, Hkv=2, Tc=300, D=64, dtype=0):
    L = ne.load()
    p = ptrs or [A] * 7
    return L.ne_attn_decode(*[VP(x) for x in p], B, Hq, Hkv, Tc, D, dtype, VP(0))


def test_decode_workspace_bytes(ne):
    """Splits of 256 cached keys: outputs [S][B][Hq][D] then lse [S][B][Hq], fp32, each region
    on a 256-byte boundary."""
    B, Hq, Hkv, Tc, D = 3, 6, 2, 700, 64
    S = (Tc + 255) // 256
    for dtype in (0, 1):
        assert ne.ne_attn_decode_workspace_bytes(B, Hq, Hkv, Tc, D, dtype) == (
            up256(4 * S * B * Hq * D) + up256(4 * S * B * Hq))
    assert ne.ne_attn_decode_workspace_bytes(B, Hq, 4, Tc, D, 0) == 0     # Hq % Hkv
    assert ne.ne_attn_decode_workspace_bytes(B, Hq, Hkv, 0, D, 0) == 0    # empty cache
    assert ne.ne_attn_decode_workspace_bytes(B, Hq, Hkv, Tc, 256, 0) == 0  # unsupported D
    for dtype in (0, 1):  # head size 128 in both dtypes
        assert ne.ne_attn_decode_workspace_bytes(B, Hq, Hkv, Tc, 128, dtype) == (
            up256(4 * S * B * Hq * 128) + up256(4 * S * B * Hq))


@pytest.mark.parametrize("which", range(7))
def test_decode_validates(ne, which):
    p = [A] * 7
    p[which] = 0
    assert decode_call(ne, p) == ne.NE_ERR_NULL
    p[which] = A + 4
    assert decode_call(ne, p) == ne.NE_ERR_ALIGN
    assert decode_call(ne, Hkv=3) == ne.NE_ERR_SHAPE
    assert decode_call(ne, Tc=0) == ne.NE_ERR_SHAPE
    assert decode_call(ne, B=70000, Hq=1, Hkv=1) == ne.NE_ERR_SHAPE   # grid rows past 65535
    assert decode_call(ne, D=48) == ne.NE_ERR_UNSUPPORTED
    assert decode_call(ne, D=256) == ne.NE_ERR_UNSUPPORTED
    assert decode_call(ne, dtype=3) == ne.NE_ERR_UNSUPPORTED


def prefill_call(ne, ptrs=None, B=1, Hq=4, Hkv=2, Tq=16, Tk=40, D=64, dtype=0):
    L = ne.load()
    p = ptrs or [A] * 5
    return L.ne_attn_prefill(*[VP(x) for x in p], B, Hq, Hkv, Tq, Tk, D, dtype, VP(0))


@pytest.mark.parametrize("which", range(5))
def test_prefill_validates(ne, which):
    p = [A] * 5
    p[which] = 0
    assert prefill_call(ne, p) == ne.NE_ERR_NULL
    p[which] = A + 4
    assert prefill_call(ne, p) == ne.NE_ERR_ALIGN
    assert prefill_call(ne, Tq=41) == ne.NE_ERR_SHAPE    # longer than the cache
    assert prefill_call(ne, Tq=0) == ne.NE_ERR_SHAPE
    assert prefill_call(ne, Hkv=3) == ne.NE_ERR_SHAPE
    assert prefill_call(ne, D=256) == ne.NE_ERR_UNSUPPORTED


def fused(ne, ptrs=None, **kw):
    L = ne.load()
    p = ptrs or [A] * 10
    a = dict(B=1, Hq=4, Hkv=2, T=64, D=32, causal=1, dtype=0, rope=0.0)
    a.update(kw)
    return L.ne_attn_bwd_fused(*[VP(x) for x in p], a["B"], a["Hq"], a["Hkv"], a["T"], a["D"],
                               a["causal"], a["dtype"], a["rope"], VP(0))


@pytest.mark.parametrize("which", range(10))
def test_fused_backward_validates(ne, which):
    p = [A] * 10
    p[which] = 0
    assert fused(ne, p) == ne.NE_ERR_NULL
    p[which] = A + 4
    assert fused(ne, p) == ne.NE_ERR_ALIGN
    assert fused(ne, Hkv=3) == ne.NE_ERR_SHAPE
    assert fused(ne, T=0) == ne.NE_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(dtype=1), dict(dtype=1, rope=10000.0), dict(D=256),
                                dict(D=48), dict(rope=-1.0)])
def test_fused_backward_limits(ne, kw):
    """float32 only; D 32, 64 or 128."""
    assert fused(ne, **kw) == ne.NE_ERR_UNSUPPORTED


def block_call(ne, which, ptrs=None, B=1, T=16, Hq=4, Hkv=2, D=32, eps=1e-5, rope=0.0):
    L = ne.load()
    if which == "fwd":
        p = ptrs or [A] * 6
        return L.ne_attn_block_fwd(*[VP(x) for x in p], B, T, Hq, Hkv, D, eps, rope, VP(0))
    p = ptrs or [A] * 10
    return L.ne_attn_block_bwd(*[VP(x) for x in p], B, T, Hq, Hkv, D, eps, rope, VP(0))


@pytest.mark.parametrize("which,n", [("fwd", 6), ("bwd", 10)])
def test_block_validates(ne, which, n):
    for j in range(n):
        p = [A] * n
        p[j] = 0
        assert block_call(ne, which, p) == ne.NE_ERR_NULL
        p[j] = A + 4
        assert block_call(ne, which, p) == ne.NE_ERR_ALIGN
    assert block_call(ne, which, Hkv=3) == ne.NE_ERR_SHAPE
    assert block_call(ne, which, T=0) == ne.NE_ERR_SHAPE
    assert block_call(ne, which, D=48) == ne.NE_ERR_UNSUPPORTED
    assert block_call(ne, which, eps=0.0) == ne.NE_ERR_UNSUPPORTED
    assert block_call(ne, which, eps=float("nan")) == ne.NE_ERR_UNSUPPORTED
    assert block_call(ne, which, rope=-1.0) == ne.NE_ERR_UNSUPPORTED
    assert block_call(ne, which, Hq=130, Hkv=2, D=64) == ne.NE_ERR_SHAPE  # C = 8320 > 8192
    # the attention reads one batch element's projection rows with 32-bit offsets: T W < 2^31
    assert block_call(ne, which, T=1 << 20, Hq=64, Hkv=8, D=128) == ne.NE_ERR_SHAPE


def test_block_workspace_bytes(ne):
    n = ne.ne_attn_block_workspace_bytes(2, 64, 4, 2, 32, 0.0)
    n_rope = ne.ne_attn_block_workspace_bytes(2, 64, 4, 2, 32, 10000.0)
    C, N = 4 * 32, 2 * 64
    assert n > 4 * N * C * 4 and n_rope > n          # RoPE adds the rotated q, k
    assert ne.ne_attn_block_workspace_bytes(2, 64, 4, 3, 32, 0.0) == 0  # Hq % Hkv
    assert ne.ne_attn_block_workspace_bytes(2, 64, 4, 2, 48, 0.0) == 0  # unsupported D


def test_block_binding_checks_output_shapes(ne):
    """The binding rejects outputs whose shape or dtype differs from what the entry points write
    (before any device call, so host tensors serve)."""
    import torch
    B, T, Hq, Hkv, D = 1, 16, 4, 2, 32
    C, W = Hq * D, (Hq + 2 * Hkv) * D
    x, g = torch.zeros(B, T, C), torch.zeros(C)
    wqkv, wo = torch.zeros(C, W), torch.zeros(C, C)
    ws = torch.zeros(1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="y must be"):
        ne.ne_attn_block_fwd(x, g, wqkv, wo, torch.zeros(B, T - 1, C), ws, Hq, Hkv, D)
    with pytest.raises(ValueError, match="y must be"):
        ne.ne_attn_block_fwd(x, g, wqkv, wo, torch.zeros(B, T, C, dtype=torch.float64), ws, Hq,
                             Hkv, D)
    good = dict(dy=x, dx=torch.zeros_like(x), dgamma=torch.zeros_like(g),
                dw_qkv=torch.zeros_like(wqkv), dw_o=torch.zeros_like(wo))
    for name, bad in (("dy", torch.zeros(B, T, C + 4)), ("dx", torch.zeros(B * T, C)),
                      ("dgamma", torch.zeros(C + 1)), ("dw_qkv", torch.zeros(W, C)),
                      ("dw_o", torch.zeros(C, C, dtype=torch.float16))):
        args = dict(good, **{name: bad})
        with pytest.raises(ValueError, match=f"{name} must be"):
            ne.ne_attn_block_bwd(x, g, wqkv, wo, args["dy"], args["dx"], args["dgamma"],
                                 args["dw_qkv"], args["dw_o"], ws, Hq, Hkv, D)


def noalloc(ne, ptrs=None, B=1, Hq=4, Hkv=2, T=64, D=32, causal=1, dtype=0, rope=0.0):
    p = ptrs or [A] * 9
    return ne.load().ne_attn_bwd_noalloc(*[VP(x) for x in p], B, Hq, Hkv, T, D, causal, dtype,
                                         rope, VP(0))


@pytest.mark.parametrize("which", range(9))
def test_noalloc_backward_validates(ne, which):
    p = [A] * 9
    p[which] = 0
    assert noalloc(ne, p) == ne.NE_ERR_NULL
    p[which] = A + 4
    assert noalloc(ne, p) == ne.NE_ERR_ALIGN
    assert noalloc(ne, Hq=4, Hkv=3) == ne.NE_ERR_SHAPE
    assert noalloc(ne, D=48) == ne.NE_ERR_UNSUPPORTED


def test_noalloc_backward_scratch_limit(ne):
    """Shapes whose scratch (ne_attn_workspace_bytes) exceeds the static 64 MiB are refused
    before any launch; the largest workloads it is meant for fit."""
    lim = 64 << 20
    big = dict(B=64, Hq=16, Hkv=4, T=1024, D=64, dtype=1, rope=10000.0)
    assert ne.ne_attn_workspace_bytes(64, 16, 4, 1024, 64, 1, 10000.0) > lim
    assert noalloc(ne, **big) == ne.NE_ERR_SCRATCH
    assert noalloc(ne, B=64, Hq=16, Hkv=4, T=1 << 15, D=64, dtype=0) == ne.NE_ERR_SCRATCH
    for shape in [(16, 16, 4, 1024, 64, 1, 10000.0), (16, 12, 4, 512, 64, 0, 0.0),
                  (4, 12, 4, 4096, 64, 0, 0.0), (8, 16, 4, 1024, 128, 1, 10000.0)]:
        assert 0 < ne.ne_attn_workspace_bytes(*shape) <= lim, shape
