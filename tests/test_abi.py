"""The C ABI on the CPU: the library loads, exports every entry point that
include/hga.h declares, the ctypes struct matches the C layout, and invalid
arguments are rejected with the documented codes before any device work."""
import ctypes
import os
import re
import subprocess

import pytest

from hierarchical_sparse_attention_build_amd import hga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hga.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hga.LIB_PATH):
        from hierarchical_sparse_attention_build_amd import build
        build.build()
    return hga.lib()


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(hga_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 12, names
    out = subprocess.run(["nm", "-D", "--defined-only", hga.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (hga_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None
    assert set(names) == set(hga.EXPORTS)


def test_params_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "hga.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu\\n", sizeof(hga_params),'
                   ' offsetof(hga_params, top_g), offsetof(hga_params, rope_base),'
                   ' offsetof(hga_params, hf_threshold), offsetof(hga_params, out_dtype));return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()))
    P = hga.HGAParams
    assert got == [ctypes.sizeof(P), P.top_g.offset, P.rope_base.offset, P.hf_threshold.offset,
                   P.out_dtype.offset]


def good(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, chunk_size=64, group_size=16,
                n_sink=1, n_local=2, top_k=4, top_g=8, rope_base=5e5)
    base.update(kw)
    return hga.params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -2), (dict(n_kv_heads=3), -2), (dict(n_q_heads=24, n_kv_heads=8), -5),
    (dict(head_dim=96), -5), (dict(chunk_size=0), -2), (dict(chunk_size=512), -2),
    (dict(group_size=24), -2), (dict(group_size=0), -2), (dict(chunk_size=128, group_size=1), -5),
    (dict(n_sink=-1), -1), (dict(top_k=2000), -1), (dict(top_g=-3), -1), (dict(rope_base=1.0), -1),
    (dict(rope_base=float("inf")), -1), (dict(hf_threshold=-0.5), -1), (dict(qkv_dtype=7), -1),
])
def test_invalid_params_rejected(L, kw, code):
    p = good(**kw)
    assert hga.lib().hga_workspace_size(ctypes.byref(p), hga.OP_DECODE, 1, 4096) == 0
    assert hga.last_error()
    st = L.hga_route(ctypes.byref(p), None, 1, None, None, None, 4096, None, None, None, None, 0, None)
    assert st == code, (kw, st, hga.last_error())


def test_null_misaligned_and_workspace_errors(L):
    p = good()
    fake = 0x10000  # aligned, never dereferenced: every call below fails validation first
    P = ctypes.byref(p)
    # null pointer
    assert L.hga_decode(P, None, fake, fake, 4096, fake, fake, fake, fake, None, None, fake, 1 << 30, None) == -1
    # misaligned
    assert L.hga_decode(P, fake + 2, fake, fake, 4096, fake, fake, fake, fake, None, None, fake, 1 << 30, None) == -3
    # workspace too small / missing
    need = hga.workspace_size(p, hga.OP_DECODE, 1, 4096)
    assert need > 0
    assert L.hga_decode(P, fake, fake, fake, 4096, fake, fake, fake, fake, None, None, fake, need - 1, None) == -4
    assert L.hga_decode(P, fake, fake, fake, 4096, fake, fake, fake, fake, None, None, None, 0, None) == -4
    # capacity not a multiple of C, nq not a multiple of C in prefill
    assert L.hga_decode(P, fake, fake, fake, 4000, fake, fake, fake, fake, None, None, fake, 1 << 30, None) == -2
    assert L.hga_route(P, fake, 100, fake, fake, fake, 4096, fake, fake, None, fake, 1 << 30, None) == -2
    # scores_out is a decode-only output
    assert L.hga_route(P, fake, 128, fake, fake, fake, 4096, fake, fake, fake, fake, 1 << 30, None) == -1
    # summary range outside the capacity; K_rot_out with rotated keys
    assert L.hga_build_summaries(P, fake, 4096, 0, 65, 1, None, fake, fake, None) == -2
    assert L.hga_build_summaries(P, fake, 4096, 0, 8, 1, fake, fake, fake, None) == -1
    # offload: staging too small
    st = L.hga_decode_offload(P, fake, fake, fake, fake, fake, 4096, fake, fake, fake, fake, None, None,
                              fake, 16, fake, 1 << 30, None, None)
    assert st == -4 and "staging" in hga.last_error()


def test_workspace_sizes_grow_with_problem(L):
    p = good()
    a = hga.workspace_size(p, hga.OP_DECODE, 1, 4096)
    b = hga.workspace_size(p, hga.OP_DECODE, 1, 65536)
    assert 0 < a < b
    c = hga.workspace_size(p, hga.OP_PREFILL, 4096, 4096)
    assert 0 < c < hga.workspace_size(p, hga.OP_PREFILL, 8192, 8192)
    assert hga.workspace_size(p, hga.OP_ROUTE, 1, 4096) < a
    assert hga.lib().hga_workspace_size(ctypes.byref(p), 9, 1, 4096) == 0


def test_warm_tier_argument_errors(L):
    """The warm-tier entry point rejects a missing state and a slot count below
    top_g (or above the limit) before launching anything."""
    p = good()
    fake = 0x10000
    P = ctypes.byref(p)
    args = (fake, fake, fake, fake, fake, 4096, fake, fake, fake, fake, None, None)
    assert L.hga_decode_offload_warm(P, *args, None, fake, 1 << 30, None, None) == -1
    assert "warm" in hga.last_error()
    for slots in (p.top_g - 1, 4096):
        w = hga.HGAWarm(fake, fake, fake, fake, fake, None, None, slots)
        assert L.hga_decode_offload_warm(P, *args, ctypes.byref(w), fake, 1 << 30, None, None) == -1
        assert "slots" in hga.last_error()
    w = hga.HGAWarm(None, fake, fake, fake, fake, None, None, p.top_g)
    assert L.hga_decode_offload_warm(P, *args, ctypes.byref(w), fake, 1 << 30, None, None) == -1


def test_prefill_workspace_holds_the_converted_tables(L):
    """With bf16 inputs a prefill's workspace holds the fp16 copy of V and the
    summary tables split into bf16 high and low parts; with fp32 inputs it does
    not (those kernels do not run)."""
    kw = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, chunk_size=64, group_size=16,
              n_sink=1, n_local=2, top_k=32, top_g=64, rope_base=5e5)
    n = 8192
    pb = hga.params(**kw, qkv_dtype=hga.HGA_BF16)
    pf = hga.params(**kw, qkv_dtype=hga.HGA_F32)
    v16 = 1 * 8 * n * 128 * 2
    split = 1 * 8 * (n // 64) * (1 + 4) * 128 * 2 * 2
    for op in (hga.OP_ATTEND, hga.OP_PREFILL):
        assert hga.workspace_size(pb, op, n, n) >= hga.workspace_size(pf, op, n, n) + v16
    assert hga.workspace_size(pb, hga.OP_PREFILL, n, n) >= hga.workspace_size(pf, hga.OP_PREFILL, n, n) + v16 + split
    # one query per sequence: neither table
    assert hga.workspace_size(pb, hga.OP_ATTEND, 1, n) < v16



def test_decode_static_rejects_unsupported_shapes(L):
    """The no-workspace decode rejects, before any device work, shapes outside
    its one-launch kernel and more units than its static scratch holds."""
    fake = 0x10000
    args = (fake, fake, fake, 4096, fake, fake, fake, fake, None, None, None)
    p = good(n_q_heads=16, n_kv_heads=2)  # 8 query heads per KV head
    assert L.hga_decode_static(ctypes.byref(p), *args) == -5
    assert "hga_decode_static" in hga.last_error()
    p = good(batch=600, n_q_heads=8, n_kv_heads=2)  # 1200 units
    assert L.hga_decode_static(ctypes.byref(p), *args) == -2
    assert "B*Hkv" in hga.last_error()
    p = good()
    assert L.hga_decode_static(ctypes.byref(p), None, *args[1:]) == -1


def test_prefill_row_cap_only_for_the_splitk_path(L):
    """A 64K prefill is accepted by validation; with fp32 inputs (the split-K
    attention, which carries the row in grid.y) more than 65535 rows are
    rejected with HGA_ERR_UNSUPPORTED before anything is launched."""
    fake = 0x10000
    n = 65536
    pf = hga.params(1, 32, 8, 128, 64, 16, 1, 2, 32, 64, 5e5, qkv_dtype=hga.HGA_F32)
    assert hga.workspace_size(pf, hga.OP_PREFILL, n, n) > 0
    st = L.hga_prefill(ctypes.byref(pf), fake, fake, fake, n, fake, fake, fake, None, None, fake, 1 << 40, None)
    assert st == -5 and "65535" in hga.last_error()
    pb = hga.params(1, 32, 8, 128, 64, 16, 1, 2, 32, 64, 5e5, qkv_dtype=hga.HGA_BF16)
    assert hga.workspace_size(pb, hga.OP_PREFILL, n, n) > 0
