"""C ABI checks that need no GPU: the library loads, exports every entry
point the header declares, its structs match the binding's mirror, and host
argument checks return the documented status codes before touching a GPU."""

import ctypes as C
import os
import re
import subprocess

import pytest
import torch

import top_reduce_amd as tr
from top_reduce_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topreduce.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_entry_points():
    names = _declared()
    for n in ("moe_workspace_size", "moe_plan", "moe_forward", "moe_expand", "moe_grouped_gemm",
              "moe_combine_reduce", "moe_plan_stats", "moe_grouped_gemm_up", "moe_grouped_gemm_down",
              "moe_combine_epilogue", "moe_grouped_gemm_up_x", "moe_grouped_gemm_down_y",
              "moe_combine_reduce_multi", "moe_plan_padded", "moe_compact_rows", "moe_last_error",
              "moe_abi_version", "moe_forward_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = tr.load_library()
    out = subprocess.run(["nm", "-D", "--defined-only", tr.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.moe_abi_version() == B.ABI_VERSION


def test_struct_layout_matches_binding(tmp_path):
    prog = tmp_path / "layout.c"
    fields_d = [f for f, _ in B.Desc._fields_]
    fields_p = [f for f, _ in B.PlanStruct._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "topreduce.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(tr_moe_desc), sizeof(tr_moe_plan));']
    lines += [f'printf("%zu\\n", offsetof(tr_moe_desc, {f}));' for f in fields_d]
    lines += [f'printf("%zu\\n", offsetof(tr_moe_plan, {f}));' for f in fields_p]
    lines += ["return 0;}"]
    prog.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(prog), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == C.sizeof(B.Desc) and vals[1] == C.sizeof(B.PlanStruct)
    got = [getattr(B.Desc, f).offset for f in fields_d] + [getattr(B.PlanStruct, f).offset for f in fields_p]
    assert vals[2:] == got


def _ws(desc):
    return tr.load_library().moe_workspace_size(C.byref(desc))


def test_workspace_size_and_desc_checks():
    lib = tr.load_library()
    good = tr.make_desc(T=16384, K=8, E=32, H=7168, I=2048)
    n = _ws(good)
    # T*K expanded rows of Xe and O (bf16) and of h, plus metadata
    assert n >= 2 * 16384 * 8 * (2 * 7168 + 2048)
    assert _ws(tr.make_desc(T=0, K=8, E=32, H=7168, I=2048)) > 0
    bad = [dict(K=0), dict(K=33), dict(E=0), dict(E=1025), dict(T=-1)]
    for kw in bad:
        args = dict(T=64, K=2, E=8, H=256, I=128)
        args.update(kw)
        assert _ws(tr.make_desc(**args)) == 0, kw
        assert lib.moe_last_error()
    # both dtypes need H a multiple of 8 (16-byte row pieces); any I
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=100, I=128)) == 0
    assert b"multiple of 8" in lib.moe_last_error()
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=100, I=128, dtype=torch.float32)) == 0
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=512, I=64)) > 0
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=2880, I=2880)) > 0
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=136, I=70)) > 0
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=512, I=128)) > 0
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=104, I=72, dtype=torch.float32)) > 0
    d = tr.make_desc(T=8, K=2, E=4, H=64, I=64, flags=3)
    assert _ws(d) == 0


def test_plan_rejects_bad_arguments_before_any_launch():
    lib = tr.load_library()
    d = tr.make_desc(T=64, K=2, E=8, H=256, I=128)
    st = B.PlanStruct()
    need = _ws(d)
    fake = C.c_void_p(1 << 40)          # never dereferenced: checks fail first
    assert lib.moe_plan(C.byref(d), fake, None, need, None, C.byref(st)) == -1
    assert lib.moe_plan(C.byref(d), fake, C.c_void_p((1 << 40) + 8), need, None, C.byref(st)) == -1
    assert lib.moe_plan(C.byref(d), fake, fake, need - 1, None, C.byref(st)) == -3
    assert b"needs" in lib.moe_last_error()
    assert lib.moe_plan(C.byref(d), None, fake, need, None, C.byref(st)) == -1
    assert lib.moe_plan(C.byref(d), fake, fake, need, None, None) == -1
    bad = tr.make_desc(T=64, K=2, E=8, H=256, I=128, dtype=7)
    assert lib.moe_plan(C.byref(bad), fake, fake, need, None, C.byref(st)) == -1


def test_entry_points_reject_null_plan():
    lib = tr.load_library()
    assert lib.moe_forward(None, None, None, None, None, None, None) == -1
    assert lib.moe_expand(None, None, None) == -1
    assert lib.moe_grouped_gemm(None, None, None, None) == -1
    assert lib.moe_grouped_gemm_up(None, None, None) == -1
    assert lib.moe_grouped_gemm_up_x(None, None, None, None) == -1
    assert lib.moe_grouped_gemm_down(None, None, None) == -1
    assert lib.moe_grouped_gemm_down_y(None, None, None, None, None) == -1
    assert lib.moe_combine_reduce_multi(None, None, None, None) == -1
    assert lib.moe_combine_reduce(None, None, None, None, None) == -1
    assert lib.moe_plan_stats(None, None, None) == -1
    empty = B.PlanStruct()            # no workspace
    assert lib.moe_forward(C.byref(empty), None, None, None, None, None, None) == -1
    assert b"workspace" in lib.moe_last_error()


def test_fused_down_is_bf16_only_and_checked_on_the_host():
    lib = tr.load_library()
    st = B.PlanStruct()
    st.d = tr.make_desc(T=8, K=2, E=4, H=104, I=72, dtype=torch.float32)
    fake = C.c_void_p(1 << 40)           # never dereferenced: checks fail first
    st.ws = fake
    assert lib.moe_grouped_gemm_down_y(C.byref(st), fake, None, fake, None) == -2
    assert b"bf16" in lib.moe_last_error()
    st.d = tr.make_desc(T=8, K=2, E=4, H=512, I=128)
    assert lib.moe_grouped_gemm_down_y(C.byref(st), fake, None, None, None) == -1
    assert b"y" in lib.moe_last_error()
    st.d = tr.make_desc(T=150016, K=2, E=2, H=7168, I=128)   # y past 2 GiB
    assert lib.moe_grouped_gemm_down_y(C.byref(st), fake, None, fake, None) == -2


def test_no_xe_flag_drops_the_expanded_buffer():
    lib = tr.load_library()
    T, K, H = 16384, 8, 7168
    full = _ws(tr.make_desc(T=T, K=K, E=32, H=H, I=2048))
    lean = _ws(tr.make_desc(T=T, K=K, E=32, H=H, I=2048, flags=tr.FLAG_NO_XE))
    assert full - lean == (T * K + 256) * H * 2
    # the tiled/stream choice still combines with it
    assert _ws(tr.make_desc(T=64, K=2, E=8, H=256, I=128,
                            flags=tr.FLAG_NO_XE | tr.FLAG_GEMM_FORCE_TILED)) > 0
    # only the gathering GEMM1 can run without Xe: bf16 with x under 2 GiB
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=104, I=72, dtype=torch.float32,
                            flags=tr.FLAG_NO_XE)) == 0
    assert b"TR_FLAG_NO_XE" in lib.moe_last_error()
    assert _ws(tr.make_desc(T=150016, K=2, E=2, H=7168, I=128, flags=tr.FLAG_NO_XE)) == 0
    assert _ws(tr.make_desc(T=8, K=2, E=4, H=64, I=64, flags=0x8)) == 0
    # the entry points over Xe refuse such a plan before any launch
    st = B.PlanStruct()
    st.d = tr.make_desc(T=64, K=2, E=8, H=256, I=128, flags=tr.FLAG_NO_XE)
    fake = C.c_void_p(1 << 40)           # never dereferenced: checks fail first
    st.ws = fake
    assert lib.moe_expand(C.byref(st), fake, None) == -2
    assert b"expanded buffer" in lib.moe_last_error()
    assert lib.moe_grouped_gemm(C.byref(st), fake, fake, None) == -2
    assert lib.moe_grouped_gemm_up(C.byref(st), fake, None) == -2


def test_padded_plan_and_compaction_check_arguments_on_the_host():
    lib = tr.load_library()
    d = tr.make_desc(T=960, K=8, E=32, H=256, I=128)
    st = B.PlanStruct()
    need = _ws(d)
    fake = C.c_void_p(1 << 40)           # never dereferenced: checks fail first
    assert lib.moe_plan_padded(C.byref(d), fake, 0, fake, fake, need, None, C.byref(st)) == -1
    assert b"block_rows" in lib.moe_last_error()
    assert lib.moe_plan_padded(C.byref(d), fake, 120, None, fake, need, None, C.byref(st)) == -1
    assert b"block_counts" in lib.moe_last_error()
    mis = C.c_void_p((1 << 40) + 2)
    assert lib.moe_plan_padded(C.byref(d), fake, 120, mis, fake, need, None, C.byref(st)) == -1
    # at most 4096 blocks
    big = tr.make_desc(T=4097, K=1, E=4, H=256, I=128)
    assert lib.moe_plan_padded(C.byref(big), fake, 1, fake, fake, _ws(big), None,
                               C.byref(st)) == -2
    assert lib.moe_plan_padded(C.byref(d), fake, 120, fake, fake, need - 1, None,
                               C.byref(st)) == -3
    # compaction
    cr = lib.moe_compact_rows
    assert cr(-1, 1, fake, 16, fake, fake, 0, None, None) == -1
    assert cr(8, 0, fake, 16, fake, fake, 0, None, None) == -1
    assert cr(8, 4, fake, 6, fake, fake, 0, None, None) == -1          # row bytes % 4
    assert b"row_bytes" in lib.moe_last_error()
    assert cr(8, 4, fake, 0, fake, fake, 0, None, None) == -1
    assert cr(8, 4, fake, 16, fake, fake, 2, None, None) == -1
    assert cr(8, 4, None, 16, fake, fake, 0, None, None) == -1
    assert cr(8, 4, fake, 16, None, fake, 0, None, None) == -1
    assert cr(8, 4, fake, 16, fake, mis, 0, None, None) == -1
    assert cr(8, 4, fake, 16, fake, fake, 0, mis, None) == -1
    assert cr(4097, 1, fake, 16, fake, fake, 0, None, None) == -2
    assert cr((1 << 31) - 1, 1 << 20, fake, 1 << 40, fake, fake, 0, None, None) == -1
    assert cr(1 << 31, 1 << 20, fake, 16, fake, fake, 0, None, None) == -2   # 32-bit rows
    assert b"2^31" in lib.moe_last_error()
    assert cr(0, 4, None, 16, None, None, 0, None, None) == 0         # nothing to do


def test_forward_rejects_misaligned_buffers():
    lib = tr.load_library()
    st = B.PlanStruct()
    st.d = tr.make_desc(T=64, K=2, E=8, H=256, I=128)
    st.ws = C.c_void_p(1 << 40)
    ok = C.c_void_p(1 << 41)
    mis = C.c_void_p((1 << 41) + 4)
    assert lib.moe_forward(C.byref(st), mis, None, ok, ok, ok, None) == -1
    assert b"aligned" in lib.moe_last_error()
    assert lib.moe_forward(C.byref(st), ok, None, None, ok, ok, None) == -1


def test_combine_epilogue_checks_arguments_on_the_host():
    """Every bad argument is rejected before any launch (no GPU needed);
    T == 0 is a no-op that touches no pointer."""
    lib = tr.load_library()
    ok = C.c_void_p(1 << 41)
    src = C.c_void_p(1 << 42)
    bf16 = B.BF16
    assert lib.moe_combine_epilogue(0, 4, 256, bf16, None, None, 0, None, None) == 0
    assert lib.moe_combine_epilogue(-1, 4, 256, bf16, src, ok, 8, ok, None) == -1
    assert lib.moe_combine_epilogue(2, 0, 256, bf16, src, ok, 8, ok, None) == -1
    assert lib.moe_combine_epilogue(2, 70000, 256, bf16, src, ok, 8, ok, None) == -1
    assert lib.moe_combine_epilogue(2, 4, 12, bf16, src, ok, 8, ok, None) == -2
    assert b"multiple of 8" in lib.moe_last_error()
    assert lib.moe_combine_epilogue(2, 4, 256, 9, src, ok, 8, ok, None) == -1
    assert lib.moe_combine_epilogue(2, 4, 256, bf16, None, ok, 8, ok, None) == -1
    assert lib.moe_combine_epilogue(2, 4, 256, bf16, src, ok, 8, None, None) == -1
    assert lib.moe_combine_epilogue(2, 4, 256, bf16, src, C.c_void_p((1 << 41) + 8), 8, ok, None) == -1
    assert b"aligned" in lib.moe_last_error()
    assert lib.moe_combine_epilogue(2, 4, 256, bf16, src, ok, -1, ok, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_HERE", str(tmp_path))
    monkeypatch.delenv("TOP_REDUCE_LIB", raising=False)
    with pytest.raises(ImportError):
        B.load_library()


def test_noalloc_refuses_batch_past_scratch_on_host():
    """moe_forward_noalloc checks the batch against its static workspace
    before it touches a device: a prefill-sized batch is TR_EUNSUPPORTED (no
    pointer is read), an invalid descriptor TR_EINVAL."""
    lib = tr.load_library()
    big = tr.make_desc(T=16384, K=8, E=32, H=7168, I=2048)
    null = C.c_void_p(None)
    st = lib.moe_forward_noalloc(C.byref(big), null, null, null, null, null, null, null)
    assert st == -2
    assert b"static scratch" in lib.moe_last_error()
    bad = tr.make_desc(T=64, K=0, E=8, H=256, I=128)
    assert lib.moe_forward_noalloc(C.byref(bad), null, null, null, null, null, null, null) == -1
    # the decode batch fits: its descriptor (bf16, no expanded rows) needs
    # less than the scratch holds
    dec = tr.make_desc(T=64, K=16, E=28, H=3584, I=2048, flags=tr.FLAG_NO_XE)
    assert 0 < _ws(dec) <= tr.NOALLOC_SCRATCH_BYTES
