"""CPU-side checks of the C-ABI library: it loads, exports every function the header
declares, agrees with the binding's struct layout, and rejects bad arguments on the host
(these calls return before any GPU work is enqueued)."""
import ctypes as C
import os
import re

import pytest

import asynchronous_moe_expert_amd as M
from asynchronous_moe_expert_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_step.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        from asynchronous_moe_expert_amd import build

        build.build()
    return M.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_three_calls_and_helpers():
    d = _declared()
    for name in ["moe_assemble", "moe_expert_ffn_grouped", "moe_combine_release", "moe_state_reset",
                 "moe_pack_ffn_weights", "moe_ffn_workspace_size", "moe_combine_workspace_size", "moe_strerror",
                 "moe_version", "moe_struct_size"]:
        assert name in d
    assert sorted(N.EXPORTS) == d


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {M.LIB_PATH}").read()
    for name in _declared():
        assert re.search(rf"\bT {name}\b", out), name


def test_struct_layout_and_version(lib):
    for k, s in enumerate(N._STRUCTS):
        assert lib.moe_struct_size(k) == C.sizeof(s)
    assert lib.moe_struct_size(99) == 0
    assert M.moe_version() == 2  # 2: moe_ffn_args.index
    assert M.moe_strerror(0) == "ok" and "NULL" in M.moe_strerror(-1)


def test_workspace_size(lib):
    assert M.moe_ffn_workspace_size(256, 8, 2880, 2880, M.MOE_BF16) == 256 * 2880 * 2
    assert M.moe_ffn_workspace_size(64, 8, 64, 128, M.MOE_F32) == 64 * 128 * 4
    assert M.moe_ffn_workspace_size(3, 1, 64, 64, M.MOE_BF16) == 512  # rounded up to 256 B
    assert M.moe_ffn_workspace_size(1, 1, 64, 64, 7) == 0
    # batches that can take the tiled GEMM path (>= 96 rows per local expert, bf16 activations)
    # also hold 512 fp32 partial tiles of 128 KiB for the split tail units (one per workgroup
    # of a grid of up to 2 workgroups x 256 CUs)
    parts = 512 * 128 * 1024
    assert M.moe_ffn_workspace_size(6554, 32, 4096, 2048, M.MOE_BF16) == 6554 * 2048 * 2 + parts
    assert M.moe_ffn_workspace_size(96 * 32, 32, 4096, 2048, M.MOE_BF16) == 96 * 32 * 2048 * 2 + parts
    assert M.moe_ffn_workspace_size(96 * 32 - 1, 32, 4096, 2048, M.MOE_BF16) == (96 * 32 - 1) * 2048 * 2
    assert M.moe_ffn_workspace_size(4096, 8, 64, 128, M.MOE_F32) == 4096 * 128 * 4  # fp32 path: no GEMM
    # plan path: a 16-byte header, a 16-byte record and an 8-byte list entry per arrival
    assert M.moe_combine_workspace_size(256) == 6160 and M.moe_combine_workspace_size(3) == 96


def test_host_validation_rejects_bad_arguments(lib):
    null = None
    assert lib.moe_assemble(None, null) == -1
    a = N.AssembleArgs(n=4, E_loc=0, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_BF16)
    assert lib.moe_assemble(C.byref(a), null) == -2  # E_loc < 1
    a = N.AssembleArgs(n=4, E_loc=300, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_BF16)
    assert lib.moe_assemble(C.byref(a), null) == -2  # E_loc > 256
    a = N.AssembleArgs(n=4, E_loc=4, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_FP8_E4M3)
    assert lib.moe_assemble(C.byref(a), null) == -3  # fp8 activations not supported
    a = N.AssembleArgs(n=4, E_loc=4, H=60, P=10, pool_pitch=60, act_dtype=M.MOE_BF16, counts=8, offsets=8, err=8)
    assert lib.moe_assemble(C.byref(a), null) == -4  # 120-byte rows are not 16-byte multiples
    a = N.AssembleArgs(n=4, E_loc=4, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_BF16, counts=16, offsets=16, err=16)
    assert lib.moe_assemble(C.byref(a), null) == -1  # slot/expert/pool missing

    f = N.FfnArgs(n=4, E_loc=2, H=96, I=64, act_dtype=M.MOE_BF16, w_dtype=M.MOE_BF16)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -5  # H % 64
    f = N.FfnArgs(n=4, E_loc=2, H=64, I=64, act_dtype=M.MOE_F32, w_dtype=M.MOE_BF16)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -3
    f = N.FfnArgs(n=4, E_loc=2, H=64, I=64, act_dtype=M.MOE_BF16, w_dtype=M.MOE_FP8_E4M3, xb=16, offsets=16,
                  w_gu=16, w_d=16, y=16)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -1  # fp8 scales missing
    f = N.FfnArgs(n=4, E_loc=2, H=64, I=64, act_dtype=M.MOE_BF16, w_dtype=M.MOE_BF16, xb=16, offsets=16,
                  w_gu=16, w_d=16, y=16, workspace=16, workspace_bytes=8)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -6  # workspace too small

    st = N.StateC(acc=16, mask=16, head=16, tgen=16, rflag=16, T_cap=8, H=64)
    c = N.CombineArgs(m=1, K=33, state=st)
    assert lib.moe_combine_release(C.byref(c), null) == -2  # K > 32
    c = N.CombineArgs(m=1, K=4, row_dtype=M.MOE_FP8_E4M3, state=st)
    assert lib.moe_combine_release(C.byref(c), null) == -3
    st2 = N.StateC(acc=16, mask=16, head=16, tgen=16, rflag=16, T_cap=8, H=60)
    c = N.CombineArgs(m=1, K=4, state=st2)
    assert lib.moe_combine_release(C.byref(c), null) == -5  # H % 8
    st3 = N.StateC(acc=0, mask=16, head=16, tgen=16, rflag=16, T_cap=8, H=64)
    assert lib.moe_state_reset(C.byref(st3), 0, null) == -1

    c = N.CombineArgs(m=4, K=2, row_dtype=M.MOE_F32, row_pitch=64, n_rows=4, rows=16, row_idx=16, tok=16,
                      kslot=16, w=16, gen=16, out=16, out_dtype=M.MOE_F32, out_pitch=64, rel_list=16, rel_count=16,
                      err=16, state=st, workspace=16, workspace_bytes=8)
    assert lib.moe_combine_release(C.byref(c), null) == -6  # workspace too small for 4 arrivals

    p = N.PackArgs(E_loc=2, H=64, I=96, w_dtype=M.MOE_BF16)
    assert lib.moe_pack_ffn_weights(C.byref(p), null) == -5


def test_host_validation_of_fused_arguments_and_other_entry_points(lib):
    """Further host-side checks, all returning before anything is enqueued: the FFN's size limits,
    a queue index or combine plan handed to the FFN that does not fit the call, the two halves of
    the combine, and the allocation-free combine's arrival limit."""
    null = None
    base = dict(E_loc=2, H=64, I=64, act_dtype=M.MOE_BF16, w_dtype=M.MOE_BF16, xb=16, offsets=16, w_gu=16,
                w_d=16, y=16, workspace=16, workspace_bytes=1 << 20)
    for n in (-1, (1 << 24) + 1):
        f = N.FfnArgs(n=n, **base)
        assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -2, n
    f = N.FfnArgs(n=4, **dict(base, E_loc=257))
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -2
    # a queue index whose call does not match the FFN's (n, xb given) is MOE_EINVAL_SIZE; one that
    # moe_assemble itself would reject returns moe_assemble's status
    ptrs = dict(slot=16, expert=16, pool=16, perm=16, pos=16, counts=16, offsets=16, err=16, row_slot=16)
    ix = N.AssembleArgs(n=4, E_loc=2, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_BF16, **ptrs)
    f = N.FfnArgs(n=8, index=C.addressof(ix), **base)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -2
    ix_xb = N.AssembleArgs(n=4, E_loc=2, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_BF16, xb=16, **ptrs)
    f = N.FfnArgs(n=4, index=C.addressof(ix_xb), **base)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -2
    ix_bad = N.AssembleArgs(n=4, E_loc=0, H=64, P=10, pool_pitch=64, act_dtype=M.MOE_BF16, **ptrs)
    f = N.FfnArgs(n=4, index=C.addressof(ix_bad), **base)
    assert lib.moe_expert_ffn_grouped(C.byref(f), null) == -2
    # a combine plan handed to the FFN is validated like moe_combine_plan (K > 32, fp8 rows)
    st = N.StateC(acc=16, mask=16, head=16, tgen=16, rflag=16, T_cap=8, H=64)
    for kw, code in ((dict(K=33), -2), (dict(K=4, row_dtype=M.MOE_FP8_E4M3), -3)):
        plan = N.CombineArgs(m=1, state=st, **kw)
        f = N.FfnArgs(n=4, plan=C.addressof(plan), **base)
        assert lib.moe_expert_ffn_grouped(C.byref(f), null) == code, kw
        assert lib.moe_combine_plan(C.byref(plan), null) == code, kw
        assert lib.moe_combine_apply(C.byref(plan), null) == code, kw
    assert lib.moe_combine_plan(None, null) == -1 and lib.moe_combine_apply(None, null) == -1
    # the allocation-free combine: its static scratch holds a fixed number of arrivals
    assert lib.moe_combine_release_noalloc(None, null) == -1
    over = N.CombineArgs(m=int(lib.moe_combine_noalloc_max_arrivals()) + 1, K=4, state=st)
    assert lib.moe_combine_release_noalloc(C.byref(over), null) == -8
