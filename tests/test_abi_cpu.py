"""The C ABI on the CPU: the library loads, exports every function include/idx.h declares,
and rejects bad arguments on the host before touching a device (no GPU needed)."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_score_amd as sai
from sparse_attention_indexer_score_amd import IdxProblem, IdxDebug, IdxStats

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "idx.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sai.LIB_PATH), reason="libidx.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(idx_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("idx_score", "idx_score_workspace", "idx_select", "idx_fused_topk", "idx_select_workspace",
              "idx_fused_workspace", "idx_page_slots", "idx_sparse_attn",
              "idx_strerror", "idx_row_split", "idx_select_split", "idx_version"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(sai.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_struct_sizes_match_the_header_layout():
    # idx_problem: 4 ints, 8 pointers, int64, 2 pointers, 2 ints, 1 pointer (LP64, natural alignment)
    assert ctypes.sizeof(IdxProblem) == 16 + 8 * 8 + 8 + 16 + 8 + 8
    assert ctypes.sizeof(IdxDebug) == 16
    assert ctypes.sizeof(IdxStats) == 6 * 4 + 8 + 4 * 4


def test_version_and_strerror():
    lib = sai.library()
    assert lib.idx_version() == 10000
    assert lib.idx_strerror(0) == b"success"
    for code in (-1, -2, -3, -4, -5, -6):
        assert lib.idx_strerror(code) not in (b"success", b"unknown error")


@pytest.mark.parametrize("rows,row_len,cu,expect", [
    (64, 131072, 256, 4),      # the selection workload: 256 / 64 = 4 workgroups per row
    (1, 65536, 256, 32),       # capped at 32
    (8, 1 << 20, 256, 32),
    (16, 1 << 20, 256, 16),
    (100, 1 << 20, 256, 0),    # 256 / 100 = 2 < 4
    (64, 65535, 256, 0),       # row shorter than 65536
    (0, 1 << 20, 256, 32),     # rows clamped to 1
    (512, 262144, 256, 0),
])
def test_row_split_rule(rows, row_len, cu, expect):
    assert sai.idx_row_split(rows, row_len, cu) == expect


def _problem(**kw):
    p = IdxProblem()
    p.rows, p.heads, p.head_dim, p.fmt = 4, 32, 128, sai.IDX_FMT_E4M3
    fake = 0x10000
    p.q = p.k = p.w = p.ks = p.ke = ctypes.c_void_p(fake)
    p.num_keys = 100
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("mut,code", [
    (dict(heads=48), sai.IDX_EINVAL),
    (dict(head_dim=64), sai.IDX_EINVAL),
    (dict(fmt=3), sai.IDX_EINVAL),
    (dict(rows=-1), sai.IDX_EINVAL),
    (dict(q=None), sai.IDX_EINVAL),
    (dict(q_sf=ctypes.c_void_p(0x20000)), sai.IDX_EFMT),          # block scales with e4m3
    (dict(fmt=sai.IDX_FMT_MXFP4), sai.IDX_EFMT),                   # MXFP4 without block scales
    (dict(q=ctypes.c_void_p(0x10008)), sai.IDX_EALIGN),            # q must be 16-byte aligned
    (dict(ks=ctypes.c_void_p(0x10002)), sai.IDX_EALIGN),
    (dict(page_table=ctypes.c_void_p(0x30000)), sai.IDX_EINVAL),   # paged without row_req
    (dict(num_keys=0), sai.IDX_EINVAL),                              # rows but no keys to read
])
def test_problem_validation_on_host(mut, code):
    lib = sai.library()
    p = _problem(**mut)
    assert lib.idx_score(ctypes.byref(p), ctypes.c_void_p(0x40000), 128, None, 0, None) == code
    assert lib.idx_fused_workspace(ctypes.byref(p), 16) == 0


def test_paged_mxfp4_is_a_format_error():
    lib = sai.library()
    p = _problem(fmt=sai.IDX_FMT_MXFP4, q_sf=ctypes.c_void_p(0x20000), k_sf=ctypes.c_void_p(0x20000),
                 page_table=ctypes.c_void_p(0x30000), row_req=ctypes.c_void_p(0x30000), num_req=1, max_pages=2,
                 num_keys=128)
    assert lib.idx_score(ctypes.byref(p), ctypes.c_void_p(0x40000), 128, None, 0, None) == sai.IDX_EFMT


def test_fused_argument_checks():
    lib = sai.library()
    p = _problem()
    out = ctypes.c_void_p(0x40000)
    assert lib.idx_fused_topk(ctypes.byref(p), 0, out, None, 0, None, None) == sai.IDX_EINVAL
    assert lib.idx_fused_topk(ctypes.byref(p), 2049, out, None, 0, None, None) == sai.IDX_EINVAL
    need = lib.idx_fused_workspace(ctypes.byref(p), 16)
    assert need > 0
    assert lib.idx_fused_topk(ctypes.byref(p), 16, out, ctypes.c_void_p(0x100000), need - 1, None, None) == sai.IDX_EWS
    assert lib.idx_fused_topk(ctypes.byref(p), 16, out, ctypes.c_void_p(0x100080), need, None, None) == sai.IDX_EALIGN
    st = IdxStats()
    p0 = _problem(rows=0)
    assert lib.idx_fused_topk(ctypes.byref(p0), 16, None, None, 0, ctypes.byref(st), None) == 0
    assert st.cap == 64 and st.sample_stride == 1


def test_score_workspace_and_check():
    lib = sai.library()
    assert lib.idx_score_workspace(ctypes.byref(_problem(rows=64, num_keys=4096))) == 0   # e4m3: none
    sf = ctypes.c_void_p(0x20000)
    p = _problem(rows=64, num_keys=4096, fmt=sai.IDX_FMT_MXFP4, q_sf=sf, k_sf=sf)
    need = lib.idx_score_workspace(ctypes.byref(p))
    assert need >= 64 * 780                          # six fp6 pieces of u per row, and their scales
    out = ctypes.c_void_p(0x40000)
    assert lib.idx_score(ctypes.byref(p), out, 4096, None, 0, None) == sai.IDX_EWS
    assert lib.idx_score(ctypes.byref(p), out, 4096, ctypes.c_void_p(0x100000), need - 1, None) == sai.IDX_EWS
    assert lib.idx_score(ctypes.byref(p), out, 4096, ctypes.c_void_p(0x100080), need, None) == sai.IDX_EALIGN
    paged = _problem(rows=4, page_table=ctypes.c_void_p(0x30000), row_req=ctypes.c_void_p(0x30000), num_req=1,
                     max_pages=2, num_keys=128)
    assert lib.idx_score_workspace(ctypes.byref(paged)) == 0        # paged keys are e4m3


def test_fused_workspace_grows_with_k_and_cap():
    lib = sai.library()
    p = _problem(rows=64, num_keys=4096)
    a = lib.idx_fused_workspace(ctypes.byref(p), 512)
    b = lib.idx_fused_workspace(ctypes.byref(p), 2048)
    assert 0 < a < b
    dbg = IdxDebug(cap=16, threshold_mode=0, threshold_row_mod=0)
    p.debug = ctypes.pointer(dbg)
    assert lib.idx_fused_workspace(ctypes.byref(p), 512) < a


def test_select_argument_checks():
    lib = sai.library()
    x = ctypes.c_void_p(0x10000)
    n = ctypes.c_void_p(0x20000)
    o = ctypes.c_void_p(0x30000)
    assert lib.idx_select(x, 1024, None, n, 4, 0, o, None, 0, None) == sai.IDX_EINVAL
    assert lib.idx_select(x, 1024, None, n, 4, 4096, o, None, 0, None) == sai.IDX_EINVAL
    assert lib.idx_select(None, 1024, None, n, 4, 16, o, None, 0, None) == sai.IDX_EINVAL
    assert lib.idx_select(ctypes.c_void_p(0x10002), 1024, None, n, 4, 16, o, None, 0, None) == sai.IDX_EALIGN
    assert lib.idx_select_split(x, 1024, None, n, 4, 16, o, None, 0, 1, None) == sai.IDX_EINVAL
    assert lib.idx_select_split(x, 1024, None, n, 4, 16, o, None, 0, 33, None) == sai.IDX_EINVAL
    assert lib.idx_select(x, 1024, None, n, 0, 16, o, None, 0, None) == 0     # zero rows: nothing to do
    assert lib.idx_select_workspace(64, 131072, 2048) > 64 * 4096 * 4


def test_sample_stride_is_odd():
    lib = sai.library()
    for k, s in ((2048, 71), (1024, 35), (512, 17), (16, 1)):
        p = _problem(rows=4, num_keys=1000)
        st = IdxStats()
        p0 = _problem(rows=0)
        assert lib.idx_fused_topk(ctypes.byref(p0), k, None, None, 0, ctypes.byref(st), None) == 0
        assert st.sample_stride == s and st.sample_stride % 2 == 1


def test_page_slots_argument_checks():
    lib = sai.library()
    a = ctypes.c_void_p(0x10000)
    assert lib.idx_page_slots(a, -1, 4, None, a, a, 2, a, None) == sai.IDX_EINVAL
    assert lib.idx_page_slots(a, 2, 0, None, a, a, 2, a, None) == sai.IDX_EINVAL
    assert lib.idx_page_slots(a, 2, 4, None, a, a, 0, a, None) == sai.IDX_EINVAL
    assert lib.idx_page_slots(None, 2, 4, None, a, a, 2, a, None) == sai.IDX_EINVAL
    assert lib.idx_page_slots(ctypes.c_void_p(0x10002), 2, 4, None, a, a, 2, a, None) == sai.IDX_EALIGN
    assert lib.idx_page_slots(None, 0, 4, None, None, None, 2, None, None) == 0    # nothing to do


def test_sparse_attn_argument_checks():
    """Host-side validation of idx_sparse_attn; every case returns before any device call."""
    lib = sai.library()
    a = ctypes.c_void_p(0x10000)
    f = lambda q=a, kc=a, vc=a, ns=100, sl=a, rows=2, hq=24, hkv=2, width=8, ss=0.1, os_=1.0, out=a: \
        lib.idx_sparse_attn(q, kc, vc, ns, sl, rows, hq, hkv, width, ss, os_, out, None)
    assert f(rows=-1) == sai.IDX_EINVAL
    assert f(width=-1) == sai.IDX_EINVAL
    assert f(hkv=0) == sai.IDX_EINVAL
    assert f(hq=25) == sai.IDX_EINVAL                    # not a multiple of hkv
    assert f(hq=66, hkv=2) == sai.IDX_EINVAL             # 33 query heads per KV head
    assert f(ns=0) == sai.IDX_EINVAL
    assert f(ss=float("nan")) == sai.IDX_EINVAL
    assert f(os_=float("inf")) == sai.IDX_EINVAL
    assert f(q=None) == sai.IDX_EINVAL
    assert f(sl=None) == sai.IDX_EINVAL                  # slots needed when width > 0
    assert f(q=ctypes.c_void_p(0x10008)) == sai.IDX_EALIGN
    assert f(kc=ctypes.c_void_p(0x10004)) == sai.IDX_EALIGN
    assert f(out=ctypes.c_void_p(0x10002)) == sai.IDX_EALIGN
    assert f(rows=0, q=None, kc=None, vc=None, sl=None, out=None) == 0   # nothing to do


def test_debug_hooks_are_validated_on_the_host():
    """Out-of-range debug overrides are rejected before any device work (tie_cap within
    1..4096, 0 = default; threshold_mode 0..2; cap >= 0)."""
    lib = sai.library()
    p = _problem(rows=4, num_keys=1000)
    out = ctypes.c_void_p(0x40000)
    ws = ctypes.c_void_p(0x100000)
    for dbg in (IdxDebug(tie_cap=-1), IdxDebug(tie_cap=4097), IdxDebug(threshold_mode=3), IdxDebug(cap=-5)):
        p.debug = ctypes.pointer(dbg)
        assert lib.idx_fused_topk(ctypes.byref(p), 64, out, ws, 1 << 30, None, None) == sai.IDX_EINVAL


def test_split_gate_of_the_workloads():
    """Row split on 256 CUs: the selection workload (64 rows of pitch 131072) gets g = 4;
    the decode batch (512 rows) and the prefill batch (4096 rows of 65536) get 256 / rows < 4
    workgroups per row, so the split is off; 8 rows split 32 ways once a row reaches 65536."""
    assert sai.idx_row_split(64, 131072, 256) == 4
    assert sai.idx_row_split(512, 262144, 256) == 0
    assert sai.idx_row_split(4096, 65536, 256) == 0
    assert sai.idx_row_split(8, 65535, 256) == 0
    assert sai.idx_row_split(8, 65536, 256) == 32


def test_noalloc_checks_on_the_host():
    """idx_fused_topk_noalloc validates like idx_fused_topk and rejects problems whose
    workspace exceeds the fixed scratch before any device work."""
    lib = sai.library()
    out = ctypes.c_void_p(0x40000)
    assert lib.idx_fused_topk_noalloc(ctypes.byref(_problem(heads=48)), 64, out, None) == sai.IDX_EINVAL
    assert lib.idx_fused_topk_noalloc(ctypes.byref(_problem()), 0, out, None) == sai.IDX_EINVAL
    big = _problem(rows=4096, num_keys=65536, heads=64)
    assert lib.idx_fused_workspace(ctypes.byref(big), 2048) > sai.IDX_NOALLOC_SCRATCH_BYTES
    assert lib.idx_fused_topk_noalloc(ctypes.byref(big), 2048, out, None) == sai.IDX_ESCRATCH
    assert b"scratch" in lib.idx_strerror(sai.IDX_ESCRATCH)
