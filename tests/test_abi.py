"""The C ABI on the host: the library loads, exports every entry point that
include/dsa.h declares, and rejects bad arguments with the documented status
before anything reaches the GPU (these calls never launch a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_05_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    from sparse_attention_05_amd import dsa as mod
    return mod


def test_header_lists_the_entry_points():
    fns = header_functions()
    for name in ("dsa_index_scores", "dsa_index_scores_decode", "dsa_topk", "dsa_sparse_mla_attn",
                 "dsa_decode_fused",
                 "dsa_workspace_size", "dsa_status_string", "dsa_last_error"):
        assert name in fns


def test_library_exports_every_declared_symbol(dsa):
    lib = ctypes.CDLL(dsa.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name
    assert sorted(dsa.SIGNATURES) == header_functions()


def test_status_strings(dsa):
    for s in range(8):
        assert dsa.dsa_status_string(s) and dsa.dsa_status_string(s) != "unknown status"
    assert dsa.dsa_status_string(99) == "unknown status"


# Fake device addresses: validation fails before any pointer is used.
A = 0x10000      # 16-B aligned
MIS = 0x10004    # misaligned


def _index(lib, **kw):
    args = dict(q=A, qdt=1, w=A, k=A, kdt=1, ks=None, rows=100, off=A, B=1, qseq=None, qpos=A, R=1,
                HI=64, DI=128, max_n=100, sc=A, ld=100)
    args.update(kw)
    return lib.dsa_index_scores(args["q"], args["qdt"], args["w"], args["k"], args["kdt"], args["ks"],
                                args["rows"], args["off"], args["B"], args["qseq"], args["qpos"], args["R"],
                                args["HI"], args["DI"], args["max_n"], args["sc"], args["ld"], None)


def test_index_scores_rejects(dsa):
    lib = dsa.lib
    assert _index(lib, q=None) == dsa.DSA_ERR_NULL
    assert _index(lib, kdt=2) == dsa.DSA_ERR_NULL          # fp8 keys need a scale array
    assert _index(lib, HI=65) == dsa.DSA_ERR_UNSUPPORTED
    assert _index(lib, DI=96) == dsa.DSA_ERR_UNSUPPORTED
    assert _index(lib, qdt=0, kdt=1) == dsa.DSA_ERR_DTYPE
    assert _index(lib, qdt=0, kdt=2, ks=A) == dsa.DSA_ERR_DTYPE
    assert _index(lib, k=MIS) == dsa.DSA_ERR_ALIGN
    assert _index(lib, sc=MIS) == dsa.DSA_ERR_ALIGN
    assert _index(lib, ld=99) == dsa.DSA_ERR_SHAPE            # ld < max_n
    assert _index(lib, ld=102, max_n=100) == dsa.DSA_ERR_SHAPE  # ld % 4 != 0
    assert _index(lib, R=2, B=1) == dsa.DSA_ERR_SHAPE         # no q_seq needs R == B
    assert _index(lib, max_n=0) == dsa.DSA_ERR_SHAPE


def test_index_scores_decode_rejects(dsa):
    lib = dsa.lib
    def call(**kw):
        a = dict(q=A, qdt=1, w=A, keys=A, kdt=1, ksc=None, rows=4 * 32768, off=A, sl=A, B=4, m=4, HI=64, DI=128,
                 ml=32768, sc=A, ld=32768)
        a.update(kw)
        return lib.dsa_index_scores_decode(a["q"], a["qdt"], a["w"], a["keys"], a["kdt"], a["ksc"], a["rows"],
                                           a["off"], a["sl"], a["B"], a["m"], a["HI"], a["DI"], a["ml"], a["sc"],
                                           a["ld"], None)
    assert call(sl=None) == dsa.DSA_ERR_NULL
    assert call(m=0) == dsa.DSA_ERR_UNSUPPORTED
    assert call(m=9) == dsa.DSA_ERR_UNSUPPORTED
    assert call(ld=32766) == dsa.DSA_ERR_SHAPE
    assert call(kdt=2) == dsa.DSA_ERR_NULL         # fp8 keys without their row scales
    assert call(sc=MIS) == dsa.DSA_ERR_ALIGN


def test_topk_rejects(dsa):
    lib = dsa.lib
    assert lib.dsa_topk(None, 128, A, 1, 100, 64, A, None, 0, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_topk(A, 128, A, 1, 100, 0, A, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(A, 4096, A, 1, 4000, 2049, A, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(A, 1 << 21, A, 1, (1 << 20) + 1, 64, A, None, 0, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(A, 99, A, 1, 100, 64, A, None, 0, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_topk(MIS, 128, A, 1, 100, 64, A, None, 0, None) == dsa.DSA_ERR_ALIGN


def test_sparse_mla_rejects(dsa):
    lib = dsa.lib
    def call(**kw):
        a = dict(q=A, dt=1, lat=A, ldt=1, lsc=None, rows=100, off=A, B=4, qseq=None, idx=A, k=2048, R=4, H=64,
                 out=A, ws=None, wsb=0)
        a.update(kw)
        return lib.dsa_sparse_mla_attn(a["q"], a["dt"], a["lat"], a["ldt"], a["lsc"], a["rows"], a["off"], a["B"],
                                       a["qseq"], a["idx"], a["k"], a["R"], a["H"], 0.1, a["out"], None, a["ws"],
                                       a["wsb"], None)
    assert call(idx=None) == dsa.DSA_ERR_NULL
    assert call(dt=2, ldt=2) == dsa.DSA_ERR_DTYPE
    assert call(ldt=0) == dsa.DSA_ERR_DTYPE                  # latent dtype differs, not fp8
    assert call(ldt=2) == dsa.DSA_ERR_NULL                   # fp8 latent without its row scales
    assert call(dt=0, ldt=2, lsc=A) == dsa.DSA_ERR_DTYPE     # fp8 latent needs bf16 queries
    assert call(ldt=2, lsc=A + 2) == dsa.DSA_ERR_ALIGN
    assert call(k=4096) == dsa.DSA_ERR_UNSUPPORTED
    assert call(H=129) == dsa.DSA_ERR_UNSUPPORTED
    assert call(lat=MIS) == dsa.DSA_ERR_ALIGN
    need = dsa.dsa_workspace_size(dsa.DSA_ENTRY_SPARSE_MLA, 4, 0, 2048, 64)
    assert need > 0
    assert call(ws=A, wsb=need - 256) == dsa.DSA_ERR_WORKSPACE


def test_decode_rejects_small_workspace(dsa):
    lib = dsa.lib
    need = dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, 4, 32768, 2048, 64)
    assert need % 256 == 0 and need >= 4 * 32768 * 4 + 4 * 2048 * 4
    st = lib.dsa_decode_fused(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, A, A, 4, 1, 32768, 64, 128, 64, 2048,
                              0.07, A, None, None, A, need - 1, None)
    assert st == dsa.DSA_ERR_WORKSPACE
    st = lib.dsa_decode_fused(A, A, A, 1, None, A, A, 1, 2, A, 4 * 32768, A, A, 4, 1, 32768, 64, 128, 64, 2048,
                              0.07, A, None, None, A, need - 1, None)
    assert st == dsa.DSA_ERR_WORKSPACE                       # fp8 latent accepted up to the workspace
    st = lib.dsa_decode_fused(A, A, A, 1, None, A, A, 1, 2, None, 4 * 32768, A, A, 4, 1, 32768, 64, 128, 64, 2048,
                              0.07, A, None, None, A, need, None)
    assert st == dsa.DSA_ERR_NULL
    st = lib.dsa_decode_fused(A, A, A, 1, None, A, A, 2, 2, A, 4 * 32768, A, A, 4, 1, 32768, 64, 128, 64, 2048,
                              0.07, A, None, None, A, need, None)
    assert st == dsa.DSA_ERR_DTYPE
    # several new tokens per sequence: the workspace is sized by rows = B * q_per_seq
    need4 = dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, 16, 32768, 2048, 64)
    assert need4 > need
    st = lib.dsa_decode_fused(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, A, A, 4, 4, 32768, 64, 128, 64,
                              2048, 0.07, A, None, None, A, need, None)
    assert st == dsa.DSA_ERR_WORKSPACE
    for bad in (0, 9):
        st = lib.dsa_decode_fused(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, A, A, 4, bad, 32768, 64, 128,
                                  64, 2048, 0.07, A, None, None, A, need4, None)
        assert st == dsa.DSA_ERR_UNSUPPORTED


def test_decode_noalloc_rejects_before_any_device_call(dsa):
    """The no-allocation step refuses bad shapes and steps larger than its
    per-device scratch on the host (no device call is made for these)."""
    lib = dsa.lib
    limit = dsa.dsa_decode_noalloc_limit()
    assert limit == 64 << 20
    # 16 rows of 2^20 keys need more workspace than the scratch holds
    big = dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, 16, 1 << 20, 2048, 64)
    assert big > limit
    st = lib.dsa_decode_fused_noalloc(A, A, A, 1, None, A, A, 1, 1, None, 16 << 20, A, A, 16, 1, 1 << 20, 64, 128,
                                      64, 2048, 0.07, A, None, None, None)
    assert st == dsa.DSA_ERR_WORKSPACE
    assert b"scratch" in lib.dsa_last_error()
    for bad in (0, 9):
        st = lib.dsa_decode_fused_noalloc(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, A, A, 4, bad, 32768, 64,
                                          128, 64, 2048, 0.07, A, None, None, None)
        assert st == dsa.DSA_ERR_UNSUPPORTED
    st = lib.dsa_decode_fused_noalloc(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, A, A, 0, 1, 32768, 64, 128,
                                      64, 2048, 0.07, A, None, None, None)
    assert st == dsa.DSA_ERR_SHAPE
    st = lib.dsa_decode_fused_noalloc(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, A, A, 4, 1, 32768, 64, 128,
                                      64, 4096, 0.07, A, None, None, None)
    assert st == dsa.DSA_ERR_UNSUPPORTED


def test_check_indices_rejects(dsa):
    lib = dsa.lib
    assert lib.dsa_check_indices(A, A, 4, 2048, None, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_check_indices(None, A, 4, 2048, A, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_check_indices(A, A, -1, 2048, A, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_check_indices(A, A, 4, 0, A, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_check_indices(A, A, 4, 2049, A, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_check_indices(None, None, 0, 64, A, None) == dsa.DSA_OK  # nothing to check


def test_read_probe_rejects_before_any_device_call(dsa):
    lib = dsa.lib
    assert lib.dsa_read_probe(None, 1024, A, 256, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_read_probe(A, 1024, None, 256, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_read_probe(A, 0, A, 256, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_read_probe(A, 1000, A, 256, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_read_probe(A + 8, 1024, A, 256, None) == dsa.DSA_ERR_ALIGN


def test_workspace_sizes_are_aligned(dsa):
    for rows, k, H in [(1, 64, 8), (4, 2048, 64), (16, 2048, 64), (8192, 2048, 64)]:
        assert dsa.dsa_workspace_size(dsa.DSA_ENTRY_SPARSE_MLA, rows, 0, k, H) % 256 == 0
    # top-k: few long rows get a split-selection workspace (candidates + state),
    # short rows or many rows need none
    need = dsa.dsa_workspace_size(dsa.DSA_ENTRY_TOPK, 4, 32768, 2048, 64)
    assert need >= 4 * 4096 * 8 + 4 * 16
    assert dsa.dsa_workspace_size(dsa.DSA_ENTRY_TOPK, 4, 8192, 2048, 64) == 0
    assert dsa.dsa_workspace_size(dsa.DSA_ENTRY_TOPK, 4096, 32768, 2048, 64) == 0


def test_context_parallel_entries_reject(dsa):
    lib = dsa.lib
    assert lib.dsa_topk_pairs(None, 8, A, 1, 4, 0, A, A, None) == dsa.DSA_ERR_NULL
    assert lib.dsa_topk_pairs(A, 8, A, 1, 4, -1, A, A, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_topk_merge(A, A, 9, 1, 4, A, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_merge(A, A, 0, 1, 4, A, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_merge(A, A, 2, 1, 0, A, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_shard_indices(A, 1, 4, 5, 3, A, None) == dsa.DSA_ERR_SHAPE
    assert lib.dsa_attn_merge(A, A, 9, 1, 4, A, None, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_attn_merge(MIS, A, 2, 1, 4, A, None, None) == dsa.DSA_ERR_ALIGN


def test_paged_entries_reject(dsa):
    lib = dsa.lib
    need = dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, 4, 32768, 2048, 64)

    def fused(table=A, max_pages=512, page=64, ws=need):
        return lib.dsa_decode_fused_paged(A, A, A, 1, None, A, A, 1, 1, None, 4 * 32768, table, max_pages, page,
                                          A, 4, 1, 32768, 64, 128, 64, 2048, 0.07, A, None, None, A, ws, None)
    assert fused(table=None) == dsa.DSA_ERR_NULL
    assert fused(page=96) == dsa.DSA_ERR_UNSUPPORTED       # not a power of two
    assert fused(page=32) == dsa.DSA_ERR_UNSUPPORTED       # below one 64-key group
    assert fused(max_pages=511) == dsa.DSA_ERR_SHAPE       # the table cannot hold max_len
    assert fused(ws=need - 1) == dsa.DSA_ERR_WORKSPACE

    def attn(table=A, page=64):
        return lib.dsa_sparse_mla_attn_paged(A, 1, A, 1, None, 100000, table, 64, page, 4, None, A, 2048, 4, 64,
                                             0.1, A, None, None, 0, None)
    assert attn(table=None) == dsa.DSA_ERR_NULL
    assert attn(page=100) == dsa.DSA_ERR_UNSUPPORTED
