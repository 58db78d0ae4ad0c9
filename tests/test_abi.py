"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sparse_attn.h, and rejects bad arguments on the host before
anything is enqueued (validation runs before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def lib():
    from top_indexer_sparse_amd import api
    return api.load()


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared()
    for n in ("sparse_attn_indexer_scores", "sparse_attn_topk", "sparse_attn_mla_forward",
              "sparse_attn_decode", "sparse_attn_workspace_bytes", "sparse_attn_status_string",
              "sparse_attn_last_error", "sparse_attn_block_pool", "sparse_attn_block_decode",
              "sparse_attn_csa_decode", "sparse_attn_prefill_select", "sparse_attn_prefill"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from top_indexer_sparse_amd import api
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sparse_attn_\w+)", out))
    for n in declared():
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(api.EXPORTS) == set(declared())


def test_library_carries_gfx950_code_objects():
    from top_indexer_sparse_amd import api
    blob = open(api.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def _err(lib):
    return lib.sparse_attn_last_error().decode()


def test_status_strings(lib):
    assert lib.sparse_attn_status_string(0) == b"SA_OK"
    assert lib.sparse_attn_status_string(7) == b"SA_ERR_HIP"
    assert lib.sparse_attn_status_string(99) == b"SA_UNKNOWN_STATUS"


P = ctypes.c_void_p
A = P(0x10000)  # aligned dummy device address; never dereferenced by validation
M = P(0x10004)  # misaligned


def test_indexer_validation(lib):
    f = lib.sparse_attn_indexer_scores
    # NULL required pointer
    assert f(None, 1, A, A, 1, None, None, None, 1, 1, 8, 64, 128, A, None) == 1
    # bad dtype
    assert f(A, 5, A, A, 1, None, None, None, 1, 1, 8, 64, 128, A, None) == 3
    # fp8 keys without scales
    assert f(A, 1, A, A, 2, None, None, None, 1, 1, 8, 64, 128, A, None) == 1
    # unsupported dI
    assert f(A, 1, A, A, 1, None, None, None, 1, 1, 8, 64, 96, A, None) == 5
    assert "dI=96" in _err(lib)
    # misaligned
    assert f(M, 1, A, A, 1, None, None, None, 1, 1, 8, 64, 128, A, None) == 4
    # negative size
    assert f(A, 1, A, A, 1, None, None, None, -1, 1, 8, 64, 128, A, None) == 2


def test_topk_validation(lib):
    f = lib.sparse_attn_topk
    assert f(None, None, None, 1, 1, 8, 4, A, None, None, 0, None) == 1
    assert f(A, None, None, 1, 1, 8, 0, A, None, None, 0, None) == 2
    assert f(A, None, None, 1, 1, 8, 5000, A, None, None, 0, None) == 5
    # a long row needs a workspace
    assert f(A, None, None, 1, 1, 100000, 2048, A, None, None, 0, None) == 6
    assert lib.sparse_attn_workspace_bytes(0, 1, 1, 100000, 2048, 0, 0) > 0
    # few rows of >= 8192 positions are split over work-groups: per row and
    # 4096-position chunk, four counts, the bracket and 4096 (key, position)
    assert lib.sparse_attn_workspace_bytes(0, 1, 1, 32768, 2048, 0, 0) == 8 * (24 + 8 * 4096)
    assert f(A, None, None, 1, 1, 32768, 2048, A, None, None, 0, None) == 6
    # rows that fill the GPU, and short rows, need none
    assert lib.sparse_attn_workspace_bytes(0, 1, 200, 32768, 2048, 0, 0) == 0
    assert lib.sparse_attn_workspace_bytes(0, 1, 1, 4096, 2048, 0, 0) == 0


def test_mla_validation(lib):
    f = lib.sparse_attn_mla_forward
    F = ctypes.c_float(0.1)
    # dtype mismatch
    assert f(A, A, 1, A, A, 0, 576, 576, A, 64, 1, 1, 10, 128, 512, 64, F, A, None, None, 0, None) == 3
    # unsupported shape on the bf16 path (H not a multiple of 64 and too big for the vector path)
    assert f(A, A, 1, A, A, 1, 576, 576, A, 64, 1, 1, 10, 100, 512, 64, F, A, None, None, 0, None) == 5
    # stride shorter than the row
    assert f(A, A, 1, A, A, 1, 500, 576, A, 64, 1, 1, 10, 128, 512, 64, F, A, None, None, 0, None) == 2
    # row stride breaking alignment (fp32, 161 elements)
    assert f(A, A, 0, A, A, 0, 161, 161, A, 64, 1, 1, 10, 8, 128, 32, F, A, None, None, 0, None) == 4
    # missing workspace for a KV split (B=1, k=2048 splits over work-groups)
    assert lib.sparse_attn_workspace_bytes(1, 1, 1, 32768, 2048, 128, 512) > 0
    assert f(A, A, 1, A, A, 1, 576, 576, A, 2048, 1, 1, 32768, 128, 512, 64, F, A, None, None, 0, None) == 6


def test_decode_validation(lib):
    f = lib.sparse_attn_decode
    F = ctypes.c_float(0.1)
    args = [A, 1, A, A, 1, None, None, 2, 4096, 64, 128, 2048, A, A, 1, A, A, 1, 576, 576, 128,
            512, 64, F, A, None, None]
    assert f(*args, None, 0, None) == 6
    need = lib.sparse_attn_workspace_bytes(2, 2, 1, 4096, 2048, 128, 512)
    assert need >= 2 * 4096 * 4
    assert f(*args, A, need - 256, None) == 6


def test_decode_workspace_holds_scores_lists_and_partials(lib):
    # decode, B=32, L=32768, k=2048, H=128: the fp32 score rows (4 bytes per
    # position), the score kernel's candidate lists ((key, position) pairs, up
    # to every position: 8 bytes), and the MLA's KV-split partials (4 splits x
    # 128 heads x (512 + 2) floats per query)
    B, L, k, H = 32, 32768, 2048, 128
    need = lib.sparse_attn_workspace_bytes(2, B, 1, L, k, H, 512)
    assert need >= B * L * (4 + 8) + B * H * 4 * 514 * 4


def test_block_validation(lib):
    f = lib.sparse_attn_block_decode
    F = ctypes.c_float(0.1)
    # d outside the compiled set
    assert f(A, A, A, A, 1, 4096, 8, 2, 64, 64, 16, 64, 512, F, 0, A, None, A, 1 << 20, None) == 5
    # group size 3 is not compiled
    assert f(A, A, A, A, 1, 4096, 6, 2, 128, 64, 16, 64, 512, F, 0, A, None, A, 1 << 20, None) == 5
    # shared_choice is a flag
    assert f(A, A, A, A, 1, 4096, 8, 2, 128, 64, 16, 64, 512, F, 2, A, None, A, 1 << 20, None) == 2
    # workspace too small: the block scores [B, Hq, L / blk]
    need = lib.sparse_attn_workspace_bytes(3, 1, 8, 4096, 16, 2, 128)
    assert need >= 8 * 16 * 4
    assert f(A, A, A, A, 1, 4096, 8, 2, 128, 64, 16, 64, 512, F, 0, A, None, A, 16, None) == 6
    pool = lib.sparse_attn_block_pool
    assert pool(A, 1, 4096, 2, 128, 48, A, None) == 5  # block size not compiled
    assert pool(None, 1, 4096, 2, 128, 64, A, None) == 1
    assert pool(A, 1, 4096, 2, 128, 64, None, None) == 1
    # no complete block (L < blk): krep may be NULL, and nothing is enqueued
    assert pool(A, 1, 40, 2, 128, 64, None, None) == 0
    # the decode still needs krep when blocks exist
    assert f(A, A, A, None, 1, 4096, 8, 2, 128, 64, 16, 64, 512, F, 0, A, None, A, 1 << 20,
             None) == 1


def test_prefill_select_validation(lib):
    f = lib.sparse_attn_prefill_select
    # fp32 queries run only on the vector score path: not fused
    assert f(A, 0, A, A, 1, None, A, None, 1, 16, 4096, 64, 128, 64, A, None, None) == 5
    # the row must fit on chip
    assert f(A, 1, A, A, 1, None, A, None, 1, 16, 40000, 64, 128, 64, A, None, None) == 5
    assert "L <= 32768" in _err(lib)
    assert f(A, 1, A, A, 1, None, A, None, 1, 16, 4096, 64, 128, 0, A, None, None) == 2
    assert f(A, 1, A, A, 1, None, A, None, 1, 16, 4096, 64, 128, 64, None, None, None) == 1
    assert f(A, 1, A, A, 1, None, A, None, 1, 16, 4096, 64, 128, 64, A, M, None) == 4


def test_prefill_validation(lib):
    f = lib.sparse_attn_prefill
    F = ctypes.c_float(0.1)
    idx_args = [A, 1, A, A, 1, None, A, None, 1, 1024, 4096, 64, 128, 2048]
    mla_args = [A, A, A, A, 576, 576, 128, 512, 64, F]
    need = lib.sparse_attn_workspace_bytes(5, 1, 1024, 4096, 2048, 128, 512)
    assert need >= 1024 * 2048 * 4
    # unknown mode
    assert f(*idx_args, *mla_args, 3, A, None, None, A, need, None) == 2
    # no workspace, short workspace
    assert f(*idx_args, *mla_args, 0, A, None, None, None, 0, None) == 6
    assert f(*idx_args, *mla_args, 1, A, None, None, A, need - 256, None) == 6
    # the dense mode needs no indexer inputs, but still the bf16 attention shapes
    bad_h = [A, A, A, A, 576, 576, 100, 512, 64, F]
    assert f(None, 1, None, None, 1, None, A, None, 1, 1024, 4096, 0, 0, 2048, *bad_h, 1, A, None,
             None, A, need, None) == 5
    # the sparse mode needs them
    assert f(None, 1, None, None, 1, None, A, None, 1, 1024, 4096, 0, 0, 2048, *mla_args, 0, A,
             None, None, A, need, None) == 1
