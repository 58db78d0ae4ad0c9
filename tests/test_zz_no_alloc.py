"""The decode entry point without a workspace argument (sparse_attn_decode_noalloc):
its scratch is the library's fixed per-GPU array.  Two calls in a row, the
second with smaller sizes, each equal bit for bit to sparse_attn_decode with a
workspace on the same inputs; sizes beyond the scratch are refused on the host."""
import ctypes

import pytest
import torch

from top_indexer_sparse_amd import api, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _both(wl):
    t = wl.to(DEV)
    c, r = t.kv[..., :wl.dc], t.kv[..., wl.dc:]
    o1, l1, i1 = api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, t.k_scale, t.kv_len, wl.topk, t.q_lat,
                                        t.q_rope, c, r, wl.sm_scale)
    o2, l2, i2 = api.sparse_attn_decode_noalloc(t.q_idx, t.w, t.k_idx, t.k_scale, t.kv_len, wl.topk,
                                                t.q_lat, t.q_rope, c, r, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2), "index sets differ from sparse_attn_decode"
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "outputs differ from sparse_attn_decode"
    return i2


def test_noalloc_decode_equals_workspace_decode_twice():
    # first call: 5 sequences of 5000 positions (ragged); second: 2 of 2600
    _announce("decode_noalloc B=5 L=5000 then B=2 L=2600")
    wl1 = workloads.decode_32k(B=5, L=5000, kv_len=[5000, 4000, 2100, 1500, 3333])
    i1 = _both(wl1)
    assert (i1 >= 0).sum().item() == sum(min(2048, n) for n in (5000, 4000, 2100, 1500, 3333))
    wl2 = workloads.decode_32k(B=2, L=2600, kv_len=[2600, 1999])
    _both(wl2)


def test_noalloc_decode_fp8_keys():
    _announce("decode_noalloc fp8 keys B=2 L=9000")
    wl = workloads.decode_128k_fp8(B=2, L=9000, H=128, boost_frac=0.02)
    _both(wl)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    # 64 sequences of 131072 positions need more than the fixed scratch:
    # refused on the host (nothing enqueued, no pointer dereferenced)
    lib = api.load()
    A = ctypes.c_void_p(16)
    need = lib.sparse_attn_workspace_bytes(api.SA_OP_DECODE, 64, 1, 131072, 2048, 128, 512)
    assert need > 64 << 20
    st = lib.sparse_attn_decode_noalloc(A, 1, A, A, 1, None, None, 64, 131072, 64, 128, 2048, A, A,
                                        1, A, A, 1, 576, 576, 128, 512, 64, ctypes.c_float(0.04),
                                        A, None, None, None)
    assert st == 6  # SA_ERR_WORKSPACE
    assert b"scratch" in lib.sparse_attn_last_error()
