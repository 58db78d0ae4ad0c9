"""GPU parity of the block-sparse GQA decode against the oracle.

Block choice is an argmax decided in floating point, so both sides decide it
on the same pooled keys: the oracle receives the GPU's fp32 pooled keys (and
scores them in double).  Chosen sets must have equal sizes and may differ only
by blocks whose oracle score is within 1e-3 of the nsel-th score (relative);
the attention output is compared (max-abs 2e-3, bf16 inputs) for every head
whose chosen set equals the oracle's, which on continuous random data is every
head.  With a shared choice the scores are the KV group's sums, and every head
of a group must carry the same set.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_indexer_sparse_amd import api, workloads

from parity import ATTN_ATOL_BF16

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _announce(msg):
    print(f"\n[block] {msg}", file=sys.stderr, flush=True)


def _block_scores(q, krep, Hkv, shared=False):
    """Oracle-precision block scores q_h . krep[b, n, g(h)] -> [B, Hq, nblk];
    with shared=True each head gets its KV group's sum."""
    qd = oracle.decode(q)
    kr = oracle.decode(krep)
    B, Hq, d = qd.shape
    G = Hq // Hkv
    krg = np.repeat(kr, G, axis=2)  # [B, nblk, Hq, d]
    sc = np.einsum("bhd,bnhd->bhn", qd, krg)
    if shared:
        sc = np.repeat(sc.reshape(B, Hkv, G, -1).sum(axis=2), G, axis=1)
    return sc


def _check_choice(g_blocks, o_blocks, scores, nsel):
    """Equal sizes; differences only between near-tied blocks.  Returns the
    mask of (b, h) whose chosen sets are identical."""
    gb = g_blocks.cpu().numpy().astype(np.int64)
    ob = np.asarray(o_blocks, np.int64)
    B, Hq, _ = gb.shape
    same = np.zeros((B, Hq), bool)
    for b in range(B):
        for h in range(Hq):
            gs = [x for x in gb[b, h] if x >= 0]
            os_ = [x for x in ob[b, h] if x >= 0]
            assert gs == sorted(gs), "chosen blocks not ascending"
            assert len(gs) == len(os_), "chosen set sizes differ"
            assert all(x == -1 for x in gb[b, h, len(gs):]), "padding is not -1"
            diff = set(gs) ^ set(os_)
            if diff:
                sc = scores[b, h]
                tau = np.sort(sc)[::-1][min(nsel, sc.size) - 1]
                for x in diff:
                    assert abs(sc[x] - tau) <= 1e-3 * max(abs(tau), 1e-30), \
                        f"block {x} differs but is not a near tie (b={b}, h={h})"
            same[b, h] = not diff
    return same


def _same_within_groups(blocks, Hkv):
    b = blocks.cpu().numpy()
    B, Hq, nsel = b.shape
    g = b.reshape(B, Hkv, Hq // Hkv, nsel)
    assert (g == g[:, :, :1]).all(), "heads of a KV group chose different blocks"


def _run_case(wl, shared=False):
    t = wl.to(DEV)
    krep = api.sparse_attn_block_pool(t.k, wl.blk)
    out, blocks = api.sparse_attn_block_decode(t.q, t.k, t.v, krep, wl.blk, wl.nsel, wl.n_sink,
                                               wl.n_win, wl.sm_scale, shared_choice=shared)
    torch.cuda.synchronize()
    if shared:
        _same_within_groups(blocks, wl.Hkv)
    # pooled keys against the oracle's mean in double
    okr = oracle.block_pool(wl.k, wl.blk)
    gkr = krep.cpu().numpy().astype(np.float64)
    assert np.allclose(gkr, okr, rtol=1e-5, atol=1e-6), "pooled keys differ"
    ro, rb = oracle.block_sparse_decode(wl.q, wl.k, wl.v, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                        wl.sm_scale, krep=krep.cpu(), shared=shared)
    sc = _block_scores(wl.q, krep.cpu(), wl.Hkv, shared)
    same = _check_choice(blocks, rb, sc, wl.nsel)
    assert same.mean() > 0.9, "too many heads with near-tie choices"
    err = np.abs(out.cpu().numpy().astype(np.float64) - ro)
    worst = err.max(axis=-1)[same].max()
    assert worst <= ATTN_ATOL_BF16, f"attention max-abs {worst:.3g}"


def test_block_sparse_small_ragged():
    # L not a multiple of the block: the last partial block is never chosen,
    # the window reaches into it; sinks and window overlap chosen blocks
    _announce("block sparse B=2 L=2085 Hq=8 Hkv=2 blk=64 nsel=8")
    wl = workloads.block_sparse_64k(B=2, L=2085, Hq=8, Hkv=2, blk=64, nsel=8, n_sink=64,
                                    n_win=200)
    _run_case(wl)


@pytest.mark.parametrize("blk,G", [(32, 1), (128, 8)])
def test_block_sparse_block_sizes_and_groups(blk, G):
    _announce(f"block sparse blk={blk} G={G}")
    Hkv = 2
    wl = workloads.block_sparse_64k(B=2, L=4096, Hq=G * Hkv, Hkv=Hkv, blk=blk, nsel=12,
                                    n_sink=16, n_win=100)
    _run_case(wl)


def test_block_sparse_fewer_blocks_than_nsel():
    # 3 complete blocks, nsel 16: every block chosen, -1 padding after them
    _announce("block sparse L=200 blk=64 nsel=16")
    wl = workloads.block_sparse_64k(B=1, L=200, Hq=4, Hkv=1, blk=64, nsel=16, n_sink=0,
                                    n_win=0)
    _run_case(wl)


@pytest.mark.parametrize("L,blk,nsel", [(131109, 64, 64), (262144, 32, 40)])
def test_block_sparse_long_rows_and_max_nsel(L, blk, nsel):
    # 2048 and 8192 blocks per row (the selection's 8- and 32-keys-per-thread
    # variants), the largest nsel, a ragged tail; one KV group, B * Hq = 4
    # attention work-groups (fewer than the XCDs: no XCD layout)
    _announce(f"block sparse L={L} blk={blk} nsel={nsel}")
    wl = workloads.block_sparse_64k(B=1, L=L, Hq=4, Hkv=1, blk=blk, nsel=nsel, n_sink=32,
                                    n_win=300)
    _run_case(wl)


def test_block_sparse_fullsize_sampled():
    """The block-sparse workload at full size (B=16, L=65536, 32/8 heads,
    block 64, top 16 + 64 sinks + 512 window); two sequences go to the oracle."""
    _announce("block sparse full size B=16 L=65536")
    wl = workloads.block_sparse_64k()
    t = wl.to(DEV)
    krep = api.sparse_attn_block_pool(t.k, wl.blk)
    out, blocks = api.sparse_attn_block_decode(t.q, t.k, t.v, krep, wl.blk, wl.nsel, wl.n_sink,
                                               wl.n_win, wl.sm_scale)
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        _announce(f"oracle on sequence {b}")
        q, k, v = wl.q[b:b + 1], wl.k[b:b + 1], wl.v[b:b + 1]
        kr = krep[b:b + 1].cpu()
        okr = oracle.block_pool(k, wl.blk)
        assert np.allclose(kr.numpy().astype(np.float64), okr, rtol=1e-5, atol=1e-6)
        ro, rb = oracle.block_sparse_decode(q, k, v, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                            wl.sm_scale, krep=kr)
        sc = _block_scores(q, kr, wl.Hkv)
        same = _check_choice(blocks[b:b + 1], rb, sc, wl.nsel)
        err = np.abs(out[b:b + 1].cpu().numpy().astype(np.float64) - ro)
        assert err.max(axis=-1)[same].max() <= ATTN_ATOL_BF16


@pytest.mark.parametrize("blk,G", [(64, 4), (32, 8), (128, 2)])
def test_block_sparse_shared_choice(blk, G):
    _announce(f"block sparse, group-shared choice, blk={blk} G={G}")
    Hkv = 2
    wl = workloads.block_sparse_64k(B=2, L=4133, Hq=G * Hkv, Hkv=Hkv, blk=blk, nsel=10,
                                    n_sink=16, n_win=150)
    _run_case(wl, shared=True)


def test_block_sparse_shared_choice_fullsize_sampled():
    """The block-sparse workload at full size with the group-shared choice;
    one sequence goes to the oracle."""
    _announce("block sparse full size, group-shared choice")
    wl = workloads.block_sparse_64k()
    t = wl.to(DEV)
    krep = api.sparse_attn_block_pool(t.k, wl.blk)
    out, blocks = api.sparse_attn_block_decode(t.q, t.k, t.v, krep, wl.blk, wl.nsel, wl.n_sink,
                                               wl.n_win, wl.sm_scale, shared_choice=True)
    torch.cuda.synchronize()
    _same_within_groups(blocks, wl.Hkv)
    b = wl.B // 2
    _announce(f"oracle on sequence {b}")
    q, k, v = wl.q[b:b + 1], wl.k[b:b + 1], wl.v[b:b + 1]
    kr = krep[b:b + 1].cpu()
    ro, rb = oracle.block_sparse_decode(q, k, v, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                        wl.sm_scale, krep=kr, shared=True)
    sc = _block_scores(q, kr, wl.Hkv, shared=True)
    same = _check_choice(blocks[b:b + 1], rb, sc, wl.nsel)
    err = np.abs(out[b:b + 1].cpu().numpy().astype(np.float64) - ro)
    assert err.max(axis=-1)[same].max() <= ATTN_ATOL_BF16
