"""GPU parity of the block-sparse GQA decode against the oracle.

The oracle pools the block keys itself (in double) and chooses its own blocks
from its own scores; nothing the GPU produced enters that choice. The GPU's
pooled keys (bf16: the fp32 mean rounded to nearest even) are checked against
the oracle's mean to within half a bf16 unit. Block choice is a ranking decided
in floating point, so the two chosen sets must have equal sizes and may differ
only by blocks whose oracle score is within the bound on the GPU's score error
of the oracle's nsel-th score: 1e-3 relative, plus twice the largest error the
rounded pooled keys allow, 2^-8 sum_d |q_d| |krep_d| per block. The attention
output of EVERY head is then compared (max-abs 2e-3, bf16 inputs) with the
oracle's attention evaluated on the blocks the GPU chose (the oracle's
given-blocks mode), which is only passed in after that choice has passed the
rule above. With a shared choice the scores are the KV group's sums, and every head
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


def _pooled_close(g_krep, okr):
    """The GPU's bf16 pooled keys against the oracle's mean: round to nearest
    even moves a value by at most 2^-8 of itself (8 significant bits)."""
    gkr = g_krep.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gkr - okr) <= 2.0 ** -8 * np.abs(okr) + 1e-6), "pooled keys differ"


def _score_slack(q, okr, Hkv, shared=False):
    """Per (b, h): twice the largest score error that the bf16 rounding of the
    pooled keys allows over the blocks, 2 * 2^-8 * max_n sum_d |q_d| |krep_d|
    (with a shared choice, summed over the group's heads)."""
    qa = np.abs(oracle.decode(q))
    ka = np.abs(okr)
    B, Hq, d = qa.shape
    G = Hq // Hkv
    kag = np.repeat(ka, G, axis=2)  # [B, nblk, Hq, d]
    e = np.einsum("bhd,bnhd->bhn", qa, kag)
    if shared:
        e = np.repeat(e.reshape(B, Hkv, G, -1).sum(axis=2), G, axis=1)
    return 2.0 * 2.0 ** -8 * (e.max(axis=2) if e.shape[2] else np.zeros((B, Hq)))


def _check_choice(g_blocks, o_blocks, scores, nsel, slack):
    """Equal sizes; ascending, -1 padded; differences only between blocks
    that are near-tied on the oracle's scores (within slack[b, h] plus 1e-3
    relative)."""
    gb = g_blocks.cpu().numpy().astype(np.int64)
    ob = np.asarray(o_blocks, np.int64)
    B, Hq, _ = gb.shape
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
                    assert abs(sc[x] - tau) <= 1e-3 * abs(tau) + slack[b, h], \
                        f"block {x} differs but is not a near tie (b={b}, h={h})"


def _check_attention(wl, out, blocks, shared, b0=0, b1=None):
    """Every head of sequences b0..b1-1 against the oracle's attention over
    the GPU's chosen blocks."""
    b1 = wl.B if b1 is None else b1
    sl = slice(b0, b1)
    ro, _ = oracle.block_sparse_decode(wl.q[sl], wl.k[sl], wl.v[sl], wl.blk, wl.nsel,
                                       wl.n_sink, wl.n_win, wl.sm_scale, shared=shared,
                                       given_blocks=blocks[sl].cpu(), allow_empty=True)
    err = np.abs(out[sl].cpu().numpy().astype(np.float64) - ro)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= ATTN_ATOL_BF16, f"attention max-abs {worst:.3g}"


def _same_within_groups(blocks, Hkv):
    b = blocks.cpu().numpy()
    B, Hq, nsel = b.shape
    g = b.reshape(B, Hkv, Hq // Hkv, nsel)
    assert (g == g[:, :, :1]).all(), "heads of a KV group chose different blocks"


def _run_case(wl, shared=False, ws=None):
    t = wl.to(DEV)
    krep = api.sparse_attn_block_pool(t.k, wl.blk)
    out, blocks = api.sparse_attn_block_decode(t.q, t.k, t.v, krep, wl.blk, wl.nsel, wl.n_sink,
                                               wl.n_win, wl.sm_scale, shared_choice=shared,
                                               ws=ws)
    torch.cuda.synchronize()
    if shared:
        _same_within_groups(blocks, wl.Hkv)
    # pooled keys against the oracle's mean in double
    okr = oracle.block_pool(wl.k, wl.blk)
    _pooled_close(krep, okr)
    # the oracle's own choice, on its own pooled keys
    _, rb = oracle.block_sparse_decode(wl.q, wl.k, wl.v, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                       wl.sm_scale, shared=shared, allow_empty=True)
    sc = _block_scores(wl.q, okr, wl.Hkv, shared)
    _check_choice(blocks, rb, sc, wl.nsel, _score_slack(wl.q, okr, wl.Hkv, shared))
    _check_attention(wl, out, blocks, shared)
    return out, blocks


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
        okr = oracle.block_pool(k, wl.blk)
        _pooled_close(krep[b:b + 1], okr)
        _, rb = oracle.block_sparse_decode(q, k, v, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                           wl.sm_scale)
        _check_choice(blocks[b:b + 1], rb, _block_scores(q, okr, wl.Hkv), wl.nsel,
                      _score_slack(q, okr, wl.Hkv))
        _check_attention(wl, out, blocks, False, b, b + 1)


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
    okr = oracle.block_pool(k, wl.blk)
    _, rb = oracle.block_sparse_decode(q, k, v, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                       wl.sm_scale, shared=True)
    _check_choice(blocks[b:b + 1], rb, _block_scores(q, okr, wl.Hkv, shared=True), wl.nsel,
                  _score_slack(q, okr, wl.Hkv, shared=True))
    _check_attention(wl, out, blocks, True, b, b + 1)


@pytest.mark.parametrize("n_sink,n_win", [(16, 20), (0, 0)])
def test_block_sparse_no_complete_block(n_sink, n_win):
    # L < blk: no block exists, so krep is empty and the decode needs no
    # workspace; both go in as NULL, straight through the C ABI.  With sinks
    # and a window the output attends to those tokens only; with neither,
    # nothing is visible: out = 0 and every chosen-block slot is -1.
    import ctypes
    _announce(f"block sparse L=40 < blk=64, sinks {n_sink}, window {n_win}")
    wl = workloads.block_sparse_64k(B=2, L=40, Hq=8, Hkv=2, blk=64, nsel=4, n_sink=n_sink,
                                    n_win=n_win)
    t = wl.to(DEV)
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=DEV)
    blocks = torch.full((wl.B, wl.Hq, wl.nsel), 7, dtype=torch.int32, device=DEV)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = api.load()
    assert lib.sparse_attn_block_pool(p(t.k), wl.B, wl.L, wl.Hkv, wl.d, wl.blk, None,
                                      stream) == 0
    st = lib.sparse_attn_block_decode(p(t.q), p(t.k), p(t.v), None, wl.B, wl.L, wl.Hq, wl.Hkv,
                                      wl.d, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                      ctypes.c_float(wl.sm_scale), 0, p(out), p(blocks), None,
                                      ctypes.c_size_t(0), stream)
    assert st == 0, lib.sparse_attn_last_error()
    torch.cuda.synchronize()
    assert (blocks.cpu() == -1).all()
    if n_sink == 0 and n_win == 0:
        assert (out.cpu() == 0).all()
    _check_attention(wl, out, blocks, False)
