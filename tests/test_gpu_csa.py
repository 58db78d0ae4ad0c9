"""GPU parity of the selection over compressed entries (CSA-style decode):
the indexer and top-k over the entries' index keys (set rule of the other
parity tests), then the core attention (keys = values = entries, the selected
entries plus the window, one softmax) against the oracle's attention on the
GPU's own selection (max-abs 2e-3, bf16 inputs)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from top_indexer_sparse_amd import api, workloads

from parity import ATTN_ATOL_BF16, assert_attention_close, assert_index_sets

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _announce(msg):
    print(f"\n[csa] {msg}", file=sys.stderr, flush=True)


def _check(wl, seqs=None):
    t = wl.to(DEV)
    out, lse, idx = api.sparse_attn_csa_decode(t.q_idx, t.w, t.k_idx, None, t.n_comp, wl.topk, t.q,
                                               t.comp, t.win, wl.sm_scale)
    torch.cuda.synchronize()
    seqs = range(wl.B) if seqs is None else seqs
    for b in seqs:
        sl = slice(b, b + 1)
        nc = None if wl.n_comp is None else wl.n_comp[sl]
        rs = oracle.indexer(wl.q_idx[sl, None], wl.w[sl, None], wl.k_idx[sl], kv_len=nc)
        oi, oc = oracle.topk(rs, wl.topk, kv_len=nc)
        gi = idx[sl].cpu().numpy()
        gc = (gi >= 0).sum(-1)
        assert_index_sets(gi[:, None], gc[:, None], oi, oc, rs)
        win = None if wl.win is None else wl.win[sl]
        ro, rl = oracle.csa_attention(wl.q[sl], wl.comp[sl], win, gi, wl.sm_scale)
        assert_attention_close(out[sl], ro, ATTN_ATOL_BF16, lse[sl], rl)


def test_csa_small_ragged():
    # three sequences: all entries, part of them, fewer than k (every entry taken)
    _announce("csa B=3 Lc=5000 k=256 H=64 n_win=48")
    wl = workloads.csa_decode(B=3, Lc=5000, topk=256, H=64, n_win=48, n_comp=[5000, 3001, 100])
    _check(wl)


def test_csa_no_window():
    _announce("csa B=2 Lc=9000 k=512 H=128 no window")
    wl = workloads.csa_decode(B=2, Lc=9000, topk=512, H=128, n_win=0)
    _check(wl)


def test_csa_window_only():
    # no entry present: the window alone is attended
    _announce("csa B=2 Lc=600 n_comp=0 n_win=40")
    wl = workloads.csa_decode(B=2, Lc=600, topk=64, H=64, n_win=40, n_comp=[0, 600])
    _check(wl)


def test_csa_fullsize_sampled():
    """B=32, Lc=32768 entries (a 131072-token context at m = 4), k=2048, H=128,
    128 window entries; two sequences go to the oracle."""
    _announce("csa full size B=32 Lc=32768")
    wl = workloads.csa_decode()
    _check(wl, seqs=[0, wl.B - 1])
