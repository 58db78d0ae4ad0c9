"""GPU parity of the decode Top-K that reads the score kernel's per-work-group
candidate lists (sparse_attn_decode and sparse_attn_csa_decode with the MFMA
indexer).

Whichever way the select goes -- from the lists; from the lists with the
deficient lists' keys read back from the score row (a work-group held more
of the row's top k than its floor kept); from the score row alone (more kept
keys than fit on chip, fewer kept keys than k, fewer candidates than k with
keys dropped) -- the selected set must equal, bit for bit, the oracle's top-k
of the same scores: those of sparse_attn_indexer_scores, which runs the same
contraction (its scores are parity-checked against the oracle's indexer in
test_gpu_parity.py and test_gpu_fullsize.py).  `select_path` restates the
lists' geometry and floors on the CPU so each case can assert which way it
goes.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from top_indexer_sparse_amd import api, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
H, DC, DR = 64, 512, 64


def _announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


def _index_inputs(kind, B, L, seed, HI=64, dI=128):
    """(q_idx [B,1,HI,dI] bf16, w [B,1,HI] f32, k_idx [B,L,dI] bf16) on the CPU."""
    g = torch.Generator().manual_seed(seed)
    if kind == "ties":
        # integers in {-1, 0, 1} and weights in {0, 1}: integer scores, exact
        # in fp32, with many ties at the k-th score
        HI, dI = 16, 64
        q = torch.randint(-1, 2, (B, 1, HI, dI), generator=g).to(torch.bfloat16)
        w = torch.randint(0, 2, (B, 1, HI), generator=g).float()
        k = torch.randint(-1, 2, (B, L, dI), generator=g).to(torch.bfloat16)
        return q, w, k
    q = torch.randn(B, 1, HI, dI, generator=g).to(torch.bfloat16)
    w = torch.rand(B, 1, HI, generator=g)
    k = torch.randn(B, L, dI, generator=g).to(torch.bfloat16)
    if kind == "clustered":
        # 64-position runs every 8192 positions scaled by 8 (scores scale with
        # the key, ReLU being positively homogeneous): every score work-group
        # takes its positions in 64-position runs, so these all land in one
        # work-group per row, which then holds far more of the top k than its
        # share
        pos = torch.arange(L)
        k[:, (pos % 8192) < 64] *= 8
    elif kind == "phase":
        # the same 64-position phase of every 1024 positions scaled by 4: one
        # list per row holds most of the top k, so it is read back
        pos = torch.arange(L)
        k[:, (pos % 1024) < 64] *= 4
    elif kind == "halfphase":
        # half the phases scaled by 16: the keys above the read-back bound
        # outgrow the select's LDS, so the row is read directly
        pos = torch.arange(L)
        k[:, (pos % 1024) < 512] *= 16
    elif kind == "allequal":
        k[:] = k[:, :1]  # one key row everywhere: every score ties
    return q, w, k


def _keys(f):
    """Order-preserving uint32 keys of fp32 scores; 0 (no candidate) for NaN
    and -inf, one key for +0 and -0."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.int64)
    u = np.where(u == 0x80000000, 0, u)
    key = np.where(u & 0x80000000, (~u) & 0xffffffff, u | 0x80000000)
    return np.where(np.isnan(f) | (u == 0xff800000), 0, key)


def _rank_floor(keys, lo, r):
    """Floor of the bin (of a 2048-bin histogram fitted to [lo, max]) that
    holds the r-th largest of `keys` (all >= lo)."""
    span = int(keys.max()) - lo
    sh = max(0, span.bit_length() - 11)
    hist = np.bincount((keys - lo) >> sh, minlength=2048)
    above = np.cumsum(hist[::-1])
    return lo + ((2047 - int(np.argmax(above >= r))) << sh)


def select_path(srow, lim, k, rows, L):
    """Which way the decode select takes one row: 'all' (at most k
    candidates), 'lists', 'reread' (deficient lists read back) or 'row'."""
    s = 1024
    while s > 64 and rows * -(-L // (4 * s)) < 512:
        s //= 2
    nwg = -(-L // (4 * s))
    keys = _keys(srow[:lim])
    lst = (np.arange(lim) // 64) % nwg
    p = np.float32(min(1.0, np.float32(k) / np.float32(max(lim, 1))))
    info, kept = [], []
    for j in range(nwg):
        kj = keys[(lst == j) & (keys != 0)]
        n = len(kj)
        if n == 0:
            info.append((0, 0, None))
            kept.append(kj)
            continue
        mean = np.float32(p * np.float32(n))
        r1 = min(n, int(math.ceil(np.float32(np.float32(mean + np.float32(5) * np.sqrt(
            np.float32(mean * np.float32(1 - p)), dtype=np.float32)) + np.float32(2)))))
        lo = int(kj.min()) if n <= r1 else _rank_floor(kj, int(kj.min()), r1)
        info.append((int((kj >= lo).sum()), n, lo))
        kept.append(kj[kj >= lo])
    K, V = sum(i[0] for i in info), sum(i[1] for i in info)
    if V <= k:
        return "all" if K == V else "row"
    if K < k or K > 12288:
        return "row"
    allk = np.concatenate(kept)
    lomin = min(i[2] for i in info if i[0] > 0)
    lo0 = max([lomin] + [i[2] for i in info if i[0] < i[1]])
    if (allk >= lo0).sum() >= k:
        return "lists"
    t = _rank_floor(allk, lomin, k)
    extra = sum(int(((keys >= t) & (keys < i[2]) & (lst == j)).sum())
                for j, i in enumerate(info) if i[0] < i[1] and i[2] > t)
    return "reread" if K + extra <= 12288 else "row"


def _check_decode(q, w, k, k_scale, kv_len, topk, expect=None):
    B, L = k.shape[0], k.shape[1]
    gm = torch.Generator(device=DEV).manual_seed(11)
    q_lat = torch.randn(B, 1, H, DC, device=DEV, generator=gm).to(torch.bfloat16)
    q_rope = torch.randn(B, 1, H, DR, device=DEV, generator=gm).to(torch.bfloat16)
    kv = torch.randn(B, L, DC + DR, device=DEV, generator=gm).to(torch.bfloat16)
    qd, wd, kd = q.to(DEV), w.to(DEV), k.to(DEV)
    sd = None if k_scale is None else k_scale.to(DEV)
    kl = None if kv_len is None else kv_len.to(DEV)
    out, lse, idx = api.sparse_attn_decode(qd, wd, kd, sd, kl, topk, q_lat, q_rope,
                                           kv[..., :DC], kv[..., DC:], 0.04)
    s = api.sparse_attn_indexer_scores(qd, wd, kd, k_scale=sd, kv_len=kl)
    torch.cuda.synchronize()
    sc = s.cpu()
    oi, oc = oracle.topk(sc.double().numpy(), topk, kv_len=kv_len)
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, oi), \
        f"rows differ: {sorted(set(np.nonzero((gi != oi).any(-1))[0].tolist()))}"
    assert torch.isfinite(out).all().item()
    if expect is not None:  # the case exercises the path it is meant for
        sn = sc.numpy()
        paths = [select_path(sn[b, 0], L if kv_len is None else int(kv_len[b]), topk, B, L)
                 for b in range(B)]
        assert expect in paths, paths


@pytest.mark.parametrize("kind,B,L,topk,kv,path", [
    ("spread", 4, 32768, 2048, None, "lists"),
    ("clustered", 4, 32768, 2048, None, "reread"),
    ("clustered", 32, 32768, 2048, None, "reread"),  # the benchmark's launch geometry
    ("phase", 4, 32768, 2048, None, "reread"),
    ("phase", 32, 32768, 2048, None, "reread"),
    # read back with ragged candidate limits (and rows with at most k candidates)
    ("phase", 6, 32768, 2048, [32768, 20000, 9000, 2048, 1, 0], "reread"),
    # the keys above the read-back bound outgrow LDS: the score row is read
    ("halfphase", 32, 32768, 2048, None, "row"),
    ("ties", 3, 20037, 512, None, "lists"),
    ("allequal", 2, 10000, 300, None, "lists"),
    ("spread", 6, 9000, 2048, [9000, 2047, 2048, 0, 1, 5000], "all"),
    ("spread", 2, 3000, 4096, None, "all"),  # fewer candidates than k
    ("spread", 2, 131072, 2048, [131072, 100000], "lists"),
    # every key equal: each list keeps all of its keys, 40000 in all, more
    # than the select holds on chip, so it reads the score row
    ("allequal", 2, 40000, 2048, None, "row"),
    # one short list per row; rows shorter than k, a single position, k = 64
    ("spread", 5, 777, 64, [777, 500, 64, 63, 1], "lists"),
])
def test_decode_select_equals_oracle_topk_of_the_same_scores(kind, B, L, topk, kv, path):
    _announce(f"decode select {kind} B={B} L={L} k={topk} kv_len={kv}")
    q, w, k = _index_inputs(kind, B, L, seed=B * 1000 + L % 997)
    kv_len = None if kv is None else torch.tensor(kv, dtype=torch.int32)
    _check_decode(q, w, k, None, kv_len, topk, expect=path)


@pytest.mark.parametrize("HI,dI", [(16, 128), (32, 128), (128, 128), (64, 64)])
def test_decode_select_other_indexer_shapes(HI, dI):
    # every compiled score kernel leaves its lists the same way (the 128-head
    # query block runs a four-deep key ring instead of eight)
    _announce(f"decode select H^I={HI} d^I={dI} B=3 L=20000 k=1024")
    q, w, k = _index_inputs("clustered", 3, 20000, seed=HI * 7 + dI, HI=HI, dI=dI)
    kv_len = torch.tensor([20000, 12345, 900], dtype=torch.int32)
    _check_decode(q, w, k, None, kv_len, 1024)


def test_decode_select_fp8_keys_small_query_block():
    _announce("decode select fp8 keys H^I=16 B=2 L=30000 k=2048")
    wl = workloads.decode_128k_fp8(B=2, L=30000, HI=16)
    _check_decode(wl.q_idx, wl.w, wl.k_idx, wl.k_scale, wl.kv_len, wl.topk)


def test_decode_beyond_the_lists_limit_takes_the_split_select():
    # rows longer than 131072 positions: the score kernel leaves no lists and
    # the chunked split select runs over the scores, with the same result rule
    _announce("decode select L=140000 (split path) B=2 k=2048")
    q, w, k = _index_inputs("spread", 2, 140000, seed=140)
    _check_decode(q, w, k, None, torch.tensor([140000, 131100], dtype=torch.int32), 2048)


@pytest.mark.parametrize("nnan,path", [
    (700, "lists"),
    # 85% NaN: the lists keep fewer than k keys in all, so the row is read
    (27853, "row"),
])
def test_decode_select_never_takes_nan_scores(nnan, path):
    # NaN index scores are never selected (documented: the library excludes
    # non-finite index scores).  The ReLU maps a NaN product to 0, so NaN
    # scores come from the fp8 path's per-token scale, which multiplies the
    # finished score.  The oracle refuses non-finite scores, so the fused
    # decode is checked against the staged top-k over the same scores, and
    # against the oracle's top-k over the finite positions.
    _announce(f"decode select with {nnan} NaN scores B=3 L=32768 k=2048")
    k = 2048
    wl = workloads.decode_128k_fp8(B=3, L=32768)
    B, L = wl.B, wl.L
    g = torch.Generator().manual_seed(5)
    nanpos = torch.randperm(L, generator=g)[:nnan]
    scale = wl.k_scale.clone()
    scale[:, nanpos] = float("nan")
    qd, wd, kd, sd = wl.q_idx.to(DEV), wl.w.to(DEV), wl.k_idx.to(DEV), scale.to(DEV)
    gm = torch.Generator(device=DEV).manual_seed(11)
    q_lat = torch.randn(B, 1, H, DC, device=DEV, generator=gm).to(torch.bfloat16)
    q_rope = torch.randn(B, 1, H, DR, device=DEV, generator=gm).to(torch.bfloat16)
    kv = torch.randn(B, L, DC + DR, device=DEV, generator=gm).to(torch.bfloat16)
    _, _, idx = api.sparse_attn_decode(qd, wd, kd, sd, None, k, q_lat, q_rope,
                                       kv[..., :DC], kv[..., DC:], 0.04)
    s = api.sparse_attn_indexer_scores(qd, wd, kd, k_scale=sd)
    si, sc = api.sparse_attn_topk(s, k)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, si.cpu().numpy())
    sn = s.cpu().double().numpy()
    assert np.isnan(sn[:, 0, nanpos.numpy()]).all()  # the case is really exercised
    for b in range(B):
        sel = gi[b, 0][gi[b, 0] >= 0]
        assert np.isfinite(sn[b, 0, sel]).all()
        fin = np.nonzero(np.isfinite(sn[b, 0]))[0]
        assert len(sel) == min(k, len(fin))
        # the oracle on the finite positions only, mapped back to positions
        oi, _ = oracle.topk(sn[b:b + 1, :, fin], k)
        assert np.array_equal(np.sort(fin[oi[0, 0][oi[0, 0] >= 0]]), sel)
    paths = [select_path(s.cpu().numpy()[b, 0], L, k, B, L) for b in range(B)]
    assert path in paths, paths


def test_decode_select_fp8_keys_read_back():
    # fp8 keys whose per-token scale is 4x on one 64-position phase of every
    # 1024: the read-back path reads scaled scores, as the lists hold them
    _announce("decode select fp8 keys, phase pattern through the scales, B=3 L=40000")
    wl = workloads.decode_128k_fp8(B=3, L=40000)
    scale = wl.k_scale.clone()
    pos = torch.arange(wl.L)
    scale[:, (pos % 1024) < 64] *= 4
    _check_decode(wl.q_idx, wl.w, wl.k_idx, scale, wl.kv_len, wl.topk, expect="reread")


def test_decode_select_fp8_keys():
    _announce("decode select fp8 keys B=3 L=40000 k=2048")
    wl = workloads.decode_128k_fp8(B=3, L=40000)
    _check_decode(wl.q_idx, wl.w, wl.k_idx, wl.k_scale, wl.kv_len, wl.topk)


def test_csa_decode_select_equals_oracle_topk():
    _announce("csa decode select B=3 Lc=12000 k=1024")
    B, Lc, k, n_win = 3, 12000, 1024, 128
    q, w, kidx = _index_inputs("clustered", B, Lc, seed=77)
    g = torch.Generator(device=DEV).manual_seed(3)
    qa = torch.randn(B, H, DC, device=DEV, generator=g).to(torch.bfloat16)
    comp = torch.randn(B, Lc, DC, device=DEV, generator=g).to(torch.bfloat16)
    win = torch.randn(B, n_win, DC, device=DEV, generator=g).to(torch.bfloat16)
    n_comp = torch.tensor([Lc, 7000, 1500], dtype=torch.int32)
    qd, wd, kd, nc = q.to(DEV), w.to(DEV), kidx.to(DEV), n_comp.to(DEV)
    out, lse, idx = api.sparse_attn_csa_decode(qd[:, 0].contiguous(), wd[:, 0].contiguous(), kd,
                                               None, nc, k, qa, comp, win, 0.04)
    s = api.sparse_attn_indexer_scores(qd, wd, kd, kv_len=nc)
    torch.cuda.synchronize()
    oi, oc = oracle.topk(s.cpu().double().numpy(), k, kv_len=n_comp)
    assert np.array_equal(idx.cpu().numpy(), oi[:, 0])
