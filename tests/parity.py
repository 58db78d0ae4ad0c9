"""Comparison rules between the GPU path and the oracle.

Index scores: |g - o| <= 1e-3 |o| + 1e-5 * sum_h |w_h| |q_h| |k_s|  (the second
term is the scale of fp32 rounding in the dot products; it only matters for
scores near zero, where cancellation makes a relative bound meaningless).
Non-candidates must be -inf on both sides, exactly.

Index sets: bit-exact where the scores are exact (small-integer workload).
Elsewhere equal sizes, and every position in the symmetric difference has an
oracle score within 1e-3 |tau| of tau, the oracle's k-th score: the two sides
may only disagree about near-ties at the boundary.

Attention: max-abs error given identical index sets (2e-3 for bf16 inputs).
"""
import numpy as np
import torch

SCORE_RTOL = 1e-3
SCORE_FLOOR = 1e-5
SET_RTOL = 1e-3
ATTN_ATOL_BF16 = 2e-3
ATTN_ATOL_FP8 = 5e-2


def to_np(t):
    return t.detach().float().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def score_floor(q_idx, w, k_deq):
    """1e-5 * sum_h |w_h| ||q_h|| ||k_s||  -> [B,T,L]."""
    import oracle
    q = oracle.decode(q_idx)
    wd = oracle.decode(w)
    a = (np.abs(wd) * np.linalg.norm(q, axis=-1)).sum(-1)  # [B,T]
    kn = np.linalg.norm(k_deq, axis=-1)                     # [B,L]
    return SCORE_FLOOR * a[:, :, None] * kn[:, None, :]


def assert_scores_close(gpu, ref, floor, rtol=SCORE_RTOL):
    g = to_np(gpu).astype(np.float64)
    assert g.shape == ref.shape
    ninf_r = np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), ninf_r), "candidate masks differ"
    ok = ~ninf_r
    err = np.abs(g[ok] - ref[ok])
    bound = rtol * np.abs(ref[ok]) + floor[ok]
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} scores out of tolerance; worst err/bound "
                           f"{(err / bound).max():.3g}")
    return float((err / np.maximum(np.abs(ref[ok]), 1e-30)).max()) if err.size else 0.0


def assert_index_sets(g_idx, g_cnt, o_idx, o_cnt, o_scores, rtol=SET_RTOL, exact=False):
    gi, gc = to_np(g_idx).astype(np.int64), to_np(g_cnt).astype(np.int64)
    oi, oc = np.asarray(o_idx, np.int64), np.asarray(o_cnt, np.int64)
    assert np.array_equal(gc, oc), "selected counts differ"
    rows = gi.reshape(-1, gi.shape[-1])
    orows = oi.reshape(-1, oi.shape[-1])
    sc = o_scores.reshape(-1, o_scores.shape[-1])
    cnt = oc.reshape(-1)
    n_diff = 0
    for r in range(rows.shape[0]):
        c = cnt[r]
        g = rows[r]
        # the GPU writes its positions ascending and pads with -1
        assert np.all(g[c:] == -1), f"row {r}: padding"
        assert np.all(np.diff(g[:c]) > 0), f"row {r}: not strictly ascending"
        if exact:
            assert np.array_equal(g, orows[r]), f"row {r}: index sets differ"
            continue
        gs, os_ = set(g[:c].tolist()), set(orows[r, :c].tolist())
        diff = gs ^ os_
        if not diff:
            continue
        tau = np.sort(sc[r, orows[r, :c]])[0]  # the oracle's k-th (smallest kept) score
        for p in diff:
            assert abs(sc[r, p] - tau) <= rtol * abs(tau) + 1e-12, (
                f"row {r}: position {p} (oracle score {sc[r, p]}) is not a near-tie of "
                f"tau = {tau}")
        n_diff += len(diff)
    return n_diff


def assert_attention_close(g_out, o_out, atol, g_lse=None, o_lse=None, lse_atol=1e-3):
    g = to_np(g_out).astype(np.float64)
    err = np.abs(g - o_out)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, f"max-abs attention error {worst:.3g} > {atol}"
    if g_lse is not None:
        gl = to_np(g_lse).astype(np.float64)
        both_inf = np.isneginf(gl) & np.isneginf(o_lse)
        assert np.array_equal(np.isneginf(gl), np.isneginf(o_lse))
        e2 = np.abs(np.where(both_inf, 0.0, gl - np.where(both_inf, 0.0, o_lse)))
        assert float(e2.max()) <= lse_atol, f"lse error {float(e2.max()):.3g}"
    return worst
