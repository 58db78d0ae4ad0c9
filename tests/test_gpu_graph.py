"""HIP graph capture of the fused entry points.

A serving loop captures a decode step once and replays it.  The library's
launches take only the caller's stream, allocate nothing and record no
memory sets, so a captured step must replay to the eager result: each test
captures a call, replays it several times with eager work and
synchronisations in between, and checks every replay bit for bit against
the eager call.
"""
import pytest
import torch

from top_indexer_sparse_amd import api, workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _replays_match(fn, outs, n=4):
    # eager reference
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        for o in outs:
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {i} differs from the eager call"
        # eager work of the program between replays
        fn()
        torch.cuda.synchronize()


def test_graph_replay_decode():
    _announce("graph capture: sparse_attn_decode B=4 L=8192")
    wl = workloads.decode_32k(B=4, L=8192)
    t = wl.to(DEV)
    B, L, k = wl.B, wl.L, wl.topk
    out = torch.empty((B, 1, wl.H, wl.dc), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, wl.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    ws = torch.empty(api.sparse_attn_workspace_bytes(api.SA_OP_DECODE, B, 1, L, k, wl.H, wl.dc),
                     dtype=torch.uint8, device=DEV)
    c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]

    def fn():
        api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, None, None, k, t.q_lat, t.q_rope, c_kv,
                               k_rope, wl.sm_scale, out=out, lse=lse, idx_out=idx, ws=ws)

    _replays_match(fn, [out, lse, idx])


def test_graph_replay_prefill_sparse():
    _announce("graph capture: sparse_attn_prefill (fused select) B=1 T=L=2048")
    wl = workloads.prefill_batch(B=1, T=2048, L=2048, HI=64, dI=128, topk=256, H=64)
    t = wl.to(DEV)
    B, T, L, k = wl.B, wl.T, wl.L, wl.topk
    out = torch.empty((B, T, wl.H, wl.dc), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, T, wl.H), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    ws = torch.empty(api.sparse_attn_workspace_bytes(api.SA_OP_PREFILL, B, T, L, k, wl.H, wl.dc),
                     dtype=torch.uint8, device=DEV)
    c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]

    def fn():
        api.sparse_attn_prefill(t.q_idx, t.w, t.k_idx, k, t.q_lat, t.q_rope, c_kv, k_rope,
                                wl.sm_scale, q_pos=t.q_pos, mode=api.SA_PREFILL_SPARSE, out=out,
                                lse=lse, idx_out=idx, ws=ws)

    _replays_match(fn, [out, lse, idx])
