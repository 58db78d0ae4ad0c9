"""Seeded synthetic workloads (the input bytes both the GPU path and the CPU
oracle consume).

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no index score, no selection, no attention).  Everything
is generated on the CPU from torch.Generator seeds, in fp32, then cast once by
torch (round to nearest even) to the storage dtype, so every machine produces
the same bytes.  Seed of tensor `tid` in workload `wid`:
20260900 + 16 * wid + tid.

Workload shapes follow the workloads the source pages describe (DSA top-k
k = 2048 over long contexts, a small-integer exact case, an fp8-key long
context, block-sparse selection with sinks and a window).  No benchmark suite
items are reproduced; "needles" only imitate the structure of a
needle-in-a-haystack probe: a few planted cache rows whose keys align with the
query, so a correct selector must find them.
"""
from dataclasses import dataclass, field
import math
from typing import Optional

import torch

SEED_BASE = 20260900

# workload ids (for seeding)
W_TINY_PREFILL, W_DECODE_32K, W_PREFILL_16K, W_DECODE_128K_FP8, W_BLOCK_64K = 1, 2, 3, 4, 5


def _g(wid: int, tid: int) -> torch.Generator:
    return torch.Generator().manual_seed(SEED_BASE + 16 * wid + tid)


def _randn(shape, wid, tid):
    return torch.randn(*shape, generator=_g(wid, tid), dtype=torch.float32)


def _rand(shape, wid, tid):
    return torch.rand(*shape, generator=_g(wid, tid), dtype=torch.float32)


def _distinct_positions(n_rows, L, count, wid, tid):
    """count distinct positions in [0, L) per row, seeded, ascending."""
    g = _g(wid, tid)
    rows = []
    for _ in range(n_rows):
        rows.append(torch.sort(torch.randperm(L, generator=g)[:count]).values)
    return torch.stack(rows) if rows else torch.empty(0, count, dtype=torch.int64)


def _unit(v):
    return v / v.norm()


@dataclass
class DsaWorkload:
    """Inputs of one pass of the DSA hot path.

    q_idx [B,T,HI,dI], w [B,T,HI] fp32, k_idx [B,L,dI] (+ k_scale [B,L] fp32
    for fp8 keys), q_pos [B,T] int32 (None: decode, every cached position is a
    candidate), kv_len [B] int32 (None: all L valid), q_lat [B,T,H,dc],
    q_rope [B,T,H,dR], kv [B,L,dc+dR] packed latent row (c_kv then k_rope).
    """
    name: str
    B: int
    T: int
    L: int
    HI: int
    dI: int
    topk: int
    H: int
    dc: int
    dR: int
    sm_scale: float
    q_idx: torch.Tensor
    w: torch.Tensor
    k_idx: torch.Tensor
    k_scale: Optional[torch.Tensor]
    q_pos: Optional[torch.Tensor]
    kv_len: Optional[torch.Tensor]
    q_lat: torch.Tensor
    q_rope: torch.Tensor
    kv: torch.Tensor
    needles: Optional[torch.Tensor] = None
    boosted: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    def to(self, device):
        def mv(t):
            return None if t is None else t.to(device)
        out = DsaWorkload(**{**self.__dict__})
        for f in ("q_idx", "w", "k_idx", "k_scale", "q_pos", "kv_len", "q_lat",
                  "q_rope", "kv"):
            setattr(out, f, mv(getattr(self, f)))
        return out

    def slice_batch(self, b0, b1):
        """The same workload restricted to sequences b0..b1-1 (CPU tensors)."""
        def sl(t):
            return None if t is None else t[b0:b1].contiguous()
        out = DsaWorkload(**{**self.__dict__})
        for f in ("q_idx", "w", "k_idx", "k_scale", "q_pos", "kv_len", "q_lat",
                  "q_rope", "kv", "needles", "boosted"):
            setattr(out, f, sl(getattr(self, f)))
        out.B = b1 - b0
        return out


def tiny_prefill(L: int = 1024, HI: int = 4, dI: int = 64, topk: int = 64,
                 H: int = 8, dc: int = 128, dR: int = 32, B: int = 1,
                 wid: int = W_TINY_PREFILL) -> DsaWorkload:
    """Exact small causal prefill: every position is a query (q_pos = t).
    q^I, k^I uniform integers in [-2, 2]; w uniform in {1/4, 1/2, 1}; all fp32,
    so every index score is an exact multiple of 1/4.  Sparse MLA inputs
    N(0,1) fp32; sm_scale = 1/sqrt(dc + dR)."""
    T = L
    g = _g(wid, 0)
    q_idx = torch.randint(-2, 3, (B, T, HI, dI), generator=g).to(torch.float32)
    k_idx = torch.randint(-2, 3, (B, L, dI), generator=_g(wid, 1)).to(torch.float32)
    wsel = torch.tensor([0.25, 0.5, 1.0])
    w = wsel[torch.randint(0, 3, (B, T, HI), generator=_g(wid, 2))].contiguous()
    q_pos = torch.arange(T, dtype=torch.int32).repeat(B, 1).contiguous()
    q_lat = _randn((B, T, H, dc), wid, 3)
    q_rope = _randn((B, T, H, dR), wid, 4)
    kv = _randn((B, L, dc + dR), wid, 5)
    return DsaWorkload("tiny_prefill", B, T, L, HI, dI, topk, H, dc, dR,
                       1.0 / math.sqrt(dc + dR), q_idx, w, k_idx, None, q_pos,
                       None, q_lat, q_rope, kv)


def _plant_needles(q_idx, w, k_idx, q_lat, q_rope, kv, dc, positions, t_align):
    """Write aligned rows at the needle positions of every sequence:
    k^I_p = 4 sqrt(dI) unit(sum_h w_h q^I_h), c_p = 4 sqrt(dc) unit(sum_h q_lat_h),
    k^R_p = 4 sqrt(dR) unit(sum_h q_rope_h), using the stored (rounded) query
    values of query t_align."""
    B = q_idx.shape[0]
    dI = k_idx.shape[-1]
    dR = kv.shape[-1] - dc
    for b in range(B):
        qi = q_idx[b, t_align].float()
        wi = w[b, t_align].float()
        ki = 4.0 * math.sqrt(dI) * _unit((wi[:, None] * qi).sum(0))
        cl = 4.0 * math.sqrt(dc) * _unit(q_lat[b, t_align].float().sum(0))
        kr = 4.0 * math.sqrt(dR) * _unit(q_rope[b, t_align].float().sum(0)) if dR else None
        for p in positions[b].tolist():
            k_idx[b, p] = ki.to(k_idx.dtype)
            kv[b, p, :dc] = cl.to(kv.dtype)
            if dR:
                kv[b, p, dc:] = kr.to(kv.dtype)


def decode_32k(B: int = 32, L: int = 32768, HI: int = 64, dI: int = 128,
               topk: int = 2048, H: int = 128, dc: int = 512, dR: int = 64,
               n_needles: int = 16, kv_len=None,
               wid: int = W_DECODE_32K) -> DsaWorkload:
    """Batched decode: one query per sequence over L cached tokens, bf16
    indexer (HI heads of dim dI, w ~ U(0,1) fp32) and bf16 latent cache
    (c_kv dc + k_rope dR, N(0,1)), 16 planted needle rows per sequence."""
    T = 1
    q_idx = _randn((B, T, HI, dI), wid, 0).to(torch.bfloat16)
    w = _rand((B, T, HI), wid, 1)
    k_idx = _randn((B, L, dI), wid, 2).to(torch.bfloat16)
    q_lat = _randn((B, T, H, dc), wid, 3).to(torch.bfloat16)
    q_rope = _randn((B, T, H, dR), wid, 4).to(torch.bfloat16)
    kv = _randn((B, L, dc + dR), wid, 5).to(torch.bfloat16)
    kl = None
    if kv_len is not None:
        kl = torch.as_tensor(kv_len, dtype=torch.int32).reshape(B).contiguous()
    needles = None
    if n_needles:
        needles = _distinct_positions(B, L if kl is None else int(kl.min()),
                                      n_needles, wid, 6)
        _plant_needles(q_idx, w, k_idx, q_lat, q_rope, kv, dc, needles, 0)
    return DsaWorkload("decode_32k", B, T, L, HI, dI, topk, H, dc, dR,
                       1.0 / math.sqrt(dc + dR), q_idx, w, k_idx, None, None, kl,
                       q_lat, q_rope, kv, needles=needles)


def prefill_16k(L: int = 16384, HI: int = 64, dI: int = 128, topk: int = 2048,
                H: int = 128, dc: int = 512, dR: int = 64, n_needles: int = 16,
                with_mla: bool = True, wid: int = W_PREFILL_16K) -> DsaWorkload:
    """Causal prefill chunk, B = 1, T = L queries (q_pos = t), bf16 everywhere,
    needles aligned with the last query.  with_mla=False leaves the (large)
    MLA query tensors empty for indexer-only runs."""
    B, T = 1, L
    q_idx = _randn((B, T, HI, dI), wid, 0).to(torch.bfloat16)
    w = _rand((B, T, HI), wid, 1)
    k_idx = _randn((B, L, dI), wid, 2).to(torch.bfloat16)
    if with_mla:
        q_lat = _randn((B, T, H, dc), wid, 3).to(torch.bfloat16)
        q_rope = _randn((B, T, H, dR), wid, 4).to(torch.bfloat16)
    else:
        q_lat = torch.empty((B, 0, H, dc), dtype=torch.bfloat16)
        q_rope = torch.empty((B, 0, H, dR), dtype=torch.bfloat16)
    kv = _randn((B, L, dc + dR), wid, 5).to(torch.bfloat16)
    q_pos = torch.arange(T, dtype=torch.int32).reshape(1, T).contiguous()
    needles = None
    if n_needles and with_mla:
        needles = _distinct_positions(B, L, n_needles, wid, 6)
        _plant_needles(q_idx, w, k_idx, q_lat, q_rope, kv, dc, needles, T - 1)
    return DsaWorkload("prefill_16k", B, T, L, HI, dI, topk, H, dc, dR,
                       1.0 / math.sqrt(dc + dR), q_idx, w, k_idx, None, q_pos,
                       None, q_lat, q_rope, kv, needles=needles)


FP8_MAX = 448.0


def decode_128k_fp8(B: int = 8, L: int = 131072, HI: int = 64, dI: int = 128,
                    topk: int = 2048, H: int = 128, dc: int = 512, dR: int = 64,
                    boost_frac: float = 0.01, boost: float = 6.0,
                    wid: int = W_DECODE_128K_FP8) -> DsaWorkload:
    """Long-context decode with fp8 (OCP e4m3fn) indexer keys and one fp32
    scale per token (scale = max|k|/448, chosen before the cast), bf16 queries
    and bf16 latent cache.  round(boost_frac * L) positions per sequence have
    their indexer key and RoPE key multiplied by `boost` (a heavy-tailed score
    distribution); c_kv stays N(0,1)."""
    T = 1
    q_idx = _randn((B, T, HI, dI), wid, 0).to(torch.bfloat16)
    w = _rand((B, T, HI), wid, 1)
    k32 = _randn((B, L, dI), wid, 2)
    q_lat = _randn((B, T, H, dc), wid, 3).to(torch.bfloat16)
    q_rope = _randn((B, T, H, dR), wid, 4).to(torch.bfloat16)
    kv32 = _randn((B, L, dc + dR), wid, 5)
    nb = int(round(boost_frac * L))
    boosted = _distinct_positions(B, L, nb, wid, 6) if nb else None
    if boosted is not None:
        for b in range(B):
            k32[b, boosted[b]] *= boost
            kv32[b, boosted[b], dc:] *= boost
    scale = k32.abs().amax(dim=-1) / FP8_MAX
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    k8 = (k32 / scale[..., None]).to(torch.float8_e4m3fn)
    kv = kv32.to(torch.bfloat16)
    return DsaWorkload("decode_128k_fp8", B, T, L, HI, dI, topk, H, dc, dR,
                       1.0 / math.sqrt(dc + dR), q_idx, w, k8,
                       scale.contiguous(), None, None, q_lat, q_rope, kv,
                       boosted=boosted)


@dataclass
class BlockWorkload:
    """GQA block-sparse decode: q [B,Hq,d], k/v [B,L,Hkv,d] bf16."""
    name: str
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    blk: int
    nsel: int
    n_sink: int
    n_win: int
    sm_scale: float
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor

    def to(self, device):
        out = BlockWorkload(**{**self.__dict__})
        for f in ("q", "k", "v"):
            setattr(out, f, getattr(self, f).to(device))
        return out


def block_sparse_64k(B: int = 16, L: int = 65536, Hq: int = 32, Hkv: int = 8,
                     d: int = 128, blk: int = 64, nsel: int = 16,
                     n_sink: int = 64, n_win: int = 512,
                     wid: int = W_BLOCK_64K) -> BlockWorkload:
    q = _randn((B, Hq, d), wid, 0).to(torch.bfloat16)
    k = _randn((B, L, Hkv, d), wid, 1).to(torch.bfloat16)
    v = _randn((B, L, Hkv, d), wid, 2).to(torch.bfloat16)
    return BlockWorkload("block_sparse_64k", B, L, Hq, Hkv, d, blk, nsel,
                         n_sink, n_win, 1.0 / math.sqrt(d), q, k, v)


W_CSA_DECODE = 6


@dataclass
class CsaWorkload:
    """Selection over compressed entries, one query per sequence.

    q_idx [B,HI,dI] bf16, w [B,HI] fp32, k_idx [B,Lc,dI] bf16: the indexer over
    the entries' index keys; q [B,H,c] bf16; comp [B,Lc,c] bf16 compressed
    entries (keys = values); win [B,n_win,c] bf16 the most recent raw entries;
    n_comp [B] int32 entries present (None: Lc)."""
    name: str
    B: int
    Lc: int
    HI: int
    dI: int
    topk: int
    H: int
    c: int
    n_win: int
    sm_scale: float
    q_idx: torch.Tensor
    w: torch.Tensor
    k_idx: torch.Tensor
    q: torch.Tensor
    comp: torch.Tensor
    win: Optional[torch.Tensor]
    n_comp: Optional[torch.Tensor] = None

    def to(self, device):
        out = CsaWorkload(**{**self.__dict__})
        for f in ("q_idx", "w", "k_idx", "q", "comp", "win", "n_comp"):
            v = getattr(self, f)
            if v is not None:
                setattr(out, f, v.to(device))
        return out


def csa_decode(B: int = 32, Lc: int = 32768, HI: int = 64, dI: int = 128,
               topk: int = 2048, H: int = 128, c: int = 512, n_win: int = 128,
               n_comp=None, wid: int = W_CSA_DECODE) -> CsaWorkload:
    """Decode over Lc = n/m compressed entries (a 131072-token context at
    m = 4 by default) plus a window of the n_win most recent raw entries.
    The entries are synthetic N(0,1): the learned compression is the caller's."""
    q_idx = _randn((B, HI, dI), wid, 0).to(torch.bfloat16)
    w = _rand((B, HI), wid, 1)
    k_idx = _randn((B, Lc, dI), wid, 2).to(torch.bfloat16)
    q = _randn((B, H, c), wid, 3).to(torch.bfloat16)
    comp = _randn((B, Lc, c), wid, 4).to(torch.bfloat16)
    win = _randn((B, n_win, c), wid, 5).to(torch.bfloat16) if n_win else None
    nc = None
    if n_comp is not None:
        nc = torch.as_tensor(n_comp, dtype=torch.int32).reshape(B).contiguous()
    return CsaWorkload("csa_decode", B, Lc, HI, dI, topk, H, c, n_win,
                       1.0 / math.sqrt(c), q_idx, w, k_idx, q, comp, win, nc)


W_PREFILL_BATCH = 7


def prefill_batch(B: int = 2, T: int = 3000, L: int = 3000, HI: int = 64, dI: int = 128,
                  topk: int = 256, H: int = 64, dc: int = 512, dR: int = 64,
                  fp8: bool = False, q_pos: str = "causal", kv_len=None,
                  with_mla: bool = True, wid: int = W_PREFILL_BATCH) -> DsaWorkload:
    """Batched prefill with ragged candidate ranges, for the fused prefill select
    and the prefill modes.  q_pos "causal": query t sits at position t + L - T
    (the last T positions of the context); "spread": sorted random positions in
    [0, L).  kv_len: optional per-sequence cache lengths.  fp8: e4m3fn index
    keys with a per-token scale max|k|/448 (as decode_128k_fp8).  N(0,1)
    values, w U(0,1)."""
    q_idx = _randn((B, T, HI, dI), wid, 0).to(torch.bfloat16)
    w = _rand((B, T, HI), wid, 1)
    k32 = _randn((B, L, dI), wid, 2)
    scale = None
    if fp8:
        scale = k32.abs().amax(dim=-1) / FP8_MAX
        scale = torch.where(scale > 0, scale, torch.ones_like(scale)).contiguous()
        k_idx = (k32 / scale[..., None]).to(torch.float8_e4m3fn)
    else:
        k_idx = k32.to(torch.bfloat16)
    if q_pos == "causal":
        qp = (torch.arange(T, dtype=torch.int32) + (L - T)).reshape(1, T).repeat(B, 1)
    else:
        g = _g(wid, 6)
        qp = torch.sort(torch.randint(0, L, (B, T), generator=g, dtype=torch.int64), dim=1).values
        qp = qp.to(torch.int32)
    kvl = None if kv_len is None else torch.as_tensor(kv_len, dtype=torch.int32).reshape(B)
    if with_mla:
        q_lat = _randn((B, T, H, dc), wid, 3).to(torch.bfloat16)
        q_rope = _randn((B, T, H, dR), wid, 4).to(torch.bfloat16)
        kv = _randn((B, L, dc + dR), wid, 5).to(torch.bfloat16)
    else:
        q_lat = torch.empty((B, 0, H, dc), dtype=torch.bfloat16)
        q_rope = torch.empty((B, 0, H, dR), dtype=torch.bfloat16)
        kv = torch.empty((B, 0, dc + dR), dtype=torch.bfloat16)
    return DsaWorkload("prefill_batch", B, T, L, HI, dI, topk, H, dc, dR,
                       1.0 / math.sqrt(dc + dR), q_idx, w, k_idx, scale,
                       qp.contiguous(), kvl, q_lat, q_rope, kv)
