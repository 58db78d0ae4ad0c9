"""Python face of the CPU oracle (TEST INFRASTRUCTURE).

Only tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py may
import this package.  The GPU library never does, and this package imports
nothing from it.

Inputs are torch CPU tensors in their storage dtype (the exact bytes the GPU
receives).  They are decoded to float64 by the oracle's own C decoders (bf16
bit layout, OCP E4M3 definition); fp32 widens exactly.  All arithmetic happens
in liboracle.so (see sa_oracle.c), in double precision.
"""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_ORACLE_LIB selects another build of the same source (the sanitizer build)
_LIB_PATH = os.environ.get("SA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_ARG, ERR_NONFINITE, ERR_EMPTY, ERR_NOMEM = 0, -1, -2, -3, -4


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        D = ctypes.c_double
        L.orc_num_threads.restype = I
        L.orc_decode_bf16.argtypes = [P, P, I64]
        L.orc_decode_e4m3fn.argtypes = [P, P, I64]
        L.orc_indexer.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
        L.orc_topk.argtypes = [P, P, P, I, I, I, I, P, P]
        L.orc_sparse_mla.argtypes = [P, P, P, P, I64, I64, P, I, I, I, I, I,
                                     I, I, D, P, P]
        L.orc_masked_mla.argtypes = [P, P, P, P, I64, I64, P, I, I, I, I, I,
                                     I, D, P, P]
        L.orc_block_pool.argtypes = [P, I, I, I, I, I, P]
        L.orc_block_sparse_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, I,
                                              I, I, D, I, P, P, P]
        for f in ("orc_indexer", "orc_topk", "orc_sparse_mla", "orc_masked_mla",
                  "orc_block_pool", "orc_block_sparse_decode"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().orc_num_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(code, what):
    if code != OK:
        raise OracleError(code, what)


# --------------------------------------------------------------------------
# decoding
# --------------------------------------------------------------------------

def decode(t) -> np.ndarray:
    """Exact float64 value of every element of a CPU tensor (bf16, e4m3fn,
    fp32, fp64) or numpy array, decoded by the oracle's own decoders."""
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t, dtype=np.float64)
    t = t.detach().cpu().contiguous()
    out = np.empty(tuple(t.shape), dtype=np.float64)
    n = t.numel()
    if t.dtype == torch.bfloat16:
        raw = t.view(torch.int16).numpy().view(np.uint16)
        lib().orc_decode_bf16(_ptr(raw), _ptr(out), n)
    elif t.dtype == torch.float8_e4m3fn:
        raw = t.view(torch.uint8).numpy()
        lib().orc_decode_e4m3fn(_ptr(raw), _ptr(out), n)
    elif t.dtype in (torch.float32, torch.float64):
        out[...] = t.numpy().astype(np.float64)
    else:
        raise TypeError(f"oracle cannot decode {t.dtype}")
    return out


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().orc_decode_bf16(_ptr(bits), _ptr(out), bits.size)
    return out


def decode_e4m3fn_bits(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().orc_decode_e4m3fn(_ptr(bits), _ptr(out), bits.size)
    return out


def dequantized_keys(k_idx, k_scale=None) -> np.ndarray:
    """Indexer keys as stored: fp8 code value times the row's fp32 scale."""
    k = decode(k_idx)
    if k_scale is not None:
        k = k * decode(k_scale)[..., None]
    return k


def _i32(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(t, dtype=np.int32)


# --------------------------------------------------------------------------
# the method
# --------------------------------------------------------------------------

def indexer(q_idx, w, k_idx, k_scale=None, q_pos=None, kv_len=None):
    """I[b,t,s] (float64, -inf for non-candidates).  Shapes as the GPU API:
    q_idx[B,T,HI,dI], w[B,T,HI], k_idx[B,L,dI], k_scale[B,L]."""
    q = decode(q_idx)
    wd = decode(w)
    k = dequantized_keys(k_idx, k_scale)
    B, T, HI, dI = q.shape
    L = k.shape[1]
    qp, kl = _i32(q_pos), _i32(kv_len)
    out = np.empty((B, T, L), dtype=np.float64)
    _check(lib().orc_indexer(_ptr(q), _ptr(wd), _ptr(k), _ptr(qp), _ptr(kl),
                             B, T, L, HI, dI, _ptr(out)), "indexer")
    return out


def topk(scores, k, q_pos=None, kv_len=None):
    """(idx[B,T,k] int32 ascending, -1 padded; count[B,T] int32)."""
    s = decode(scores) if isinstance(scores, torch.Tensor) else \
        np.ascontiguousarray(scores, dtype=np.float64)
    B, T, L = s.shape
    qp, kl = _i32(q_pos), _i32(kv_len)
    idx = np.empty((B, T, k), dtype=np.int32)
    cnt = np.empty((B, T), dtype=np.int32)
    _check(lib().orc_topk(_ptr(s), _ptr(qp), _ptr(kl), B, T, L, k, _ptr(idx),
                          _ptr(cnt)), "topk")
    return idx, cnt


def _split_cache(kv, dc, k_rope=None):
    """Return (c_kv rows, k_rope rows, c_stride, r_stride) as float64 arrays.
    kv is either the packed [B,L,dc+dR] cache (k_rope None) or c_kv[B,L,dc]
    with a separate k_rope[B,L,dR]."""
    if k_rope is None:
        full = decode(kv)
        B, L, D = full.shape
        dR = D - dc
        return full, (full[..., dc:] if dR > 0 else None), D, D, dR
    c = decode(kv)
    r = decode(k_rope)
    return c, r, c.shape[-1], r.shape[-1], r.shape[-1]


def sparse_mla(q_lat, q_rope, kv, idx, sm_scale, dc=None, k_rope=None,
               allow_empty=False):
    """Sparse MLA on the gathered set idx[B,T,k] -> (out[B,T,H,dc], lse[B,T,H])."""
    ql = decode(q_lat)
    B, T, H, dcq = ql.shape
    dc = dcq if dc is None else dc
    c, r, cs, rs, dR = _split_cache(kv, dc, k_rope)
    qr = decode(q_rope) if dR > 0 else None
    L = c.shape[1]
    ix = _i32(idx)
    k = ix.shape[-1]
    out = np.empty((B, T, H, dc), dtype=np.float64)
    lse = np.empty((B, T, H), dtype=np.float64)
    rptr = None
    if dR > 0:
        # the rope rows start dc elements into the packed row
        rbase = r if k_rope is not None else c
        rptr = rbase.ctypes.data + (0 if k_rope is not None else dc * 8)
    code = lib().orc_sparse_mla(_ptr(ql), _ptr(qr), _ptr(c),
                                ctypes.c_void_p(rptr) if rptr else None, cs, rs,
                                _ptr(ix), k, B, T, L, H, dc, dR, sm_scale,
                                _ptr(out), _ptr(lse))
    if not (allow_empty and code == ERR_EMPTY):
        _check(code, "sparse_mla")
    return out, lse


def masked_mla(q_lat, q_rope, kv, visible, sm_scale, dc=None, k_rope=None):
    """Mask form softmax(s + M) over all L positions (dense when all visible)."""
    ql = decode(q_lat)
    B, T, H, dcq = ql.shape
    dc = dcq if dc is None else dc
    c, r, cs, rs, dR = _split_cache(kv, dc, k_rope)
    qr = decode(q_rope) if dR > 0 else None
    L = c.shape[1]
    vis = np.ascontiguousarray(np.asarray(visible, dtype=np.uint8))
    assert vis.shape == (B, T, L)
    out = np.empty((B, T, H, dc), dtype=np.float64)
    lse = np.empty((B, T, H), dtype=np.float64)
    rptr = None
    if dR > 0:
        rbase = r if k_rope is not None else c
        rptr = rbase.ctypes.data + (0 if k_rope is not None else dc * 8)
    _check(lib().orc_masked_mla(_ptr(ql), _ptr(qr), _ptr(c),
                                ctypes.c_void_p(rptr) if rptr else None, cs, rs,
                                _ptr(vis), B, T, L, H, dc, dR, sm_scale,
                                _ptr(out), _ptr(lse)), "masked_mla")
    return out, lse


def csa_decode(q_idx, w, k_idx, q, comp, win, k, sm_scale, k_scale=None, n_comp=None,
               allow_empty=False):
    """Selection over compressed entries, one query per sequence
    ("LLM注意力优化：稀疏注意力", DeepSeek CSA & HCA section):
      1. index scores of the query against the Lc entries' index keys (the DSA
         indexer, over n_comp[b] present entries);
      2. the top-k entries by the DSA rule;
      3. core attention as MQA with the entries as both keys and values, over
         the selected entries and the n_win most recent raw entries (win),
         one softmax over the union: o_h = sum_j softmax_j(q_h . e_j * scale) e_j.
    q_idx [B,HI,dI], w [B,HI], k_idx [B,Lc,dI]; q [B,H,c]; comp [B,Lc,c];
    win [B,n_win,c] or None.
    -> (out[B,H,c], lse[B,H], idx[B,k] ascending -1 padded, count[B])"""
    qi, wi = q_idx[:, None], w[:, None]
    s = indexer(qi, wi, k_idx, k_scale=k_scale, kv_len=n_comp)
    idx, cnt = topk(s, k, kv_len=n_comp)
    out, lse = csa_attention(q, comp, win, _i32(idx)[:, 0], sm_scale, allow_empty=allow_empty)
    return out, lse, _i32(idx)[:, 0], np.asarray(cnt)[:, 0]


def csa_attention(q, comp, win, idx, sm_scale, allow_empty=False):
    """Core attention of csa_decode given the selected entries idx[B,k]
    (-1 = none): keys = values = entries, over the selected entries and every
    window entry, one softmax.  -> (out[B,H,c], lse[B,H])"""
    cd = decode(comp)
    B, Lc, c = cd.shape
    if win is not None and win.shape[1] > 0:
        wd = decode(win)
        rows = np.concatenate([cd, wd], axis=1)
        n_win = wd.shape[1]
    else:
        rows, n_win = cd, 0
    wslots = np.broadcast_to(Lc + np.arange(n_win, dtype=np.int32), (B, n_win))
    full = np.concatenate([_i32(idx), wslots], axis=-1)[:, None]
    out, lse = sparse_mla(decode(q)[:, None], None, rows, full, sm_scale, dc=c,
                          allow_empty=allow_empty)
    return out[:, 0], lse[:, 0]


def block_pool(k, blk):
    """Mean-pooled block keys krep[B, L//blk, Hkv, d] over complete blocks."""
    kd = decode(k)
    B, L, Hkv, d = kd.shape
    out = np.empty((B, L // blk, Hkv, d), dtype=np.float64)
    _check(lib().orc_block_pool(_ptr(kd), B, L, Hkv, d, blk, _ptr(out)),
           "block_pool")
    return out


def block_sparse_decode(q, k, v, blk, nsel, n_sink, n_win, sm_scale, krep=None,
                        shared=False, given_blocks=None, allow_empty=False):
    """GQA block-sparse decode -> (out[B,Hq,d], blocks[B,Hq,nsel]).

    shared=True: the query heads of a KV group share one block choice, by the
    sum of their block scores ("MLA 与稀疏注意力", block choice and merging).
    given_blocks[B,Hq,nsel]: attend over these blocks (entries outside
    [0, L // blk) ignored) instead of choosing; blocks then echoes the given
    valid blocks in ascending order.  allow_empty: a head with an empty
    visible set gets out = 0 instead of raising."""
    qd, kd, vd = decode(q), decode(k), decode(v)
    B, Hq, d = qd.shape
    L, Hkv = kd.shape[1], kd.shape[2]
    kr = block_pool(k, blk) if krep is None else decode(krep)
    out = np.empty((B, Hq, d), dtype=np.float64)
    blocks = np.empty((B, Hq, max(nsel, 1)), dtype=np.int32)
    gb = None
    if given_blocks is not None:
        gb = _i32(given_blocks)
        assert gb.shape == (B, Hq, nsel), "given_blocks must be [B, Hq, nsel]"
    code = lib().orc_block_sparse_decode(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(kr),
                                         B, L, Hq, Hkv, d, blk, nsel, n_sink,
                                         n_win, sm_scale, int(bool(shared)),
                                         _ptr(gb), _ptr(out), _ptr(blocks))
    if not (allow_empty and code == ERR_EMPTY):
        _check(code, "block_sparse_decode")
    return out, blocks[..., :nsel]
