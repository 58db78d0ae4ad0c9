"""Thin Python binding of libsparse_attn.so (gfx950).

Each function carries the name of the C entry point it calls and does only
argument marshalling: it checks device, dtype, shape and layout of the torch
tensors, allocates outputs (and a workspace) when the caller passes none, and
hands raw device pointers plus torch's current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  Import fails loudly if the library has not been built.
"""
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_LIB selects another build of the same sources (the host-sanitizer build)
LIB_PATH = os.environ.get("SA_LIB") or os.path.join(_HERE, "libsparse_attn.so")

SA_OK = 0
SA_F32, SA_BF16, SA_FP8_E4M3 = 0, 1, 2
SA_OP_TOPK, SA_OP_MLA_FORWARD, SA_OP_DECODE, SA_OP_BLOCK_DECODE, SA_OP_CSA_DECODE = 0, 1, 2, 3, 4
SA_OP_PREFILL = 5
SA_PREFILL_SPARSE, SA_PREFILL_DENSE, SA_PREFILL_AUTO = 0, 1, 2

_DTYPE = {torch.float32: SA_F32, torch.bfloat16: SA_BF16, torch.float8_e4m3fn: SA_FP8_E4M3}

EXPORTS = (
    "sparse_attn_indexer_scores", "sparse_attn_topk", "sparse_attn_mla_forward",
    "sparse_attn_decode", "sparse_attn_decode_noalloc", "sparse_attn_block_pool",
    "sparse_attn_block_decode",
    "sparse_attn_csa_decode", "sparse_attn_prefill_select", "sparse_attn_prefill",
    "sparse_attn_workspace_bytes", "sparse_attn_status_string", "sparse_attn_last_error",
)

_lib = None


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        name = lib.sparse_attn_status_string(status).decode()
        detail = lib.sparse_attn_last_error().decode()
        super().__init__(f"{where}: {name}: {detail}")
        self.status = status


def load():
    """Load libsparse_attn.so (raises if it is missing: no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python top_indexer_sparse_amd/build.py` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                        ctypes.c_size_t)
    L.sparse_attn_indexer_scores.argtypes = [P, I, P, P, I, P, P, P, I, I, I, I, I, P, P]
    L.sparse_attn_topk.argtypes = [P, P, P, I, I, I, I, P, P, P, SZ, P]
    L.sparse_attn_mla_forward.argtypes = [P, P, I, P, P, I, I64, I64, P, I, I, I, I, I, I,
                                          I, F, P, P, P, SZ, P]
    L.sparse_attn_decode.argtypes = [P, I, P, P, I, P, P, I, I, I, I, I, P, P, I, P, P, I,
                                     I64, I64, I, I, I, F, P, P, P, P, SZ, P]
    L.sparse_attn_decode_noalloc.argtypes = [P, I, P, P, I, P, P, I, I, I, I, I, P, P, I, P, P,
                                             I, I64, I64, I, I, I, F, P, P, P, P]
    L.sparse_attn_block_pool.argtypes = [P, I, I, I, I, I, P, P]
    L.sparse_attn_block_decode.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, P,
                                           P, P, SZ, P]
    L.sparse_attn_csa_decode.argtypes = [P, I, P, P, I, P, P, I, I, I, I, I, P, P, P, I, I, I, F,
                                         P, P, P, P, SZ, P]
    L.sparse_attn_prefill_select.argtypes = [P, I, P, P, I, P, P, P, I, I, I, I, I, I, P, P, P]
    L.sparse_attn_prefill.argtypes = [P, I, P, P, I, P, P, P, I, I, I, I, I, I, P, P, P, P, I64,
                                      I64, I, I, I, F, I, P, P, P, P, SZ, P]
    L.sparse_attn_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    L.sparse_attn_workspace_bytes.restype = SZ
    L.sparse_attn_status_string.argtypes = [I]
    L.sparse_attn_status_string.restype = ctypes.c_char_p
    L.sparse_attn_last_error.argtypes = []
    L.sparse_attn_last_error.restype = ctypes.c_char_p
    for f in ("sparse_attn_indexer_scores", "sparse_attn_topk", "sparse_attn_mla_forward",
              "sparse_attn_decode", "sparse_attn_decode_noalloc", "sparse_attn_block_pool",
              "sparse_attn_block_decode", "sparse_attn_csa_decode", "sparse_attn_prefill_select", "sparse_attn_prefill"):
        getattr(L, f).restype = I
    _lib = L
    return L


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, shape=None, contiguous=True, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _call(fn_name, *args):
    s = getattr(load(), fn_name)(*args)
    if s != SA_OK:
        raise SparseAttnError(s, fn_name)


def _rows(t: torch.Tensor, name: str, B: int, L: int):
    """(row stride in elements) of a [B, L, d] view whose rows may be strided."""
    if t.dim() != 3 or t.shape[0] != B or t.shape[1] != L:
        raise ValueError(f"{name} must be [B={B}, L={L}, d], got {tuple(t.shape)}")
    if t.stride(2) != 1 or (B > 1 and t.stride(0) != L * t.stride(1)):
        raise ValueError(f"{name}: rows must be unit-stride and laid out as [B*L] rows")
    return t.stride(1)


def sparse_attn_workspace_bytes(op: int, B: int, T: int, L: int, k: int, H: int, dc: int) -> int:
    return int(load().sparse_attn_workspace_bytes(op, B, T, L, k, H, dc))


def _workspace(ws, nbytes, device):
    if nbytes == 0:
        return ws, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws, ws.numel() * ws.element_size()


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def sparse_attn_indexer_scores(q_idx, w, k_idx, k_scale=None, q_pos=None, kv_len=None,
                               scores=None, stream=None):
    """Index scores [B,T,L] fp32 (-inf for non-candidates)."""
    B, T, HI, dI = q_idx.shape
    L = k_idx.shape[1]
    _need(q_idx, "q_idx", (torch.float32, torch.bfloat16))
    _need(w, "w", (torch.float32,), (B, T, HI))
    _need(k_idx, "k_idx", (torch.float32, torch.bfloat16, torch.float8_e4m3fn), (B, L, dI))
    _need(k_scale, "k_scale", (torch.float32,), (B, L), optional=True)
    _need(q_pos, "q_pos", (torch.int32,), (B, T), optional=True)
    _need(kv_len, "kv_len", (torch.int32,), (B,), optional=True)
    if scores is None:
        scores = torch.empty((B, T, L), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", (torch.float32,), (B, T, L))
    _call("sparse_attn_indexer_scores", _ptr(q_idx), _DTYPE[q_idx.dtype], _ptr(w),
          _ptr(k_idx), _DTYPE[k_idx.dtype], _ptr(k_scale), _ptr(q_pos), _ptr(kv_len),
          B, T, L, HI, dI, _ptr(scores), _stream(stream))
    return scores


def sparse_attn_topk(scores, k, q_pos=None, kv_len=None, idx=None, count=None, ws=None,
                     stream=None):
    """(idx [B,T,k] int32 ascending, -1 padded; count [B,T] int32)."""
    B, T, L = scores.shape
    _need(scores, "scores", (torch.float32,))
    _need(q_pos, "q_pos", (torch.int32,), (B, T), optional=True)
    _need(kv_len, "kv_len", (torch.int32,), (B,), optional=True)
    dev = scores.device
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, T), dtype=torch.int32, device=dev)
    _need(idx, "idx", (torch.int32,), (B, T, k))
    _need(count, "count", (torch.int32,), (B, T))
    ws, nb = _workspace(ws, sparse_attn_workspace_bytes(SA_OP_TOPK, B, T, L, k, 0, 0), dev)
    _call("sparse_attn_topk", _ptr(scores), _ptr(q_pos), _ptr(kv_len), B, T, L, k, _ptr(idx),
          _ptr(count), _ptr(ws), nb, _stream(stream))
    return idx, count


def sparse_attn_mla_forward(q_lat, q_rope, c_kv, k_rope, idx, sm_scale, out=None, lse=None,
                            ws=None, stream=None):
    """Sparse MLA over idx -> (out [B,T,H,dc] fp32, lse [B,T,H] fp32).

    c_kv [B,L,dc] and k_rope [B,L,dR] may be strided row views of one packed
    [B,L,dc+dR] cache (kv[..., :dc], kv[..., dc:])."""
    B, T, H, dc = q_lat.shape
    L = c_kv.shape[1]
    dR = q_rope.shape[-1] if q_rope is not None else 0
    dt = q_lat.dtype
    _need(q_lat, "q_lat", (torch.float32, torch.bfloat16))
    if dR:
        _need(q_rope, "q_rope", (dt,), (B, T, H, dR))
        _need(k_rope, "k_rope", (dt,), contiguous=False)
    _need(c_kv, "c_kv", (dt,), contiguous=False)
    _need(idx, "idx", (torch.int32,))
    if idx.dim() != 3 or idx.shape[:2] != (B, T):
        raise ValueError(f"idx must be [B,T,k], got {tuple(idx.shape)}")
    k = idx.shape[2]
    cs = _rows(c_kv, "c_kv", B, L)
    rs = _rows(k_rope, "k_rope", B, L) if dR else 0
    if dR and k_rope.shape[2] != dR:
        raise ValueError("k_rope width != q_rope width")
    if c_kv.shape[2] != dc:
        raise ValueError("c_kv width != q_lat width")
    dev = q_lat.device
    if out is None:
        out = torch.empty((B, T, H, dc), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), (B, T, H, dc))
    _need(lse, "lse", (torch.float32,), (B, T, H))
    ws, nb = _workspace(ws, sparse_attn_workspace_bytes(SA_OP_MLA_FORWARD, B, T, L, k, H, dc),
                        dev)
    _call("sparse_attn_mla_forward", _ptr(q_lat), _ptr(q_rope) if dR else None, _DTYPE[dt],
          _ptr(c_kv), _ptr(k_rope) if dR else None, _DTYPE[dt], cs, rs, _ptr(idx), k, B, T, L,
          H, dc, dR, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), nb, _stream(stream))
    return out, lse


def _decode_args(q_idx, w, k_idx, k_scale, kv_len, topk, q_lat, q_rope, c_kv, k_rope, sm_scale,
                 out, lse, idx_out):
    """Checked arguments of the fused decode, up to the workspace."""
    B, T, HI, dI = q_idx.shape
    if T != 1:
        raise ValueError("sparse_attn_decode takes one query per sequence (T = 1)")
    L = k_idx.shape[1]
    _, _, H, dc = q_lat.shape
    dR = q_rope.shape[-1]
    dt = q_lat.dtype
    _need(q_idx, "q_idx", (torch.float32, torch.bfloat16))
    _need(w, "w", (torch.float32,), (B, 1, HI))
    _need(k_idx, "k_idx", (torch.float32, torch.bfloat16, torch.float8_e4m3fn), (B, L, dI))
    _need(k_scale, "k_scale", (torch.float32,), (B, L), optional=True)
    _need(kv_len, "kv_len", (torch.int32,), (B,), optional=True)
    _need(q_lat, "q_lat", (torch.float32, torch.bfloat16), (B, 1, H, dc))
    _need(q_rope, "q_rope", (dt,), (B, 1, H, dR))
    _need(c_kv, "c_kv", (dt,), contiguous=False)
    _need(k_rope, "k_rope", (dt,), contiguous=False)
    cs, rs = _rows(c_kv, "c_kv", B, L), _rows(k_rope, "k_rope", B, L)
    dev = q_idx.device
    if out is None:
        out = torch.empty((B, 1, H, dc), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=dev)
    if idx_out is None:
        idx_out = torch.empty((B, 1, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.float32,), (B, 1, H, dc))
    _need(lse, "lse", (torch.float32,), (B, 1, H))
    _need(idx_out, "idx_out", (torch.int32,), (B, 1, topk))
    args = (_ptr(q_idx), _DTYPE[q_idx.dtype], _ptr(w), _ptr(k_idx), _DTYPE[k_idx.dtype],
            _ptr(k_scale), _ptr(kv_len), B, L, HI, dI, topk, _ptr(q_lat), _ptr(q_rope), _DTYPE[dt],
            _ptr(c_kv), _ptr(k_rope), _DTYPE[dt], cs, rs, H, dc, dR, float(sm_scale), _ptr(out),
            _ptr(lse), _ptr(idx_out))
    return args, out, lse, idx_out, (B, L, H, dc, dev)


def sparse_attn_decode(q_idx, w, k_idx, k_scale, kv_len, topk, q_lat, q_rope, c_kv, k_rope,
                       sm_scale, out=None, lse=None, idx_out=None, ws=None, stream=None):
    """Fused decode step (T = 1) -> (out [B,1,H,dc], lse [B,1,H], idx [B,1,k])."""
    args, out, lse, idx_out, (B, L, H, dc, dev) = _decode_args(
        q_idx, w, k_idx, k_scale, kv_len, topk, q_lat, q_rope, c_kv, k_rope, sm_scale, out, lse,
        idx_out)
    ws, nb = _workspace(ws, sparse_attn_workspace_bytes(SA_OP_DECODE, B, 1, L, topk, H, dc), dev)
    _call("sparse_attn_decode", *args, _ptr(ws), nb, _stream(stream))
    return out, lse, idx_out


def sparse_attn_decode_noalloc(q_idx, w, k_idx, k_scale, kv_len, topk, q_lat, q_rope, c_kv,
                               k_rope, sm_scale, out=None, lse=None, idx_out=None, stream=None):
    """sparse_attn_decode with the library's fixed per-GPU scratch instead of a
    workspace; with out, lse and idx_out given, nothing is allocated."""
    args, out, lse, idx_out, _ = _decode_args(
        q_idx, w, k_idx, k_scale, kv_len, topk, q_lat, q_rope, c_kv, k_rope, sm_scale, out, lse,
        idx_out)
    _call("sparse_attn_decode_noalloc", *args, _stream(stream))
    return out, lse, idx_out


def sparse_attn_prefill_select(q_idx, w, k_idx, topk, k_scale=None, q_pos=None, kv_len=None,
                               idx=None, count=None, stream=None):
    """Fused indexer + Top-K, no score tensor -> (idx [B,T,k] int32 ascending,
    -1 padded; count [B,T] int32)."""
    B, T, HI, dI = q_idx.shape
    L = k_idx.shape[1]
    _need(q_idx, "q_idx", (torch.bfloat16,))
    _need(w, "w", (torch.float32,), (B, T, HI))
    _need(k_idx, "k_idx", (torch.bfloat16, torch.float8_e4m3fn), (B, L, dI))
    _need(k_scale, "k_scale", (torch.float32,), (B, L), optional=True)
    _need(q_pos, "q_pos", (torch.int32,), (B, T), optional=True)
    _need(kv_len, "kv_len", (torch.int32,), (B,), optional=True)
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((B, T, topk), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((B, T), dtype=torch.int32, device=dev)
    _need(idx, "idx", (torch.int32,), (B, T, topk))
    _need(count, "count", (torch.int32,), (B, T))
    _call("sparse_attn_prefill_select", _ptr(q_idx), _DTYPE[q_idx.dtype], _ptr(w), _ptr(k_idx),
          _DTYPE[k_idx.dtype], _ptr(k_scale), _ptr(q_pos), _ptr(kv_len), B, T, L, HI, dI, topk,
          _ptr(idx), _ptr(count), _stream(stream))
    return idx, count


def sparse_attn_prefill(q_idx, w, k_idx, topk, q_lat, q_rope, c_kv, k_rope, sm_scale,
                        k_scale=None, q_pos=None, kv_len=None, mode=SA_PREFILL_SPARSE, out=None,
                        lse=None, idx_out=None, ws=None, stream=None):
    """Whole causal prefill -> (out [B,T,H,dc] fp32, lse [B,T,H] fp32).

    mode SA_PREFILL_SPARSE: fused select + sparse MLA (idx_out, if given,
    receives the sets); SA_PREFILL_DENSE: MLA over every causal candidate
    (q_idx, w, k_idx may be None); SA_PREFILL_AUTO: dense when L <= topk (the
    two modes then attend to the same rows).  c_kv / k_rope as in
    sparse_attn_mla_forward."""
    B, T, H, dc = q_lat.shape
    L = c_kv.shape[1]
    dR = q_rope.shape[-1]
    _need(q_lat, "q_lat", (torch.bfloat16,))
    _need(q_rope, "q_rope", (torch.bfloat16,), (B, T, H, dR))
    _need(c_kv, "c_kv", (torch.bfloat16,), contiguous=False)
    _need(k_rope, "k_rope", (torch.bfloat16,), contiguous=False)
    cs, rs = _rows(c_kv, "c_kv", B, L), _rows(k_rope, "k_rope", B, L)
    dense = mode == SA_PREFILL_DENSE or (mode == SA_PREFILL_AUTO and L <= topk)
    HI = dI = 0
    if q_idx is not None:
        _, _, HI, dI = q_idx.shape
        _need(q_idx, "q_idx", (torch.bfloat16,), (B, T, HI, dI))
        _need(w, "w", (torch.float32,), (B, T, HI))
        _need(k_idx, "k_idx", (torch.bfloat16, torch.float8_e4m3fn), (B, L, dI))
        _need(k_scale, "k_scale", (torch.float32,), (B, L), optional=True)
    elif not dense:
        raise ValueError("the sparse mode needs q_idx, w and k_idx")
    _need(q_pos, "q_pos", (torch.int32,), (B, T), optional=True)
    _need(kv_len, "kv_len", (torch.int32,), (B,), optional=True)
    dev = q_lat.device
    if out is None:
        out = torch.empty((B, T, H, dc), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    _need(out, "out", (torch.float32,), (B, T, H, dc))
    _need(lse, "lse", (torch.float32,), (B, T, H))
    _need(idx_out, "idx_out", (torch.int32,), (B, T, topk), optional=True)
    ws, nb = _workspace(ws, sparse_attn_workspace_bytes(SA_OP_PREFILL, B, T, L, topk, H, dc), dev)
    kd = _DTYPE[k_idx.dtype] if k_idx is not None else SA_BF16
    _call("sparse_attn_prefill", _ptr(q_idx), SA_BF16, _ptr(w), _ptr(k_idx), kd, _ptr(k_scale),
          _ptr(q_pos), _ptr(kv_len), B, T, L, HI, dI, topk, _ptr(q_lat), _ptr(q_rope), _ptr(c_kv),
          _ptr(k_rope), cs, rs, H, dc, dR, float(sm_scale), int(mode), _ptr(out), _ptr(lse),
          _ptr(idx_out), _ptr(ws), nb, _stream(stream))
    return out, lse


def sparse_attn_csa_decode(q_idx, w, k_idx, k_scale, n_comp, topk, q, comp, win, sm_scale,
                           out=None, lse=None, idx_out=None, ws=None, stream=None):
    """Selection over compressed entries (T = 1) -> (out [B,H,c], lse [B,H], idx [B,k]).

    q_idx [B,HI,dI], w [B,HI], k_idx [B,Lc,dI] (+ k_scale [B,Lc] for fp8): the
    indexer over the entries' index keys; q [B,H,c] bf16; comp [B,Lc,c] bf16
    entries; win [B,n_win,c] bf16 raw window entries or None."""
    B, HI, dI = q_idx.shape
    Lc = k_idx.shape[1]
    _, H, c = q.shape
    n_win = 0 if win is None else win.shape[1]
    _need(q_idx, "q_idx", (torch.float32, torch.bfloat16))
    _need(w, "w", (torch.float32,), (B, HI))
    _need(k_idx, "k_idx", (torch.float32, torch.bfloat16, torch.float8_e4m3fn), (B, Lc, dI))
    _need(k_scale, "k_scale", (torch.float32,), (B, Lc), optional=True)
    _need(n_comp, "n_comp", (torch.int32,), (B,), optional=True)
    _need(q, "q", (torch.bfloat16,), (B, H, c))
    _need(comp, "comp", (torch.bfloat16,), (B, Lc, c))
    _need(win, "win", (torch.bfloat16,), (B, n_win, c), optional=True)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if idx_out is None:
        idx_out = torch.empty((B, topk), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.float32,), (B, H, c))
    _need(lse, "lse", (torch.float32,), (B, H))
    _need(idx_out, "idx_out", (torch.int32,), (B, topk))
    ws, nb = _workspace(ws, sparse_attn_workspace_bytes(SA_OP_CSA_DECODE, B, n_win, Lc, topk, H, c),
                        dev)
    _call("sparse_attn_csa_decode", _ptr(q_idx), _DTYPE[q_idx.dtype], _ptr(w), _ptr(k_idx),
          _DTYPE[k_idx.dtype], _ptr(k_scale), _ptr(n_comp), B, Lc, HI, dI, topk, _ptr(q),
          _ptr(comp), _ptr(win), n_win, H, c, float(sm_scale), _ptr(out), _ptr(lse),
          _ptr(idx_out), _ptr(ws), nb, _stream(stream))
    return out, lse, idx_out


def sparse_attn_block_pool(k, blk, krep=None, stream=None):
    """Mean-pooled block keys krep [B, L//blk, Hkv, d] bf16 (the fp32 mean,
    rounded to nearest even)."""
    B, L, Hkv, d = k.shape
    _need(k, "k", (torch.bfloat16,))
    if krep is None:
        krep = torch.empty((B, L // blk, Hkv, d), dtype=torch.bfloat16, device=k.device)
    _need(krep, "krep", (torch.bfloat16,), (B, L // blk, Hkv, d))
    _call("sparse_attn_block_pool", _ptr(k), B, L, Hkv, d, blk, _ptr(krep) if krep.numel() else None,
          _stream(stream))
    return krep


def sparse_attn_block_decode(q, k, v, krep, blk, nsel, n_sink, n_win, sm_scale, out=None,
                             blocks_out=None, ws=None, stream=None, shared_choice=False):
    """GQA block-sparse decode -> (out [B,Hq,d] fp32, blocks [B,Hq,nsel] int32).
    shared_choice: the heads of a KV group share one block choice."""
    B, Hq, d = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    _need(q, "q", (torch.bfloat16,))
    _need(k, "k", (torch.bfloat16,), (B, L, Hkv, d))
    _need(v, "v", (torch.bfloat16,), (B, L, Hkv, d))
    _need(krep, "krep", (torch.bfloat16,), (B, L // blk, Hkv, d))
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if blocks_out is None:
        blocks_out = torch.empty((B, Hq, nsel), dtype=torch.int32, device=dev)
    _need(out, "out", (torch.float32,), (B, Hq, d))
    _need(blocks_out, "blocks_out", (torch.int32,), (B, Hq, nsel))
    ws, nb = _workspace(ws, sparse_attn_workspace_bytes(SA_OP_BLOCK_DECODE, B, Hq, L, nsel, Hkv,
                                                        d), dev)
    _call("sparse_attn_block_decode", _ptr(q), _ptr(k), _ptr(v),
          _ptr(krep) if krep.numel() else None, B, L, Hq, Hkv, d,
          blk, nsel, n_sink, n_win, float(sm_scale), int(bool(shared_choice)), _ptr(out),
          _ptr(blocks_out), _ptr(ws), nb, _stream(stream))
    return out, blocks_out
