"""ctypes binding of libsas (C ABI declared in include/sas.h).

Argument marshalling only: shapes are read off the torch tensors, outputs and
workspaces are allocated with torch when the caller does not pass them, and
every call goes to the HIP library on the current torch stream.  There is no
fallback: if libsas.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsas.so")

SAS_OK, SAS_ERR_INVALID_ARGUMENT, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE_TOO_SMALL, SAS_ERR_HIP = range(5)
SAS_F32, SAS_BF16 = 0, 1
SAS_SELECT_DECODE, SAS_SELECT_TILES, SAS_SELECT_QUERIES = 0, 1, 2
(SAS_OP_SELECT_DECODE, SAS_OP_SELECT_TILES, SAS_OP_DECODE_FWD, SAS_OP_PREFILL_FWD, SAS_OP_BWD,
 SAS_OP_DECODE_STEP, SAS_OP_SELECTOR_BWD, SAS_OP_SELECT_QUERIES, SAS_OP_PREFILL_FWD_QUERIES,
 SAS_OP_BWD_QUERIES, SAS_OP_SELECTOR_BWD_QUERIES) = range(11)
BLOCK = 64
SIZE_MAX = 2 ** 64 - 1


class SasDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "sel_dim", "block_size", "top_k",
        "t_max", "dtype")]


class SasError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_PD = ctypes.POINTER(SasDims)
_SIGNATURES = {
    "sas_block_summaries": (_i32, [_PD, _vp, _vp, _vp, _i32, _i32, _vp, _vp]),
    "sas_select": (_i32, [_PD, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sas_decode_fwd": (_i32, [_PD, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp]),
    "sas_decode_step": (_i32, [_PD, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32, _vp, _vp, _vp,
                               _vp, _vp, _vp, _sz, _vp]),
    "sas_block_summaries_paged": (_i32, [_PD, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp]),
    "sas_decode_step_paged": (_i32, [_PD, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32,
                                     _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "sas_prefill_fwd": (_i32, [_PD, _vp, _vp, _vp, _i32, _vp, _vp, _f32, _vp, _vp, _vp, _sz, _vp]),
    "sas_prefill_fwd_queries": (_i32, [_PD, _vp, _vp, _vp, _i32, _vp, _vp, _f32, _vp, _vp, _vp,
                                       _sz, _vp]),
    "sas_bwd": (_i32, [_PD, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _f32, _vp, _vp, _vp,
                       _vp, _vp, _sz, _vp]),
    "sas_bwd_queries": (_i32, [_PD, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _f32, _vp, _vp,
                               _vp, _vp, _vp, _sz, _vp]),
    "sas_selector_bwd": (_i32, [_PD, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _sz, _vp]),
    "sas_selector_bwd_queries": (_i32, [_PD, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _sz, _vp]),
    "sas_workspace_bytes": (_sz, [_i32, _PD, _i32]),
    "sas_status_str": (ctypes.c_char_p, [_i32]),
    "sas_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load_library():
    """Load libsas.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gated_block_sparse_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _status_name(status: int) -> str:
    names = {0: "SAS_OK", 1: "SAS_ERR_INVALID_ARGUMENT", 2: "SAS_ERR_UNSUPPORTED",
             3: "SAS_ERR_WORKSPACE_TOO_SMALL", 4: "SAS_ERR_HIP"}
    return names.get(status, f"status {status}")


def _check(status: int):
    if status != SAS_OK:
        raise SasError(status, load_library().sas_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SAS_F32
    if t.dtype == torch.bfloat16:
        return SAS_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def make_dims(batch, n_q_heads, n_kv_heads, head_dim, sel_dim, top_k, t_max, dtype,
              block_size=BLOCK) -> SasDims:
    return SasDims(batch, n_q_heads, n_kv_heads, head_dim, sel_dim, block_size, top_k, t_max,
                   dtype)


def sas_workspace_bytes(op: int, dims: SasDims, q_len: int = 0) -> int:
    n = load_library().sas_workspace_bytes(op, ctypes.byref(dims), q_len)
    if n == SIZE_MAX:
        _check(SAS_ERR_INVALID_ARGUMENT)
    return n


def _workspace(op, dims, q_len, ws, device):
    need = sas_workspace_bytes(op, dims, q_len)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


# --------------------------------------------------------------------------
def sas_block_summaries(K, seq_lens, Wk_sel, blk_begin=0, blk_end=None, summ=None):
    """summ[b,r,m,:] = Wk_sel . mean(K[b,r,64m:64m+64,:]) for complete history blocks.

    K [B,Hkv,t_max,d]; seq_lens int32 [B]; Wk_sel fp32 [d_sel,d].  Returns summ
    fp32 [B,Hkv,t_max//64,d_sel] (zeros where not written when allocated here)."""
    B, Hkv, t_max, d = K.shape
    ds = Wk_sel.shape[0]
    dims = make_dims(B, Hkv, Hkv, d, ds, 0, t_max, _dtype_code(K))
    if summ is None:
        summ = torch.zeros(B, Hkv, t_max // BLOCK, ds, dtype=torch.float32, device=K.device)
    if blk_end is None:
        blk_end = t_max // BLOCK
    _check(load_library().sas_block_summaries(ctypes.byref(dims), _ptr(K), _ptr(seq_lens),
                                              _ptr(Wk_sel), blk_begin, blk_end, _ptr(summ),
                                              _stream()))
    return summ


def sas_select(mode, Q, seq_lens, Wq_sel, summ, top_k, t_max=None, q_len=None,
               idx=None, log_gate=None, score_lse=None, scores=None, want_scores=False,
               ws=None):
    """Selector scores, gate and Top-K.  Returns (idx, log_gate, score_lse, scores|None).

    mode SAS_SELECT_DECODE: Q is q [B,Hq,d]; SAS_SELECT_TILES and
    SAS_SELECT_QUERIES: Q is [B,Hq,S,d] (rows: ceil(S/64) tiles, or S queries).
    t_max: K/V row capacity (default: the largest one whose summary buffer has
    summ.shape[2] rows, so no sequence length that fits the buffer is clipped)."""
    B, Hkv, c_max, ds = summ.shape
    if t_max is None:
        t_max = c_max * BLOCK + BLOCK - 1
    Hq, d = Q.shape[1], Q.shape[-1]
    if mode == SAS_SELECT_TILES:
        q_len = Q.shape[2] if q_len is None else q_len
        rows = -(-q_len // BLOCK)
    elif mode == SAS_SELECT_QUERIES:
        q_len = Q.shape[2] if q_len is None else q_len
        rows = q_len
    else:
        q_len, rows = 0, 1
    dims = make_dims(B, Hq, Hkv, d, ds, top_k, t_max, _dtype_code(Q))
    dev = Q.device
    if idx is None:
        idx = torch.empty(B, Hkv, rows, top_k, dtype=torch.int32, device=dev)
    if log_gate is None:
        log_gate = torch.empty(B, Hkv, rows, top_k, dtype=torch.float32, device=dev)
    if score_lse is None:
        score_lse = torch.empty(B, Hkv, rows, dtype=torch.float32, device=dev)
    if want_scores and scores is None:
        scores = torch.full((B, Hkv, rows, c_max), float("nan"), dtype=torch.float32, device=dev)
    op = {SAS_SELECT_TILES: SAS_OP_SELECT_TILES,
          SAS_SELECT_QUERIES: SAS_OP_SELECT_QUERIES}.get(mode, SAS_OP_SELECT_DECODE)
    ws, ws_bytes = _workspace(op, dims, q_len, ws, dev)
    _check(load_library().sas_select(ctypes.byref(dims), mode, _ptr(Q), q_len, _ptr(seq_lens),
                                     _ptr(Wq_sel), _ptr(summ), _ptr(idx), _ptr(log_gate),
                                     _ptr(score_lse), _ptr(scores), _ptr(ws), ws_bytes,
                                     _stream()))
    return idx, log_gate, score_lse, scores


def sas_decode_fwd(q, K, V, seq_lens, idx, log_gate, scale=None, o=None, lse=None, ws=None,
                   want_lse=True):
    """Gated sparse decode attention.  q [B,Hq,d]; K,V [B,Hkv,t_max,d]; idx/log_gate
    [B,Hkv,1,k] (log_gate None = ungated).  Returns (o [B,Hq,d], lse [B,Hq] | None)."""
    B, Hq, d = q.shape
    _, Hkv, t_max, _ = K.shape
    k = idx.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, 64, k, t_max, _dtype_code(q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    ws, ws_bytes = _workspace(SAS_OP_DECODE_FWD, dims, 0, ws, q.device)
    _check(load_library().sas_decode_fwd(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V),
                                         _ptr(seq_lens), _ptr(idx), _ptr(log_gate), scale, _ptr(o),
                                         _ptr(lse), _ptr(ws), ws_bytes, _stream()))
    return o, lse


def sas_decode_step(q, K, V, seq_lens, Wq_sel, summ, top_k, gated=True, scale=None, idx=None,
                    log_gate=None, score_lse=None, o=None, lse=None, ws=None, want_lse=True,
                    Wk_sel=None):
    """Fused selection + gated sparse decode attention (the outputs of
    sas_select(SAS_SELECT_DECODE) followed by sas_decode_fwd).  q [B,Hq,d];
    K,V [B,Hkv,t_max,d]; summ [B,Hkv,t_max//64,d_sel].  With Wk_sel, the
    summary of each sequence's newest complete block is refreshed into summ
    first (as sas_block_summaries over that block).
    Returns (idx, log_gate, score_lse, o, lse | None)."""
    B, Hq, d = q.shape
    _, Hkv, t_max, _ = K.shape
    ds = summ.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, ds, top_k, t_max, _dtype_code(q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dev = q.device
    if idx is None:
        idx = torch.empty(B, Hkv, 1, top_k, dtype=torch.int32, device=dev)
    if log_gate is None:
        log_gate = torch.empty(B, Hkv, 1, top_k, dtype=torch.float32, device=dev)
    if score_lse is None:
        score_lse = torch.empty(B, Hkv, 1, dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(SAS_OP_DECODE_STEP, dims, 0, ws, dev)
    _check(load_library().sas_decode_step(ctypes.byref(dims), _ptr(q), _ptr(K), _ptr(V),
                                          _ptr(seq_lens), _ptr(Wq_sel), _ptr(Wk_sel), _ptr(summ),
                                          int(gated),
                                          scale, _ptr(idx), _ptr(log_gate), _ptr(score_lse),
                                          _ptr(o), _ptr(lse), _ptr(ws), ws_bytes, _stream()))
    return idx, log_gate, score_lse, o, lse


def sas_block_summaries_paged(K_pages, page_table, seq_lens, Wk_sel, t_max, blk_begin=0,
                              blk_end=None, summ=None):
    """sas_block_summaries on a paged cache: K_pages [n_pages,Hkv,64,d];
    page_table int32 [B,max_pages]; summaries [B,Hkv,t_max//64,d_sel]
    (logical blocks, allocated if None)."""
    _, Hkv, _, d = K_pages.shape
    B, max_pages = page_table.shape
    ds = Wk_sel.shape[0]
    c_max = t_max // BLOCK
    if summ is None:
        summ = torch.zeros(B, Hkv, c_max, ds, dtype=torch.float32, device=K_pages.device)
    blk_end = c_max if blk_end is None else blk_end
    dims = make_dims(B, Hkv, Hkv, d, ds, 0, t_max, _dtype_code(K_pages))
    _check(load_library().sas_block_summaries_paged(
        ctypes.byref(dims), _ptr(K_pages), _ptr(page_table), int(max_pages), _ptr(seq_lens),
        _ptr(Wk_sel), int(blk_begin), int(blk_end), _ptr(summ), _stream()))
    return summ


def sas_decode_step_paged(q, K_pages, V_pages, page_table, seq_lens, Wq_sel, summ, top_k,
                          t_max, Wk_sel=None, gated=True, scale=None, idx=None, log_gate=None,
                          score_lse=None, o=None, lse=None, ws=None):
    """sas_decode_step on a paged cache: q [B,Hq,d]; K_pages/V_pages
    [n_pages,Hkv,64,d]; page_table int32 [B,max_pages]; summ fp32
    [B,Hkv,t_max//64,d_sel] (logical blocks); t_max = logical capacity per
    sequence.  Returns (idx, log_gate, score_lse, o, lse)."""
    B, Hq, d = q.shape
    _, Hkv, _, _ = K_pages.shape
    ds = summ.shape[-1]
    max_pages = page_table.shape[1]
    dims = make_dims(B, Hq, Hkv, d, ds, top_k, t_max, _dtype_code(q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dev = q.device
    if idx is None:
        idx = torch.empty(B, Hkv, 1, top_k, dtype=torch.int32, device=dev)
    if log_gate is None:
        log_gate = torch.empty(B, Hkv, 1, top_k, dtype=torch.float32, device=dev)
    if score_lse is None:
        score_lse = torch.empty(B, Hkv, 1, dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(SAS_OP_DECODE_STEP, dims, 0, ws, dev)
    _check(load_library().sas_decode_step_paged(
        ctypes.byref(dims), _ptr(q), _ptr(K_pages), _ptr(V_pages), _ptr(page_table),
        int(max_pages), _ptr(seq_lens), _ptr(Wq_sel), _ptr(Wk_sel), _ptr(summ), int(gated),
        scale, _ptr(idx), _ptr(log_gate), _ptr(score_lse), _ptr(o), _ptr(lse), _ptr(ws),
        ws_bytes, _stream()))
    return idx, log_gate, score_lse, o, lse


def sas_prefill_fwd(Q, K, V, idx, log_gate, scale=None, seq_len=None, O=None, lse=None, ws=None):
    """Causal gated block-sparse prefill forward (bf16).  Q [B,Hq,S,d]; K,V
    [B,Hkv,t_max,d]; idx/log_gate [B,Hkv,ceil(S/64),k].  Returns (O, lse)."""
    B, Hq, S, d = Q.shape
    _, Hkv, t_max, _ = K.shape
    seq_len = S if seq_len is None else seq_len
    k = idx.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, 64, k, t_max, _dtype_code(Q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if O is None:
        O = torch.empty_like(Q)
    if lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=Q.device)
    ws, ws_bytes = _workspace(SAS_OP_PREFILL_FWD, dims, seq_len, ws, Q.device)
    _check(load_library().sas_prefill_fwd(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), seq_len,
                                          _ptr(idx), _ptr(log_gate), scale, _ptr(O), _ptr(lse),
                                          _ptr(ws), ws_bytes, _stream()))
    return O, lse


def sas_prefill_fwd_queries(Q, K, V, idx, log_gate, scale=None, seq_len=None, O=None,
                            lse=None, ws=None):
    """Causal prefill forward with one selection per query (bf16).  Q
    [B,Hq,S,d]; K,V [B,Hkv,t_max,d]; idx/log_gate [B,Hkv,S,k].  Returns (O, lse)."""
    B, Hq, S, d = Q.shape
    _, Hkv, t_max, _ = K.shape
    seq_len = S if seq_len is None else seq_len
    k = idx.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, 64, k, t_max, _dtype_code(Q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if O is None:
        O = torch.empty_like(Q)
    if lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=Q.device)
    ws, ws_bytes = _workspace(SAS_OP_PREFILL_FWD_QUERIES, dims, seq_len, ws, Q.device)
    _check(load_library().sas_prefill_fwd_queries(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V),
                                                  seq_len, _ptr(idx), _ptr(log_gate), scale,
                                                  _ptr(O), _ptr(lse), _ptr(ws), ws_bytes,
                                                  _stream()))
    return O, lse


def sas_bwd(Q, K, V, O, dO, lse, idx, log_gate, scale=None, seq_len=None, dQ=None, dK=None,
            dV=None, dlog_gate=None, ws=None):
    """Backward of sas_prefill_fwd.  Returns (dQ, dK, dV, dlog_gate)."""
    B, Hq, S, d = Q.shape
    _, Hkv, t_max, _ = K.shape
    seq_len = S if seq_len is None else seq_len
    k = idx.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, 64, k, t_max, _dtype_code(Q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.zeros_like(K) if dK is None else dK
    dV = torch.zeros_like(V) if dV is None else dV
    if dlog_gate is None:
        dlog_gate = torch.empty(idx.shape, dtype=torch.float32, device=Q.device)
    ws, ws_bytes = _workspace(SAS_OP_BWD, dims, seq_len, ws, Q.device)
    _check(load_library().sas_bwd(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                  _ptr(lse), seq_len, _ptr(idx), _ptr(log_gate), scale, _ptr(dQ),
                                  _ptr(dK), _ptr(dV), _ptr(dlog_gate), _ptr(ws), ws_bytes,
                                  _stream()))
    return dQ, dK, dV, dlog_gate


def sas_bwd_queries(Q, K, V, O, dO, lse, idx, log_gate, scale=None, seq_len=None, dQ=None,
                    dK=None, dV=None, dlog_gate=None, ws=None):
    """Backward of sas_prefill_fwd_queries (idx/log_gate [B,Hkv,S,k]).
    Returns (dQ, dK, dV, dlog_gate [B,Hkv,S,k])."""
    B, Hq, S, d = Q.shape
    _, Hkv, t_max, _ = K.shape
    seq_len = S if seq_len is None else seq_len
    k = idx.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, 64, k, t_max, _dtype_code(Q))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dQ = torch.empty_like(Q) if dQ is None else dQ
    dK = torch.zeros_like(K) if dK is None else dK
    dV = torch.zeros_like(V) if dV is None else dV
    if dlog_gate is None:
        dlog_gate = torch.empty(idx.shape, dtype=torch.float32, device=Q.device)
    ws, ws_bytes = _workspace(SAS_OP_BWD_QUERIES, dims, seq_len, ws, Q.device)
    _check(load_library().sas_bwd_queries(ctypes.byref(dims), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                          _ptr(dO), _ptr(lse), seq_len, _ptr(idx),
                                          _ptr(log_gate), scale, _ptr(dQ), _ptr(dK), _ptr(dV),
                                          _ptr(dlog_gate), _ptr(ws), ws_bytes, _stream()))
    return dQ, dK, dV, dlog_gate


def sas_selector_bwd(Q, K, Wq_sel, summ, idx, score_lse, dlog_gate, q_len=None, t_max=None,
                     ds=None, want_ds=False, dWq=None, dWk=None, ws=None):
    """Selector weight gradients for the tile rows of a prefill.  Q [B,Hq,S,d];
    K [B,Hkv,t_max,d]; summ [B,Hkv,t_max//64,d_sel]; idx/dlog_gate [B,Hkv,rows,k];
    score_lse [B,Hkv,rows].  Returns (dWq_sel, dWk_sel, ds | None)."""
    B, Hq, S, d = Q.shape
    _, Hkv, tm, _ = K.shape
    t_max = tm if t_max is None else t_max
    q_len = S if q_len is None else q_len
    ds_dim = Wq_sel.shape[0]
    k = idx.shape[-1]
    rows = -(-q_len // BLOCK)
    dims = make_dims(B, Hq, Hkv, d, ds_dim, k, t_max, _dtype_code(Q))
    dev = Q.device
    if want_ds and ds is None:
        ds = torch.full((B, Hkv, rows, t_max // BLOCK), float("nan"), dtype=torch.float32,
                        device=dev)
    if dWq is None:
        dWq = torch.empty_like(Wq_sel)
    if dWk is None:
        dWk = torch.empty_like(Wq_sel)
    ws, ws_bytes = _workspace(SAS_OP_SELECTOR_BWD, dims, q_len, ws, dev)
    _check(load_library().sas_selector_bwd(ctypes.byref(dims), _ptr(Q), q_len, _ptr(K),
                                           _ptr(Wq_sel), _ptr(summ), _ptr(idx), _ptr(score_lse),
                                           _ptr(dlog_gate), _ptr(ds), _ptr(dWq), _ptr(dWk),
                                           _ptr(ws), ws_bytes, _stream()))
    return dWq, dWk, ds


def sas_selector_bwd_queries(Q, K, Wq_sel, Wk_sel, summ, idx, score_lse, dlog_gate, q_len=None,
                             t_max=None, ds=None, want_ds=False, dWq=None, dWk=None, ws=None):
    """Selector weight gradients for per-query rows.  Q [B,Hq,S,d]; K
    [B,Hkv,t_max,d]; summ [B,Hkv,t_max//64,d_sel]; idx/dlog_gate [B,Hkv,S,k];
    score_lse [B,Hkv,S].  Returns (dWq_sel, dWk_sel, ds | None)."""
    B, Hq, S, d = Q.shape
    _, Hkv, tm, _ = K.shape
    t_max = tm if t_max is None else t_max
    q_len = S if q_len is None else q_len
    ds_dim = Wq_sel.shape[0]
    k = idx.shape[-1]
    dims = make_dims(B, Hq, Hkv, d, ds_dim, k, t_max, _dtype_code(Q))
    dev = Q.device
    if want_ds and ds is None:
        ds = torch.full((B, Hkv, q_len, t_max // BLOCK), float("nan"), dtype=torch.float32,
                        device=dev)
    if dWq is None:
        dWq = torch.empty_like(Wq_sel)
    if dWk is None:
        dWk = torch.empty_like(Wq_sel)
    ws, ws_bytes = _workspace(SAS_OP_SELECTOR_BWD_QUERIES, dims, q_len, ws, dev)
    _check(load_library().sas_selector_bwd_queries(
        ctypes.byref(dims), _ptr(Q), q_len, _ptr(K), _ptr(Wq_sel), _ptr(Wk_sel), _ptr(summ),
        _ptr(idx), _ptr(score_lse), _ptr(dlog_gate), _ptr(ds), _ptr(dWq), _ptr(dWk), _ptr(ws),
        ws_bytes, _stream()))
    return dWq, dWk, ds
