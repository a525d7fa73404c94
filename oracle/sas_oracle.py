"""Plain float64 CPU oracle for SAS (Simple Attention Sparsification).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP library
and its Python binding) never calls it, and this module imports nothing from
the product package.

What it computes, in the order the method states it
---------------------------------------------------
Sources are cited by page and section; the short names are:

* *SAS close reading* -- liuzhao09.github.io, "SAS：用最终预测损失学习有限注意力预算下的上下文排序"
  (sections 2.1-2.4: selection, gate, sparse scope, fused kernel).
* *SAS reproduction note* -- daiwk.github.io, "SAS：用语言模型损失端到端学习稀疏注意力排序"
  (section "核心公式", the attention formula with the 1/sqrt(d) scale).
* *SAS summary* -- hyper.ai, Chinese summary of paper 2609.13141 (section "方法").
* *MSA notes* -- papercache.org notes on MiniMax Sparse Attention (section 2.1 on
  GQA head grouping; section 4.1 on selecting Top-k on raw scores).

1. Blocks (SAS close reading, 2.1): a query at position ``T-1`` sees the current
   block ``B0 = [b*C, T)`` (always kept, causal, unit gate) and ``C = (T-1)//b``
   complete history blocks ``B_m = [b*m, b*m+b)``.  In prefill, the query tile
   ``t`` covers queries ``[b*t, b*t+b)``; its history is blocks ``m < t`` and its
   B0 is block ``t`` under the causal mask ``j <= i``.
2. Block summaries (SAS close reading, 2.1, block summary; pooled by the mean):
   ``summ_m = mean_{j in B_m} (Wk_sel @ k_j)`` per KV head.
3. Selector score per GQA group ``r`` (SAS summary, Method: ``s = R_theta(q, {K_Bm})``;
   MSA notes 2.1: adjacent query heads share a KV head, so head ``h`` is in group
   ``h // G``): ``s_m = mean_{h in r} (Wq_sel @ q_h) . summ_m / sqrt(d_sel)``.  In
   prefill the mean also runs over the tile's queries.
4. Gate (SAS close reading, 2.2, gate equation): ``g = softmax(s)`` over all C
   history blocks, ``log g_m = s_m - LSE(s)``, ``g_0 = 1``.
5. Selection (SAS close reading, 2.1): ``I = TopK(s, k)``; ``S = B0 U (U_{m in I} B_m)``.
   Top-K runs on the raw scores (MSA notes 4.1: softmax keeps the order); ties
   go to the lower block index; ``min(k, C)`` blocks are chosen and listed in
   ascending block order.
6. Attention (SAS reproduction note, core formula; SAS close reading 2.2):
   ``o = softmax(q K_S^T / sqrt(d) + log g_S) V_S`` with the log-gate broadcast to
   every token of a selected block and 0 on B0.  With ``gated=False`` the bias is
   0 everywhere (the inference rule of SAS close reading 2.1/2.3).
7. Backward (SAS close reading 2.4 and 2.2 eq. 5; SAS summary, Method): recompute
   ``p``; ``D = do . o``; ``dz = p * (do . v_j - D)``; ``dq = scale * dz K_S``;
   ``dk_j += scale * dz_j q``; ``dv_j += p_j do``; ``dlog g_m`` is the sum of ``dz``
   over the tokens of block ``m`` (all heads of the group, all queries of the
   tile).  B0 has no gate and gets no gradient; unselected blocks get none
   (sparse scope, SAS close reading 2.3).

8. Selector backward (SAS close reading 2.2, gate equation; 2.3, eq. 8, sparse
   scope; 2.4 and the training description after it: the selector's own
   parameters are what the loss trains): with ``dlog g`` of the selected
   slots from step 7 and the selection held fixed, ``log g = s - LSE(s)`` gives
   ``ds_m = dlog g_m [m in I] - g_m * sum_{l in I} dlog g_l`` over all C
   history blocks (for ``m`` not in ``I`` this is eq. 8's sparse-scope term,
   since ``dlog g_l = g_l dL/dg_l``), and the score definition of step 3
   carries ``ds`` to ``Wq_sel`` and ``Wk_sel``.  The selector's own chain into
   the backbone's Q and K is not formed: the backbone is held fixed while the
   selector trains.
9. Per-query selection (a next row; SAS close reading 2.4: the training
   kernel masks unselected blocks by each query's own gate threshold): query
   i of a prefill has its own scores over its C_i = i // b history blocks
   (step 3 with the query alone), its own gate and Top-K, and attends like a
   decode query at position i.  Its backward is step 7 on the query's own
   token set, with one log-gate gradient per (query, slot).

Every stage is its own function so a test can feed one stage's inputs
independently of the others.  All arithmetic is float64 NumPy; loops are kept
per block / per head so the code reads like the definitions above.
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import numpy as np

BLOCK = 64
NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# 1. Blocks
# --------------------------------------------------------------------------
def n_history_blocks(T: int, b: int = BLOCK) -> int:
    """Complete history blocks before the block holding position T-1."""
    return (int(T) - 1) // b


def current_block(T: int, b: int = BLOCK) -> Tuple[int, int]:
    """[start, end) of B0 for a query at position T-1."""
    C = n_history_blocks(T, b)
    return b * C, int(T)


# --------------------------------------------------------------------------
# 2. Block summaries
# --------------------------------------------------------------------------
def block_summaries(K: np.ndarray, T: int, Wk_sel: np.ndarray, b: int = BLOCK) -> np.ndarray:
    """Summaries of the complete history blocks of one sequence.

    K: [Hkv, >=T, d] float64; Wk_sel: [d_sel, d].  Returns [Hkv, C, d_sel]:
    every key is projected by Wk_sel, then the projections of a block are
    averaged (the wording of the tiny fp32 workload: mean_pool(Wk_sel K)).
    """
    C = n_history_blocks(T, b)
    Hkv = K.shape[0]
    out = np.zeros((Hkv, C, Wk_sel.shape[0]))
    for r in range(Hkv):
        proj = K[r, :C * b] @ Wk_sel.T
        for m in range(C):
            out[r, m] = proj[m * b:(m + 1) * b].mean(axis=0)
    return out


# --------------------------------------------------------------------------
# 3. Selector scores
# --------------------------------------------------------------------------
def decode_scores(q: np.ndarray, Wq_sel: np.ndarray, summ: np.ndarray, G: int) -> np.ndarray:
    """Per-group scores for one decode query.  q: [Hq, d]; summ: [Hkv, C, d_sel].

    Returns [Hkv, C]: mean over the group's heads of (Wq_sel q_h) . summ_m / sqrt(d_sel).
    """
    d_sel = Wq_sel.shape[0]
    Hkv, C, _ = summ.shape
    s = np.zeros((Hkv, C))
    for r in range(Hkv):
        acc = np.zeros(C)
        for h in range(r * G, (r + 1) * G):
            acc += summ[r] @ (Wq_sel @ q[h])
        s[r] = acc / G / math.sqrt(d_sel)
    return s


def tile_scores(Q: np.ndarray, S: int, Wq_sel: np.ndarray, summ: np.ndarray, G: int,
                b: int = BLOCK, tiles=None) -> List[np.ndarray]:
    """Per-tile, per-group scores in prefill.  Q: [Hq, >=S, d]; summ: [Hkv, >=n_tiles-1, d_sel].

    Returns a list over tiles t of arrays [Hkv, t]: the score of history block
    m < t is the mean over the group's heads and the tile's queries of
    (Wq_sel q_{h,i}) . summ_m / sqrt(d_sel).  With ``tiles`` only those tiles
    are computed (the others are None).
    """
    d_sel = Wq_sel.shape[0]
    Hkv = summ.shape[0]
    n_tiles = -(-S // b)
    out = []
    for t in range(n_tiles):
        if tiles is not None and t not in tiles:
            out.append(None)
            continue
        i0, i1 = b * t, min(b * t + b, S)
        s = np.zeros((Hkv, t))
        for r in range(Hkv):
            acc = np.zeros(t)
            n = 0
            for h in range(r * G, (r + 1) * G):
                for i in range(i0, i1):
                    acc += summ[r, :t] @ (Wq_sel @ Q[h, i])
                    n += 1
            s[r] = acc / n / math.sqrt(d_sel)
        out.append(s)
    return out


# --------------------------------------------------------------------------
# 4. Gate
# --------------------------------------------------------------------------
def gate(s: np.ndarray) -> Tuple[float, np.ndarray]:
    """LSE(s) and log g = s - LSE(s) over all history blocks of one row."""
    if s.size == 0:
        return NEG_INF, np.zeros(0)
    mx = float(np.max(s))
    lse = mx + math.log(float(np.sum(np.exp(s - mx))))
    return lse, s - lse


# --------------------------------------------------------------------------
# 5. Top-K
# --------------------------------------------------------------------------
def topk(s: np.ndarray, k: int) -> Tuple[List[int], float]:
    """The min(k, C) highest-scoring blocks (ties -> lower index), ascending.

    Also returns the gap between the k-th and (k+1)-th largest scores
    (+inf when nothing is left out or k == 0).
    """
    C = int(s.size)
    kk = max(0, min(int(k), C))
    order = sorted(range(C), key=lambda m: (-float(s[m]), m))
    chosen = sorted(order[:kk])
    if kk >= 1 and C > kk:
        gap = float(s[order[kk - 1]] - s[order[kk]])
    else:
        gap = float("inf")
    return chosen, gap


def select_rows(score_rows: List[np.ndarray], k: int):
    """Gate + Top-K for a list of score rows.  Returns (idx, log_gate, lse, gap),
    idx int64 [rows, k] padded with -1, log_gate [rows, k] padded with -inf."""
    n = len(score_rows)
    idx = np.full((n, k), -1, dtype=np.int64)
    lg = np.full((n, k), NEG_INF)
    lse = np.full(n, NEG_INF)
    gap = np.full(n, np.inf)
    for row, s in enumerate(score_rows):
        lse_r, logg = gate(s)
        chosen, gp = topk(s, k)
        lse[row] = lse_r
        gap[row] = gp
        for slot, m in enumerate(chosen):
            idx[row, slot] = m
            lg[row, slot] = logg[m]
    return idx, lg, lse, gap


# --------------------------------------------------------------------------
# 6. Attention
# --------------------------------------------------------------------------
def _selected_tokens(idx_row, lg_row, b, gated):
    toks, bias = [], []
    for m, lgm in zip(idx_row, lg_row):
        if m < 0:
            continue
        toks.extend(range(b * int(m), b * int(m) + b))
        bias.extend([float(lgm) if gated else 0.0] * b)
    return toks, bias


def decode_attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, T: int, idx: np.ndarray,
                  log_gate: np.ndarray, scale: float, G: int, b: int = BLOCK,
                  gated: bool = True):
    """One decode step of one sequence.

    q: [Hq, d]; K, V: [Hkv, >=T, d]; idx, log_gate: [Hkv, k].
    Returns o [Hq, d] and lse [Hq] (natural log of the softmax normaliser).
    """
    Hq, d = q.shape
    o = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    b0, b1 = current_block(T, b)
    for h in range(Hq):
        r = h // G
        toks, bias = _selected_tokens(idx[r], log_gate[r], b, gated)
        toks = list(range(b0, b1)) + toks
        bias = [0.0] * (b1 - b0) + bias
        z = K[r, toks] @ q[h] * scale + np.asarray(bias)
        mx = z.max()
        e = np.exp(z - mx)
        l = e.sum()
        o[h] = (e / l) @ V[r, toks]
        lse[h] = mx + math.log(l)
    return o, lse


def _tile_logits(Qt, K, r, t, S, idx_row, lg_row, scale, b, gated):
    """Logits of the queries of tile t against the tile's token set.

    Returns (Z [nq, ntok], token list, per-token slot (-1 for the diagonal block))."""
    i0, i1 = b * t, min(b * t + b, S)
    toks, bias = _selected_tokens(idx_row, lg_row, b, gated)
    slots = []
    for slot, m in enumerate(idx_row):
        if m >= 0:
            slots.extend([slot] * b)
    diag = list(range(i0, i1))
    all_toks = toks + diag
    slots = slots + [-1] * len(diag)
    Z = Qt @ K[r, all_toks].T * scale + np.asarray(bias + [0.0] * len(diag))[None, :]
    nsel = len(toks)
    for qi in range(i1 - i0):
        for dj in range(len(diag)):
            if dj > qi:                      # causal mask inside the diagonal block
                Z[qi, nsel + dj] = NEG_INF
    return Z, all_toks, np.asarray(slots)


def prefill_attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, S: int, idx: np.ndarray,
                   log_gate: np.ndarray, scale: float, G: int, b: int = BLOCK,
                   gated: bool = True, tiles=None):
    """Causal gated block-sparse attention of one sequence, one selection per tile.

    Q: [Hq, >=S, d]; K, V: [Hkv, >=S, d]; idx, log_gate: [Hkv, n_tiles, k].
    Returns O [Hq, S, d] and lse [Hq, S] (with ``tiles``, only the queries of
    those tiles are filled in).
    """
    Hq, _, d = Q.shape
    O = np.zeros((Hq, S, d))
    lse = np.zeros((Hq, S))
    n_tiles = -(-S // b)
    for t in (range(n_tiles) if tiles is None else tiles):
        i0, i1 = b * t, min(b * t + b, S)
        for h in range(Hq):
            r = h // G
            Z, toks, _ = _tile_logits(Q[h, i0:i1], K, r, t, S, idx[r, t], log_gate[r, t],
                                      scale, b, gated)
            mx = Z.max(axis=1, keepdims=True)
            E = np.exp(Z - mx)
            L = E.sum(axis=1, keepdims=True)
            O[h, i0:i1] = (E / L) @ V[r, toks]
            lse[h, i0:i1] = (mx + np.log(L))[:, 0]
    return O, lse


# --------------------------------------------------------------------------
# 7. Backward
# --------------------------------------------------------------------------
def prefill_backward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray, S: int,
                     idx: np.ndarray, log_gate: np.ndarray, scale: float, G: int,
                     b: int = BLOCK, tiles=None):
    """Gradients of L = <dO, O> for prefill_attend (gated).

    Returns dQ [Hq,S,d], dK [Hkv,S,d], dV [Hkv,S,d], dlog_gate [Hkv, n_tiles, k]
    (zero on empty slots).  The log-gate is treated as an independent input.
    With ``tiles``, only the terms of those query tiles are accumulated (so
    dQ/dlog_gate are exact on those tiles and dK/dV hold their contribution).
    """
    Hq, _, d = Q.shape
    Hkv = K.shape[0]
    n_tiles = -(-S // b)
    k = idx.shape[2]
    dQ = np.zeros((Hq, S, d))
    dK = np.zeros((Hkv, S, d))
    dV = np.zeros((Hkv, S, d))
    dlg = np.zeros((Hkv, n_tiles, k))
    for t in (range(n_tiles) if tiles is None else tiles):
        i0, i1 = b * t, min(b * t + b, S)
        for h in range(Hq):
            r = h // G
            Qt = Q[h, i0:i1]
            Z, toks, slots = _tile_logits(Qt, K, r, t, S, idx[r, t], log_gate[r, t],
                                          scale, b, True)
            mx = Z.max(axis=1, keepdims=True)
            E = np.exp(Z - mx)
            P = E / E.sum(axis=1, keepdims=True)
            Vs = V[r, toks]
            Ot = P @ Vs
            dOt = dO[h, i0:i1]
            D = np.sum(dOt * Ot, axis=1, keepdims=True)
            dP = dOt @ Vs.T
            dZ = P * (dP - D)
            dQ[h, i0:i1] += scale * dZ @ K[r, toks]
            np.add.at(dK[r], toks, scale * dZ.T @ Qt)
            np.add.at(dV[r], toks, P.T @ dOt)
            colsum = dZ.sum(axis=0)
            for slot in range(k):
                sel = slots == slot
                if np.any(sel):
                    dlg[r, t, slot] += colsum[sel].sum()
    return dQ, dK, dV, dlg


# --------------------------------------------------------------------------
# 8. Selector backward
# --------------------------------------------------------------------------
def score_grad(s: np.ndarray, idx_row: np.ndarray, dlg_row: np.ndarray) -> np.ndarray:
    """dL/ds for one row from the log-gate gradients of its selected slots.

    log g_m = s_m - LSE(s), so d(log g_l)/d(s_m) = [l == m] - g_m and
    dL/ds_m = sum over selected l of dlog g_l ([l == m] - g_m).
    """
    if s.size == 0:
        return np.zeros(0)
    _, logg = gate(s)
    g = np.exp(logg)
    total = 0.0
    ds = np.zeros(s.size)
    for m, dl in zip(idx_row, dlg_row):
        if m >= 0:
            ds[m] += dl
            total += dl
    return ds - g * total


def selector_backward(Q: np.ndarray, K: np.ndarray, S: int, Wq_sel: np.ndarray,
                      Wk_sel: np.ndarray, idx: np.ndarray, dlog_gate: np.ndarray, G: int,
                      b: int = BLOCK):
    """Gradients of the loss with respect to the selector weights (prefill tiles).

    Q: [Hq,>=S,d], K: [Hkv,>=S,d]; idx/dlog_gate [Hkv, n_tiles, k] (the
    selection is held fixed).  Returns (ds rows: list over tiles of [Hkv, t],
    dWq_sel [d_sel,d], dWk_sel [d_sel,d]).

    The score of tile t and block m is s = mean_{h,i} (Wq_sel q_{h,i}) . summ_m
    / sqrt(d_sel) with summ_m = mean_{j in B_m} Wk_sel k_j, so
      ds/dWq_sel = summ_m qbar^T / sqrt(d_sel),  qbar = mean_{h,i} q_{h,i},
      ds/dWk_sel = (Wq_sel qbar / sqrt(d_sel)) kbar_m^T,  kbar_m = mean_{j in B_m} k_j.
    """
    d_sel, d = Wq_sel.shape
    Hkv = K.shape[0]
    n_tiles = -(-S // b)
    summ = block_summaries(K, S, Wk_sel, b)
    rows = tile_scores(Q, S, Wq_sel, summ, G, b)
    dWq = np.zeros((d_sel, d))
    dWk = np.zeros((d_sel, d))
    ds_rows = []
    for t in range(n_tiles):
        i0, i1 = b * t, min(b * t + b, S)
        ds_t = np.zeros((Hkv, t))
        for r in range(Hkv):
            ds = score_grad(rows[t][r], idx[r, t], dlog_gate[r, t])
            ds_t[r] = ds
            qbar = Q[r * G:(r + 1) * G, i0:i1].reshape(-1, d).mean(axis=0)
            u = Wq_sel @ qbar / math.sqrt(d_sel)
            for m in range(t):
                kbar = K[r, b * m:b * m + b].mean(axis=0)
                dWq += ds[m] * np.outer(summ[r, m], qbar) / math.sqrt(d_sel)
                dWk += ds[m] * np.outer(u, kbar)
        ds_rows.append(ds_t)
    return ds_rows, dWq, dWk


# --------------------------------------------------------------------------
# Whole-problem drivers (batch loops over the stages above)
# --------------------------------------------------------------------------
def decode_step(q, K, V, seq_lens, Wq_sel, Wk_sel, k, scale=None, G=None, b=BLOCK,
                gated=True, want_scores=False):
    """Summaries -> scores -> gate -> Top-K -> attention for a batch of decode queries.

    q: [B,Hq,d]; K,V: [B,Hkv,t_max,d] (float64).  Returns a dict with idx/log_gate
    [B,Hkv,k], score_lse [B,Hkv], gap [B,Hkv], o [B,Hq,d], lse [B,Hq] and
    optionally the score rows.
    """
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = G or Hq // Hkv
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    out = {"idx": np.full((B, Hkv, k), -1, np.int64), "log_gate": np.full((B, Hkv, k), NEG_INF),
           "score_lse": np.zeros((B, Hkv)), "gap": np.zeros((B, Hkv)),
           "o": np.zeros((B, Hq, d)), "lse": np.zeros((B, Hq)), "scores": [], "summ": []}
    for bi in range(B):
        T = int(seq_lens[bi])
        summ = block_summaries(K[bi], T, Wk_sel, b)
        s = decode_scores(q[bi], Wq_sel, summ, G)
        idx, lg, lse_s, gap = select_rows([s[r] for r in range(Hkv)], k)
        out["idx"][bi], out["log_gate"][bi] = idx, lg
        out["score_lse"][bi], out["gap"][bi] = lse_s, gap
        o, lse = decode_attend(q[bi], K[bi], V[bi], T, idx, lg, scale, G, b, gated)
        out["o"][bi], out["lse"][bi] = o, lse
        if want_scores:
            out["scores"].append(s)
            out["summ"].append(summ)
    return out


def prefill_select(Q, K, S, Wq_sel, Wk_sel, k, G, b=BLOCK):
    """Summaries -> per-tile scores -> gate -> Top-K for one sequence.

    Q: [Hq,>=S,d], K: [Hkv,>=S,d].  Returns idx/log_gate [Hkv,n_tiles,k],
    score_lse/gap [Hkv,n_tiles] and the per-tile score rows.
    """
    Hkv = K.shape[0]
    n_tiles = -(-S // b)
    summ = block_summaries(K, S, Wk_sel, b)
    rows = tile_scores(Q, S, Wq_sel, summ, G, b)
    idx = np.full((Hkv, n_tiles, k), -1, np.int64)
    lg = np.full((Hkv, n_tiles, k), NEG_INF)
    lse = np.zeros((Hkv, n_tiles))
    gap = np.zeros((Hkv, n_tiles))
    for r in range(Hkv):
        i_r, lg_r, lse_r, gap_r = select_rows([rows[t][r] for t in range(n_tiles)], k)
        idx[r], lg[r], lse[r], gap[r] = i_r, lg_r, lse_r, gap_r
    return {"idx": idx, "log_gate": lg, "score_lse": lse, "gap": gap, "scores": rows,
            "summ": summ}


# --------------------------------------------------------------------------
# 9. Per-query selection in prefill (a next row: oracle only, no kernel yet)
# --------------------------------------------------------------------------
def query_scores(Q, S, Wq_sel, summ, G, b=BLOCK, queries=None):
    """Per-query, per-group scores for a prefill with one selection per query
    (SAS close reading 2.4: the training kernel masks the unselected blocks by
    each query's own gate threshold).  Query i has the C_i = i // b complete
    blocks before its own block as history, and its score of block m is step 3
    with the query alone in place of a tile: the mean over its group's heads
    of (Wq_sel q_{h,i}) . summ_m / sqrt(d_sel), i.e. the decode score of a
    query at position i.  Q: [Hq, >=S, d]; summ: [Hkv, >=C, d_sel].
    Returns {i: array [Hkv, C_i]} for the queries asked for (all by default).
    """
    out = {}
    for i in (range(S) if queries is None else queries):
        C = i // b
        out[i] = decode_scores(Q[:, i], Wq_sel, summ[:, :C], G)
    return out


def query_select(Q, K, S, Wq_sel, Wk_sel, k, G, b=BLOCK, queries=None):
    """Summaries -> per-query scores -> gate -> Top-K for one sequence (the
    threshold of query i is its k-th largest score, ties to the lower block).

    Returns idx/log_gate [Hkv, S, k] (-1 / -inf padded), score_lse and gap
    [Hkv, S]; with ``queries`` only those rows are filled in."""
    Hkv = K.shape[0]
    summ = block_summaries(K, S, Wk_sel, b)
    rows = query_scores(Q, S, Wq_sel, summ, G, b, queries)
    idx = np.full((Hkv, S, k), -1, np.int64)
    lg = np.full((Hkv, S, k), NEG_INF)
    lse = np.zeros((Hkv, S))
    gap = np.zeros((Hkv, S))
    for i, s in rows.items():
        i_r, lg_r, lse_r, gap_r = select_rows([s[r] for r in range(Hkv)], k)
        idx[:, i], lg[:, i], lse[:, i], gap[:, i] = i_r, lg_r, lse_r, gap_r
    return {"idx": idx, "log_gate": lg, "score_lse": lse, "gap": gap, "scores": rows,
            "summ": summ}


def query_attend(Q, K, V, S, idx, log_gate, scale, G, b=BLOCK, gated=True, queries=None):
    """Causal gated block-sparse attention with one selection per query: query
    i attends to the blocks idx[r, i] (bias log g) and to tokens b*(i//b)..i of
    its own block (bias 0) -- a decode step at T = i + 1.

    Q: [Hq, >=S, d]; K, V: [Hkv, >=S, d]; idx, log_gate: [Hkv, S, k].
    Returns O [Hq, S, d] and lse [Hq, S] (only the requested queries)."""
    Hq, _, d = Q.shape
    O = np.zeros((Hq, S, d))
    lse = np.zeros((Hq, S))
    for i in (range(S) if queries is None else queries):
        o, l = decode_attend(Q[:, i], K, V, i + 1, idx[:, i], log_gate[:, i], scale, G, b, gated)
        O[:, i], lse[:, i] = o, l
    return O, lse


def _query_tokens(i, idx_row, lg_row, b):
    """Token set of query i under per-query selection: its own block up to i
    (bias 0, slot -1), then the tokens of its selected blocks (bias log g,
    the block's slot)."""
    j0 = b * (i // b)
    toks = list(range(j0, i + 1))
    bias = [0.0] * len(toks)
    slots = [-1] * len(toks)
    for slot, (m, lgm) in enumerate(zip(idx_row, lg_row)):
        if m >= 0:
            toks.extend(range(b * int(m), b * int(m) + b))
            bias.extend([float(lgm)] * b)
            slots.extend([slot] * b)
    return toks, np.asarray(bias), np.asarray(slots)


def _slot_sums(dz, slots, k):
    """Sum of the logit gradients over the tokens of each selected slot (the
    query's own block, slot -1, has no gate)."""
    out = np.zeros(k)
    for slot in range(k):
        out[slot] = dz[slots == slot].sum()
    return out


def query_backward(Q, K, V, dO, S, idx, log_gate, scale, G, b=BLOCK, queries=None):
    """Gradients of L = <dO, O> for query_attend (gated): step 7 on each
    query's own token set.  With p the softmax row of query i and head h,
    D = do . o, dz = p (do . v_j - D), dq = scale dz K_S, dk_j += scale dz_j q,
    dv_j += p_j do, and the log-gate gradient of query i's slot is the sum of
    dz over that block's tokens and the group's heads (the gates are per
    query, so the sum runs over one query only).

    Q, dO: [Hq, >=S, d]; K, V: [Hkv, >=S, d]; idx, log_gate: [Hkv, S, k].
    Returns dQ [Hq,S,d], dK [Hkv,S,d], dV [Hkv,S,d], dlog_gate [Hkv,S,k]
    (zero on empty slots).  With ``queries``, only the terms of those queries
    are accumulated."""
    Hq, _, d = Q.shape
    Hkv = K.shape[0]
    k = idx.shape[2]
    dQ = np.zeros((Hq, S, d))
    dK = np.zeros((Hkv, S, d))
    dV = np.zeros((Hkv, S, d))
    dlg = np.zeros((Hkv, S, k))
    for i in (range(S) if queries is None else queries):
        for h in range(Hq):
            r = h // G
            toks, bias, slots = _query_tokens(i, idx[r, i], log_gate[r, i], b)
            Ks, Vs = K[r, toks], V[r, toks]
            z = Ks @ Q[h, i] * scale + bias
            e = np.exp(z - z.max())
            p = e / e.sum()
            o = p @ Vs
            D = float(dO[h, i] @ o)
            dz = p * (Vs @ dO[h, i] - D)
            dQ[h, i] += scale * dz @ Ks
            np.add.at(dK[r], toks, scale * np.outer(dz, Q[h, i]))
            np.add.at(dV[r], toks, np.outer(p, dO[h, i]))
            dlg[r, i] += _slot_sums(dz, slots, k)
    return dQ, dK, dV, dlg


def query_selector_backward(Q, K, S, Wq_sel, Wk_sel, idx, dlog_gate, G, b=BLOCK):
    """Step 8 for per-query rows: the selector weights' gradients from the
    per-query log-gate gradients (the selection held fixed).  Row (i, r) has
    the C_i = i // b blocks before query i's block, the score
    s_m = (Wq_sel qbar) . summ_m / sqrt(d_sel) with qbar the mean of query i
    over the group's heads, and ds = score_grad(s, idx, dlog_gate) over all
    C_i blocks; then, as for the tile rows,
      dWq_sel += ds_m summ_m qbar^T / sqrt(d_sel),
      dWk_sel += ds_m (Wq_sel qbar / sqrt(d_sel)) kbar_m^T.
    Q: [Hq,>=S,d], K: [Hkv,>=S,d]; idx/dlog_gate [Hkv, S, k].  Returns
    (ds rows: dict i -> [Hkv, C_i], dWq_sel [d_sel,d], dWk_sel [d_sel,d])."""
    d_sel, d = Wq_sel.shape
    Hkv = K.shape[0]
    summ = block_summaries(K, S, Wk_sel, b)
    rows = query_scores(Q, S, Wq_sel, summ, G, b)
    dWq = np.zeros((d_sel, d))
    dWk = np.zeros((d_sel, d))
    ds_rows = {}
    for i in range(S):
        C = i // b
        ds_i = np.zeros((Hkv, C))
        for r in range(Hkv):
            ds = score_grad(rows[i][r], idx[r, i], dlog_gate[r, i])
            ds_i[r] = ds
            qbar = Q[r * G:(r + 1) * G, i].mean(axis=0)
            u = Wq_sel @ qbar / math.sqrt(d_sel)
            for m in range(C):
                kbar = K[r, b * m:b * m + b].mean(axis=0)
                dWq += ds[m] * np.outer(summ[r, m], qbar) / math.sqrt(d_sel)
                dWk += ds[m] * np.outer(u, kbar)
        ds_rows[i] = ds_i
    return ds_rows, dWq, dWk


# --------------------------------------------------------------------------
# Second formulation for tiny inputs: dense logits with a block mask
# --------------------------------------------------------------------------
def dense_masked_decode(q, K, V, T, idx, log_gate, scale, G, b=BLOCK, gated=True):
    """Same result as decode_attend, computed over all T positions with a bias
    vector: log g (selected history block), 0 (B0), -inf (everything else)."""
    Hq, d = q.shape
    C = n_history_blocks(T, b)
    o = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        r = h // G
        bias = np.full(T, NEG_INF)
        bias[b * C:T] = 0.0
        for m, lgm in zip(idx[r], log_gate[r]):
            if m >= 0:
                bias[b * m:b * m + b] = lgm if gated else 0.0
        z = K[r, :T] @ q[h] * scale + bias
        w = np.exp(z - z.max())
        o[h] = w @ V[r, :T] / w.sum()
        lse[h] = z.max() + math.log(w.sum())
    return o, lse


def dense_masked_prefill(Q, K, V, S, idx, log_gate, scale, G, b=BLOCK, gated=True):
    """Same result as prefill_attend via a dense [S x S] bias matrix per group."""
    Hq, _, d = Q.shape
    Hkv = K.shape[0]
    O = np.zeros((Hq, S, d))
    lse = np.zeros((Hq, S))
    for r in range(Hkv):
        bias = np.full((S, S), NEG_INF)
        for i in range(S):
            t = i // b
            for m, lgm in zip(idx[r, t], log_gate[r, t]):
                if m >= 0:
                    bias[i, b * m:b * m + b] = lgm if gated else 0.0
            bias[i, b * t:i + 1] = 0.0
        for h in range(r * G, (r + 1) * G):
            Z = Q[h, :S] @ K[r, :S].T * scale + bias
            mx = Z.max(axis=1, keepdims=True)
            W = np.exp(Z - mx)
            O[h] = W @ V[r, :S] / W.sum(axis=1, keepdims=True)
            lse[h] = (mx + np.log(W.sum(axis=1, keepdims=True)))[:, 0]
    return O, lse
