"""Pins for the CPU oracle: each test checks it against something other than itself.

* hand-worked closed-form cases (tests/golden/hand_worked.json);
* Top-K against NumPy's lexsort and against exhaustive search over subsets;
* the gathered-token formulation against a dense masked one (tiny inputs);
* k = C with all gates equal, and k = 0, against torch's CPU
  scaled_dot_product_attention (library routine, float64);
* gate shift invariance and normalisation;
* the log-gate gradient, eq. 5's g-space gradient and dQ/dK/dV against central
  finite differences, plus exact identities of the backward;
* summaries and scores on inputs with closed-form answers, a planted-key
  recall check, and decode/prefill score consistency;
* the selector backward: dL/ds of the attention loss by central differences on
  the scores (eq. 8's sparse-scope term for unselected blocks, sum ds = 0), and
  dWq_sel / dWk_sel by central differences on the weights;
* per-query selection: dense causal attention with a per-query log-gate bias
  when k covers the history, local causal attention at k = 0, and the tile
  scores when the queries of each tile are equal;
* planted mistakes: each mutation of the oracle must make some pin fail.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from gated_block_sparse_amd import synth
from oracle import sas_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))


# --------------------------------------------------------------------------
# helpers (plain NumPy / torch library calls, no oracle arithmetic)
# --------------------------------------------------------------------------
def _rand_prefill(seed, Hq=4, Hkv=2, d=8, S=20):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Hq, S, d))
    K = rng.standard_normal((Hkv, S, d))
    V = rng.standard_normal((Hkv, S, d))
    dO = rng.standard_normal((Hq, S, d))
    return Q, K, V, dO


def _random_selection(rng, Hkv, n_tiles, k):
    idx = np.full((Hkv, n_tiles, k), -1, np.int64)
    lg = np.full((Hkv, n_tiles, k), -np.inf)
    for r in range(Hkv):
        for t in range(n_tiles):
            n = min(k, t)
            ch = np.sort(rng.choice(t, size=n, replace=False)) if n else []
            for s, m in enumerate(ch):
                idx[r, t, s] = m
                lg[r, t, s] = -abs(rng.standard_normal()) - 0.5
    return idx, lg


def _sdpa(q, k, v, mask, scale):
    """torch CPU SDPA in float64; q [H,L,d], k/v [H,S,d], mask [H or 1, L, S] additive."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(mask)[None], scale=scale)
    return out[0].numpy()


# --------------------------------------------------------------------------
# hand-worked cases
# --------------------------------------------------------------------------
def check_hand_worked():
    g = GOLDEN["gate"]
    lse, logg = O.gate(np.asarray(g["s"]))
    assert abs(lse - g["lse"]) < 1e-12
    np.testing.assert_allclose(logg, g["log_g"], atol=1e-12)
    for case in GOLDEN["decode"]:
        b, T = case["b"], case["T"]
        q = np.asarray(case["q"]).reshape(1, 1)
        K = np.asarray(case["K"]).reshape(1, T, 1)
        V = np.asarray(case["V"]).reshape(1, T, 1)
        idx, lg, _, _ = O.select_rows([np.asarray(case["s"])], case["k"])
        assert [int(m) for m in idx[0] if m >= 0] == case["idx"], case["name"]
        o, l = O.decode_attend(q, K, V, T, idx, lg, 1.0, 1, b=b, gated=case["gated"])
        assert abs(o[0, 0] - case["o"]) < 1e-12, case["name"]
        assert abs(l[0] - case["lse"]) < 1e-12, case["name"]
    pb = GOLDEN["prefill_backward"]
    b, S = pb["b"], pb["S"]
    Q = np.asarray(pb["Q"]).reshape(1, S, 1)
    K = np.asarray(pb["K"]).reshape(1, S, 1)
    V = np.asarray(pb["V"]).reshape(1, S, 1)
    dO = np.asarray(pb["dO"]).reshape(1, S, 1)
    idx = np.asarray(pb["idx"]).reshape(1, S, 2)
    lg = np.asarray([[np.nan if x is None else x for x in row] for row in pb["log_gate"]])
    lg = np.where(np.isnan(lg), -np.inf, lg).reshape(1, S, 2)
    Ot, _ = O.prefill_attend(Q, K, V, S, idx, lg, 1.0, 1, b=b)
    np.testing.assert_allclose(Ot[0, :, 0], pb["O"], atol=1e-12)
    _, _, _, dlg = O.prefill_backward(Q, K, V, dO, S, idx, lg, 1.0, 1, b=b)
    np.testing.assert_allclose(dlg[0], pb["dlog_gate"], atol=1e-12)


def test_hand_worked_cases():
    check_hand_worked()


# --------------------------------------------------------------------------
# Top-K
# --------------------------------------------------------------------------
def check_topk_lexsort(seed=0):
    rng = np.random.default_rng(seed)
    for trial in range(200):
        C = int(rng.integers(0, 300))
        k = int(rng.integers(0, 40))
        # coarse values make exact ties common
        s = np.round(rng.standard_normal(C) * 4) / 4 if trial % 2 else rng.standard_normal(C)
        chosen, gap = O.topk(s, k)
        ref = np.lexsort((np.arange(C), -s))[:min(k, C)]
        assert chosen == sorted(ref.tolist())
        if 0 < k < C:
            srt = np.sort(s)[::-1]
            assert gap == srt[k - 1] - srt[k]
        else:
            assert gap == math.inf


def test_topk_matches_lexsort():
    check_topk_lexsort()


def check_topk_exhaustive(seed=1):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        C = int(rng.integers(1, 11))
        k = int(rng.integers(0, C + 2))
        s = rng.integers(-3, 4, size=C).astype(np.float64)   # integer scores: exact sums, many ties
        kk = min(k, C)
        best = None
        for sub in itertools.combinations(range(C), kk):
            key = (-sum(s[list(sub)]), sub)                  # max sum, then lexicographically smallest
            if best is None or key < best:
                best = key
        chosen, _ = O.topk(s, k)
        assert tuple(chosen) == best[1]


def test_topk_exhaustive_small():
    check_topk_exhaustive()


def test_topk_on_scores_equals_topk_on_gate():
    rng = np.random.default_rng(2)
    for _ in range(50):
        s = rng.standard_normal(100) * 3
        _, logg = O.gate(s)
        g = np.exp(logg)
        assert O.topk(s, 16)[0] == sorted(np.argsort(-g, kind="stable")[:16].tolist())


# --------------------------------------------------------------------------
# two formulations agree (brute force on tiny inputs)
# --------------------------------------------------------------------------
def check_gather_vs_dense(seed=3):
    rng = np.random.default_rng(seed)
    for b in (4, 64):
        for T in (1, b - 1, b, b + 1, 3 * b + 5, 7 * b):
            Hq, Hkv, d = 4, 2, 8
            q = rng.standard_normal((Hq, d))
            K = rng.standard_normal((Hkv, T, d))
            V = rng.standard_normal((Hkv, T, d))
            C = O.n_history_blocks(T, b)
            for k in (0, 1, 3, C + 2):
                s = [rng.standard_normal(C) for _ in range(Hkv)]
                idx, lg, _, _ = O.select_rows(s, k)
                for gated in (True, False):
                    o1, l1 = O.decode_attend(q, K, V, T, idx, lg, 0.35, 2, b, gated)
                    o2, l2 = O.dense_masked_decode(q, K, V, T, idx, lg, 0.35, 2, b, gated)
                    np.testing.assert_allclose(o1, o2, atol=1e-12)
                    np.testing.assert_allclose(l1, l2, atol=1e-12)
    for b, S in ((4, 1), (4, 7), (4, 17), (4, 24), (8, 45)):
        Q, K, V, _ = _rand_prefill(seed + S, S=S)
        n_tiles = -(-S // b)
        for k in (0, 2, n_tiles):
            idx, lg = _random_selection(rng, 2, n_tiles, k)
            o1, l1 = O.prefill_attend(Q, K, V, S, idx, lg, 0.3, 2, b)
            o2, l2 = O.dense_masked_prefill(Q, K, V, S, idx, lg, 0.3, 2, b)
            np.testing.assert_allclose(o1, o2, atol=1e-12)
            np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_gather_equals_dense_masked():
    check_gather_vs_dense()


# --------------------------------------------------------------------------
# k = C with equal gates, and k = 0, against torch SDPA
# --------------------------------------------------------------------------
def _decode_problem(seed, T, b=64, k=None, zero_wq=False, Hq=4, Hkv=2, d=16):
    wl = synth.custom_workload("decode", n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, sel_dim=d,
                               top_k=k if k is not None else 4, seq_len=T)
    return synth.make_problem(wl, seed, zero_wq=zero_wq)


def check_uniform_gate_is_dense_with_bias(seed=4):
    for T in (65, 200, 257, 64 * 6):
        C = O.n_history_blocks(T)
        p = _decode_problem(seed, T, k=C + 3, zero_wq=True)
        q, K, V = p.f64("q")[0], p.f64("K")[0], p.f64("V")[0]
        d = q.shape[1]
        res = O.decode_step(p.f64("q"), p.f64("K"), p.f64("V"), p.seq_lens, p.f64("Wq_sel"),
                            p.f64("Wk_sel"), C + 3)
        mask = np.zeros((1, 1, T))
        mask[..., :64 * C] = -math.log(C) if C else 0.0
        for h in range(4):
            r = h // 2
            ref = _sdpa(q[h][None, None], K[r][None, :T], V[r][None, :T], mask, 1 / math.sqrt(d))
            np.testing.assert_allclose(res["o"][0, h], ref[0, 0], atol=1e-10)
    # prefill: every tile selects all its history with log g = -ln t
    S, b = 23, 4
    Q, K, V, _ = _rand_prefill(seed, S=S)
    Wk = np.random.default_rng(seed).standard_normal((8, 8))
    sel = O.prefill_select(Q, K, S, np.zeros((8, 8)), Wk, k=10, G=2, b=b)
    Ot, _ = O.prefill_attend(Q, K, V, S, sel["idx"], sel["log_gate"], 0.4, 2, b)
    mask = np.full((1, S, S), -np.inf)
    for i in range(S):
        t = i // b
        if t:
            mask[0, i, :b * t] = -math.log(t)
        mask[0, i, b * t:i + 1] = 0.0
    for h in range(4):
        ref = _sdpa(Q[h][None], K[h // 2][None], V[h // 2][None], mask, 0.4)
        np.testing.assert_allclose(Ot[h], ref[0], atol=1e-10)


def test_k_equals_C_uniform_gate_is_dense_attention_with_bias():
    check_uniform_gate_is_dense_with_bias()


def check_k0_is_local_causal(seed=5):
    for T in (1, 63, 64, 65, 130):
        p = _decode_problem(seed, T, k=0)
        q, K, V = p.f64("q")[0], p.f64("K")[0], p.f64("V")[0]
        res = O.decode_step(p.f64("q"), p.f64("K"), p.f64("V"), p.seq_lens, p.f64("Wq_sel"),
                            p.f64("Wk_sel"), 0)
        b0 = 64 * O.n_history_blocks(T)
        for h in range(4):
            r = h // 2
            ref = _sdpa(q[h][None, None], K[r][None, b0:T], V[r][None, b0:T],
                        np.zeros((1, 1, T - b0)), 0.25)
            np.testing.assert_allclose(res["o"][0, h], ref[0, 0], atol=1e-10)
    S, b = 22, 4
    Q, K, V, _ = _rand_prefill(seed, S=S)
    idx = np.full((2, 6, 0), -1, np.int64)
    lg = np.zeros((2, 6, 0))
    Ot, _ = O.prefill_attend(Q, K, V, S, idx, lg, 0.5, 2, b)
    for t in range(6):
        i0, i1 = b * t, min(b * t + b, S)
        n = i1 - i0
        causal = np.triu(np.full((n, n), -np.inf), 1)[None]
        for h in range(4):
            ref = _sdpa(Q[h][None, i0:i1], K[h // 2][None, i0:i1], V[h // 2][None, i0:i1],
                        causal, 0.5)
            np.testing.assert_allclose(Ot[h, i0:i1], ref[0], atol=1e-10)


def test_k0_is_local_causal_attention():
    check_k0_is_local_causal()


# --------------------------------------------------------------------------
# gate properties
# --------------------------------------------------------------------------
def test_gate_shift_invariance_and_normalisation():
    rng = np.random.default_rng(6)
    p = _decode_problem(6, 64 * 9 + 3, k=3)
    q, K, V = p.f64("q")[0], p.f64("K")[0], p.f64("V")[0]
    T = int(p.seq_lens[0])
    for _ in range(10):
        s = rng.standard_normal(9) * 2
        c = rng.standard_normal() * 50
        l1, g1 = O.gate(s)
        l2, g2 = O.gate(s + c)
        np.testing.assert_allclose(g1, g2, atol=1e-12)
        assert abs(l2 - l1 - c) < 1e-9
        assert abs(np.exp(g1).sum() - 1.0) < 1e-12
        i1, lg1, _, _ = O.select_rows([s, s[::-1].copy()], 3)
        i2, lg2, _, _ = O.select_rows([s + c, s[::-1] + c], 3)
        assert (i1 == i2).all()
        o1, _ = O.decode_attend(q, K, V, T, i1, lg1, 0.25, 2)
        o2, _ = O.decode_attend(q, K, V, T, i2, lg2, 0.25, 2)
        np.testing.assert_allclose(o1, o2, atol=1e-12)


# --------------------------------------------------------------------------
# backward: finite differences and identities
# --------------------------------------------------------------------------
def _loss(Q, K, V, dO, S, idx, lg, scale, G, b):
    Ot, _ = O.prefill_attend(Q, K, V, S, idx, lg, scale, G, b)
    return float(np.sum(Ot * dO))


def check_dlog_gate_fd(seed=7):
    S, b, k, G, scale = 21, 4, 2, 2, 0.37
    Q, K, V, dO = _rand_prefill(seed, S=S)
    rng = np.random.default_rng(seed)
    idx, lg = _random_selection(rng, 2, 6, k)
    _, _, _, dlg = O.prefill_backward(Q, K, V, dO, S, idx, lg, scale, G, b)
    h = 1e-6
    fd = np.zeros_like(dlg)
    fd_g = np.zeros_like(dlg)
    for r, t, s in zip(*np.nonzero(idx >= 0)):
        lp, lm = lg.copy(), lg.copy()
        lp[r, t, s] += h
        lm[r, t, s] -= h
        fd[r, t, s] = (_loss(Q, K, V, dO, S, idx, lp, scale, G, b) -
                       _loss(Q, K, V, dO, S, idx, lm, scale, G, b)) / (2 * h)
        # eq. 5 lives in g-space: dL/dg_m; log g is the input, so perturb g itself
        g = math.exp(lg[r, t, s])
        lp[r, t, s] = math.log(g + h)
        lm[r, t, s] = math.log(g - h)
        dLdg = (_loss(Q, K, V, dO, S, idx, lp, scale, G, b) -
                _loss(Q, K, V, dO, S, idx, lm, scale, G, b)) / (2 * h)
        fd_g[r, t, s] = g * dLdg
    assert np.abs(fd).max() > 1e-3
    np.testing.assert_allclose(dlg, fd, atol=1e-6 * np.abs(fd).max(), rtol=1e-6)
    np.testing.assert_allclose(dlg, fd_g, atol=1e-6 * np.abs(fd).max(), rtol=1e-6)
    assert (dlg[idx < 0] == 0).all()


def test_dlog_gate_matches_finite_differences():
    check_dlog_gate_fd()


def check_qkv_grads_fd(seed=8):
    S, b, k, G, scale = 19, 4, 2, 2, 0.41
    Q, K, V, dO = _rand_prefill(seed, S=S)
    rng = np.random.default_rng(seed + 1)
    idx, lg = _random_selection(rng, 2, 5, k)
    dQ, dK, dV, _ = O.prefill_backward(Q, K, V, dO, S, idx, lg, scale, G, b)
    h = 1e-6
    for name, X, grad in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for _ in range(12):
            pos = tuple(int(rng.integers(0, n)) for n in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[pos] += h
            Xm[pos] -= h
            args_p = {"Q": Q, "K": K, "V": V}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            fd = (_loss(args_p["Q"], args_p["K"], args_p["V"], dO, S, idx, lg, scale, G, b) -
                  _loss(args_m["Q"], args_m["K"], args_m["V"], dO, S, idx, lg, scale, G, b)) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-6 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


def test_qkv_grads_match_finite_differences():
    check_qkv_grads_fd()


def test_backward_identities():
    """Sum_j dV_j = Sum_rows dO per group (softmax rows sum to 1) and
    Sum_j dK_j = 0 per group (a shift of every key leaves each row unchanged)."""
    S, b, k, G = 30, 4, 3, 2
    Q, K, V, dO = _rand_prefill(9, S=S)
    idx, lg = _random_selection(np.random.default_rng(9), 2, 8, k)
    dQ, dK, dV, _ = O.prefill_backward(Q, K, V, dO, S, idx, lg, 0.3, G, b)
    for r in range(2):
        np.testing.assert_allclose(dV[r].sum(axis=0), dO[r * G:(r + 1) * G].sum(axis=(0, 1)),
                                   atol=1e-12)
        np.testing.assert_allclose(dK[r].sum(axis=0), 0.0, atol=1e-12)


# --------------------------------------------------------------------------
# summaries and scores
# --------------------------------------------------------------------------
def check_summaries(seed=10):
    rng = np.random.default_rng(seed)
    d, ds, b = 8, 6, 4
    W = rng.standard_normal((ds, d))
    for T in (1, 4, 5, 17, 32, 33):
        C = O.n_history_blocks(T, b)
        consts = rng.standard_normal((2, C + 2, d))
        K = np.repeat(consts, b, axis=1)[:, :T + b]          # constant keys inside each block
        K = K + 0.0
        summ = O.block_summaries(K, T, W, b)
        assert summ.shape == (2, C, ds)
        for r in range(2):
            for m in range(C):
                np.testing.assert_allclose(summ[r, m], W @ consts[r, m], atol=1e-12)
        # reordering keys inside a block, or changing B0 / later tokens, changes nothing
        K2 = K.copy()
        for m in range(C):
            K2[:, b * m:b * m + b] = K2[:, b * m:b * m + b][:, ::-1]
        K2[:, b * C:] = rng.standard_normal(K2[:, b * C:].shape)
        np.testing.assert_allclose(O.block_summaries(K2, T, W, b), summ, atol=1e-12)


def test_summaries_closed_forms():
    check_summaries()


def test_scores_closed_form_identity_projection():
    """Wq_sel = Wk_sel = I and block-constant keys c_m: s_m = mean_h(q_h).c_m / sqrt(d)."""
    rng = np.random.default_rng(11)
    d, b, T, G = 8, 4, 23, 3
    C = O.n_history_blocks(T, b)
    c = rng.standard_normal((1, C + 1, d))
    K = np.repeat(c, b, axis=1)
    q = rng.standard_normal((G, d))
    summ = O.block_summaries(K, T, np.eye(d), b)
    s = O.decode_scores(q, np.eye(d), summ, G)
    expect = np.array([q.mean(axis=0) @ c[0, m] for m in range(C)]) / math.sqrt(d)
    np.testing.assert_allclose(s[0], expect, atol=1e-12)


def test_tile_scores_match_decode_scores():
    """A prefill tile whose queries all equal one decode query scores history
    blocks exactly like that decode query."""
    rng = np.random.default_rng(12)
    d, ds, b, G, S = 8, 5, 4, 2, 20
    K = rng.standard_normal((2, S, d))
    Wq, Wk = rng.standard_normal((ds, d)), rng.standard_normal((ds, d))
    qdec = rng.standard_normal((4, d))
    Q = np.repeat(qdec[:, None, :], S, axis=1)
    summ = O.block_summaries(K, S, Wk, b)
    rows = O.tile_scores(Q, S, Wq, summ, G, b)
    for t in range(1, -(-S // b)):
        sd = O.decode_scores(qdec, Wq, summ[:, :t], G)
        np.testing.assert_allclose(rows[t], sd, atol=1e-12)


def test_planted_blocks_are_recalled():
    """With identity selector projections, blocks whose keys carry a strong copy
    of the group query outrank random blocks, so Top-k lands inside the plant."""
    wl = synth.custom_workload("decode", n_q_heads=8, n_kv_heads=2, head_dim=32, sel_dim=32,
                               top_k=8, seq_len=64 * 400 + 1, plant_frac=0.03)
    p = synth.make_problem(wl, 0)
    d = 32
    res = O.decode_step(p.f64("q"), p.f64("K"), p.f64("V"), p.seq_lens, np.eye(d), np.eye(d), 8)
    for r in range(2):
        chosen = res["idx"][0, r]
        assert p.planted[0, r, chosen].all()


# --------------------------------------------------------------------------
# planted mistakes: every mutation must break at least one pin
# --------------------------------------------------------------------------
# selector backward: finite differences through the scores and the weights
# --------------------------------------------------------------------------
def _sel_problem(seed, S=21, b=4, Hq=4, Hkv=2, d=8, d_sel=6, k=2):
    rng = np.random.default_rng(seed)
    Q, K, V, dO = _rand_prefill(seed, Hq=Hq, Hkv=Hkv, d=d, S=S)
    Wq = rng.standard_normal((d_sel, d)) / math.sqrt(d)
    Wk = rng.standard_normal((d_sel, d)) / math.sqrt(d)
    n_tiles = -(-S // b)
    idx, _ = _random_selection(rng, Hkv, n_tiles, k)
    return Q, K, V, dO, Wq, Wk, idx, S, b, Hq // Hkv


def _lg_from_scores(rows, idx):
    """log g of the selected slots from explicit score rows (softmax over the row)."""
    Hkv, n_tiles, k = idx.shape
    lg = np.full(idx.shape, -np.inf)
    for t in range(n_tiles):
        for r in range(Hkv):
            s = rows[t][r]
            if s.size:
                ls = s - (s.max() + np.log(np.exp(s - s.max()).sum()))
                for slot in range(k):
                    if idx[r, t, slot] >= 0:
                        lg[r, t, slot] = ls[idx[r, t, slot]]
    return lg


def _attn_loss_of_weights(Q, K, V, dO, S, b, G, idx, Wq, Wk, scale):
    summ = O.block_summaries(K, S, Wk, b)
    rows = O.tile_scores(Q, S, Wq, summ, G, b)
    return _loss(Q, K, V, dO, S, idx, _lg_from_scores(rows, idx), scale, G, b)


def check_selector_score_grad_fd(seed=21):
    """dL/ds over every history block (selected or not) of the attention loss,
    by central differences on the scores themselves; eq. 8's sparse-scope term
    for the unselected blocks and sum_m ds_m = 0 come with it."""
    Q, K, V, dO, Wq, Wk, idx, S, b, G = _sel_problem(seed)
    scale = 0.43
    summ = O.block_summaries(K, S, Wk, b)
    rows = O.tile_scores(Q, S, Wq, summ, G, b)
    lg = _lg_from_scores(rows, idx)
    _, _, _, dlg = O.prefill_backward(Q, K, V, dO, S, idx, lg, scale, G, b)
    h = 1e-6
    checked = 0
    for t in range(len(rows)):
        for r in range(idx.shape[0]):
            ds = O.score_grad(rows[t][r], idx[r, t], dlg[r, t])
            if ds.size:
                assert abs(ds.sum()) <= 1e-12 * max(1.0, np.abs(ds).max())
            for m in range(rows[t][r].size):
                rp = [x.copy() for x in rows]
                rm = [x.copy() for x in rows]
                rp[t][r, m] += h
                rm[t][r, m] -= h
                fd = (_loss(Q, K, V, dO, S, idx, _lg_from_scores(rp, idx), scale, G, b) -
                      _loss(Q, K, V, dO, S, idx, _lg_from_scores(rm, idx), scale, G, b)) / (2 * h)
                assert abs(ds[m] - fd) <= 1e-6 * max(1.0, abs(fd)), (t, r, m, ds[m], fd)
                if m not in idx[r, t]:
                    g = np.exp(rows[t][r][m] - (rows[t][r].max() + np.log(
                        np.exp(rows[t][r] - rows[t][r].max()).sum())))
                    assert abs(ds[m] + g * dlg[r, t][idx[r, t] >= 0].sum()) <= 1e-12
                checked += 1
    assert checked > 20


def check_selector_weights_fd(seed=22):
    """dWq_sel / dWk_sel of the attention loss through gate, scores and
    summaries, by central differences on every weight."""
    Q, K, V, dO, Wq, Wk, idx, S, b, G = _sel_problem(seed)
    scale = 0.39
    summ = O.block_summaries(K, S, Wk, b)
    rows = O.tile_scores(Q, S, Wq, summ, G, b)
    lg = _lg_from_scores(rows, idx)
    _, _, _, dlg = O.prefill_backward(Q, K, V, dO, S, idx, lg, scale, G, b)
    _, dWq, dWk = O.selector_backward(Q, K, S, Wq, Wk, idx, dlg, G, b)
    h = 1e-6
    for W, dW, which in ((Wq, dWq, "q"), (Wk, dWk, "k")):
        fd = np.zeros_like(W)
        for j, c in itertools.product(range(W.shape[0]), range(W.shape[1])):
            Wp, Wm = W.copy(), W.copy()
            Wp[j, c] += h
            Wm[j, c] -= h
            args = (Wp, Wk) if which == "q" else (Wq, Wp)
            lp = _attn_loss_of_weights(Q, K, V, dO, S, b, G, idx, *args, scale)
            args = (Wm, Wk) if which == "q" else (Wq, Wm)
            lm = _attn_loss_of_weights(Q, K, V, dO, S, b, G, idx, *args, scale)
            fd[j, c] = (lp - lm) / (2 * h)
        assert np.abs(fd).max() > 1e-4
        np.testing.assert_allclose(dW, fd, atol=1e-6 * np.abs(fd).max(), rtol=1e-5)


def test_selector_score_gradient_matches_finite_differences():
    check_selector_score_grad_fd()


def test_selector_weight_gradients_match_finite_differences():
    check_selector_weights_fd()


# --------------------------------------------------------------------------
# per-query selection (a next row): dense causal attention with a per-query
# bias, k = 0, and consistency with the tile selection
def _query_problem(seed, S=150, b=16, Hq=4, Hkv=2, d=8, d_sel=6):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Hq, S, d))
    K = rng.standard_normal((Hkv, S, d))
    V = rng.standard_normal((Hkv, S, d))
    Wq = rng.standard_normal((d_sel, d)) / math.sqrt(d_sel)
    Wk = rng.standard_normal((d_sel, d)) / math.sqrt(d_sel)
    return Q, K, V, Wq, Wk


def check_query_selection_dense(seed=31):
    """k >= every C_i: each query selects all its history blocks, so the
    attention is dense causal attention whose logits carry, per query row, the
    log-gate of the key's block (0 in the query's own block)."""
    S, b, Hq, Hkv, d = 150, 16, 4, 2, 8
    G = Hq // Hkv
    Q, K, V, Wq, Wk = _query_problem(seed, S, b, Hq, Hkv, d)
    scale = 1.0 / math.sqrt(d)
    sel = O.query_select(Q, K, S, Wq, Wk, 100, G, b)
    Oq, _ = O.query_attend(Q, K, V, S, sel["idx"], sel["log_gate"], scale, G, b)
    for h in range(Hq):
        r = h // G
        bias = np.full((S, S), -np.inf)
        for i in range(S):
            C = i // b
            assert list(sel["idx"][r, i, :C]) == list(range(C))
            lg = sel["log_gate"][r, i, :C]
            if C:
                assert abs(np.exp(lg).sum() - 1.0) < 1e-12     # the gate is a softmax
            for j in range(i + 1):
                bias[i, j] = lg[j // b] if j // b < C else 0.0
        Z = Q[h, :S] @ K[r, :S].T * scale + bias
        P = np.exp(Z - Z.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        assert np.abs(P @ V[r, :S] - Oq[h]).max() < 1e-12


def check_query_k0_local(seed=32):
    """k = 0: every query attends to its own block only, causally."""
    S, b, Hq, Hkv, d = 100, 16, 4, 2, 8
    G = Hq // Hkv
    Q, K, V, Wq, Wk = _query_problem(seed, S, b, Hq, Hkv, d)
    scale = 1.0 / math.sqrt(d)
    sel = O.query_select(Q, K, S, Wq, Wk, 0, G, b)
    Oq, lse = O.query_attend(Q, K, V, S, sel["idx"], sel["log_gate"], scale, G, b)
    for h in range(Hq):
        r = h // G
        for i in range(S):
            j0 = b * (i // b)
            z = K[r, j0:i + 1] @ Q[h, i] * scale
            p = np.exp(z - z.max())
            assert np.abs(p @ V[r, j0:i + 1] / p.sum() - Oq[h, i]).max() < 1e-12
            assert abs(lse[h, i] - (z.max() + math.log(p.sum()))) < 1e-12


def check_query_scores_vs_tiles(seed=33):
    """Queries that are equal within each tile give the tile's scores: the
    tile's pooling then averages identical rows."""
    S, b, Hq, Hkv, d = 96, 16, 4, 2, 8
    G = Hq // Hkv
    Q, K, V, Wq, Wk = _query_problem(seed, S, b, Hq, Hkv, d)
    for t in range(S // b):
        Q[:, b * t:b * t + b] = Q[:, b * t:b * t + 1]
    summ = O.block_summaries(K, S, Wk, b)
    rows_q = O.query_scores(Q, S, Wq, summ, G, b)
    rows_t = O.tile_scores(Q, S, Wq, summ, G, b)
    for i in range(S):
        assert rows_q[i].shape == rows_t[i // b].shape
        assert np.abs(rows_q[i] - rows_t[i // b]).max(initial=0.0) < 1e-12


def _random_query_selection(rng, Hkv, S, b, k):
    idx = np.full((Hkv, S, k), -1, np.int64)
    lg = np.full((Hkv, S, k), -np.inf)
    for r in range(Hkv):
        for i in range(S):
            n = min(k, i // b)
            if n:
                idx[r, i, :n] = np.sort(rng.choice(i // b, size=n, replace=False))
                lg[r, i, :n] = -rng.uniform(0.2, 3.0, size=n)
    return idx, lg


def _query_loss(Q, K, V, dO, S, idx, lg, scale, G, b):
    Oq, _ = O.query_attend(Q, K, V, S, idx, lg, scale, G, b)
    return float(np.sum(Oq[:, :S] * dO[:, :S]))


def check_query_backward_fd(seed=34):
    """Per-query backward against central differences of L = <dO, O>: every
    log-gate entry of every query, and sampled entries of Q, K and V."""
    S, b, Hq, Hkv, d, k, scale = 22, 4, 4, 2, 3, 2, 0.43
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal(sh) for sh in ((Hq, S, d), (Hkv, S, d), (Hkv, S, d)))
    dO = rng.standard_normal((Hq, S, d))
    idx, lg = _random_query_selection(rng, Hkv, S, b, k)
    dQ, dK, dV, dlg = O.query_backward(Q, K, V, dO, S, idx, lg, scale, G, b)
    h = 1e-6
    fd = np.zeros_like(dlg)
    for r, i, sl in zip(*np.nonzero(idx >= 0)):
        lp, lm = lg.copy(), lg.copy()
        lp[r, i, sl] += h
        lm[r, i, sl] -= h
        fd[r, i, sl] = (_query_loss(Q, K, V, dO, S, idx, lp, scale, G, b) -
                        _query_loss(Q, K, V, dO, S, idx, lm, scale, G, b)) / (2 * h)
    assert np.abs(fd).max() > 1e-3
    np.testing.assert_allclose(dlg, fd, atol=1e-6 * np.abs(fd).max(), rtol=1e-6)
    assert (dlg[idx < 0] == 0).all()
    for name, X, grad in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for _ in range(12):
            pos = tuple(int(rng.integers(0, n)) for n in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[pos] += h
            Xm[pos] -= h
            args_p = {"Q": Q, "K": K, "V": V}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            fdx = (_query_loss(args_p["Q"], args_p["K"], args_p["V"], dO, S, idx, lg, scale, G, b) -
                   _query_loss(args_m["Q"], args_m["K"], args_m["V"], dO, S, idx, lg, scale, G, b)) / (2 * h)
            assert abs(fdx - grad[pos]) <= 1e-6 * max(1.0, abs(fdx)), (name, pos, fdx, grad[pos])


def check_query_backward_vs_tiles(seed=35):
    """Queries that carry their tile's selection: the per-query backward gives
    the tile backward's dQ, dK and dV, and its per-query log-gate gradients
    sum over each tile's queries to the tile's."""
    S, b, Hq, Hkv, d, k, scale = 45, 8, 4, 2, 5, 3, 0.31
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal(sh) for sh in ((Hq, S, d), (Hkv, S, d), (Hkv, S, d)))
    dO = rng.standard_normal((Hq, S, d))
    n_tiles = -(-S // b)
    idx_t, lg_t = _random_selection(rng, Hkv, n_tiles, k)
    tile_of = np.arange(S) // b
    qQ, qK, qV, qlg = O.query_backward(Q, K, V, dO, S, idx_t[:, tile_of], lg_t[:, tile_of],
                                       scale, G, b)
    tQ, tK, tV, tlg = O.prefill_backward(Q, K, V, dO, S, idx_t, lg_t, scale, G, b)
    for a, c in ((qQ, tQ), (qK, tK), (qV, tV)):
        assert np.abs(a - c).max() < 1e-12
    summed = np.zeros_like(tlg)
    for i in range(S):
        summed[:, i // b] += qlg[:, i]
    assert np.abs(summed - tlg).max() < 1e-12


def _query_lg_from_scores(rows, idx):
    """Per-query log g of the selected slots from explicit score rows."""
    Hkv, S, k = idx.shape
    lg = np.full(idx.shape, -np.inf)
    for i in range(S):
        for r in range(Hkv):
            s = rows[i][r]
            if s.size:
                ls = s - (s.max() + np.log(np.exp(s - s.max()).sum()))
                for slot in range(k):
                    if idx[r, i, slot] >= 0:
                        lg[r, i, slot] = ls[idx[r, i, slot]]
    return lg


def _query_loss_of_weights(Q, K, V, dO, S, b, G, idx, Wq, Wk, scale):
    summ = O.block_summaries(K, S, Wk, b)
    rows = O.query_scores(Q, S, Wq, summ, G, b)
    return _query_loss(Q, K, V, dO, S, idx, _query_lg_from_scores(rows, idx), scale, G, b)


def check_query_selector_weights_fd(seed=36):
    """Per-query rows: dWq_sel / dWk_sel of the attention loss through the
    per-query gates, scores and summaries, by central differences on every
    weight (the selection held fixed)."""
    S, b, Hq, Hkv, d, d_sel, k, scale = 22, 4, 4, 2, 5, 3, 2, 0.41
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal(sh) for sh in ((Hq, S, d), (Hkv, S, d), (Hkv, S, d)))
    dO = rng.standard_normal((Hq, S, d))
    Wq = rng.standard_normal((d_sel, d)) / math.sqrt(d)
    Wk = rng.standard_normal((d_sel, d)) / math.sqrt(d)
    idx, _ = _random_query_selection(rng, Hkv, S, b, k)
    summ = O.block_summaries(K, S, Wk, b)
    lg = _query_lg_from_scores(O.query_scores(Q, S, Wq, summ, G, b), idx)
    _, _, _, dlg = O.query_backward(Q, K, V, dO, S, idx, lg, scale, G, b)
    _, dWq, dWk = O.query_selector_backward(Q, K, S, Wq, Wk, idx, dlg, G, b)
    h = 1e-6
    for W, dW, which in ((Wq, dWq, "q"), (Wk, dWk, "k")):
        fd = np.zeros_like(W)
        for j, c in itertools.product(range(W.shape[0]), range(W.shape[1])):
            Wp, Wm = W.copy(), W.copy()
            Wp[j, c] += h
            Wm[j, c] -= h
            args = (Wp, Wk) if which == "q" else (Wq, Wp)
            lp = _query_loss_of_weights(Q, K, V, dO, S, b, G, idx, *args, scale)
            args = (Wm, Wk) if which == "q" else (Wq, Wm)
            lm = _query_loss_of_weights(Q, K, V, dO, S, b, G, idx, *args, scale)
            fd[j, c] = (lp - lm) / (2 * h)
        assert np.abs(fd).max() > 1e-4
        np.testing.assert_allclose(dW, fd, atol=1e-6 * np.abs(fd).max(), rtol=1e-5)


def check_query_selector_vs_tiles(seed=37):
    """Queries equal within each tile and carrying their tile's selection: the
    per-query selector gradients equal the tile rows' gradients taken with
    each tile's log-gate gradients summed over its queries."""
    S, b, Hq, Hkv, d, d_sel, k = 40, 8, 4, 2, 5, 3, 2
    G = Hq // Hkv
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Hq, S, d))
    for t in range(S // b):
        Q[:, b * t:b * t + b] = Q[:, b * t:b * t + 1]
    K = rng.standard_normal((Hkv, S, d))
    Wq = rng.standard_normal((d_sel, d)) / math.sqrt(d)
    Wk = rng.standard_normal((d_sel, d)) / math.sqrt(d)
    n_tiles = S // b
    idx_t, _ = _random_selection(rng, Hkv, n_tiles, k)
    tile_of = np.arange(S) // b
    dlg_q = rng.standard_normal((Hkv, S, k)) * (idx_t[:, tile_of] >= 0)
    _, qWq, qWk = O.query_selector_backward(Q, K, S, Wq, Wk, idx_t[:, tile_of], dlg_q, G, b)
    dlg_t = np.zeros((Hkv, n_tiles, k))
    for i in range(S):
        dlg_t[:, i // b] += dlg_q[:, i]
    _, tWq, tWk = O.selector_backward(Q, K, S, Wq, Wk, idx_t, dlg_t, G, b)
    assert np.abs(qWq - tWq).max() < 1e-12 and np.abs(qWk - tWk).max() < 1e-12


def test_query_selector_weight_gradients_match_finite_differences():
    check_query_selector_weights_fd()


def test_query_selector_gradients_reduce_to_tile_rows():
    check_query_selector_vs_tiles()


def test_query_backward_matches_finite_differences():
    check_query_backward_fd()


def test_query_backward_reduces_to_tile_backward():
    check_query_backward_vs_tiles()


def test_query_selection_is_dense_when_k_covers_history():
    check_query_selection_dense()


def test_query_selection_k0_is_local_causal():
    check_query_k0_local()


def test_query_scores_match_tile_scores_on_tile_constant_queries():
    check_query_scores_vs_tiles()


# --------------------------------------------------------------------------
PINS = [check_hand_worked, check_topk_lexsort, check_topk_exhaustive, check_gather_vs_dense,
        check_uniform_gate_is_dense_with_bias, check_k0_is_local_causal, check_dlog_gate_fd,
        check_qkv_grads_fd, check_summaries, check_selector_score_grad_fd,
        check_selector_weights_fd, check_query_selection_dense, check_query_k0_local,
        check_query_scores_vs_tiles, check_query_backward_fd, check_query_backward_vs_tiles,
        check_query_selector_weights_fd, check_query_selector_vs_tiles]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            return True
    return False


def _wrong_gate_sign(s):
    lse, logg = _ORIG["gate"](s)
    return lse, -logg


def _topk_highest_index_ties(s, k):
    C = int(s.size)
    kk = max(0, min(int(k), C))
    order = sorted(range(C), key=lambda m: (-float(s[m]), -m))
    return sorted(order[:kk]), _ORIG["topk"](s, k)[1]


def _summaries_sum_not_mean(K, T, Wk, b=O.BLOCK):
    return _ORIG["block_summaries"](K, T, Wk, b) * b


_ORIG = {"gate": O.gate, "topk": O.topk, "block_summaries": O.block_summaries,
         "_selected_tokens": O._selected_tokens, "score_grad": O.score_grad,
         "query_scores": O.query_scores, "_slot_sums": O._slot_sums}


def _query_history_includes_own_block(Q, S, Wq, summ, G, b=O.BLOCK, queries=None):
    """Lets query i score its own (incomplete) block as history."""
    out = {}
    for i in (range(S) if queries is None else queries):
        C = min(i // b + 1, summ.shape[1])
        out[i] = O.decode_scores(Q[:, i], Wq, summ[:, :C], G)
    return out


def _score_grad_no_normaliser(s, idx_row, dlg_row):
    """Forgets the -g_m sum dlog g term of the log-softmax."""
    out = np.zeros(s.size)
    for m, dl in zip(idx_row, dlg_row):
        if m >= 0:
            out[m] += dl
    return out


def _slot_sums_with_own_block(dz, slots, k):
    """Credits the query's own block (no gate) to its first slot as well."""
    out = _ORIG["_slot_sums"](dz, slots, k)
    if k:
        out[0] += dz[slots == -1].sum()
    return out


def _drop_gate_bias(idx_row, lg_row, b, gated):
    return _ORIG["_selected_tokens"](idx_row, lg_row, b, False)


def _off_by_one_block(idx_row, lg_row, b, gated):
    toks, bias = _ORIG["_selected_tokens"](idx_row, lg_row, b, gated)
    return [t + 1 if t + 1 < 10 ** 9 else t for t in toks], bias


@pytest.mark.parametrize("name,fn", [
    ("gate", _wrong_gate_sign),
    ("topk", _topk_highest_index_ties),
    ("block_summaries", _summaries_sum_not_mean),
    ("_selected_tokens", _drop_gate_bias),
    ("_selected_tokens", _off_by_one_block),
    ("score_grad", _score_grad_no_normaliser),
    ("query_scores", _query_history_includes_own_block),
    ("_slot_sums", _slot_sums_with_own_block),
])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    assert _some_pin_fails()
