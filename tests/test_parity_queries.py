"""GPU parity of the per-query selection path against the CPU oracle, through
the C ABI: sas_block_summaries -> sas_select(QUERIES) -> sas_prefill_fwd_queries.

Per-query selection is the training kernel's own masking rule (SAS close
reading 2.4: every query is masked by its own gate threshold): query i keeps
the Top-k of its own scores over the i // 64 blocks before its block, which
is the decode selection of a query at position i.

The selection is checked row by row against the oracle's query_select (the
index rule with the near-tie band, log-gate, LSE and the raw scores).  The
forward gets a selection that does not come from the GPU (the oracle's own
per-query Top-K on small shapes, a seeded random valid per-query selection at
full size) and is compared with the oracle's query_attend.  A property that
holds at any size: when every query carries its tile's selection, the
per-query forward equals sas_prefill_fwd bit for bit."""
import math

import numpy as np
import pytest
import torch

from gated_block_sparse_amd import synth
from oracle import sas_oracle as O
from tests.gpu_util import (TOL_F32_OUT, TOL_GRAD_REL, TOL_OUT, check_selection_row, dev, host,
                            idx_dev, lg_dev, log, needs_gpu)

pytestmark = [pytest.mark.gpu, needs_gpu]
TOL_LSE = 1e-3


def _sas():
    from gated_block_sparse_amd import binding
    return binding


def _problem(S, Hq=4, Hkv=1, d=128, ds=128, k=4, dtype="bf16", seed=0):
    wl = synth.custom_workload("prefill", n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, sel_dim=ds,
                               top_k=k, dtype=dtype, seq_len=S)
    return synth.make_problem(wl, seed)


def random_query_selection(rng, Hkv, S, k):
    """A seeded valid per-query selection: row i holds min(k, i // 64) distinct
    blocks below i // 64, ascending, -1 padded, with log g < 0."""
    idx = np.full((Hkv, S, k), -1, np.int64)
    lg = np.full((Hkv, S, k), -np.inf)
    for r in range(Hkv):
        for i in range(S):
            C = i // 64
            n = min(k, C)
            if n:
                idx[r, i, :n] = np.sort(rng.choice(C, size=n, replace=False))
                lg[r, i, :n] = -rng.uniform(0.5, 8.0, size=n)
    return idx, lg


def check_select_queries(p, summ_g, queries):
    """GPU per-query selection vs the oracle on the given queries."""
    S_ = _sas()
    wl = p.wl
    S, Hkv, G, k, dt = int(p.seq_lens[0]), wl.n_kv_heads, wl.group, wl.top_k, wl.dtype
    idx_g, lg_g, slse_g, sc_g = S_.sas_select(S_.SAS_SELECT_QUERIES, dev(p.q), None,
                                              dev(p.Wq_sel), summ_g, k, t_max=p.K.shape[2],
                                              want_scores=True)
    idx_h, lg_h, slse_h, sc_h = idx_g.cpu().numpy(), host(lg_g), host(slse_g), host(sc_g)
    Qf, Kf = synth.to_f64(p.q[0], dt), synth.to_f64(p.K[0], dt)
    ref = O.query_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G, queries=queries)
    tol = TOL_F32_OUT[dt]
    n_exact = n_rows = 0
    for i in queries:
        C = i // 64
        for r in range(Hkv):
            s = ref["scores"][i][r]
            if C:
                err = np.abs(sc_h[0, r, i, :C] - s).max()
                assert err <= tol, (i, r, err)
                assert abs(slse_h[0, r, i] - ref["score_lse"][r, i]) <= tol, (i, r)
            else:
                assert np.isneginf(slse_h[0, r, i])
            n_exact += check_selection_row(idx_h[0, r, i], lg_h[0, r, i], s, ref["idx"][r, i],
                                           ref["gap"][r, i], k, ref["score_lse"][r, i], tol)
            n_rows += 1
    return idx_g, lg_g, n_exact, n_rows


def run_queries_case(p, queries=None, selection="oracle", gated=True, label=""):
    S_ = _sas()
    wl = p.wl
    S, Hq, Hkv, d, k, G = int(p.seq_lens[0]), wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k, wl.group
    queries = list(range(S)) if queries is None else sorted(queries)
    log(f"[queries {label}] S={S} Hq={Hq} Hkv={Hkv} d={d} k={k} {len(queries)} queries checked")
    Q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.tensor([S], dtype=torch.int32).cuda()
    summ_g = S_.sas_block_summaries(K, lens, dev(p.Wk_sel))
    _, _, n_exact, n_rows = check_select_queries(p, summ_g, queries)
    log(f"[queries {label}] per-query selection exact on {n_exact}/{n_rows} rows")

    Qf, Kf, Vf = (synth.to_f64(x[0], "bf16") for x in (p.q, p.K, p.V))
    if selection == "oracle":
        sel = O.query_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
        idx, lg = sel["idx"], sel["log_gate"]
    else:
        idx, lg = random_query_selection(np.random.default_rng(2024), Hkv, S, k)
    scale = 1.0 / math.sqrt(d)
    O_g, lse_g = S_.sas_prefill_fwd_queries(Q, K, V, idx_dev(idx[None]),
                                            lg_dev(lg[None]) if gated else None)
    Or, lser = O.query_attend(Qf, Kf, Vf, S, idx, lg, scale, G, gated=gated, queries=queries)
    O_h, lse_h = host(O_g)[0], host(lse_g)[0]
    err_o = np.abs(O_h[:, queries] - Or[:, queries]).max()
    err_l = np.abs(lse_h[:, queries] - lser[:, queries]).max()
    log(f"[queries {label}] max|O-O_ref|={err_o:.3g} max|lse-lse_ref|={err_l:.3g}")
    assert err_o <= TOL_OUT["bf16"], err_o
    assert err_l <= TOL_LSE, err_l


@pytest.mark.parametrize("S,Hq,Hkv,d,ds,k", [
    (64, 4, 1, 128, 128, 4), (100, 4, 1, 128, 128, 4), (1000, 8, 2, 128, 128, 3),
    (2048, 8, 2, 128, 128, 16), (777, 2, 2, 64, 128, 5), (640, 8, 1, 128, 64, 4),
    (700, 16, 2, 64, 64, 6), (1, 4, 1, 128, 128, 2), (1300, 4, 4, 128, 128, 64),
])
def test_queries_small(S, Hq, Hkv, d, ds, k):
    run_queries_case(_problem(S, Hq, Hkv, d, ds, k, seed=S + Hq + 7), label=f"S={S}")


def test_queries_ungated_and_k0():
    run_queries_case(_problem(500, 8, 2, 128, 128, 4, seed=5), gated=False, label="ungated")
    run_queries_case(_problem(333, 8, 2, 128, 128, 0, seed=6), label="k=0")


@pytest.mark.parametrize("S,Hq,Hkv,d,ds,k", [(900, 4, 1, 64, 64, 8), (300, 8, 2, 128, 128, 5)])
def test_select_queries_fp32(S, Hq, Hkv, d, ds, k):
    """The per-query selection on fp32 queries and keys (fp32 tolerances)."""
    p = _problem(S, Hq, Hkv, d, ds, k, dtype="f32", seed=S)
    K = dev(p.K)
    summ_g = _sas().sas_block_summaries(K, torch.tensor([S], dtype=torch.int32).cuda(),
                                        dev(p.Wk_sel))
    _, _, n_exact, n_rows = check_select_queries(p, summ_g, list(range(S)))
    log(f"[queries fp32 S={S}] exact on {n_exact}/{n_rows} rows")


def _tile_vs_query_bitwise(p, label):
    S_ = _sas()
    wl = p.wl
    S, Hkv, k = int(p.seq_lens[0]), wl.n_kv_heads, wl.top_k
    n_tiles = -(-S // 64)
    rng = np.random.default_rng(99)
    idx_t = np.full((Hkv, n_tiles, k), -1, np.int64)
    lg_t = np.full((Hkv, n_tiles, k), -np.inf)
    for r in range(Hkv):
        for t in range(n_tiles):
            n = min(k, t)
            if n:
                idx_t[r, t, :n] = np.sort(rng.choice(t, size=n, replace=False))
                lg_t[r, t, :n] = -rng.uniform(0.5, 8.0, size=n)
    tile_of = np.arange(S) // 64
    idx_q, lg_q = idx_t[:, tile_of], lg_t[:, tile_of]
    Q, K, V = dev(p.q), dev(p.K), dev(p.V)
    O_t, lse_t = S_.sas_prefill_fwd(Q, K, V, idx_dev(idx_t[None]), lg_dev(lg_t[None]))
    O_q, lse_q = S_.sas_prefill_fwd_queries(Q, K, V, idx_dev(idx_q[None]), lg_dev(lg_q[None]))
    torch.cuda.synchronize()
    log(f"[queries {label}] tile-selection broadcast: O equal={torch.equal(O_t, O_q)} "
        f"lse equal={torch.equal(lse_t, lse_q)}")
    assert torch.equal(O_t, O_q) and torch.equal(lse_t, lse_q)


def test_queries_equal_tile_forward_small():
    _tile_vs_query_bitwise(_problem(1024, 8, 2, 128, 128, 5, seed=11), "S=1024")
    _tile_vs_query_bitwise(_problem(640, 4, 1, 64, 64, 3, seed=12), "S=640 d=64")


@pytest.mark.timeout(900)
def test_queries_full_workload():
    """The training-style workload (S=16384, Qwen3-4B head shape, k=16): the
    per-query selection on sampled queries (first, tile edges, last), the
    forward with a random per-query selection on those queries, and the
    bitwise equality with the tile forward under a broadcast tile selection."""
    p = synth.make_problem(synth.WORKLOADS["qwen3_4b_prefill_16k"], seed=0)
    queries = [0, 1, 63, 64, 65, 1023, 1024, 1087, 4095, 8200, 12345, 16320, 16383]
    run_queries_case(p, queries=queries, selection="random", label="qwen3_4b_prefill_16k")
    _tile_vs_query_bitwise(p, "qwen3_4b_prefill_16k")


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def run_queries_bwd_case(p, queries=None, selection="oracle", label=""):
    """sas_bwd_queries on the per-query forward's outputs vs the oracle's
    query_backward.  With sampled queries, dQ and dlog_gate are compared on
    those queries and dK/dV through identities that hold at any size."""
    S_ = _sas()
    wl = p.wl
    S, Hq, Hkv, d, k, G = int(p.seq_lens[0]), wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k, wl.group
    full = queries is None
    queries = list(range(S)) if full else sorted(queries)
    log(f"[queries bwd {label}] S={S} Hq={Hq} Hkv={Hkv} d={d} k={k} {len(queries)} queries checked")
    Q, K, V, dO = dev(p.q), dev(p.K), dev(p.V), dev(p.dO)
    Qf, Kf, Vf, dOf = (synth.to_f64(x[0], "bf16") for x in (p.q, p.K, p.V, p.dO))
    if selection == "oracle":
        sel = O.query_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
        idx, lg = sel["idx"], sel["log_gate"]
    else:
        idx, lg = random_query_selection(np.random.default_rng(77), Hkv, S, k)
    idx_d, lg_d = idx_dev(idx[None]), lg_dev(lg[None])
    O_g, lse_g = S_.sas_prefill_fwd_queries(Q, K, V, idx_d, lg_d)
    dQ, dK, dV, dlg = S_.sas_bwd_queries(Q, K, V, O_g, dO, lse_g, idx_d, lg_d)
    scale = 1.0 / math.sqrt(d)
    rQ, rK, rV, rlg = O.query_backward(Qf, Kf, Vf, dOf, S, idx, lg, scale, G,
                                       queries=None if full else queries)
    gQ, gK, gV, glg = host(dQ)[0], host(dK)[0][:, :S], host(dV)[0][:, :S], host(dlg)[0]
    floor = 1e-2 * np.linalg.norm(dOf[:, queries])

    def rel_l2(x, ref):
        return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), floor))

    e_q = rel_l2(gQ[:, queries], rQ[:, queries])
    valid = np.zeros_like(idx, bool)
    valid[:, queries] = idx[:, queries] >= 0
    e_lg = 0.0
    if valid.any():
        e_lg = float(np.linalg.norm(glg[valid] - rlg[valid]) / max(np.linalg.norm(rlg[valid]), 1e-30))
    assert (glg[idx < 0] == 0).all()
    msg = f"[queries bwd {label}] rel dQ={e_q:.3g} dlog_gate={e_lg:.3g}"
    if full:
        e_k, e_v = rel_l2(gK, rK), rel_l2(gV, rV)
        msg += f" dK={e_k:.3g} dV={e_v:.3g}"
        assert max(e_k, e_v) <= TOL_GRAD_REL
    # identities at any size: sum_j dV_j = sum over the group's rows of dO
    # (softmax rows sum to 1), sum_j dK_j = 0 (shifting every key leaves each
    # softmax row unchanged)
    # (exactly 0: its GPU value is rounding residue, hence the absolute slack)
    for r in range(Hkv):
        so = dOf[r * G:(r + 1) * G, :S].sum(axis=(0, 1))
        assert np.linalg.norm(gV[r].sum(axis=0) - so) <= TOL_GRAD_REL * max(np.linalg.norm(so), floor)
        assert np.linalg.norm(gK[r].sum(axis=0)) <= TOL_GRAD_REL * np.linalg.norm(gK[r]) + 1e-3
    log(msg)
    assert max(e_q, e_lg) <= TOL_GRAD_REL


@pytest.mark.parametrize("S,Hq,Hkv,d,k", [
    (64, 4, 1, 128, 4), (100, 4, 1, 128, 4), (1000, 8, 2, 128, 3), (777, 2, 2, 64, 5),
    (700, 16, 2, 64, 6), (1, 4, 1, 128, 2), (900, 4, 4, 128, 64), (640, 8, 1, 128, 16),
])
def test_queries_bwd_small(S, Hq, Hkv, d, k):
    run_queries_bwd_case(_problem(S, Hq, Hkv, d, 128, k, seed=S + 2 * Hq), label=f"S={S}")


def test_queries_bwd_k0():
    run_queries_bwd_case(_problem(333, 8, 2, 128, 128, 0, seed=8), label="k=0")


def _tile_vs_query_bwd(p, label):
    """Every query carries its tile's selection: dQ, dK and dV equal the tile
    backward's bit for bit, and the per-query log-gate gradients sum over each
    tile's queries to the tile's (fp32 sums in another order)."""
    S_ = _sas()
    wl = p.wl
    S, Hkv, k = int(p.seq_lens[0]), wl.n_kv_heads, wl.top_k
    n_tiles = -(-S // 64)
    rng = np.random.default_rng(98)
    idx_t = np.full((Hkv, n_tiles, k), -1, np.int64)
    lg_t = np.full((Hkv, n_tiles, k), -np.inf)
    for r in range(Hkv):
        for t in range(n_tiles):
            n = min(k, t)
            if n:
                idx_t[r, t, :n] = np.sort(rng.choice(t, size=n, replace=False))
                lg_t[r, t, :n] = -rng.uniform(0.5, 8.0, size=n)
    tile_of = np.arange(S) // 64
    Q, K, V, dO = dev(p.q), dev(p.K), dev(p.V), dev(p.dO)
    it, lt = idx_dev(idx_t[None]), lg_dev(lg_t[None])
    iq, lq = idx_dev(idx_t[:, tile_of][None]), lg_dev(lg_t[:, tile_of][None])
    O_t, lse_t = S_.sas_prefill_fwd(Q, K, V, it, lt)
    tQ, tK, tV, tlg = S_.sas_bwd(Q, K, V, O_t, dO, lse_t, it, lt)
    qQ, qK, qV, qlg = S_.sas_bwd_queries(Q, K, V, O_t, dO, lse_t, iq, lq)
    torch.cuda.synchronize()
    same = [torch.equal(a, b) for a, b in ((tQ, qQ), (tK[:, :, :S], qK[:, :, :S]),
                                           (tV[:, :, :S], qV[:, :, :S]))]
    summed = np.zeros((Hkv, n_tiles, k))
    ql = host(qlg)[0]
    for i in range(S):
        summed[:, i // 64] += ql[:, i]
    tl = host(tlg)[0]
    e = float(np.linalg.norm(summed - tl) / max(np.linalg.norm(tl), 1e-30))
    log(f"[queries bwd {label}] tile selection broadcast: dQ/dK/dV equal={same} "
        f"dlog_gate tile sums rel={e:.3g}")
    assert all(same)
    assert e <= 1e-4


def test_queries_bwd_equal_tile_backward_small():
    _tile_vs_query_bwd(_problem(1024, 8, 2, 128, 128, 5, seed=13), "S=1024")
    _tile_vs_query_bwd(_problem(640, 4, 1, 64, 128, 3, seed=14), "S=640 d=64")


@pytest.mark.timeout(900)
def test_queries_bwd_full_workload():
    """The training-style workload (S=16384, Qwen3-4B head shape, k=16) with a
    random per-query selection: dQ and dlog_gate on sampled queries, the dK/dV
    identities, and the bitwise equality with the tile backward."""
    p = synth.make_problem(synth.WORKLOADS["qwen3_4b_prefill_16k"], seed=0)
    queries = [0, 63, 64, 1000, 4095, 8200, 12345, 16383]
    run_queries_bwd_case(p, queries=queries, selection="random", label="qwen3_4b_prefill_16k")
    _tile_vs_query_bwd(p, "qwen3_4b_prefill_16k")


def test_queries_batch2_select_fwd_bwd():
    """Two sequences in one call (grid z) with a t_max above S: the per-query
    selection, forward and backward of each sequence against the oracle run on
    that sequence alone."""
    S_ = _sas()
    S, Hq, Hkv, d, k = 650, 8, 2, 128, 5
    wl = synth.custom_workload("prefill", batch=2, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                               sel_dim=128, top_k=k, dtype="bf16", seq_len=S)
    p = synth.make_problem(wl, 41)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    t_max = S + 100     # K/V rows past S are never read
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (t_max - S, d), x.dtype)], axis=2)
    Qd, dOd = dev(p.q), dev(p.dO)
    Kd, Vd = dev(pad(p.K)), dev(pad(p.V))
    lens = torch.tensor([S, S], dtype=torch.int32).cuda()
    summ = S_.sas_block_summaries(Kd, lens, dev(p.Wk_sel))
    gidx, glg, _, _ = S_.sas_select(S_.SAS_SELECT_QUERIES, Qd, None, dev(p.Wq_sel), summ, k,
                                    t_max=t_max)
    sels, refs = [], []
    for b in range(2):
        Qf, Kf, Vf, dOf = (synth.to_f64(x[b], "bf16") for x in (p.q, p.K, p.V, p.dO))
        sel = O.query_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
        gi = gidx.cpu().numpy()[b]
        exact = (gi == sel["idx"]).all(axis=-1) | (sel["gap"] <= 1e-4)
        assert exact.all(), b
        sels.append(sel)
        Or, lser = O.query_attend(Qf, Kf, Vf, S, sel["idx"], sel["log_gate"], scale, G)
        gr = O.query_backward(Qf, Kf, Vf, dOf, S, sel["idx"], sel["log_gate"], scale, G)
        refs.append((Or, lser, gr))
    idx = idx_dev(np.stack([s["idx"] for s in sels]))
    lg = lg_dev(np.stack([s["log_gate"] for s in sels]))
    O_g, lse_g = S_.sas_prefill_fwd_queries(Qd, Kd, Vd, idx, lg)
    dQ, dK, dV, dlg = S_.sas_bwd_queries(Qd, Kd, Vd, O_g, dOd, lse_g, idx, lg)
    torch.cuda.synchronize()
    for b in range(2):
        Or, lser, (rQ, rK, rV, rlg) = refs[b]
        err = np.abs(host(O_g)[b] - Or).max()
        assert err <= TOL_OUT["bf16"], (b, err)
        for g, r in ((dQ, rQ), (dK, rK), (dV, rV)):
            x = host(g)[b][:, :S]
            assert np.linalg.norm(x - r) <= TOL_GRAD_REL * np.linalg.norm(r), b
        valid = sels[b]["idx"] >= 0
        e = np.linalg.norm(host(dlg)[b][valid] - rlg[valid]) / np.linalg.norm(rlg[valid])
        assert e <= TOL_GRAD_REL, (b, e)
        log(f"[queries batch2] sequence {b}: max|O-O_ref|={err:.3g} rel dlog_gate={e:.3g}")


# --------------------------------------------------------------------------
# selector backward for per-query rows
# --------------------------------------------------------------------------
def run_selector_queries_case(p, dlg_from="random", label=""):
    """sas_selector_bwd_queries against the oracle's query_selector_backward;
    both sides get the oracle's per-query selection, score LSE and log-gate
    gradients (seeded random ones, or the oracle's query_backward of the
    attention loss)."""
    S_ = _sas()
    wl = p.wl
    S, Hkv, G, k, dt, d = int(p.seq_lens[0]), wl.n_kv_heads, wl.group, wl.top_k, wl.dtype, wl.head_dim
    t_max = p.K.shape[2]
    log(f"[selector bwd queries {label}] S={S} Hq={wl.n_q_heads} Hkv={Hkv} d={d} "
        f"d_sel={wl.sel_dim} k={k} {dt}")
    Qf, Kf = synth.to_f64(p.q[0], dt), synth.to_f64(p.K[0], dt)
    sel = O.query_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
    idx, lse = sel["idx"], sel["score_lse"]
    if dlg_from == "random":
        rng = np.random.default_rng(S + k)
        dlg = rng.standard_normal(idx.shape) * 0.1 * (idx >= 0)
    else:
        Vf, dOf = synth.to_f64(p.V[0], dt), synth.to_f64(p.dO[0], dt)
        dlg = O.query_backward(Qf, Kf, Vf, dOf, S, idx, sel["log_gate"], 1.0 / math.sqrt(d), G)[3]
    Q, K = dev(p.q), dev(p.K)
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    summ = S_.sas_block_summaries(K, torch.tensor([S], dtype=torch.int32).cuda(), Wk)
    dWq_g, dWk_g, ds_g = S_.sas_selector_bwd_queries(
        Q, K, Wq, Wk, summ, idx_dev(idx[None]), lg_dev(lse[None]), lg_dev(dlg[None]),
        t_max=t_max, want_ds=True)
    torch.cuda.synchronize()
    ds_rows, dWq_r, dWk_r = O.query_selector_backward(Qf, Kf, S, p.f64("Wq_sel"),
                                                      p.f64("Wk_sel"), idx, dlg, G)
    ds_h = host(ds_g)[0]
    got = np.concatenate([ds_h[:, i, :i // 64].ravel() for i in range(S)])
    ref = np.concatenate([ds_rows[i].ravel() for i in range(S)])
    e_ds = rel_l2(got, ref) if ref.size else 0.0
    e_q, e_k = rel_l2(host(dWq_g), dWq_r), rel_l2(host(dWk_g), dWk_r)
    log(f"[selector bwd queries {label}] rel ds={e_ds:.3g} dWq={e_q:.3g} dWk={e_k:.3g}")
    assert max(e_ds, e_q, e_k) <= TOL_GRAD_REL
    return dWq_g, dWk_g


def rel_l2(x, ref):
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))


@pytest.mark.parametrize("S,Hq,Hkv,d,ds,k,dtype", [
    (64, 4, 1, 128, 128, 4, "bf16"), (100, 4, 1, 128, 128, 4, "bf16"),
    (1000, 8, 2, 128, 128, 3, "bf16"), (700, 16, 2, 64, 64, 6, "bf16"),
    (777, 2, 2, 64, 128, 5, "f32"), (640, 8, 1, 128, 64, 16, "bf16"), (1, 4, 1, 128, 128, 2, "bf16"),
    (333, 8, 2, 128, 128, 0, "bf16"), (900, 4, 4, 128, 128, 64, "bf16"),
])
def test_selector_bwd_queries_small(S, Hq, Hkv, d, ds, k, dtype):
    run_selector_queries_case(_problem(S, Hq, Hkv, d, ds, k, dtype=dtype, seed=S + 3 * Hq),
                              label=f"S={S}")


def test_selector_bwd_queries_from_attention_backward():
    run_selector_queries_case(_problem(640, 4, 1, 128, 128, 4, seed=17), dlg_from="attention",
                              label="end to end")


@pytest.mark.timeout(900)
def test_selector_bwd_queries_full_workload():
    """S = 16384 (Qwen3-4B head shape, k = 16): (1) with queries equal within
    each tile and every query carrying its tile's selection, the per-query
    selector gradients equal the tile rows' (sas_selector_bwd) with each
    tile's log-gate gradients summed over its queries; (2) ds of sampled rows
    against the oracle; (3) two runs give the same bits."""
    S_ = _sas()
    p = synth.make_problem(synth.WORKLOADS["qwen3_4b_prefill_16k"], seed=0)
    wl = p.wl
    S, Hkv, G, k = int(p.seq_lens[0]), wl.n_kv_heads, wl.group, wl.top_k
    n_tiles = S // 64
    q_tile = p.q.copy()
    for t in range(n_tiles):
        q_tile[:, :, 64 * t:64 * t + 64] = q_tile[:, :, 64 * t:64 * t + 1]
    Q, K = dev(q_tile), dev(p.K)
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    summ = S_.sas_block_summaries(K, torch.tensor([S], dtype=torch.int32).cuda(), Wk)
    idx_t, _, lse_t, _ = S_.sas_select(S_.SAS_SELECT_TILES, Q, None, Wq, summ, k, t_max=S)
    _, _, lse_q, _ = S_.sas_select(S_.SAS_SELECT_QUERIES, Q, None, Wq, summ, k, t_max=S)
    rng = np.random.default_rng(5)
    it = idx_t.cpu().numpy()
    tile_of = np.arange(S) // 64
    dlg_q = (rng.standard_normal((1, Hkv, S, k)) * 0.1 * (it[:, :, tile_of] >= 0)).astype(np.float32)
    dlg_t = dlg_q.reshape(1, Hkv, n_tiles, 64, k).sum(axis=3, dtype=np.float64).astype(np.float32)
    iq = idx_t[:, :, tile_of].contiguous()
    qWq, qWk, qds = S_.sas_selector_bwd_queries(Q, K, Wq, Wk, summ, iq, lse_q,
                                                torch.from_numpy(dlg_q).cuda(), want_ds=True)
    tWq, tWk, _ = S_.sas_selector_bwd(Q, K, Wq, summ, idx_t, lse_t, torch.from_numpy(dlg_t).cuda())
    torch.cuda.synchronize()
    e_q, e_k = rel_l2(host(qWq), host(tWq)), rel_l2(host(qWk), host(tWk))
    log(f"[selector bwd queries S=16384] per-query vs tile rows: rel dWq={e_q:.3g} dWk={e_k:.3g}")
    assert max(e_q, e_k) <= 1e-4
    # ds of sampled rows against the oracle's score gradient of those rows
    Qf, Kf = synth.to_f64(q_tile[0], "bf16"), synth.to_f64(p.K[0], "bf16")
    summ_f = O.block_summaries(Kf, S, p.f64("Wk_sel"))
    rows = [0, 64, 65, 1000, 4097, 9999, 16383]
    sc = O.query_scores(Qf, S, p.f64("Wq_sel"), summ_f, G, queries=rows)
    ds_h = host(qds)[0]
    iq_h = iq.cpu().numpy()[0]
    for i in rows:
        for r in range(Hkv):
            ref = O.score_grad(sc[i][r], iq_h[r, i], dlg_q[0, r, i].astype(np.float64))
            got = ds_h[r, i, :i // 64]
            if ref.size:
                assert rel_l2(got, ref) <= TOL_GRAD_REL, (i, r)
    # determinism
    qWq2, qWk2, _ = S_.sas_selector_bwd_queries(Q, K, Wq, Wk, summ, iq, lse_q,
                                                torch.from_numpy(dlg_q).cuda())
    torch.cuda.synchronize()
    assert torch.equal(qWq, qWq2) and torch.equal(qWk, qWk2)
