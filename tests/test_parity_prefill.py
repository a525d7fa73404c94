"""GPU parity of the prefill path against the CPU oracle, through the C ABI:
sas_block_summaries -> sas_select(TILES) -> sas_prefill_fwd (-> sas_bwd).

Small shapes are checked on every tile; the full training-style workload
(S=16384, Qwen3-4B head shape, per-tile k=16) is checked on sampled tiles
(first, last, around the k boundary and in the middle).  The attention stage
gets a selection that does not come from the GPU: the oracle's own Top-K on
small shapes, a seeded random valid selection at full size.  Also covered: a
sink-heavy selection (hot-block chunking of the dK/dV pass), two sequences in
one call, the largest k (64) and the largest sequence (1024 tiles, sampled)."""
import math

import numpy as np
import pytest
import torch

from gated_block_sparse_amd import synth
from oracle import sas_oracle as O
from tests.gpu_util import (TOL_GRAD_REL, TOL_OUT, check_selection_row, dev, host, idx_dev,
                            lg_dev, log, needs_gpu)

pytestmark = [pytest.mark.gpu, needs_gpu]
TOL_LSE = 1e-3


def _sas():
    from gated_block_sparse_amd import binding
    return binding


def _problem(S, Hq=4, Hkv=1, d=128, ds=128, k=4, seed=0):
    wl = synth.custom_workload("prefill", n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, sel_dim=ds,
                               top_k=k, dtype="bf16", seq_len=S)
    return synth.make_problem(wl, seed)


def random_selection(rng, Hkv, n_tiles, k):
    """A seeded valid per-tile selection (ascending, -1 padded) with log g < 0."""
    idx = np.full((Hkv, n_tiles, k), -1, np.int64)
    lg = np.full((Hkv, n_tiles, k), -np.inf)
    for r in range(Hkv):
        for t in range(n_tiles):
            n = min(k, t)
            if n:
                ch = np.sort(rng.choice(t, size=n, replace=False))
                idx[r, t, :n] = ch
                lg[r, t, :n] = -rng.uniform(0.5, 8.0, size=n)
    return idx, lg


def sink_selection(rng, Hkv, n_tiles, k):
    """Like random_selection, but every tile that can selects blocks 0 and 1
    (sink-heavy: those blocks are read by every tile)."""
    idx = np.full((Hkv, n_tiles, k), -1, np.int64)
    lg = np.full((Hkv, n_tiles, k), -np.inf)
    for r in range(Hkv):
        for t in range(n_tiles):
            n = min(k, t)
            if n:
                sinks = [m for m in (0, 1) if m < t][:n]
                rest = rng.choice(np.arange(len(sinks), t), size=n - len(sinks), replace=False)
                ch = np.sort(np.concatenate([sinks, rest]).astype(np.int64))
                idx[r, t, :n] = ch
                lg[r, t, :n] = -rng.uniform(0.5, 8.0, size=n)
    return idx, lg


def check_select_tiles(p, summ_g, tiles):
    """GPU per-tile selection vs the oracle on the given tiles."""
    S_ = _sas()
    wl = p.wl
    S, Hkv, G, k = int(p.seq_lens[0]), wl.n_kv_heads, wl.group, wl.top_k
    Q = dev(p.q)
    idx_g, lg_g, slse_g, sc_g = S_.sas_select(S_.SAS_SELECT_TILES, Q, None, dev(p.Wq_sel), summ_g, k,
                                              t_max=p.K.shape[2], want_scores=True)
    idx_h, lg_h, slse_h, sc_h = idx_g.cpu().numpy(), host(lg_g), host(slse_g), host(sc_g)
    Qf, Kf = synth.to_f64(p.q[0], "bf16"), synth.to_f64(p.K[0], "bf16")
    summ = O.block_summaries(Kf, S, p.f64("Wk_sel"))
    rows = O.tile_scores(Qf, S, p.f64("Wq_sel"), summ, G, tiles=set(tiles))
    n_exact = 0
    for t in tiles:
        for r in range(Hkv):
            s = rows[t][r]
            lse_r, _ = O.gate(s)
            oidx, gap = O.topk(s, k)
            if t:
                assert np.abs(sc_h[0, r, t, :t] - s).max() <= 1e-4
                assert abs(slse_h[0, r, t] - lse_r) <= 1e-4
            else:
                assert np.isneginf(slse_h[0, r, t])
            n_exact += check_selection_row(idx_h[0, r, t], lg_h[0, r, t], s,
                                           np.asarray(oidx + [-1] * (k - len(oidx))), gap, k,
                                           lse_r, 1e-4)
    return idx_g, lg_g, n_exact


def run_prefill_case(p, tiles=None, selection="oracle", gated=True, label=""):
    S_ = _sas()
    wl = p.wl
    S, Hq, Hkv, d, k, G = int(p.seq_lens[0]), wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k, wl.group
    n_tiles = -(-S // 64)
    tiles = list(range(n_tiles)) if tiles is None else tiles
    log(f"[prefill {label}] S={S} Hq={Hq} Hkv={Hkv} d={d} k={k} tiles={tiles[:6]}...")
    Q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.tensor([S], dtype=torch.int32).cuda()
    summ_g = S_.sas_block_summaries(K, lens, dev(p.Wk_sel))
    idx_g, lg_g, n_exact = check_select_tiles(p, summ_g, tiles)
    log(f"[prefill {label}] tile selection exact on {n_exact}/{len(tiles) * Hkv} rows")

    Qf, Kf, Vf = (synth.to_f64(x[0], "bf16") for x in (p.q, p.K, p.V))
    if selection == "oracle":
        sel = O.prefill_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
        idx, lg = sel["idx"], sel["log_gate"]
    elif selection == "sink":
        idx, lg = sink_selection(np.random.default_rng(4321), Hkv, n_tiles, k)
    else:
        idx, lg = random_selection(np.random.default_rng(1234), Hkv, n_tiles, k)
    scale = 1.0 / math.sqrt(d)
    O_g, lse_g = S_.sas_prefill_fwd(Q, K, V, idx_dev(idx[None]), lg_dev(lg[None]) if gated else None)
    Or, lser = O.prefill_attend(Qf, Kf, Vf, S, idx, lg, scale, G, gated=gated, tiles=tiles)
    O_h, lse_h = host(O_g)[0], host(lse_g)[0]
    rows = np.concatenate([np.arange(64 * t, min(64 * t + 64, S)) for t in tiles])
    err_o = np.abs(O_h[:, rows] - Or[:, rows]).max()
    err_l = np.abs(lse_h[:, rows] - lser[:, rows]).max()
    log(f"[prefill {label}] max|O-O_ref|={err_o:.3g} max|lse-lse_ref|={err_l:.3g}")
    assert err_o <= TOL_OUT["bf16"], err_o
    assert err_l <= TOL_LSE, err_l
    return dict(Q=Q, K=K, V=V, O=O_g, lse=lse_g, idx=idx, lg=lg, Qf=Qf, Kf=Kf, Vf=Vf, rows=rows,
                tiles=tiles)


@pytest.mark.parametrize("S,Hq,Hkv,d,k", [
    (64, 4, 1, 128, 4), (100, 4, 1, 128, 4), (1000, 8, 2, 128, 3), (2048, 8, 2, 128, 16),
    (777, 2, 2, 64, 5), (640, 8, 1, 128, 4), (700, 16, 2, 64, 6), (1, 4, 1, 128, 2),
])
def test_prefill_small(S, Hq, Hkv, d, k):
    run_prefill_case(_problem(S, Hq, Hkv, d, 128, k, seed=S + Hq), label=f"S={S}")


def test_prefill_ungated_and_k0():
    run_prefill_case(_problem(500, 8, 2, 128, 128, 4, seed=3), gated=False, label="ungated")
    run_prefill_case(_problem(333, 8, 2, 128, 128, 0, seed=4), label="k=0")


@pytest.mark.timeout(900)
def test_prefill_full_workload_sampled_tiles():
    p = synth.make_problem(synth.WORKLOADS["qwen3_4b_prefill_16k"], seed=0)
    run_prefill_case(p, tiles=[0, 1, 2, 15, 16, 17, 100, 200, 254, 255], selection="random",
                     label="qwen3_4b_prefill_16k")


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def run_bwd_case(p, ctx, exact_blocks=None, label=""):
    """sas_bwd on the forward's outputs vs prefill_backward of the oracle.

    ctx: what run_prefill_case returned.  With sampled tiles, dQ and dlog_gate
    are compared on those tiles and dK/dV on `exact_blocks` (blocks whose every
    reader is a sampled tile); otherwise everything is compared."""
    S_ = _sas()
    wl = p.wl
    S, Hq, Hkv, d, k, G = int(p.seq_lens[0]), wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k, wl.group
    n_tiles = -(-S // 64)
    idx, lg, tiles = ctx["idx"], ctx["lg"], ctx["tiles"]
    full = len(tiles) == n_tiles
    dO = dev(p.dO)
    dQ, dK, dV, dlg = S_.sas_bwd(ctx["Q"], ctx["K"], ctx["V"], ctx["O"], dO, ctx["lse"],
                                 idx_dev(idx[None]), lg_dev(lg[None]))
    dOf = synth.to_f64(p.dO[0], "bf16")
    scale = 1.0 / math.sqrt(d)
    rQ, rK, rV, rlg = O.prefill_backward(ctx["Qf"], ctx["Kf"], ctx["Vf"], dOf, S, idx, lg, scale,
                                         G, tiles=None if full else tiles)
    gQ, gK, gV, glg = host(dQ)[0], host(dK)[0][:, :S], host(dV)[0][:, :S], host(dlg)[0]
    rows = ctx["rows"]
    # relative L2 per tensor; the floor keeps an exactly-zero reference (one
    # query and one key: dQ = dK = 0) from dividing by zero
    floor = 1e-2 * np.linalg.norm(dOf[:, rows])

    def rel_l2(x, ref):
        return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), floor))

    e_q = rel_l2(gQ[:, rows], rQ[:, rows])
    sel = np.zeros_like(idx, bool)
    sel[:, tiles] = True
    valid = (idx >= 0) & sel
    e_lg = 0.0
    if valid.any():   # the log-gate gradient has no zero-reference case: plain relative L2
        e_lg = float(np.linalg.norm(glg[valid] - rlg[valid]) / max(np.linalg.norm(rlg[valid]), 1e-30))
    assert (glg[idx < 0] == 0).all()
    if full:
        kv_rows = np.arange(S)
    else:
        kv_rows = np.concatenate([np.arange(64 * m, min(64 * m + 64, S)) for m in exact_blocks])
    e_k = rel_l2(gK[:, kv_rows], rK[:, kv_rows])
    e_v = rel_l2(gV[:, kv_rows], rV[:, kv_rows])
    log(f"[bwd {label}] rel dQ={e_q:.3g} dK={e_k:.3g} dV={e_v:.3g} dlog_gate={e_lg:.3g}")
    assert max(e_q, e_k, e_v, e_lg) <= TOL_GRAD_REL
    # identities that hold at any size: sum_j dV_j = sum over the group's rows of dO,
    # sum_j dK_j = 0 (a shift of every key leaves each softmax row unchanged)
    for r in range(Hkv):
        sv = gV[r].sum(axis=0)
        so = dOf[r * G:(r + 1) * G].sum(axis=(0, 1))
        assert np.linalg.norm(sv - so) <= TOL_GRAD_REL * max(np.linalg.norm(so), floor)
        assert np.linalg.norm(gK[r].sum(axis=0)) <= TOL_GRAD_REL * np.linalg.norm(gK[r]) + 1e-3


@pytest.mark.parametrize("S,Hq,Hkv,d,k", [
    (64, 4, 1, 128, 4), (100, 4, 1, 128, 4), (1000, 8, 2, 128, 3), (2048, 8, 2, 128, 16),
    (777, 2, 2, 64, 5), (700, 16, 2, 64, 6), (1, 4, 1, 128, 2), (333, 8, 2, 128, 0),
    (500, 2, 2, 128, 5), (300, 4, 2, 128, 3), (640, 8, 1, 128, 4), (129, 16, 2, 128, 2),
])
def test_bwd_small(S, Hq, Hkv, d, k):
    p = _problem(S, Hq, Hkv, d, 128, k, seed=S + 7 * Hq)
    ctx = run_prefill_case(p, label=f"S={S}")
    run_bwd_case(p, ctx, label=f"S={S}")


@pytest.mark.timeout(900)
def test_bwd_full_workload_sampled_tiles():
    p = synth.make_problem(synth.WORKLOADS["qwen3_4b_prefill_16k"], seed=0)
    ctx = run_prefill_case(p, tiles=[0, 1, 2, 15, 16, 17, 100, 200, 253, 254, 255],
                           selection="random", label="qwen3_4b_prefill_16k")
    run_bwd_case(p, ctx, exact_blocks=[253, 254, 255], label="qwen3_4b_prefill_16k")


def test_bwd_hot_blocks_split():
    """Sink-heavy selection: blocks 0 and 1 are read by all 200 tiles, so for
    d = 128 the dK/dV pass splits them into chunks of reading tiles whose
    fp32 partials are summed by the reduction kernel; everything is compared."""
    p = _problem(64 * 200, 8, 2, 128, 128, 8, seed=77)
    ctx = run_prefill_case(p, selection="sink", label="sink")
    run_bwd_case(p, ctx, label="sink")


def test_bwd_deterministic():
    S_ = _sas()
    p = _problem(1500, 8, 2, 128, 128, 6, seed=11)
    ctx = run_prefill_case(p, label="det")
    outs = []
    for _ in range(2):
        r = S_.sas_bwd(ctx["Q"], ctx["K"], ctx["V"], ctx["O"], dev(p.dO), ctx["lse"],
                       idx_dev(ctx["idx"][None]), lg_dev(ctx["lg"][None]))
        outs.append([x.clone() for x in r])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_prefill_batch2_fwd_bwd():
    """Two sequences in one call (grid z): each checked against the oracle run
    on its own, with the oracle's selection of that sequence."""
    S_ = _sas()
    S, Hq, Hkv, d, k = 700, 8, 2, 128, 5
    wl = synth.custom_workload("prefill", batch=2, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                               sel_dim=128, top_k=k, dtype="bf16", seq_len=S)
    p = synth.make_problem(wl, 31)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    Qd, Kd, Vd, dOd = dev(p.q), dev(p.K), dev(p.V), dev(p.dO)
    sels, refs = [], []
    for b in range(2):
        Qf, Kf, Vf, dOf = (synth.to_f64(x[b], "bf16") for x in (p.q, p.K, p.V, p.dO))
        sel = O.prefill_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
        sels.append(sel)
        Or, lser = O.prefill_attend(Qf, Kf, Vf, S, sel["idx"], sel["log_gate"], scale, G)
        gr = O.prefill_backward(Qf, Kf, Vf, dOf, S, sel["idx"], sel["log_gate"], scale, G)
        refs.append((Or, lser, gr))
    idx = idx_dev(np.stack([s["idx"] for s in sels]))
    lg = lg_dev(np.stack([s["log_gate"] for s in sels]))
    O_g, lse_g = S_.sas_prefill_fwd(Qd, Kd, Vd, idx, lg)
    dQ, dK, dV, dlg = S_.sas_bwd(Qd, Kd, Vd, O_g, dOd, lse_g, idx, lg)
    torch.cuda.synchronize()
    for b in range(2):
        Or, lser, (rQ, rK, rV, rlg) = refs[b]
        assert np.abs(host(O_g)[b] - Or).max() <= TOL_OUT["bf16"]
        for g, r in ((dQ, rQ), (dK, rK), (dV, rV)):
            x = host(g)[b][:, :S]
            assert np.linalg.norm(x - r) <= TOL_GRAD_REL * np.linalg.norm(r), b
        valid = sels[b]["idx"] >= 0
        e = np.linalg.norm(host(dlg)[b][valid] - rlg[valid]) / np.linalg.norm(rlg[valid])
        assert e <= TOL_GRAD_REL, (b, e)


@pytest.mark.parametrize("S,Hq,Hkv,d,k,B", [
    (1000, 32, 4, 64, 5, 3), (1000, 16, 4, 128, 6, 5), (1000, 8, 4, 128, 4, 5),
    (1000, 4, 4, 64, 3, 5),
])
def test_prefill_fwd_more_items_than_cus(S, Hq, Hkv, d, k, B):
    """More (tile, group, head chunk, sequence) items than the GPU has CUs, so
    the tile forward's workgroups each take several items in turn, ragged last
    tile and tile 0 (diagonal only) among them; every tile of every sequence
    against the oracle with the oracle's own selection."""
    S_ = _sas()
    G = Hq // Hkv
    n_items = -(-S // 64) * Hkv * B * max(1, G // 4)
    assert n_items > torch.cuda.get_device_properties(0).multi_processor_count
    wl = synth.custom_workload("prefill", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                               sel_dim=128, top_k=k, dtype="bf16", seq_len=S)
    p = synth.make_problem(wl, 17 + B)
    scale = 1.0 / math.sqrt(d)
    log(f"[prefill items] S={S} Hq={Hq} Hkv={Hkv} d={d} k={k} B={B} items={n_items}")
    sels, refs = [], []
    for b in range(B):
        Qf, Kf, Vf = (synth.to_f64(x[b], "bf16") for x in (p.q, p.K, p.V))
        sel = O.prefill_select(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"), k, G)
        sels.append(sel)
        refs.append(O.prefill_attend(Qf, Kf, Vf, S, sel["idx"], sel["log_gate"], scale, G))
    idx = idx_dev(np.stack([s["idx"] for s in sels]))
    lg = lg_dev(np.stack([s["log_gate"] for s in sels]))
    O_g, lse_g = S_.sas_prefill_fwd(dev(p.q), dev(p.K), dev(p.V), idx, lg)
    O_h, lse_h = host(O_g), host(lse_g)
    for b in range(B):
        Or, lser = refs[b]
        err_o = np.abs(O_h[b] - Or).max()
        err_l = np.abs(lse_h[b] - lser).max()
        assert err_o <= TOL_OUT["bf16"], (b, err_o)
        assert err_l <= TOL_LSE, (b, err_l)


def test_prefill_k64_fwd_bwd():
    """The largest k built (64): tiles past the 64th select 64 history blocks."""
    p = _problem(64 * 70 + 17, 4, 1, 128, 128, 64, seed=64)
    ctx = run_prefill_case(p, selection="random", label="k=64")
    run_bwd_case(p, ctx, label="k=64")


@pytest.mark.timeout(900)
def test_prefill_max_tiles_sampled():
    """The largest sequence the tile selector supports (1024 tiles, S = 65536),
    forward and backward on sampled tiles / exact blocks."""
    p = _problem(65536, 4, 1, 128, 128, 16, seed=65)
    ctx = run_prefill_case(p, tiles=[0, 1, 511, 1021, 1022, 1023], selection="random",
                           label="S=65536")
    run_bwd_case(p, ctx, exact_blocks=[1021, 1022, 1023], label="S=65536")
