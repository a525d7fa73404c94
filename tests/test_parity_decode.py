"""GPU parity of the decode path against the CPU oracle, through the C ABI:
sas_block_summaries -> sas_select(DECODE) -> sas_decode_fwd, and the fused
sas_decode_step, which must reproduce the last two bit for bit.

Full-size workloads (tiny fp32 4K; Qwen3-4B shape at 64K; batch 8 at
32K-64K; 512K with planted blocks) plus a sweep of edge cases: contexts of
1, 63, 64, 65, 129, 4097 tokens, k = 0, 1, C-1, C, C+5, varied batch lengths,
group sizes, head dims and dtypes, a t_max that is not a multiple of 64, and
bitwise run-to-run determinism.

The attention stage is always fed the ORACLE's selection, so its check never
depends on the GPU's Top-K; the end-to-end check then uses the GPU's own
selection on rows whose indices matched the oracle exactly."""
import dataclasses
import math

import numpy as np
import pytest
import torch

from gated_block_sparse_amd import synth
from oracle import sas_oracle as O
from tests.gpu_util import (GAP_TIE, TOL_F32_OUT, TOL_OUT, check_selection_row, dev, host,
                            idx_dev, lg_dev, log, needs_gpu)

pytestmark = [pytest.mark.gpu, needs_gpu]


def _sas():
    from gated_block_sparse_amd import binding
    return binding


def oracle_decode(p: synth.Problem, gated=True, sel=None):
    """Runs the oracle stage by stage, one (sequence, group) at a time, in float64."""
    wl = p.wl
    B, Hq, Hkv, d, k = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    Wq, Wk = p.f64("Wq_sel"), p.f64("Wk_sel")
    out = {"summ": [], "scores": [], "idx": np.full((B, Hkv, k), -1, np.int64),
           "lg": np.full((B, Hkv, k), -np.inf), "slse": np.zeros((B, Hkv)),
           "gap": np.zeros((B, Hkv)), "o": np.zeros((B, Hq, d)), "lse": np.zeros((B, Hq))}
    for b in range(B):
        T = int(p.seq_lens[b])
        q = synth.to_f64(p.q[b], wl.dtype)
        summ_b, scores_b = [], []
        for r in range(Hkv):
            Kr = synth.to_f64(p.K[b, r:r + 1, :T], wl.dtype)
            Vr = synth.to_f64(p.V[b, r:r + 1, :T], wl.dtype)
            summ = O.block_summaries(Kr, T, Wk)
            qg = q[r * G:(r + 1) * G]
            s = O.decode_scores(qg, Wq, summ, G)[0]
            idx, lg, slse, gap = O.select_rows([s], k)
            if sel is not None:
                idx, lg = sel[0][b, r][None], sel[1][b, r][None]
            o, lse = O.decode_attend(qg, Kr, Vr, T, idx, lg, scale, G, gated=gated)
            out["idx"][b, r], out["lg"][b, r] = idx[0], lg[0]
            out["slse"][b, r], out["gap"][b, r] = slse[0], gap[0]
            out["o"][b, r * G:(r + 1) * G], out["lse"][b, r * G:(r + 1) * G] = o, lse
            summ_b.append(summ[0])
            scores_b.append(s)
        out["summ"].append(summ_b)
        out["scores"].append(scores_b)
    return out


def run_decode_case(p: synth.Problem, t_max=None, check_e2e=True, label=""):
    S = _sas()
    wl = p.wl
    B, Hq, Hkv, d, k = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.top_k
    tol_o, tol_f = TOL_OUT[wl.dtype], TOL_F32_OUT[wl.dtype]
    log(f"[decode {label}] B={B} Hq={Hq} Hkv={Hkv} d={d} k={k} dtype={wl.dtype} "
        f"lens={p.seq_lens.tolist()[:8]} t_max={p.K.shape[2]}")
    q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.from_numpy(p.seq_lens).cuda()
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)

    summ = S.sas_block_summaries(K, lens, Wk)
    idx_g, lg_g, slse_g, sc_g = S.sas_select(S.SAS_SELECT_DECODE, q, lens, Wq, summ, k,
                                             want_scores=True)
    torch.cuda.synchronize()
    ref = oracle_decode(p)
    summ_h, sc_h = host(summ), host(sc_g)
    idx_h, lg_h, slse_h = idx_g.cpu().numpy(), host(lg_g), host(slse_g)
    exact_rows = np.zeros((B, Hkv), bool)
    for b in range(B):
        C = O.n_history_blocks(int(p.seq_lens[b]))
        for r in range(Hkv):
            if C:
                err = np.abs(summ_h[b, r, :C] - ref["summ"][b][r]).max()
                assert err <= 1e-5, f"summaries b={b} r={r}: {err}"
                err = np.abs(sc_h[b, r, 0, :C] - ref["scores"][b][r]).max()
                assert err <= tol_f, f"scores b={b} r={r}: {err}"
                assert abs(slse_h[b, r, 0] - ref["slse"][b, r]) <= tol_f
            else:
                assert np.isneginf(slse_h[b, r, 0])
            exact_rows[b, r] = check_selection_row(
                idx_h[b, r, 0], lg_h[b, r, 0], ref["scores"][b][r], ref["idx"][b, r],
                ref["gap"][b, r], k, ref["slse"][b, r], tol_f)

    # the fused step reproduces select + decode_fwd bit for bit (gated and ungated)
    for gated in (True, False):
        idx_f, lg_f, slse_f, o_f, lse_f = S.sas_decode_step(q, K, V, lens, Wq, summ, k,
                                                            gated=gated)
        o_r, lse_r = S.sas_decode_fwd(q, K, V, lens, idx_g, lg_g if gated else None)
        torch.cuda.synchronize()
        assert torch.equal(idx_f, idx_g) and torch.equal(lg_f, lg_g), label
        assert torch.equal(slse_f, slse_g), label
        assert torch.equal(o_f, o_r) and torch.equal(lse_f, lse_r), (label, gated)

    # the step with its fused refresh: summ starts with every newest complete
    # block's summary spoiled, and must end equal to sas_block_summaries' bits
    # with the same selection and attention as before
    summ_s = summ.clone()
    for b in range(B):
        C = O.n_history_blocks(int(p.seq_lens[b]))
        if C:
            summ_s[b, :, C - 1] = 1e3
    idx_f, lg_f, slse_f, o_f, lse_f = S.sas_decode_step(q, K, V, lens, Wq, summ_s, k, Wk_sel=Wk)
    o_r, lse_r = S.sas_decode_fwd(q, K, V, lens, idx_g, lg_g)
    torch.cuda.synchronize()
    assert torch.equal(summ_s, summ), label
    assert torch.equal(idx_f, idx_g) and torch.equal(lg_f, lg_g), label
    assert torch.equal(slse_f, slse_g), label
    assert torch.equal(o_f, o_r) and torch.equal(lse_f, lse_r), label

    # attention on the oracle's selection
    oidx, olg = idx_dev(ref["idx"][:, :, None]), lg_dev(ref["lg"][:, :, None])
    o, lse = S.sas_decode_fwd(q, K, V, lens, oidx, olg)
    o_h, lse_h = host(o), host(lse)
    err_o = np.abs(o_h - ref["o"]).max()
    err_l = np.abs(lse_h - ref["lse"]).max()
    log(f"[decode {label}] max|o-o_ref|={err_o:.3g} max|lse-lse_ref|={err_l:.3g} "
        f"exact rows {exact_rows.sum()}/{exact_rows.size}")
    assert err_o <= tol_o and err_l <= tol_f

    # ungated inference rule on the same selection
    o_u, lse_u = S.sas_decode_fwd(q, K, V, lens, oidx, None)
    ref_u = oracle_decode(p, gated=False, sel=(ref["idx"], ref["lg"]))
    assert np.abs(host(o_u) - ref_u["o"]).max() <= tol_o
    assert np.abs(host(lse_u) - ref_u["lse"]).max() <= tol_f

    if check_e2e:
        o_e, _ = S.sas_decode_fwd(q, K, V, lens, idx_g, lg_g)
        o_eh = host(o_e)
        G = Hq // Hkv
        for b in range(B):
            for r in range(Hkv):
                if exact_rows[b, r]:
                    e = np.abs(o_eh[b, r * G:(r + 1) * G] - ref["o"][b, r * G:(r + 1) * G]).max()
                    assert e <= tol_o, (b, r, e)
    return exact_rows


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_f32_decode_4k", "qwen3_4b_decode_64k",
                                  "qwen3_4b_decode_b8_32k_64k", "qwen3_4b_decode_512k"])
def test_decode_workload(name):
    p = synth.make_problem(synth.WORKLOADS[name], seed=0)
    exact = run_decode_case(p, label=name)
    assert exact.mean() >= 0.5


def test_planted_blocks_recalled_on_gpu():
    """512K-style plant at a smaller size with identity selector projections:
    every selected block must be a planted one."""
    S = _sas()
    wl = synth.custom_workload("decode", n_q_heads=8, n_kv_heads=2, head_dim=128, sel_dim=128,
                               top_k=16, dtype="bf16", seq_len=64 * 2000 + 7, plant_frac=0.02)
    p = synth.make_problem(wl, 0)
    eye = torch.eye(128, dtype=torch.float32).cuda()
    lens = torch.from_numpy(p.seq_lens).cuda()
    summ = S.sas_block_summaries(dev(p.K), lens, eye)
    idx, _, _, _ = S.sas_select(S.SAS_SELECT_DECODE, dev(p.q), lens, eye, summ, 16)
    idx = idx.cpu().numpy()
    for r in range(2):
        assert p.planted[0, r, idx[0, r, 0]].all()


EDGE_T = [1, 63, 64, 65, 129, 4097]


def _edge_problem(T, k, dtype="f32", Hq=4, Hkv=2, d=64, ds=64, batch=1, lens=None,
                  t_max=None, seed=0):
    wl = synth.custom_workload("decode", batch=batch, n_q_heads=Hq, n_kv_heads=Hkv,
                               head_dim=d, sel_dim=ds, top_k=k, dtype=dtype, seq_len=T)
    return synth.make_problem(wl, seed, seq_lens=lens, t_max=t_max)


@pytest.mark.parametrize("T", EDGE_T)
def test_decode_edge_lengths_and_k(T):
    C = O.n_history_blocks(T)
    for k in sorted({0, 1, max(C - 1, 0), C, C + 5}):
        if k > 64:
            continue
        run_decode_case(_edge_problem(T, k, seed=T + k), label=f"T={T} k={k}")


@pytest.mark.parametrize("dtype,d,ds,Hq,Hkv", [
    ("bf16", 128, 128, 32, 8), ("bf16", 64, 128, 8, 8), ("bf16", 128, 64, 16, 2),
    ("f32", 128, 128, 8, 1), ("f32", 64, 64, 16, 8), ("bf16", 64, 64, 2, 2),
])
def test_decode_shapes(dtype, d, ds, Hq, Hkv):
    run_decode_case(_edge_problem(3000, 7, dtype=dtype, Hq=Hq, Hkv=Hkv, d=d, ds=ds, seed=d + Hq),
                    label=f"{dtype} d={d} ds={ds} Hq={Hq} Hkv={Hkv}")


def test_decode_varlen_batch_and_ragged_tmax():
    lens = [1, 65, 700, 128, 699, 64]
    p = _edge_problem(700, 5, dtype="bf16", Hq=8, Hkv=2, d=128, ds=128, batch=6, lens=lens,
                      t_max=700)
    run_decode_case(p, label="varlen")


@pytest.mark.parametrize("k", [7, 8])
def test_decode_two_blocks_per_unit_ragged(k):
    """Grids of at least 1024 (sequence, group, slot) units take two blocks per
    split workgroup: cover an odd and an even slot count, empty history slots
    (C < k) and single-token B0s."""
    lens = [1, 64, 65, 130, 300, 511, 512, 513, 700, 1000, 2049, 3000, 4000, 4095, 4096, 4097]
    p = _edge_problem(4097, k, dtype="bf16", Hq=32, Hkv=8, d=128, ds=128, batch=16, lens=lens,
                      seed=100 + k)
    run_decode_case(p, label=f"two-block units k={k}")


@pytest.mark.parametrize("T,k", [(64 * 200 + 3, 64), (64 * 3000 + 17, 64), (64 * 9000 + 1, 32),
                                 (64 * 3000 + 17, 16)])
def test_decode_large_k_and_many_chunks(T, k):
    """Rows of many selection chunks; the chunk length follows the grid and
    k (two groups here): 64 blocks for the first case, 256 for the second and
    third, 128 for the last."""
    run_decode_case(_edge_problem(T, k, dtype="bf16", Hq=8, Hkv=2, d=128, ds=128, seed=T),
                    label=f"T={T} k={k}")


def test_decode_deterministic():
    S = _sas()
    p = _edge_problem(20000, 16, dtype="bf16", Hq=32, Hkv=8, d=128, ds=128)
    q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.from_numpy(p.seq_lens).cuda()
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    outs = []
    for _ in range(2):
        summ = S.sas_block_summaries(K, lens, Wk)
        idx, lg, slse, _ = S.sas_select(S.SAS_SELECT_DECODE, q, lens, Wq, summ, 16)
        o, lse = S.sas_decode_fwd(q, K, V, lens, idx, lg)
        outs.append([t.clone() for t in (summ, idx, lg, slse, o, lse)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,T,k", [(1, 20000, 16), (8, 40000, 32)])
def test_decode_step_reused_workspace(B, T, k):
    """The fused step's merge counts arrivals per row in its workspace: one
    workspace filled with junk bytes, then reused by several steps in a row
    (the last one on a shorter batch), gives select + decode_fwd's bits each
    time.  Covers the one-block and two-block split units."""
    S = _sas()
    wl = synth.custom_workload("decode", batch=B, n_q_heads=32, n_kv_heads=8, head_dim=128,
                               sel_dim=128, top_k=k, dtype="bf16", seq_len=T,
                               seq_len_range=(T // 2, T) if B > 1 else None)
    p = synth.make_problem(wl, 5 + B)
    q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.from_numpy(p.seq_lens).cuda()
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    summ = S.sas_block_summaries(K, lens, Wk)
    dims = S.make_dims(B, 32, 8, 128, 128, k, K.shape[2], S.SAS_BF16)
    ws = torch.randint(0, 256, (S.sas_workspace_bytes(S.SAS_OP_DECODE_STEP, dims),),
                       dtype=torch.uint8, device="cuda")
    for rep, nb in enumerate((B, B, max(1, B // 2))):
        qq, KK, VV, ll, ss = q[:nb], K[:nb], V[:nb], lens[:nb], summ[:nb]
        idx_g, lg_g, slse_g, _ = S.sas_select(S.SAS_SELECT_DECODE, qq, ll, Wq, ss, k)
        o_r, lse_r = S.sas_decode_fwd(qq, KK, VV, ll, idx_g, lg_g)
        idx_f, lg_f, slse_f, o_f, lse_f = S.sas_decode_step(qq, KK, VV, ll, Wq, ss, k, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(idx_f, idx_g) and torch.equal(lg_f, lg_g), rep
        assert torch.equal(o_f, o_r) and torch.equal(lse_f, lse_r), rep


@pytest.mark.parametrize("B,T,k", [(1, 20000, 16), (8, 40000, 32)])
def test_decode_step_graph_replays(B, T, k):
    """The fused step captured in a HIP graph and replayed several times, with
    eager work (outputs spoiled) and synchronisations between the replays:
    every replay gives the eager step's bits.  The merge's arrival counts are
    reset by a kernel of the step itself (no memset node in the graph)."""
    S = _sas()
    wl = synth.custom_workload("decode", batch=B, n_q_heads=32, n_kv_heads=8, head_dim=128,
                               sel_dim=128, top_k=k, dtype="bf16", seq_len=T,
                               seq_len_range=(T // 2, T) if B > 1 else None)
    p = synth.make_problem(wl, 9 + B)
    q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.from_numpy(p.seq_lens).cuda()
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    summ = S.sas_block_summaries(K, lens, Wk)
    ref = [t.clone() for t in S.sas_decode_step(q, K, V, lens, Wq, summ, k)]
    dims = S.make_dims(B, 32, 8, 128, 128, k, K.shape[2], S.SAS_BF16)
    ws = torch.empty(S.sas_workspace_bytes(S.SAS_OP_DECODE_STEP, dims), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty_like(t) for t in ref]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g.capture_begin()
        S.sas_decode_step(q, K, V, lens, Wq, summ, k, idx=outs[0], log_gate=outs[1],
                          score_lse=outs[2], o=outs[3], lse=outs[4], ws=ws)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(-3)
        ws.fill_(rep + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("idx", "log_gate", "score_lse", "o", "lse"), ref, outs):
            assert torch.equal(a, b), (rep, name)


def test_block_summaries_range_leaves_other_rows():
    """Refreshing one block range writes exactly those rows."""
    S = _sas()
    p = _edge_problem(64 * 20 + 1, 4, dtype="bf16", Hq=8, Hkv=2, d=128, ds=128)
    K, lens, Wk = dev(p.K), torch.from_numpy(p.seq_lens).cuda(), dev(p.Wk_sel)
    full = S.sas_block_summaries(K, lens, Wk)
    part = torch.full_like(full, 7.0)
    S.sas_block_summaries(K, lens, Wk, blk_begin=5, blk_end=9, summ=part)
    torch.cuda.synchronize()
    assert torch.equal(part[:, :, 5:9], full[:, :, 5:9])
    assert (part[:, :, :5] == 7.0).all() and (part[:, :, 9:] == 7.0).all()
