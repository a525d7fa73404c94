"""GPU parity of the selector backward (sas_selector_bwd) against the CPU
oracle's selector_backward, through the C ABI.

The GPU's own tile selection (sas_select) is the input of both sides, so the
check never depends on Top-K near-ties.  The log-gate gradients come either
from a seeded random draw (zero on empty slots, as sas_bwd leaves them) or,
end to end, from sas_bwd on the GPU against the oracle's prefill_backward.
Covered: both dtypes, d and d_sel of 64 and 128, G = 1..8, ragged sequence
ends, k = 0 and k >= C, the full S = 16384 training workload, and bitwise
run-to-run determinism."""
import math

import numpy as np
import pytest
import torch

from gated_block_sparse_amd import synth
from oracle import sas_oracle as O
from tests.gpu_util import TOL_GRAD_REL, dev, host, log, needs_gpu, rel_l2

pytestmark = [pytest.mark.gpu, needs_gpu]


def _sas():
    from gated_block_sparse_amd import binding
    return binding


def _problem(S, Hq=4, Hkv=1, d=128, ds=128, k=4, dtype="bf16", seed=0, t_max=None):
    wl = synth.custom_workload("prefill", n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, sel_dim=ds,
                               top_k=k, dtype=dtype, seq_len=S)
    return synth.make_problem(wl, seed, t_max=t_max)


def _random_dlg(idx_h, seed):
    rng = np.random.default_rng(seed)
    dlg = rng.standard_normal(idx_h.shape) * 0.1
    dlg[idx_h < 0] = 0.0
    return dlg


def run_case(p, dlg_from="random", label=""):
    S_ = _sas()
    wl = p.wl
    S, Hkv, G, k, dt = int(p.seq_lens[0]), wl.n_kv_heads, wl.group, wl.top_k, wl.dtype
    t_max = p.K.shape[2]
    log(f"[selector bwd {label}] S={S} Hq={wl.n_q_heads} Hkv={Hkv} d={wl.head_dim} "
        f"d_sel={wl.sel_dim} k={k} {dt} t_max={t_max}")
    Q, K, V = dev(p.q), dev(p.K), dev(p.V)
    lens = torch.tensor([S], dtype=torch.int32, device="cuda")
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    summ = S_.sas_block_summaries(K, lens, Wk)
    idx_g, lg_g, slse_g, _ = S_.sas_select(S_.SAS_SELECT_TILES, Q, None, Wq, summ, k,
                                           t_max=t_max)
    idx_h = idx_g.cpu().numpy().astype(np.int64)[0]
    Qf, Kf = synth.to_f64(p.q[0], dt), synth.to_f64(p.K[0], dt)
    if dlg_from == "random":
        dlg_h = _random_dlg(idx_h, seed=S + k)
        dlg_g = torch.from_numpy(dlg_h[None].astype(np.float32)).cuda()
        dlg_ref = dlg_h
    else:  # the attention backward on both sides
        dO = dev(p.dO)
        O_g, lse_g = S_.sas_prefill_fwd(Q, K, V, idx_g, lg_g)
        dlg_g = S_.sas_bwd(Q, K, V, O_g, dO, lse_g, idx_g, lg_g)[3]
        Vf, dOf = synth.to_f64(p.V[0], dt), synth.to_f64(p.dO[0], dt)
        lg_h = host(lg_g)[0]
        dlg_ref = O.prefill_backward(Qf, Kf, Vf, dOf, S, idx_h, lg_h, 1.0 / math.sqrt(wl.head_dim),
                                     G)[3]
    dWq_g, dWk_g, ds_g = S_.sas_selector_bwd(Q, K, Wq, summ, idx_g, slse_g, dlg_g, want_ds=True)
    torch.cuda.synchronize()
    ds_rows, dWq_r, dWk_r = O.selector_backward(Qf, Kf, S, p.f64("Wq_sel"), p.f64("Wk_sel"),
                                                idx_h, dlg_ref, G)
    ds_h = host(ds_g)[0]
    n_tiles = len(ds_rows)
    got = np.concatenate([ds_h[:, t, :t].ravel() for t in range(n_tiles)])
    ref = np.concatenate([ds_rows[t].ravel() for t in range(n_tiles)])
    e_ds = rel_l2(got, ref) if ref.size else 0.0
    e_q, e_k = rel_l2(host(dWq_g), dWq_r), rel_l2(host(dWk_g), dWk_r)
    log(f"[selector bwd {label}] rel ds={e_ds:.3g} dWq={e_q:.3g} dWk={e_k:.3g}")
    assert max(e_ds, e_q, e_k) <= TOL_GRAD_REL
    # every row's ds sums to zero (the gate's normaliser): a property at any size
    for t in range(1, n_tiles):
        row = ds_h[:, t, :t]
        assert np.abs(row.sum(axis=1)).max() <= 1e-4 * max(1.0, np.abs(row).sum(axis=1).max())
    return dWq_g, dWk_g, ds_g


@pytest.mark.parametrize("S,Hq,Hkv,d,ds,k,dtype", [
    (64, 4, 1, 128, 128, 4, "bf16"), (100, 4, 1, 128, 128, 4, "bf16"),
    (1000, 8, 2, 128, 128, 3, "bf16"), (2048, 8, 2, 128, 64, 16, "bf16"),
    (777, 2, 2, 64, 128, 5, "f32"), (700, 16, 2, 64, 64, 6, "bf16"),
    (1, 4, 1, 128, 128, 2, "bf16"), (333, 8, 2, 128, 128, 0, "f32"),
    (450, 4, 4, 64, 64, 64, "bf16"),
])
def test_selector_bwd_small(S, Hq, Hkv, d, ds, k, dtype):
    run_case(_problem(S, Hq, Hkv, d, ds, k, dtype, seed=S + Hq), label=f"S={S}")


def test_selector_bwd_ragged_tmax():
    """K/V rows beyond the sequence (t_max > S) are never read."""
    run_case(_problem(900, 8, 2, 128, 128, 8, "bf16", seed=5, t_max=2000), label="t_max>S")


@pytest.mark.parametrize("S,Hq,Hkv,d,k", [(640, 4, 1, 128, 4), (1300, 8, 2, 64, 7)])
def test_selector_bwd_from_attention_backward(S, Hq, Hkv, d, k):
    run_case(_problem(S, Hq, Hkv, d, 128, k, "bf16", seed=S), dlg_from="bwd", label=f"e2e S={S}")


@pytest.mark.timeout(900)
def test_selector_bwd_full_workload():
    p = synth.make_problem(synth.WORKLOADS["qwen3_4b_prefill_16k"], seed=0)
    run_case(p, label="qwen3_4b_prefill_16k")


def test_selector_bwd_deterministic():
    S_ = _sas()
    p = _problem(3000, 8, 2, 128, 128, 16, "bf16", seed=9)
    S = 3000
    Q, K = dev(p.q), dev(p.K)
    lens = torch.tensor([S], dtype=torch.int32, device="cuda")
    Wq, Wk = dev(p.Wq_sel), dev(p.Wk_sel)
    summ = S_.sas_block_summaries(K, lens, Wk)
    idx, lg, slse, _ = S_.sas_select(S_.SAS_SELECT_TILES, Q, None, Wq, summ, 16, t_max=S)
    dlg = torch.from_numpy(_random_dlg(idx.cpu().numpy(), 1).astype(np.float32)).cuda()
    a = S_.sas_selector_bwd(Q, K, Wq, summ, idx, slse, dlg, want_ds=True)
    b = S_.sas_selector_bwd(Q, K, Wq, summ, idx, slse, dlg, want_ds=True)
    for x, y in zip(a, b):
        assert torch.equal(torch.nan_to_num(x, nan=0.0), torch.nan_to_num(y, nan=0.0))
