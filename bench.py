#!/usr/bin/env python3
"""Benchmark of the SAS hot path on one MI355X (prints ONE JSON line).

Default workload: one decode step of one attention layer at the Qwen3-4B
attention shape (32 query heads, 8 KV heads, d=128, bf16 KV cache, fp32
accumulation), 64K context, block 64, top-k=16 + the current block, selector
dim 128, synthetic seeded inputs.  A step is the whole decode-time path, one
sas_decode_step call with Wk_sel given:

  1. the summary of the newest complete block (the steady-state refresh; it
     is due once every 64 steps, run here every step), fused into the
     selection's first kernel,
  2. selector score over every history-block summary, softmax-gate LSE,
     Top-K, then split-KV gated attention over the selected blocks + B0 and
     the LSE merge (the selection's final merge runs inside the attention's
     split kernel).

The same step is also timed through the separate entry points
(sas_block_summaries, sas_select, then sas_decode_fwd) for the per-op
breakdown; the two give identical outputs (checked before timing).  The
roofline figure is sas_decode_fwd's.

Inputs are resident in HBM before timing starts.  Each timed step is
bracketed by HIP events on the stream the library launches on; between steps
(outside the events) a 512 MiB write and a 1 GiB read sweep evict the L2s and
the 256 MB Infinity Cache, so every step reads its bytes from HBM.
``--workload qwen3_4b_prefill_16k`` times the training-style prefill forward,
backward and selector backward instead.

Extra fields beside the contract keys: ``breakdown_us`` (per-op medians),
``roofline`` for the dominant kernel, ``cpu_baseline`` (the float64 CPU
oracle on a bounded sample of the same step, timed on this host).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def _args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_4b_decode_64k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of the CPU oracle sample")
    ap.add_argument("--no-flush", action="store_true", help="hot-cache timing only")
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the hot-cache HIP-graph figure (profiling runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for PMC byte calibration)")
    return ap.parse_args()


DECODE_KERNELS = ("sas::decode_split_kernel", "sas::decode_merge_kernel")
PREFILL_KERNELS = ("sas::prefill_fwd_persistent_kernel<128, 4>",)   # the tile forward
# the sources those kernels are built from
DECODE_SOURCES = ("decode.hip", "sas_device.h", "sas_internal.h", "sas_select_dev.h")
PREFILL_SOURCES = ("prefill.hip", "sas_device.h", "sas_internal.h", "sas_mfma.h")


def measured_traffic(workload, prefixes, sources):
    """HBM bytes per launch of the roofline kernel(s), from the committed
    PMC summary of this workload (FETCH_SIZE + WRITE_SIZE, copy-calibrated);
    None when there is none or one of the kernels' sources changed since it
    was taken."""
    from gated_block_sparse_amd import profsum
    blob = profsum.load_traffic(os.path.join(ROOT, "profiles", f"traffic_{workload}.md"), sources)
    if blob is None:
        return None
    tot, hit = 0, False
    for name, v in blob["kernels"].items():
        if name.startswith(prefixes):
            tot += v["fetch_bytes"] + v["write_bytes"]
            hit = True
    return tot if hit else None


class CacheFlush:
    """Evicts the L2s and the 256 MB Infinity Cache between timed steps: a
    512 MiB scratch write, then a 1 GiB read sweep.  The read sweep matters:
    after the write alone the Infinity Cache holds ~256 MB of dirty lines,
    whose write-back then competes with the next timed kernel's reads (a
    64 MB cold streaming read measured 26 us after a write flush against
    15 us after a read sweep and 13 us hot).  A decode step in a model never
    follows such a write burst, so the sweep is what makes the figure cold
    without that artefact."""
    LABEL = "cold (L2 + Infinity Cache evicted: 512 MiB write, then 1 GiB read sweep)"

    def __init__(self, dev):
        import torch
        self.w = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        self.r = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        self.out = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self, i):
        import torch
        self.w.fill_(float(i))
        torch.amax(self.r, dim=0, out=self.out)


def calibrate_copy():
    """A plain 1 GiB device-to-device copy: the known-size reference that the
    PMC byte counters are scaled by."""
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    bb = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    bb.copy_(a)
    torch.cuda.synchronize()
    return {"read": a.numel() * 4, "write": bb.numel() * 4}


def _pct(xs, q):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))
    return xs[i]


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def decode_bytes(wl, lens):
    """Algorithmic bytes of one decode step, split by stage."""
    es = 2 if wl.dtype == "bf16" else 4
    d, Hq, Hkv, k, ds = wl.head_dim, wl.n_q_heads, wl.n_kv_heads, wl.top_k, wl.sel_dim
    kv = 0
    summ = 0
    for T in lens:
        C = (int(T) - 1) // 64
        n0 = int(T) - 64 * C
        kv += Hkv * (min(k, C) * 64 + n0) * d * es * 2
        summ += Hkv * C * ds * 4
    B = len(lens)
    attn = kv + 2 * B * Hq * d * es + 2 * B * Hkv * k * 4 + B * Hq * 4
    select = summ + ds * d * 4 + B * Hq * d * es + 2 * B * Hkv * k * 4 + B * Hkv * 4
    refresh = B * Hkv * 64 * d * es + ds * d * 4 + B * Hkv * ds * 4
    return {"attention": attn, "kv": kv, "select": select, "refresh": refresh,
            "step": attn + select + refresh}


def run_decode(args, wl):
    import torch
    from gated_block_sparse_amd import binding as S
    from gated_block_sparse_amd import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    p = synth.make_problem(wl, seed=0)
    B, Hq, Hkv, d, ds, k = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.sel_dim, wl.top_k
    t_max = p.K.shape[2]

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, K, V = up(p.q), up(p.K), up(p.V)
    lens = torch.from_numpy(p.seq_lens).to(dev)
    Wq, Wk = up(p.Wq_sel), up(p.Wk_sel)
    # prefilled state: summaries of every complete block
    summ = S.sas_block_summaries(K, lens, Wk)
    idx, lg, slse, _ = S.sas_select(S.SAS_SELECT_DECODE, q, lens, Wq, summ, k)
    o, lse = S.sas_decode_fwd(q, K, V, lens, idx, lg)
    torch.cuda.synchronize()

    lib = S.load_library()
    import ctypes
    dims = S.make_dims(B, Hq, Hkv, d, ds, k, t_max, S.SAS_BF16 if wl.dtype == "bf16" else S.SAS_F32)
    pd = ctypes.byref(dims)
    ws_sel = torch.empty(max(1, S.sas_workspace_bytes(S.SAS_OP_SELECT_DECODE, dims)), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(1, S.sas_workspace_bytes(S.SAS_OP_DECODE_FWD, dims)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    c_new = int(min((int(T) - 1) // 64 for T in p.seq_lens))
    blk0, blk1 = max(c_new - 1, 0), max(c_new, 0)
    scale = 1.0 / math.sqrt(d)
    a_sum = (pd, K.data_ptr(), lens.data_ptr(), Wk.data_ptr(), blk0, blk1, summ.data_ptr(), sp)
    a_sel = (pd, S.SAS_SELECT_DECODE, q.data_ptr(), 0, lens.data_ptr(), Wq.data_ptr(),
             summ.data_ptr(), idx.data_ptr(), lg.data_ptr(), slse.data_ptr(), None,
             ws_sel.data_ptr(), ws_sel.numel(), sp)
    a_dec = (pd, q.data_ptr(), K.data_ptr(), V.data_ptr(), lens.data_ptr(), idx.data_ptr(),
             lg.data_ptr(), scale, o.data_ptr(), lse.data_ptr(), ws_dec.data_ptr(),
             ws_dec.numel(), sp)

    ws_step = torch.empty(max(1, S.sas_workspace_bytes(S.SAS_OP_DECODE_STEP, dims)), dtype=torch.uint8, device=dev)
    idx2, lg2, slse2 = torch.empty_like(idx), torch.empty_like(lg), torch.empty_like(slse)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    a_step = (pd, q.data_ptr(), K.data_ptr(), V.data_ptr(), lens.data_ptr(), Wq.data_ptr(),
              Wk.data_ptr(), summ.data_ptr(), 1, scale, idx2.data_ptr(), lg2.data_ptr(), slse2.data_ptr(),
              o2.data_ptr(), lse2.data_ptr(), ws_step.data_ptr(), ws_step.numel(), sp)

    def step_fused(evs=None):
        """The production step: one sas_decode_step (refresh fused in)."""
        if evs:
            evs[0].record(stream)
        st = lib.sas_decode_step(*a_step)
        if evs:
            evs[1].record(stream)
        if st:
            raise S.SasError(st, lib.sas_last_error().decode())

    # the same step on a paged cache: every block in its own page of a
    # shuffled pool (sas_block_summaries_paged, sas_decode_step_paged)
    n_blk = -(-t_max // 64)
    n_pages = B * n_blk
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(0)).view(B, n_blk)
    table = perm.to(torch.int32).to(dev).contiguous()
    pools = []
    for X in (K, V):
        pad = n_blk * 64 - t_max
        Xp = torch.nn.functional.pad(X, (0, 0, 0, pad)) if pad else X
        pool = torch.empty((n_pages, Hkv, 64, d), dtype=X.dtype, device=dev)
        pool[perm.view(-1).to(dev)] = Xp.view(B, Hkv, n_blk, 64, d).permute(0, 2, 1, 3, 4).reshape(
            n_pages, Hkv, 64, d)
        pools.append(pool)
    Kp, Vp = pools
    summ_p = S.sas_block_summaries_paged(Kp, table, lens, Wk, t_max)
    idx3, lg3, slse3 = torch.empty_like(idx), torch.empty_like(lg), torch.empty_like(slse)
    o3, lse3 = torch.empty_like(o), torch.empty_like(lse)
    a_paged = (pd, q.data_ptr(), Kp.data_ptr(), Vp.data_ptr(), table.data_ptr(), n_blk,
               lens.data_ptr(), Wq.data_ptr(), Wk.data_ptr(), summ_p.data_ptr(), 1, scale,
               idx3.data_ptr(), lg3.data_ptr(), slse3.data_ptr(), o3.data_ptr(), lse3.data_ptr(),
               ws_step.data_ptr(), ws_step.numel(), sp)

    def step_paged(evs=None):
        if evs:
            evs[0].record(stream)
        st = lib.sas_decode_step_paged(*a_paged)
        if evs:
            evs[1].record(stream)
        if st:
            raise S.SasError(st, lib.sas_last_error().decode())

    def step(evs=None):
        """The same step through the separate entry points (per-op timing)."""
        if evs:
            evs[0].record(stream)
        st = lib.sas_block_summaries(*a_sum)
        if evs:
            evs[1].record(stream)
        st |= lib.sas_select(*a_sel)
        if evs:
            evs[2].record(stream)
        st |= lib.sas_decode_fwd(*a_dec)
        if evs:
            evs[3].record(stream)
        if st:
            raise S.SasError(st, lib.sas_last_error().decode())

    flush = CacheFlush(dev)
    for _ in range(args.warmup):
        step()
        step_fused()
        step_paged()
    torch.cuda.synchronize()
    if not (torch.equal(o, o2) and torch.equal(idx, idx2) and torch.equal(lse, lse2)):
        raise RuntimeError("fused decode step differs from select + decode_fwd")
    if not (torch.equal(o, o3) and torch.equal(idx, idx3) and torch.equal(lse, lse3)):
        raise RuntimeError("paged decode step differs from the contiguous one")

    K_steps = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K_steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K_steps):
        if not args.no_flush:
            flush(i)          # evict MALL/L2; also covers host launch latency
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tot = [e[0].elapsed_time(e[3]) * 1e3 for e in evs]
    t_sum = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    t_sel = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    t_dec = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]

    # the fused production step, cold the same way
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K_steps)]
    for i in range(K_steps):
        if not args.no_flush:
            flush(i)
        step_fused(evf[i])
    torch.cuda.synchronize()
    tot_f = [e[0].elapsed_time(e[1]) * 1e3 for e in evf]
    evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K_steps)]
    for i in range(K_steps):
        if not args.no_flush:
            flush(i)
        step_paged(evp[i])
    torch.cuda.synchronize()
    tot_p = [e[0].elapsed_time(e[1]) * 1e3 for e in evp]

    # hot-cache figures: the same steps with no eviction in between
    evh = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K_steps)]
    for i in range(K_steps):
        step(evh[i])
    evhf = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K_steps)]
    for i in range(K_steps):
        step_fused(evhf[i])
    torch.cuda.synchronize()
    hot_step = statistics.median([e[0].elapsed_time(e[1]) * 1e3 for e in evhf])
    hot_step_unfused = statistics.median([e[0].elapsed_time(e[3]) * 1e3 for e in evh])
    hot_dec = statistics.median([e[2].elapsed_time(e[3]) * 1e3 for e in evh])

    # hot-cache figure: the same step replayed back to back from a HIP graph
    hot_us = None
    try:
        if args.no_hot:
            raise RuntimeError("--no-hot")
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(stream)
        with torch.cuda.stream(s2):
            sp2 = s2.cuda_stream
            a2 = a_step[:-1] + (sp2,)   # the stream is the last argument
            g.capture_begin()
            sts = [lib.sas_decode_step(*a2)]
            g.capture_end()
        if any(sts):
            raise S.SasError(max(sts), lib.sas_last_error().decode())
        stream.wait_stream(s2)
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        n_hot = 200
        for _ in range(n_hot):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        hot_us = e0.elapsed_time(e1) * 1e3 / n_hot
    except Exception as exc:  # graph capture is a reported extra, never the headline
        if not args.no_hot:
            print(f"# hot-cache graph timing skipped: {exc}", file=sys.stderr)

    by = decode_bytes(wl, p.seq_lens)
    med = statistics.median
    us_step, us_dec = med(tot_f), med(t_dec)
    achieved = by["attention"] / (us_dec * 1e-6) / 1e9
    res = {
        "metric": "SAS decode attn us/step + achieved HBM GB/s (% peak), Qwen3-4B shape @64K",
        "value": round(us_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) q/K/V, K x U(0.5,2) per channel; random selector weights)",
        "config": {"workload": wl.name, "batch": B, "context": [int(x) for x in p.seq_lens][:8],
                   "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "sel_dim": ds,
                   "block": 64, "top_k": k, "cache": "hot" if args.no_flush else CacheFlush.LABEL},
        "tokens_per_s": round(B / (us_step * 1e-6), 1),
        "breakdown_us": {
            "summary_refresh": {"median": round(med(t_sum), 3)},
            "select": {"median": round(med(t_sel), 3), "p10": round(_pct(t_sel, .1), 3), "p90": round(_pct(t_sel, .9), 3)},
            "decode_attention": {"median": round(us_dec, 3), "p10": round(_pct(t_dec, .1), 3), "p90": round(_pct(t_dec, .9), 3)},
            "step": {"median": round(us_step, 3), "p10": round(_pct(tot_f, .1), 3), "p90": round(_pct(tot_f, .9), 3)},
            "step_unfused": {"median": round(med(tot), 3), "p10": round(_pct(tot, .1), 3), "p90": round(_pct(tot, .9), 3)},
            "step_paged_cache": {"median": round(med(tot_p), 3), "p10": round(_pct(tot_p, .1), 3), "p90": round(_pct(tot_p, .9), 3)},
            "step_hot": round(hot_step, 3),
            "step_unfused_hot": round(hot_step_unfused, 3),
            "decode_attention_hot": round(hot_dec, 3),
            "step_hot_graph": None if hot_us is None else round(hot_us, 3),
        },
        "bytes": by,
        "step_GBps": round(by["step"] / (us_step * 1e-6) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": "sas_decode_fwd (split-KV + merge)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name, DECODE_KERNELS, DECODE_SOURCES),
                     "algorithmic_bytes": by["attention"]},
        "wall_s_timed_region": round(wall, 3),
    }
    return res, p


# --------------------------------------------------------------------------
# prefill (training-style forward + backward)
# --------------------------------------------------------------------------
def prefill_pairs(S, G_heads, idx_h):
    """Causally visible selected (query, key) pairs summed over query heads."""
    Hkv = idx_h.shape[1]
    Hq_per = G_heads
    total = 0
    n_tiles = -(-S // 64)
    for r in range(Hkv):
        for t in range(n_tiles):
            nq = min(64, S - 64 * t)
            nsel = int((idx_h[0, r, t] >= 0).sum())
            total += Hq_per * (nsel * 64 * nq + nq * (nq + 1) // 2)
    return total


def query_pairs(S, G_heads, qidx):
    """Per-query selection: causally visible selected (query, key) pairs and
    the pairs the forward visits (each tile's queries against the union of
    their selected blocks, plus the causal diagonal), summed over query heads."""
    Hkv = qidx.shape[1]
    sel = vis = 0
    for r in range(Hkv):
        rows = qidx[0, r]
        nsel = (rows >= 0).sum(axis=1)
        for t in range(-(-S // 64)):
            i0, i1 = 64 * t, min(64 * t + 64, S)
            nq = i1 - i0
            diag = nq * (nq + 1) // 2
            u = np.unique(rows[i0:i1][rows[i0:i1] >= 0]).size
            sel += G_heads * (int(nsel[i0:i1].sum()) * 64 + diag)
            vis += G_heads * (u * 64 * nq + diag)
    return sel, vis


def run_prefill(args, wl):
    import torch
    from gated_block_sparse_amd import binding as Sb
    from gated_block_sparse_amd import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    p = synth.make_problem(wl, seed=0)
    B, Hq, Hkv, d, ds, k = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.sel_dim, wl.top_k
    S = int(p.seq_lens[0])

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    Q, K, V, dO = up(p.q), up(p.K), up(p.V), up(p.dO)
    Wq, Wk = up(p.Wq_sel), up(p.Wk_sel)
    lens = torch.tensor([S], dtype=torch.int32, device=dev)
    summ = Sb.sas_block_summaries(K, lens, Wk)
    idx, lg, slse, _ = Sb.sas_select(Sb.SAS_SELECT_TILES, Q, None, Wq, summ, k, t_max=S)
    O, lse = Sb.sas_prefill_fwd(Q, K, V, idx, lg)
    dQ, dK, dV, dlg = Sb.sas_bwd(Q, K, V, O, dO, lse, idx, lg)
    torch.cuda.synchronize()
    pairs = prefill_pairs(S, Hq // Hkv, idx.cpu().numpy())
    fwd_flop = 4.0 * d * pairs
    bwd_flop = 10.0 * d * pairs

    stream = torch.cuda.current_stream()
    flush = CacheFlush(dev)
    dims = Sb.make_dims(B, Hq, Hkv, d, ds, k, S, Sb.SAS_BF16)
    ws_sel = torch.zeros(max(1, Sb.sas_workspace_bytes(Sb.SAS_OP_SELECT_TILES, dims, S)), dtype=torch.uint8, device=dev)
    ws_fwd = torch.zeros(max(1, Sb.sas_workspace_bytes(Sb.SAS_OP_PREFILL_FWD, dims, S)), dtype=torch.uint8, device=dev)
    ws_bwd = torch.zeros(max(1, Sb.sas_workspace_bytes(Sb.SAS_OP_BWD, dims, S)), dtype=torch.uint8, device=dev)
    ws_sb = torch.zeros(max(1, Sb.sas_workspace_bytes(Sb.SAS_OP_SELECTOR_BWD, dims, S)), dtype=torch.uint8, device=dev)
    dWq, dWk = torch.empty_like(Wq), torch.empty_like(Wq)

    def step(evs=None):
        rec = (lambda i: evs[i].record(stream)) if evs else (lambda i: None)
        rec(0)
        Sb.sas_block_summaries(K, lens, Wk, summ=summ)
        Sb.sas_select(Sb.SAS_SELECT_TILES, Q, None, Wq, summ, k, t_max=S, idx=idx, log_gate=lg,
                      score_lse=slse, ws=ws_sel)
        rec(1)
        Sb.sas_prefill_fwd(Q, K, V, idx, lg, O=O, lse=lse, ws=ws_fwd)
        rec(2)
        Sb.sas_bwd(Q, K, V, O, dO, lse, idx, lg, dQ=dQ, dK=dK, dV=dV, dlog_gate=dlg, ws=ws_bwd)
        rec(3)
        Sb.sas_selector_bwd(Q, K, Wq, summ, idx, slse, dlg, dWq=dWq, dWk=dWk, ws=ws_sb)
        rec(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        if not args.no_flush:
            flush(i)
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_sel = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    t_fwd = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    t_bwd = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]
    t_sb = [e[3].elapsed_time(e[4]) * 1e3 for e in evs]
    tot = [e[0].elapsed_time(e[4]) * 1e3 for e in evs]

    # the backward once more with a sink-heavy selection (every tile also
    # selects blocks 0 and 1, which every tile then reads): the case the
    # dK/dV pass splits hot blocks for
    rng = np.random.default_rng(7)
    sidx = idx.cpu().numpy().copy()
    n_tiles = sidx.shape[2]
    for r in range(Hkv):
        for t in range(2, n_tiles):
            row = [int(x) for x in sidx[0, r, t] if x >= 0]
            keep = [x for x in row if x not in (0, 1)]
            rng.shuffle(keep)
            row = sorted([0, 1] + keep[:max(0, len(row) - 2)])
            sidx[0, r, t, :len(row)] = row
    sidx_d = torch.from_numpy(sidx).to(dev)
    Os, lses = Sb.sas_prefill_fwd(Q, K, V, sidx_d, lg)
    t_sink = []
    for i in range(n):
        if not args.no_flush:
            flush(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        Sb.sas_bwd(Q, K, V, Os, dO, lses, sidx_d, lg, dQ=dQ, dK=dK, dV=dV, dlog_gate=dlg, ws=ws_bwd)
        e1.record(stream)
        torch.cuda.synchronize()
        t_sink.append(e0.elapsed_time(e1) * 1e3)
    # one selection per query (the training kernel's own masking rule): the
    # per-query selection, then the forward over the union of each tile's
    # per-query selections with a per-query mask
    qidx, qlg, qlse, _ = Sb.sas_select(Sb.SAS_SELECT_QUERIES, Q, None, Wq, summ, k, t_max=S)
    Oq, lseq = Sb.sas_prefill_fwd_queries(Q, K, V, qidx, qlg)
    ws_qbwd = torch.zeros(max(1, Sb.sas_workspace_bytes(Sb.SAS_OP_BWD_QUERIES, dims, S)), dtype=torch.uint8, device=dev)
    qdlg = torch.empty(qidx.shape, dtype=torch.float32, device=dev)
    ws_qsb = torch.zeros(max(1, Sb.sas_workspace_bytes(Sb.SAS_OP_SELECTOR_BWD_QUERIES, dims, S)), dtype=torch.uint8, device=dev)
    t_qsel, t_qfwd, t_qbwd, t_qsb = [], [], [], []
    for i in range(n):
        if not args.no_flush:
            flush(i)
        e0, e1, e2, e3, e4 = (torch.cuda.Event(enable_timing=True) for _ in range(5))
        e0.record(stream)
        Sb.sas_select(Sb.SAS_SELECT_QUERIES, Q, None, Wq, summ, k, t_max=S, idx=qidx,
                      log_gate=qlg, score_lse=qlse)
        e1.record(stream)
        Sb.sas_prefill_fwd_queries(Q, K, V, qidx, qlg, O=Oq, lse=lseq)
        e2.record(stream)
        Sb.sas_bwd_queries(Q, K, V, Oq, dO, lseq, qidx, qlg, dQ=dQ, dK=dK, dV=dV, dlog_gate=qdlg,
                           ws=ws_qbwd)
        e3.record(stream)
        Sb.sas_selector_bwd_queries(Q, K, Wq, Wk, summ, qidx, qlse, qdlg, dWq=dWq, dWk=dWk,
                                    ws=ws_qsb)
        e4.record(stream)
        torch.cuda.synchronize()
        t_qsel.append(e0.elapsed_time(e1) * 1e3)
        t_qfwd.append(e1.elapsed_time(e2) * 1e3)
        t_qbwd.append(e2.elapsed_time(e3) * 1e3)
        t_qsb.append(e3.elapsed_time(e4) * 1e3)
    qsel_pairs, qvis_pairs = query_pairs(S, Hq // Hkv, qidx.cpu().numpy())

    med = statistics.median
    us_fwd, us_bwd, us_step = med(t_fwd), med(t_bwd), med(tot)
    us_qfwd = med(t_qfwd)
    fwd_tf = fwd_flop / (us_fwd * 1e-6) / 1e12
    bwd_tf = bwd_flop / (us_bwd * 1e-6) / 1e12
    res = {
        "metric": "SAS prefill fwd+bwd us/step + achieved bf16 MFMA TFLOP/s (% peak), Qwen3-4B shape, S=16384",
        "value": round(us_step, 1),
        "unit": "us/step",
        "n_gpus": 1, "steps": n, "warmup": args.warmup,
        "ms_per_step": round(us_step / 1e3, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO, random selector weights)",
        "config": {"workload": wl.name, "batch": B, "seq_len": S, "n_q_heads": Hq,
                   "n_kv_heads": Hkv, "head_dim": d, "sel_dim": ds, "block": 64, "top_k": k,
                   "cache": "hot" if args.no_flush else CacheFlush.LABEL},
        "tokens_per_s": round(B * S / (us_step * 1e-6), 1),
        "breakdown_us": {
            "summaries_and_select": round(med(t_sel), 2),
            "prefill_fwd": {"median": round(us_fwd, 2), "p10": round(_pct(t_fwd, .1), 2), "p90": round(_pct(t_fwd, .9), 2)},
            "bwd": {"median": round(us_bwd, 2), "p10": round(_pct(t_bwd, .1), 2), "p90": round(_pct(t_bwd, .9), 2)},
            "selector_bwd": {"median": round(med(t_sb), 2), "p10": round(_pct(t_sb, .1), 2), "p90": round(_pct(t_sb, .9), 2)},
            "bwd_sink_heavy_selection": {"median": round(med(t_sink), 2), "p10": round(_pct(t_sink, .1), 2), "p90": round(_pct(t_sink, .9), 2)},
            "per_query_select": {"median": round(med(t_qsel), 2), "p10": round(_pct(t_qsel, .1), 2), "p90": round(_pct(t_qsel, .9), 2)},
            "per_query_fwd": {"median": round(us_qfwd, 2), "p10": round(_pct(t_qfwd, .1), 2), "p90": round(_pct(t_qfwd, .9), 2)},
            "per_query_bwd": {"median": round(med(t_qbwd), 2), "p10": round(_pct(t_qbwd, .1), 2), "p90": round(_pct(t_qbwd, .9), 2)},
            "per_query_selector_bwd": {"median": round(med(t_qsb), 2), "p10": round(_pct(t_qsb, .1), 2), "p90": round(_pct(t_qsb, .9), 2)},
        },
        "per_query": {
            "selected_pairs": qsel_pairs, "visited_pairs": qvis_pairs,
            "fwd_TFLOPs_selected": round(4.0 * d * qsel_pairs / (us_qfwd * 1e-6) / 1e12, 1),
            "fwd_TFLOPs_visited": round(4.0 * d * qvis_pairs / (us_qfwd * 1e-6) / 1e12, 1),
            "bwd_TFLOPs_selected": round(10.0 * d * qsel_pairs / (med(t_qbwd) * 1e-6) / 1e12, 1),
            "note": "selected = the causally visible (query, key) pairs each query selected "
                    "(algorithmic); visited = the pairs the forward and the backward's dQ pass "
                    "multiply: every query of a tile against the union of the tile's "
                    "selections (the backward's dK/dV pass multiplies selected pairs only, "
                    "from per-block query lists)",
        },
        "flops": {"visible_selected_pairs": pairs, "fwd": fwd_flop, "bwd": bwd_flop},
        "bwd_TFLOPs": round(bwd_tf, 1),
        "roofline": {"bound": "mfma", "kernel": "prefill_fwd_persistent_kernel (sas_prefill_fwd)",
                     "achieved": round(fwd_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fwd_tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name, PREFILL_KERNELS, PREFILL_SOURCES)},
        "roofline_bwd": {"bound": "mfma", "kernel": "sas_bwd (dQ pass with D, dK/dV pass)",
                         "achieved": round(bwd_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(bwd_tf / BF16_PEAK_TFLOPS, 4)},
        "wall_s_timed_region": round(wall, 3),
    }
    return res, p


def cpu_baseline_prefill(p, budget_s):
    """The float64 oracle forward on a sample of tiles, scaled to one full forward."""
    from oracle import sas_oracle as O
    from gated_block_sparse_amd import synth
    wl = p.wl
    S = int(p.seq_lens[0])
    G = wl.n_q_heads // wl.n_kv_heads
    n_tiles = -(-S // 64)
    Qf, Kf, Vf = (synth.to_f64(x[0], wl.dtype) for x in (p.q, p.K, p.V))
    rng = np.random.default_rng(0)
    idx = np.full((wl.n_kv_heads, n_tiles, wl.top_k), -1, np.int64)
    lg = np.full(idx.shape, -np.inf)
    for r in range(wl.n_kv_heads):
        for t in range(n_tiles):
            c = min(wl.top_k, t)
            if c:
                idx[r, t, :c] = np.sort(rng.choice(t, size=c, replace=False))
                lg[r, t, :c] = -2.0
    done = 0
    t0 = time.perf_counter()
    tiles = list(range(n_tiles - 1, -1, -1))   # full tiles first
    while time.perf_counter() - t0 < budget_s and done < n_tiles:
        O.prefill_attend(Qf, Kf, Vf, S, idx, lg, 1.0 / math.sqrt(wl.head_dim), G, tiles=[tiles[done]])
        done += 1
    el = time.perf_counter() - t0
    return el / done * n_tiles * 1e6, done, n_tiles


def cpu_baseline_decode(p, budget_s):
    """The float64 oracle on the same decode step, repeated for ~budget_s."""
    from oracle import sas_oracle as O
    from gated_block_sparse_amd import synth
    wl = p.wl
    G = wl.n_q_heads // wl.n_kv_heads
    d = wl.head_dim
    b = 0
    T = int(p.seq_lens[b])
    # prefilled state for the oracle: its own summaries of every history block
    per = []
    for r in range(wl.n_kv_heads):
        Kr = synth.to_f64(p.K[b, r:r + 1, :T], wl.dtype)
        Vr = synth.to_f64(p.V[b, r:r + 1, :T], wl.dtype)
        per.append((Kr, Vr, O.block_summaries(Kr, T, p.f64("Wk_sel"))))
    q = synth.to_f64(p.q[b], wl.dtype)
    Wq, Wk = p.f64("Wq_sel"), p.f64("Wk_sel")
    C = O.n_history_blocks(T)
    n = 0
    t0 = time.perf_counter()
    while True:
        for r, (Kr, Vr, summ) in enumerate(per):
            # refresh the newest block, score, gate, Top-K, attend
            O.block_summaries(Kr[:, 64 * (C - 1):64 * C + 1], 65, Wk)
            qg = q[r * G:(r + 1) * G]
            s = O.decode_scores(qg, Wq, summ, G)[0]
            idx, lg, _, _ = O.select_rows([s], wl.top_k)
            O.decode_attend(qg, Kr, Vr, T, idx, lg, 1.0 / math.sqrt(d), G)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    us = el / n * 1e6
    return us, n


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"])
    except Exception:
        pass
    return 1


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(the sharding plan is described in DESIGN.md)"}))
        sys.exit(2)
    from gated_block_sparse_amd import synth
    wl = synth.WORKLOADS[args.workload]
    if wl.mode != "decode":
        res, p = run_prefill(args, wl)
        if args.calibrate_copy:
            res["copy_calibration_bytes"] = calibrate_copy()
        if not args.no_cpu_baseline:
            us, done, n_tiles = cpu_baseline_prefill(p, args.cpu_seconds)
            res["cpu_baseline"] = {
                "value": round(us, 1), "unit": "us per prefill forward", "cores": blas_threads(),
                "kind": "oracle",
                "sample": f"oracle forward on {done} of {n_tiles} query tiles (all heads), "
                          f"scaled to the full sequence; float64 NumPy",
            }
        print(json.dumps(res))
        return
    res, p = run_decode(args, wl)
    if args.calibrate_copy:
        res["copy_calibration_bytes"] = calibrate_copy()
    if not args.no_cpu_baseline:
        us, n = cpu_baseline_decode(p, args.cpu_seconds)
        res["cpu_baseline"] = {
            "value": round(us, 1), "unit": "us/step", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} full decode steps of sequence 0 (all {wl.n_kv_heads} groups: newest-"
                      f"block summary, scores over every block, gate, Top-K, attention), float64 "
                      f"NumPy, host CPUs available: {len(os.sched_getaffinity(0))}",
        }
        res["gpu_speedup_vs_cpu_oracle"] = round(us / res["value"], 1)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
