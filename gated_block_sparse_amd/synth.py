"""Seeded synthetic inputs for the SAS gated block-sparse attention path.

This module only draws random tensors; it holds none of the method's arithmetic.
Both the CPU oracle (in tests) and the HIP path consume exactly the arrays built
here, so the two sides always see identical inputs.

Workloads stand in for the settings measured on the pages (no model weights or
datasets are used): the Qwen3-4B attention shape (32 query heads, 8 KV heads,
head dim 128), block size 64 ("SAS: context ranking", section 3.1), 64K/512K
contexts and batches 1/8 (section 3.6, Figure 7), and 1024/2048-token budgets
(section 3.2, Table 2).

Conventions
-----------
* Layouts are row-major, head-major: q ``[B,Hq,d]`` (decode), Q/dO
  ``[B,Hq,S,d]`` (prefill), K/V ``[B,Hkv,t_max,d]``, selector weights
  ``[d_sel,d]`` fp32.
* bf16 tensors are produced by round-to-nearest-even of fp32 draws and kept as
  raw ``uint16`` bit patterns; :func:`to_f64` gives their exact values.
* Every tensor gets an independent child of ``SeedSequence(seed)``, spawned in
  the fixed order q, K, V, Wq_sel, Wk_sel, scales, lens, plants, dO.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BLOCK = 64

F32 = "f32"
BF16 = "bf16"

_STREAMS = ("q", "K", "V", "Wq_sel", "Wk_sel", "scales", "lens", "plants", "dO")


# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored tensor (fp32 array or bf16 bits)."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == BF16 else np.ascontiguousarray(x32, np.float32)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mode: str                 # "decode" or "prefill"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    sel_dim: int
    top_k: int
    dtype: str                # dtype of Q/K/V/O
    seq_len: int = 0          # decode: context T (fixed); prefill: S
    seq_len_range: Optional[tuple] = None   # decode: per-sequence T ~ U{lo..hi}
    k_channel_skew: bool = False            # K *= U(0.5,2) per (kv head, channel)
    plant_frac: float = 0.0                 # fraction of history blocks with a planted key
    plant_gain: float = 8.0
    w_std: Optional[float] = None           # selector weight std (default 1/sqrt(d_sel))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def t_max(self) -> int:
        if self.seq_len_range is not None:
            return int(self.seq_len_range[1])
        return int(self.seq_len)


WORKLOADS = {
    # Tiny fp32 single decode step: 63 history blocks + current block, k=16.
    "tiny_f32_decode_4k": Workload(
        "tiny_f32_decode_4k", "decode", 1, 4, 1, 64, 64, 16, F32, seq_len=4096),
    # Qwen3-4B attention shape, 64K context, 1024-token budget.
    "qwen3_4b_decode_64k": Workload(
        "qwen3_4b_decode_64k", "decode", 1, 32, 8, 128, 128, 16, BF16,
        seq_len=65536, k_channel_skew=True),
    # Batch 8, per-sequence contexts U{32768..65536}, 2048-token budget.
    "qwen3_4b_decode_b8_32k_64k": Workload(
        "qwen3_4b_decode_b8_32k_64k", "decode", 8, 32, 8, 128, 128, 32, BF16,
        seq_len_range=(32768, 65536)),
    # 512K context (8191 history blocks), 2048-token budget, 1% planted blocks.
    "qwen3_4b_decode_512k": Workload(
        "qwen3_4b_decode_512k", "decode", 1, 32, 8, 128, 128, 32, BF16,
        seq_len=524288, plant_frac=0.01),
    # Training-style causal prefill forward + backward, S=16384, per-tile k=16.
    "qwen3_4b_prefill_16k": Workload(
        "qwen3_4b_prefill_16k", "prefill", 1, 32, 8, 128, 128, 16, BF16,
        seq_len=16384),
}

# Workloads in the order they are listed for this method (0-based index).
WORKLOAD_ORDER = [
    "tiny_f32_decode_4k",
    "qwen3_4b_decode_64k",
    "qwen3_4b_decode_b8_32k_64k",
    "qwen3_4b_decode_512k",
    "qwen3_4b_prefill_16k",
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[WORKLOAD_ORDER[name_or_index]]
    return WORKLOADS[name_or_index]


# --------------------------------------------------------------------------
# Problem instances
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    wl: Workload
    q: np.ndarray            # decode [B,Hq,d]; prefill [B,Hq,S,d]  (storage dtype)
    K: np.ndarray            # [B,Hkv,t_max,d] storage dtype
    V: np.ndarray            # [B,Hkv,t_max,d] storage dtype
    seq_lens: np.ndarray     # int32 [B]
    Wq_sel: np.ndarray       # fp32 [d_sel,d]
    Wk_sel: np.ndarray       # fp32 [d_sel,d]
    dO: Optional[np.ndarray] = None      # prefill [B,Hq,S,d] storage dtype
    planted: Optional[np.ndarray] = None  # decode: bool [B,Hkv,C_max] planted blocks

    def f64(self, name: str) -> np.ndarray:
        arr = getattr(self, name)
        if name in ("Wq_sel", "Wk_sel"):
            return arr.astype(np.float64)
        return to_f64(arr, self.wl.dtype)


def _rngs(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.default_rng(c) for name, c in zip(_STREAMS, children)}


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_problem(wl: Workload, seed: int = 0, *, batch: Optional[int] = None,
                 seq_len: Optional[int] = None, seq_lens=None,
                 t_max: Optional[int] = None, top_k: Optional[int] = None,
                 zero_wq: bool = False) -> Problem:
    """Draw one seeded instance of a workload.

    Optional overrides shrink or reshape it (tests use them for small and
    ragged cases); ``zero_wq`` sets ``Wq_sel = 0`` (all selector scores equal).
    """
    if batch is not None or seq_len is not None or seq_lens is not None or top_k is not None:
        wl = dataclasses.replace(
            wl,
            batch=batch if batch is not None else wl.batch,
            seq_len=seq_len if seq_len is not None else wl.seq_len,
            seq_len_range=None if (seq_len is not None or seq_lens is not None) else wl.seq_len_range,
            top_k=top_k if top_k is not None else wl.top_k,
        )
    r = _rngs(seed)
    B, Hq, Hkv, d, ds = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.sel_dim

    # sequence lengths
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32)
        assert lens.shape == (B,)
    elif wl.seq_len_range is not None:
        lo, hi = wl.seq_len_range
        lens = r["lens"].integers(lo, hi + 1, size=B).astype(np.int32)
    else:
        lens = np.full(B, wl.seq_len, dtype=np.int32)
    tm = int(t_max) if t_max is not None else int(max(lens.max(), 1))
    if wl.mode == "prefill":
        tm = int(t_max) if t_max is not None else int(lens.max())

    if wl.mode == "decode":
        q32 = _normal(r["q"], (B, Hq, d))
    else:
        q32 = _normal(r["q"], (B, Hq, int(lens.max()), d))
    K32 = _normal(r["K"], (B, Hkv, tm, d))
    V32 = _normal(r["V"], (B, Hkv, tm, d))
    w_std = wl.w_std if wl.w_std is not None else 1.0 / np.sqrt(ds)
    Wq = (_normal(r["Wq_sel"], (ds, d)) * np.float32(w_std)).astype(np.float32)
    Wk = (_normal(r["Wk_sel"], (ds, d)) * np.float32(w_std)).astype(np.float32)
    if zero_wq:
        Wq[:] = 0.0
    if wl.k_channel_skew:
        sc = r["scales"].uniform(0.5, 2.0, size=(B, Hkv, 1, d)).astype(np.float32)
        K32 *= sc

    planted = None
    if wl.plant_frac > 0.0 and wl.mode == "decode":
        G = Hq // Hkv
        c_max = (int(lens.max()) - 1) // BLOCK
        planted = np.zeros((B, Hkv, c_max), dtype=bool)
        for b in range(B):
            C = (int(lens[b]) - 1) // BLOCK
            n_plant = int(round(wl.plant_frac * C))
            for h in range(Hkv):
                qg = q32[b, h * G:(h + 1) * G].astype(np.float64).mean(axis=0)
                qhat = (qg / np.linalg.norm(qg)).astype(np.float32)
                blocks = r["plants"].choice(C, size=n_plant, replace=False)
                planted[b, h, blocks] = True
                for m in blocks:
                    K32[b, h, m * BLOCK:(m + 1) * BLOCK, :] += np.float32(wl.plant_gain) * qhat

    dO = None
    if wl.mode == "prefill":
        dO = _store(_normal(r["dO"], q32.shape), wl.dtype)

    return Problem(wl=wl, q=_store(q32, wl.dtype), K=_store(K32, wl.dtype),
                   V=_store(V32, wl.dtype), seq_lens=lens, Wq_sel=Wq, Wk_sel=Wk,
                   dO=dO, planted=planted)


def custom_workload(mode: str, *, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64,
                    sel_dim=64, top_k=4, dtype=F32, seq_len=256, **kw) -> Workload:
    """A small ad-hoc workload (tests use it for edge cases)."""
    return Workload(f"custom_{mode}", mode, batch, n_q_heads, n_kv_heads, head_dim,
                    sel_dim, top_k, dtype, seq_len=seq_len, **kw)
