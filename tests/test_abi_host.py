"""Host-side checks of the C ABI: the library loads, exports every function
include/sas.h declares, and rejects invalid arguments during validation,
before anything is enqueued (no GPU needed: these calls return before any HIP
call is made)."""
import ctypes
import os
import re

import pytest

from gated_block_sparse_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from gated_block_sparse_amd import build
        build.build(verbose=False)
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("sas_block_summaries", "sas_select", "sas_decode_fwd", "sas_prefill_fwd",
              "sas_bwd", "sas_workspace_bytes", "sas_status_str", "sas_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.sas_status_str(0) == b"SAS_OK"
    assert lib.sas_status_str(3) == b"SAS_ERR_WORKSPACE_TOO_SMALL"
    assert lib.sas_status_str(99) == b"SAS_UNKNOWN_STATUS"


def _dims(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, sel_dim=128, top_k=16,
                t_max=65536, dtype=B.SAS_BF16)
    base.update(kw)
    return B.make_dims(**base)


def _decode(lib, dims, ws_bytes=1 << 30, q=FAKE, idx=FAKE, scale=0.1):
    return lib.sas_decode_fwd(ctypes.byref(dims) if dims is not None else None, q, FAKE, FAKE,
                              FAKE, idx, FAKE, scale, FAKE, FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=30), B.SAS_ERR_INVALID_ARGUMENT),   # Hq % Hkv != 0
    (dict(top_k=-1), B.SAS_ERR_INVALID_ARGUMENT),
    (dict(batch=0), B.SAS_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.SAS_ERR_INVALID_ARGUMENT),
    (dict(block_size=32), B.SAS_ERR_UNSUPPORTED),
    (dict(head_dim=96), B.SAS_ERR_UNSUPPORTED),
    (dict(sel_dim=32), B.SAS_ERR_UNSUPPORTED),
    (dict(n_q_heads=48, n_kv_heads=8), B.SAS_ERR_UNSUPPORTED),   # G = 6
    (dict(top_k=65), B.SAS_ERR_UNSUPPORTED),
])
def test_decode_rejects_bad_dims(lib, kw, status):
    assert _decode(lib, _dims(**kw)) == status
    assert lib.sas_last_error() != b""


def test_decode_rejects_nulls_scale_and_small_workspace(lib):
    assert _decode(lib, None) == B.SAS_ERR_INVALID_ARGUMENT
    assert b"dims" in lib.sas_last_error()
    assert _decode(lib, _dims(), q=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert b"q is NULL" in lib.sas_last_error()
    assert _decode(lib, _dims(), idx=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert _decode(lib, _dims(), scale=0.0) == B.SAS_ERR_INVALID_ARGUMENT
    assert _decode(lib, _dims(), scale=float("nan")) == B.SAS_ERR_INVALID_ARGUMENT
    need = B.sas_workspace_bytes(B.SAS_OP_DECODE_FWD, _dims())
    assert need > 0
    assert _decode(lib, _dims(), ws_bytes=need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL


def test_decode_step_validation(lib):
    d = _dims()
    need = B.sas_workspace_bytes(B.SAS_OP_DECODE_STEP, d)
    # the selection's chunk state and the attention partials, each 256-byte
    # aligned, then one int arrival count per (sequence, group) row
    sel = B.sas_workspace_bytes(B.SAS_OP_SELECT_DECODE, d)
    part = B.sas_workspace_bytes(B.SAS_OP_DECODE_FWD, d)
    assert need == (sel + 255) // 256 * 256 + (part + 255) // 256 * 256 + 4 * d.batch * d.n_kv_heads
    step = lambda dims, ws_bytes, scale=0.1, q=FAKE, lg=FAKE, wk=None: lib.sas_decode_step(
        ctypes.byref(dims), q, FAKE, FAKE, FAKE, FAKE, wk, FAKE, 1, scale, FAKE, lg, FAKE, FAKE,
        FAKE, FAKE, ws_bytes, None)
    assert step(d, need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL
    assert step(d, need, scale=-1.0) == B.SAS_ERR_INVALID_ARGUMENT
    assert step(d, need, q=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert step(d, need, lg=None) == B.SAS_ERR_INVALID_ARGUMENT   # k > 0 needs log_gate
    assert step(_dims(head_dim=96), 1 << 40) == B.SAS_ERR_UNSUPPORTED
    assert step(_dims(head_dim=96), 1 << 40, wk=FAKE) == B.SAS_ERR_UNSUPPORTED


def test_paged_validation(lib):
    d = _dims()
    need = B.sas_workspace_bytes(B.SAS_OP_DECODE_STEP, d)

    def step(dims, max_pages, table=FAKE, summ=FAKE, ws_bytes=need):
        return lib.sas_decode_step_paged(
            ctypes.byref(dims), FAKE, FAKE, FAKE, table, max_pages, FAKE, FAKE, None, summ, 1,
            0.1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert step(d, 1024, ws_bytes=need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL
    assert step(d, 1023) == B.SAS_ERR_INVALID_ARGUMENT    # 65536 tokens need 1024 pages
    assert step(d, 0) == B.SAS_ERR_INVALID_ARGUMENT
    assert step(d, 1024, table=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert step(d, 1024, summ=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert step(_dims(head_dim=96), 1 << 20) == B.SAS_ERR_UNSUPPORTED
    psum = lambda b0, b1, table=FAKE, mp=1024: lib.sas_block_summaries_paged(
        ctypes.byref(d), FAKE, table, mp, FAKE, FAKE, b0, b1, FAKE, None)
    assert psum(-1, 4) == B.SAS_ERR_INVALID_ARGUMENT
    assert psum(5, 4) == B.SAS_ERR_INVALID_ARGUMENT
    assert psum(0, 4, mp=1000) == B.SAS_ERR_INVALID_ARGUMENT
    assert psum(0, 4, table=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert psum(2000, 3000, table=None) == B.SAS_OK       # beyond t_max/64: nothing to do


def test_selector_bwd_validation(lib):
    d = _dims()
    need = B.sas_workspace_bytes(B.SAS_OP_SELECTOR_BWD, d, 16384)
    # ds of every (row, block), per row a_row, qbar, u, per block e_m, kbar_m, then the
    # chunk partials of the two weight sums
    rows, grp, c_max = 256, 8, 65536 // 64
    sel = (grp * rows * c_max * 4 + 255) // 256 * 256
    rowb = (grp * rows * (2 * 128 + 128) * 4 + 255) // 256 * 256
    blkb = (grp * rows * (128 + 128) * 4 + 255) // 256 * 256
    chunks = (grp * rows + 15) // 16      # outer-product partials of 16 entries each
    assert need == sel + rowb + blkb + 2 * chunks * 128 * 128 * 4
    sb = lambda dims, q_len, ws_bytes, dlg=FAKE, dwk=FAKE: lib.sas_selector_bwd(
        ctypes.byref(dims), FAKE, q_len, FAKE, FAKE, FAKE, FAKE, FAKE, dlg, None, FAKE, dwk,
        FAKE, ws_bytes, None)
    assert sb(d, 16384, need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL
    assert sb(d, 0, need) == B.SAS_ERR_INVALID_ARGUMENT
    assert sb(d, 65537, 1 << 40) == B.SAS_ERR_INVALID_ARGUMENT     # q_len > t_max
    assert sb(d, 16384, need, dlg=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert sb(d, 16384, need, dwk=None) == B.SAS_ERR_INVALID_ARGUMENT
    big = _dims(t_max=64 * 1025 * 64)
    assert sb(big, 64 * 1025, 1 << 40) == B.SAS_ERR_UNSUPPORTED


def test_prefill_and_bwd_validation(lib):
    d = _dims()
    pf = lambda dims, seq_len: lib.sas_prefill_fwd(ctypes.byref(dims), FAKE, FAKE, FAKE, seq_len,
                                                   FAKE, FAKE, 0.1, FAKE, FAKE, FAKE, 1 << 40, None)
    assert pf(d, 0) == B.SAS_ERR_INVALID_ARGUMENT
    assert pf(d, 65537) == B.SAS_ERR_INVALID_ARGUMENT          # seq_len > t_max
    assert pf(_dims(dtype=B.SAS_F32), 128) == B.SAS_ERR_UNSUPPORTED
    bw = lambda dims, seq_len, dlg: lib.sas_bwd(ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, seq_len, FAKE, FAKE, 0.1, FAKE, FAKE, FAKE,
                                                dlg, FAKE, 1 << 40, None)
    assert bw(d, 0, FAKE) == B.SAS_ERR_INVALID_ARGUMENT
    assert bw(d, 128, None) == B.SAS_ERR_INVALID_ARGUMENT       # dlog_gate NULL with k > 0
    assert bw(_dims(dtype=B.SAS_F32), 128, FAKE) == B.SAS_ERR_UNSUPPORTED


def test_select_and_summaries_validation(lib):
    d = _dims()
    sel = lambda dims, mode, q_len, ws_bytes: lib.sas_select(
        ctypes.byref(dims), mode, FAKE, q_len, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
        ws_bytes, None)
    assert sel(d, 5, 0, 1 << 30) == B.SAS_ERR_INVALID_ARGUMENT
    assert sel(d, B.SAS_SELECT_TILES, 0, 0) == B.SAS_ERR_INVALID_ARGUMENT
    assert sel(d, B.SAS_SELECT_TILES, 70000, 0) == B.SAS_ERR_INVALID_ARGUMENT
    need = B.sas_workspace_bytes(B.SAS_OP_SELECT_DECODE, d)
    assert sel(d, B.SAS_SELECT_DECODE, 0, need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL
    big = _dims(t_max=64 * 1025 * 64)
    assert sel(big, B.SAS_SELECT_TILES, 64 * 1025, 0) == B.SAS_ERR_UNSUPPORTED
    summ = lambda dims, b0, b1: lib.sas_block_summaries(ctypes.byref(dims), FAKE, FAKE, FAKE, b0,
                                                        b1, FAKE, None)
    assert summ(d, -1, 4) == B.SAS_ERR_INVALID_ARGUMENT
    assert summ(d, 5, 4) == B.SAS_ERR_INVALID_ARGUMENT
    assert summ(d, 7, 7) == B.SAS_OK                              # empty range: nothing to do


def test_workspace_sizes(lib):
    d = _dims()
    assert B.sas_workspace_bytes(B.SAS_OP_SELECT_TILES, d, 16384) == 0
    # decode: one partial (acc[d] + max + sum) per head and per unit (k slots + B0)
    assert B.sas_workspace_bytes(B.SAS_OP_DECODE_FWD, d) == 1 * 8 * 17 * 4 * 130 * 4
    with pytest.raises(B.SasError):
        B.sas_workspace_bytes(B.SAS_OP_DECODE_FWD, _dims(head_dim=96))
    with pytest.raises(B.SasError):
        B.sas_workspace_bytes(B.SAS_OP_PREFILL_FWD, d, 0)


def test_per_query_calls_validation(lib):
    """The per-query selection path: the QUERIES select mode, the forward,
    the backward and the selector backward reject what they do not support
    before enqueueing anything, and size their workspaces."""
    d = _dims()
    sel = lambda dims, q_len: lib.sas_select(
        ctypes.byref(dims), B.SAS_SELECT_QUERIES, FAKE, q_len, None, FAKE, FAKE, FAKE, FAKE,
        FAKE, None, None, 0, None)
    assert sel(d, 0) == B.SAS_ERR_INVALID_ARGUMENT
    assert sel(d, 65537) == B.SAS_ERR_INVALID_ARGUMENT               # q_len > t_max
    big = _dims(t_max=64 * 1025 * 64)
    assert sel(big, 64 * 1025) == B.SAS_ERR_UNSUPPORTED               # more than 1024 tiles
    assert B.sas_workspace_bytes(B.SAS_OP_SELECT_QUERIES, d, 16384) == 0

    pf = lambda dims, seq_len, idx=FAKE: lib.sas_prefill_fwd_queries(
        ctypes.byref(dims), FAKE, FAKE, FAKE, seq_len, idx, FAKE, 0.1, FAKE, FAKE, None, 0, None)
    assert pf(d, 0) == B.SAS_ERR_INVALID_ARGUMENT
    assert pf(d, 128, idx=None) == B.SAS_ERR_INVALID_ARGUMENT          # idx NULL with k > 0
    assert pf(_dims(dtype=B.SAS_F32), 128) == B.SAS_ERR_UNSUPPORTED
    assert pf(big, 64 * 1025) == B.SAS_ERR_UNSUPPORTED
    assert B.sas_workspace_bytes(B.SAS_OP_PREFILL_FWD_QUERIES, d, 16384) == 0

    # backward workspace: that of sas_bwd plus the per-head log-gate partials,
    # the union bitmaps and their prefix counts, the gate rows and the
    # per-block query lists (each region 256-byte aligned)
    S, k, grp, n_tiles = 16384, 16, 8, 256
    al = lambda x: (x + 255) // 256 * 256
    need_tile = B.sas_workspace_bytes(B.SAS_OP_BWD, d, S)
    qcap = S * k + 64 * n_tiles
    extra = (al(32 * S * k * 4) + al(grp * n_tiles * 32 * 4) + al(grp * n_tiles * 32 * 4)
             + al(grp * (1 + n_tiles * (n_tiles - 1) // 2) * 64 * 4) + al(grp * n_tiles * 4)
             + al(grp * (n_tiles + 1) * 4) + al(grp * qcap * 4) + grp * qcap * 4)
    need = B.sas_workspace_bytes(B.SAS_OP_BWD_QUERIES, d, S)
    assert need == al(need_tile) + extra
    bw = lambda dims, seq_len, ws_bytes, dlg=FAKE: lib.sas_bwd_queries(
        ctypes.byref(dims), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, seq_len, FAKE, FAKE, 0.1, FAKE,
        FAKE, FAKE, dlg, FAKE, ws_bytes, None)
    assert bw(d, S, need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL
    assert bw(d, 0, need) == B.SAS_ERR_INVALID_ARGUMENT
    assert bw(d, S, need, dlg=None) == B.SAS_ERR_INVALID_ARGUMENT
    assert bw(_dims(dtype=B.SAS_F32), 128, 1 << 40) == B.SAS_ERR_UNSUPPORTED

    # selector backward of per-query rows: mean keys, per-row (h, qbar), the
    # H partials of 512-row chunks and H
    need = B.sas_workspace_bytes(B.SAS_OP_SELECTOR_BWD_QUERIES, d, S)
    c_max = 65536 // 64
    chunks = (grp * S + 511) // 512
    assert need == (al(grp * c_max * 128 * 4) + al(grp * S * 2 * 128 * 4)
                    + al(chunks * 128 * 128 * 4) + 128 * 128 * 4)
    sb = lambda dims, q_len, ws_bytes, wk=FAKE: lib.sas_selector_bwd_queries(
        ctypes.byref(dims), FAKE, q_len, FAKE, FAKE, wk, FAKE, FAKE, FAKE, FAKE, None, FAKE,
        FAKE, FAKE, ws_bytes, None)
    assert sb(d, S, need - 1) == B.SAS_ERR_WORKSPACE_TOO_SMALL
    assert sb(d, S, need, wk=None) == B.SAS_ERR_INVALID_ARGUMENT       # Wk_sel is required
    assert sb(d, 65537, 1 << 40) == B.SAS_ERR_INVALID_ARGUMENT
    assert sb(big, 64 * 1025, 1 << 40) == B.SAS_ERR_UNSUPPORTED
