"""The C-ABI library loads, exports what include/flashsample.h declares, and
rejects bad arguments on the host before any HIP call (CPU only: no call in
this file launches a kernel -- the calls with valid arguments run under
FS_FAULT_INJECT=launch, or only where no GPU is present)."""
import ctypes

import pytest

from conftest import gpu_available
from lm_head_exact_amd import binding as bd

ALIGNED = 0x10000            # fake, never dereferenced: every call below fails validation
WS_ALIGNED = 0x20000


@pytest.fixture(scope="module")
def L():
    return bd.lib()


def test_exports_every_declared_symbol(L):
    names = bd.exported_names_from_header()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), f"{n} declared in flashsample.h but not exported"


def test_status_strings(L):
    assert L.fs_status_string(0) == b"FS_OK"
    assert L.fs_status_string(4) == b"FS_ERR_HIP"
    assert L.fs_status_string(99) == b"FS_ERR_UNKNOWN"


def _sample(L, fn="fs_sample", h=ALIGNED, W=ALIGNED, B=4, D=256, V=1000, off=0,
            T=ALIGNED, ids=ALIGNED, val=ALIGNED, ws=WS_ALIGNED, wsb=1 << 30):
    return getattr(L, fn)(h, W, B, D, V, off, T, 1, 2, ids, val, ws, wsb, None)


@pytest.mark.parametrize("fn", ["fs_sample", "fs_sample_partial", "fs_sample_unfused"])
@pytest.mark.parametrize("kw,status", [
    (dict(D=7), bd.FS_ERR_INVALID_ARG),
    (dict(D=0), bd.FS_ERR_INVALID_ARG),
    (dict(D=260), bd.FS_ERR_INVALID_ARG),
    (dict(V=0), bd.FS_ERR_INVALID_ARG),
    (dict(B=-1), bd.FS_ERR_INVALID_ARG),
    (dict(off=-5), bd.FS_ERR_INVALID_ARG),
    (dict(off=2**31 - 1000, V=1000), bd.FS_ERR_INVALID_ARG),
    (dict(h=None), bd.FS_ERR_INVALID_ARG),
    (dict(W=None), bd.FS_ERR_INVALID_ARG),
    (dict(T=None), bd.FS_ERR_INVALID_ARG),
    (dict(ids=None), bd.FS_ERR_INVALID_ARG),
    (dict(ws=None), bd.FS_ERR_INVALID_ARG),
    (dict(h=ALIGNED + 8), bd.FS_ERR_INVALID_ARG),
    (dict(W=ALIGNED + 2), bd.FS_ERR_INVALID_ARG),
    (dict(T=ALIGNED + 1), bd.FS_ERR_INVALID_ARG),
    (dict(ws=WS_ALIGNED + 16), bd.FS_ERR_INVALID_ARG),
    (dict(wsb=16), bd.FS_ERR_WORKSPACE),
    (dict(B=0, h=None, W=None, T=None, ids=None, val=None, ws=None), bd.FS_OK),
])
def test_argument_errors(L, fn, kw, status):
    assert _sample(L, fn, **kw) == status
    if status != bd.FS_OK:
        assert len(L.fs_last_error()) > 0


def test_workspace_sizes(L):
    # B = 0 is a valid no-op and needs no workspace
    assert L.fs_workspace_bytes(0, 256, 1000) == 0
    assert L.fs_workspace_bytes(4, 7, 1000) == 0          # invalid D
    ws = L.fs_workspace_bytes(32, 4096, 128256)
    assert ws >= 8 * 32 * (128256 // 64) and ws % 256 == 0
    unf = L.fs_unfused_workspace_bytes(32, 4096, 128256)
    assert unf >= 2 * 4 * 32 * 128256                     # logits + probabilities
    # exactly-sized workspace passes the size check (then fails on alignment)
    need = L.fs_workspace_bytes(4, 256, 1000)
    assert _sample(L, wsb=need - 1) == bd.FS_ERR_WORKSPACE
    assert _sample(L, wsb=need, ws=WS_ALIGNED + 4) == bd.FS_ERR_INVALID_ARG


def test_merge_argument_errors(L):
    assert L.fs_merge(ALIGNED, ALIGNED, 0, 4, ALIGNED, ALIGNED, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_merge(ALIGNED, ALIGNED, 2, -1, ALIGNED, ALIGNED, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_merge(None, ALIGNED, 2, 4, ALIGNED, ALIGNED, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_merge(ALIGNED + 2, ALIGNED, 2, 4, ALIGNED, ALIGNED, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_merge(None, None, 3, 0, None, None, None) == bd.FS_OK


def test_debug_argument_errors(L):
    assert L.fs_debug_noise(0, 0, 0, 0, -1, ALIGNED, ALIGNED, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_debug_noise(0, 0, 0, 2**32 - 4, 5, ALIGNED, ALIGNED, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_debug_noise(0, 0, 0, 0, 0, None, None, None) == bd.FS_OK
    assert L.fs_debug_gumbel(None, 5, ALIGNED, None) == bd.FS_ERR_INVALID_ARG


def test_configs(L):
    n = L.fs_num_configs()
    assert n >= 5
    names = [L.fs_config_name(i).decode() for i in range(n)]
    assert len(set(names)) == n
    assert L.fs_config_name(n) is None
    assert L.fs_force_config(n) == bd.FS_ERR_INVALID_ARG
    assert L.fs_force_config(-2) == bd.FS_ERR_INVALID_ARG
    auto = [L.fs_selected_config(B, 4096, 128256) for B in (1, 32, 64, 128, 256)]
    assert all(0 <= c < n for c in auto)
    assert L.fs_force_config(n - 1) == bd.FS_OK
    assert L.fs_selected_config(1, 4096, 128256) == n - 1
    assert L.fs_force_config(-1) == bd.FS_OK
    assert L.fs_selected_config(1, 4096, 128256) == auto[0]
    assert L.fs_selected_config(1, 7, 10) == -1


def _sample_lse(L, h=ALIGNED, W=ALIGNED, B=4, D=256, V=1000, off=0, T=ALIGNED, val=ALIGNED,
                ids=ALIGNED, lse=ALIGNED, ws=WS_ALIGNED, wsb=1 << 30):
    return L.fs_sample_partial_lse(h, W, B, D, V, off, T, 1, 2, val, ids, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=7), bd.FS_ERR_INVALID_ARG),
    (dict(V=0), bd.FS_ERR_INVALID_ARG),
    (dict(B=-1), bd.FS_ERR_INVALID_ARG),
    (dict(off=-5), bd.FS_ERR_INVALID_ARG),
    (dict(h=None), bd.FS_ERR_INVALID_ARG),
    (dict(lse=None), bd.FS_ERR_INVALID_ARG),
    (dict(lse=ALIGNED + 2), bd.FS_ERR_INVALID_ARG),
    (dict(ids=ALIGNED + 1), bd.FS_ERR_INVALID_ARG),
    (dict(W=ALIGNED + 8), bd.FS_ERR_INVALID_ARG),
    (dict(wsb=16), bd.FS_ERR_WORKSPACE),
    (dict(B=0, h=None, W=None, T=None, ids=None, val=None, lse=None, ws=None), bd.FS_OK),
])
def test_sample_partial_lse_argument_errors(L, kw, status):
    assert _sample_lse(L, **kw) == status
    if status != bd.FS_OK:
        assert len(L.fs_last_error()) > 0


def _merge_lse(L, val=ALIGNED, ids=ALIGNED, lse=ALIGNED, P=2, B=4, T=ALIGNED, out_ids=ALIGNED,
               out_val=ALIGNED, out_lse=ALIGNED):
    return L.fs_merge_lse(val, ids, lse, P, B, T, 1, 2, out_ids, out_val, out_lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(P=0), bd.FS_ERR_INVALID_ARG),
    (dict(B=-1), bd.FS_ERR_INVALID_ARG),
    (dict(lse=None), bd.FS_ERR_INVALID_ARG),
    (dict(T=None), bd.FS_ERR_INVALID_ARG),
    (dict(out_lse=None), bd.FS_ERR_INVALID_ARG),
    (dict(val=ALIGNED + 2), bd.FS_ERR_INVALID_ARG),
    (dict(out_lse=ALIGNED + 1), bd.FS_ERR_INVALID_ARG),
    (dict(P=1 << 20, B=1 << 21), bd.FS_ERR_INVALID_ARG),
    (dict(B=0, val=None, ids=None, lse=None, T=None, out_ids=None, out_val=None, out_lse=None),
     bd.FS_OK),
])
def test_merge_lse_argument_errors(L, kw, status):
    assert _merge_lse(L, **kw) == status


def test_workspace_covers_the_shifted_grid(L):
    """Unaligned vocabulary offsets shift the tile grid by up to 3 rows, which
    can add one block of 16 rows: the workspace is sized for it."""
    for V in (13, 16, 17, 1000, 16032):
        ws = L.fs_workspace_bytes(5, 256, V)
        assert ws >= 3 * 4 * 5 * ((V + 3 + 15) // 16)


# ---- online sampler with early finalisation ----
def _cuts(*c):
    return (ctypes.c_int32 * len(c))(*c)


def _online(L, h=ALIGNED, W=ALIGNED, B=4, D=256, V=1000, off=0, T=ALIGNED, cuts=None, n=2,
            later=ALIGNED, ids=ALIGNED, val=ALIGNED, chunks=ALIGNED, ws=WS_ALIGNED,
            wsb=1 << 30):
    cuts = _cuts(0, 500, 1000) if cuts is None else cuts
    return L.fs_sample_online(h, W, B, D, V, off, T, 1, 2, cuts, n, later, ids, val, chunks, ws,
                              wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cuts=_cuts(0, 500, 999)), bd.FS_ERR_INVALID_ARG),        # does not end at V
    (dict(cuts=_cuts(1, 500, 1000)), bd.FS_ERR_INVALID_ARG),       # does not start at 0
    (dict(cuts=_cuts(0, 600, 600, 1000), n=3), bd.FS_ERR_INVALID_ARG),  # empty chunk
    (dict(cuts=_cuts(0, 700, 300, 1000), n=3), bd.FS_ERR_INVALID_ARG),  # decreasing
    (dict(n=0), bd.FS_ERR_INVALID_ARG),
    (dict(n=70000), bd.FS_ERR_INVALID_ARG),
    (dict(later=None), bd.FS_ERR_INVALID_ARG),
    (dict(later=ALIGNED + 4), bd.FS_ERR_INVALID_ARG),
    (dict(chunks=None), bd.FS_ERR_INVALID_ARG),
    (dict(chunks=ALIGNED + 2), bd.FS_ERR_INVALID_ARG),
    (dict(D=7), bd.FS_ERR_INVALID_ARG),
    (dict(h=None), bd.FS_ERR_INVALID_ARG),
    (dict(W=ALIGNED + 8), bd.FS_ERR_INVALID_ARG),
    (dict(D=32776, cuts=_cuts(0, 500, 1000)), bd.FS_ERR_UNSUPPORTED),
    (dict(wsb=16), bd.FS_ERR_WORKSPACE),
    (dict(B=0, h=None, W=None, T=None, later=None, ids=None, val=None, chunks=None, ws=None),
     bd.FS_OK),
])
def test_online_argument_errors(L, kw, status):
    assert _online(L, **kw) == status
    if status != bd.FS_OK:
        assert len(L.fs_last_error()) > 0


def test_online_workspace_sizes(L):
    assert L.fs_online_workspace_bytes(4, 7, 1000, 2) == 0
    assert L.fs_online_workspace_bytes(4, 256, 1000, 0) == 0
    need = L.fs_online_workspace_bytes(4, 256, 1000, 2)
    assert need >= L.fs_workspace_bytes(4, 256, 1000) + 4 * (8 + 4) + 2 * 4
    assert need % 256 == 0
    assert _online(L, wsb=need - 1) == bd.FS_ERR_WORKSPACE
    assert _online(L, wsb=need, ws=WS_ALIGNED + 4) == bd.FS_ERR_INVALID_ARG
    assert L.fs_online_bounds_workspace_bytes(0, 2) == 0
    assert L.fs_online_bounds_workspace_bytes(1000, 2) >= 8 * 1000 + 8 * 2


def test_online_bounds_argument_errors(L):
    c = _cuts(0, 500, 1000)
    ok = dict(W=ALIGNED, V=1000, D=256, cuts=c, n=2, later=ALIGNED, ws=WS_ALIGNED, wsb=1 << 30)

    def call(**kw):
        a = {**ok, **kw}
        return L.fs_online_bounds(a["W"], a["V"], a["D"], a["cuts"], a["n"], a["later"], a["ws"],
                                  a["wsb"], None)
    assert call(cuts=_cuts(0, 500, 900)) == bd.FS_ERR_INVALID_ARG
    assert call(W=None) == bd.FS_ERR_INVALID_ARG
    assert call(W=ALIGNED + 2) == bd.FS_ERR_INVALID_ARG
    assert call(later=ALIGNED + 4) == bd.FS_ERR_INVALID_ARG
    assert call(D=12) == bd.FS_ERR_INVALID_ARG
    assert call(ws=WS_ALIGNED + 8) == bd.FS_ERR_INVALID_ARG
    assert call(wsb=8) == bd.FS_ERR_WORKSPACE


# ---- fragment-order weights ----
def test_packed_sizes_and_errors(L):
    assert L.fs_packed_weights_bytes(1000, 256, 0) == 63 * 16 * 256 * 2   # 1000 rows -> 63 groups
    assert L.fs_packed_weights_bytes(1000, 256, 7) == 63 * 16 * 256 * 2   # shift 3: 1003 rows
    assert L.fs_packed_weights_bytes(1024, 256, 1) == 65 * 16 * 256 * 2
    assert L.fs_packed_weights_bytes(1000, 264, 0) == 0                   # D % 32 != 0
    assert L.fs_packed_weights_bytes(0, 256, 0) == 0
    need = L.fs_packed_weights_bytes(1000, 256, 0)
    assert L.fs_pack_weights(ALIGNED, 1000, 264, 0, ALIGNED, 1 << 30, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_pack_weights(None, 1000, 256, 0, ALIGNED, 1 << 30, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_pack_weights(ALIGNED, 1000, 256, 0, ALIGNED + 8, 1 << 30, None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_pack_weights(ALIGNED, 1000, 256, 0, ALIGNED, need - 1, None) == bd.FS_ERR_WORKSPACE
    # the packed sampler validates like fs_sample, plus D % 32
    assert _sample(L, "fs_sample_packed", D=264) == bd.FS_ERR_INVALID_ARG
    assert _sample(L, "fs_sample_packed", h=None) == bd.FS_ERR_INVALID_ARG
    assert _sample(L, "fs_sample_packed", wsb=16) == bd.FS_ERR_WORKSPACE
    assert _sample(L, "fs_sample_packed", B=0, h=None, W=None, T=None, ids=None, val=None,
                   ws=None) == bd.FS_OK


def test_online_packed_argument_errors(L):
    def call(cuts, n=2, D=256, **kw):
        a = dict(h=ALIGNED, W=ALIGNED, B=4, V=1000, off=0, T=ALIGNED, later=ALIGNED, ids=ALIGNED,
                 val=ALIGNED, chunks=ALIGNED, ws=WS_ALIGNED, wsb=1 << 30)
        a.update(kw)
        return L.fs_sample_online_packed(a["h"], a["W"], a["B"], D, a["V"], a["off"], a["T"], 1, 2,
                                         cuts, n, a["later"], a["ids"], a["val"], a["chunks"],
                                         a["ws"], a["wsb"], None)
    assert call(_cuts(0, 500, 1000)) == bd.FS_ERR_INVALID_ARG        # 500 % 16 != 0
    assert call(_cuts(0, 512, 1000), D=264) == bd.FS_ERR_INVALID_ARG  # D % 32 != 0
    assert call(_cuts(0, 512, 999)) == bd.FS_ERR_INVALID_ARG          # does not end at V
    assert call(_cuts(0, 512, 1000), wsb=16) == bd.FS_ERR_WORKSPACE


def test_partial_lse_packed_argument_errors(L):
    def call(**kw):
        a = dict(h=ALIGNED, W=ALIGNED, B=4, D=256, V=1000, off=0, T=ALIGNED, pv=ALIGNED,
                 pi=ALIGNED, pl=ALIGNED, ws=WS_ALIGNED, wsb=1 << 30)
        a.update(kw)
        return L.fs_sample_partial_lse_packed(a["h"], a["W"], a["B"], a["D"], a["V"], a["off"],
                                              a["T"], 1, 2, a["pv"], a["pi"], a["pl"], a["ws"],
                                              a["wsb"], None)
    assert call(D=264) == bd.FS_ERR_INVALID_ARG
    assert call(pl=None) == bd.FS_ERR_INVALID_ARG
    assert call(wsb=16) == bd.FS_ERR_WORKSPACE
    assert call(B=0, h=None, W=None, T=None, pv=None, pi=None, pl=None, ws=None) == bd.FS_OK


def test_online_bounds_packed_argument_errors(L):
    c = _cuts(0, 512, 1000)
    assert L.fs_online_bounds_packed(ALIGNED, 1000, 264, 0, c, 2, ALIGNED, WS_ALIGNED, 1 << 30,
                                     None) == bd.FS_ERR_INVALID_ARG      # D % 32
    assert L.fs_online_bounds_packed(None, 1000, 256, 0, c, 2, ALIGNED, WS_ALIGNED, 1 << 30,
                                     None) == bd.FS_ERR_INVALID_ARG
    assert L.fs_online_bounds_packed(ALIGNED, 1000, 256, -1, c, 2, ALIGNED, WS_ALIGNED, 1 << 30,
                                     None) == bd.FS_ERR_INVALID_ARG      # negative offset
    assert L.fs_online_bounds_packed(ALIGNED, 1000, 256, 0, c, 2, ALIGNED, WS_ALIGNED, 8,
                                     None) == bd.FS_ERR_WORKSPACE


def test_selected_config_packed(L):
    """The packed choice is a valid configuration that reads packed W wherever
    one applies (host-side logic only; without a device the CU count is
    unknown and the DMA grids count as unfilled)."""
    n = L.fs_num_configs()
    assert L.fs_selected_config_packed(4, 7, 1000) == -1          # invalid D
    for B, D, V in [(1, 4096, 128256), (32, 4096, 128256), (4, 256, 1000), (1, 5120, 151936),
                    (64, 8192, 16032), (300, 4096, 128256)]:
        cp, cr = L.fs_selected_config_packed(B, D, V), L.fs_selected_config(B, D, V)
        assert 0 <= cp < n and 0 <= cr < n
        name = L.fs_config_name(cp).decode()
        assert not name.startswith("ksplit"), name                # K-split reads row-major W only
        if name.startswith("persist"):
            assert name.endswith("_ntl1"), name                   # packed persistent twins
    # the persistent choices at the Llama-3 head
    assert L.fs_config_name(L.fs_selected_config_packed(1, 4096, 128256)) == \
        b"persist_nt1_nw16_ks8_p4_ntl1"
    assert L.fs_config_name(L.fs_selected_config_packed(32, 4096, 128256)) == \
        b"persist_nt2_nw8_ks16_p4_ntl1"


def test_unfused_workspace_size_does_not_wrap(L):
    """Sizes are computed in size_t: at B = 2^29 the logits alone take
    4 * B * ldz bytes, past the range of a 32-bit product."""
    B, V = 1 << 29, 64
    need = L.fs_unfused_workspace_bytes(B, 8, V)
    assert need >= 2 * 4 * B * V
    assert L.fs_unfused_workspace_bytes(2 * B, 8, V) >= 2 * need - 4096


def test_batch_limits_are_refused_on_the_host(L):
    # the unfused baseline puts one batch row per grid row (at most 65535)
    assert _sample(L, "fs_sample_unfused", B=65536, wsb=1 << 62) == bd.FS_ERR_UNSUPPORTED
    assert b"65535" in L.fs_last_error()
    # the samplers' batch blocks (>= 16 rows) form the grid's y dimension
    for fn in ("fs_sample", "fs_sample_partial", "fs_sample_packed"):
        assert _sample(L, fn, B=16 * 65535 + 1, wsb=1 << 62) == bd.FS_ERR_UNSUPPORTED, fn
        assert b"1048560" in L.fs_last_error()


@pytest.fixture
def inject(monkeypatch):
    monkeypatch.setenv("FS_FAULT_INJECT", "launch")
    yield


def test_injected_launch_failure_every_entry_point(L, inject):
    """With FS_FAULT_INJECT=launch a call whose arguments pass the checks
    returns FS_ERR_HIP with the reason in fs_last_error, and launches
    nothing (the fake pointers below are never touched)."""
    A, WS, big = ALIGNED, WS_ALIGNED, 1 << 40
    cuts = (ctypes.c_int32 * 3)(0, 512, 1000)
    calls = {
        "fs_sample": lambda: _sample(L, "fs_sample"),
        "fs_sample_partial": lambda: _sample(L, "fs_sample_partial"),
        "fs_sample_packed": lambda: _sample(L, "fs_sample_packed"),
        "fs_sample_packed_noalloc": lambda: L.fs_sample_packed_noalloc(A, A, 4, 256, 1000, 0, A, 1,
                                                                       2, A, A, None),
        "fs_sample_unfused": lambda: _sample(L, "fs_sample_unfused"),
        "fs_sample_partial_lse": lambda: _sample_lse(L),
        "fs_merge": lambda: L.fs_merge(A, A, 3, 4, A, A, None),
        "fs_merge_lse": lambda: L.fs_merge_lse(A, A, A, 3, 4, A, 1, 2, A, A, A, None),
        "fs_pack_weights": lambda: L.fs_pack_weights(A, 1000, 256, 0, A, big, None),
        "fs_online_bounds": lambda: L.fs_online_bounds(A, 1000, 256, cuts, 2, A, WS, big, None),
        "fs_sample_online": lambda: L.fs_sample_online(A, A, 4, 256, 1000, 0, A, 1, 2, cuts, 2,
                                                       A, A, A, A, WS, big, None),
        "fs_sample_groups_lse": lambda: L.fs_sample_groups_lse(A, A, 4, 256, 1000, 0, A, 1, 2, cuts,
                                                               2, A, A, A, WS, big, None),
        "fs_sample_groups_lse_packed": lambda: L.fs_sample_groups_lse_packed(
            A, A, 4, 256, 1000, 0, A, 1, 2, cuts, 2, A, A, A, WS, big, None),
        "fs_debug_noise": lambda: L.fs_debug_noise(0, 0, 0, 0, 16, A, A, None),
        "fs_debug_gumbel": lambda: L.fs_debug_gumbel(A, 16, A, None),
    }
    for name, call in calls.items():
        assert call() == bd.FS_ERR_HIP, name
        msg = L.fs_last_error()
        assert name.encode() in msg and b"FS_FAULT_INJECT" in msg, (name, msg)


def test_injection_does_not_mask_argument_errors(L, inject):
    assert _sample(L, D=7) == bd.FS_ERR_INVALID_ARG
    assert _sample(L, wsb=16) == bd.FS_ERR_WORKSPACE
    assert _sample(L, B=0, h=None, W=None, T=None, ids=None, val=None, ws=None) == bd.FS_OK


@pytest.mark.skipif(gpu_available(), reason="needs a machine without a GPU")
def test_launch_without_a_device_reports_the_runtime_error(L, monkeypatch):
    """Where no device exists the launch itself fails: FS_ERR_HIP carries
    the runtime's message."""
    monkeypatch.delenv("FS_FAULT_INJECT", raising=False)
    assert _sample(L) == bd.FS_ERR_HIP
    assert len(L.fs_last_error()) > 0 and b"FS_FAULT_INJECT" not in L.fs_last_error()


def _noalloc(L, h=ALIGNED, W=ALIGNED, B=4, D=256, V=1000, off=0, T=ALIGNED, ids=ALIGNED,
             val=ALIGNED):
    return L.fs_sample_packed_noalloc(h, W, B, D, V, off, T, 1, 2, ids, val, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=7), bd.FS_ERR_INVALID_ARG),
    (dict(D=72), bd.FS_ERR_INVALID_ARG),            # packed weights need D % 32 == 0
    (dict(V=0), bd.FS_ERR_INVALID_ARG),
    (dict(B=-1), bd.FS_ERR_INVALID_ARG),
    (dict(h=None), bd.FS_ERR_INVALID_ARG),
    (dict(T=ALIGNED + 2), bd.FS_ERR_INVALID_ARG),
    (dict(W=ALIGNED + 8), bd.FS_ERR_INVALID_ARG),
    (dict(B=16 * 65535 + 1), bd.FS_ERR_UNSUPPORTED),
    # partials beyond the 8 MiB scratch array, refused before any launch
    (dict(B=2048, V=200000), bd.FS_ERR_WORKSPACE),
    (dict(B=1 << 19, V=1 << 20), bd.FS_ERR_WORKSPACE),
    (dict(B=0, h=None, W=None, T=None, ids=None, val=None), bd.FS_OK),
])
def test_noalloc_argument_errors(L, kw, status):
    assert _noalloc(L, **kw) == status
    if status != bd.FS_OK:
        assert len(L.fs_last_error()) > 0
    if status == bd.FS_ERR_WORKSPACE:
        assert b"scratch" in L.fs_last_error()


def _groups(L, fn="fs_sample_groups_lse", h=ALIGNED, W=ALIGNED, B=4, D=256, V=1000, off=0,
            T=ALIGNED, cuts=(0, 512, 1000), n=None, val=ALIGNED, ids=ALIGNED, lse=ALIGNED,
            ws=WS_ALIGNED, wsb=1 << 40):
    c = (ctypes.c_int32 * len(cuts))(*cuts) if cuts is not None else None
    n = len(cuts) - 1 if n is None else n
    return getattr(L, fn)(h, W, B, D, V, off, T, 1, 2, c, n, val, ids, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cuts=None, n=2), bd.FS_ERR_INVALID_ARG),
    (dict(cuts=(0, 600, 600, 1000)), bd.FS_ERR_INVALID_ARG),         # empty group
    (dict(cuts=(1, 500, 1000)), bd.FS_ERR_INVALID_ARG),              # does not start at 0
    (dict(cuts=(0, 500, 999)), bd.FS_ERR_INVALID_ARG),               # does not end at V
    (dict(n=0), bd.FS_ERR_INVALID_ARG),
    (dict(cuts=tuple(range(0, 1001, 15)) + (1000,), n=None), bd.FS_ERR_INVALID_ARG),  # 67 groups
    (dict(lse=None), bd.FS_ERR_INVALID_ARG),
    (dict(lse=ALIGNED + 2), bd.FS_ERR_INVALID_ARG),
    (dict(D=7), bd.FS_ERR_INVALID_ARG),
    (dict(wsb=16), bd.FS_ERR_WORKSPACE),
    (dict(fn="fs_sample_groups_lse_packed", cuts=(0, 500, 1000)), bd.FS_ERR_INVALID_ARG),
    (dict(fn="fs_sample_groups_lse_packed", D=72, cuts=(0, 512, 1000)), bd.FS_ERR_INVALID_ARG),
    (dict(B=0, h=None, W=None, T=None, val=None, ids=None, lse=None, ws=None), bd.FS_OK),
])
def test_groups_argument_errors(L, kw, status):
    assert _groups(L, **kw) == status
    if status != bd.FS_OK:
        assert len(L.fs_last_error()) > 0


def test_groups_refuse_a_forced_configuration_that_does_not_fit(L):
    names = [L.fs_config_name(i).decode() for i in range(L.fs_num_configs())]
    persist = names.index("persist_nt1_nw8_ks16_p8")   # needs D = 4096
    assert L.fs_force_config(persist) == bd.FS_OK
    try:
        assert _groups(L, D=256) == bd.FS_ERR_UNSUPPORTED
        assert b"does not support" in L.fs_last_error()
    finally:
        L.fs_force_config(-1)


def test_groups_workspace_sizes(L):
    assert L.fs_groups_workspace_bytes(4, 256, 1000, 0) == 0
    assert L.fs_groups_workspace_bytes(4, 256, 1000, 65) == 0
    need = L.fs_groups_workspace_bytes(4, 256, 1000, 2)
    assert need >= L.fs_workspace_bytes(4, 256, 1000) and need % 256 == 0
    assert _groups(L, wsb=need - 1) == bd.FS_ERR_WORKSPACE
    assert _groups(L, wsb=need, ws=WS_ALIGNED + 4) == bd.FS_ERR_INVALID_ARG


def test_groups_automatic_choice_is_the_plain_one(L):
    """A grouped launch takes the configuration fs_sample (fs_sample_packed)
    takes, persistent ones included."""
    assert L.fs_selected_config_groups(4, 7, 1000, 0) == -1
    for packed in (0, 1):
        for B in (1, 4, 8, 32, 64, 256, 512):
            for D, V in ((4096, 128256), (8192, 16032), (256, 1000)):
                c = L.fs_selected_config_groups(B, D, V, packed)
                plain = (L.fs_selected_config_packed if packed else L.fs_selected_config)(B, D, V)
                assert c == plain, (B, D, V, packed)
