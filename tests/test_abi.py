"""The C ABI without a GPU: the library loads, exports every entry point that
include/entmax.h declares, and rejects bad arguments before any launch (the
pointers used here are never dereferenced: validation fails first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "entmax.h")
LIB = os.path.join(ROOT, "adaptive_sparse_attention_row_amd", "libentmax.so")

FAKE = 4096  # non-null, 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(entmax_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def api():
    if not os.path.exists(LIB):
        pytest.fail("libentmax.so is not built (run __graft_entry__.build())")
    from adaptive_sparse_attention_row_amd import api as a
    a.lib()
    return a


def test_header_symbols_exported(api):
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(api):
    for s in range(11):
        assert api.status_str(s) and api.status_str(s) != "unknown status"
    assert api.status_str(99) == "unknown status"


def test_tile_shape(api):
    assert api.tile_shape(64, api.BF16) == (64, 64)
    assert api.tile_shape(128, api.F32) == (64, 64)
    L = api.lib()
    br, bc = ctypes.c_int(), ctypes.c_int()
    assert L.entmax_tile_shape(96, 1, ctypes.byref(br), ctypes.byref(bc)) == api.ERR_SHAPE
    assert L.entmax_tile_shape(64, 7, ctypes.byref(br), ctypes.byref(bc)) == api.ERR_DTYPE
    assert L.entmax_tile_shape(64, 1, None, ctypes.byref(bc)) == api.ERR_NULL


def test_tau_rows_validation(api):
    L = api.lib()
    f = L.entmax_tau_rows
    assert f(None, None, FAKE, 4, 8, 8, 1.5, None) == api.ERR_NULL
    assert f(FAKE, None, None, 4, 8, 8, 1.5, None) == api.ERR_NULL
    for bad in (2.5, 1.0, 0.0, float("nan")):
        assert f(FAKE, None, FAKE, 4, 8, 8, bad, None) == api.ERR_ALPHA
    assert f(FAKE, None, FAKE, -1, 8, 8, 1.5, None) == api.ERR_SHAPE
    assert f(FAKE, None, FAKE, 4, 0, 8, 1.5, None) == api.ERR_SHAPE
    assert f(FAKE, None, FAKE, 4, 9, 8, 1.5, None) == api.ERR_SHAPE
    assert f(None, None, None, 0, 8, 8, 1.5, None) == api.OK   # empty: no-op


def fwd(L, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, tau=FAKE, bm=FAKE, B=1, H=1, Ls=128, d=64,
             scale=0.125, alpha=1.5, dtype=1, mask=0, window=0, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return L.entmax_attn_fwd(a["Q"], a["K"], a["V"], a["O"], a["tau"], a["bm"], a["B"], a["H"],
                             a["Ls"], a["d"], a["scale"], a["alpha"], a["dtype"], a["mask"],
                             a["window"], a["ws"], a["wsb"], None)


def test_attn_fwd_validation(api):
    L = api.lib()
    assert fwd(L, Q=None) == api.ERR_NULL
    assert fwd(L, tau=None) == api.ERR_NULL
    for bad in (2.5, 1.0, float("nan")):
        assert fwd(L, alpha=bad) == api.ERR_ALPHA
    assert fwd(L, dtype=5) == api.ERR_DTYPE
    assert fwd(L, mask=3) == api.ERR_MASK
    assert fwd(L, mask=2, window=-1) == api.ERR_MASK
    assert fwd(L, d=96) == api.ERR_SHAPE
    assert fwd(L, Ls=0) == api.ERR_SHAPE
    assert fwd(L, Ls=65537) == api.ERR_SHAPE
    assert fwd(L, B=0) == api.ERR_SHAPE
    assert fwd(L, scale=0.0) == api.ERR_ARG
    assert fwd(L, scale=float("nan")) == api.ERR_ARG
    assert fwd(L, Q=FAKE + 4) == api.ERR_ALIGN
    assert fwd(L, O=FAKE + 8) == api.ERR_ALIGN
    need = L.entmax_attn_fwd_workspace(1, 1, 128, 64, 1, 0, 0)
    need_thr = L.entmax_attn_threshold_workspace(1, 1, 128, 64, 1, 0, 0)
    assert need > need_thr > 0
    assert fwd(L, ws=None) == api.ERR_WORKSPACE
    assert fwd(L, bm=None, wsb=need - 1) == api.ERR_WORKSPACE
    assert fwd(L, wsb=need_thr - 1) == api.ERR_WORKSPACE
    assert fwd(L, ws=FAKE + 8) == api.ERR_ALIGN
    assert L.entmax_attn_fwd_workspace(1, 1, 128, 96, 1, 0, 0) == 0
    thr = L.entmax_attn_threshold
    base = [FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.125, 1.5, 1, 0, 0, FAKE, need_thr, None]
    def tcall(i, v):
        a = list(base)
        a[i] = v
        return thr(*a)
    assert tcall(3, None) == api.ERR_NULL
    assert tcall(9, 1.0) == api.ERR_ALPHA
    assert tcall(13, None) == api.ERR_WORKSPACE
    assert tcall(14, need_thr - 1) == api.ERR_WORKSPACE
    out = L.entmax_attn_output
    assert out(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 128, 64, 0.125, 1.5, 1, 0, 0, None) == api.ERR_NULL
    assert out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.125, 1.5, 1, 3, 0, None) == api.ERR_MASK


def test_attn_bwd_validation(api):
    L = api.lib()
    f = L.entmax_attn_bwd
    need = L.entmax_attn_bwd_workspace(1, 2, 100, 64, 1, 1, 0)
    assert need >= 2 * 100 * 4
    base = [FAKE] * 9 + [1, 2, 100, 64, 0.125, 1.5, 1, 1, 0, FAKE, need, None]
    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(0, None) == api.ERR_NULL      # Q
    assert call(5, None) == api.ERR_NULL      # block mask
    assert call(8, None) == api.ERR_NULL      # dV
    assert call(14, 1.0) == api.ERR_ALPHA
    assert call(15, 9) == api.ERR_DTYPE
    assert call(16, 4) == api.ERR_MASK
    assert call(12, 32) == api.ERR_SHAPE
    assert call(13, -1.0) == api.ERR_ARG
    assert call(18, None) == api.ERR_WORKSPACE
    assert call(19, need - 1) == api.ERR_WORKSPACE
    assert call(6, FAKE + 4) == api.ERR_ALIGN


def test_gv_validation(api):
    """The training pair: bf16 and L <= 16384 only; GV and gsum required."""
    L = api.lib()
    # a caller-held mask: the threshold workspace suffices
    need = L.entmax_attn_threshold_workspace(1, 2, 100, 64, 1, 1, 0)
    f = L.entmax_attn_fwd_gv
    base = [FAKE] * 8 + [1, 2, 100, 64, 0.125, 1.5, 1, 1, 0, FAKE, need, None]
    def call(i, v):
        a = list(base)
        a[i] = v
        return f(*a)
    assert call(6, None) == api.ERR_NULL      # GV
    assert call(7, None) == api.ERR_NULL      # gsum
    assert call(14, 0) == api.ERR_DTYPE       # fp32
    assert call(10, 16448) == api.ERR_SHAPE   # L above the fused kernel's range
    assert call(6, FAKE + 4) == api.ERR_ALIGN
    assert call(0, None) == api.ERR_NULL      # Q, as in entmax_attn_fwd
    assert call(18, need - 1) == api.ERR_WORKSPACE
    bneed = L.entmax_attn_bwd_workspace(1, 2, 100, 64, 1, 1, 0)
    b = L.entmax_attn_bwd_gv
    bbase = [FAKE] * 11 + [1, 2, 100, 64, 0.125, 1.5, 1, 1, 0, FAKE, bneed, None]
    def bcall(i, v):
        a = list(bbase)
        a[i] = v
        return b(*a)
    assert bcall(6, None) == api.ERR_NULL     # GV
    assert bcall(7, None) == api.ERR_NULL     # gsum
    assert bcall(17, 0) == api.ERR_DTYPE
    assert bcall(13, 16448) == api.ERR_SHAPE
    assert bcall(10, None) == api.ERR_NULL    # dV
    assert bcall(21, bneed - 1) == api.ERR_WORKSPACE


def test_options_validation(api):
    """Per-call options: out-of-range values are rejected before any launch."""
    import ctypes as C
    L = api.lib()
    bad = [api.Options(-1, 0), api.Options(129, 0), api.Options(0, 2)]
    for o in bad:
        assert L.entmax_tau_rows_ex(FAKE, None, FAKE, 4, 8, 8, 1.5, C.byref(o), None) == api.ERR_ARG
        assert L.entmax_attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.125, 1.5, 1, 0, 0,
                                    FAKE, 1 << 24, C.byref(o), None) == api.ERR_ARG
        assert L.entmax_attn_threshold_ex(FAKE, FAKE, FAKE, FAKE, 1, 1, 128, 64, 0.125, 1.5, 1, 0, 0,
                                          FAKE, 1 << 24, C.byref(o), None) == api.ERR_ARG
    # NULL options and an all-zero struct are the defaults: rows == 0 is a no-op either way
    assert L.entmax_tau_rows_ex(None, None, None, 0, 8, 8, 1.5, None, None) == api.OK
    assert L.entmax_tau_rows_ex(None, None, None, 0, 8, 8, 1.5, C.byref(api.Options(0, 0)), None) == api.OK


def test_decode_validation(api):
    L = api.lib()

    def call(q=FAKE, K=FAKE, V=FAKE, O=FAKE, tau=FAKE, B=1, H=2, Lk=100, cap=128, d=64, scale=0.125,
             alpha=1.5, dtype=1, mask=1, window=0, ws=FAKE, wsb=1 << 20):
        return L.entmax_attn_decode(q, K, V, O, tau, B, H, Lk, cap, d, scale, alpha, dtype, mask, window,
                                    ws, wsb, None)

    assert call(q=None) == api.ERR_NULL
    assert call(tau=None) == api.ERR_NULL
    assert call(alpha=2.5) == api.ERR_ALPHA
    assert call(dtype=7) == api.ERR_DTYPE
    assert call(mask=3) == api.ERR_MASK
    assert call(mask=2, window=-1) == api.ERR_MASK
    assert call(Lk=0) == api.ERR_SHAPE
    assert call(Lk=200, cap=100) == api.ERR_SHAPE   # L beyond the cache
    assert call(d=96) == api.ERR_SHAPE
    assert call(scale=0.0) == api.ERR_ARG
    assert call(q=FAKE + 4) == api.ERR_ALIGN
    assert call(wsb=10) == api.ERR_WORKSPACE
    assert call(ws=None) == api.ERR_WORKSPACE
    # 4 bytes per active key per head; the window keeps key 0 and W + 1 recent keys
    assert L.entmax_attn_decode_workspace(2, 3, 1000, 64, 1, 1, 0) == 2 * 3 * 1000 * 4
    assert L.entmax_attn_decode_workspace(2, 3, 1000, 64, 1, 2, 32) == 2 * 3 * 34 * 4
    assert L.entmax_attn_decode_workspace(2, 3, 20, 64, 1, 2, 32) == 2 * 3 * 20 * 4
    assert L.entmax_attn_decode_workspace(1, 1, 10, 96, 1, 1, 0) == 0


def test_decode_noalloc_validation(api):
    """The allocation-free decode checks its arguments like the decode, and
    rejects inputs whose scores do not fit its static scratch, all before
    touching the device."""
    L = api.lib()

    def call(q=FAKE, K=FAKE, V=FAKE, O=FAKE, tau=FAKE, B=1, H=2, Lk=100, cap=128, d=64, scale=0.125,
             alpha=1.5, dtype=1, mask=1, window=0):
        return L.entmax_attn_decode_noalloc(q, K, V, O, tau, B, H, Lk, cap, d, scale, alpha, dtype, mask,
                                            window, None)

    assert call(q=None) == api.ERR_NULL
    assert call(alpha=0.9) == api.ERR_ALPHA
    assert call(Lk=200, cap=100) == api.ERR_SHAPE
    assert call(scale=float("inf")) == api.ERR_ARG
    assert call(K=FAKE + 8) == api.ERR_ALIGN
    limit = 32 << 20                        # ENTMAX_DECODE_SCRATCH_BYTES
    keys = limit // 4                       # active keys over all heads that fit
    assert call(B=1, H=1, Lk=keys + 1, cap=keys + 1) == api.ERR_SCRATCH
    assert call(B=2, H=4, Lk=keys // 8 + 1, cap=keys // 8 + 1) == api.ERR_SCRATCH
    # a window keeps the active keys per head small whatever the cache length
    assert L.entmax_attn_decode_workspace(64, 64, 1 << 20, 64, 1, 2, 32) <= limit
