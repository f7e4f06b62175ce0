"""C-ABI checks that need no GPU: the library loads, exports every function
include/ffn.h declares, and rejects bad arguments before launching anything.

Pointers used here are fake non-null addresses; every call below fails
validation (or is an M == 0 no-op) before any device access, which is the
documented contract ("validated before anything is launched")."""
import ctypes
import os
import re

import pytest

from transformer_ffn_block_amd import ffn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "ffn.h")

A = 0x10000000      # fake 256-byte-aligned device addresses, never dereferenced
B = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000
Y = 0x60000000
WS = 0x70000000


def declared_functions():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ffn_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ffn.LIB_PATH):
        pytest.fail("libffn.so not built: run `python -m transformer_ffn_block_amd.build`")
    return ffn.lib()


def test_header_declares_the_three_block_entry_points():
    names = declared_functions()
    for n in ("ffn_rmsnorm", "ffn_swiglu_block", "ffn_swiglu_block_q8", "ffn_swiglu_block_q4"):
        assert n in names


def test_library_exports_every_declared_function(L):
    names = declared_functions()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # and the binding's signature table covers exactly the header
    assert sorted(ffn.exported_symbols()) == names


def test_status_strings(L):
    for code, name in enumerate(["FFN_OK", "FFN_ERR_INVALID_ARGUMENT", "FFN_ERR_UNSUPPORTED",
                                 "FFN_ERR_WORKSPACE", "FFN_ERR_LAUNCH"]):
        assert L.ffn_status_string(code).decode() == name
    assert L.ffn_status_string(99).decode() == "FFN_ERR_UNKNOWN"


def _block(L, dt=ffn.FFN_BF16, x=A, g=B, wg=C, wu=D, wd=E, y=Y, M=16, d=4096, f=11008,
           eps=1e-6, v=0, ws=WS, wsb=None):
    if wsb is None:
        wsb = L.ffn_swiglu_block_workspace_size(dt, M, d, f, v)
    return L.ffn_swiglu_block(dt, x, g, wg, wu, wd, y, M, d, f, eps, v, ws, wsb, None)


def test_block_validation(L):
    INV, UNS, WSE = ffn.FFN_ERR_INVALID_ARGUMENT, ffn.FFN_ERR_UNSUPPORTED, ffn.FFN_ERR_WORKSPACE
    assert _block(L, x=0) == INV
    assert _block(L, wd=0) == INV
    assert _block(L, dt=7) == INV
    assert _block(L, v=9) == INV
    assert _block(L, M=-1) == INV
    assert _block(L, d=0) == INV
    assert _block(L, f=-8) == INV
    assert _block(L, eps=-1.0) == INV
    assert _block(L, eps=float("nan")) == INV
    assert _block(L, d=4100) == UNS                    # bf16 needs d % 8 == 0
    assert _block(L, dt=ffn.FFN_F32, d=258, f=704) == UNS
    assert _block(L, x=A + 2) == UNS                   # misaligned
    assert _block(L, ws=WS + 16) == UNS                # workspace must be 256-aligned
    assert _block(L, wsb=100) == WSE
    assert _block(L, ws=0) == WSE
    assert _block(L, y=A) == INV                       # y aliases x
    assert _block(L, y=WS) == INV                      # y inside the workspace
    assert "overlaps" in L.ffn_last_error().decode()
    assert _block(L, wsb=100) == WSE
    assert "workspace" in L.ffn_last_error().decode()


def test_persistent_variant_scope(L):
    UNS = ffn.FFN_ERR_UNSUPPORTED
    P = ffn.VARIANTS["persistent"]
    assert _block(L, v=P, M=17) == UNS                       # at most 16 tokens
    assert _block(L, v=P, dt=ffn.FFN_F32, d=256, f=704) == UNS  # bf16 only
    assert _block(L, v=5) == ffn.FFN_ERR_INVALID_ARGUMENT
    assert _block(L, v=P, M=0, ws=0, wsb=0) == ffn.FFN_OK


def test_block_zero_tokens_is_a_noop(L):
    assert _block(L, M=0, ws=0, wsb=0) == ffn.FFN_OK
    assert L.ffn_last_error().decode() == ""


def _tile_m(M):
    """Token tile of the prefill GEMMs: 128 up to 128 tokens, else 256."""
    return 128 if M <= 128 else 256


def _prefill_splits_rule(M, N, K, bno, cus=256):
    """The documented split rule for a prefill GEMM (128- or 256-token tiles,
    bno weight rows per tile, 64-deep K tiles in ranges of two when they pair
    up)."""
    if K % 64:
        return 1
    bm = _tile_m(M)
    tiles = -(-M // bm) * -(-N // bno)
    nk = K // 64
    pp = M % bm == 0 and N % bno == 0 and K % 128 == 0
    units = nk // 2 if (pp or nk % 2 == 0) else nk
    z = min(cus // tiles, 16, units)
    return max(z, 1)


def _prefill_plan_rule(M, N, K, bno, slots=256):
    """(main, z): output columns [0, main) unsplit, the rest over z K ranges.
    A GEMM with fewer tiles than compute units splits whole; past one round
    of `slots` resident tiles (whole tiles, K in pairs of 64-deep tiles), the
    columns filling the earlier rounds run unsplit and the rest -- at most
    half a round -- split into as many ranges as fill one round."""
    z = _prefill_splits_rule(M, N, K, bno)
    if z > 1:
        return 0, z
    bm = _tile_m(M)
    if not (M % bm == 0 and N % bno == 0 and K % 128 == 0):
        return N, 1
    mt, nt = M // bm, N // bno
    if mt * nt <= slots:
        return N, 1
    nm = (-(-mt * nt // slots) - 1) * slots // mt
    if nm < 1 or nm >= nt:
        return N, 1
    zt = min(slots // (mt * (nt - nm)), 16, K // 128)
    return (nm * bno, zt) if zt >= 2 else (N, 1)


@pytest.mark.parametrize("M,d,f", [(65, 4096, 11008), (128, 4096, 11008), (256, 1024, 2048),
                                   (300, 512, 768), (512, 4096, 14336), (1000, 4096, 11008),
                                   (2048, 5120, 13824), (4096, 4096, 14336), (100, 1032, 576),
                                   (777, 2048, 704), (768, 4096, 11008), (1024, 4096, 11008),
                                   (4352, 4096, 1024), (1536, 4096, 11008), (128, 512, 38400),
                                   (128, 512, 76800), (96, 4096, 11008)])
def test_prefill_split_workspace(L, M, d, f):
    """Above 64 tokens the bf16 workspace adds one fp32 region for split-K
    partials: 2 Z_gu [M, f - main] planes (fused gate/up) or Z_dn
    [M, d - main] planes (down), whichever is larger, with the plans from the
    documented rule on 256 CUs (the count assumed without a device); SPLIT
    plans only the down GEMM."""
    def r256(n):
        return (n + 255) // 256 * 256
    cg, zg = _prefill_plan_rule(M, f, d, 128)
    cd, zd = _prefill_plan_rule(M, d, f, 256)
    pg = 2 * zg * M * (f - cg) * 4 if zg > 1 else 0
    pd = zd * M * (d - cd) * 4 if zd > 1 else 0
    base = r256(M * d * 2) + r256(M * f * 2)
    part = r256(max(pg, pd)) if max(pg, pd) else 0
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, 1) == base + part
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, 2) == \
        base + 2 * r256(M * f * 2) + (r256(pd) if pd else 0)
    # fp32 blocks never split
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_F32, M, d, f, 1) == r256(M * d * 4) + r256(M * f * 4)


def test_prefill_tail_plans():
    """The plans the rule gives for shapes just past whole rounds: 768 tokens
    at f = 11008 have 258 gate/up tiles, so 85 column tiles (255 tiles) run
    unsplit and the last 3 split 16 ways; 4352 tokens at d = 4096 have 272
    down tiles, the last column's 17 split over all 8 K ranges of f = 1024."""
    assert _prefill_plan_rule(768, 11008, 4096, 128) == (85 * 128, 16)
    assert _prefill_plan_rule(1024, 11008, 4096, 128) == (64 * 128, 2)
    assert _prefill_plan_rule(4352, 4096, 1024, 256) == (15 * 256, 8)
    assert _prefill_plan_rule(768, 4096, 11008, 256) == (0, 5)
    # 128 tokens take 128-token tiles: 300 fused gate/up tiles at f = 38400
    # are 44 past a round, split over the 4 K ranges of d = 512
    assert _prefill_plan_rule(128, 38400, 512, 128) == (256 * 128, 4)
    # whole rounds: no split
    assert _prefill_plan_rule(8192, 14336, 4096, 128) == (14336, 1)
    assert _prefill_plan_rule(8192, 4096, 14336, 256) == (4096, 1)


def test_workspace_sizes(L):
    def r256(n):
        return (n + 255) // 256 * 256
    M, d, f = 16, 4096, 11008
    fused = L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, 1)
    split = L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, 2)
    assert fused == r256(M * d * 2) + r256(M * f * 2)
    assert split == fused + 2 * r256(M * f * 2)
    # bf16 decode regime (M <= 64, fused schedule): h in the decode kernels'
    # blocked layout, whole 16-token tiles of ceil(f / 128) 128-k stages;
    # SPLIT and prefill keep h row-major [M, f]
    for m, ff in ((1, 11008), (20, 704), (64, 1000)):
        blk = ((m + 15) // 16 * 16) * ((ff + 127) // 128 * 128) * 2
        assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, m, d, ff, 0) == r256(m * d * 2) + r256(blk)
        assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, m, d, ff, 2) == r256(m * d * 2) + 3 * r256(m * ff * 2)
    # prefill (M > 64) GEMMs whose tiles leave compute units idle split K and
    # add fp32 partial planes: at M = 65, d = 4096, f = 704 on 256 CUs (the
    # count assumed without a device) the fused gate/up GEMM has 6 tiles ->
    # 16 ranges (2 x 16 planes of [65, 704]), the down GEMM 16 tiles -> 11
    # ranges (its K = 704 holds 11 K tiles of 64): one region for the larger
    base = r256(65 * d * 2) + r256(65 * 704 * 2)
    part = max(2 * 16 * 65 * 704 * 4, 11 * 65 * d * 4)
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, 65, d, 704, 0) == base + r256(part)
    # SPLIT: only the down GEMM splits; 8192 tokens fill the chip: no partials
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, 65, d, 704, 2) == base + 2 * r256(65 * 704 * 2) + r256(11 * 65 * d * 4)
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, 8192, d, 14336, 0) == r256(8192 * d * 2) + r256(8192 * 14336 * 2)
    assert L.ffn_swiglu_block_workspace_size(ffn.FFN_F32, 8, 256, 704, 0) == r256(8 * 256 * 4) + r256(8 * 704 * 4)
    assert L.ffn_swiglu_block_workspace_size(5, M, d, f, 0) == 0
    # persistent: plus [S, M, d] fp32 partials and 2 + S + d/16 counter words
    pers = L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, 3)
    assert any(pers == fused + r256(s * M * d * 4) + r256((2 + s + d // 16) * 4) for s in range(1, 9))
    # quantised blocks: plus the split-K partials of the down projection, 4 K
    # ranges for 320 output tiles, [4, min(M, 32), d] fp32; Q8 with up to 8
    # tokens (Q4: narrow projections only) folds the norm and needs no n
    assert L.ffn_swiglu_block_q8_workspace_size(8, 5120, 17408) == \
        r256(8 * 17408 * 2) + 4 * 8 * 5120 * 4
    sp = 4  # ceil(1024 / 320) ranges for the 320 row tiles of the down projection
    assert L.ffn_swiglu_block_q8_workspace_size(8, 5120, 2176) == \
        r256(8 * 2176 * 2) + r256(sp * 8 * 5120 * 4)
    assert L.ffn_swiglu_block_q8_workspace_size(9, 5120, 2176) == \
        r256(9 * 5120 * 2) + r256(9 * 2176 * 2) + r256(sp * 9 * 5120 * 4)
    assert L.ffn_swiglu_block_q4_workspace_size(8, 5120, 17408) == \
        r256(8 * 5120 * 2) + r256(8 * 17408 * 2) + 4 * 8 * 5120 * 4
    assert L.ffn_swiglu_block_q4_workspace_size(64, 5120, 17408) == \
        r256(64 * 5120 * 2) + r256(64 * 17408 * 2) + 4 * 32 * 5120 * 4
    assert L.ffn_swiglu_block_q4_workspace_size(-1, 5120, 17408) == 0
    # d = 4096: 256 row tiles fill a round of 256 CUs, so up to 16 tokens the
    # down projection runs unsplit (no partials); 32 tokens split 4 ways
    assert L.ffn_swiglu_block_q8_workspace_size(8, 4096, 11008) == r256(8 * 11008 * 2)
    assert L.ffn_swiglu_block_q8_workspace_size(16, 4096, 11008) == \
        r256(16 * 4096 * 2) + r256(16 * 11008 * 2)
    assert L.ffn_swiglu_block_q8_workspace_size(32, 4096, 11008) == \
        r256(32 * 4096 * 2) + r256(32 * 11008 * 2) + r256(4 * 32 * 4096 * 4)
    assert L.ffn_swiglu_block_q4_workspace_size(16, 4096, 11008) == \
        r256(16 * 4096 * 2) + r256(16 * 11008 * 2)
    # beyond the weight-streaming regime the quantised blocks take no call
    assert L.ffn_swiglu_block_q4_workspace_size(65, 5120, 17408) == 0
    assert L.ffn_swiglu_block_q8_workspace_size(65, 5120, 17408) == 0


def test_rmsnorm_validation(L):
    INV, UNS = ffn.FFN_ERR_INVALID_ARGUMENT, ffn.FFN_ERR_UNSUPPORTED
    f = L.ffn_rmsnorm
    assert f(ffn.FFN_BF16, 0, B, Y, 4, 64, 1e-6, None) == INV
    assert f(3, A, B, Y, 4, 64, 1e-6, None) == INV
    assert f(ffn.FFN_BF16, A, B, Y, -1, 64, 1e-6, None) == INV
    assert f(ffn.FFN_BF16, A, B, Y, 4, 0, 1e-6, None) == INV
    assert f(ffn.FFN_BF16, A, B, Y, 4, 60, 1e-6, None) == UNS
    assert f(ffn.FFN_F32, A, B, Y, 4, 6, 1e-6, None) == UNS
    assert f(ffn.FFN_BF16, A, B + 8, Y, 4, 64, 1e-6, None) == UNS
    assert f(ffn.FFN_BF16, A, B, A + 64, 4, 64, 1e-6, None) == INV   # overlap
    assert f(ffn.FFN_BF16, A, B, Y, 0, 64, 1e-6, None) == ffn.FFN_OK


def test_q8_validation(L):
    INV, UNS = ffn.FFN_ERR_INVALID_ARGUMENT, ffn.FFN_ERR_UNSUPPORTED
    good = ffn.Q8Matrix(C, D)
    g2 = ffn.Q8Matrix(E, E + 0x1000000)
    g3 = ffn.Q8Matrix(E + 0x2000000, E + 0x3000000)
    ref = ctypes.byref

    def call(M=8, d=5120, f=17408, mg=good, mu=g2, md=g3, ws=WS, wsb=None, x=A):
        if wsb is None:
            wsb = L.ffn_swiglu_block_q8_workspace_size(M, d, f)
        return L.ffn_swiglu_block_q8(x, B, ref(mg), ref(mu), ref(md), Y, M, d, f, 1e-6, ws, wsb, None)

    assert call(d=5128) == UNS                       # d % 32 != 0
    assert call(mg=ffn.Q8Matrix(0, D)) == INV
    assert call(mg=ffn.Q8Matrix(C + 8, D)) == UNS     # quants 16-byte aligned
    assert call(x=0) == INV
    assert call(wsb=10) == ffn.FFN_ERR_WORKSPACE
    assert call(M=0, ws=0, wsb=0) == ffn.FFN_OK
    assert call(M=65, wsb=1 << 30) == UNS            # more tokens than the streaming regime
    assert "at most 64 tokens" in L.ffn_last_error().decode()
    assert L.ffn_swiglu_block_q8(A, B, None, ref(g2), ref(g3), Y, 8, 5120, 17408, 1e-6, WS, 1 << 30, None) == INV


def test_q4_validation(L):
    INV, UNS = ffn.FFN_ERR_INVALID_ARGUMENT, ffn.FFN_ERR_UNSUPPORTED
    good = ffn.Q4Matrix(C, D)
    g2 = ffn.Q4Matrix(E, E + 0x1000000)
    g3 = ffn.Q4Matrix(E + 0x2000000, E + 0x3000000)
    ref = ctypes.byref

    def call(M=8, d=5120, f=17408, mg=good, mu=g2, md=g3, ws=WS, wsb=None, x=A, y=Y):
        if wsb is None:
            wsb = L.ffn_swiglu_block_q4_workspace_size(M, d, f)
        return L.ffn_swiglu_block_q4(x, B, ref(mg), ref(mu), ref(md), y, M, d, f, 1e-6, ws, wsb, None)

    assert call(d=5136) == UNS                       # d % 32 != 0
    assert call(f=17400) == UNS                      # f % 32 != 0
    assert call(mg=ffn.Q4Matrix(0, D)) == INV
    assert call(md=ffn.Q4Matrix(E, 0)) == INV
    assert call(mu=ffn.Q4Matrix(E + 8, E + 0x1000000)) == UNS   # nibbles 16-byte aligned
    assert call(mu=ffn.Q4Matrix(E, E + 0x1000001)) == UNS       # scales 2-byte aligned
    assert call(x=0) == INV
    assert call(wsb=10) == ffn.FFN_ERR_WORKSPACE
    assert call(M=0, ws=0, wsb=0) == ffn.FFN_OK
    assert call(M=65, wsb=1 << 30) == UNS            # more tokens than the streaming regime
    # 2^31 bytes of nibbles: d * f = 2^32 weights
    assert call(M=1, d=65536, f=65536) == UNS
    # just under the limit passes validation up to the aliasing check: y inside qs
    assert call(M=1, d=65536, f=32768 - 32, y=C) == INV
    assert L.ffn_swiglu_block_q4(A, B, None, ref(g2), ref(g3), Y, 8, 5120, 17408, 1e-6, WS, 1 << 30, None) == INV


def test_persistent_status_offset(L):
    def r256(n):
        return (n + 255) // 256 * 256
    M, d, f = 16, 4096, 11008
    need = L.ffn_swiglu_block_workspace_size(ffn.FFN_BF16, M, d, f, 3)
    off = L.ffn_swiglu_block_persistent_status_offset(M, d, f)
    # word 1 of the counter region, which ends the workspace: 2 + S + d/16 words
    assert any(off == need - r256((2 + s + d // 16) * 4) + 4 for s in range(1, 9))
    assert off > r256(M * d * 2) + r256(M * f * 2)
    assert L.ffn_swiglu_block_persistent_status_offset(17, d, f) == 0
    assert L.ffn_swiglu_block_persistent_status_offset(0, d, f) == 0


def test_timing_state_is_per_thread(L):
    """Timing switched on in one thread is invisible to another; the other
    thread's calls and its own switch are unaffected (no process-global
    mutable state besides the library's code)."""
    import threading
    seen = {}
    ev_on, ev_checked = threading.Event(), threading.Event()

    def a():
        seen["a_enable"] = L.ffn_timing_enable(1, 64)
        seen["a_on"] = L.ffn_timing_enabled()
        ev_on.set()
        ev_checked.wait(10)
        seen["a_still_on"] = L.ffn_timing_enabled()
        seen["a_disable"] = L.ffn_timing_enable(0, 0)
        seen["a_off"] = L.ffn_timing_enabled()

    def b():
        ev_on.wait(10)
        seen["b_on"] = L.ffn_timing_enabled()
        seen["b_count"] = L.ffn_timing_count()
        # validation errors on this thread leave the other thread's state alone
        seen["b_call"] = _block(L, x=0)
        seen["b_err"] = L.ffn_last_error().decode()
        seen["b_disable"] = L.ffn_timing_enable(0, 0)
        ev_checked.set()

    ta, tb = threading.Thread(target=a), threading.Thread(target=b)
    ta.start(); tb.start(); ta.join(20); tb.join(20)
    assert seen["a_enable"] == ffn.FFN_OK and seen["a_on"] == 1
    assert seen["b_on"] == 0 and seen["b_count"] == 0
    assert seen["b_call"] == ffn.FFN_ERR_INVALID_ARGUMENT and "null" in seen["b_err"]
    assert seen["b_disable"] == ffn.FFN_OK
    assert seen["a_still_on"] == 1                    # b's switch did not touch a's
    assert seen["a_disable"] == ffn.FFN_OK and seen["a_off"] == 0
    assert L.ffn_timing_enabled() == 0                # nor the main thread's


def test_error_text_is_per_thread(L):
    import threading
    got = {}
    assert _block(L, d=4100) == ffn.FFN_ERR_UNSUPPORTED
    main_err = L.ffn_last_error().decode()

    def other():
        got["fresh"] = L.ffn_last_error().decode()
        _block(L, x=0)
        got["own"] = L.ffn_last_error().decode()
    t = threading.Thread(target=other)
    t.start(); t.join(10)
    assert got["fresh"] == ""
    assert "null" in got["own"]
    assert L.ffn_last_error().decode() == main_err


def test_probe_and_timing_validation(L):
    INV = ffn.FFN_ERR_INVALID_ARGUMENT
    assert L.ffn_probe_read(A, 15, B, 4, None) == INV
    assert L.ffn_probe_read(A, 1 << 20, B, 0, None) == INV
    assert L.ffn_probe_copy(A, A + 16, 64, 0, 0, None) == INV     # overlap
    assert L.ffn_probe_copy(A, B, 64, 65, 0, None) == INV         # groups per CU 0..64
    assert L.ffn_probe_copy(A, B, 24, 0, 0, None) == INV          # multiple of 16
    assert L.ffn_probe_copy(A, B, 0, 0, 1, None) == ffn.FFN_OK    # nothing to copy
    assert L.ffn_probe_mfma(0, 8, A, None) == INV
    assert L.ffn_probe_mfma(10, 33, A, None) == INV
    assert L.ffn_probe_mfma(10, 8, 0, None) == INV
    assert L.ffn_probe_mfma_groups(0) == 0
    assert L.ffn_timing_enable(1, 0) == INV
    assert L.ffn_timing_enable(0, 0) == ffn.FFN_OK
    assert L.ffn_timing_count() == 0
