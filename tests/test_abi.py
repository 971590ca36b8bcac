"""Host-side checks of the C-ABI library (no GPU compute): it loads, exports
every function include/ec.h declares, and rejects bad descriptors on the host."""
import ctypes
import math

import pytest

import error_bounded_lossy_amd as ec


def test_library_exports_every_declared_symbol():
    L = ec.lib()
    names = ec.declared_functions()
    assert {"ec_plan", "ec_compress", "ec_decompress", "ec_ratio"} <= set(names)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings():
    assert ec.status_string(ec.EC_OK) == "ok"
    assert ec.status_string(ec.EC_ERR_CORRUPT) == "corrupt stream"
    assert ec.status_string(99) == "unknown status"


def test_workspace_sizing_and_descriptor_validation():
    ok = ec.workspace_bytes(26, 8192, 128, 1, ec.EB_REL_RANGE, 0.005,
                            schedule={"kind": ec.SCHED_INV_SQRT, "t0": 1000.0})
    assert ok > 0 and ok % 256 == 0
    # hash tables alone: 26 segments x 16384 slots x 8 bytes
    assert ok > 26 * 16384 * 8
    bad = [
        dict(T=0, B=10, D=4),
        dict(T=1, B=10, D=0),
        dict(T=1, B=10, D=4, P=0),
        dict(T=1, B=10, D=4, eb=0.0),
        dict(T=1, B=10, D=4, eb=math.nan),
        dict(T=1, B=10, D=4, eb=math.inf),
        dict(T=1, B=10, D=4, eb=3e38),                     # 2*eb overflows
        dict(T=1, B=10, D=4, eb_mode=1, eb=-0.1),
        dict(T=1, B=10, D=4, eb_mode=7),
        dict(T=1, B=10, D=4, table_mult=[0.0]),
        dict(T=1, B=10, D=4, schedule={"kind": ec.SCHED_INV_SQRT, "t0": 0.0}),
        dict(T=1, B=10, D=4, schedule={"kind": ec.SCHED_STEP, "phase": 0}),
        dict(T=1, B=10, D=4, schedule={"kind": 9}),
    ]
    for kw in bad:
        kw = dict(kw)
        T, B, D = kw.pop("T"), kw.pop("B"), kw.pop("D")
        assert ec.workspace_bytes(T, B, D, **kw) == 0, kw
    # D beyond what one workgroup's LDS can stage is unsupported
    assert ec.workspace_bytes(1, 10, 1 << 16) == 0


def test_plan_rejects_bad_arguments_before_touching_the_device():
    L = ec.lib()
    keep = []
    d = ec._desc(1, 10, 4, 1, ec.EB_ABS, 0.0, None, None, 0, keep)
    h = ctypes.c_void_p()
    assert L.ec_plan(ctypes.byref(d), ctypes.byref(h)) == ec.EC_ERR_INVALID
    assert not h.value
    assert L.ec_plan(None, ctypes.byref(h)) == ec.EC_ERR_INVALID
    assert L.ec_compress(None, 0, None, None, 0, None) == ec.EC_ERR_INVALID
    assert L.ec_decompress(None, None, 0, None, None) == ec.EC_ERR_INVALID
    assert L.ec_ratio(None, None, None, None) == ec.EC_ERR_INVALID
    assert L.ec_max_compressed_bytes(None) == 0
    # a descriptor that gives a workspace size but no workspace, or a
    # misaligned workspace, is rejected on the host (no workspace at all, size
    # 0, is a plan for ec_compress_static)
    d = ec._desc(1, 10, 4, 1, ec.EB_ABS, 1e-3, None, None, 0, keep)
    d.workspace_bytes = 1 << 20
    assert L.ec_plan(ctypes.byref(d), ctypes.byref(h)) == ec.EC_ERR_INVALID
    d.d_workspace = 0x1010
    assert L.ec_plan(ctypes.byref(d), ctypes.byref(h)) == ec.EC_ERR_INVALID
    assert not h.value
    assert L.ec_compress_static(None, 0, None, None, 0, None) == ec.EC_ERR_INVALID


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    monkeypatch.setattr(ec, "_lib", None)
    monkeypatch.setattr(ec, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        ec.lib()


def test_huffman_entry_points_check_arguments_on_the_host():
    L = ec.lib()
    assert L.ec_huff_workspace_bytes() > 4 * 4096
    # 12 bits per symbol, each 256-symbol chunk rounded up to whole words
    assert L.ec_huff_max_words(0) == 0
    assert L.ec_huff_max_words(1) == 1
    assert L.ec_huff_max_words(256) == 96
    assert L.ec_huff_max_words(257) == 97
    assert L.ec_huff_max_words(256 * 1000 + 3) == 96 * 1000 + 2
    wb = L.ec_huff_workspace_bytes()
    fake = 1 << 20  # never dereferenced: every call below fails its host checks
    enc = L.ec_huff_encode
    assert enc(fake, 1000, None, fake, fake, 10**6, fake, wb, None) == ec.EC_ERR_INVALID
    assert enc(fake, 1 << 31, fake, fake, fake, 1 << 40, fake, wb, None) == ec.EC_ERR_INVALID
    assert enc(fake + 2, 1000, fake, fake, fake, 10**6, fake, wb, None) == ec.EC_ERR_INVALID
    assert enc(fake, 1000, fake, fake, fake, 10**6, fake + 16, wb, None) == ec.EC_ERR_INVALID
    assert enc(fake, 1000, fake, fake, fake, 374, fake, wb, None) == ec.EC_ERR_CAPACITY
    assert enc(fake, 1000, fake, fake, fake, 10**6, fake, wb - 1, None) == ec.EC_ERR_CAPACITY
    dec = L.ec_huff_decode
    assert dec(None, 4, fake, fake, 10, 10, fake, fake, wb, None) == ec.EC_ERR_INVALID
    assert dec(fake, 4, fake, fake, 10, 10, fake, fake, wb - 1, None) == ec.EC_ERR_CAPACITY
    assert L.ec_huff_status(None, None) == ec.EC_ERR_INVALID
    # segments: a workspace per segment count, limits checked on the host
    assert L.ec_huff_workspace_bytes_segments(0) == 0
    assert L.ec_huff_workspace_bytes_segments(2049) == 0
    assert L.ec_huff_workspace_bytes_segments(1) == wb
    w26 = L.ec_huff_workspace_bytes_segments(26)
    assert w26 > wb and w26 - wb >= 25 * 10 * 4096  # histogram, codes, table per segment
    es = L.ec_huff_encode_segments
    assert es(fake, 0, 100, fake, fake, fake, 10**6, fake, w26, None) == ec.EC_ERR_INVALID
    assert es(fake, 2049, 100, fake, fake, fake, 10**8, fake, 1 << 30, None) == ec.EC_ERR_INVALID
    assert es(fake, 26, 1 << 27, fake, fake, fake, 1 << 40, fake, w26, None) == ec.EC_ERR_INVALID
    assert es(fake, 26, 1000, fake, fake, fake, 26 * 375 - 1, fake, w26, None) == ec.EC_ERR_CAPACITY
    assert es(fake, 26, 1000, fake, fake, fake, 10**6, fake, wb, None) == ec.EC_ERR_CAPACITY
    ds = L.ec_huff_decode_segments
    assert ds(fake, fake, fake, 10, 0, 10, fake, fake, w26, None) == ec.EC_ERR_INVALID
    assert ds(fake, fake, fake, 10, 26, 10, fake, fake, wb, None) == ec.EC_ERR_CAPACITY


def test_table_classification_matches_the_oracle():
    """ec_classify_tables (host code in the library) against the oracle's
    Algorithm 1 on random homogenization indices, thresholds and multipliers,
    threshold ties included; invalid arguments are rejected."""
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(7)
    for _ in range(50):
        T = int(rng.integers(1, 40))
        lo, hi = sorted(rng.uniform(0, 1, 2))
        h = rng.uniform(0, 1, T)
        h[: T // 4] = lo
        h[T // 4: T // 2] = hi
        alpha, beta = float(rng.uniform(1, 4)), float(rng.uniform(1, 4))
        cls, mult = ec.classify_tables(h, lo, hi, alpha, beta)
        ocls, omult = O.classify(h, lo, hi, alpha, beta)
        assert cls == [int(c) for c in ocls]
        assert np.array_equal(np.array(mult, np.float32), omult)
    for bad in [(0.5, 0.4, 2.0, 2.0), (0.1, 0.3, 0.0, 2.0), (0.1, 0.3, 2.0, float("inf"))]:
        with pytest.raises(ec.ECError):
            ec.classify_tables([0.2], *bad)


def test_speedup_and_selection_match_the_oracle():
    """ec_speedup / ec_select_coders (host code in the library) against the
    oracle's eq. (2) and Algorithm 2 on random pools, ties included (the
    earlier compressor wins); invalid pools are rejected."""
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(11)
    for _ in range(200):
        cr, bw, tc, td = (float(v) for v in rng.uniform(0.5, 50, 4))
        assert ec.speedup(cr, bw, tc, td) == O.speedup(cr, bw, tc, td)
    for _ in range(50):
        C, T = int(rng.integers(1, 5)), int(rng.integers(1, 30))
        cr = rng.uniform(1, 20, (C, T))
        tc, td = rng.uniform(10, 400, C), rng.uniform(10, 400, C)
        if C > 1:
            cr[1, : T // 3] = cr[0, : T // 3]  # a tie where the pool's
            tc[1], td[1] = tc[0], td[0]        # first two are the same
        bw = float(rng.uniform(0.5, 50))
        best, sp = ec.select_coders(cr.tolist(), tc.tolist(), td.tolist(), bw)
        obest, osp = O.select(cr, tc, td, bw)
        assert best == [int(b) for b in obest]
        assert np.array_equal(np.array(sp), osp)
    for bad in [([[2.0]], [0.0], [1.0], 1.0), ([[2.0]], [1.0], [1.0], float("nan")),
                ([[-1.0]], [1.0], [1.0], 1.0), ([[2.0]], [1.0], [float("inf")], 1.0)]:
        with pytest.raises(ec.ECError):
            ec.select_coders(*bad)
    with pytest.raises(ec.ECError):
        ec.select_coders([], [], [], 1.0)


def test_table_coder_validation():
    """A per-table coder array is checked like the plan's coder; Huffman
    tables need the wave64 paths (D = 64, 128, 256)."""
    assert ec.workspace_bytes(3, 100, 128, table_coder=[1, 2, 3]) > 0
    assert ec.workspace_bytes(3, 100, 24, table_coder=[1, 1, 1]) > 0
    assert ec.workspace_bytes(3, 100, 24, table_coder=[1, 2, 1]) == 0
    assert ec.workspace_bytes(3, 100, 128, table_coder=[1, 4, 1]) == 0
    assert ec.workspace_bytes(2, 100, 128, table_coder=[0, 1]) == 0


def test_window_validation():
    """Windowed references: W <= 255, wave64 dims only, at most 32768 rows per
    segment."""
    assert ec.workspace_bytes(2, 100, 128, window=255) > 0
    assert ec.workspace_bytes(2, 100, 64, window=1, coder=ec.CODER_AUTO) > 0
    assert ec.workspace_bytes(2, 100, 128, window=256) == 0
    assert ec.workspace_bytes(2, 100, 24, window=8) == 0
    assert ec.workspace_bytes(1, 32768, 64, window=8) > 0
    assert ec.workspace_bytes(1, 32769, 64, window=8) == 0
    assert ec.workspace_bytes(1, 65536, 64, P=2, window=8) > 0
