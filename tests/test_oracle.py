"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
rational arithmetic, closed forms, brute force on tiny inputs, an
independent stream reader written from the layout spec, or numbers printed
on the pages (arXiv 2407.04272).
"""
from fractions import Fraction
import math
import os

import numpy as np
import pytest

import oracle as O
import streamfmt as SF

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(v):
    return float(np.float32(v))


# --------------------------------------------------------------------------
# quantization encoder (section III-D): q = round(x / 2eb), |x - x^| <= eb
# --------------------------------------------------------------------------
def test_ties_round_half_to_even():
    # eb = 0.5 -> bin width 1: exact ties go to the even bin
    for x, q in [(0.5, 0), (1.5, 2), (2.5, 2), (3.5, 4), (-0.5, 0), (-1.5, -2), (-2.5, -2)]:
        got, out = O.quantize(x, 0.5)
        assert (got, out) == (q, False), x


def test_quantizer_matches_exact_rounding_away_from_ties():
    rng = np.random.default_rng(1)
    for _ in range(4000):
        eb = f32(10.0 ** rng.uniform(-8, 1))
        x = f32(rng.uniform(-2040, 2040) * 2 * eb)
        ratio = Fraction(x) / (2 * Fraction(eb))
        frac = ratio - math.floor(ratio)
        if abs(frac - Fraction(1, 2)) < Fraction(1, 1000):
            continue  # near a tie: covered by the bound test below
        want = round(ratio)
        got, out = O.quantize(x, eb)
        assert not out and got == want, (x, eb)


def test_bound_holds_exactly_for_every_value():
    rng = np.random.default_rng(2)
    n_out = 0
    for _ in range(6000):
        eb = f32(10.0 ** rng.uniform(-10, 2))
        x = f32(rng.choice([1.0, -1.0]) * 10.0 ** rng.uniform(-12, 4))
        q, out = O.quantize(x, eb)
        if out:
            n_out += 1
            assert q == 0
            continue
        assert abs(q) <= 2047
        xh = O.dequantize(q, eb)
        assert abs(Fraction(x) - Fraction(xh)) <= Fraction(eb), (x, eb, q)
    assert n_out > 0


def test_float_quotient_on_a_tie_that_is_not_a_tie():
    # Search values whose rounded quotient fl(x/s) is exactly k + 1/2 while the
    # true quotient is not: round-half-even may pick the far bin.  The value is
    # an outlier exactly when its fp32 reconstruction fl(q*s) misses eb, judged
    # here in exact rational arithmetic.
    rng = np.random.default_rng(3)
    found_far = 0
    for _ in range(200000):
        eb = f32(rng.uniform(0.5, 1.0))
        s = np.float32(eb) + np.float32(eb)
        k = int(rng.integers(1, 2000))
        x = np.float32((k + 0.5) * float(s))
        x = np.nextafter(x, np.float32(np.inf) if rng.random() < 0.5 else np.float32(-np.inf))
        t = np.float32(x) / s
        if float(t) != k + 0.5:
            continue
        exact = Fraction(float(x)) / Fraction(float(s))
        if exact == Fraction(2 * k + 1, 2):
            continue
        q, out = O.quantize(float(x), eb)
        near = math.floor(exact + Fraction(1, 2))          # the correct bin
        rne = k if k % 2 == 0 else k + 1                   # what RNE of k + 1/2 picks
        xh = np.float32(rne) * s                           # reconstruction is fl(q * s)
        misses = abs(Fraction(float(x)) - Fraction(float(xh))) > Fraction(eb)
        assert out == misses, (float(x), eb, k)
        if not out:
            assert q == rne        # kept: its fp32 reconstruction still meets eb
            assert abs(q - near) <= 1
        else:
            found_far += 1
            assert q == 0          # stored verbatim instead
    assert found_far > 0


def test_out_of_range_nan_inf_are_outliers():
    for x in [math.nan, math.inf, -math.inf, 1e30, -1e30]:
        q, out = O.quantize(x, 1e-3)
        assert out and q == 0
    # 2047 bins is the largest code
    assert O.quantize(2047.0, 0.5) == (2047, False)
    assert O.quantize(2048.0, 0.5) == (0, True)


def test_integer_values_with_dyadic_eb_round_trip_exactly():
    for k in range(0, 6):
        eb = 2.0 ** (-1 - k)            # bin width 2^-k
        xs = np.arange(-(2047 >> k), (2047 >> k) + 1, dtype=np.float32)
        for x in xs[:: max(1, xs.size // 200)]:
            q, out = O.quantize(float(x), eb)
            assert not out and O.dequantize(q, eb) == float(x)


def test_zigzag_is_a_bijection_on_the_code_range():
    zs = [O.zigzag(q) for q in range(-2047, 2048)]
    assert sorted(zs) == list(range(0, 4095))
    assert all(O.unzigzag(O.zigzag(q)) == q for q in range(-2047, 2048))
    assert max(zs).bit_length() == 12


# --------------------------------------------------------------------------
# error-bound policy (section III-C, Algorithm 1)
# --------------------------------------------------------------------------
def test_inverse_sqrt_schedule_closed_forms():
    cfg = O.Config(T=1, B=1, D=1, sched_kind=O.SCHED_INV_SQRT, sched_t0=1000.0)
    assert O.schedule(cfg, 0) == 1.0
    assert O.schedule(cfg, 3000) == 0.5      # 4^-1/2
    assert O.schedule(cfg, 15000) == 0.25    # 16^-1/2
    vals = [O.schedule(cfg, i) for i in range(10)]
    assert all(a > b for a, b in zip(vals, vals[1:]))
    assert O.schedule(cfg, -5) == 1.0        # negative iterations clamp to 0


def test_staircase_schedule_closed_forms():
    # Decay_2x (Fig. 10 caption): from twice the base eb down to the base eb
    cfg = O.Config(T=1, B=1, D=1, sched_kind=O.SCHED_STEP, sched_k=2.0, sched_phase=100,
                   sched_steps=4)
    want = {0: 2.0, 24: 2.0, 25: 1.75, 49: 1.75, 50: 1.5, 75: 1.25, 99: 1.25, 100: 1.0,
            10 ** 6: 1.0}
    for i, v in want.items():
        assert O.schedule(cfg, i) == v, i
    none = O.Config(T=1, B=1, D=1)
    assert O.schedule(none, 12345) == 1.0


def test_drop_schedule_closed_form():
    # Drop_2x (Fig. 10 caption): twice the base eb for the whole initial phase,
    # the base eb from the end of that phase on -- the staircase with one stair
    cfg = O.Config(T=1, B=1, D=1, sched_kind=O.SCHED_STEP, sched_k=2.0, sched_phase=100,
                   sched_steps=1)
    for i in (0, 1, 50, 99):
        assert O.schedule(cfg, i) == 2.0, i
    for i in (100, 101, 10 ** 7):
        assert O.schedule(cfg, i) == 1.0, i
    # three times the base (the section's other comparison), dropped at 10
    cfg3 = O.Config(T=1, B=1, D=1, sched_kind=O.SCHED_STEP, sched_k=3.0, sched_phase=10,
                    sched_steps=1)
    assert [O.schedule(cfg3, i) for i in (9, 10)] == [3.0, 1.0]


def test_table_factor_is_one_rounding_of_the_product():
    cfg = O.Config(T=2, B=1, D=1, eb=(0.005, 0.01), table_mult=(1.0, 3.0),
                   sched_kind=O.SCHED_INV_SQRT, sched_t0=1000.0)
    assert O.table_factor(cfg, 0, 0) == f32(0.005)
    assert O.table_factor(cfg, 0, 3000) == f32(float(np.float32(0.005)) * 0.5)
    # exact product 3 * f32(0.01) rounded once to fp32
    exact = Fraction(float(np.float32(0.01))) * 3
    assert Fraction(O.table_factor(cfg, 1, 0)) == Fraction(float(np.float32(float(exact))))


def test_range_ignores_nan_and_relative_eb():
    x = np.array([np.nan, -0.25, 3.0, np.nan, 1.0], np.float32)
    assert O.value_range(x) == (-0.25, 3.0)
    assert O.value_range(np.array([np.nan, np.nan], np.float32)) == (math.inf, -math.inf)
    cfg = O.Config(T=1, B=5, D=1, eb_mode=O.EB_REL, eb=(0.01,))
    assert O.table_eb(cfg, 0, 0, x) == f32(float(np.float32(0.01)) * 3.25)


def test_eb_validity():
    assert O.eb_valid(1e-30) and O.eb_valid(1.0)
    for v in [0.0, -1.0, math.nan, math.inf, 3e38]:   # 3e38: 2 eb overflows
        assert not O.eb_valid(v)


# --------------------------------------------------------------------------
# Homogenization Index, Eq. (1), against Tables III and IV
# --------------------------------------------------------------------------
def test_homo_index_against_printed_tables():
    rows = []
    with open(os.path.join(HERE, "golden", "homo_index_tables.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            src, tab, eb, n_o, n_q, batch, printed = line.split()
            rows.append((int(n_o), int(n_q), float(printed)))
    assert len(rows) == 16
    for n_o, n_q, printed in rows:
        eta = O.homo_index(n_o, n_q)
        assert 0.0 <= eta <= 1.0
        assert round(1.0 - eta, 6) == pytest.approx(printed, abs=1e-6)
    assert O.homo_index(110, 68) == pytest.approx(42 / 110, abs=1e-15)


def _patterns(x, eb):
    """Distinct raw rows and distinct quantized rows, by Python sets over an
    independent fp32 quantizer (outliers keyed by their raw bits)."""
    raw = {x[r].tobytes() for r in range(x.shape[0])}
    q, o = SF.quantize_np(x.reshape(-1), eb)
    q, o = q.reshape(x.shape), o.reshape(x.shape)
    bits = x.view(np.uint32)
    keys = set()
    for r in range(x.shape[0]):
        keys.add(tuple(("o", int(bits[r, d])) if o[r, d] else ("q", int(q[r, d]))
                       for d in range(x.shape[1])))
    return len(raw), len(keys)


@pytest.mark.parametrize("seed", range(4))
def test_homo_counts_match_sets_of_patterns(seed):
    """Eq. (1)'s N_original and N_quantized per segment against Python sets of
    rows: repeated rows, rows differing by less than a bin, outliers, NaN."""
    rng = np.random.default_rng(40 + seed)
    T, B, D, P = 2, 37 + 11 * seed, 3 + seed, 1 + seed % 3
    eb = 0.05
    base = rng.normal(0, 0.3, (T, 9, D)).astype(np.float32)
    x = np.take_along_axis(base, rng.integers(0, 9, (T, B))[:, :, None], axis=1).copy()
    x[:, ::4] += rng.uniform(-eb / 8, eb / 8, x[:, ::4].shape).astype(np.float32)
    x[0, 1, 0] = np.float32(1e6)
    x[1, 2, -1] = np.nan
    cfg = O.Config(T=T, B=B, D=D, P=P, eb_mode=O.EB_ABS, eb=(eb,))
    no, nq = O.homo_counts(cfg, 0, x)
    for p in range(P):
        r0, r1 = p * B // P, (p + 1) * B // P
        for t in range(T):
            want_o, want_q = _patterns(x[t, r0:r1], eb)
            assert (no[p * T + t], nq[p * T + t]) == (want_o, want_q), (p, t)
            assert nq[p * T + t] <= no[p * T + t]


def test_homo_counts_closed_form_and_invalid_eb():
    """k_i raw variants of each of m quantized patterns (perturbations well
    inside a bin around bin centres): N_original = sum k_i, N_quantized = m, so
    eta = 1 - m / sum k_i; a constant table under a range-relative bound has no
    valid eb and is not quantized (N_quantized = N_original)."""
    eb = np.float32(0.25)  # bin width 0.5: centres are multiples of 0.5
    m, D = 5, 4
    ks = [1, 2, 3, 4, 6]
    rows = []
    for i in range(m):
        centre = np.float32(0.5) * np.arange(i, i + D, dtype=np.float32)
        for j in range(ks[i]):
            rows.append(centre + np.float32(0.01 * j))
    x = np.array(rows * 2, np.float32)[None]  # every variant twice
    cfg = O.Config(T=1, B=x.shape[1], D=D, eb_mode=O.EB_ABS, eb=(float(eb),))
    no, nq = O.homo_counts(cfg, 0, x)
    assert (int(no[0]), int(nq[0])) == (sum(ks), m)
    assert O.homo_index(int(no[0]), int(nq[0])) == pytest.approx(1 - m / sum(ks))
    const = np.full((1, 10, D), 3.0, np.float32)
    rel = O.Config(T=1, B=10, D=D, eb_mode=O.EB_REL, eb=(0.01,))
    no, nq = O.homo_counts(rel, 0, const)
    assert (int(no[0]), int(nq[0])) == (1, 1)
    x2 = np.array(rows, np.float32)[None]
    x2[0, 0, 0] = np.nan  # range ignores NaN: still valid
    rel2 = O.Config(T=1, B=x2.shape[1], D=D, eb_mode=O.EB_REL, eb=(0.01,))
    no, nq = O.homo_counts(rel2, 0, x2)
    assert int(no[0]) == sum(ks) and int(nq[0]) <= int(no[0])


def test_classification_of_printed_kaggle_tables():
    """Algorithm 1's classes for Table III's tables, eta read from eq. (1)
    (one minus the printed column), with thresholds 0.1 / 0.3 and the
    multipliers that give the pages' Large / Medium / Small bounds 0.05 / 0.03
    / 0.01 around a medium bound of 0.03 (alpha = 5/3, beta = 3); equality
    with a threshold is medium.  Worked by hand."""
    rows = []
    with open(os.path.join(HERE, "golden", "homo_index_tables.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            src, tab, eb, n_o, n_q, batch, printed = line.split()
            if src == "TableIII":
                rows.append((int(tab), O.homo_index(int(n_o), int(n_q))))
    eta = [e for _, e in rows]
    cls, mult = O.classify(eta, 0.1, 0.3, 5.0 / 3.0, 3.0)
    want = {20: 2, 11: 2, 2: 2, 15: 1, 3: 1, 23: 0, 25: 0, 0: 0, 1: 0}
    assert {tab: int(c) for (tab, _), c in zip(rows, cls)} == want
    m = {0: np.float32(5.0 / 3.0), 1: np.float32(1.0), 2: np.float32(1.0 / 3.0)}
    assert all(mult[i] == m[int(c)] for i, c in enumerate(cls))
    assert np.float32(0.03) * m[0] == pytest.approx(0.05, rel=1e-6)
    assert np.float32(0.03) * m[2] == pytest.approx(0.01, rel=1e-6)
    cls, _ = O.classify([0.1, 0.3, 0.0999, 0.3001], 0.1, 0.3, 2.0, 2.0)
    assert list(cls) == [1, 1, 0, 2]
    with pytest.raises(ValueError):
        O.classify([0.5], 0.4, 0.3, 2.0, 2.0)
    with pytest.raises(ValueError):
        O.classify([0.5], 0.1, 0.3, 0.0, 2.0)


# --------------------------------------------------------------------------
# vector deduplication (section III-B obs. 2): brute force on tiny inputs
# --------------------------------------------------------------------------
def brute_first(x, eb):
    rows = []
    for r in range(x.shape[0]):
        key = []
        for v in x[r]:
            q, out = O.quantize(float(v), eb)
            key.append(("o", np.float32(v).view(np.uint32).item()) if out else ("q", q))
        rows.append(tuple(key))
    first = []
    for r in range(len(rows)):
        for r2 in range(r + 1):
            if rows[r2] == rows[r]:
                first.append(r2)
                break
    return np.array(first)


@pytest.mark.parametrize("seed", range(6))
def test_dedup_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, D = int(rng.integers(1, 140)), int(rng.integers(1, 9))
    eb = 0.05
    base = rng.normal(0, 0.2, (max(1, B // 3), D)).astype(np.float32)
    x = base[rng.integers(0, base.shape[0], B)]
    x = x + rng.uniform(-0.02, 0.02, x.shape).astype(np.float32) * (rng.random((B, 1)) < 0.5)
    x = x.astype(np.float32)
    if B > 4:
        x[2, 0] = np.nan
        x[3] = x[2]
        x[4, -1] = 1e9
    cfg = O.Config(T=1, B=B, D=D, eb=(eb,))
    c = O.compress(cfg, 0, x[None])
    want = brute_first(x, eb)
    np.testing.assert_array_equal(c.first[0], want)
    # quantization only merges rows: distinct quantized rows <= distinct raw rows
    u_quant = len(set(want.tolist()))
    u_raw = np.unique(x.view(np.uint32), axis=0).shape[0]
    assert u_quant <= u_raw


# --------------------------------------------------------------------------
# stream: independent reader, zero padding, bit planes, bound, determinism
# --------------------------------------------------------------------------
def check_stream(cfg, x, it=0):
    c = O.compress(cfg, it, x)
    st = SF.parse(c.stream)
    assert not c.stream[~st.covered].any(), "non-zero padding"
    codes, outl, first, y = SF.decode(st, c.stream)
    yo = O.decompress(cfg, c.stream)
    np.testing.assert_array_equal(y.view(np.uint32), yo.view(np.uint32))
    # widths = bit length of each block's largest zigzag code
    for seg in st.segments:
        for tl in seg.tiles:
            if tl.mode != 1:
                continue
            zz = np.zeros(len(tl.widths) * 64, np.int64)
            zz[:tl.zz.size] = tl.zz
            mx = zz.reshape(-1, 64).max(axis=1)
            np.testing.assert_array_equal(tl.widths, [int(m).bit_length() for m in mx])
    # the oracle's own debug outputs agree with what the stream says
    for seg in st.segments:
        r0 = seg.p * cfg.B // cfg.P
        r1 = (seg.p + 1) * cfg.B // cfg.P
        if not seg.valid:
            continue
        mask = first[seg.t, r0:r1] >= 0
        np.testing.assert_array_equal(first[seg.t, r0:r1][mask], c.first[seg.t, r0:r1][mask])
        np.testing.assert_array_equal(codes[seg.t, r0:r1], c.codes[seg.t, r0:r1])
        np.testing.assert_array_equal(outl[seg.t, r0:r1], c.outlier[seg.t, r0:r1].astype(bool))
    # error bound on every element (outliers exact, NaN payloads preserved)
    for seg in st.segments:
        r0 = seg.p * cfg.B // cfg.P
        r1 = (seg.p + 1) * cfg.B // cfg.P
        xs, ys = x[seg.t, r0:r1], yo[seg.t, r0:r1]
        if seg.valid:
            err = np.abs(xs.astype(np.float64) - ys.astype(np.float64))
            fin = np.isfinite(xs)
            assert (err[fin] <= np.float64(seg.eb)).all()
            np.testing.assert_array_equal(xs[~fin].view(np.uint32), ys[~fin].view(np.uint32))
        else:
            np.testing.assert_array_equal(xs.view(np.uint32), ys.view(np.uint32))
    assert c.stream.size <= O.max_compressed_bytes(cfg)
    assert O.compress(cfg, it, x).stream.tobytes() == c.stream.tobytes()
    return c, st


@pytest.mark.parametrize("T,B,D,P", [(1, 1, 1, 1), (1, 63, 3, 1), (2, 64, 16, 1),
                                      (3, 65, 64, 2), (2, 130, 128, 3), (1, 200, 5, 4),
                                      (2, 3, 8, 5), (1, 0, 4, 1), (1, 129, 256, 1)])
def test_stream_shapes_and_invariants(T, B, D, P):
    rng = np.random.default_rng(T * 1000 + B * 10 + D + P)
    base = rng.normal(0, 0.1, (T, max(1, B // 2 + 1), D)).astype(np.float32)
    idx = rng.integers(0, base.shape[1], (T, B))
    x = np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)
    cfg = O.Config(T=T, B=B, D=D, P=P, eb_mode=O.EB_REL, eb=(0.01,))
    check_stream(cfg, x)


def test_special_values_and_raw_fallbacks():
    rng = np.random.default_rng(7)
    T, B, D = 4, 70, 8
    x = rng.normal(0, 1, (T, B, D)).astype(np.float32)
    x[0, 3, 2] = np.nan
    x[0, 4, 1] = np.inf
    x[0, 5, 0] = -np.inf
    x[0, 6, 3] = -0.0
    x[0, 7] = np.float32(np.uint32(0x7FC00123).view(np.float32))  # NaN payload
    x[1] = np.nan            # all-NaN table: invalid eb -> RAW segment
    x[2] = 0.25              # constant table: zero range -> RAW segment
    x[3] = rng.normal(0, 1e6, (B, D)).astype(np.float32)
    cfg = O.Config(T=T, B=B, D=D, eb_mode=O.EB_REL, eb=(0.01,))
    c, st = check_stream(cfg, x)
    assert not st.segments[1].valid and not st.segments[2].valid
    assert all(tl.mode == 0 for tl in st.segments[1].tiles)


def test_all_outliers_fall_back_to_raw_tiles():
    # eb -> 0: every nonzero value is an outlier; the tile is stored RAW and
    # the round trip is exact (the pages' "exact round-trip at eb -> 0")
    rng = np.random.default_rng(8)
    x = rng.integers(-1000, 1000, (2, 100, 16)).astype(np.float32)
    cfg = O.Config(T=2, B=100, D=16, eb=(1e-30,))
    c, st = check_stream(cfg, x)
    y = O.decompress(cfg, c.stream)
    np.testing.assert_array_equal(y, x)
    assert all(tl.mode == 0 for s in st.segments for tl in s.tiles)
    assert c.stream.size == O.max_compressed_bytes(cfg)


def test_references_into_raw_tiles_decode_by_requantization():
    # tile 0 incompressible (huge spread -> RAW), later rows repeat tile-0 rows
    rng = np.random.default_rng(9)
    B, D = 200, 32
    x = np.zeros((1, B, D), np.float32)
    x[0, :64] = rng.normal(0, 1, (64, D)) * np.float32(10.0) ** rng.integers(-3, 4, (64, D))
    x[0, 64:] = rng.normal(0, 0.01, (B - 64, D))
    x[0, 100] = x[0, 3]
    x[0, 150] = x[0, 10]
    cfg = O.Config(T=1, B=B, D=D, eb=(1e-3,))
    c, st = check_stream(cfg, x)
    assert st.segments[0].tiles[0].mode == 0
    assert c.first[0, 100] == 3 and c.first[0, 150] == 10


def test_raw_record_when_bitpack_is_not_strictly_smaller():
    """A one-row tile of D = 8 with eb = 1/2 (bin width 1, integer values):
    the RAW record is 16 + 32 = 48 bytes; the BITPACK record is 24 bytes of
    header, widths and padding plus 8 bytes per plane, padded to 16.  One plane
    (32 bytes) is smaller, so the tile is packed; two or three planes make it
    exactly 48 bytes, not smaller, so the tile stays RAW (the independent
    reader re-derives the rule for every tile it walks)."""
    cfg = O.Config(T=1, B=1, D=8, eb_mode=O.EB_ABS, eb=(0.5,))
    for vals, w, mode in [([-1, 0, 0, 0, 0, 0, 0, 0], 1, 1), ([1, 0, 0, 0, 0, 0, 0, 0], 2, 0),
                          ([-2, 0, 0, 0, 0, 0, 0, 0], 2, 0), ([2, -2, 0, 0, 0, 0, 0, 0], 3, 0),
                          ([0] * 8, 0, 1)]:
        x = np.array(vals, np.float32).reshape(1, 1, 8)
        ref = O.compress(cfg, 0, x)
        st = SF.parse(ref.stream)
        tl = st.segments[0].tiles[0]
        assert tl.mode == mode, (vals, tl.mode)
        zz = [2 * v if v >= 0 else -2 * v - 1 for v in vals]
        assert max(zz).bit_length() == w
        assert SF.bitpack_size(x[0], 1, 1, 8, 0.5, 1) == (32 if w <= 1 else 48)
        np.testing.assert_array_equal(O.decompress(cfg, ref.stream), x)


def test_compression_ratio_is_total_bytes_based():
    # Table V "avg." is the harmonic mean of per-table ratios, i.e. the ratio
    # of total bytes for equal-sized tables; the stream reports total bytes.
    rng = np.random.default_rng(10)
    x = rng.normal(0, 0.01, (3, 256, 32)).astype(np.float32)
    x[1] = x[1, :1]   # all rows identical
    cfg = O.Config(T=3, B=256, D=32, eb=(1e-3,))
    c, st = check_stream(cfg, x)
    seg_bytes = [s.nbytes for s in st.segments]
    per_cr = [4 * 256 * 32 / b for b in seg_bytes]
    overhead = c.stream.size - sum(seg_bytes)
    assert 3 * 4 * 256 * 32 / (sum(seg_bytes)) == pytest.approx(3 / sum(1 / v for v in per_cr))
    assert overhead == 64 + 16 + 32


# --------------------------------------------------------------------------
# corrupt and truncated streams never crash the decoder
# --------------------------------------------------------------------------
def test_corrupt_streams_are_rejected_or_decoded_safely():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 0.1, (2, 150, 24)).astype(np.float32)
    x[:, 80:] = x[:, :70]
    cfg = O.Config(T=2, B=150, D=24, eb=(1e-2,))
    good = O.compress(cfg, 0, x).stream
    assert O.decompress(cfg, good, status=True)[0] == O.OK
    assert O.decompress(cfg, good[:-16], status=True)[0] == O.ERR_CORRUPT
    bad = good.copy()
    bad[0] ^= 1
    assert O.decompress(cfg, bad, status=True)[0] == O.ERR_CORRUPT
    n_err = 0
    for i in range(400):
        bad = good.copy()
        for _ in range(int(rng.integers(1, 4))):
            bad[int(rng.integers(0, bad.size))] ^= np.uint8(1 << int(rng.integers(0, 8)))
        rc, _ = O.decompress(cfg, bad, status=True)
        assert rc in (O.OK, O.ERR_CORRUPT)
        n_err += rc != O.OK
        cut = int(rng.integers(0, good.size))
        assert O.decompress(cfg, good[:cut], status=True)[0] == O.ERR_CORRUPT
    assert n_err > 0
    # wrong shape
    cfg2 = O.Config(T=2, B=151, D=24, eb=(1e-2,))
    assert O.decompress(cfg2, good, status=True)[0] == O.ERR_CORRUPT


def test_invalid_configuration_is_an_error():
    x = np.zeros((1, 4, 4), np.float32)
    with pytest.raises(RuntimeError):
        O.compress(O.Config(T=1, B=4, D=4, eb=(0.0,)), 0, x)
    with pytest.raises(RuntimeError):
        O.compress(O.Config(T=1, B=4, D=4, eb=(math.nan,)), 0, x)
    with pytest.raises(RuntimeError):
        O.compress(O.Config(T=1, B=4, D=4, eb=(1e-3,), table_mult=(-1.0,)), 0, x)


# --------------------------------------------------------------------------
# the synthetic workloads (two tables each, or fewer rows) through the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_workload_subsets_meet_the_bound(name):
    import synth
    w = synth.workload(name, iteration=1, tables=None if name == "c1" else [0, 3])
    x = w.x.numpy()
    T, B, D = x.shape
    if name != "c1":
        x = np.ascontiguousarray(x[:, :1024])
        B = 1024
    cfg = O.Config(T=T, B=B, D=D, eb_mode=w.eb_mode, eb=tuple(w.eb), sched_kind=w.sched_kind,
                   sched_t0=w.sched_t0)
    c, st = check_stream(cfg, x, it=w.iteration)
    cr = x.nbytes / c.stream.size
    assert cr > 1.5, cr


# --------------------------------------------------------------------------
# the entropy coder inside the stream (section III-D "Huffman Encoding"):
# Huffman segments, per-segment choice, same reconstruction as bit planes
# --------------------------------------------------------------------------
def test_huffman_segment_bytes_by_hand():
    """One row of D = 8 values 0,0,0,1,0,0,0,0 at eb = 1/2: symbols 2047 (x7)
    and 2048 (x1) get one-bit codes 0 and 1, so E's chunk is the bits
    00010000, one word 0x10000000.  Record: 16-byte header, chunk table
    [0, 1], the word: 28 -> 32 bytes, smaller than RAW (48).  Segment:
    header 32, directory 16, codebook ff 07 00 08 11 padded to 16, record
    32 = 96 bytes.  The bit-plane form is also 96 (its record, width 2, is
    48 = RAW, not smaller), so the per-segment choice keeps bit planes."""
    x = np.array([0, 0, 0, 1, 0, 0, 0, 0], np.float32).reshape(1, 1, 8)
    cfg = O.Config(T=1, B=1, D=8, eb_mode=O.EB_ABS, eb=(0.5,), coder=O.CODER_HUFFMAN)
    st = O.compress(cfg, 0, x).stream
    assert st.size == 64 + 16 + 16 + 96
    assert int.from_bytes(st[6:8].tobytes(), "little") == 2
    sg = 64 + 16 + 16
    assert int.from_bytes(st[sg + 12:sg + 16].tobytes(), "little") == 3  # valid | Huffman
    assert int.from_bytes(st[sg + 24:sg + 32].tobytes(), "little") == 96
    assert st[sg + 48:sg + 64].tolist() == [0xFF, 0x07, 0x00, 0x08, 0x11] + [0] * 11
    assert int.from_bytes(st[sg + 32:sg + 36].tobytes(), "little") == 64  # the record
    rec = st[sg + 64:sg + 96]
    assert rec[:16].tolist() == [1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 2, 0]
    assert rec[16:28].tolist() == [0, 0, 0, 0, 1, 0, 0, 0, 0, 0, 0, 0x10]
    assert rec[28:].tolist() == [0, 0, 0, 0]
    np.testing.assert_array_equal(O.decompress(cfg, st), x)
    auto = O.Config(T=1, B=1, D=8, eb_mode=O.EB_ABS, eb=(0.5,), coder=O.CODER_AUTO)
    sa = O.compress(auto, 0, x).stream
    assert int.from_bytes(sa[sg + 12:sg + 16].tobytes(), "little") == 1  # tie: bit planes
    assert sa.size == st.size


def _huff_streams(T, B, D, P, mode, eb, seed, coder):
    rng = np.random.default_rng(seed)
    base = rng.normal(0, 0.05, (T, max(1, B // 3), D)).astype(np.float32)
    x = np.take_along_axis(base, rng.integers(0, base.shape[1], (T, B))[:, :, None], axis=1).copy()
    if B > 2:
        x[0, 1, 0] = 1e6
        x[-1, 2, -1] = np.nan
    return x, O.Config(T=T, B=B, D=D, P=P, eb_mode=mode, eb=(eb,), coder=coder)


@pytest.mark.parametrize("T,B,D,P", [(2, 130, 128, 1), (3, 200, 24, 2), (1, 64, 64, 1),
                                     (2, 1, 8, 1), (2, 0, 16, 1), (4, 300, 5, 3)])
@pytest.mark.parametrize("coder", [2, 3])
def test_huffman_streams_rules_and_reconstruction(T, B, D, P, coder):
    """The independent reader walks every Huffman structure (zero padding,
    complete tight codebooks, chunk tables, chunk bits), re-derives each
    record's and each segment's choice, and finds the codebook built from the
    histogram of E; the reconstruction is bitwise the bit-plane stream's."""
    x, cfg = _huff_streams(T, B, D, P, O.EB_REL, 0.02, T * 31 + B + D, coder)
    ref = O.compress(cfg, 3, x)
    st = SF.parse(ref.stream)
    assert st.coder == coder
    assert not np.any(ref.stream[~st.covered])
    SF.check_coder_choice(st, ref.stream, O.huff_lengths)
    y = O.decompress(cfg, ref.stream)
    codes, outl, first, yr = SF.decode(st, ref.stream)
    np.testing.assert_array_equal(yr.view(np.uint32), y.view(np.uint32))
    np.testing.assert_array_equal(codes, ref.codes)
    assert ref.stream.size <= O.max_compressed_bytes(cfg)
    # the bound on every element; and rows of tiles coded under both coders
    # (a tile may be RAW under one and coded under the other) reconstruct
    # bitwise alike
    bp = O.Config(**{**cfg.__dict__, "coder": O.CODER_BITPACK})
    sb = SF.parse(O.compress(bp, 3, x).stream)
    yb = O.decompress(bp, O.compress(bp, 3, x).stream)
    for sh, sp in zip(st.segments, sb.segments):
        r0 = sh.p * B // P
        xs = x[sh.t, r0:r0 + sh.rows].astype(np.float64)
        fin = np.isfinite(xs)
        ys = y[sh.t, r0:r0 + sh.rows].astype(np.float64)
        assert np.all(np.abs(xs - ys)[fin] <= np.float64(np.float32(sh.eb)) if sh.valid else xs[fin] == ys[fin])
        for k, (th, tp) in enumerate(zip(sh.tiles, sp.tiles)):
            if th.mode and tp.mode:
                a = y[sh.t, r0 + 64 * k:r0 + 64 * k + th.n]
                b = yb[sh.t, r0 + 64 * k:r0 + 64 * k + th.n]
                np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_per_segment_choice_follows_the_data():
    """A table whose codes are all 0 costs no bit planes at all but one bit per
    code under Huffman: bit planes win.  A table of wide Gaussian codes costs
    about its entropy under Huffman and the width of each block's largest
    code as bit planes: Huffman wins.  The per-segment choice is never larger
    than either forced coder."""
    rng = np.random.default_rng(5)
    T, B, D = 2, 512, 64
    x = np.zeros((T, B, D), np.float32)
    x[1] = rng.normal(0, 40.0, (B, D)).astype(np.float32)
    mk = lambda c: O.Config(T=T, B=B, D=D, eb_mode=O.EB_ABS, eb=(0.5,), coder=c)
    sizes = {c: O.compress(mk(c), 0, x).stream for c in (1, 2, 3)}
    st = SF.parse(sizes[3])
    assert [s.huff for s in st.segments] == [False, True]
    assert sizes[3].size <= min(sizes[1].size, sizes[2].size)
    assert sizes[3].size < sizes[1].size
    for c in (1, 2, 3):
        np.testing.assert_array_equal(O.decompress(mk(c), sizes[c]), x.round())


def test_all_raw_huffman_segment_stays_within_the_bound():
    """Values that are all outliers leave every tile RAW; a forced Huffman
    segment then carries its codebook on top of the RAW records, which the
    size bound allows for."""
    rng = np.random.default_rng(9)
    x = rng.normal(0, 1e6, (2, 100, 32)).astype(np.float32)
    cfg = O.Config(T=2, B=100, D=32, eb_mode=O.EB_ABS, eb=(1e-3,), coder=O.CODER_HUFFMAN)
    st = O.compress(cfg, 0, x).stream
    assert st.size <= O.max_compressed_bytes(cfg)
    p = SF.parse(st)
    assert all(s.huff for s in p.segments) and all(t.mode == 0 for s in p.segments for t in s.tiles)
    np.testing.assert_array_equal(O.decompress(cfg, st), x)


def test_corrupt_huffman_streams_are_rejected():
    x, cfg = _huff_streams(2, 200, 32, 1, O.EB_ABS, 0.01, 3, O.CODER_HUFFMAN)
    good = O.compress(cfg, 0, x).stream
    st = SF.parse(good)
    seg = st.segments[0]
    cases = []
    b = good.copy(); b[6] = 1; cases.append(("Huffman segment in a bit-plane stream", b))
    bo = seg.offset + 32 + (4 * seg.ntiles + 15) // 16 * 16
    b = good.copy(); b[bo + 4] &= 0xF0; cases.append(("codebook range not tight", b))
    tl = [t for t in seg.tiles if t.mode == 2][0]
    oop = tl.offset + (16 + 2 * (tl.n - tl.U) + 3) // 4 * 4
    oct_ = oop + 8 * tl.n_out
    b = good.copy(); b[oct_:oct_ + 4] = 1; cases.append(("chunk table start", b))
    b = good.copy(); b[oct_ + 4:oct_ + 8] = 0; cases.append(("chunk table order", b))
    b = good.copy(); b[tl.offset + 14] = 1; cases.append(("bit-plane record in a Huffman segment", b))
    for label, bad in cases:
        rc, _ = O.decompress(cfg, bad, status=True)
        assert rc == O.ERR_CORRUPT, label
    rng = np.random.default_rng(0)
    for i in range(200):
        bad = good.copy()
        bad[int(rng.integers(0, bad.size))] ^= np.uint8(1 << int(rng.integers(0, 8)))
        rc, _ = O.decompress(cfg, bad, status=True)
        assert rc in (O.OK, O.ERR_CORRUPT)


# --------------------------------------------------------------------------
# compressor selection (section III-D "Selection Between Two Encoders":
# eq. (2) and Algorithm 2), and coders chosen per table
# --------------------------------------------------------------------------
def test_speedup_closed_forms():
    """eq. (2) at round numbers worked by hand, and its limits: infinitely
    fast coders (or a free link) give the compression ratio itself, an
    infinite ratio gives the coders' own bound."""
    assert O.speedup(4.0, 1.0, 8.0, 8.0) == 2.0          # 1 / (1/4 + 1/8 + 1/8)
    assert O.speedup(2.0, 2.0, 4.0, 4.0) == pytest.approx(2.0 / 3.0)  # 1 / (1/2 + 1)
    assert O.speedup(5.0, 4.0, 1e300, 1e300) == pytest.approx(5.0)
    assert O.speedup(5.0, 1e-300, 40.5, 205.4) == pytest.approx(5.0)
    assert O.speedup(1e300, 2.0, 10.0, 10.0) == pytest.approx(2.5)    # 1 / (2 * 0.2)
    # faster coders or a higher ratio never lower the speed-up
    assert O.speedup(6.0, 4.0, 80.0, 40.0) > O.speedup(6.0, 4.0, 40.0, 40.0)
    assert O.speedup(7.0, 4.0, 40.0, 40.0) > O.speedup(6.0, 4.0, 40.0, 40.0)


def test_selection_takes_the_largest_speedup_per_table():
    """Three tables, two compressors: A (ratio 4, 8, 10; coders at 8 GB/s),
    B (ratio 8, 8, 5; coders at 16 GB/s), link 1 GB/s.  Speed-ups by hand:
    A = 1/(1/r + 1/4), B = 1/(1/r + 1/8): table 0 A 2, B 4 -> B; table 1
    A 8/3, B 4 -> B; table 2 A 1/(0.1 + 0.25) = 2.857, B 1/(0.2 + 0.125) =
    3.077 -> B.  With B's coders at 4 GB/s (B = 1/(1/r + 1/2)): table 0 A 2,
    B 1.6 -> A; table 1 8/3 vs 1.6 -> A; table 2 2.857 vs 1.429 -> A.  Equal
    speed-ups keep the earlier compressor."""
    best, sp = O.select([[4, 8, 10], [8, 8, 5]], [8, 16], [8, 16], 1.0)
    assert best.tolist() == [1, 1, 1]
    np.testing.assert_allclose(sp, [4.0, 4.0, 1 / 0.325])
    best, sp = O.select([[4, 8, 10], [8, 8, 5]], [8, 4], [8, 4], 1.0)
    assert best.tolist() == [0, 0, 0]
    np.testing.assert_allclose(sp, [2.0, 8 / 3, 1 / 0.35])
    best, _ = O.select([[4, 4], [4, 4]], [8, 8], [8, 8], 1.0)
    assert best.tolist() == [0, 0]
    with pytest.raises(ValueError):
        O.select([[4, 0]], [8], [8], 1.0)


def test_coders_chosen_per_table():
    """Algorithm 2's per-table configuration in the stream: each table's
    segments follow its own coder's rule; the stream's coder is 1 when every
    table is bit planes, 2 when every table is Huffman, else 3."""
    rng = np.random.default_rng(21)
    T, B, D = 4, 300, 64
    x = rng.normal(0, 0.05, (T, B, D)).astype(np.float32)
    x[2] = 0.0
    for tc in [(1, 2, 3, 3), (2, 2, 2, 2), (1, 1, 1, 1), (3, 1, 2, 1)]:
        cfg = O.Config(T=T, B=B, D=D, eb_mode=O.EB_REL, eb=(0.02,), table_coder=tc)
        st_bytes = O.compress(cfg, 0, x).stream
        st = SF.parse(st_bytes)
        SF.check_coder_choice(st, st_bytes, O.huff_lengths, table_coder=tc)
        y = O.decompress(cfg, st_bytes)
        assert np.all(np.abs(y.astype(np.float64) - x) <= 0.02 * (x.max(axis=(1, 2)) - x.min(axis=(1, 2)))[:, None, None] + 1e-9)
    bp = O.Config(T=T, B=B, D=D, eb_mode=O.EB_REL, eb=(0.02,))
    allbp = O.Config(T=T, B=B, D=D, eb_mode=O.EB_REL, eb=(0.02,), table_coder=(1, 1, 1, 1))
    assert np.array_equal(O.compress(bp, 0, x).stream, O.compress(allbp, 0, x).stream)


# --------------------------------------------------------------------------
# windowed vector-LZ (section III-D "Vector-based LZ Encoding" with the
# extended window of section III-E, Table VI)
# --------------------------------------------------------------------------
def row_keys(x, eb):
    """Each row's key, quantized element by element with the pinned scalar
    quantizer: ('q', code) or ('o', raw bits) per element."""
    keys = []
    for r in range(x.shape[0]):
        key = []
        for v in x[r]:
            q, out = O.quantize(float(v), eb)
            key.append(("o", np.float32(v).view(np.uint32).item()) if out else ("q", q))
        keys.append(tuple(key))
    return keys


def brute_window(keys, W):
    """Nearest earlier row within W rows with the same key, else the row."""
    out = []
    for r in range(len(keys)):
        m = r
        for r2 in range(r - 1, max(-1, r - W - 1), -1):
            if keys[r2] == keys[r]:
                m = r2
                break
        out.append(m)
    return np.array(out)


def zipf_rows(rng, B, D, distinct, a=1.1, scale=0.2):
    """B rows drawn from `distinct` base rows with Zipf-like popularity."""
    base = rng.normal(0, scale, (distinct, D)).astype(np.float32)
    p = 1.0 / np.arange(1, distinct + 1) ** a
    idx = rng.choice(distinct, size=B, p=p / p.sum())
    return base[idx].astype(np.float32)


@pytest.mark.parametrize("W", [1, 2, 7, 64, 255])
@pytest.mark.parametrize("seed", range(2))
def test_window_matches_brute_force(W, seed):
    """The match of every row is the nearest earlier row within W with its
    key (brute force over the window), the stream stores its distance, and
    the reader's reconstruction is the oracle's."""
    rng = np.random.default_rng(100 * W + seed)
    B, D, P = 300, int(rng.integers(2, 9)), 2
    eb = 0.05
    x = np.stack([zipf_rows(rng, B, D, 40) for _ in range(2)])
    x[0, 5, 0] = np.nan
    x[0, 9] = x[0, 5]
    x[1, 7, -1] = 1e9
    cfg = O.Config(T=2, B=B, D=D, P=P, eb=(eb,), window=W)
    c, st = check_stream(cfg, x)
    for seg in st.segments:
        assert seg.window == W
        r0, r1 = seg.p * B // P, (seg.p + 1) * B // P
        want = brute_window(row_keys(x[seg.t, r0:r1], eb), W)
        np.testing.assert_array_equal(c.first[seg.t, r0:r1], want)
        assert seg.U == int((want == np.arange(r1 - r0)).sum())
        for k, tl in enumerate(seg.tiles):
            if tl.mode == 0:
                continue
            rows = [64 * k + i for i in range(tl.n) if not (tl.bitmap >> i) & 1]
            np.testing.assert_array_equal(tl.refs, [r - want[r] for r in rows])


@pytest.mark.parametrize("coder", [1, 2, 3])
def test_window_reconstruction_is_the_whole_segment_one(coder):
    """Rows with one key reconstruct identically wherever their reference
    points, so every window gives the values of the whole-segment
    references, and a window covering the segment gives its literals."""
    rng = np.random.default_rng(coder)
    T, B, D = 3, 250, 16
    x = np.stack([zipf_rows(rng, B, D, d) for d in (5, 30, 200)])
    x[1, 64:128] = rng.normal(0, 1e4, (64, D)).astype(np.float32)  # RAW tiles
    x[1, 200] = x[1, 70]
    x[2, 130] = x[2, 10]
    cfg0 = O.Config(T=T, B=B, D=D, eb_mode=O.EB_REL, eb=(0.01,), coder=coder)
    y0 = O.decompress(cfg0, O.compress(cfg0, 0, x, debug=False).stream)
    u_prev = None
    for W in (1, 3, 16, 64, 128, 255):
        cfg = O.Config(T=T, B=B, D=D, eb_mode=O.EB_REL, eb=(0.01,), coder=coder, window=W)
        c, st = check_stream(cfg, x)
        np.testing.assert_array_equal(O.decompress(cfg, c.stream).view(np.uint32),
                                      y0.view(np.uint32))
        u = sum(seg.U for seg in st.segments)
        assert u_prev is None or u <= u_prev  # a wider window never adds literals
        u_prev = u
    st0 = SF.parse(O.compress(cfg0, 0, x, debug=False).stream)
    assert u_prev == sum(seg.U for seg in st0.segments)  # 255 >= rows - 1


def test_window_chains_through_raw_tiles():
    """A match may itself be a repeated row, also one stored in a RAW tile
    (whose raw values give its key): every row of a hot key chains back."""
    rng = np.random.default_rng(9)
    B, D, W = 400, 8, 40
    x = rng.normal(0, 0.3, (1, B, D)).astype(np.float32)
    hot = x[0, 3].copy()
    x[0, 3::30] = hot                                              # a chain, step 30
    x[0, 128:192] = rng.normal(0, 1e5, (64, D)).astype(np.float32)  # a RAW tile...
    x[0, 153] = hot                                                # ...on the chain
    x[0, 128 + 5] = hot
    cfg = O.Config(T=1, B=B, D=D, eb=(1e-3,), window=W)
    c, st = check_stream(cfg, x)
    assert any(tl.mode == 0 for tl in st.segments[0].tiles)
    want = brute_window(row_keys(x[0], 1e-3), W)
    np.testing.assert_array_equal(c.first[0], want)
    y = O.decompress(cfg, c.stream)
    for r in range(3, B, 30):
        if not 128 <= r < 192:
            np.testing.assert_array_equal(y[0, r].view(np.uint32), y[0, 3].view(np.uint32))


def test_corrupt_window_distances_are_rejected():
    rng = np.random.default_rng(4)
    B, D, W = 200, 8, 10
    x = np.stack([zipf_rows(rng, B, D, 12)])
    cfg = O.Config(T=1, B=B, D=D, eb=(0.02,), window=W)
    good = O.compress(cfg, 0, x, debug=False).stream
    st = SF.parse(good)
    seg = st.segments[0]
    tl = next(t for t in seg.tiles if t.mode == 1 and t.U < t.n)
    orf = tl.offset + 16 + (len(tl.widths) + 3) // 4 * 4
    for v in (0, W + 1, 255):
        bad = good.copy()
        bad[orf] = v
        assert O.decompress(cfg, bad, status=True)[0] == O.ERR_CORRUPT
    # the first tile: a distance reaching before the segment
    t0 = seg.tiles[0]
    rows = [i for i in range(t0.n) if not (t0.bitmap >> i) & 1]
    if t0.mode == 1 and rows and rows[0] < W:
        bad = good.copy()
        bad[t0.offset + 16 + (len(t0.widths) + 3) // 4 * 4] = rows[0] + 1
        assert O.decompress(cfg, bad, status=True)[0] == O.ERR_CORRUPT
    # window bits without the windowed flag, and the flag without a window
    for flags in (1 | (W << 8), 5):
        bad = good.copy()
        bad[seg.offset + 12:seg.offset + 16] = np.frombuffer(np.uint32(flags).tobytes(), np.uint8)
        assert O.decompress(cfg, bad, status=True)[0] == O.ERR_CORRUPT
    with pytest.raises(ValueError):
        O.compress(O.Config(T=1, B=B, D=D, eb=(0.02,), window=256), 0, x)


# --------------------------------------------------------------------------
# codebook reuse across calls (stable distributions over training, Fig. 14)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("coder", [2, 3])
def test_codebook_reuse_rule(coder):
    """A segment keeps its previous code while that code has a length for
    every symbol it now holds, else builds and keeps a new one; the stored
    codebook is the code used; bit-plane tables keep nothing.  Streams stay
    within the bound and decode like any other."""
    rng = np.random.default_rng(40 + coder)
    T, B, D = 3, 400, 32
    tc = (coder, 1, coder)
    books = O.BookState(O.Config(T=T, B=B, D=D))
    for it, scale in enumerate([0.05, 0.04, 0.05, 0.3, 0.05]):
        x = rng.normal(0, scale, (T, B, D)).astype(np.float32)
        cfg = O.Config(T=T, B=B, D=D, eb=(0.01,), coder=coder, table_coder=tc, books=books)
        before = books.copy()
        c, st = check_stream(cfg, x)
        cfg0 = O.Config(T=T, B=B, D=D, eb=(0.01,), coder=coder, table_coder=tc)
        for seg in st.segments:
            s = seg.p * T + seg.t
            if tc[seg.t] == 1:
                assert books.have[s] == 0
                continue
            # the symbols the segment holds, by the independent reader
            freq = np.zeros(4095, np.int64)
            for tl in seg.tiles:
                qq, _ = SF._tile_codes(seg, tl, c.stream, D)
                freq += np.bincount(qq + 2047, minlength=4095)
            covered = before.have[s] and np.all((freq == 0) | (before.lengths[s] > 0))
            fresh = O.huff_lengths(freq)
            want = before.lengths[s] if covered else fresh
            assert books.have[s] == 1
            np.testing.assert_array_equal(books.lengths[s], want)
            if seg.huff:
                np.testing.assert_array_equal(seg.lengths, want)
            if not covered:
                # a fresh code is the one the call without reuse builds
                st0 = SF.parse(O.compress(cfg0, 0, x, debug=False).stream)
                s0 = st0.segments[s]
                if s0.huff and seg.huff:
                    np.testing.assert_array_equal(s0.lengths, fresh)
        if it == 1:
            assert books.have[0] and np.array_equal(books.lengths[0], before.lengths[0])  # reused


def test_codebook_reuse_needs_both_arrays():
    import ctypes
    books = O.BookState(O.Config(T=1, B=4, D=4))
    cfg = O.Config(T=1, B=4, D=4, eb=(0.1,), coder=2, books=books)
    c, keep = cfg._c()
    c.book_have = None
    assert O.lib().ebo_max_compressed_bytes(ctypes.byref(c)) == 0
