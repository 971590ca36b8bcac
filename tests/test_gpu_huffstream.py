"""GPU parity of Huffman segments inside the stream (section III-D's entropy
coder as a segment coder, with the per-segment choice): streams byte for
byte against the oracle with the same coder, reconstructions bitwise the
oracle's, full-size workloads, plans reused across calls, and damaged
streams rejected exactly when the oracle's reader rejects them."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import error_bounded_lossy_amd as ec  # noqa: E402
import oracle as O  # noqa: E402
import streamfmt as SF  # noqa: E402


def say(*a):
    print(*a, flush=True)


def dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.4):
    base = rng.normal(0, scale, (T, max(1, int(B * frac_unique) + 1), D)).astype(np.float32)
    idx = rng.integers(0, base.shape[1], (T, B))
    return np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)


def cfg_of(T, B, D, P, mode, eb, coder, sched=None):
    sched = sched or {}
    return O.Config(T=T, B=B, D=D, P=P, eb_mode=mode, eb=(eb,), coder=coder,
                    sched_kind=sched.get("kind", 0), sched_t0=sched.get("t0", 1000.0))


def gpu_round_trip(plan, x_t, it):
    out = plan.empty_stream()
    plan.compress(x_t, out, it)
    cr, nbytes, per, st = plan.ratio(per_segment=True)
    y = torch.full_like(x_t, float("nan"))
    plan.decompress(out[:nbytes], y)
    plan.ratio()
    return out[:nbytes].cpu().numpy(), y.cpu().numpy(), cr


def check(cfg, x, it=0, bits=0, label=""):
    say(f"[huffstream] {label} T={cfg.T} B={cfg.B} D={cfg.D} P={cfg.P} coder={cfg.coder} bits={bits}")
    ref = O.compress(cfg, it, x, debug=False)
    plan = ec.Plan(cfg.T, cfg.B, cfg.D, cfg.P, cfg.eb_mode, cfg.eb[0], debug_hash_bits=bits,
                   coder=cfg.coder)
    got, y, cr = gpu_round_trip(plan, torch.from_numpy(x).cuda(), it)
    assert got.size == ref.stream.size, (got.size, ref.stream.size)
    if not np.array_equal(got, ref.stream):
        bad = np.nonzero(got != ref.stream)[0]
        raise AssertionError(f"stream differs at {bad.size} bytes, first {bad[:8]}")
    yo = O.decompress(cfg, ref.stream)
    np.testing.assert_array_equal(y.view(np.uint32), yo.view(np.uint32))
    return ref


SHAPES = [(2, 130, 128, 1, 1), (3, 200, 64, 2, 1), (1, 64, 256, 1, 0), (2, 1, 64, 1, 1),
          (2, 0, 128, 1, 0), (4, 300, 128, 3, 1), (2, 1000, 256, 1, 1), (3, 700, 64, 1, 0)]


@pytest.mark.parametrize("T,B,D,P,mode", SHAPES)
@pytest.mark.parametrize("coder", [2, 3])
def test_shapes(T, B, D, P, mode, coder):
    rng = np.random.default_rng(T * 1000 + B + D + P + coder)
    x = dup_rows(rng, T, B, D)
    if B > 4:
        x[0, 3, 1] = 1e6      # an outlier
        x[-1, 4, -1] = np.nan
        x[0, 2] = x[0, 0]     # a repeat inside a tile
    check(cfg_of(T, B, D, P, mode, 0.02 if mode else 2e-3, coder), x, it=2, label="shape")


@pytest.mark.parametrize("D,bits", [(64, 2), (128, 0), (256, 4)])
def test_raw_tiles_hot_rows_and_weak_hashes(D, bits):
    """Hot rows repeated across many tiles, references into a RAW tile, a RAW
    segment, and a table whose all-zero codes keep bit planes under AUTO."""
    rng = np.random.default_rng(D + bits)
    T, B = 4, 2100
    base = rng.normal(0, 0.1, (T, 6, D)).astype(np.float32)
    idx = rng.choice(6, size=(T, B), p=[0.55, 0.2, 0.1, 0.08, 0.05, 0.02])
    x = np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)
    x[1, 64:128] = rng.normal(0, 1e4, (64, D)).astype(np.float32)  # a RAW tile
    x[1, 300] = x[1, 70]                                            # a reference into it
    x[2] = np.nan                                                   # no valid eb: RAW segment
    x[3] = 0.0
    x[3, 0, 0] = 1.0                                                # nearly all-zero codes
    for coder in (2, 3):
        ref = check(cfg_of(T, B, D, 1, 1, 0.01, coder), x, bits=bits, label="hot/raw")
        st = SF.parse(ref.stream)
        SF.check_coder_choice(st, ref.stream, O.huff_lengths)
        if coder == 3:
            assert not st.segments[3].huff


@pytest.mark.parametrize("name,coder", [("c2", 3), ("c3", 3), ("c3", 2), ("c4", 3), ("c4", 2)])
def test_workloads_full_size(name, coder):
    """Full-size batches, whole stream byte for byte against the oracle."""
    import synth
    w = synth.workload(name, iteration=1, device="cuda")
    T, B, D = w.shape
    sched = {"kind": w.sched_kind, "t0": w.sched_t0} if w.sched_kind else None
    cfg = cfg_of(T, B, D, 1, w.eb_mode, 0, coder, sched={"kind": w.sched_kind, "t0": w.sched_t0})
    cfg.eb = tuple(w.eb)
    plan = ec.Plan(T, B, D, 1, w.eb_mode, w.eb, schedule=sched, coder=coder)
    say(f"[huffstream] {name} coder={coder} full size")
    got, y, cr = gpu_round_trip(plan, w.x, w.iteration)
    xs = w.x.cpu().numpy()
    ref = O.compress(cfg, w.iteration, xs, debug=False)
    assert got.size == ref.stream.size, (got.size, ref.stream.size)
    assert np.array_equal(got, ref.stream)
    yo = O.decompress(cfg, ref.stream)
    assert np.array_equal(y.view(np.uint32), yo.view(np.uint32))
    st = SF.parse_segments(got)
    say(f"[huffstream] {name} coder={coder} CR={cr:.3f}, Huffman segments "
        f"{sum(1 for s in st if s.valid and _flags(got, s) & 2)}/{len(st)}")


@pytest.mark.parametrize("tcoder", [(1, 2, 3, 3), (2, 2, 2, 2), (1, 1, 1, 1), (3, 1, 2, 1)])
def test_per_table_coders(tcoder):
    """Algorithm 2's table-wise configuration: each table coded by its own
    coder; the stream's coder field follows from them; byte for byte the
    oracle with the same per-table coders."""
    rng = np.random.default_rng(sum(tcoder) * 7 + tcoder[0])
    T, B, D = 4, 900, 128
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.3)
    x[2] = rng.normal(0, 1, (B, D)).astype(np.float32)   # few repeats, wide codes
    x[3, :, 1:] = 0.0                                     # nearly all-zero codes
    cfg = cfg_of(T, B, D, 2, 1, 0.01, 1)
    cfg.table_coder = tuple(tcoder)
    say(f"[huffstream] table coders {tcoder}")
    ref = O.compress(cfg, 1, x, debug=False)
    plan = ec.Plan(T, B, D, 2, ec.EB_REL_RANGE, 0.01, coder=ec.CODER_BITPACK,
                   table_coder=tcoder)
    got, y, cr = gpu_round_trip(plan, torch.from_numpy(x).cuda(), 1)
    assert np.array_equal(got, ref.stream)
    np.testing.assert_array_equal(y.view(np.uint32), O.decompress(cfg, ref.stream).view(np.uint32))
    st = SF.parse(ref.stream)
    SF.check_coder_choice(st, ref.stream, O.huff_lengths, table_coder=tcoder)


def test_offline_comp_config_selects_and_compresses():
    """Algorithm 2 end to end: the pool's ratios and throughputs measured on
    a sample, the selection equal to the oracle's on those figures, and a
    plan with the selected coders byte for byte the oracle's."""
    rng = np.random.default_rng(5)
    T, B, D = 6, 4096, 128
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.05)
    x[1] = rng.normal(0, 1, (B, D)).astype(np.float32)
    x[4] = rng.normal(0, 3, (B, D)).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    for bw in (1e9, 1e12):
        r = ec.offline_comp_config(xt, bw, eb_mode=ec.EB_REL_RANGE, eb=0.01, reps=3)
        say(f"[huffstream] offline selection bw={bw:g}: {r['table_coder']} "
            f"tc={[round(v / 1e9, 1) for v in r['tc']]} GB/s td={[round(v / 1e9, 1) for v in r['td']]} GB/s")
        obest, osp = O.select(np.array(r["cr"]), r["tc"], r["td"], bw)
        assert r["best"] == [int(b) for b in obest]
        assert np.array_equal(np.array(r["speedup"]), osp)
        cfg = cfg_of(T, B, D, 1, 1, 0.01, 1)
        cfg.table_coder = tuple(r["table_coder"])
        plan = ec.Plan(T, B, D, 1, ec.EB_REL_RANGE, 0.01, table_coder=r["table_coder"])
        got, y, _ = gpu_round_trip(plan, xt, 0)
        assert np.array_equal(got, O.compress(cfg, 0, x, debug=False).stream)


def _flags(buf, seg):
    return int.from_bytes(buf[seg.offset + 12:seg.offset + 16].tobytes(), "little")


def test_plan_reused_across_calls():
    """Histograms, codebooks and choices are rebuilt every call."""
    rng = np.random.default_rng(77)
    T, B, D = 3, 1500, 128
    plan = ec.Plan(T, B, D, 1, ec.EB_REL_RANGE, 0.01, coder=ec.CODER_AUTO)
    cfg = cfg_of(T, B, D, 1, 1, 0.01, 3)
    out = plan.empty_stream()
    for call, (scale, fu) in enumerate([(1.0, 0.4), (100.0, 0.05), (0.01, 0.9), (3.0, 0.4)]):
        x = dup_rows(rng, T, B, D, scale=scale, frac_unique=fu)
        if call == 1:
            x[0] = 0.0
        plan.compress(torch.from_numpy(x).cuda(), out, call)
        _, nbytes, _ = plan.ratio()
        ref = O.compress(cfg, call, x, debug=False)
        assert np.array_equal(out[:nbytes].cpu().numpy(), ref.stream), call
        y = torch.empty(T, B, D, device="cuda")
        plan.decompress(out[:nbytes], y)
        plan.ratio()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                      O.decompress(cfg, ref.stream).view(np.uint32))


def test_bitplane_plan_rejects_huffman_streams_and_decodes_its_own():
    rng = np.random.default_rng(3)
    T, B, D = 2, 300, 64
    x = dup_rows(rng, T, B, D)
    huff = O.compress(cfg_of(T, B, D, 1, 0, 1e-3, 2), 0, x, debug=False).stream
    plan = ec.Plan(T, B, D, 1, ec.EB_ABS, 1e-3)
    y = torch.empty(T, B, D, device="cuda")
    plan.decompress(torch.from_numpy(huff).cuda(), y)
    assert plan.ratio(raise_on_error=False)[-1] == ec.EC_ERR_CORRUPT
    # a Huffman plan decodes bit-plane streams too
    bp = O.compress(cfg_of(T, B, D, 1, 0, 1e-3, 1), 0, x, debug=False).stream
    hplan = ec.Plan(T, B, D, 1, ec.EB_ABS, 1e-3, coder=ec.CODER_AUTO)
    hplan.decompress(torch.from_numpy(bp).cuda(), y)
    assert hplan.ratio(raise_on_error=False)[-1] == ec.EC_OK
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                  O.decompress(cfg_of(T, B, D, 1, 0, 1e-3, 1), bp).view(np.uint32))


@pytest.mark.parametrize("D", [64, 128])
def test_corrupt_huffman_streams(D):
    """Targeted damage (the stream's coder, a codebook that is not a complete
    code, chunk tables that do not start at 0 or go backwards, a chunk's
    bits, a bit-plane record in a Huffman segment, outliers out of order) is
    reported corrupt as the oracle's reader reports it; random flips and cuts
    end in OK or corrupt, and every stream the oracle accepts decodes to the
    same bits."""
    rng = np.random.default_rng(11 + D)
    T, B = 2, 300
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.3)
    x[0, 5, 7], x[0, 5, 9] = 1e6, -1e6
    x[1, 64:128] = rng.normal(0, 1e4, (64, D)).astype(np.float32)
    x[1, 130] = x[1, 70]
    cfg = cfg_of(T, B, D, 1, 0, 1e-2, 2)
    good = O.compress(cfg, 0, x).stream
    st = SF.parse(good)
    plan = ec.Plan(T, B, D, 1, ec.EB_ABS, 1e-2, coder=ec.CODER_HUFFMAN)
    y = torch.empty(T, B, D, device="cuda")

    def gpu_decode(buf):
        t = torch.from_numpy(np.ascontiguousarray(buf, np.uint8)).cuda()
        y.fill_(float("nan"))
        plan.decompress(t, y)
        return plan.ratio(raise_on_error=False)[-1], y.cpu().numpy()

    rc, yg = gpu_decode(good)
    assert rc == ec.EC_OK
    np.testing.assert_array_equal(yg.view(np.uint32), O.decompress(cfg, good).view(np.uint32))
    seg = st.segments[0]
    cases = []
    b = good.copy(); b[6] = 1; cases.append(("coder 1 with Huffman segments", b))
    bo = seg.offset + 32 + (4 * seg.ntiles + 15) // 16 * 16
    b = good.copy(); b[bo + 4] &= 0xF0; cases.append(("codebook range not tight", b))
    tl = [t for t in seg.tiles if t.mode == 2][0]
    oop = tl.offset + (16 + 2 * (tl.n - tl.U) + 3) // 4 * 4
    oct_ = oop + 8 * tl.n_out
    b = good.copy(); b[oct_:oct_ + 4] = 1; cases.append(("chunk table start", b))
    b = good.copy(); b[oct_ + 4:oct_ + 8] = 0; cases.append(("chunk table order", b))
    b = good.copy(); b[tl.offset + 14] = 1; cases.append(("bit-plane record", b))
    tlo = [t for s in st.segments for t in s.tiles if t.mode == 2 and t.n_out >= 2][0]
    oop2 = tlo.offset + (16 + 2 * (tlo.n - tlo.U) + 3) // 4 * 4
    b = good.copy(); b[oop2 + 4:oop2 + 8] = b[oop2:oop2 + 4]; cases.append(("outlier order", b))
    for label, bad in cases:
        say(f"[huffstream corrupt] {label}")
        rc_o, _ = O.decompress(cfg, bad, status=True)
        assert rc_o == O.ERR_CORRUPT, label
        rc_g, _ = gpu_decode(bad)
        assert rc_g == ec.EC_ERR_CORRUPT, label
    n_ok = n_bad = 0
    for i in range(60):
        bad = good.copy()
        for _ in range(int(rng.integers(1, 4))):
            bad[int(rng.integers(0, bad.size))] ^= np.uint8(1 << int(rng.integers(0, 8)))
        if i % 3 == 2:
            bad = bad[:int(rng.integers(64, bad.size))].copy()
        rc_o, yo = O.decompress(cfg, bad, status=True)
        rc_g, yg = gpu_decode(bad)
        assert rc_g in (ec.EC_OK, ec.EC_ERR_CORRUPT), (i, rc_g)
        if rc_o == O.OK:
            assert rc_g == ec.EC_OK, i
            np.testing.assert_array_equal(yg.view(np.uint32), yo.view(np.uint32))
        n_ok += rc_g == ec.EC_OK
        n_bad += rc_g != ec.EC_OK
    say(f"[huffstream corrupt] random: {n_ok} decoded, {n_bad} rejected")


@pytest.mark.parametrize("D,coder,tcoder", [(128, 2, None), (64, 3, None), (256, 3, (2, 1, 3))])
def test_codebook_reuse_across_calls(D, coder, tcoder):
    """Codebook reuse: a plan's calls keep each segment's code while it
    covers the segment's symbols; every call's stream is byte for byte the
    oracle's given the oracle's own kept codes, with decompressions (which
    build their tables elsewhere in the workspace) between the calls."""
    rng = np.random.default_rng(D + coder)
    T, B, P = 3, 700, 2
    cfg0 = cfg_of(T, B, D, P, 0, 0.01, coder)
    cfg0.table_coder = tcoder
    books = O.BookState(cfg0)
    plan = ec.Plan(T, B, D, P, ec.EB_ABS, 0.01, coder=coder, table_coder=tcoder, reuse_books=True)
    out = plan.empty_stream()
    y = torch.empty(T, B, D, device="cuda")
    reused = 0
    for it, scale in enumerate([0.05, 0.045, 0.05, 0.4, 0.04, 0.05]):
        x = dup_rows(rng, T, B, D, scale=scale, frac_unique=0.5)
        if it == 2:
            x[0, 5, 7] = 1e6  # an outlier (code 0, already in the code)
        cfg = cfg_of(T, B, D, P, 0, 0.01, coder)
        cfg.table_coder = tcoder
        cfg.books = books
        have_before = books.have.copy()
        len_before = books.lengths.copy()
        say(f"[huffstream] reuse D={D} coder={coder} call {it}")
        ref = O.compress(cfg, it, x, debug=False)
        plan.compress(torch.from_numpy(x).cuda(), out, it)
        _, nbytes, _ = plan.ratio()
        assert np.array_equal(out[:nbytes].cpu().numpy(), ref.stream), it
        plan.decompress(out[:nbytes], y)
        plan.ratio()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                      O.decompress(cfg, ref.stream).view(np.uint32))
        reused += int(np.sum(have_before.astype(bool) & books.have.astype(bool) &
                             np.all(len_before == books.lengths, axis=1)))
    assert reused > 0
