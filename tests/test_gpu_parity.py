"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Streams must match byte for byte (which fixes codes, first-occurrence maps and
every packed bit), the debug outputs (codes, outlier flags, first occurrences,
segment eb) must match exactly, and the decompressed tensor must be bitwise
identical to the oracle's reconstruction (hence within eb of the input)."""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import error_bounded_lossy_amd as ec  # noqa: E402
import oracle as O  # noqa: E402
import streamfmt as SF  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_cfg(T, B, D, P=1, eb_mode=0, eb=(1e-3,), mult=None, sched=None):
    sched = sched or {}
    return O.Config(T=T, B=B, D=D, P=P, eb_mode=eb_mode, eb=tuple(eb), table_mult=mult,
                    sched_kind=sched.get("kind", 0), sched_t0=sched.get("t0", 1000.0),
                    sched_k=sched.get("k", 2.0), sched_phase=sched.get("phase", 1),
                    sched_steps=sched.get("steps", 1))


def run_gpu(cfg, x_np, it=0, hash_bits=0, debug=True, sched=None):
    T, B, D, P = cfg.T, cfg.B, cfg.D, cfg.P
    plan = ec.Plan(T, B, D, P, cfg.eb_mode, list(cfg.eb) if len(cfg.eb) > 1 else cfg.eb[0],
                   table_mult=cfg.table_mult, schedule=sched, debug_hash_bits=hash_bits)
    x = torch.from_numpy(np.ascontiguousarray(x_np, np.float32)).cuda()
    out = plan.empty_stream()
    dbg = None
    if debug:
        dbg = (torch.full((T * B * D,), -7, dtype=torch.int32, device="cuda"),
               torch.full((T * B * D,), 9, dtype=torch.uint8, device="cuda"),
               torch.full((T * B,), 0xFFFF, dtype=torch.int32, device="cuda"),
               torch.full((P * T,), -1.0, dtype=torch.float32, device="cuda"))
        plan.debug_attach(*dbg)
    plan.compress(x, out, it)
    cr, nbytes, per, st = plan.ratio(per_segment=True)
    stream = out[:nbytes].cpu().numpy()
    y = torch.full_like(x, float("nan"))
    plan.decompress(out[:nbytes], y)
    plan.ratio()
    res = dict(stream=stream, y=y.cpu().numpy(), cr=cr, per=per, plan=plan, out=out, x=x)
    if debug:
        res.update(codes=dbg[0].cpu().numpy().reshape(T, B, D),
                   outlier=dbg[1].cpu().numpy().reshape(T, B, D),
                   first=dbg[2].cpu().numpy().view(np.uint32).reshape(T, B),
                   eb=dbg[3].cpu().numpy())
    return res


def assert_parity(cfg, x, it=0, hash_bits=0, sched=None, label=""):
    say(f"[parity] {label} T={cfg.T} B={cfg.B} D={cfg.D} P={cfg.P} mode={cfg.eb_mode} "
        f"it={it} hash_bits={hash_bits}")
    ref = O.compress(cfg, it, x)
    yo = O.decompress(cfg, ref.stream)
    g = run_gpu(cfg, x, it, hash_bits, sched=sched)
    np.testing.assert_array_equal(g["eb"], ref.eb)
    np.testing.assert_array_equal(g["codes"], ref.codes)
    np.testing.assert_array_equal(g["outlier"], ref.outlier)
    np.testing.assert_array_equal(g["first"], ref.first)
    assert g["stream"].size == ref.stream.size
    if not np.array_equal(g["stream"], ref.stream):
        bad = np.nonzero(g["stream"] != ref.stream)[0]
        raise AssertionError(f"stream differs at {bad.size} bytes, first {bad[:8]}")
    np.testing.assert_array_equal(g["y"].view(np.uint32), yo.view(np.uint32))
    assert g["cr"] == pytest.approx(x.nbytes / ref.stream.size if x.size else 0.0, rel=1e-12) \
        or x.size == 0
    return g, ref


def dup_rows(rng, T, B, D, scale=0.1, frac_unique=0.4):
    base = rng.normal(0, scale, (T, max(1, int(B * frac_unique) + 1), D)).astype(np.float32)
    idx = rng.integers(0, base.shape[1], (T, B))
    return np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)


SHAPES = [(1, 1, 1, 1), (1, 63, 3, 1), (2, 64, 16, 1), (3, 65, 64, 2), (2, 130, 128, 3),
          (1, 200, 5, 4), (2, 3, 8, 5), (1, 129, 256, 1), (4, 257, 32, 1), (2, 1000, 100, 1),
          (1, 4096, 128, 1)]


@pytest.mark.parametrize("T,B,D,P", SHAPES)
def test_shapes_rel(T, B, D, P):
    rng = np.random.default_rng(T * 7919 + B * 31 + D * 3 + P)
    x = dup_rows(rng, T, B, D)
    assert_parity(make_cfg(T, B, D, P, eb_mode=1, eb=(0.01,)), x, label="rel")


@pytest.mark.parametrize("T,B,D,P", SHAPES[:8])
def test_shapes_abs_schedule(T, B, D, P):
    rng = np.random.default_rng(100 + T * 7919 + B * 31 + D * 3 + P)
    x = dup_rows(rng, T, B, D, scale=0.05)
    sched = {"kind": ec.SCHED_STEP, "k": 2.0, "phase": 10, "steps": 4}
    cfg = make_cfg(T, B, D, P, eb_mode=0, eb=[1e-3 * (1 + t) for t in range(T)],
                   mult=[1.0 + 0.5 * t for t in range(T)], sched=sched)
    assert_parity(cfg, x, it=5, sched=sched, label="abs+step")


def test_empty_batch():
    cfg = make_cfg(2, 0, 8, 1, eb_mode=1, eb=(0.01,))
    assert_parity(cfg, np.zeros((2, 0, 8), np.float32), label="B=0")


def test_more_chunks_than_rows():
    rng = np.random.default_rng(5)
    x = dup_rows(rng, 2, 3, 8)
    assert_parity(make_cfg(2, 3, 8, 7, eb_mode=0, eb=(1e-2,)), x, label="P>B")


@pytest.mark.parametrize("D", [8, 64, 128])
def test_special_values_and_raw_segments(D):
    rng = np.random.default_rng(7)
    T, B = 4, 70
    x = rng.normal(0, 1, (T, B, D)).astype(np.float32)
    x[0, 3, 2] = np.nan
    x[0, 4, 1] = np.inf
    x[0, 5, 0] = -np.inf
    x[0, 6, 3] = -0.0
    x[0, 7] = np.float32(np.uint32(0x7FC00123).view(np.float32))
    x[0, 40] = x[0, 7]
    x[1] = np.nan
    x[2] = 0.25
    x[3] = rng.normal(0, 1e6, (B, D)).astype(np.float32)
    assert_parity(make_cfg(T, B, D, eb_mode=1, eb=(0.01,)), x, label="special")


@pytest.mark.parametrize("D", [32, 128, 256])
def test_raw_tiles_and_references_into_them(D):
    rng = np.random.default_rng(9)
    B = 200
    x = np.zeros((1, B, D), np.float32)
    x[0, :64] = rng.normal(0, 1, (64, D)) * np.float32(10.0) ** rng.integers(-3, 4, (64, D))
    x[0, 64:] = rng.normal(0, 0.01, (B - 64, D))
    x[0, 100] = x[0, 3]
    x[0, 150] = x[0, 10]
    g, ref = assert_parity(make_cfg(1, B, D, eb=(1e-3,)), x, label="raw-refs")
    assert SF.parse(ref.stream).segments[0].tiles[0].mode == 0


@pytest.mark.parametrize("D", [16, 64])
def test_eb_to_zero_is_exact(D):
    rng = np.random.default_rng(8)
    x = rng.integers(-1000, 1000, (2, 100, D)).astype(np.float32)
    g, _ = assert_parity(make_cfg(2, 100, D, eb=(1e-30,)), x, label="eb->0")
    np.testing.assert_array_equal(g["y"], x)


@pytest.mark.parametrize("bits,D", [(1, 24), (4, 24), (12, 24), (1, 64), (4, 128), (12, 256)])
def test_weak_hash_gives_identical_bytes(bits, D):
    rng = np.random.default_rng(11 + bits + D)
    x = dup_rows(rng, 2, 700, D, frac_unique=0.3)
    # near-duplicates: rows that differ in one element by less than a bin
    x[:, 500:] = x[:, :200]
    x[:, 500:, 3] += np.float32(1e-7)
    assert_parity(make_cfg(2, 700, D, eb_mode=1, eb=(0.02,)), x, hash_bits=bits,
                  label=f"weak-hash-{bits}")


def test_rounding_boundaries_and_code_range_edges():
    """Values on and next to bin edges and at the ends of the code range,
    where the fast multiply-by-reciprocal quantizer must defer to division."""
    eb = np.float32(0.001)
    s = eb + eb
    ks = np.arange(-2048, 2049, dtype=np.float32)
    base = np.concatenate([(ks + 0.5) * s, ks * s, (ks + 0.25) * s])
    vals = np.concatenate([base, np.nextafter(base, np.float32(np.inf)),
                           np.nextafter(base, np.float32(-np.inf))]).astype(np.float32)
    D = 128
    n = (vals.size + D - 1) // D
    x = np.zeros(n * D, np.float32)
    x[:vals.size] = vals
    x = x.reshape(1, n, D)
    for d in (128, 16):
        xx = x.reshape(1, -1, d)
        assert_parity(make_cfg(1, xx.shape[1], d, eb=(float(eb),)), xx, label=f"edges-D{d}")


def test_determinism_across_runs():
    rng = np.random.default_rng(12)
    x = dup_rows(rng, 3, 3000, 64, frac_unique=0.2)
    cfg = make_cfg(3, 3000, 64, eb_mode=1, eb=(0.01,))
    first = run_gpu(cfg, x, debug=False)["stream"]
    for _ in range(3):
        assert np.array_equal(run_gpu(cfg, x, debug=False)["stream"], first)


def test_ratio_waits_for_queued_calls():
    """ec_ratio waits for the plan's last call however much work is queued
    before it: on a side stream behind a little work (the call's completion
    number seen in the pinned report), and on the current stream behind more
    than 200 ms of work (then the wait falls back to the whole device).  The
    report it returns (bytes, then a decoder's corrupt status) is the call's."""
    rng = np.random.default_rng(31)
    T, B, D = 4, 4096, 128
    x = torch.from_numpy(dup_rows(rng, T, B, D, frac_unique=0.3)).cuda()
    plan = ec.Plan(T, B, D, 1, 1, 0.01)
    out = plan.empty_stream()
    plan.compress(x, out, 3)
    torch.cuda.synchronize()
    _, nb0, _ = plan.ratio()
    ref = out[:nb0].clone()
    a = torch.randn(4096, 4096, device="cuda")

    def busy(ms, stream):
        # matrix products on `stream` until about `ms` of work is queued
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            c = a
            e0.record()
            c = a @ c
            e1.record()
        e1.synchronize()
        per = max(e0.elapsed_time(e1), 1e-3)
        with torch.cuda.stream(stream):
            e0.record()
            for _ in range(int(ms / per) + 1):
                c = (a @ c) * 1e-3
            e1.record()
        return e0, e1

    side = torch.cuda.Stream()
    for ms, stream in ((20.0, side), (400.0, torch.cuda.current_stream())):
        out.zero_()
        stream.wait_stream(torch.cuda.current_stream())
        e0, e1 = busy(ms, stream)
        plan.compress(x, out, 3, stream=stream)
        cr, nb, st = plan.ratio()
        assert st == ec.EC_OK and nb == nb0, (ms, nb, nb0)
        torch.cuda.synchronize()
        say(f"[ratio wait] queued {e0.elapsed_time(e1):.1f} ms on "
            f"{'the side' if stream is side else 'the current'} stream")
        assert torch.equal(out[:nb], ref)
    # a corrupt stream's status, reported after a queued decompression
    bad = ref.clone()
    bad[0] ^= 1
    y = torch.empty(T, B, D, device="cuda")
    busy(250.0, torch.cuda.current_stream())
    plan.decompress(bad, y)
    assert plan.ratio(raise_on_error=False)[-1] == ec.EC_ERR_CORRUPT
    plan.decompress(ref, y)
    assert plan.ratio(raise_on_error=False)[-1] == ec.EC_OK


def test_per_segment_ratio_and_chunk_sizes():
    rng = np.random.default_rng(13)
    x = dup_rows(rng, 3, 500, 32)
    cfg = make_cfg(3, 500, 32, P=4, eb_mode=1, eb=(0.01,))
    g, ref = assert_parity(cfg, x, label="ratio")
    st = SF.parse(ref.stream)
    for seg in st.segments:
        rows = (seg.p + 1) * 500 // 4 - seg.p * 500 // 4
        assert g["per"][seg.p * 3 + seg.t] == pytest.approx(4 * rows * 32 / seg.nbytes)


def describe_segment_diff(g, r, D):
    """Where two segment byte strings (same length) first differ: header field,
    tile directory entry, or tile record and the part of it."""
    idx = np.flatnonzero(g != r)
    if idx.size == 0:
        return "identical"
    i = int(idx[0])
    nt = int(r[4:8].view(np.uint32)[0])
    head = f"{idx.size} bytes differ, first at {i}"
    if i < 32:
        return f"{head}: segment header word {i // 4}"
    if i < 32 + 4 * nt:
        return f"{head}: tile directory entry {(i - 32) // 4}"
    dirs = r[32:32 + 4 * nt].view(np.uint32).astype(np.int64)
    if nt == 0 or i < dirs[0]:
        return f"{head}: tile directory padding"
    j = int(np.searchsorted(dirs, i, side="right") - 1)
    o = i - int(dirs[j])
    rec = r[dirs[j]:]
    n_out = int(rec[8:12].view(np.uint32)[0])
    u_t = int(rec[12:14].view(np.uint16)[0])
    mode = int(rec[14])
    if o < 16:
        part = "record header"
    elif mode == 0:
        part = "raw rows"
    else:
        rows = int(r[0:4].view(np.uint32)[0])
        n = min(64, rows - 64 * j)
        nblk = (u_t * D + 63) // 64
        rb = 2 if rows <= 65536 else 4
        o_refs = (16 + nblk + 3) // 4 * 4
        o_opos = (o_refs + rb * (n - u_t) + 3) // 4 * 4
        o_pl = (o_opos + 8 * n_out + 7) // 8 * 8
        part = ("widths" if o < o_refs else "refs" if o < o_opos else
                "outliers" if o < o_pl else "planes")
    return f"{head}: tile {j} (U_t={u_t}, n_out={n_out}, mode={mode}) {part} byte {o}"


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c5d40"])
def test_workloads_full_size_whole_stream(name):
    """Full-size batch on the GPU, in the launch configuration the benchmark
    times.  The oracle compresses the whole batch: the complete GPU stream
    (header, chunk table, every segment header, tile directory and record) must
    equal it byte for byte, and the GPU reconstruction of every table must be
    bitwise the oracle's (hence within eb of the input)."""
    import synth
    say(f"[workload] {name} full size")
    w = synth.workload(name, iteration=3, device="cuda")
    T, B, D = w.shape
    sched = {"kind": w.sched_kind, "t0": w.sched_t0} if w.sched_kind else None
    plan = ec.Plan(T, B, D, 1, w.eb_mode, w.eb, schedule=sched)
    out = plan.empty_stream()
    plan.compress(w.x, out, w.iteration)
    cr, nbytes, per, _ = plan.ratio(per_segment=True)
    y = torch.empty_like(w.x)
    plan.decompress(out[:nbytes], y)
    plan.ratio()
    gst = out[:nbytes].cpu().numpy()
    del out
    xs = w.x.cpu().numpy()
    cfg = make_cfg(T, B, D, 1, eb_mode=w.eb_mode, eb=tuple(w.eb),
                   sched={"kind": w.sched_kind, "t0": w.sched_t0})
    say(f"[workload] {name} oracle on {xs.nbytes >> 20} MiB")
    ref = O.compress(cfg, w.iteration, xs, debug=False)
    assert gst.size == ref.stream.size, (gst.size, ref.stream.size)
    if not np.array_equal(gst, ref.stream):
        gsegs, rsegs = SF.parse_segments(gst), SF.parse_segments(ref.stream)
        for t in range(T):
            gs, rs = gsegs[t], rsegs[t]
            gb = gst[gs.offset:gs.offset + gs.nbytes]
            rb = ref.stream[rs.offset:rs.offset + rs.nbytes]
            assert gs.offset == rs.offset and np.array_equal(gb, rb), \
                f"table {t}: " + describe_segment_diff(gb, rb, D)
        raise AssertionError("stream headers differ")
    del xs
    yo = O.decompress(cfg, ref.stream)
    yg = y.cpu().numpy()
    assert np.array_equal(yg.view(np.uint32), yo.view(np.uint32)), "reconstruction differs"
    # the bound on every element of the whole batch
    gsegs = SF.parse_segments(gst)
    xg = w.x
    ebs = torch.tensor([s.eb for s in gsegs], device="cuda").view(T, 1, 1)
    fin = torch.isfinite(xg)
    err = (xg.double() - y.double()).abs()
    assert bool((err[fin] <= ebs.expand_as(xg).double()[fin]).all())
    assert cr == pytest.approx(4.0 * T * B * D / ref.stream.size, rel=1e-12)
    say(f"[workload] {name} CR={cr:.3f} ({ref.stream.size} bytes, whole stream equal)")


@pytest.mark.parametrize("T,B,D,mode", [(3, 1000, 128, 1), (2, 8192, 64, 1), (5, 4096, 64, 1),
                                        (3, 16448, 64, 1), (9, 2100, 256, 1), (2, 1000, 128, 0)])
def test_plan_reused_across_calls(T, B, D, mode):
    """One plan, consecutive calls on the same stream whose value ranges and
    duplicate structure change: every call must match the oracle (nothing of
    an earlier call's range partials or hash tables may leak into a later one).
    Shapes from 48 to 771 tiles, one to 257 tiles per table."""
    say(f"[reuse] T={T} B={B} D={D} mode={mode}")
    rng = np.random.default_rng(B + D + T)
    cfg = make_cfg(T, B, D, eb_mode=mode, eb=(0.01,))
    plan = ec.Plan(T, B, D, 1, mode, 0.01)
    out = plan.empty_stream()
    for call, (scale, fu) in enumerate([(1.0, 0.4), (100.0, 0.05), (0.01, 0.9), (3.0, 0.4)]):
        x = dup_rows(rng, T, B, D, scale=scale, frac_unique=fu)
        if call == 2:
            x[0, 5, 3] = np.nan  # NaN is excluded from the range
        plan.compress(torch.from_numpy(x).cuda(), out, call)
        _, nbytes, _, _ = plan.ratio(per_segment=True)
        ref = O.compress(cfg, call, x, debug=False)
        got = out[:nbytes].cpu().numpy()
        assert got.size == ref.stream.size, (call, got.size, ref.stream.size)
        assert np.array_equal(got, ref.stream), f"call {call}"
        y = torch.empty(T, B, D, device="cuda")
        plan.decompress(out[:nbytes], y)
        plan.ratio()
        yo = O.decompress(cfg, ref.stream)
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))


@pytest.mark.parametrize("D,mode,bits", [(64, 0, 4), (128, 1, 3), (256, 0, 0)])
def test_hash_tables_clean_between_calls(D, mode, bits):
    """The hash tables are cleared on a plan's first call only; afterwards the
    write pass clears the slots it used.  Calls alternate duplicate-heavy and
    duplicate-free batches, with weakened row hashes (long probe chains, many
    tag collisions), a segment stored raw and a tile stored raw: every call
    must still match the oracle byte for byte."""
    T, B = 3, 700
    say(f"[clean] D={D} mode={mode} bits={bits}")
    rng = np.random.default_rng(D + mode + bits)
    cfg = make_cfg(T, B, D, eb_mode=mode, eb=(0.01,))
    plan = ec.Plan(T, B, D, 1, mode, 0.01, debug_hash_bits=bits)
    out = plan.empty_stream()
    for call in range(5):
        if call % 2 == 0:
            x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.1)
        else:
            x = rng.normal(0, 0.05, (T, B, D)).astype(np.float32)
        if call == 2:
            x[1] = np.nan  # an invalid error bound (range mode) or outliers only
        if call == 3:
            x[2, 64:128] = rng.normal(0, 1e4, (64, D)).astype(np.float32)  # a raw tile
        plan.compress(torch.from_numpy(x).cuda(), out, call)
        _, nbytes, _, _ = plan.ratio(per_segment=True)
        ref = O.compress(cfg, call, x, debug=False)
        got = out[:nbytes].cpu().numpy()
        assert got.size == ref.stream.size and np.array_equal(got, ref.stream), f"call {call}"
        y = torch.empty(T, B, D, device="cuda")
        plan.decompress(out[:nbytes], y)
        plan.ratio()
        yo = O.decompress(cfg, ref.stream)
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))


@pytest.mark.parametrize("D,bits", [(64, 0), (128, 0), (256, 0), (128, 2)])
def test_hot_rows_many_duplicates(D, bits):
    """A few rows repeated thousands of times across many tiles (one-hot
    lookups of a hot index), with near-duplicates that differ by less than a
    bin and, with few hash bits, tag collisions between different rows: every
    duplicate must point at the smallest equal row of its segment."""
    rng = np.random.default_rng(D + bits)
    T, B = 2, 4096
    base = rng.normal(0, 0.1, (T, 6, D)).astype(np.float32)
    idx = rng.choice(6, size=(T, B), p=[0.55, 0.2, 0.1, 0.08, 0.05, 0.02])
    x = np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)
    x[:, 1000:1100, 5] += np.float32(1e-7)  # same codes, other bits
    x[:, 3000] = rng.normal(0, 0.1, (T, D))  # a unique row late in the segment
    assert_parity(make_cfg(T, B, D, eb_mode=1, eb=(0.02,)), x, hash_bits=bits, label=f"hot-{D}-{bits}")


@pytest.mark.parametrize("D", [128, 24])
def test_corrupt_streams_are_rejected_or_decoded_like_the_oracle(D):
    """The decoders validate every field they use (D = 128 runs the wave64
    decoder, D = 24 the generic one).  Targeted corruptions (magic,
    truncation, wrong shape, a segment offset, a tile directory entry, a block
    width above 12, a forward reference, an outlier position past its record's
    rows, outlier positions out of order, a segment header's U or n_out that
    disagrees with its records, a stream total that disagrees with the chunk
    sizes) must be reported as corrupt, as the oracle's reader reports them;
    random bit flips and cuts must end in OK or corrupt, and a stream the
    oracle's reader accepts must decode to the same bits."""
    rng = np.random.default_rng(23 + D)
    T, B = 2, 300
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.3)
    x[0, 5, 7], x[0, 5, 9], x[1, 200, 3] = 1e6, -1e6, np.nan  # outliers
    x[1, 64:128] = rng.normal(0, 1e4, (64, D)).astype(np.float32)  # a raw tile
    x[1, 130] = x[1, 70]  # a reference into it
    cfg = make_cfg(T, B, D, eb_mode=0, eb=(1e-2,))
    plan = ec.Plan(T, B, D, 1, 0, 1e-2)
    good = O.compress(cfg, 0, x).stream
    st = SF.parse(good)
    y = torch.empty(T, B, D, device="cuda")

    def gpu_decode(buf, plan=plan, y=y):
        t = torch.from_numpy(np.ascontiguousarray(buf, np.uint8)).cuda()
        y.fill_(float("nan"))
        plan.decompress(t, y)
        return plan.ratio(raise_on_error=False)[-1], y.cpu().numpy()

    rc, yg = gpu_decode(good)
    assert rc == ec.EC_OK
    np.testing.assert_array_equal(yg.view(np.uint32), O.decompress(cfg, good).view(np.uint32))

    seg0 = st.segments[0]
    packed = [tl for s in st.segments for tl in s.tiles if tl.mode == 1]
    with_refs = [tl for tl in packed if tl.n - tl.U > 0]
    with_out = [tl for tl in packed if tl.n_out > 0]
    assert packed and with_refs and with_out
    cases = []
    b = good.copy(); b[0] ^= 1; cases.append(("magic", b))
    cases.append(("truncated", good[:-16].copy()))
    b = good.copy(); c0 = 64 + 16; b[c0:c0 + 8] = np.frombuffer(np.uint64(1 << 40).tobytes(), np.uint8)
    cases.append(("segment offset", b))
    b = good.copy(); d = seg0.offset + 32 + 4 * (seg0.ntiles - 1)
    b[d:d + 4] = np.frombuffer(np.uint32(0xFFFFFFF0).tobytes(), np.uint8); cases.append(("tile entry", b))
    b = good.copy(); b[packed[0].offset + 16] = 13; cases.append(("width 13", b))
    tl = with_refs[0]; nblk = (tl.U * D + 63) // 64; orf = tl.offset + (16 + nblk + 3) // 4 * 4
    b = good.copy(); b[orf:orf + 2] = np.frombuffer(np.uint16(0xFFFF).tobytes(), np.uint8)
    cases.append(("forward reference", b))
    tl = with_out[0]; nblk = (tl.U * D + 63) // 64
    oop = tl.offset + ((16 + nblk + 3) // 4 * 4 + 2 * (tl.n - tl.U) + 3) // 4 * 4
    b = good.copy(); b[oop:oop + 4] = np.frombuffer(np.uint32(tl.U * D + 5).tobytes(), np.uint8)
    cases.append(("outlier position", b))
    tl = [t for t in with_out if t.n_out >= 2][0]; nblk = (tl.U * D + 63) // 64
    oop = tl.offset + ((16 + nblk + 3) // 4 * 4 + 2 * (tl.n - tl.U) + 3) // 4 * 4
    b = good.copy(); b[oop + 4:oop + 8] = b[oop:oop + 4]
    cases.append(("outlier order", b))
    sg = [s for s in st.segments if s.n_out > 0][0]
    b = good.copy(); b[seg0.offset + 16] ^= 1; cases.append(("segment U", b))
    b = good.copy(); b[sg.offset + 20] ^= 2; cases.append(("segment n_out", b))
    b = np.concatenate([good, np.zeros(16, np.uint8)])
    b[48:56] = np.frombuffer(np.uint64(good.size + 16).tobytes(), np.uint8)
    cases.append(("total vs chunk sizes", b))
    for label, bad in cases:
        say(f"[corrupt] {label}")
        rc_o, _ = O.decompress(cfg, bad, status=True)
        assert rc_o == O.ERR_CORRUPT, label
        rc_g, _ = gpu_decode(bad)
        assert rc_g == ec.EC_ERR_CORRUPT, label
    say("[corrupt] wrong shape")
    plan2 = ec.Plan(T, B + 1, D, 1, 0, 1e-2)
    y2 = torch.empty(T, B + 1, D, device="cuda")
    assert gpu_decode(good, plan2, y2)[0] == ec.EC_ERR_CORRUPT

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
    say(f"[corrupt] random: {n_ok} decoded, {n_bad} rejected")
    assert n_bad > 0


@pytest.mark.parametrize("coder", [ec.CODER_BITPACK, ec.CODER_HUFFMAN, ec.CODER_AUTO])
def test_graph_replays_match_eager_calls(coder):
    """Compression and decompression captured in HIP graphs (one per input)
    and replayed several times, with eager calls of the same plan in between:
    every replay's stream and output equal the eager results for its input
    (nothing in either call allocates, clears with a memset or synchronizes),
    with bit planes, with Huffman segments, and with the automatic choice."""
    T, B, D = 3, 1000, 128
    rng = np.random.default_rng(31)
    xs = [torch.from_numpy(dup_rows(rng, T, B, D, scale=sc, frac_unique=fu)).cuda()
          for sc, fu in ((1.0, 0.4), (0.01, 0.9))]
    xs[1][0, 7, 5] = float("nan")
    plan = ec.Plan(T, B, D, 1, ec.EB_REL_RANGE, 0.01, coder=coder)
    out = plan.empty_stream()
    y = torch.empty(T, B, D, device="cuda")
    refs = []
    for i, x in enumerate(xs):
        plan.compress(x, out, i)
        _, nb, _ = plan.ratio()
        plan.decompress(out[:nb], y)
        plan.ratio()
        refs.append((out[:nb].clone(), y.clone(), nb))
    say("[graph] capture")
    side = torch.cuda.Stream()
    graphs = []
    for i, x in enumerate(xs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            plan.compress(x, out, i)
            plan.decompress(out, y)
        graphs.append(g)
    torch.cuda.synchronize()
    for r, i in enumerate([0, 1, 1, 0, 1, 0]):
        say(f"[graph] replay {r} of graph {i}")
        graphs[i].replay()
        torch.cuda.synchronize()
        ref_s, ref_y, nb = refs[i]
        assert torch.equal(out[:nb], ref_s), f"replay {r}: stream"
        assert torch.equal(y.view(torch.int32), ref_y.view(torch.int32)), f"replay {r}: values"
        if r % 2 == 0:  # eager work of the same plan between replays
            plan.compress(xs[1 - i], out, 1 - i)
            plan.ratio()
    assert plan.ratio(raise_on_error=False)[-1] == ec.EC_OK


@pytest.mark.parametrize("D", [64, 24])
def test_segment_beyond_65536_rows(D):
    """A segment of 70,000 rows: references are stored as 32-bit row indices,
    and first occurrences lie up to 70,000 rows back (fast path for D = 64,
    generic path for D = 24)."""
    rng = np.random.default_rng(D)
    x = dup_rows(rng, 1, 70000, D, scale=0.05, frac_unique=0.02)
    assert_parity(make_cfg(1, 70000, D, eb_mode=1, eb=(0.01,)), x, label=f"rows>65536 D={D}")


@pytest.mark.parametrize("D", [512, 700, 0])
def test_large_dims(D):
    """Large D on the generic kernels, up to the library's limit (0: the limit,
    set by their LDS): a tile record holds more than 256 blocks, so the
    decoder's scan of the widths reads other threads' writes."""
    D = D or int(ec.lib().ec_max_dim())
    say(f"[large D] D={D}")
    rng = np.random.default_rng(5)
    x = dup_rows(rng, 2, 130, D, scale=0.05, frac_unique=0.5)
    assert_parity(make_cfg(2, 130, D, eb_mode=0, eb=(1e-3,)), x, label=f"large D={D}")


@pytest.mark.parametrize("D", [100, 128])
def test_many_outliers_per_tile(D):
    """About 5 % of the elements far outside the code range: a packed tile
    record holds more outliers than the generic decoder stages in LDS (256),
    and the fast decoder's outlier runs span several 64-position chunks."""
    rng = np.random.default_rng(D + 1)
    T, B = 2, 200
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.6)
    hit = rng.random((T, B, D)) < 0.05
    x[hit] = rng.choice(np.array([-1e5, 1e5], np.float32), size=int(hit.sum()))
    cfg = make_cfg(T, B, D, eb_mode=0, eb=(1e-3,))
    st = SF.parse(O.compress(cfg, 0, x).stream)
    assert max(tl.n_out for s in st.segments for tl in s.tiles if tl.mode == 1) > 256
    assert_parity(cfg, x, label=f"outliers D={D}")


@pytest.mark.parametrize("T,B,D,P,mode", [(300, 70, 64, 1, 1), (40, 1, 128, 1, 0), (7, 64, 256, 2, 1),
                                          (33, 65, 128, 5, 0)])
def test_many_small_segments(T, B, D, P, mode):
    """Hundreds of segments of one or two tiles, one-row tables and chunks of
    a few rows on the D = 64*C kernels: most tiles are a segment's first and
    write its header and its entry in the chunk table."""
    rng = np.random.default_rng(T + B + D + P)
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.5)
    assert_parity(make_cfg(T, B, D, P, eb_mode=mode, eb=(0.01,)), x, label="small segments")


@pytest.mark.parametrize("D,P", [(128, 1), (256, 2), (24, 1)])
def test_rel_mode_with_classes_and_staircase(D, P):
    """Range-relative eb with per-table class multipliers (Algorithm 1's
    large / medium / small tables) and the staircase decay, mid-schedule."""
    rng = np.random.default_rng(D * 3 + P)
    T, B = 4, 300
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.5)
    x[1] *= 40.0  # tables with different ranges
    sched = {"kind": ec.SCHED_STEP, "k": 4.0, "phase": 100, "steps": 3}
    cfg = make_cfg(T, B, D, P, eb_mode=1, eb=[0.01, 0.02, 0.005, 0.01], mult=[1.0, 1.5, 0.5, 2.0],
                   sched=sched)
    assert_parity(cfg, x, it=60, sched=sched, label="rel+classes+step")


def test_special_values_wide_rows():
    """NaN payloads, infinities, signed zeros, an all-NaN table (stored raw)
    and a constant table at D = 256."""
    rng = np.random.default_rng(17)
    T, B, D = 3, 90, 256
    x = rng.normal(0, 1, (T, B, D)).astype(np.float32)
    x[0, 3, 200] = np.nan
    x[0, 4, 7] = np.inf
    x[0, 5, 255] = -np.inf
    x[0, 6, 3] = -0.0
    x[0, 7] = np.float32(np.uint32(0x7FC00123).view(np.float32))
    x[0, 70] = x[0, 7]
    x[1] = np.nan
    x[2] = 0.25
    assert_parity(make_cfg(T, B, D, eb_mode=1, eb=(0.01,)), x, label="special D=256")


@pytest.mark.parametrize("T,B,D,P", [(3, 129, 64, 2), (5, 300, 128, 7), (4, 3, 64, 5), (2, 1000, 256, 3),
                                     (40, 200, 128, 1)])
def test_ranges_found_by_the_quantize_pass(T, B, D, P):
    """Range-relative eb on D = 64*C: the quantize pass's range items run
    ahead of its tiles, which take tables in table-major order across
    chunks of different tile counts (and chunks without rows).  A table whose
    extremes are one NaN-free row, one all-NaN table, one whose values are
    zeros of both signs and one with an infinity are among them."""
    rng = np.random.default_rng(T * 101 + B + D + P)
    x = dup_rows(rng, T, B, D, scale=0.2)
    x[0, -1, 0] = 7.5            # the maximum in the last row of the last chunk
    x[0, 0, 1] = -3.25           # the minimum in the first row
    if T > 1:
        x[1] = np.nan
        x[1, B // 2, 3] = 0.5    # one value: zero range, eb not valid
    if T > 2:
        x[2] = 0.0
        x[2, ::2] = -0.0
    if T > 3:
        x[3, 0, 0] = np.inf
    assert_parity(make_cfg(T, B, D, P, eb_mode=1, eb=(0.02,)), x, label="fused range")
