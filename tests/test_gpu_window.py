"""GPU parity of windowed references (the vector-based LZ of section III-D
with the extended window of section III-E): streams byte for byte against
the oracle with the same window, reconstructions bitwise the oracle's, the
matches the oracle's, chains through RAW tiles, weak row hashes, Huffman
segments, and damaged distances reported as the oracle's reader reports
them."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import error_bounded_lossy_amd as ec  # noqa: E402
import oracle as O  # noqa: E402
import streamfmt as SF  # noqa: E402


def say(*a):
    print(*a, flush=True)


def zipf_rows(rng, T, B, D, distinct, a=1.1, scale=0.05):
    base = rng.normal(0, scale, (T, distinct, D)).astype(np.float32)
    p = 1.0 / np.arange(1, distinct + 1) ** a
    idx = rng.choice(distinct, size=(T, B), p=p / p.sum())
    return np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)


def run(cfg, x, it=0, bits=0, label=""):
    say(f"[window] {label} T={cfg.T} B={cfg.B} D={cfg.D} P={cfg.P} W={cfg.window} "
        f"coder={cfg.coder} bits={bits}")
    ref = O.compress(cfg, it, x, debug=True)
    plan = ec.Plan(cfg.T, cfg.B, cfg.D, cfg.P, cfg.eb_mode, cfg.eb[0], debug_hash_bits=bits,
                   coder=cfg.coder, window=cfg.window,
                   schedule={"kind": cfg.sched_kind, "t0": cfg.sched_t0} if cfg.sched_kind else None)
    xt = torch.from_numpy(x).cuda()
    first = torch.zeros(cfg.T, cfg.B, dtype=torch.int32, device="cuda")
    plan.debug_attach(first=first)
    out = plan.empty_stream()
    plan.compress(xt, out, it)
    cr, nbytes, st = plan.ratio()
    got = out[:nbytes].cpu().numpy()
    assert got.size == ref.stream.size, (got.size, ref.stream.size)
    if not np.array_equal(got, ref.stream):
        bad = np.nonzero(got != ref.stream)[0]
        raise AssertionError(f"stream differs at {bad.size} bytes, first {bad[:8]}")
    np.testing.assert_array_equal(first.cpu().numpy().astype(np.uint32), ref.first)
    y = torch.full_like(xt, float("nan"))
    plan.decompress(out[:nbytes], y)
    assert plan.ratio(raise_on_error=False)[-1] == ec.EC_OK
    yo = O.decompress(cfg, ref.stream)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))
    return ref, plan


def cfg_of(T, B, D, P, W, coder=1, mode=1, eb=0.01):
    return O.Config(T=T, B=B, D=D, P=P, eb_mode=mode, eb=(eb,), coder=coder, window=W)


CASES = [(2, 300, 128, 1, 1), (3, 700, 64, 2, 7), (2, 1000, 256, 1, 64), (4, 2100, 128, 3, 255),
         (1, 64, 64, 1, 255), (2, 1, 128, 1, 3), (2, 0, 64, 1, 5), (3, 4096, 64, 1, 32)]


@pytest.mark.parametrize("T,B,D,P,W", CASES)
@pytest.mark.parametrize("coder", [1, 3])
def test_shapes(T, B, D, P, W, coder):
    rng = np.random.default_rng(T * 7919 + B + D + W + coder)
    x = zipf_rows(rng, T, B, D, max(2, B // 8))
    if B > 8:
        x[0, 3, 1] = 1e6       # an outlier
        x[-1, 4, -1] = np.nan
        x[0, 5] = x[0, 3]      # a repeated row holding an outlier
    run(cfg_of(T, B, D, P, W, coder), x, it=1, label="shape")


@pytest.mark.parametrize("D,bits", [(64, 2), (128, 5), (256, 0)])
def test_raw_tiles_chains_and_weak_hashes(D, bits):
    """Matches that are repeated rows themselves, chains through RAW tiles,
    a RAW segment, and hash collisions that the row comparison rejects."""
    rng = np.random.default_rng(D + bits)
    T, B, W = 3, 1500, 40
    x = zipf_rows(rng, T, B, D, 30, scale=0.1)
    hot = x[0, 3].copy()
    x[0, 3::30] = hot
    x[0, 128:192] = rng.normal(0, 1e5, (64, D)).astype(np.float32)  # a RAW tile on the chain
    x[0, 153] = hot
    x[1] = np.nan                                                   # no valid eb: RAW segment
    for coder in (1, 3):
        run(cfg_of(T, B, D, 1, W, coder), x, bits=bits, label="raw/chain")


def test_full_size_c3_stream_and_table_vi_trend():
    """The 26-table dim-128 pooled batch at full size for W = 32 .. 255:
    whole streams byte for byte; the literals never grow with W."""
    import synth
    w = synth.workload("c3", iteration=1, device="cuda")
    T, B, D = w.shape
    xs = w.x.cpu().numpy()
    prev = None
    for W in (32, 64, 128, 255):
        cfg = O.Config(T=T, B=B, D=D, P=1, eb_mode=w.eb_mode, eb=tuple(w.eb), window=W,
                       sched_kind=w.sched_kind, sched_t0=w.sched_t0)
        say(f"[window] c3 full size W={W}")
        ref = O.compress(cfg, w.iteration, xs, debug=False)
        plan = ec.Plan(T, B, D, 1, w.eb_mode, w.eb, window=W,
                       schedule={"kind": w.sched_kind, "t0": w.sched_t0})
        out = plan.empty_stream()
        plan.compress(w.x, out, w.iteration)
        cr, nbytes, _ = plan.ratio()
        assert np.array_equal(out[:nbytes].cpu().numpy(), ref.stream)
        y = torch.empty_like(w.x)
        plan.decompress(out[:nbytes], y)
        plan.ratio()
        assert np.array_equal(y.cpu().numpy().view(np.uint32),
                              O.decompress(cfg, ref.stream).view(np.uint32))
        u = sum(s.U for s in SF.parse_segments(ref.stream))
        say(f"[window] c3 W={W}: CR {cr:.3f}, literal rows {u}")
        assert prev is None or u <= prev
        prev = u


def test_plans_and_streams():
    """A windowed plan decodes whole-segment streams; a plan without a window
    reports windowed segments corrupt; homo_counts needs whole-segment U."""
    rng = np.random.default_rng(3)
    T, B, D = 2, 500, 64
    x = zipf_rows(rng, T, B, D, 40)
    plain = O.compress(cfg_of(T, B, D, 1, 0), 0, x, debug=False).stream
    win = O.compress(cfg_of(T, B, D, 1, 16), 0, x, debug=False).stream
    y = torch.empty(T, B, D, device="cuda")
    wplan = ec.Plan(T, B, D, 1, ec.EB_REL_RANGE, 0.01, window=16)
    wplan.decompress(torch.from_numpy(plain).cuda(), y)
    assert wplan.ratio(raise_on_error=False)[-1] == ec.EC_OK
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                  O.decompress(cfg_of(T, B, D, 1, 0), plain).view(np.uint32))
    # another window's stream decodes too (the distances carry their own W)
    w8 = O.compress(cfg_of(T, B, D, 1, 8), 0, x, debug=False).stream
    wplan.decompress(torch.from_numpy(w8).cuda(), y)
    assert wplan.ratio(raise_on_error=False)[-1] == ec.EC_OK
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32),
                                  O.decompress(cfg_of(T, B, D, 1, 8), w8).view(np.uint32))
    pplan = ec.Plan(T, B, D, 1, ec.EB_REL_RANGE, 0.01)
    pplan.decompress(torch.from_numpy(win).cuda(), y)
    assert pplan.ratio(raise_on_error=False)[-1] == ec.EC_ERR_CORRUPT
    out = wplan.empty_stream()
    with pytest.raises(ec.ECError):
        wplan.homo_counts(torch.from_numpy(x).cuda(), out)


@pytest.mark.parametrize("coder", [1, 2])
def test_corrupt_distances(coder):
    """Distances 0, past W or before the segment, and flags that do not
    match, are reported corrupt as the oracle's reader reports them; random
    flips end in OK or corrupt with the oracle's reconstruction when OK."""
    rng = np.random.default_rng(21 + coder)
    T, B, D, W = 2, 400, 64, 12
    x = zipf_rows(rng, T, B, D, 20)
    cfg = cfg_of(T, B, D, 1, W, coder)
    good = O.compress(cfg, 0, x, debug=False).stream
    st = SF.parse(good)
    plan = ec.Plan(T, B, D, 1, ec.EB_REL_RANGE, 0.01, window=W, coder=3)
    y = torch.empty(T, B, D, device="cuda")

    def gpu_rc(buf):
        plan.decompress(torch.from_numpy(buf).cuda(), y)
        return plan.ratio(raise_on_error=False)[-1]

    seg = st.segments[0]
    tl = next(t for t in seg.tiles if t.mode != 0 and t.U < t.n)
    orf = tl.offset + (16 if tl.mode == 2 else 16 + (len(tl.widths) + 3) // 4 * 4)
    cases = []
    for v in (0, W + 1, 255):
        bad = good.copy()
        bad[orf] = v
        cases.append(bad)
    t0 = seg.tiles[0]
    if t0.mode != 0 and t0.U < t0.n:
        i0 = next(i for i in range(t0.n) if not (t0.bitmap >> i) & 1)
        if i0 < W:
            bad = good.copy()
            bad[t0.offset + (16 if t0.mode == 2 else 16 + (len(t0.widths) + 3) // 4 * 4)] = i0 + 1
            cases.append(bad)
    for flags in (1 | (W << 8), 5, 0x10005):
        bad = good.copy()
        bad[seg.offset + 12:seg.offset + 16] = np.frombuffer(np.uint32(flags).tobytes(), np.uint8)
        cases.append(bad)
    for k, bad in enumerate(cases):
        say(f"[window] targeted damage {k}")
        assert O.decompress(cfg, bad, status=True)[0] == O.ERR_CORRUPT
        assert gpu_rc(bad) == ec.EC_ERR_CORRUPT, k
    for i in range(60):
        bad = good.copy()
        for _ in range(int(rng.integers(1, 3))):
            bad[int(rng.integers(0, bad.size))] ^= np.uint8(1 << int(rng.integers(0, 8)))
        rc_o, yo = O.decompress(cfg, bad, status=True)
        rc_g = gpu_rc(bad)
        assert rc_g in (ec.EC_OK, ec.EC_ERR_CORRUPT)
        if rc_o == O.OK:
            assert rc_g == ec.EC_OK, i
            np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))
