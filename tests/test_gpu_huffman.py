"""GPU parity of the canonical Huffman coder (include/ec_huffman.h) against
the oracle's coder: codebook bytes, chunk table and words must be identical,
decoding must return the input, and a damaged stream must be rejected exactly
when the oracle rejects it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import error_bounded_lossy_amd as ec  # noqa: E402


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def coder():
    return ec.Huffman("cuda")


def oracle_encode(sym: np.ndarray):
    f = np.bincount(sym.astype(np.int64), minlength=O.HUFF_NSYM).astype(np.uint64)
    ln = O.huff_lengths(f)
    words, off = O.huff_encode(sym, ln)
    return O.huff_book_write(ln), off, words, ln


def gpu_encode(coder, sym: np.ndarray):
    n = sym.size
    book, off, words = coder.buffers(n)
    s = torch.from_numpy(sym.astype(np.uint16).view(np.int16)).cuda()
    coder.encode(s, book, off, words)
    st = coder.status()
    bk = book.cpu().numpy()
    nb = ec.huff_book_bytes(bk)
    o = off.cpu().numpy().view(np.uint32)
    w = words.cpu().numpy().view(np.uint32)[: int(o[-1])]
    return st, bk[:nb], o, w


def gpu_decode(coder, book: np.ndarray, off: np.ndarray, words: np.ndarray, n: int):
    b = torch.zeros(ec.HUFF_BOOK_MAX, dtype=torch.uint8, device="cuda")
    b[: book.size] = torch.from_numpy(book.astype(np.uint8))
    o = torch.from_numpy(off.astype(np.uint32).view(np.int32)).cuda()
    w = torch.from_numpy(np.ascontiguousarray(words, dtype=np.uint32).view(np.int32)).cuda()
    out = torch.zeros(max(n, 1), dtype=torch.int16, device="cuda")
    coder.decode(b, book.size, o, w, n, out)
    st = coder.status()
    return st, out[:n].cpu().numpy().view(np.uint16)


def check_parity(coder, sym: np.ndarray, what: str):
    say(f"[huffman] {what} n={sym.size}")
    rb, ro, rw, _ = oracle_encode(sym)
    st, gb, go, gw = gpu_encode(coder, sym)
    assert st == ec.EC_OK
    assert np.array_equal(gb, rb), "codebook differs"
    assert np.array_equal(go, ro), "chunk table differs"
    assert np.array_equal(gw, rw), f"words differ at {np.flatnonzero(gw != rw)[:8]}"
    st, back = gpu_decode(coder, gb, go, gw, sym.size)
    assert st == ec.EC_OK
    assert np.array_equal(back, sym.astype(np.uint16))


def laplace_codes(rng, n, scale):
    q = np.clip(np.rint(rng.laplace(0, scale, n)), -2047, 2047).astype(np.int64)
    return (q + 2047).astype(np.uint16)


@pytest.mark.parametrize("n", [1, 7, 8, 255, 256, 257, 1000, 65536 + 3, 1_000_003])
@pytest.mark.parametrize("scale", [0.3, 5.0, 200.0])
def test_laplace_codes(coder, n, scale):
    rng = np.random.default_rng(n + int(scale * 10))
    check_parity(coder, laplace_codes(rng, n, scale), f"laplace scale={scale}")


def test_empty_input(coder):
    check_parity(coder, np.zeros(0, np.uint16), "empty")


@pytest.mark.parametrize("n", [1, 300, 4096])
def test_single_symbol(coder, n):
    check_parity(coder, np.full(n, 2047, np.uint16), "one symbol")
    check_parity(coder, np.full(n, 0, np.uint16), "symbol 0")
    check_parity(coder, np.full(n, 4094, np.uint16), "symbol 4094")


def test_two_symbols_and_extremes(coder):
    rng = np.random.default_rng(2)
    check_parity(coder, rng.choice(np.array([0, 4094], np.uint16), 5000), "extremes")
    check_parity(coder, rng.choice(np.array([10, 11], np.uint16), 777, p=[0.999, 0.001]), "skewed")


def test_whole_alphabet_equal_and_random(coder):
    sym = np.tile(np.arange(4095, dtype=np.uint16), 3)
    np.random.default_rng(3).shuffle(sym)
    check_parity(coder, sym, "whole alphabet, equal")
    check_parity(coder, np.random.default_rng(4).integers(0, 4095, 300_000).astype(np.uint16),
                 "whole alphabet, uniform")


@pytest.mark.parametrize("m", [14, 20, 27])
def test_length_limit_with_fibonacci_weights(coder, m):
    a, b, f = 1, 1, []
    for _ in range(m):
        f.append(a)
        a, b = b, a + b
    syms = np.arange(2047 - m // 2, 2047 - m // 2 + m)
    sym = np.repeat(syms, f).astype(np.uint16)
    np.random.default_rng(m).shuffle(sym)
    check_parity(coder, sym, f"fibonacci m={m}")


@pytest.mark.parametrize("m,alpha", [(100, 3.0), (128, 3.0), (129, 3.0), (300, 1.6), (900, 2.0),
                                     (4095, 1.1)])
def test_heavy_tailed_counts(coder, m, alpha):
    """Power-law counts (rank r used about 2e5 / r^alpha times, at least
    once): trees far deeper than 12, so the length limit moves many codes,
    on both sides of 128 used symbols."""
    rng = np.random.default_rng(m)
    used = rng.choice(4095, m, replace=False)
    counts = np.maximum(1, (2e5 / np.arange(1, m + 1) ** alpha).astype(np.int64))
    sym = np.repeat(used, counts).astype(np.uint16)
    rng.shuffle(sym)
    check_parity(coder, sym, f"power law m={m}")


@pytest.mark.parametrize("n", [3 * 128 * 256, 3 * 128 * 256 + 77])
def test_wide_codes_overflow_the_stage(coder, n):
    """Near-uniform codes over the whole alphabet (about 12 bits each, about
    96 words per chunk): every 128-chunk decode group exceeds the LDS stage
    and is staged one wave at a time, with a ragged last chunk; then a last
    group of 100 chunks (about 9600 words, still too many) whose second wave
    holds 36 chunks, the last one partial."""
    rng = np.random.default_rng(n)
    sym = rng.integers(0, 4095, n).astype(np.uint16)
    check_parity(coder, sym, f"wide codes n={n}")
    tail = rng.integers(0, 4095, 128 * 256 + 100 * 256 - 100).astype(np.uint16)
    check_parity(coder, tail, "wide codes, short last group")


def test_many_ties(coder):
    rng = np.random.default_rng(9)
    used = rng.choice(4095, 600, replace=False)
    sym = np.repeat(used, rng.integers(1, 4, 600)).astype(np.uint16)
    rng.shuffle(sym)
    check_parity(coder, sym, "ties")


@pytest.mark.parametrize("m", [2, 3, 63, 64, 65, 66, 100, 126, 127, 128])
@pytest.mark.parametrize("pattern", ["small", "equal"])
def test_ties_in_the_small_tree(coder, m, pattern):
    """Up to 127 used symbols the tree is built by selects on one wave, from
    both queues in registers (two registers each, lanes 0-63 and 64-127);
    128 symbols take the rounds form.  Counts of 1-3 (or all equal) make
    leaves and internal nodes tie at almost every step, where the leaf must
    be taken first: the code lengths, hence the codebook bytes, must be the
    oracle's on both sides of 64 and of 127/128."""
    rng = np.random.default_rng(1000 + m)
    used = rng.choice(4095, m, replace=False)
    counts = rng.integers(1, 4, m) if pattern == "small" else np.full(m, 5)
    sym = np.repeat(used, counts).astype(np.uint16)
    rng.shuffle(sym)
    check_parity(coder, sym, f"small-tree ties m={m} {pattern}")


def test_symbol_outside_the_alphabet_is_reported(coder):
    sym = np.full(1000, 2047, np.uint16)
    sym[517] = 4095
    st, _, _, _ = gpu_encode(coder, sym)
    assert st == ec.EC_ERR_INVALID
    st, _, _, _ = gpu_encode(coder, np.full(1000, 2047, np.uint16))
    assert st == ec.EC_OK  # the status belongs to the last call


def test_workload_codes_full_size(coder):
    """Quantization codes of the 26x8192x128 pooled-lookup batch (range-
    relative eb 0.005 of each table's range), outliers counted as code 0:
    27.3 M symbols, the size the benchmark times."""
    import synth
    w = synth.workload("c3", iteration=3, device="cuda")
    x = w.x
    T = x.shape[0]
    flat = x.view(T, -1)
    fin = torch.isfinite(flat)
    lo = torch.where(fin, flat, torch.full_like(flat, float("inf"))).amin(1)
    hi = torch.where(fin, flat, torch.full_like(flat, float("-inf"))).amax(1)
    eb = (0.005 * (hi.double() - lo.double())).float().clamp_min(1e-30)
    q = torch.round(flat.double() / (2.0 * eb.double()[:, None]))
    q = torch.where(fin & (q.abs() <= 2047), q, torch.zeros_like(q))
    sym = (q + 2047).to(torch.int32).reshape(-1).cpu().numpy().astype(np.uint16)
    check_parity(coder, sym, "c3 codes")


def test_damaged_streams_are_rejected_like_the_oracle(coder):
    rng = np.random.default_rng(11)
    sym = laplace_codes(rng, 3000, 4.0)
    book, off, words, ln = oracle_encode(sym)
    n = sym.size

    def oracle_accepts(b, o, w):
        rc, l2 = O.huff_book_read(b)
        if rc != 0:
            return False, None
        if o[0] != 0:
            return False, None
        rc, out = O.huff_decode(w, o, n, l2, status=True)
        return rc == 0, out

    cases = []
    w = words.copy(); w[off[1] - 1] ^= 1; cases.append(("padding bit", book, off, w))
    o = off.copy(); o[1] += 1; cases.append(("chunk too long", book, o, words))
    o = off.copy(); o[2] = o[1] - 1; cases.append(("decreasing table", book, o, words))
    o = off.copy(); o[0] = 1; cases.append(("table not from 0", book, o, words))
    cases.append(("truncated words", book, off, words[:-1]))
    b = book.copy(); b[4] ^= 0x10; cases.append(("book not complete", b, off, words))
    cases.append(("short book", book[:-1], off, words))
    b = book.copy(); b[2] = 0xFF; b[3] = 0x0F; cases.append(("book past alphabet", b, off, words))
    for k in range(40):
        w = words.copy()
        i = int(rng.integers(0, w.size))
        w[i] ^= np.uint32(1 << int(rng.integers(0, 32)))
        cases.append((f"flip {k}", book, off, w))
    for name, b, o, w in cases:
        ok, ref = oracle_accepts(b, o, w)
        st, out = gpu_decode(coder, b, o, w, n)
        assert (st == ec.EC_OK) == ok, name
        assert st in (ec.EC_OK, ec.EC_ERR_CORRUPT), name
        if ok:
            assert np.array_equal(out, ref), name


def oracle_encode_segments(sym: np.ndarray, nseg: int):
    """The oracle's coder applied to each segment alone; chunk tables and
    words concatenated with the earlier segments' word counts added."""
    L = sym.size // nseg
    books, offs, words, base = [], [], [], 0
    for s in range(nseg):
        b, o, w, _ = oracle_encode(sym[s * L:(s + 1) * L])
        books.append(b)
        offs.append(o[:-1].astype(np.int64) + base)
        words.append(w)
        base += w.size
    off = np.concatenate(offs + [np.array([base])]).astype(np.uint32)
    return books, off, np.concatenate(words).astype(np.uint32) if words else np.zeros(0, np.uint32)


def check_segments(nseg: int, sym: np.ndarray, what: str):
    say(f"[huffman segments] {what} nseg={nseg} seg_len={sym.size // nseg}")
    coder = ec.Huffman("cuda", nseg=nseg)
    books, ro, rw = oracle_encode_segments(sym, nseg)
    n = sym.size
    book, off, words = coder.buffers(n)
    s = torch.from_numpy(sym.astype(np.uint16).view(np.int16)).cuda()
    coder.encode(s, book, off, words)
    assert coder.status() == ec.EC_OK
    go = off.cpu().numpy().view(np.uint32)
    gw = words.cpu().numpy().view(np.uint32)[: int(go[-1])]
    gb = book.cpu().numpy()
    for k in range(nseg):
        bk = gb[k * ec.HUFF_BOOK_MAX:(k + 1) * ec.HUFF_BOOK_MAX]
        assert np.array_equal(bk[: ec.huff_book_bytes(bk)], books[k]), f"codebook {k}"
    assert np.array_equal(go, ro), "chunk table differs"
    assert np.array_equal(gw, rw), f"words differ at {np.flatnonzero(gw != rw)[:8]}"
    out = torch.zeros(max(n, 1), dtype=torch.int16, device="cuda")
    coder.decode(book, ec.HUFF_BOOK_MAX, off, words, n, out)
    assert coder.status() == ec.EC_OK
    assert np.array_equal(out[:n].cpu().numpy().view(np.uint16), sym.astype(np.uint16))
    return coder, book, off, words


@pytest.mark.parametrize("nseg,L", [(2, 1000), (5, 256), (3, 257), (7, 1), (4, 13), (26, 4096),
                                    (6, 0), (3, 70_003), (40, 300)])
def test_segments_have_codebooks_of_their_own(nseg, L):
    """Segments of different widths and offsets (so that codebooks differ),
    lengths that are and are not multiples of 4, 8 and 256."""
    rng = np.random.default_rng(nseg * 1000 + L)
    parts = []
    for k in range(nseg):
        scale = [0.3, 4.0, 60.0][k % 3]
        q = np.clip(np.rint(rng.laplace(5 * k, scale, L)), -2047, 2047).astype(np.int64)
        parts.append((q + 2047).astype(np.uint16))
    sym = np.concatenate(parts) if parts else np.zeros(0, np.uint16)
    check_segments(nseg, sym, "laplace")


def test_segments_with_degenerate_members():
    """One segment with a single symbol, one with the whole alphabet, one with
    Fibonacci weights that hit the 12-bit limit."""
    L = 4095 * 3
    rng = np.random.default_rng(5)
    a = np.full(L, 100, np.uint16)
    b = np.tile(np.arange(4095, dtype=np.uint16), 3)
    rng.shuffle(b)
    f, x, y = [], 1, 1
    while sum(f) < L:
        f.append(x)
        x, y = y, x + y
    c = np.repeat(np.arange(2000, 2000 + len(f)), f)[:L].astype(np.uint16)
    rng.shuffle(c)
    check_segments(3, np.concatenate([a, b, c]), "degenerate")


def test_segments_full_size_per_table_codebooks():
    """The 26x8192x128 batch's codes with one codebook per table."""
    import synth
    import bench
    w = synth.workload("c3", iteration=3, device="cuda")
    sym = bench.workload_codes(w, torch).cpu().numpy().view(np.uint16)
    check_segments(26, sym, "c3 per table")


def test_segments_reject_a_damaged_codebook():
    rng = np.random.default_rng(8)
    sym = np.concatenate([laplace_codes(rng, 3000, 3.0), laplace_codes(rng, 3000, 30.0)])
    coder, book, off, words = check_segments(2, sym, "for damage")
    bad = book.clone()
    bad[ec.HUFF_BOOK_MAX + 4] ^= 0x10  # a length in segment 1's codebook: no longer complete
    out = torch.zeros(sym.size, dtype=torch.int16, device="cuda")
    coder.decode(bad, ec.HUFF_BOOK_MAX, off, words, sym.size, out)
    assert coder.status() == ec.EC_ERR_CORRUPT
    coder.decode(book, ec.HUFF_BOOK_MAX, off, words, sym.size, out)
    assert coder.status() == ec.EC_OK


def test_groups_of_more_than_256_chunks():
    """Past 2048 * 256 chunks a group of the size and write passes holds more
    than 256 chunks, so the write pass scans its offsets in several rounds
    (134.7 M codes)."""
    coder = ec.Huffman("cuda")
    rng = np.random.default_rng(21)
    n = 256 * 257 * 2048 + 5
    sym = laplace_codes(rng, n, 3.0)
    check_parity(coder, sym, "two-pass packing")
