"""Pins of the oracle's canonical Huffman coder (CPU only).

The coder is the entropy stage of section III-D of arXiv 2407.04272; the
pages fix no construction, so these tests pin the oracle to outside facts:
RFC 1951 section 3.2.2's worked example of canonical codes, brute-force
optimality on small alphabets, Shannon's bounds, the Kraft equality of a
complete code, hand-worked results of ITU-T T.81 Annex K.3's length limiting,
closed forms for equal and Fibonacci frequencies, and hand-encoded words.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle as O

NSYM, MAXLEN, CHUNK = O.HUFF_NSYM, O.HUFF_MAXLEN, O.HUFF_CHUNK


def freq_of(pairs):
    f = np.zeros(NSYM, np.uint64)
    for s, v in pairs.items():
        f[s] = v
    return f


def kraft(lengths):
    return sum(2.0 ** -int(l) for l in lengths if l)


def test_rfc1951_canonical_codes_example():
    # RFC 1951 section 3.2.2: lengths (3,3,3,3,3,2,4,4) for A..H give
    # 010 011 100 101 110 00 1110 1111
    ln = np.zeros(NSYM, np.uint8)
    ln[:8] = [3, 3, 3, 3, 3, 2, 4, 4]
    code = O.huff_codes(ln)
    want = ["010", "011", "100", "101", "110", "00", "1110", "1111"]
    got = [format(int(code[i]), f"0{int(ln[i])}b") for i in range(8)]
    assert got == want


def brute_min_cost(f):
    """Minimum sum f*l over length vectors satisfying Kraft (exhaustive)."""
    m = len(f)
    best = None
    best_sets = []
    for ls in itertools.product(range(1, m), repeat=m):
        if sum(2.0 ** -l for l in ls) > 1.0 + 1e-12:
            continue
        c = sum(a * b for a, b in zip(f, ls))
        if best is None or c < best:
            best, best_sets = c, [ls]
        elif c == best:
            best_sets.append(ls)
    return best, best_sets


@pytest.mark.parametrize("seed", range(40))
def test_optimal_on_small_alphabets(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(2, 7))
    f = [int(v) for v in rng.integers(1, 6 if seed % 2 else 40, size=m)]
    syms = sorted(rng.choice(NSYM, size=m, replace=False).tolist())
    ln = O.huff_lengths(freq_of(dict(zip(syms, f))))
    got = [int(ln[s]) for s in syms]
    best, sets = brute_min_cost(f)
    assert sum(a * b for a, b in zip(f, got)) == best
    # taking the leaf first on equal weights gives, among the optimal codes,
    # the smallest longest code and the smallest sum of squared lengths
    assert max(got) == min(max(s) for s in sets)
    assert sum(l * l for l in got) == min(sum(l * l for l in s) for s in sets)
    assert abs(kraft(got) - 1.0) < 1e-12
    assert int(np.count_nonzero(ln)) == m


def test_lengths_follow_frequency_then_symbol_order():
    rng = np.random.default_rng(5)
    f = np.zeros(NSYM, np.uint64)
    used = rng.choice(NSYM, size=300, replace=False)
    f[used] = rng.integers(1, 30, size=300)  # many ties
    ln = O.huff_lengths(f)
    order = sorted(used.tolist(), key=lambda s: (-int(f[s]), s))
    seq = [int(ln[s]) for s in order]
    assert seq == sorted(seq)


def test_zero_and_one_used_symbols():
    assert not O.huff_lengths(np.zeros(NSYM, np.uint64)).any()
    ln = O.huff_lengths(freq_of({2047: 10}))
    assert ln[2047] == 1 and int(np.count_nonzero(ln)) == 1
    assert O.huff_codes(ln)[2047] == 0


def test_equal_frequencies_over_the_whole_alphabet():
    # 4095 equal weights: a complete code with a lengths of 11 and b of 12 has
    # a + b = 4095 and 2a + b = 4096, so one code of 11 bits; the tie goes to
    # the smallest symbol
    ln = O.huff_lengths(np.ones(NSYM, np.uint64))
    assert ln[0] == 11 and (ln[1:] == 12).all()


def fib(n):
    a, b = 1, 1
    out = []
    for _ in range(n):
        out.append(a)
        a, b = b, a + b
    return out


def test_fibonacci_frequencies_without_limit():
    # m Fibonacci weights give lengths 1, 2, ..., m-2, m-1, m-1 (largest
    # weight shortest); m = 13 reaches exactly the 12-bit limit
    m = 13
    f = fib(m)
    ln = O.huff_lengths(freq_of({100 + i: v for i, v in enumerate(f)}))
    got = [int(ln[100 + i]) for i in range(m)]
    assert got == [12, 12] + list(range(11, 0, -1))


def test_annex_k3_length_limit_by_hand():
    # m = 14 Fibonacci weights: the tree has depths 1..12 once and two leaves
    # at 13.  Annex K.3 moves the pair at 13: one to 12 (beside its
    # prefix), and the only code at 11 splits into two codes at 12.  Result:
    # lengths 1..10 once, four codes at 12.
    m = 14
    f = fib(m)
    ln = O.huff_lengths(freq_of({i: v for i, v in enumerate(f)}))
    got = [int(ln[i]) for i in range(m)]
    # lengths go to weights in descending order, smallest symbol first on ties
    assert sorted(got) == list(range(1, 11)) + [12] * 4
    assert got[::-1][:10] == list(range(1, 11))
    assert abs(kraft(got) - 1.0) < 1e-12


@pytest.mark.parametrize("m", [20, 40, 90])
def test_length_limit_keeps_the_code_complete(m):
    f = fib(m)  # unlimited depth m-1 > 12
    ln = O.huff_lengths(freq_of({3 * i: v for i, v in enumerate(f)}))
    got = [int(ln[3 * i]) for i in range(m)]
    assert max(got) == MAXLEN and min(got) >= 1
    assert abs(kraft(got) - 1.0) < 1e-12
    assert got == sorted(got, reverse=True)  # weights ascend with i


@pytest.mark.parametrize("sigma", [0.7, 3.0, 40.0, 300.0])
def test_shannon_bounds_on_gaussian_codes(sigma):
    rng = np.random.default_rng(int(sigma * 10))
    q = np.clip(np.rint(rng.normal(0, sigma, 200_000)), -2047, 2047).astype(np.int64)
    f = np.bincount(q + 2047, minlength=NSYM).astype(np.uint64)
    ln = O.huff_lengths(f)
    p = f[f > 0] / f.sum()
    H = float(-(p * np.log2(p)).sum())
    L = float((f * ln).sum() / f.sum())
    assert H - 1e-9 <= L <= H + 1.0
    assert ln.max() <= MAXLEN


def test_hand_encoded_word():
    # RFC example codes, symbols F A H -> 00 010 1111, MSB first in bit 31
    ln = np.zeros(NSYM, np.uint8)
    ln[:8] = [3, 3, 3, 3, 3, 2, 4, 4]
    words, off = O.huff_encode([5, 0, 7], ln)
    assert words.tolist() == [0x17800000]
    assert off.tolist() == [0, 1]


def test_chunks_start_on_word_boundaries():
    # a single used symbol codes as one 0 bit: 256 bits fill 8 words, the
    # 257th symbol starts word 8
    ln = O.huff_lengths(freq_of({2047: 1}))
    words, off = O.huff_encode(np.full(257, 2047), ln)
    assert off.tolist() == [0, 8, 9] and (words == 0).all() and words.size == 9
    # 300 codes of 3 bits: chunk 0 is 768 bits = 24 words; chunk 1 holds 44
    # codes = 132 bits, padded with zeros to 5 words
    ln = np.zeros(NSYM, np.uint8)
    ln[:8] = [3, 3, 3, 3, 3, 2, 4, 4]
    words, off = O.huff_encode(np.full(300, 4), ln)  # code 110
    assert off.tolist() == [0, 24, 29]
    bits = "".join(format(int(w), "032b") for w in words[24:29])
    assert bits == "110" * 44 + "0" * (160 - 132)


@pytest.mark.parametrize("n", [0, 1, 255, 256, 257, 1000, 4096 + 17])
def test_round_trip_and_independent_bit_reader(n):
    rng = np.random.default_rng(n)
    q = np.clip(np.rint(rng.laplace(0, 6, n)), -2047, 2047).astype(np.int64)
    sym = (q + 2047).astype(np.uint16)
    f = np.bincount(sym, minlength=NSYM).astype(np.uint64)
    ln = O.huff_lengths(f)
    words, off = O.huff_encode(sym, ln)
    assert off[-1] == words.size
    out = O.huff_decode(words, off, n, ln)
    assert (out == sym).all()
    # read the bits back with a dictionary of code strings
    code = O.huff_codes(ln)
    book = {format(int(code[s]), f"0{int(ln[s])}b"): s for s in range(NSYM) if ln[s]}
    dec = []
    for c in range(len(off) - 1):
        bits = "".join(format(int(w), "032b") for w in words[off[c]:off[c + 1]])
        cur = ""
        k = 0
        for _ in range(min(CHUNK, n - c * CHUNK)):
            while cur not in book:
                cur += bits[k]
                k += 1
            dec.append(book[cur])
            cur = ""
        assert set(bits[k:]) <= {"0"} and len(bits) - k < 32
    assert dec == sym.tolist()
    # total size: sum of code lengths per chunk, rounded up to words
    per = [int(ln[sym[c:c + CHUNK]].astype(np.int64).sum()) for c in range(0, n, CHUNK)]
    assert words.size == sum((b + 31) // 32 for b in per)


def test_codebook_bytes_by_hand_and_round_trip():
    ln = np.zeros(NSYM, np.uint8)
    ln[2046], ln[2047], ln[2048] = 2, 1, 2
    book = O.huff_book_write(ln)
    assert book.tolist() == [0xFE, 0x07, 0x00, 0x08, 0x12, 0x02]
    rc, back = O.huff_book_read(book)
    assert rc == 0 and (back == ln).all()
    assert O.huff_book_write(np.zeros(NSYM, np.uint8)).tolist() == [1, 0, 0, 0]
    rc, back = O.huff_book_read(np.array([1, 0, 0, 0], np.uint8))
    assert rc == 0 and not back.any()
    rng = np.random.default_rng(1)
    f = np.zeros(NSYM, np.uint64)
    f[rng.choice(NSYM, 700, replace=False)] = rng.integers(1, 1000, 700)
    ln = O.huff_lengths(f)
    rc, back = O.huff_book_read(O.huff_book_write(ln))
    assert rc == 0 and (back == ln).all()


def test_codebook_rejects_malformed_books():
    good = np.array([0xFE, 0x07, 0x00, 0x08, 0x12, 0x02], np.uint8)
    assert O.huff_book_read(good[:5])[0] != 0            # short
    assert O.huff_book_read(np.array([0xFE, 0x07, 0x00, 0x08, 0x12, 0x12], np.uint8))[0] != 0  # pad
    assert O.huff_book_read(np.array([0xFE, 0x07, 0x00, 0x08, 0x22, 0x02], np.uint8))[0] != 0  # Kraft
    assert O.huff_book_read(np.array([0xFE, 0x07, 0x00, 0x08, 0x10, 0x02], np.uint8))[0] != 0  # lo unused
    assert O.huff_book_read(np.array([0xFF, 0x0F, 0xFF, 0x0F, 0x01], np.uint8))[0] != 0  # sym 4095
    assert O.huff_book_read(np.array([5, 0, 5, 0, 0x02], np.uint8))[0] != 0  # lone symbol, length 2
    assert O.huff_book_read(np.array([5, 0, 5, 0, 0x0D], np.uint8))[0] != 0  # length 13
    assert O.huff_book_read(np.array([5, 0, 5, 0, 0x01], np.uint8))[0] == 0


def test_decode_rejects_malformed_chunks():
    ln = np.zeros(NSYM, np.uint8)
    ln[:8] = [3, 3, 3, 3, 3, 2, 4, 4]
    sym = np.array([5, 0, 7] * 100, np.uint16)
    words, off = O.huff_encode(sym, ln)
    assert O.huff_decode(words, off, sym.size, ln, status=True)[0] == 0
    w = words.copy()
    w[off[1] - 1] |= 1  # a padding bit
    assert O.huff_decode(w, off, sym.size, ln, status=True)[0] != 0
    o = off.copy()
    o[1] += 1  # chunk 0 no longer ends in its last word
    assert O.huff_decode(words, o, sym.size, ln, status=True)[0] != 0
    assert O.huff_decode(words[:-1], off, sym.size, ln, status=True)[0] != 0  # truncated
    # an incomplete book leaves code words that decode to nothing
    ln2 = ln.copy()
    ln2[7] = 0
    assert O.huff_decode(np.array([0xFFFFFFFF], np.uint32), np.array([0, 1], np.uint32), 1, ln2,
                         status=True)[0] != 0
