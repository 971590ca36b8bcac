"""Independent reader of the compressed stream, written from the layout spec
(not from either implementation).  It walks every structure, records which
bytes it interpreted, and rebuilds codes, outlier flags, first-occurrence
maps and reconstructed values with numpy, so tests can check that:
  - every byte not covered by a structure is a zero pad byte;
  - the bit planes are the bit transpose of the zigzag codes;
  - widths are the bit length of each block's largest zigzag code;
  - the reconstruction meets the error bound.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def _u(buf, off, n):
    return int.from_bytes(bytes(buf[off:off + n]), "little")


def _a(v, a):
    return (v + a - 1) // a * a


@dataclass
class Tile:
    offset: int
    size: int
    bitmap: int
    n_out: int
    U: int
    mode: int
    n: int
    widths: np.ndarray | None = None
    refs: np.ndarray | None = None
    opos: np.ndarray | None = None
    oval: np.ndarray | None = None
    zz: np.ndarray | None = None       # zigzag codes of E (U*D), BITPACK only


@dataclass
class Segment:
    p: int
    t: int
    offset: int
    rows: int
    ntiles: int
    eb: float
    valid: bool
    U: int
    n_out: int
    nbytes: int
    tiles: list = field(default_factory=list)
    huff: bool = False
    window: int = 0
    lengths: np.ndarray | None = None
    codes: dict | None = None


@dataclass
class Stream:
    T: int
    B: int
    D: int
    P: int
    eb_mode: int
    iter: int
    total: int
    chunk_bytes: list
    segments: list
    covered: np.ndarray
    coder: int = 1


def unzigzag(z):
    z = z.astype(np.int64)
    return np.where(z & 1, -((z + 1) // 2), z // 2)


def parse(buf: np.ndarray) -> Stream:
    buf = np.asarray(buf, dtype=np.uint8)
    cov = np.zeros(buf.size, dtype=bool)

    def mark(off, n):
        assert off + n <= buf.size, "structure runs past the end of the stream"
        assert not cov[off:off + n].any(), "overlapping structures"
        cov[off:off + n] = True

    assert _u(buf, 0, 4) == 0x434C4245 and _u(buf, 4, 2) == 1
    coder = _u(buf, 6, 2)
    assert coder in (1, 2, 3)
    T, B, D, P = (_u(buf, o, 4) for o in (8, 12, 16, 20))
    assert _u(buf, 24, 4) == 64
    eb_mode = _u(buf, 28, 4)
    it = int(np.int64(np.uint64(_u(buf, 32, 8))))
    assert _u(buf, 40, 8) == 4 * T * B * D
    total = _u(buf, 48, 8)
    assert total == buf.size
    mark(0, 64)
    chunk_bytes = [_u(buf, 64 + 8 * p, 8) for p in range(P)]
    mark(64, 8 * P)
    at = 64 + _a(8 * P, 16)
    segs = []
    rb = None
    for p in range(P):
        c0 = at
        r0 = p * B // P
        rows = (p + 1) * B // P - r0
        mark(c0, 8 * T)
        for t in range(T):
            so = _u(buf, c0 + 8 * t, 8)
            s0 = c0 + so
            assert s0 % 16 == 0
            seg = Segment(p, t, s0, _u(buf, s0, 4), _u(buf, s0 + 4, 4),
                          float(np.frombuffer(bytes(buf[s0 + 8:s0 + 12]), np.float32)[0]),
                          bool(_u(buf, s0 + 12, 4) & 1), _u(buf, s0 + 16, 4),
                          _u(buf, s0 + 20, 4), _u(buf, s0 + 24, 8))
            flags = _u(buf, s0 + 12, 4)
            seg.window = (flags >> 8) & 0xFF
            assert flags >> 16 == 0
            assert (flags & 0xFF) in ((0, 1, 3) if seg.window == 0 else (5, 7))
            seg.huff = bool(flags & 2)
            # coder 1: no Huffman segment; coder 2: every valid segment is one
            assert not (seg.huff and coder == 1)
            assert not (coder == 2 and seg.valid and not seg.huff)
            assert seg.rows == rows and seg.ntiles == (rows + 63) // 64
            mark(s0, 32)
            mark(s0 + 32, 4 * seg.ntiles)
            rb = ref_bytes(rows, seg.window)
            rdt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[rb]
            if seg.huff:
                bo = s0 + 32 + _a(4 * seg.ntiles, 16)
                seg.lengths, nbook = read_book(buf, bo)
                mark(bo, nbook)
                seg.codes = canonical_codes(seg.lengths)
            for k in range(seg.ntiles):
                ro = s0 + _u(buf, s0 + 32 + 4 * k, 4)
                assert ro % 16 == 0
                n = min(64, rows - 64 * k)
                tl = Tile(ro, 0, _u(buf, ro, 8), _u(buf, ro + 8, 4), _u(buf, ro + 12, 2),
                          int(buf[ro + 14]), n)
                mark(ro, 15)
                assert bin(tl.bitmap).count("1") == tl.U
                raw_size = 16 + _a(4 * n * D, 16)
                if tl.mode == 0:
                    mark(ro + 16, 4 * n * D)
                    tl.size = raw_size
                    if seg.valid:
                        # the rule: a coded record only when strictly smaller than RAW
                        raw = np.frombuffer(bytes(buf[ro + 16:ro + 16 + 4 * n * D]),
                                            np.float32).reshape(n, D)
                        us = [i for i in range(n) if (tl.bitmap >> i) & 1]
                        q, o = quantize_np(raw[us].reshape(-1), seg.eb)
                        if seg.huff:
                            coded = huff_size(q, o, n, len(us), D, rows, seg.lengths, seg.window)
                        else:
                            coded = bitpack_size(raw, tl.bitmap, n, D, seg.eb, rows, seg.window)
                        assert coded >= raw_size, "RAW tile whose coded record would be smaller"
                elif tl.mode == 2:
                    assert seg.huff and seg.valid
                    nE = tl.U * D
                    nd = n - tl.U
                    tl.refs = np.frombuffer(bytes(buf[ro + 16:ro + 16 + rb * nd]),
                                            rdt).astype(np.int64)
                    mark(ro + 16, rb * nd)
                    oop = _a(16 + rb * nd, 4)
                    tl.opos = np.frombuffer(bytes(buf[ro + oop:ro + oop + 4 * tl.n_out]),
                                            np.uint32).astype(np.int64)
                    tl.oval = np.frombuffer(bytes(buf[ro + oop + 4 * tl.n_out:
                                                      ro + oop + 8 * tl.n_out]), np.uint32)
                    mark(ro + oop, 8 * tl.n_out)
                    oct_ = oop + 8 * tl.n_out
                    nch = (nE + 255) // 256
                    ct = [_u(buf, ro + oct_ + 4 * c, 4) for c in range(nch + 1)]
                    mark(ro + oct_, 4 * (nch + 1))
                    ow = oct_ + 4 * (nch + 1)
                    mark(ro + ow, 4 * ct[-1])
                    words = np.frombuffer(bytes(buf[ro + ow:ro + ow + 4 * ct[-1]]), np.uint32)
                    sym = decode_chunks(words, ct, nE, seg.lengths, seg.codes)
                    q = sym.astype(np.int64) - 2047
                    tl.zz = np.where(q >= 0, 2 * q, -2 * q - 1)
                    tl.size = _a(ow + 4 * ct[-1], 16)
                    assert tl.size < raw_size, "Huffman tile not smaller than RAW"
                else:
                    assert tl.mode == 1 and seg.valid and not seg.huff
                    nE = tl.U * D
                    nblk = (nE + 63) // 64
                    tl.widths = buf[ro + 16:ro + 16 + nblk].copy()
                    mark(ro + 16, nblk)
                    orf = _a(16 + nblk, 4)
                    nd = n - tl.U
                    tl.refs = np.frombuffer(bytes(buf[ro + orf:ro + orf + rb * nd]),
                                            rdt).astype(np.int64)
                    mark(ro + orf, rb * nd)
                    oop = _a(orf + rb * nd, 4)
                    tl.opos = np.frombuffer(bytes(buf[ro + oop:ro + oop + 4 * tl.n_out]),
                                            np.uint32).astype(np.int64)
                    tl.oval = np.frombuffer(bytes(buf[ro + oop + 4 * tl.n_out:
                                                      ro + oop + 8 * tl.n_out]), np.uint32)
                    mark(ro + oop, 8 * tl.n_out)
                    opl = _a(oop + 8 * tl.n_out, 8)
                    sw = int(tl.widths.astype(np.int64).sum())
                    mark(ro + opl, 8 * sw)
                    planes = np.frombuffer(bytes(buf[ro + opl:ro + opl + 8 * sw]), np.uint64)
                    zz = np.zeros(nblk * 64, np.int64)
                    pos = 0
                    lane = np.arange(64, dtype=np.uint64)
                    for b in range(nblk):
                        w = int(tl.widths[b])
                        for j in range(w):
                            bits = (planes[pos + j] >> lane) & np.uint64(1)
                            zz[64 * b:64 * b + 64] |= bits.astype(np.int64) << j
                        pos += w
                    tl.zz = zz[:nE]
                    assert not zz[nE:].any()
                    tl.size = _a(opl + 8 * sw, 16)
                    assert tl.size < raw_size, "BITPACK tile not smaller than RAW"
                seg.tiles.append(tl)
            segs.append(seg)
        at += chunk_bytes[p]
    assert at == total
    return Stream(T, B, D, P, eb_mode, it, total, chunk_bytes, segs, cov, coder)


def read_book(buf, off):
    """Codebook at off: u16 lowest, u16 highest symbol, 4-bit lengths (low
    nibble first).  Returns (lengths [4095], bytes); checks it is tight and a
    complete prefix code (or one symbol of length 1)."""
    lo, hi = _u(buf, off, 2), _u(buf, off + 2, 2)
    lengths = np.zeros(4095, np.int64)
    if hi < lo:
        assert (lo, hi) == (1, 0)
        return lengths, 4
    nb = hi - lo + 1
    for k in range(nb):
        lengths[lo + k] = (int(buf[off + 4 + k // 2]) >> (4 * (k & 1))) & 15
    if nb & 1:
        assert int(buf[off + 4 + nb // 2]) >> 4 == 0
    assert lengths[lo] and lengths[hi] and lengths.max() <= 12
    used = lengths[lengths > 0]
    if used.size == 1:
        assert used[0] == 1
    else:
        assert sum(2 ** (12 - int(l)) for l in used) == 2 ** 12
    return lengths, 4 + (nb + 1) // 2


def canonical_codes(lengths):
    """Bit strings of the canonical code (shorter first, then by symbol;
    consecutive values, shifted left at each longer length)."""
    syms = sorted((int(l), s) for s, l in enumerate(lengths) if l)
    out, code, prev = {}, 0, None
    for l, s in syms:
        if prev is not None:
            code = (code + 1) << (l - prev)
        out[format(code, f"0{l}b")] = s
        prev = l
    return out


def decode_chunks(words, ct, n, lengths, codes):
    """Symbols of n Huffman-coded values in 256-symbol chunks (chunk c in
    words[ct[c]:ct[c+1]], MSB first, the rest of its last word zero)."""
    assert ct[0] == 0
    out = []
    for c in range(len(ct) - 1):
        assert ct[c] <= ct[c + 1]
        bits = "".join(format(int(w), "032b") for w in words[ct[c]:ct[c + 1]])
        k = 0
        for _ in range(min(256, n - 256 * c)):
            cur = ""
            while cur not in codes:
                cur += bits[k]
                k += 1
            out.append(codes[cur])
        assert set(bits[k:]) <= {"0"} and len(bits) - k < 32
    assert len(out) == n
    return np.array(out, np.int64)


def ref_bytes(rows, window=0):
    """Bytes of one reference: a u8 distance in windowed segments, else the
    referenced row as u16 (segments up to 65536 rows) or u32."""
    return 1 if window else (2 if rows <= 65536 else 4)


def huff_size(q, o, n, U, D, rows, lengths, window=0):
    """Bytes of a tile's Huffman record for the codes q (outliers o) of its U
    first-occurrence rows."""
    sym = np.asarray(q, np.int64).reshape(-1) + 2047
    nE = U * D
    words = sum((int(lengths[sym[c:c + 256]].sum()) + 31) // 32 for c in range(0, nE, 256))
    n_out = int(np.asarray(o).sum())
    rb = ref_bytes(rows, window)
    oop = _a(16 + rb * (n - U), 4)
    return _a(oop + 8 * n_out + 4 * ((nE + 255) // 256 + 1) + 4 * words, 16)


def bitpack_size(raw, bitmap, n, D, eb, rows, window=0):
    """Bytes the BITPACK record of a tile would take, rebuilt from its raw rows
    (n x D), its first-occurrence bitmap and the segment's eb."""
    us = [i for i in range(n) if (bitmap >> i) & 1]
    q, o = quantize_np(raw[us].reshape(-1), eb)
    z = np.where(q >= 0, 2 * q, -2 * q - 1)
    nE = len(us) * D
    nblk = (nE + 63) // 64
    zb = np.zeros(nblk * 64, np.int64)
    zb[:nE] = z
    m = zb.reshape(nblk, 64).max(axis=1) if nblk else np.zeros(0, np.int64)
    sw = int(sum(int(v).bit_length() for v in m))
    n_out = int(o.sum())
    rb = ref_bytes(rows, window)
    orf = _a(16 + nblk, 4)
    oop = _a(orf + rb * (n - len(us)), 4)
    opl = _a(oop + 8 * n_out, 8)
    return _a(opl + 8 * sw, 16)


def quantize_np(x, eb):
    """fp32 quantizer written for the tests: q = rint(x / 2eb) unless out of range
    or the reconstruction misses eb (then an outlier with code 0)."""
    x = np.asarray(x, np.float32)
    eb = np.float32(eb)
    s = eb + eb
    with np.errstate(all="ignore"):
        t = x / s
        out = ~(np.abs(t) <= np.float32(2047))
        qf = np.rint(np.where(out, np.float32(0), t)).astype(np.float32)
        xh = qf * s
        out |= ~(np.abs(x - xh) <= eb)
    return np.where(out, 0, qf).astype(np.int64), out


def decode(st: Stream, buf: np.ndarray):
    """Rebuild codes, outlier flags, first-occurrence maps and values."""
    buf = np.asarray(buf, dtype=np.uint8)
    T, B, D, P = st.T, st.B, st.D, st.P
    y = np.zeros((T, B, D), np.float32)
    codes = np.zeros((T, B, D), np.int64)
    outl = np.zeros((T, B, D), bool)
    first = np.zeros((T, B), np.int64)
    for seg in st.segments:
        r0 = seg.p * B // P
        eb = np.float32(seg.eb)
        s = eb + eb
        keyrow = {}   # segment row -> (codes, outlier flags, values) of its key
        rawrow = {}   # segment row -> raw values (RAW tiles)
        for k, tl in enumerate(seg.tiles):
            if tl.mode == 0:
                raw = np.frombuffer(bytes(buf[tl.offset + 16:tl.offset + 16 + 4 * tl.n * D]),
                                    np.float32).reshape(tl.n, D)
                for i in range(tl.n):
                    rawrow[64 * k + i] = raw[i]
                    if seg.valid:
                        q, o = quantize_np(raw[i], eb)
                        vals = np.where(o, raw[i], q.astype(np.float32) * s).astype(np.float32)
                        keyrow[64 * k + i] = (q, o, vals)
            else:
                us = [i for i in range(tl.n) if (tl.bitmap >> i) & 1]
                q = unzigzag(tl.zz).reshape(len(us), D)
                o = np.zeros(len(us) * D, bool)
                o[tl.opos] = True
                o = o.reshape(len(us), D)
                raw = np.zeros(len(us) * D, np.uint32)
                raw[tl.opos] = tl.oval
                raw = raw.reshape(len(us), D).view(np.float32)
                for u, i in enumerate(us):
                    vals = np.where(o[u], raw[u], q[u].astype(np.float32) * s)
                    keyrow[64 * k + i] = (q[u], o[u], vals.astype(np.float32))
        for k, tl in enumerate(seg.tiles):
            j = 0
            for i in range(tl.n):
                r = 64 * k + i
                if tl.mode == 0:
                    y[seg.t, r0 + r] = rawrow[r]
                    if seg.valid:
                        first[seg.t, r0 + r] = r if (tl.bitmap >> i) & 1 else -1
                        codes[seg.t, r0 + r], outl[seg.t, r0 + r], _ = keyrow[r]
                    else:
                        first[seg.t, r0 + r] = r
                    continue
                if (tl.bitmap >> i) & 1:
                    first[seg.t, r0 + r] = r
                    qq, oo, vv = keyrow[r]
                else:
                    ref = int(tl.refs[j])
                    j += 1
                    if seg.window:  # a distance back to the nearest row with the key
                        assert 1 <= ref <= min(seg.window, r), "distance out of the window"
                        ref = r - ref
                        qq, oo, vv = keyrow[ref]
                        keyrow[r] = (qq, oo, vv)
                    else:
                        assert ref < r, "reference to a later row"
                        qq, oo, vv = keyrow[ref]
                    first[seg.t, r0 + r] = ref
                codes[seg.t, r0 + r] = qq
                outl[seg.t, r0 + r] = oo
                y[seg.t, r0 + r] = vv
    return codes, outl, first, y


def parse_segments(buf: np.ndarray):
    """Segment headers only (no tile walk): list of Segment without tiles."""
    buf = np.asarray(buf, dtype=np.uint8)
    assert _u(buf, 0, 4) == 0x434C4245
    T, B, D, P = (_u(buf, o, 4) for o in (8, 12, 16, 20))
    chunk_bytes = [_u(buf, 64 + 8 * p, 8) for p in range(P)]
    at = 64 + _a(8 * P, 16)
    segs = []
    for p in range(P):
        c0 = at
        for t in range(T):
            s0 = c0 + _u(buf, c0 + 8 * t, 8)
            segs.append(Segment(p, t, s0, _u(buf, s0, 4), _u(buf, s0 + 4, 4),
                                float(np.frombuffer(bytes(buf[s0 + 8:s0 + 12]), np.float32)[0]),
                                bool(_u(buf, s0 + 12, 4) & 1), _u(buf, s0 + 16, 4),
                                _u(buf, s0 + 20, 4), _u(buf, s0 + 24, 8)))
        at += chunk_bytes[p]
    assert at == _u(buf, 48, 8)
    return segs


def _tile_codes(seg, tl, buf, D):
    """Codes and outlier flags of a tile's first-occurrence rows (U x D)."""
    if tl.mode == 0:
        raw = np.frombuffer(bytes(buf[tl.offset + 16:tl.offset + 16 + 4 * tl.n * D]),
                            np.float32).reshape(tl.n, D)
        us = [i for i in range(tl.n) if (tl.bitmap >> i) & 1]
        q, o = quantize_np(raw[us].reshape(-1), seg.eb)
        return q, o
    q = unzigzag(tl.zz)
    o = np.zeros(tl.U * D, bool)
    o[tl.opos] = True
    return q, o


def _bitpack_tile_size(q, o, n, U, D, rows, window=0):
    z = np.where(q >= 0, 2 * q, -2 * q - 1)
    nE = U * D
    nblk = (nE + 63) // 64
    zb = np.zeros(nblk * 64, np.int64)
    zb[:nE] = z
    sw = sum(int(v).bit_length() for v in (zb.reshape(nblk, 64).max(axis=1) if nblk else []))
    rb = ref_bytes(rows, window)
    orf = _a(16 + nblk, 4)
    oop = _a(orf + rb * (n - U), 4)
    return _a(_a(oop + 8 * int(o.sum()), 8) + 8 * sw, 16)


def segment_form_sizes(seg, buf, D, lengths_of_hist):
    """(bit-plane form bytes, Huffman form bytes, Huffman lengths) of a valid
    segment, rebuilt from its codes; lengths_of_hist(freq[4095]) is the
    Huffman construction (pinned on its own)."""
    tiles = [(tl, *_tile_codes(seg, tl, buf, D)) for tl in seg.tiles]
    freq = np.zeros(4095, np.uint64)
    for tl, q, o in tiles:
        freq += np.bincount(q + 2047, minlength=4095).astype(np.uint64)
    lengths = np.asarray(lengths_of_hist(freq), np.int64)
    used = np.nonzero(lengths)[0]
    book = 4 if used.size == 0 else 4 + (int(used[-1]) - int(used[0]) + 2) // 2
    pre = 32 + _a(4 * seg.ntiles, 16)
    bp, hf = pre, pre + _a(book, 16)
    for tl, q, o in tiles:
        raw = 16 + _a(4 * tl.n * D, 16)
        b = _bitpack_tile_size(q, o, tl.n, tl.U, D, seg.rows, seg.window)
        h = huff_size(q, o, tl.n, tl.U, D, seg.rows, lengths, seg.window)
        bp += b if b < raw else raw
        hf += h if h < raw else raw
    return bp, hf, lengths


def check_coder_choice(st, buf, lengths_of_hist, table_coder=None):
    """Every segment has the size of the form its coder rules pick: coder 1
    bit planes, coder 2 Huffman for valid segments, coder 3 Huffman iff
    strictly smaller (the stream's coder, or table_coder[t] per table); a
    Huffman segment's codebook is the histogram's."""
    picked = []
    if table_coder is not None:
        tc = list(table_coder)
        assert st.coder == (1 if all(c == 1 for c in tc) else 2 if all(c == 2 for c in tc) else 3)
    for seg in st.segments:
        if not seg.valid:
            assert not seg.huff
            continue
        bp, hf, lengths = segment_form_sizes(seg, buf, st.D, lengths_of_hist)
        coder = st.coder if table_coder is None else table_coder[seg.t]
        want_huff = {1: False, 2: True, 3: hf < bp}[coder]
        assert seg.huff == want_huff, (seg.p, seg.t, bp, hf)
        assert seg.nbytes == (hf if seg.huff else bp), (seg.p, seg.t, seg.nbytes, bp, hf)
        if seg.huff:
            assert np.array_equal(seg.lengths, lengths)
        picked.append((seg.t, seg.huff, bp, hf))
    return picked
