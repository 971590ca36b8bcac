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

    assert _u(buf, 0, 4) == 0x434C4245 and _u(buf, 4, 2) == 1 and _u(buf, 6, 2) == 1
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
            assert _u(buf, s0 + 12, 4) in (0, 1)
            assert seg.rows == rows and seg.ntiles == (rows + 63) // 64
            mark(s0, 32)
            mark(s0 + 32, 4 * seg.ntiles)
            rb = 2 if rows <= 65536 else 4
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
                        # the rule: BITPACK only when strictly smaller than RAW
                        raw = np.frombuffer(bytes(buf[ro + 16:ro + 16 + 4 * n * D]),
                                            np.float32).reshape(n, D)
                        assert bitpack_size(raw, tl.bitmap, n, D, seg.eb, rows) >= raw_size, \
                            "RAW tile whose BITPACK record would be smaller"
                else:
                    assert tl.mode == 1 and seg.valid
                    nE = tl.U * D
                    nblk = (nE + 63) // 64
                    tl.widths = buf[ro + 16:ro + 16 + nblk].copy()
                    mark(ro + 16, nblk)
                    orf = _a(16 + nblk, 4)
                    nd = n - tl.U
                    tl.refs = np.frombuffer(bytes(buf[ro + orf:ro + orf + rb * nd]),
                                            np.uint16 if rb == 2 else np.uint32).astype(np.int64)
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
    return Stream(T, B, D, P, eb_mode, it, total, chunk_bytes, segs, cov)


def bitpack_size(raw, bitmap, n, D, eb, rows):
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
    rb = 2 if rows <= 65536 else 4
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
                    assert ref < r, "reference to a later row"
                    first[seg.t, r0 + r] = ref
                    qq, oo, vv = keyrow[ref]
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
