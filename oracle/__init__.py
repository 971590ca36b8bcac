"""ctypes wrapper of the CPU oracle (``ebl_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use this module; the library and its Python
binding never import it.  The oracle is single-threaded plain C that follows
arXiv 2407.04272 (quantization encoder of section III-D, vector
homogenization of section III-B, Algorithm 1's error-bound policy) and this
project's stream layout, documented in ``ebl_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libebl_oracle.so")
SOURCES = [os.path.join(HERE, "ebl_oracle.c"), os.path.join(HERE, "ebl_huffman.c")]

EB_ABS, EB_REL = 0, 1
SCHED_NONE, SCHED_INV_SQRT, SCHED_STEP = 0, 1, 2
OK, ERR_INVALID, ERR_CAPACITY, ERR_CORRUPT, ERR_OOM = 0, 1, 2, 3, 5
CODER_BITPACK, CODER_HUFFMAN, CODER_AUTO = 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE fp32, no contraction, no fast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-o", LIB_PATH, *SOURCES, "-lm"]
    subprocess.run(cmd, check=True, cwd=HERE)
    return LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_uint32), ("B", ctypes.c_uint32), ("D", ctypes.c_uint32),
        ("P", ctypes.c_uint32), ("eb_mode", ctypes.c_uint32),
        ("eb", ctypes.POINTER(ctypes.c_float)),
        ("table_mult", ctypes.POINTER(ctypes.c_float)),
        ("sched_kind", ctypes.c_int32), ("sched_steps", ctypes.c_int32),
        ("sched_t0", ctypes.c_double), ("sched_k", ctypes.c_double),
        ("sched_phase", ctypes.c_int64), ("coder", ctypes.c_uint32),
        ("table_coder", ctypes.POINTER(ctypes.c_int32)), ("window", ctypes.c_uint32),
        ("book_len", ctypes.c_void_p), ("book_have", ctypes.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        f32p = ctypes.POINTER(ctypes.c_float)
        cfgp = ctypes.POINTER(_Cfg)
        L.ebo_schedule.restype = ctypes.c_double
        L.ebo_schedule.argtypes = [cfgp, ctypes.c_int64]
        L.ebo_table_factor.restype = ctypes.c_float
        L.ebo_table_factor.argtypes = [cfgp, ctypes.c_uint32, ctypes.c_int64]
        L.ebo_range.restype = None
        L.ebo_range.argtypes = [f32p, ctypes.c_size_t, f32p, f32p]
        L.ebo_eb_valid.restype = ctypes.c_int
        L.ebo_eb_valid.argtypes = [ctypes.c_float]
        L.ebo_quantize.restype = ctypes.c_int
        L.ebo_quantize.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_int32)]
        L.ebo_dequantize.restype = ctypes.c_float
        L.ebo_dequantize.argtypes = [ctypes.c_int32, ctypes.c_float]
        L.ebo_zigzag.restype = ctypes.c_uint32
        L.ebo_zigzag.argtypes = [ctypes.c_int32]
        L.ebo_unzigzag.restype = ctypes.c_int32
        L.ebo_unzigzag.argtypes = [ctypes.c_uint32]
        L.ebo_homo_index.restype = ctypes.c_double
        L.ebo_homo_index.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.ebo_homo_counts.restype = ctypes.c_int
        L.ebo_homo_counts.argtypes = [cfgp, ctypes.c_int64, f32p, ctypes.c_void_p, ctypes.c_void_p]
        L.ebo_speedup.restype = ctypes.c_double
        L.ebo_speedup.argtypes = [ctypes.c_double] * 4
        L.ebo_select.restype = ctypes.c_int
        L.ebo_select.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
        L.ebo_classify.restype = ctypes.c_int
        L.ebo_classify.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_double,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                   ctypes.c_void_p, ctypes.c_void_p]
        L.ebo_table_eb.restype = ctypes.c_float
        L.ebo_table_eb.argtypes = [cfgp, ctypes.c_uint32, ctypes.c_int64, f32p]
        L.ebo_max_compressed_bytes.restype = ctypes.c_size_t
        L.ebo_max_compressed_bytes.argtypes = [cfgp]
        L.ebo_compress.restype = ctypes.c_int
        L.ebo_compress.argtypes = [cfgp, ctypes.c_int64, f32p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.POINTER(ctypes.c_size_t), ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.ebo_decompress.restype = ctypes.c_int
        L.ebo_decompress.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32,
                                     ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, f32p]
        u8p, u16p, u32p = (ctypes.POINTER(t) for t in (ctypes.c_uint8, ctypes.c_uint16,
                                                        ctypes.c_uint32))
        L.ebo_huff_lengths.restype = ctypes.c_int
        L.ebo_huff_lengths.argtypes = [ctypes.POINTER(ctypes.c_uint64), u8p]
        L.ebo_huff_codes.restype = None
        L.ebo_huff_codes.argtypes = [u8p, u32p]
        L.ebo_huff_encode.restype = ctypes.c_size_t
        L.ebo_huff_encode.argtypes = [u16p, ctypes.c_size_t, u8p, u32p, u32p, u32p]
        L.ebo_huff_decode.restype = ctypes.c_int
        L.ebo_huff_decode.argtypes = [u32p, ctypes.c_size_t, u32p, ctypes.c_size_t, u8p, u16p]
        L.ebo_huff_book_bytes.restype = ctypes.c_size_t
        L.ebo_huff_book_bytes.argtypes = [u8p]
        L.ebo_huff_book_write.restype = ctypes.c_size_t
        L.ebo_huff_book_write.argtypes = [u8p, u8p]
        L.ebo_huff_book_read.restype = ctypes.c_int
        L.ebo_huff_book_read.argtypes = [u8p, ctypes.c_size_t, u8p]
        _lib = L
    return _lib


def _f32ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


@dataclass
class Config:
    """Shape and error-bound policy of one compression problem."""
    T: int
    B: int
    D: int
    P: int = 1
    eb_mode: int = EB_ABS
    eb: tuple = (1e-4,)
    table_mult: tuple | None = None
    sched_kind: int = SCHED_NONE
    sched_t0: float = 1000.0
    sched_k: float = 2.0
    sched_phase: int = 1
    sched_steps: int = 1
    coder: int = CODER_BITPACK
    table_coder: tuple | None = None
    window: int = 0
    books: "BookState | None" = None  # codebook reuse across calls (state kept here)

    def _c(self):
        eb = np.ascontiguousarray(np.asarray(self.eb, dtype=np.float32).reshape(-1))
        if eb.size == 1 and self.T > 1:
            eb = np.full(self.T, eb[0], dtype=np.float32)
        mult = None
        if self.table_mult is not None:
            mult = np.ascontiguousarray(np.asarray(self.table_mult, dtype=np.float32))
        tc = None
        if self.table_coder is not None:
            tc = np.ascontiguousarray(np.asarray(self.table_coder, dtype=np.int32))
        c = _Cfg(self.T, self.B, self.D, self.P, self.eb_mode, _f32ptr(eb),
                 _f32ptr(mult) if mult is not None else ctypes.POINTER(ctypes.c_float)(),
                 self.sched_kind, self.sched_steps, self.sched_t0, self.sched_k,
                 self.sched_phase, self.coder,
                 tc.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if tc is not None
                 else ctypes.POINTER(ctypes.c_int32)(), self.window,
                 self.books.lengths.ctypes.data if self.books is not None else None,
                 self.books.have.ctypes.data if self.books is not None else None)
        return c, (eb, mult, tc)  # keep arrays alive with the struct


def schedule(cfg: Config, it: int) -> float:
    c, keep = cfg._c()
    return lib().ebo_schedule(ctypes.byref(c), it)


def table_factor(cfg: Config, t: int, it: int) -> float:
    c, keep = cfg._c()
    return lib().ebo_table_factor(ctypes.byref(c), t, it)


def table_eb(cfg: Config, t: int, it: int, x: np.ndarray) -> float:
    c, keep = cfg._c()
    x = np.ascontiguousarray(x, dtype=np.float32)
    return lib().ebo_table_eb(ctypes.byref(c), t, it, _f32ptr(x))


def value_range(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    lo, hi = ctypes.c_float(), ctypes.c_float()
    lib().ebo_range(_f32ptr(x), x.size, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def eb_valid(eb: float) -> bool:
    return bool(lib().ebo_eb_valid(eb))


def quantize(x: float, eb: float):
    q = ctypes.c_int32()
    o = lib().ebo_quantize(x, eb, ctypes.byref(q))
    return q.value, bool(o)


def dequantize(q: int, eb: float) -> float:
    return lib().ebo_dequantize(q, eb)


def zigzag(q: int) -> int:
    return lib().ebo_zigzag(q)


def unzigzag(z: int) -> int:
    return lib().ebo_unzigzag(z)


def homo_index(n_original: int, n_compressed: int) -> float:
    return lib().ebo_homo_index(n_original, n_compressed)


def homo_counts(cfg: Config, it: int, x: np.ndarray):
    """(n_orig, n_quant) per segment p*T + t: eq. (1)'s distinct original and
    distinct quantized rows."""
    c, keep = cfg._c()
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(cfg.T, cfg.B, cfg.D)
    no = np.zeros(cfg.P * cfg.T, np.uint32)
    nq = np.zeros(cfg.P * cfg.T, np.uint32)
    rc = lib().ebo_homo_counts(ctypes.byref(c), it, _f32ptr(x), no.ctypes.data, nq.ctypes.data)
    if rc != OK:
        raise RuntimeError(f"oracle homo_counts failed with status {rc}")
    return no, nq


def speedup(cr: float, bw: float, tc: float, td: float) -> float:
    """Eq. (2)."""
    return lib().ebo_speedup(cr, bw, tc, td)


def select(cr, tc, td, bw: float):
    """Algorithm 2: per table, the index of the compressor with the largest
    eq. (2) speed-up.  cr [ncomp][T], tc / td [ncomp].  (best, speed-ups)."""
    cr = np.ascontiguousarray(cr, dtype=np.float64)
    ncomp, T = cr.shape
    tc = np.ascontiguousarray(tc, dtype=np.float64)
    td = np.ascontiguousarray(td, dtype=np.float64)
    best = np.zeros(T, np.int32)
    sp = np.zeros(T, np.float64)
    rc = lib().ebo_select(T, ncomp, cr.ctypes.data, tc.ctypes.data, td.ctypes.data, bw,
                          best.ctypes.data, sp.ctypes.data)
    if rc != 0:
        raise ValueError("invalid compressor pool")
    return best, sp


def classify(hindex, l_thresh: float, s_thresh: float, alpha: float, beta: float):
    """Algorithm 1's table classes (0 large, 1 medium, 2 small) and eb multipliers."""
    h = np.ascontiguousarray(hindex, dtype=np.float64)
    cls = np.zeros(h.size, np.int32)
    mult = np.zeros(h.size, np.float32)
    rc = lib().ebo_classify(h.size, h.ctypes.data, l_thresh, s_thresh, alpha, beta,
                            cls.ctypes.data, mult.ctypes.data)
    if rc != 0:
        raise ValueError("invalid classification thresholds or multipliers")
    return cls, mult


def max_compressed_bytes(cfg: Config) -> int:
    c, keep = cfg._c()
    return lib().ebo_max_compressed_bytes(ctypes.byref(c))


class BookState:
    """The codes kept between calls for codebook reuse: lengths [P*T][4095]
    and a have flag per segment, updated by every compress call."""

    def __init__(self, cfg):
        self.lengths = np.zeros((cfg.P * cfg.T, 4095), np.uint8)
        self.have = np.zeros(cfg.P * cfg.T, np.uint8)

    def copy(self):
        c = BookState.__new__(BookState)
        c.lengths, c.have = self.lengths.copy(), self.have.copy()
        return c


@dataclass
class Compressed:
    stream: np.ndarray          # uint8 bytes of the stream
    codes: np.ndarray | None    # int32 [T,B,D]
    outlier: np.ndarray | None  # uint8 [T,B,D]
    first: np.ndarray | None    # uint32 [T,B]
    eb: np.ndarray | None       # float32 [P*T]


def compress(cfg: Config, it: int, x: np.ndarray, debug: bool = True) -> Compressed:
    c, keep = cfg._c()
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(cfg.T, cfg.B, cfg.D)
    cap = max_compressed_bytes(cfg)
    if cap == 0:
        raise ValueError("invalid configuration")
    out = np.zeros(cap, dtype=np.uint8)
    n = ctypes.c_size_t()
    codes = np.zeros((cfg.T, cfg.B, cfg.D), np.int32) if debug else None
    outl = np.zeros((cfg.T, cfg.B, cfg.D), np.uint8) if debug else None
    first = np.zeros((cfg.T, cfg.B), np.uint32) if debug else None
    ebs = np.zeros(cfg.P * cfg.T, np.float32) if debug else None

    def p(a):
        return a.ctypes.data if a is not None else None

    rc = lib().ebo_compress(ctypes.byref(c), it, _f32ptr(x), out.ctypes.data, cap,
                            ctypes.byref(n), p(codes), p(outl), p(first), p(ebs))
    if rc != OK:
        raise RuntimeError(f"oracle compress failed with status {rc}")
    return Compressed(out[: n.value].copy(), codes, outl, first, ebs)


def decompress(cfg: Config, stream: np.ndarray, status: bool = False):
    s = np.ascontiguousarray(stream, dtype=np.uint8)
    y = np.zeros((cfg.T, cfg.B, cfg.D), np.float32)
    rc = lib().ebo_decompress(s.ctypes.data, s.size, cfg.T, cfg.B, cfg.D, cfg.P, _f32ptr(y))
    if status:
        return rc, y
    if rc != OK:
        raise RuntimeError(f"oracle decompress failed with status {rc}")
    return y


# --- canonical Huffman coder (ebl_huffman.c) -------------------------------
HUFF_NSYM, HUFF_MAXLEN, HUFF_CHUNK = 4095, 12, 256


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(ctypes.POINTER(t))


def huff_lengths(freq) -> np.ndarray:
    """Code lengths (uint8 [4095], 0 = unused) from symbol frequencies."""
    f = np.zeros(HUFF_NSYM, np.uint64)
    fr = np.asarray(freq, dtype=np.uint64).reshape(-1)
    f[: fr.size] = fr
    ln = np.zeros(HUFF_NSYM, np.uint8)
    lib().ebo_huff_lengths(_p(f, ctypes.c_uint64), _p(ln, ctypes.c_uint8))
    return ln


def huff_codes(lengths) -> np.ndarray:
    ln = np.zeros(HUFF_NSYM, np.uint8)
    l = np.asarray(lengths, dtype=np.uint8).reshape(-1)
    ln[: l.size] = l
    code = np.zeros(HUFF_NSYM, np.uint32)
    lib().ebo_huff_codes(_p(ln, ctypes.c_uint8), _p(code, ctypes.c_uint32))
    return code


def huff_encode(sym, lengths):
    """Encode uint16 symbols; returns (words uint32, chunk offsets uint32)."""
    s = np.ascontiguousarray(sym, dtype=np.uint16).reshape(-1)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    code = huff_codes(ln)
    n = s.size
    nch = (n + HUFF_CHUNK - 1) // HUFF_CHUNK
    words = np.zeros(HUFF_MAXLEN * n // 32 + nch + 1, np.uint32)
    off = np.zeros(nch + 1, np.uint32)
    nw = lib().ebo_huff_encode(_p(s, ctypes.c_uint16), n, _p(ln, ctypes.c_uint8),
                               _p(code, ctypes.c_uint32), _p(words, ctypes.c_uint32),
                               _p(off, ctypes.c_uint32))
    return words[:nw].copy(), off


def huff_decode(words, chunk_off, n, lengths, status: bool = False):
    w = np.ascontiguousarray(words, dtype=np.uint32)
    o = np.ascontiguousarray(chunk_off, dtype=np.uint32)
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    assert o.size == (n + HUFF_CHUNK - 1) // HUFF_CHUNK + 1
    out = np.zeros(n, np.uint16)
    w1 = w if w.size else np.zeros(1, np.uint32)
    rc = lib().ebo_huff_decode(_p(w1, ctypes.c_uint32), w.size, _p(o, ctypes.c_uint32), n,
                               _p(ln, ctypes.c_uint8), _p(out, ctypes.c_uint16))
    if status:
        return rc, out
    if rc != 0:
        raise RuntimeError("oracle Huffman decode: malformed chunk")
    return out


def huff_book_write(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    out = np.zeros(lib().ebo_huff_book_bytes(_p(ln, ctypes.c_uint8)), np.uint8)
    lib().ebo_huff_book_write(_p(ln, ctypes.c_uint8), _p(out, ctypes.c_uint8))
    return out


def huff_book_read(book):
    b = np.ascontiguousarray(book, dtype=np.uint8)
    b1 = b if b.size else np.zeros(1, np.uint8)
    ln = np.zeros(HUFF_NSYM, np.uint8)
    rc = lib().ebo_huff_book_read(_p(b1, ctypes.c_uint8), b.size, _p(ln, ctypes.c_uint8))
    return rc, ln
