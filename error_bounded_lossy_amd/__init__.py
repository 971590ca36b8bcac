"""Python binding of libec.so, the gfx950 error-bounded lossy compressor for
DLRM embedding traffic (arXiv 2407.04272).

This module only marshals arguments for the C ABI declared in include/ec.h:
torch supplies device memory and streams, and every step of compression and
decompression runs in the library's HIP kernels.  There is no fallback: if
libec.so cannot be loaded, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libec.so")
HEADERS = [os.path.join(ROOT, "include", h) for h in ("ec.h", "ec_huffman.h")]

EC_OK, EC_ERR_INVALID, EC_ERR_CAPACITY, EC_ERR_CORRUPT = 0, 1, 2, 3
EC_ERR_DEVICE, EC_ERR_OOM, EC_ERR_UNSUPPORTED = 4, 5, 6
EB_ABS, EB_REL_RANGE = 0, 1
SCHED_NONE, SCHED_INV_SQRT, SCHED_STEP = 0, 1, 2
CODER_BITPACK, CODER_HUFFMAN, CODER_AUTO = 1, 2, 3
KERNEL_PREP, KERNEL_ENCODE, KERNEL_DECODE, KERNEL_ASSEMBLE = 0, 1, 2, 3
ABI_VERSION = 2


class ECError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class _Schedule(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("steps", ctypes.c_int32), ("t0", ctypes.c_double),
                ("k", ctypes.c_double), ("phase", ctypes.c_int64)]


class _Desc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32), ("num_tables", ctypes.c_uint32),
        ("rows", ctypes.c_uint32), ("dim", ctypes.c_uint32), ("num_chunks", ctypes.c_uint32),
        ("eb_mode", ctypes.c_int32), ("eb", ctypes.POINTER(ctypes.c_float)),
        ("table_mult", ctypes.POINTER(ctypes.c_float)), ("sched", _Schedule),
        ("coder", ctypes.c_int32), ("debug_hash_bits", ctypes.c_uint32),
        ("d_workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("window", ctypes.c_uint32), ("reuse_books", ctypes.c_uint32),
        ("table_coder", ctypes.POINTER(ctypes.c_int32)),
    ]


_lib = None


def lib():
    """Load libec.so (raises if it is missing: there is no CPU fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with error_bounded_lossy_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(_Desc)
    L.ec_max_dim.restype = ctypes.c_uint32
    L.ec_max_dim.argtypes = []
    L.ec_workspace_bytes.restype = sz
    L.ec_workspace_bytes.argtypes = [dp]
    L.ec_plan.restype = st
    L.ec_plan.argtypes = [dp, ctypes.POINTER(vp)]
    L.ec_plan_destroy.restype = st
    L.ec_plan_destroy.argtypes = [vp]
    L.ec_max_compressed_bytes.restype = sz
    L.ec_max_compressed_bytes.argtypes = [vp]
    L.ec_compress.restype = st
    L.ec_compress.argtypes = [vp, ctypes.c_int64, vp, vp, sz, vp]
    L.ec_compress_static.restype = st
    L.ec_compress_static.argtypes = [vp, ctypes.c_int64, vp, vp, sz, vp]
    u32p = ctypes.POINTER(ctypes.c_uint32)
    L.ec_homo_counts.restype = st
    L.ec_homo_counts.argtypes = [vp, ctypes.c_int64, vp, vp, sz, u32p, u32p, vp]
    L.ec_classify_tables.restype = st
    L.ec_classify_tables.argtypes = [ctypes.c_uint32, ctypes.POINTER(ctypes.c_double),
                                     ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_double, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(ctypes.c_float)]
    dblp = ctypes.POINTER(ctypes.c_double)
    L.ec_speedup.restype = ctypes.c_double
    L.ec_speedup.argtypes = [ctypes.c_double] * 4
    L.ec_select_coders.restype = st
    L.ec_select_coders.argtypes = [ctypes.c_uint32, ctypes.c_uint32, dblp, dblp, dblp,
                                   ctypes.c_double, ctypes.POINTER(ctypes.c_int32), dblp]
    L.ec_decompress.restype = st
    L.ec_decompress.argtypes = [vp, vp, sz, vp, vp]
    L.ec_ratio.restype = st
    L.ec_ratio.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64),
                           ctypes.POINTER(ctypes.c_double)]
    L.ec_status_string.restype = ctypes.c_char_p
    L.ec_status_string.argtypes = [st]
    L.ec_debug_attach.restype = st
    L.ec_debug_attach.argtypes = [vp, vp, vp, vp, vp]
    L.ec_profile_enable.restype = st
    L.ec_profile_enable.argtypes = [vp, st, ctypes.c_uint32]
    L.ec_profile_read.restype = st
    L.ec_profile_read.argtypes = [vp, st, ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_uint64)]
    u64 = ctypes.c_uint64
    L.ec_huff_workspace_bytes.restype = sz
    L.ec_huff_workspace_bytes.argtypes = []
    L.ec_huff_max_words.restype = u64
    L.ec_huff_max_words.argtypes = [u64]
    L.ec_huff_encode.restype = st
    L.ec_huff_encode.argtypes = [vp, u64, vp, vp, vp, u64, vp, sz, vp]
    L.ec_huff_decode.restype = st
    L.ec_huff_decode.argtypes = [vp, u64, vp, vp, u64, u64, vp, vp, sz, vp]
    L.ec_huff_status.restype = st
    L.ec_huff_status.argtypes = [vp, vp]
    L.ec_huff_workspace_bytes_segments.restype = sz
    L.ec_huff_workspace_bytes_segments.argtypes = [ctypes.c_uint32]
    L.ec_huff_encode_segments.restype = st
    L.ec_huff_encode_segments.argtypes = [vp, ctypes.c_uint32, u64, vp, vp, vp, u64, vp, sz, vp]
    L.ec_huff_decode_segments.restype = st
    L.ec_huff_decode_segments.argtypes = [vp, vp, vp, u64, ctypes.c_uint32, u64, vp, vp, sz, vp]
    _lib = L
    return L


def declared_functions() -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in HEADERS:
        with open(h) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(ec_[a-z_]+)\s*\(", text))
    return sorted(names)


def status_string(status: int) -> str:
    try:
        return lib().ec_status_string(status).decode()
    except ImportError:
        return "status"


def _check(status: int, what: str):
    if status != EC_OK:
        raise ECError(status, what)


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _desc(T, B, D, P, eb_mode, eb, table_mult, schedule, debug_hash_bits, keep,
          coder=CODER_BITPACK, table_coder=None, window=0, reuse_books=False):
    ebs = [float(v) for v in (eb if hasattr(eb, "__len__") else [eb])]
    if len(ebs) == 1 and T > 1:
        ebs = ebs * T
    arr = (ctypes.c_float * len(ebs))(*ebs)
    keep.append(arr)
    mult = ctypes.POINTER(ctypes.c_float)()
    if table_mult is not None:
        m = (ctypes.c_float * len(table_mult))(*[float(v) for v in table_mult])
        keep.append(m)
        mult = ctypes.cast(m, ctypes.POINTER(ctypes.c_float))
    sch = schedule or {}
    s = _Schedule(int(sch.get("kind", SCHED_NONE)), int(sch.get("steps", 1)),
                  float(sch.get("t0", 1000.0)), float(sch.get("k", 2.0)),
                  int(sch.get("phase", 1)))
    tc = ctypes.POINTER(ctypes.c_int32)()
    if table_coder is not None:
        c = (ctypes.c_int32 * max(len(table_coder), 1))(*[int(v) for v in table_coder])
        keep.append(c)
        tc = ctypes.cast(c, ctypes.POINTER(ctypes.c_int32))
    return _Desc(ABI_VERSION, T, B, D, P, int(eb_mode), ctypes.cast(arr, ctypes.POINTER(ctypes.c_float)),
                 mult, s, int(coder), int(debug_hash_bits), None, 0, int(window),
                 1 if reuse_books else 0, tc)


def workspace_bytes(T, B, D, P=1, eb_mode=EB_ABS, eb=1e-4, table_mult=None, schedule=None,
                    debug_hash_bits=0, coder=CODER_BITPACK, table_coder=None, window=0) -> int:
    keep = []
    d = _desc(T, B, D, P, eb_mode, eb, table_mult, schedule, debug_hash_bits, keep, coder,
              table_coder, window)
    return int(lib().ec_workspace_bytes(ctypes.byref(d)))


class Plan:
    """A compression plan: shape, error-bound policy and a torch-allocated workspace.

    schedule: None, {"kind": SCHED_INV_SQRT, "t0": 1000.0} or
              {"kind": SCHED_STEP, "k": 2.0, "phase": 100, "steps": 4}.
    """

    def __init__(self, T: int, B: int, D: int, P: int = 1, eb_mode: int = EB_ABS, eb=1e-4,
                 table_mult=None, schedule=None, debug_hash_bits: int = 0, device=None,
                 workspace: bool = True, coder: int = CODER_BITPACK, table_coder=None,
                 window: int = 0, reuse_books: bool = False):
        """workspace=False builds a plan without a workspace: compress with
        compress_static (the library's static device scratch), decompress as
        usual.  coder: CODER_BITPACK, CODER_HUFFMAN or CODER_AUTO;
        table_coder: one of them per table (Algorithm 2), overriding coder;
        window: 0, or 1..255 for windowed references (section III-E);
        reuse_books: Huffman segments keep their code across calls while it
        covers their symbols."""
        import torch
        self.T, self.B, self.D, self.P = T, B, D, P
        self.coder = coder
        self._keep = []
        self._desc = _desc(T, B, D, P, eb_mode, eb, table_mult, schedule, debug_hash_bits,
                           self._keep, coder, table_coder, window, reuse_books)
        L = lib()
        nbytes = int(L.ec_workspace_bytes(ctypes.byref(self._desc)))
        if nbytes == 0:
            raise ECError(EC_ERR_INVALID, "ec_workspace_bytes")
        self.workspace_bytes = nbytes
        self.device = torch.device(device or "cuda")
        self.workspace = None
        if workspace:
            self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
            base = self.workspace.data_ptr()
            aligned = (base + 255) // 256 * 256
            self._desc.d_workspace = aligned
            self._desc.workspace_bytes = nbytes
        h = ctypes.c_void_p()
        _check(L.ec_plan(ctypes.byref(self._desc), ctypes.byref(h)), "ec_plan")
        self._h = h
        self.max_compressed_bytes = int(L.ec_max_compressed_bytes(h))

    def close(self):
        if getattr(self, "_h", None):
            lib().ec_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def empty_stream(self):
        import torch
        return torch.empty(self.max_compressed_bytes, dtype=torch.uint8, device=self.device)

    def compress(self, x, out, iteration: int = 0, stream=None):
        """Enqueue compression of fp32 x [T,B,D] into the uint8 tensor `out`."""
        import torch
        assert x.dtype == torch.float32 and x.is_contiguous() and x.numel() == self.T * self.B * self.D
        assert out.dtype == torch.uint8 and out.is_contiguous()
        _check(lib().ec_compress(self._h, int(iteration), x.data_ptr(), out.data_ptr(),
                                 out.numel(), _stream_handle(stream)), "ec_compress")

    def compress_static(self, x, out, iteration: int = 0, stream=None):
        """Enqueue compression like compress(), with the library's static
        device scratch instead of the plan's workspace (ec_compress_static)."""
        import torch
        assert x.dtype == torch.float32 and x.is_contiguous() and x.numel() == self.T * self.B * self.D
        assert out.dtype == torch.uint8 and out.is_contiguous()
        _check(lib().ec_compress_static(self._h, int(iteration), x.data_ptr(), out.data_ptr(),
                                        out.numel(), _stream_handle(stream)),
               "ec_compress_static")

    def homo_counts(self, x, out, iteration: int = 0, stream=None):
        """Compress x into out and return eq. (1)'s counts per segment p*T + t:
        (distinct raw rows, distinct quantized rows) as two lists (waits)."""
        import torch
        assert x.dtype == torch.float32 and x.is_contiguous() and x.numel() == self.T * self.B * self.D
        assert out.dtype == torch.uint8 and out.is_contiguous()
        n = self.P * self.T
        no = (ctypes.c_uint32 * n)()
        nq = (ctypes.c_uint32 * n)()
        _check(lib().ec_homo_counts(self._h, int(iteration), x.data_ptr(), out.data_ptr(),
                                    out.numel(), no, nq, _stream_handle(stream)),
               "ec_homo_counts")
        return list(no), list(nq)

    def decompress(self, stream_bytes, y, stream=None):
        """Enqueue decompression of the uint8 stream into fp32 y [T,B,D]."""
        import torch
        assert y.dtype == torch.float32 and y.is_contiguous() and y.numel() == self.T * self.B * self.D
        assert stream_bytes.dtype == torch.uint8 and stream_bytes.is_contiguous()
        _check(lib().ec_decompress(self._h, stream_bytes.data_ptr(), stream_bytes.numel(),
                                   y.data_ptr(), _stream_handle(stream)), "ec_decompress")

    def ratio(self, per_segment: bool = False, raise_on_error: bool = True):
        """Wait for the plan's work; return (total CR, stream bytes[, per-segment CR], status)."""
        cr = ctypes.c_double()
        nb = ctypes.c_uint64()
        per = (ctypes.c_double * (self.P * self.T))() if per_segment else None
        st = lib().ec_ratio(self._h, ctypes.byref(cr), ctypes.byref(nb),
                            ctypes.cast(per, ctypes.POINTER(ctypes.c_double)) if per else None)
        if raise_on_error:
            _check(st, "ec_ratio")
        out = (cr.value, int(nb.value))
        if per_segment:
            out = out + (list(per),)
        return out + (st,)

    def debug_attach(self, codes=None, outlier=None, first=None, eb=None):
        p = lambda t: t.data_ptr() if t is not None else None
        _check(lib().ec_debug_attach(self._h, p(codes), p(outlier), p(first), p(eb)),
               "ec_debug_attach")
        self._dbg = (codes, outlier, first, eb)

    def profile_enable(self, enable: bool = True, max_launches: int = 4096):
        _check(lib().ec_profile_enable(self._h, int(enable), int(max_launches)), "ec_profile_enable")

    def profile_read(self, kernel: int):
        ms = ctypes.c_double()
        n = ctypes.c_uint64()
        _check(lib().ec_profile_read(self._h, int(kernel), ctypes.byref(ms), ctypes.byref(n)),
               "ec_profile_read")
        return ms.value, int(n.value)


CLASS_LARGE, CLASS_MEDIUM, CLASS_SMALL = 0, 1, 2


def homo_index(n_orig: int, n_quant: int) -> float:
    """Eq. (1): (N_original - N_compressed) / N_original."""
    return (n_orig - n_quant) / n_orig if n_orig else 0.0


def classify_tables(homo_index_per_table, l_thresh: float, s_thresh: float, alpha: float,
                    beta: float):
    """Algorithm 1's table classes and eb multipliers (ec_classify_tables):
    returns (classes, multipliers) for ec_plan_desc.table_mult."""
    h = [float(v) for v in homo_index_per_table]
    T = len(h)
    hin = (ctypes.c_double * max(T, 1))(*h)
    cls = (ctypes.c_int32 * max(T, 1))()
    mult = (ctypes.c_float * max(T, 1))()
    _check(lib().ec_classify_tables(T, hin, float(l_thresh), float(s_thresh), float(alpha),
                                    float(beta), cls, mult), "ec_classify_tables")
    return list(cls)[:T], list(mult)[:T]


def speedup(cr: float, bw: float, tc: float, td: float) -> float:
    """Eq. (2): the communication speed-up 1 / (1/CR + B (1/Tc + 1/Td))."""
    return float(lib().ec_speedup(float(cr), float(bw), float(tc), float(td)))


def select_coders(cr, tc, td, bw: float):
    """Algorithm 2 (ec_select_coders): cr[c][t] the ratio of compressor c on
    table t, tc[c] / td[c] its throughputs; returns (best compressor per
    table, its eq. (2) speed-up)."""
    C = len(tc)
    T = len(cr[0]) if C else 0
    flat = [float(cr[c][t]) for c in range(C) for t in range(T)]
    a = (ctypes.c_double * max(len(flat), 1))(*flat)
    b = (ctypes.c_double * max(C, 1))(*[float(v) for v in tc])
    d = (ctypes.c_double * max(C, 1))(*[float(v) for v in td])
    best = (ctypes.c_int32 * max(T, 1))()
    sp = (ctypes.c_double * max(T, 1))()
    _check(lib().ec_select_coders(T, C, a, b, d, float(bw), best, sp), "ec_select_coders")
    return list(best)[:T], list(sp)[:T]


def offline_comp_config(x, bw: float, pool=(CODER_BITPACK, CODER_HUFFMAN), eb_mode: int = EB_ABS,
                        eb=1e-4, table_mult=None, schedule=None, iteration: int = 0,
                        reps: int = 5, stream=None):
    """Algorithm 2 (OfflineCompConfig) on a sample batch x [T,B,D] (fp32, on
    the GPU): every compressor of the pool compresses the sample; its
    per-table compression ratios and its compression / decompression
    throughputs (bytes of fp32 input per second, the mean of `reps` timed
    calls) enter eq. (2) with the link bandwidth bw (bytes per second), and
    each table takes the compressor with the largest speed-up.  Returns a
    dict with table_coder (ready for Plan(table_coder=...)), best (indices
    into pool), speedup, cr [c][t], tc [c] and td [c]."""
    import torch
    T, B, D = (int(v) for v in x.shape)
    if B < 1 or reps < 1 or not pool:
        raise ECError(EC_ERR_INVALID, "offline_comp_config")
    raw = 4.0 * T * B * D
    strm = stream or torch.cuda.current_stream()
    crs, tcs, tds = [], [], []
    for coder in pool:
        plan = Plan(T, B, D, 1, eb_mode, eb, table_mult=table_mult, schedule=schedule,
                    device=x.device, coder=coder)
        out = plan.empty_stream()
        y = torch.empty_like(x)
        plan.compress(x, out, iteration, stream=strm)
        _, nbytes, per, _ = plan.ratio(per_segment=True)
        plan.decompress(out[:nbytes], y, stream=strm)
        plan.ratio()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(strm)
        for _ in range(reps):
            plan.compress(x, out, iteration, stream=strm)
        ev[1].record(strm)
        for _ in range(reps):
            plan.decompress(out[:nbytes], y, stream=strm)
        ev[2].record(strm)
        plan.ratio()
        ev[2].synchronize()
        tc_s = ev[0].elapsed_time(ev[1]) / 1e3 / reps
        td_s = ev[1].elapsed_time(ev[2]) / 1e3 / reps
        crs.append(per)
        tcs.append(raw / tc_s)
        tds.append(raw / td_s)
        plan.close()
    best, sp = select_coders(crs, tcs, tds, bw)
    return {"table_coder": [int(pool[b]) for b in best], "best": best, "speedup": sp,
            "cr": crs, "tc": tcs, "td": tds}


# --- canonical Huffman coder (include/ec_huffman.h) ------------------------
HUFF_NSYM, HUFF_MAXLEN, HUFF_CHUNK, HUFF_BOOK_MAX = 4095, 12, 256, 2052


def huff_max_words(n: int) -> int:
    return int(lib().ec_huff_max_words(int(n)))


def huff_book_bytes(header4) -> int:
    """Codebook size from its first 4 bytes (u16 lowest, u16 highest symbol)."""
    b = [int(v) for v in header4[:4]]
    lo, hi = b[0] | b[1] << 8, b[2] | b[3] << 8
    return 4 if hi < lo else 4 + (hi - lo + 2) // 2


class Huffman:
    """Workspace holder for the Huffman coder on one device.

    nseg = 1 codes one array (ec_huff_encode / ec_huff_decode); nseg > 1 codes
    nseg equal segments with a codebook each (ec_huff_encode_segments /
    ec_huff_decode_segments).  Symbols travel as int16 tensors (bit patterns
    of the u16 symbols), words and chunk offsets as int32 tensors (bit
    patterns of u32), codebooks as uint8 tensors of nseg * HUFF_BOOK_MAX."""

    def __init__(self, device=None, nseg: int = 1):
        import torch
        self.device = torch.device(device or "cuda")
        self.nseg = int(nseg)
        nbytes = int(lib().ec_huff_workspace_bytes_segments(self.nseg))
        if nbytes == 0:
            raise ECError(EC_ERR_INVALID, "ec_huff_workspace_bytes_segments")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.workspace.data_ptr()
        self._work = (base + 255) // 256 * 256
        self._work_bytes = nbytes

    def buffers(self, n: int):
        """Codebooks, chunk table and words for n symbols in all (n = nseg * seg_len)."""
        import torch
        assert n % self.nseg == 0
        L = n // self.nseg
        nch = self.nseg * ((L + HUFF_CHUNK - 1) // HUFF_CHUNK)
        book = torch.zeros(self.nseg * HUFF_BOOK_MAX, dtype=torch.uint8, device=self.device)
        off = torch.zeros(nch + 1, dtype=torch.int32, device=self.device)
        words = torch.zeros(max(self.nseg * huff_max_words(L), 1), dtype=torch.int32,
                            device=self.device)
        return book, off, words

    def encode(self, sym, book, chunk_off, words, stream=None):
        """Enqueue encoding of the int16 tensor `sym` (symbols 0..4094)."""
        import torch
        assert sym.dtype == torch.int16 and sym.is_contiguous()
        n = sym.numel()
        assert n % self.nseg == 0
        L = n // self.nseg
        assert book.numel() >= self.nseg * HUFF_BOOK_MAX
        assert chunk_off.numel() >= self.nseg * ((L + 255) // 256) + 1
        args = (chunk_off.data_ptr(), words.data_ptr(), words.numel(), self._work,
                self._work_bytes, _stream_handle(stream))
        p = sym.data_ptr() if n else None
        if self.nseg == 1:
            _check(lib().ec_huff_encode(p, n, book.data_ptr(), *args), "ec_huff_encode")
        else:
            _check(lib().ec_huff_encode_segments(p, self.nseg, L, book.data_ptr(), *args),
                   "ec_huff_encode_segments")

    def decode(self, book, book_bytes: int, chunk_off, words, n: int, sym, stream=None):
        """Enqueue decoding of n symbols in all into the int16 tensor `sym`
        (book_bytes is used with nseg = 1; segments read HUFF_BOOK_MAX each)."""
        import torch
        assert sym.dtype == torch.int16 and sym.is_contiguous() and sym.numel() >= n
        assert n % self.nseg == 0
        w = words.data_ptr() if words.numel() else None
        p = sym.data_ptr() if n else None
        if self.nseg == 1:
            _check(lib().ec_huff_decode(book.data_ptr(), int(book_bytes), chunk_off.data_ptr(), w,
                                        words.numel(), n, p, self._work, self._work_bytes,
                                        _stream_handle(stream)), "ec_huff_decode")
        else:
            _check(lib().ec_huff_decode_segments(book.data_ptr(), chunk_off.data_ptr(), w,
                                                 words.numel(), self.nseg, n // self.nseg, p,
                                                 self._work, self._work_bytes,
                                                 _stream_handle(stream)),
                   "ec_huff_decode_segments")

    def status(self, stream=None) -> int:
        """Wait for the stream; status of the last call on this workspace."""
        return int(lib().ec_huff_status(self._work, _stream_handle(stream)))
