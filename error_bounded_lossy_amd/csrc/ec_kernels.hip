// ec_kernels.hip -- gfx950 (CDNA4, wave64) kernels of the error-bounded lossy
// compressor for DLRM embedding traffic (arXiv 2407.04272).
//
//  prep    clears the per-call workspace and, for range-relative error
//          bounds, reduces every table's (min, max) over non-NaN values
//          (one coalesced 128-bit-load pass over the input).
//  encode  one workgroup per 64-row tile, in stream order taken from a ticket
//          counter: quantize (section III-D), hash the quantized rows into a
//          per-segment table to find each row's first occurrence (section
//          III-B "Vector Homogenization", the vector-based LZ of III-D), pack
//          the first-occurrence rows' codes as bit planes by wavefront ballot,
//          and place the tile record with a decoupled look-back prefix scan so
//          that every tile, table and chunk lands in ONE contiguous stream in a
//          single pass (section III-E "Buffer Optimization", Fig. 7).
//  decode  one workgroup per tile; each output row is written once.
//
// Quantization uses IEEE fp32 division and round-to-nearest-even; the build
// disables FP contraction so the reconstruction check is the exact fp32
// sequence div, rint, mul, sub.
#include "ec_internal.h"

namespace ec {
namespace {

constexpr int16_t kSent = (int16_t)0x8000;  // outlier marker in LDS codes
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ uint64_t align_up(uint64_t v, uint64_t a) {
  return (v + a - 1) / a * a;
}

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// Linear quantization of one value (section III-D): q = rint(x / 2eb); values
// whose code would leave [-2047, 2047] or whose fp32 reconstruction q*2eb
// misses eb are outliers (kept verbatim, code 0).
__device__ __forceinline__ bool quantize(float x, float eb, float s, int& q) {
  float t = x / s;
  if (!(fabsf(t) <= 2047.0f)) {
    q = 0;
    return true;
  }
  float qf = rintf(t);
  float xh = qf * s;
  float err = x - xh;
  if (!(fabsf(err) <= eb)) {
    q = 0;
    return true;
  }
  q = (int)qf;
  return false;
}

__device__ __forceinline__ int16_t code_of(float x, float eb, float s) {
  int q;
  return quantize(x, eb, s, q) ? kSent : (int16_t)q;
}

__device__ __forceinline__ uint32_t zigzag(int q) { return ((uint32_t)q << 1) ^ (uint32_t)(q >> 31); }
__device__ __forceinline__ int unzigzag(uint32_t z) { return (int)(z >> 1) ^ -(int)(z & 1u); }

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xbf58476d1ce4e5b9ull;
  z ^= z >> 27;
  z *= 0x94d049bb133111ebull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint64_t ld_acq64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_acq32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_rlx64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rel64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rel32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void report_error(Report* r, uint32_t code) {
  if (r) __hip_atomic_store(&r->status, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// segment s owning scheduled tile `ticket` (seg_tile_base is non-decreasing)
__device__ __forceinline__ uint32_t find_segment(const uint32_t* base, uint32_t nseg,
                                                 uint32_t ticket) {
  uint32_t lo = 0, hi = nseg;  // base[lo] <= ticket < base[hi]
  while (hi - lo > 1) {
    uint32_t mid = (lo + hi) >> 1;
    if (base[mid] <= ticket) lo = mid;
    else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ uint32_t chunk_row0(const Shape& sh, uint32_t p) {
  return (uint32_t)((uint64_t)p * sh.B / sh.P);
}

// Exclusive scan of a[0..n) in LDS by the whole workgroup; returns the total.
// n <= kThreads * 8.
__device__ uint32_t block_exclusive_scan(uint32_t* a, uint32_t n, uint32_t* s_part) {
  const uint32_t tid = threadIdx.x;
  const uint32_t per = (n + kThreads - 1) / kThreads;
  uint32_t beg = tid * per, end = min(n, beg + per);
  uint32_t local = 0;
  for (uint32_t i = beg; i < end; i++) local += a[i];
  // workgroup scan of the per-thread sums
  const uint32_t lane = tid & 63, wv = tid >> 6;
  uint32_t incl = local;
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t v = __shfl_up(incl, o);
    if (lane >= (uint32_t)o) incl += v;
  }
  if (lane == 63) s_part[wv] = incl;
  __syncthreads();
  uint32_t wbase = 0, total = 0;
  for (uint32_t j = 0; j < kThreads / 64; j++) {
    if (j < wv) wbase += s_part[j];
    total += s_part[j];
  }
  uint32_t run = wbase + incl - local;
  for (uint32_t i = beg; i < end; i++) {
    uint32_t v = a[i];
    a[i] = run;
    run += v;
  }
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// prep: clear the dynamic workspace; per-table (min, max) partials (REL)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) ec_prep_kernel(PrepArgs a) {
  const uint64_t gtid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = gtid; i < a.w.dyn_words; i += stride) a.w.dyn[i] = 0;
  if (!a.rel) return;

  __shared__ float s_lo[kThreads / 64], s_hi[kThreads / 64];
  const uint32_t nbr = a.w.nbr;
  const uint32_t t = blockIdx.x / nbr, j = blockIdx.x % nbr;
  const uint64_t nel = (uint64_t)a.sh.B * a.sh.D;
  const float* xt = a.x + (uint64_t)t * nel;
  uint64_t per = (nel + nbr - 1) / nbr;
  per = (per + 1023) / 1024 * 1024;
  uint64_t beg = (uint64_t)j * per, end = beg + per;
  if (end > nel) end = nel;
  float lo = INFINITY, hi = -INFINITY;
  if (beg < end) {
    if ((nel & 3) == 0) {
      const float4* x4 = reinterpret_cast<const float4*>(xt);
      for (uint64_t i = beg / 4 + threadIdx.x; i < end / 4; i += kThreads) {
        float4 v = x4[i];
        float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; c++) {
          if (e[c] < lo) lo = e[c];  // NaN compares false: skipped
          if (e[c] > hi) hi = e[c];
        }
      }
    } else {
      for (uint64_t i = beg + threadIdx.x; i < end; i += kThreads) {
        float v = xt[i];
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    float l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    s_lo[wv] = lo;
    s_hi[wv] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (uint32_t k = 1; k < kThreads / 64; k++) {
      lo = s_lo[k] < lo ? s_lo[k] : lo;
      hi = s_hi[k] > hi ? s_hi[k] : hi;
    }
    a.w.range_part[2 * ((uint64_t)t * nbr + j) + 0] = lo;
    a.w.range_part[2 * ((uint64_t)t * nbr + j) + 1] = hi;
  }
}

// ---------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------
struct EncShared {
  uint32_t ticket, seg, tile, n, rows, ntiles;
  float eb;
  int valid;
  uint64_t bitmap;
  uint32_t U, nblk, sumw, nout, mode, fin_seg, fin_all;
  uint64_t rec_size, rec_abs, item, excl;
  uint32_t off_refs, off_opos, off_oval, off_pl;
  uint32_t part[kThreads / 64];
};

// Compare segment row `cand` (re-quantized from the input) with tile row `i`
// (codes in LDS); the whole wave participates, the result is uniform.
__device__ bool rows_equal(const int16_t* s_codes, const float* xs, const float* xt,
                           uint32_t i, uint32_t cand, uint32_t D, float eb, float s2) {
  const uint32_t lane = threadIdx.x & 63;
  bool eq = true;
  for (uint32_t d = lane; d < D; d += 64) {
    int16_t c = s_codes[i * D + d];
    float xo = xs[(uint64_t)cand * D + d];
    int16_t co = code_of(xo, eb, s2);
    bool e;
    if (c == kSent) e = (co == kSent) && f2u(xo) == f2u(xt[(uint64_t)i * D + d]);
    else e = (co == c);
    eq = eq && e;
  }
  return __all(eq);
}

__global__ void __launch_bounds__(kThreads) ec_encode_kernel(EncArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ EncShared sh;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t D = a.sh.D, T = a.sh.T;

  // LDS carve-up (matches encode_lds_bytes)
  int16_t* s_codes = reinterpret_cast<int16_t*>(smem);
  uint8_t* p = smem + ((size_t)2 * kTileRows * D + 15) / 16 * 16;
  uint64_t* s_hash = reinterpret_cast<uint64_t*>(p);
  p += kTileRows * 8;
  uint32_t* s_slot = reinterpret_cast<uint32_t*>(p);
  p += kTileRows * 4;
  uint32_t* s_first = reinterpret_cast<uint32_t*>(p);
  p += kTileRows * 4;
  uint32_t* s_boff = reinterpret_cast<uint32_t*>(p);   // [nblk + 1] plane word offsets
  p += (size_t)(D + 4) * 4;
  uint32_t* s_obase = reinterpret_cast<uint32_t*>(p);  // [nblk + 1] outlier offsets
  p += (size_t)(D + 4) * 4;
  uint8_t* s_width = p;                                // [nblk]
  p += D + 4;
  uint8_t* s_urow = p;                                 // [64] tile row of each uid

  // ---- which tile ----
  if (tid == 0) {
    uint32_t ticket = atomicAdd(&a.w.ctrl[0], 1u);
    uint32_t s = find_segment(a.w.seg_tile_base, a.sh.nseg, ticket);
    uint32_t pch = s / T;
    uint32_t r0 = chunk_row0(a.sh, pch), rows = chunk_row0(a.sh, pch + 1) - r0;
    uint32_t nt = (rows + kTileRows - 1) / kTileRows;
    uint32_t k = ticket - a.w.seg_tile_base[s];
    sh.ticket = ticket;
    sh.seg = s;
    sh.tile = k;
    sh.rows = rows;
    sh.ntiles = nt;
    sh.n = nt ? min(kTileRows, rows - k * kTileRows) : 0;
  }
  __syncthreads();
  const uint32_t ticket = sh.ticket, s = sh.seg, k = sh.tile, n = sh.n, rows = sh.rows;
  const uint32_t ntiles = sh.ntiles;
  const uint32_t pch = s / T, t = s % T;
  const uint32_t row0 = chunk_row0(a.sh, pch);
  const float* xs = a.x + ((uint64_t)t * a.sh.B + row0) * D;  // segment rows
  const float* xt = xs + (uint64_t)k * kTileRows * D;        // tile rows

  // ---- error bound of this table (Algorithm 1 factor, optional range) ----
  if (tid == 0) {
    double f = (double)a.w.eb_base[t] * (double)a.w.mult[t];
    f = f * a.sched;
    float eb = (float)f;
    if (a.eb_mode == 1) {
      float lo = INFINITY, hi = -INFINITY;
      const float* rp = a.w.range_part + 2 * (uint64_t)t * a.w.nbr;
      for (uint32_t j = 0; a.sh.B > 0 && j < a.w.nbr; j++) {
        float l = rp[2 * j], h = rp[2 * j + 1];
        lo = l < lo ? l : lo;
        hi = h > hi ? h : hi;
      }
      float range = hi - lo;
      eb = eb * range;
    }
    float e2 = eb + eb;
    int valid = isfinite(eb) && eb > 0.0f && isfinite(e2);
    sh.eb = eb;
    sh.valid = valid;
    if (a.dbg_eb && k == 0) a.dbg_eb[s] = valid ? eb : 0.0f;
  }
  __syncthreads();
  const float eb = sh.eb;
  const float s2 = eb + eb;
  const bool valid = sh.valid != 0;
  const uint32_t ne = n * D;

  // ---- quantize the tile into LDS (128-bit loads when rows are 16-B sized) ----
  if (valid) {
    if ((D & 3) == 0) {
      const float4* x4 = reinterpret_cast<const float4*>(xt);
      uint2* c4 = reinterpret_cast<uint2*>(s_codes);
      for (uint32_t i = tid; i < ne / 4; i += kThreads) {
        float4 v = x4[i];
        uint32_t c0 = (uint16_t)code_of(v.x, eb, s2), c1 = (uint16_t)code_of(v.y, eb, s2);
        uint32_t c2 = (uint16_t)code_of(v.z, eb, s2), c3 = (uint16_t)code_of(v.w, eb, s2);
        c4[i] = make_uint2(c0 | (c1 << 16), c2 | (c3 << 16));
      }
    } else {
      for (uint32_t i = tid; i < ne; i += kThreads) s_codes[i] = code_of(xt[i], eb, s2);
    }
  }
  __syncthreads();
  if (a.dbg_codes || a.dbg_outlier) {
    uint64_t g0 = ((uint64_t)t * a.sh.B + row0 + (uint64_t)k * kTileRows) * D;
    for (uint32_t i = tid; i < ne; i += kThreads) {
      int16_t c = valid ? s_codes[i] : kSent;
      if (a.dbg_codes) a.dbg_codes[g0 + i] = c == kSent ? 0 : c;
      if (a.dbg_outlier) a.dbg_outlier[g0 + i] = valid ? (c == kSent) : 0;
    }
  }

  uint64_t* htab = a.w.hash + (valid ? a.w.hash_off[s] : 0);
  const uint32_t cap_mask = (1u << a.w.hash_log2[s]) - 1u;

  if (valid && n > 0) {
    // ---- row hash: order-free sum of position-salted element hashes ----
    for (uint32_t i = wv; i < n; i += kThreads / 64) {
      uint64_t acc = 0;
      for (uint32_t d = lane; d < D; d += 64) {
        int16_t c = s_codes[i * D + d];
        uint64_t key = c == kSent ? ((1ull << 32) | f2u(xt[(uint64_t)i * D + d]))
                                  : (uint64_t)(uint32_t)(int32_t)c;
        acc += mix64(key ^ ((uint64_t)d << 40) ^ 0x9e3779b97f4a7c15ull);
      }
      acc = wave_sum_u64(acc);
      if (lane == 0) s_hash[i] = acc;
    }
    __syncthreads();

    // ---- insert: each wave owns 16 rows (lanes 0..15); compares use the wave ----
    {
      const uint32_t i = wv * 16 + lane;
      bool active = lane < 16 && i < n;
      uint64_t H = active ? (s_hash[i] & a.hash_keep) : 0;
      uint32_t h32 = (uint32_t)(H >> 32);
      uint32_t slot = (uint32_t)H & cap_mask;
      uint64_t mine = ((uint64_t)h32 << 32) | (uint64_t)(k * kTileRows + i + 1);
      uint32_t guard = 0;
      while (__ballot(active) != 0) {
        bool need = false;
        uint32_t cand = 0;
        if (active) {
          uint64_t v = ld_rlx64(&htab[slot]);
          if (v == 0) {
            uint64_t old = atomicCAS((unsigned long long*)&htab[slot], 0ull,
                                     (unsigned long long)mine);
            if (old == 0) {
              s_slot[i] = slot;
              active = false;
            } else {
              v = old;
            }
          }
          if (active) {
            if ((uint32_t)(v >> 32) == h32 && (uint32_t)v - 1u < rows) {
              need = true;
              cand = (uint32_t)v - 1u;
            } else {
              slot = (slot + 1) & cap_mask;
            }
          }
        }
        uint64_t m = __ballot(need);
        while (m) {
          int L = __ffsll((long long)m) - 1;
          m &= m - 1;
          uint32_t iL = __shfl(i, L), cL = __shfl(cand, L);
          bool eq = rows_equal(s_codes, xs, xt, iL, cL, D, eb, s2);
          if ((int)lane == L) {
            if (eq) {
              atomicMin((unsigned long long*)&htab[slot], (unsigned long long)mine);
              s_slot[i] = slot;
              active = false;
            } else {
              slot = (slot + 1) & cap_mask;
            }
          }
        }
        if (++guard > cap_mask + 2) {  // cannot happen: the table is at most half full
          if (active) {
            report_error(a.report, kDevErrTimeout);
            s_slot[i] = slot;
            active = false;
          }
        }
      }
    }
    __syncthreads();
    if (tid == 0) {
      __threadfence();
      st_rel32(&a.w.tile_inserted[ticket], 1u);
    }
    // ---- wait until every earlier tile of the segment has inserted its rows ----
    const uint32_t tb = a.w.seg_tile_base[s];
    for (uint32_t j = tid; j < k; j += kThreads) {
      uint32_t spins = 0;
      while (ld_acq32(&a.w.tile_inserted[tb + j]) == 0) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
          report_error(a.report, kDevErrTimeout);
          break;
        }
      }
    }
    __threadfence();
    __syncthreads();
  }

  // ---- first occurrences, bitmap, uids (wave 0, lane = tile row) ----
  if (wv == 0) {
    bool inrow = lane < n;
    uint32_t first = k * kTileRows + lane;
    if (valid && inrow) first = (uint32_t)ld_rlx64(&htab[s_slot[lane]]) - 1u;
    bool uniq = valid && inrow && first == k * kTileRows + lane;
    uint64_t bm = __ballot(uniq);
    if (inrow) s_first[lane] = first;
    if (uniq) s_urow[__popcll(bm & __lanemask_lt())] = (uint8_t)lane;
    if (lane == 0) {
      sh.bitmap = bm;
      sh.U = (uint32_t)__popcll(bm);
    }
    if (a.dbg_first && inrow)
      a.dbg_first[(uint64_t)t * a.sh.B + row0 + k * kTileRows + lane] = first;
  }
  __syncthreads();
  const uint64_t bitmap = sh.bitmap;
  const uint32_t U = sh.U;
  const uint32_t nE = U * D;
  const uint32_t nblk = (nE + 63) / 64;

  // ---- block widths and outlier counts over E (first-occurrence rows) ----
  if (valid) {
    for (uint32_t b = wv; b < nblk; b += kThreads / 64) {
      uint32_t e = b * 64 + lane;
      uint32_t zz = 0;
      bool isout = false;
      if (e < nE) {
        uint32_t u = e / D, d = e - u * D;
        int16_t c = s_codes[s_urow[u] * D + d];
        isout = c == kSent;
        zz = isout ? 0u : zigzag(c);
      }
      uint32_t mx = wave_max_u32(zz);
      uint32_t no = (uint32_t)__popcll(__ballot(isout));
      if (lane == 0) {
        uint32_t w = mx ? 32u - __clz(mx) : 0u;
        s_width[b] = (uint8_t)w;
        s_boff[b] = w;
        s_obase[b] = no;
      }
    }
  }
  __syncthreads();
  uint32_t sumw = 0, nout = 0;
  if (valid && nblk > 0) {
    sumw = block_exclusive_scan(s_boff, nblk, sh.part);
    nout = block_exclusive_scan(s_obase, nblk, sh.part);
  }

  // ---- record layout, RAW fallback, look-back placement ----
  if (tid == 0) {
    uint32_t rb = rows <= 65536 ? 2 : 4;
    uint32_t off_refs = (uint32_t)align_up(16 + nblk, 4);
    uint32_t off_opos = (uint32_t)align_up(off_refs + rb * (n - U), 4);
    uint32_t off_oval = off_opos + 4 * nout;
    uint32_t off_pl = (uint32_t)align_up(off_oval + 4 * nout, 8);
    uint64_t bp = align_up(off_pl + 8ull * sumw, 16);
    uint64_t raw = 16 + align_up(4ull * n * D, 16);
    uint32_t mode = (valid && bp < raw) ? 1u : 0u;
    uint64_t rec = n ? (mode ? bp : raw) : 0;
    uint64_t seg_prefix = 32 + align_up(4ull * ntiles, 16);
    uint64_t chunk_prefix = align_up(8ull * T, 16);
    uint64_t item = rec + (k == 0 ? seg_prefix + (t == 0 ? chunk_prefix : 0) : 0);
    sh.mode = mode;
    sh.rec_size = rec;
    sh.item = item;
    sh.off_refs = off_refs;
    sh.off_opos = off_opos;
    sh.off_oval = off_oval;
    sh.off_pl = off_pl;
    sh.sumw = sumw;
    sh.nout = nout;
    sh.nblk = nblk;
  }
  __syncthreads();

  // decoupled look-back over tiles in stream order (wave 0)
  if (wv == 0) {
    const uint64_t kAgg = 1ull << 62, kIncl = 2ull << 62, kVal = (1ull << 62) - 1;
    const uint64_t item = sh.item;
    uint64_t excl = 0;
    if (ticket == 0) {
      if (lane == 0) st_rel64(&a.w.tile_status[0], kIncl | item);
    } else {
      if (lane == 0) st_rel64(&a.w.tile_status[ticket], kAgg | item);
      int64_t top = (int64_t)ticket - 1;
      while (true) {
        int64_t idx = top - (int64_t)lane;
        uint64_t v = kIncl;  // before tile 0: inclusive prefix 0
        if (idx >= 0) {
          uint32_t spins = 0;
          while (((v = ld_acq64(&a.w.tile_status[idx])) >> 62) == 0) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
              report_error(a.report, kDevErrTimeout);
              v = kIncl;
              break;
            }
          }
        }
        uint64_t incl_mask = __ballot((v >> 62) == 2);
        if (incl_mask) {
          int L = __ffsll((long long)incl_mask) - 1;
          uint64_t mine = (int)lane <= L ? (v & kVal) : 0;
          excl += wave_sum_u64(mine);
          break;
        }
        excl += wave_sum_u64(v & kVal);
        top -= 64;
      }
      if (lane == 0) st_rel64(&a.w.tile_status[ticket], kIncl | (excl + item));
    }
    if (lane == 0) {
      uint64_t pos = a.sh.base_bytes + excl;
      if (k == 0 && t == 0) {
        st_rel64(&a.w.chunk_start[pch], pos + 1);
        pos += align_up(8ull * T, 16);
      }
      if (k == 0) {
        st_rel64(&a.w.seg_start[s], pos + 1);
        pos += 32 + align_up(4ull * ntiles, 16);
      }
      a.w.tile_rec[ticket] = pos;
      if (k + 1 >= ntiles) a.w.seg_end[s] = pos + sh.rec_size + 1;
      sh.rec_abs = pos;
      sh.fin_all = pos + sh.rec_size <= a.out_cap;  // reused as "record fits"
      if (!sh.fin_all) report_error(a.report, kDevErrTimeout);
    }
  }
  __syncthreads();

  // ---- write the tile record ----
  if (n > 0 && sh.fin_all) {
    uint8_t* rec = a.out + sh.rec_abs;
    const uint32_t mode = sh.mode;
    if (tid == 0) {
      uint64_t w1 = (uint64_t)(mode ? nout : 0u) | ((uint64_t)U << 32) | ((uint64_t)mode << 48);
      reinterpret_cast<uint64_t*>(rec)[0] = bitmap;
      reinterpret_cast<uint64_t*>(rec)[1] = w1;
    }
    if (mode == 0) {
      // RAW: rows verbatim, zero pad to 16
      float* dst = reinterpret_cast<float*>(rec + 16);
      if ((D & 3) == 0) {
        const float4* x4 = reinterpret_cast<const float4*>(xt);
        float4* d4 = reinterpret_cast<float4*>(dst);
        for (uint32_t i = tid; i < ne / 4; i += kThreads) d4[i] = x4[i];
      } else {
        for (uint32_t i = tid; i < ne; i += kThreads) dst[i] = xt[i];
        uint32_t pad = (uint32_t)(align_up(4ull * ne, 16) - 4ull * ne) / 4;
        if (tid < pad) dst[ne + tid] = 0.0f;
      }
    } else {
      const uint32_t rb = rows <= 65536 ? 2 : 4;
      const uint32_t off_refs = sh.off_refs, off_opos = sh.off_opos, off_oval = sh.off_oval;
      const uint32_t off_pl = sh.off_pl;
      // widths + zero pad up to the refs
      for (uint32_t b = tid; b < off_refs - 16; b += kThreads) rec[16 + b] = b < nblk ? s_width[b] : 0;
      // refs (first occurrence of every repeated row, row order) + pad
      if (tid < n && !((bitmap >> tid) & 1ull)) {
        uint32_t j = tid - (uint32_t)__popcll(bitmap & ((1ull << tid) - 1ull));
        if (rb == 2) reinterpret_cast<uint16_t*>(rec + off_refs)[j] = (uint16_t)s_first[tid];
        else reinterpret_cast<uint32_t*>(rec + off_refs)[j] = s_first[tid];
      }
      {
        uint32_t rend = off_refs + rb * (n - U);
        if (tid < off_opos - rend) rec[rend + tid] = 0;
        uint32_t oend = off_oval + 4 * nout;
        if (tid < off_pl - oend) rec[oend + tid] = 0;
        uint64_t pend = off_pl + 8ull * sumw;
        if (tid < sh.rec_size - pend) rec[pend + tid] = 0;
      }
      // outliers and bit planes, one wave per 64-element block
      uint64_t* planes = reinterpret_cast<uint64_t*>(rec + off_pl);
      uint32_t* opos = reinterpret_cast<uint32_t*>(rec + off_opos);
      uint32_t* oval = reinterpret_cast<uint32_t*>(rec + off_oval);
      for (uint32_t b = wv; b < nblk; b += kThreads / 64) {
        uint32_t e = b * 64 + lane;
        uint32_t zz = 0;
        bool isout = false;
        uint32_t u = 0, d = 0;
        if (e < nE) {
          u = e / D;
          d = e - u * D;
          int16_t c = s_codes[s_urow[u] * D + d];
          isout = c == kSent;
          zz = isout ? 0u : zigzag(c);
        }
        uint64_t om = __ballot(isout);
        if (isout) {
          uint32_t o = s_obase[b] + (uint32_t)__popcll(om & __lanemask_lt());
          opos[o] = e;
          oval[o] = f2u(xt[(uint64_t)s_urow[u] * D + d]);
        }
        const uint32_t w = s_width[b];
        uint64_t mine = 0;
        for (uint32_t j = 0; j < w; j++) {
          uint64_t word = __ballot((zz >> j) & 1u);
          if (lane == j) mine = word;
        }
        if (lane < w) planes[s_boff[b] + lane] = mine;
      }
    }
  }

  // ---- segment and stream completion ----
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    atomicAdd(&a.w.seg_U[s], U);
    atomicAdd(&a.w.seg_nout[s], sh.mode ? nout : 0u);
    __threadfence();
    uint32_t done = atomicAdd(&a.w.seg_done[s], 1u);
    sh.fin_seg = (done + 1 >= (ntiles ? ntiles : 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (!sh.fin_seg) return;
  __threadfence();
  const uint64_t seg_start = ld_acq64(&a.w.seg_start[s]) - 1;
  const uint64_t seg_end = ld_acq64(&a.w.seg_end[s]) - 1;
  if (seg_end > a.out_cap || seg_start + 32 + 4ull * ntiles > seg_end) {
    if (tid == 0) report_error(a.report, kDevErrTimeout);
    return;
  }
  uint64_t chunk_start = 0;
  if (t == 0) {
    chunk_start = seg_start - align_up(8ull * T, 16);
  } else {
    uint64_t v;
    uint32_t spins = 0;
    while ((v = ld_acq64(&a.w.chunk_start[pch])) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        report_error(a.report, kDevErrTimeout);
        v = 1;
        break;
      }
    }
    chunk_start = v - 1;
  }
  if (chunk_start + align_up(8ull * T, 16) > seg_start) {
    if (tid == 0) report_error(a.report, kDevErrTimeout);
    return;
  }
  uint8_t* sg = a.out + seg_start;
  const uint32_t tb = a.w.seg_tile_base[s];
  for (uint32_t j = tid; j < ntiles; j += kThreads)
    reinterpret_cast<uint32_t*>(sg + 32)[j] = (uint32_t)(a.w.tile_rec[tb + j] - seg_start);
  {
    uint32_t dend = 32 + 4 * ntiles, dpad = (uint32_t)align_up(dend, 16) - dend;
    if (tid < dpad) sg[dend + tid] = 0;
  }
  if (tid == 0) {
    const uint64_t bytes = seg_end - seg_start;
    uint32_t* h = reinterpret_cast<uint32_t*>(sg);
    h[0] = rows;
    h[1] = ntiles;
    h[2] = f2u(valid ? eb : 0.0f);
    h[3] = valid ? 1u : 0u;
    h[4] = __hip_atomic_load(&a.w.seg_U[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    h[5] = __hip_atomic_load(&a.w.seg_nout[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    reinterpret_cast<uint64_t*>(sg)[3] = bytes;
    reinterpret_cast<uint64_t*>(a.out + chunk_start)[t] = seg_start - chunk_start;
    if (a.report) a.report->seg_bytes[s] = bytes;
    __threadfence();
    uint32_t g = atomicAdd(&a.w.ctrl[1], 1u);
    sh.fin_all = (g + 1 == a.sh.nseg) ? 1u : 0u;
  }
  __syncthreads();
  if (!sh.fin_all) return;
  __threadfence();
  // the last segment to finish writes the stream header and chunk table
  const uint32_t P = a.sh.P;
  for (uint32_t q = tid; q < P; q += kThreads) {
    uint64_t cs = ld_acq64(&a.w.chunk_start[q]) - 1;
    uint64_t ce = ld_acq64(&a.w.seg_end[(uint64_t)q * T + T - 1]) - 1;
    if (cs + align_up(8ull * T, 16) > ce || ce > a.out_cap) {
      report_error(a.report, kDevErrTimeout);
      continue;
    }
    reinterpret_cast<uint64_t*>(a.out + 64)[q] = ce - cs;
    if (T & 1u) reinterpret_cast<uint64_t*>(a.out + cs)[T] = 0;  // pad of segment table
  }
  if ((P & 1u) && tid == 0) reinterpret_cast<uint64_t*>(a.out + 64)[P] = 0;
  if (tid == 0) {
    const uint64_t total = ld_acq64(&a.w.seg_end[a.sh.nseg - 1]) - 1;
    uint32_t* h = reinterpret_cast<uint32_t*>(a.out);
    h[0] = kMagic;
    h[1] = kVersion | (kCoderBitpack << 16);
    h[2] = T;
    h[3] = a.sh.B;
    h[4] = D;
    h[5] = P;
    h[6] = kTileRows;
    h[7] = a.eb_mode;
    uint64_t* h64 = reinterpret_cast<uint64_t*>(a.out);
    h64[4] = (uint64_t)a.iter;
    h64[5] = 4ull * T * a.sh.B * D;
    h64[6] = total;
    h64[7] = 0;
    if (a.report) a.report->total_bytes = total;
  }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
struct DecTile {
  const uint8_t* rec;   // record start
  uint64_t avail;       // bytes from the record start to the segment end
  uint64_t bitmap;
  uint32_t n, U, nout, mode, ok;
};

struct DecShared {
  uint32_t ok, seg, tile, n, rows, ntiles, valid;
  float eb;
  uint64_t seg_off, seg_bytes;
  DecTile tl;
};

__device__ __forceinline__ uint64_t rd64(const uint8_t* p) {
  return *reinterpret_cast<const uint64_t*>(p);
}
__device__ __forceinline__ uint32_t rd32(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

// Locate and check tile record k of a segment.  Every thread may call this;
// all reads are bounds-checked against the segment.
__device__ DecTile locate_tile(const uint8_t* seg, uint64_t seg_bytes, uint32_t ntiles,
                               uint32_t rows, uint32_t k, uint32_t D, bool valid) {
  DecTile r{};
  r.ok = 0;
  if (k >= ntiles) return r;
  const uint64_t prefix = 32 + align_up(4ull * ntiles, 16);
  uint32_t off = rd32(seg + 32 + 4ull * k);
  if (off < prefix || (off & 15u) || (uint64_t)off + 16 > seg_bytes) return r;
  r.rec = seg + off;
  r.avail = seg_bytes - off;
  r.n = min(kTileRows, rows - k * kTileRows);
  r.bitmap = rd64(r.rec);
  r.nout = rd32(r.rec + 8);
  uint32_t w3 = rd32(r.rec + 12);
  r.U = w3 & 0xffffu;
  r.mode = (w3 >> 16) & 0xffu;
  if ((w3 >> 24) != 0) return r;
  if (r.n < 64 && (r.bitmap >> r.n) != 0) return r;
  if ((uint32_t)__popcll(r.bitmap) != r.U) return r;
  if (!valid && (r.bitmap != 0 || r.mode != 0)) return r;
  if (r.mode == 0) {
    if (r.nout != 0 || 16 + 4ull * r.n * D > r.avail) return r;
  } else if (r.mode == 1) {
    uint64_t nE = (uint64_t)r.U * D;
    if (r.nout > nE) return r;
    uint64_t nblk = (nE + 63) / 64;
    uint32_t rb = rows <= 65536 ? 2 : 4;
    uint64_t off_refs = align_up(16 + nblk, 4);
    uint64_t off_opos = align_up(off_refs + (uint64_t)rb * (r.n - r.U), 4);
    uint64_t off_pl = align_up(off_opos + 8ull * r.nout, 8);
    if (off_pl > r.avail) return r;
  } else {
    return r;
  }
  r.ok = 1;
  return r;
}

// Reconstruct the key values of first-occurrence row `i` of tile `tl` into
// y[0..D) (whole wave).  Returns false on a malformed record.
__device__ bool decode_key_row(const DecTile& tl, uint32_t i, uint32_t rows, uint32_t D,
                               float eb, float s2, float* y, bool requant_raw) {
  const uint32_t lane = threadIdx.x & 63;
  if (tl.mode == 0) {
    const float* src = reinterpret_cast<const float*>(tl.rec + 16) + (uint64_t)i * D;
    for (uint32_t d = lane; d < D; d += 64) {
      float v = src[d];
      if (requant_raw) {
        int q;
        v = quantize(v, eb, s2, q) ? v : (float)q * s2;
      }
      y[d] = v;
    }
    return true;
  }
  const uint32_t u = (uint32_t)__popcll(tl.bitmap & ((1ull << i) - 1ull));
  const uint32_t nE = tl.U * D, nblk = (nE + 63) / 64;
  const uint32_t rb = rows <= 65536 ? 2 : 4;
  const uint32_t off_refs = (uint32_t)align_up(16 + nblk, 4);
  const uint32_t off_opos = (uint32_t)align_up(off_refs + rb * (tl.n - tl.U), 4);
  const uint32_t off_oval = off_opos + 4 * tl.nout;
  const uint32_t off_pl = (uint32_t)align_up(off_oval + 4 * tl.nout, 8);
  const uint8_t* widths = tl.rec + 16;
  const uint32_t e0 = u * D, b0 = e0 >> 6;
  uint32_t part = 0, bad = 0;
  for (uint32_t j = lane; j < b0; j += 64) {
    uint32_t w = widths[j];
    bad |= w > 12;
    part += w;
  }
  uint32_t run = wave_sum_u32(part);
  if (__any(bad)) return false;
  // outliers of this row: first index with position >= e0 (binary search)
  const uint32_t* opos = reinterpret_cast<const uint32_t*>(tl.rec + off_opos);
  const uint32_t* oval = reinterpret_cast<const uint32_t*>(tl.rec + off_oval);
  uint32_t olo = 0, ohi = tl.nout;
  while (olo < ohi) {
    uint32_t mid = (olo + ohi) >> 1;
    if (opos[mid] < e0) olo = mid + 1;
    else ohi = mid;
  }
  const uint64_t plane_words = (tl.avail - off_pl) / 8;
  const uint64_t* planes = reinterpret_cast<const uint64_t*>(tl.rec + off_pl);
  bool okrow = true;
  for (uint32_t m = 0; m * 64 < D; m++) {
    const uint32_t A = b0 + m;
    const uint32_t wA = A < nblk ? widths[A] : 0;
    const uint32_t wB = A + 1 < nblk ? widths[A + 1] : 0;
    const uint32_t d = m * 64 + lane;
    const uint32_t e = e0 + d;
    const bool inB = (e >> 6) != A;
    const uint32_t w = inB ? wB : wA;
    const uint32_t off = inB ? run + wA : run;
    uint32_t zz = 0;
    bool lane_ok = w <= 12 && (uint64_t)off + w <= plane_words;
    if (d < D && lane_ok) {
      const uint32_t bit = e & 63;
      for (uint32_t j = 0; j < w; j++) zz |= (uint32_t)((planes[off + j] >> bit) & 1ull) << j;
    }
    okrow = okrow && (d >= D || lane_ok);
    float v = (float)unzigzag(zz) * s2;
    while (olo < tl.nout) {
      uint32_t pos = opos[olo];
      if (pos >= e0 + min(D, m * 64 + 64)) break;
      if (pos == e) v = __uint_as_float(oval[olo]);
      olo++;
    }
    if (d < D) y[d] = v;
    run += wA;
  }
  return __all(okrow);
}

__global__ void __launch_bounds__(kThreads) ec_decode_kernel(DecArgs a) {
  __shared__ DecShared sh;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint32_t D = a.sh.D, T = a.sh.T, B = a.sh.B, P = a.sh.P;
  const uint32_t ticket = blockIdx.x;
  if (tid == 0) {
    uint32_t s = find_segment(a.seg_tile_base, a.sh.nseg, ticket);
    uint32_t pch = s / T, t = s % T;
    uint32_t r0 = chunk_row0(a.sh, pch), rows = chunk_row0(a.sh, pch + 1) - r0;
    uint32_t nt = (rows + kTileRows - 1) / kTileRows;
    uint32_t k = ticket - a.seg_tile_base[s];
    sh.seg = s;
    sh.tile = k;
    sh.rows = rows;
    sh.ntiles = nt;
    sh.n = nt ? min(kTileRows, rows - k * kTileRows) : 0;
    uint32_t ok = 1;
    const uint8_t* in = a.in;
    uint64_t total = 0;
    if (a.cap < 64) ok = 0;
    if (ok) {
      const uint32_t* h = reinterpret_cast<const uint32_t*>(in);
      total = rd64(in + 48);
      ok = h[0] == kMagic && h[1] == (kVersion | (kCoderBitpack << 16)) && h[2] == T &&
           h[3] == B && h[4] == D && h[5] == P && h[6] == kTileRows && h[7] <= 1 &&
           rd64(in + 40) == 4ull * T * B * D && rd64(in + 56) == 0 && total <= a.cap;
    }
    uint64_t base = 64 + align_up(8ull * P, 16);
    uint64_t chunk = base, cb = 0;
    if (ok && base > total) ok = 0;
    for (uint32_t q = 0; ok && q <= pch; q++) {
      cb = rd64(in + 64 + 8ull * q);
      if (cb < align_up(8ull * T, 16) || cb > total - chunk) ok = 0;
      else if (q < pch) chunk += cb;
    }
    uint64_t so = 0, sb = 0;
    if (ok) {
      so = rd64(in + chunk + 8ull * t);
      if (so < align_up(8ull * T, 16) || (so & 15u) || so + 32 > cb) ok = 0;
    }
    if (ok) {
      const uint8_t* sg = in + chunk + so;
      uint32_t flags = rd32(sg + 12);
      float eb = __uint_as_float(rd32(sg + 8));
      sb = rd64(sg + 24);
      int valid = isfinite(eb) && eb > 0.0f && isfinite(eb + eb);
      if (rd32(sg) != rows || rd32(sg + 4) != nt || flags > 1 || (int)flags != valid ||
          sb > cb - so || sb < 32 + align_up(4ull * nt, 16))
        ok = 0;
      sh.eb = eb;
      sh.valid = flags;
    }
    sh.seg_off = chunk + so;
    sh.seg_bytes = sb;
    if (ok && nt) {
      DecTile tl = locate_tile(in + chunk + so, sb, nt, rows, k, D, sh.valid != 0);
      ok = tl.ok;
      sh.tl = tl;
    }
    if (!ok) report_error(a.report, kDevErrCorrupt);
    sh.ok = ok;
  }
  __syncthreads();
  const uint32_t s = sh.seg, k = sh.tile, n = sh.n, rows = sh.rows;
  const uint32_t pch = s / T, t = s % T;
  float* yseg = a.y + ((uint64_t)t * B + chunk_row0(a.sh, pch)) * D;
  if (n == 0) return;
  if (!sh.ok) {
    float* yt = yseg + (uint64_t)k * kTileRows * D;
    for (uint32_t i = tid; i < n * D; i += kThreads) yt[i] = 0.0f;
    return;
  }
  const DecTile tl = sh.tl;
  const float eb = sh.eb, s2 = eb + eb;
  const uint8_t* sg = a.in + sh.seg_off;
  const uint64_t sbytes = sh.seg_bytes;
  const uint32_t rb = rows <= 65536 ? 2 : 4;

  if (tl.mode == 0) {  // RAW: rows verbatim
    const float* src = reinterpret_cast<const float*>(tl.rec + 16);
    float* yt = yseg + (uint64_t)k * kTileRows * D;
    if ((D & 3) == 0) {
      const float4* s4 = reinterpret_cast<const float4*>(src);
      float4* y4 = reinterpret_cast<float4*>(yt);
      for (uint32_t i = tid; i < n * D / 4; i += kThreads) y4[i] = s4[i];
    } else {
      for (uint32_t i = tid; i < n * D; i += kThreads) yt[i] = src[i];
    }
    return;
  }

  const uint32_t nblk = (tl.U * D + 63) / 64;
  const uint32_t off_refs = (uint32_t)align_up(16 + nblk, 4);
  for (uint32_t i = wv; i < n; i += kThreads / 64) {
    const uint32_t r = k * kTileRows + i;
    float* y = yseg + (uint64_t)r * D;
    bool ok;
    if ((tl.bitmap >> i) & 1ull) {
      ok = decode_key_row(tl, i, rows, D, eb, s2, y, false);
    } else {
      uint32_t j = i - (uint32_t)__popcll(tl.bitmap & ((1ull << i) - 1ull));
      uint32_t ref = rb == 2 ? reinterpret_cast<const uint16_t*>(tl.rec + off_refs)[j]
                             : reinterpret_cast<const uint32_t*>(tl.rec + off_refs)[j];
      ok = ref < r;
      if (ok) {
        const uint32_t k2 = ref / kTileRows, i2 = ref % kTileRows;
        DecTile t2 = k2 == k ? tl : locate_tile(sg, sbytes, sh.ntiles, rows, k2, D, true);
        ok = t2.ok && ((t2.bitmap >> i2) & 1ull);
        if (ok) ok = decode_key_row(t2, i2, rows, D, eb, s2, y, true);
      }
    }
    if (!ok) {
      for (uint32_t d = lane; d < D; d += 64) y[d] = 0.0f;
      if (lane == 0) report_error(a.report, kDevErrCorrupt);
    }
  }
}

}  // namespace

hipError_t launch_prep(const PrepArgs& a, uint32_t grid, hipStream_t s) {
  hipLaunchKernelGGL(ec_prep_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t set_encode_lds_limit(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&ec_encode_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_encode(const EncArgs& a, hipStream_t s) {
  size_t lds = encode_lds_bytes(a.sh.D);
  hipLaunchKernelGGL(ec_encode_kernel, dim3(a.sh.ntiles), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ec_decode_kernel, dim3(a.sh.ntiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ec
