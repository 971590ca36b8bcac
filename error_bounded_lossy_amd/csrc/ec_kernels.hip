// ec_kernels.hip -- gfx950 (CDNA4, wave64) kernels of the error-bounded lossy
// compressor for DLRM embedding traffic (arXiv 2407.04272).
//
//  prep      clears the per-call workspace and, for range-relative error
//            bounds, reduces every table's (min, max) over non-NaN values
//            (one coalesced 128-bit-load pass over the input).
//  quantize  (D = 64, 128, 256) one workgroup per 64-row tile: quantize
//            (section III-D), pack the codes of every 64-element block as bit
//            planes, stage planes and widths in the workspace, and insert the
//            tile's quantized rows into the segment's hash table (section
//            III-B "Vector Homogenization", the vector-based LZ of III-D).
//  assemble  two launches after every row is in the table: size (first
//            occurrences, record sizes, sums over blocks of tiles) and write
//            (each tile's place in ONE contiguous stream from those sums,
//            section III-E "Buffer Optimization", Fig. 7; the record and the
//            staged planes of first-occurrence rows).
//  encode    (other D) both passes in one kernel, tiles placed by a decoupled
//            look-back over earlier tiles.
//  decode    one workgroup per tile (D = 64, 128, 256: wave 0 checks and
//            indexes the record first); each output row is written once.
//
// Quantization uses IEEE fp32 division and round-to-nearest-even; the build
// disables FP contraction so the reconstruction check is the exact fp32
// sequence div, rint, mul, sub.
#include "ec_internal.h"

#include <mutex>
#include <type_traits>

#include "../../include/ec.h"
#include "ec_huff_decode.h"

#ifndef EC_PREP_LOADS
#define EC_PREP_LOADS 8  // 128-bit loads in flight per thread in the range pass
#endif

namespace ec {
namespace {

constexpr int16_t kSent = (int16_t)0x8000;  // outlier marker in LDS codes
constexpr uint32_t kSpinLimit = 1u << 22;

__device__ __forceinline__ uint64_t align_up(uint64_t v, uint64_t a) {
  return (v + a - 1) / a * a;
}

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

// Lanes below this one.  (HIP's __lanemask_lt() also masks with the lanes
// that are active, so in a divergent branch it is not this.)
__device__ __forceinline__ uint64_t lanes_below() { return (1ull << (threadIdx.x & 63)) - 1ull; }

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
// Inclusive prefix sum over a whole wave by DPP moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes with no source
// add 0), then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into
// rows 2 and 3.  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}
// Sum over a whole wave (every lane active), the same in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_u32(v), 63);
}

// Cross-workgroup communication uses only agent-scope RELAXED atomics (their
// values are coherent across the XCDs); agent-scope acquire/release would write
// back or invalidate a whole XCD L2 on every call.  Ordering is explicit:
//  * publish: every wave whose atomics a flag announces runs wait_vm() (its
//    stores and read-modify-writes are then performed at the coherence point)
//    before the barrier after which the flag is stored.  A workgroup fence or
//    barrier alone does not wait for global memory on this target, so a flag
//    could otherwise overtake the data it announces.
//  * consume: loads of the data are issued only after a load of the flag has
//    returned the published value (a spin loop or a barrier behind it).
__device__ __forceinline__ void fence_wg() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup"); }
// The wave's index in its workgroup, in a scalar register (the compiler does
// not see that threadIdx.x >> 6 is uniform: wave-indexed offsets would become
// per-lane values, and buffer offsets taken from them loops over lanes).
__device__ __forceinline__ uint32_t wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// atomic minimum whose result is awaited (the wave stalls until it is performed)
__device__ __forceinline__ void atomic_min_performed(uint64_t* p, uint64_t v) {
  const uint64_t old = __hip_atomic_fetch_min(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" ::"v"(old));
}
__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// read-modify-write read: returns the value at the coherence point
__device__ __forceinline__ uint64_t rmw_read64(uint64_t* p) {
  return __hip_atomic_fetch_or(p, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t rmw_read32(uint32_t* p) {
  return __hip_atomic_fetch_or(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Segment s and tile k of scheduled tile `ticket`: by division when every
// segment has the same number of tiles, else by search.
__device__ __forceinline__ void ticket_coords(const Shape& sh, const uint32_t* seg_tile_base,
                                              uint32_t ticket, uint32_t& s, uint32_t& k) {
  if (sh.tiles_per_seg) {
    s = ticket / sh.tiles_per_seg;
    k = ticket - s * sh.tiles_per_seg;
  } else {
    s = find_segment(seg_tile_base, sh.nseg, ticket);
    k = ticket - seg_tile_base[s];
  }
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
  if (a.clear)
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
      // eight independent 128-bit loads in flight per thread; indices past
      // the range repeat its last element, which leaves min and max unchanged
      const float4* x4 = reinterpret_cast<const float4*>(xt);
      const uint64_t e4 = end / 4;
      for (uint64_t i = beg / 4 + threadIdx.x; i < e4; i += EC_PREP_LOADS * kThreads) {
        float4 v[EC_PREP_LOADS];
#pragma unroll
        for (int u = 0; u < EC_PREP_LOADS; u++) {
          const uint64_t ii = i + (uint64_t)u * kThreads;
          v[u] = x4[ii < e4 ? ii : e4 - 1];
        }
#pragma unroll
        for (int u = 0; u < EC_PREP_LOADS; u++) {
          const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int c = 0; c < 4; c++) {
            if (e[c] < lo) lo = e[c];  // NaN compares false: skipped
            if (e[c] > hi) hi = e[c];
          }
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
// encode: pieces shared by the generic and the D = 64*C kernels
// ---------------------------------------------------------------------------
struct EncShared {
  uint32_t ticket, seg, tile, n, rows, ntiles;
  float eb;
  int valid;
  uint64_t bitmap;
  uint32_t U, nblk, sumw, nout, mode, fin_seg, fin_all, fits;
  uint64_t rec_size, rec_abs, item;
  uint32_t off_refs, off_opos, off_oval, off_pl;
  uint32_t part[kThreads / 64];
};

// Thread 0: locate this workgroup's tile.  Tiles are numbered in stream
// order and tile i runs on workgroup i; every wait in the encoder is on a
// tile with a smaller number.  Workgroups are dispatched in increasing order
// (per XCD), so the lowest unfinished tile is always resident and waits on
// nothing unfinished: the waits cannot deadlock.  They are also bounded.
__device__ __forceinline__ void take_tile(const EncArgs& a, EncShared& sh, uint32_t ticket) {
  uint32_t s, k;
  if (a.sh.tiles_per_seg) {  // every segment has the same number of tiles
    s = ticket / a.sh.tiles_per_seg;
    k = ticket - s * a.sh.tiles_per_seg;
  } else {
    s = find_segment(a.w.seg_tile_base, a.sh.nseg, ticket);
    k = ticket - a.w.seg_tile_base[s];
  }
  const uint32_t pch = s / a.sh.T;
  const uint32_t r0 = chunk_row0(a.sh, pch), rows = chunk_row0(a.sh, pch + 1) - r0;
  const uint32_t nt = (rows + kTileRows - 1) / kTileRows;
  sh.ticket = ticket;
  sh.seg = s;
  sh.tile = k;
  sh.rows = rows;
  sh.ntiles = nt;
  sh.n = nt ? min(kTileRows, rows - k * kTileRows) : 0;
}

// Order-preserving u32 key of a (non-NaN) float: keys compare as the values
// do, -0 below +0; key 0 is no value's.
__device__ __forceinline__ uint32_t f2key(float f) {
  const uint32_t i = f2u(f);
  return (i & 0x80000000u) ? ~i : (i | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// With the range folded into the quantize pass, its workgroups take range
// items and tiles in table-major order, the range items of table t + k
// (k = range_ahead) just before the tiles of table t:
//   R(0) .. R(k-1) | R(k) Q(0) | R(k+1) Q(1) | ... | Q(T-1)
// A tile waits only for range items with smaller numbers, which wait for
// nothing, so with workgroups dispatched in increasing order the waits always
// end.  Returns the tile's ticket, or ~0u for range item *ri of table *rt.
__device__ __forceinline__ uint32_t fused_item(const EncArgs& a, uint32_t i, uint32_t& rt, uint32_t& ri) {
  const uint32_t T = a.sh.T, nr = a.range_items, tpt = a.tiles_per_table;
  const uint32_t k = min(a.range_ahead, T), full = T - k;  // blocks with range items
  uint32_t t, q;
  if (i < k * nr) {
    rt = i / nr;
    ri = i - rt * nr;
    return ~0u;
  }
  const uint32_t j = i - k * nr, blk = nr + tpt;
  if (j < full * blk) {
    t = j / blk;
    q = j - t * blk;
    if (q < nr) {
      rt = t + k;
      ri = q;
      return ~0u;
    }
    q -= nr;
  } else {
    const uint32_t j2 = j - full * blk;
    t = full + j2 / tpt;
    q = j2 - (t - full) * tpt;
  }
  // tile q of table t in table-major order; segments of chunk p all have the
  // same number of scheduled tiles, seg_tile_base[pT] / T of them in each
  // table before chunk p
  uint32_t lo = 0, hi = a.sh.P;
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (a.w.seg_tile_base[mid * T] / T <= q) lo = mid;
    else hi = mid;
  }
  return a.w.seg_tile_base[lo * T + t] + (q - a.w.seg_tile_base[lo * T] / T);
}

// A range item: (min, max) without NaN of its slice of table t, stored as
// ordered keys (key(max), ~key(min)), or (0, 1) for no value.  Whole workgroup.
__device__ void range_item(const EncArgs& a, uint32_t t, uint32_t ri) {
  __shared__ uint32_t s_kh[kThreads / 64], s_kl[kThreads / 64];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const uint64_t nel = (uint64_t)a.sh.B * a.sh.D;
  uint64_t per = (nel + a.range_items - 1) / a.range_items;
  per = (per + 1023) / 1024 * 1024;
  const uint64_t beg = min((uint64_t)ri * per, nel), end = min(beg + per, nel);
  const float* xt = a.x + (uint64_t)t * nel;
  float lo = INFINITY, hi = -INFINITY;
  if ((nel & 3) == 0) {  // eight 128-bit loads in flight per thread
    const float4* x4 = reinterpret_cast<const float4*>(xt);
    for (uint64_t i = beg / 4 + tid; i < end / 4; i += 8 * kThreads) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const uint64_t ii = i + (uint64_t)u * kThreads;
        v[u] = ii < end / 4 ? x4[ii] : make_float4(NAN, NAN, NAN, NAN);
      }
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int c = 0; c < 4; c++) {
          lo = e[c] < lo ? e[c] : lo;  // NaN compares false: skipped
          hi = e[c] > hi ? e[c] : hi;
        }
      }
    }
  } else {
    for (uint64_t i = beg + tid; i < end; i += kThreads) {
      const float v = xt[i];
      lo = v < lo ? v : lo;
      hi = v > hi ? v : hi;
    }
  }
  uint32_t kh = lo <= hi ? f2key(hi) : 0u, kl = lo <= hi ? ~f2key(lo) : 0u;
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t h2 = (uint32_t)__shfl_xor((int)kh, o), l2 = (uint32_t)__shfl_xor((int)kl, o);
    kh = h2 > kh ? h2 : kh;
    kl = l2 > kl ? l2 : kl;
  }
  if (lane == 0) {
    s_kh[wv] = kh;
    s_kl[wv] = kl;
  }
  __syncthreads();
  if (tid == 0) {
    for (uint32_t q = 1; q < kThreads / 64; q++) {
      kh = s_kh[q] > kh ? s_kh[q] : kh;
      kl = s_kl[q] > kl ? s_kl[q] : kl;
    }
    st64(&a.w.range_slot[(uint64_t)t * a.range_items + ri], kh ? ((uint64_t)kh << 32) | kl : 1ull);
  }
}

// Error bound of table t (Algorithm 1's factor times the table's value range
// in range-relative mode).  Called by one whole wave; lanes reduce the range
// partials in parallel.  Result and validity are returned to every lane.
__device__ __forceinline__ float table_eb(const EncArgs& a, uint32_t t, bool& valid) {
  const uint32_t lane = threadIdx.x & 63;
  double f = (double)a.w.eb_base[t] * (double)a.w.mult[t];
  f = f * a.sched;
  float eb = (float)f;
  if (a.eb_mode == 1) {
    float lo = INFINITY, hi = -INFINITY;
    if (a.fuse_range) {
      // every range item of the table has stored its (min, max): they come
      // before the table's tiles and wait on nothing, so the wait ends
      // (bounded all the same; a timeout is reported).  Each item has a word
      // of its own: waiting waves poll plain loads, no contended atomics.
      const uint64_t* sl = a.w.range_slot + (uint64_t)t * a.range_items;
      uint32_t kh = 0, kl = 0, spins = 0;
      for (;;) {
        bool ready = true;
        kh = 0;
        kl = 0;
        for (uint32_t j = lane; j < a.range_items; j += 64) {
          const uint64_t w = ld64(&sl[j]);
          ready = ready && w != 0;
          const uint32_t h = (uint32_t)(w >> 32), l = (uint32_t)w;
          if (h != 0) {  // the tile has values: fold the keys (max key, max ~key)
            kh = h > kh ? h : kh;
            kl = l > kl ? l : kl;
          }
        }
        if (__all(ready)) break;
        __builtin_amdgcn_s_sleep(8);
        if (++spins > kSpinLimit) {
          if (lane == 0) report_error(a.report, kDevErrTimeout);
          break;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const uint32_t h2 = (uint32_t)__shfl_xor((int)kh, o), l2 = (uint32_t)__shfl_xor((int)kl, o);
        kh = h2 > kh ? h2 : kh;
        kl = l2 > kl ? l2 : kl;
      }
      if (kh != 0) {
        hi = key2f(kh);
        lo = key2f(~kl);
      }
    } else if (a.sh.B > 0) {
      const float2* rp = reinterpret_cast<const float2*>(a.w.range_part) + (uint64_t)t * a.w.nbr;
      // eight partials per lane loaded together (one round trip up to 512)
      for (uint32_t j0 = 0; j0 < a.w.nbr; j0 += 8 * 64) {
        float2 v[8];
#pragma unroll
        for (uint32_t q = 0; q < 8; q++) {
          const uint32_t j = j0 + 64 * q + lane;
          v[q] = j < a.w.nbr ? rp[j] : make_float2(INFINITY, -INFINITY);
        }
#pragma unroll
        for (uint32_t q = 0; q < 8; q++) {
          lo = v[q].x < lo ? v[q].x : lo;
          hi = v[q].y > hi ? v[q].y : hi;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        float l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
      }
    }
    float range = hi - lo;
    eb = eb * range;
  }
  float e2 = eb + eb;
  valid = isfinite(eb) && eb > 0.0f && isfinite(e2);
  return eb;
}

// Record sizes for the tile (thread 0): RAW vs BITPACK choice and the
// look-back item (record plus, for a segment's first tile, the segment and
// chunk prefixes that precede it in the stream).
__device__ __forceinline__ void size_record(const EncArgs& a, EncShared& sh, bool valid,
                                            uint32_t n, uint32_t U, uint32_t nblk,
                                            uint32_t sumw, uint32_t nout) {
  const uint32_t D = a.sh.D, T = a.sh.T;
  const uint32_t k = sh.tile, t = sh.seg % T, rows = sh.rows, ntiles = sh.ntiles;
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
  sh.mode = mode;
  sh.rec_size = rec;
  sh.item = rec + (k == 0 ? seg_prefix + (t == 0 ? chunk_prefix : 0) : 0);
  sh.off_refs = off_refs;
  sh.off_opos = off_opos;
  sh.off_oval = off_oval;
  sh.off_pl = off_pl;
  sh.sumw = sumw;
  sh.nout = nout;
  sh.nblk = nblk;
  sh.U = U;
}

// Bounded spin of one lane until a relaxed 64-bit word becomes non-zero.
__device__ __forceinline__ uint64_t spin_word(const EncArgs& a, const uint64_t* p) {
  uint64_t v = ld64(p);
  uint32_t spins = 0;
  while (v == 0) {
    __builtin_amdgcn_s_sleep(1);
    v = ld64(p);
    if (++spins > kSpinLimit) {
      report_error(a.report, kDevErrTimeout);
      return 0;
    }
  }
  return v;
}

// Wave 0: the tile's place in the stream, a two-level prefix sum over tiles in
// ticket (= stream) order.  Each tile publishes its item; the tiles of a block
// of 64 consecutive tickets sum the items before them in their block (one
// lane each); the block's last tile publishes the block sum and then the
// block's inclusive prefix, found by a decoupled look-back over the block
// words of earlier blocks, which every tile also runs.  Every wait is on a
// smaller ticket.  Publishes the segment / chunk starts and the record
// offset; sets sh.rec_abs, sh.fits.
__device__ __forceinline__ void place_record(const EncArgs& a, EncShared& sh) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t kAgg = 1ull << 62, kIncl = 2ull << 62, kVal = (1ull << 62) - 1;
  const uint32_t ticket = sh.ticket, s = sh.seg, k = sh.tile, ntiles = sh.ntiles;
  const uint32_t T = a.sh.T, pch = s / T, t = s % T;
  const uint64_t item = sh.item;
  const uint32_t blk = ticket >> 6, pos_in = ticket & 63u;
  if (lane == 0) st64(&a.w.tile_status[ticket], item + 1);
  uint64_t v = 0;
  if (lane < pos_in) v = spin_word(a, &a.w.tile_status[(blk << 6) + lane]) - 1;
  const uint64_t pre_in = wave_sum_u64(v);
  const bool last_in_blk = pos_in == 63 || ticket + 1 == a.sh.ntiles;
  if (last_in_blk && lane == 0) st64(&a.w.block_status[blk], kAgg | (pre_in + item));
  uint64_t excl_b = 0;  // items of all earlier blocks
  int64_t top = (int64_t)blk - 1;
  while (top >= 0) {
    const int64_t idx = top - (int64_t)lane;
    const uint64_t w = idx >= 0 ? spin_word(a, &a.w.block_status[idx]) : kIncl;  // before block 0: 0
    const uint64_t incl_mask = __ballot((w >> 62) == 2);
    if (incl_mask) {
      const int L = __ffsll((long long)incl_mask) - 1;
      excl_b += wave_sum_u64((int)lane <= L ? (w & kVal) : 0);
      break;
    }
    excl_b += wave_sum_u64(w & kVal);
    top -= 64;
  }
  if (last_in_blk && lane == 0) st64(&a.w.block_status[blk], kIncl | (excl_b + pre_in + item));
  const uint64_t excl = excl_b + pre_in;
  if (lane == 0) {
    uint64_t pos = a.sh.base_bytes + excl;
    if (k == 0 && t == 0) {
      st64(&a.w.chunk_start[pch], pos + 1);
      pos += align_up(8ull * T, 16);
    }
    if (k == 0) {
      st64(&a.w.seg_start[s], pos + 1);
      pos += 32 + align_up(4ull * ntiles, 16);
    }
    if (k + 1 >= ntiles) st64(&a.w.seg_end[s], pos + sh.rec_size + 1);
    sh.rec_abs = pos;
    sh.fits = pos + sh.rec_size <= a.out_cap;
    if (!sh.fits) report_error(a.report, kDevErrTimeout);
  }
}

// Bounded spin until a relaxed 64-bit word becomes non-zero.
__device__ __forceinline__ uint64_t spin_nonzero64(const EncArgs& a, const uint64_t* p) {
  uint64_t v;
  uint32_t spins = 0;
  while ((v = ld64(p)) == 0) {
    __builtin_amdgcn_s_sleep(2);
    if (++spins > kSpinLimit) {
      report_error(a.report, kDevErrTimeout);
      return 0;
    }
  }
  return v;
}

// Whole workgroup, after the record is written.  Every tile publishes its
// record offset and counts (no shared counters, so no atomic contention);
// the last tile of a segment gathers them and writes the segment header and
// tile directory; the last tile of the stream writes the stream header and
// chunk table once every segment is finished.
__device__ void complete_tile(const EncArgs& a, EncShared& sh, bool valid, float eb) {
  const uint32_t tid = threadIdx.x;
  const uint32_t ticket = sh.ticket, s = sh.seg, k = sh.tile, ntiles = sh.ntiles, rows = sh.rows;
  const uint32_t T = a.sh.T, pch = s / T, t = s % T;
  __syncthreads();
  if (tid == 0) {
    // tid 0 also stored this tile's look-back word and, for a segment's first
    // tile, the segment and chunk starts: all performed before tile_rec
    st32(&a.w.tile_U[ticket], sh.U);
    st32(&a.w.tile_nout[ticket], sh.mode ? sh.nout : 0u);
    wait_vm();
    st64(&a.w.tile_rec[ticket], sh.rec_abs + 1);
  }
  if (k + 1 < (ntiles ? ntiles : 1)) return;  // not the segment's last tile

  const uint32_t tb = ticket - k;
  uint32_t u = 0, o = 0;
  for (uint32_t j = tid; j < ntiles; j += kThreads) {
    spin_nonzero64(a, &a.w.tile_rec[tb + j]);
    u += ld32(&a.w.tile_U[tb + j]);
    o += ld32(&a.w.tile_nout[tb + j]);
  }
  u = wave_sum_u32(u);
  o = wave_sum_u32(o);
  const uint32_t lane = tid & 63, wv = tid >> 6;
  if (lane == 0) {
    sh.part[wv] = u;
  }
  __syncthreads();
  uint32_t U = 0;
  for (uint32_t j = 0; j < kThreads / 64; j++) U += sh.part[j];
  __syncthreads();
  if (lane == 0) sh.part[wv] = o;
  __syncthreads();
  uint32_t NO = 0;
  for (uint32_t j = 0; j < kThreads / 64; j++) NO += sh.part[j];
  // tile 0 published seg_start before its record offset, which the loop above
  // has seen (the barriers order this read after that observation)
  const uint64_t seg_start = ld64(&a.w.seg_start[s]) - 1;
  const uint64_t seg_end = sh.rec_abs + sh.rec_size;  // this tile ends the segment
  bool ok = seg_end <= a.out_cap && seg_start + 32 + 4ull * ntiles <= seg_end;
  uint64_t chunk_start = 0;
  if (t == 0) {
    chunk_start = seg_start - align_up(8ull * T, 16);
  } else {
    const uint64_t v = spin_nonzero64(a, &a.w.chunk_start[pch]);
    chunk_start = v ? v - 1 : 0;
  }
  ok = ok && chunk_start + align_up(8ull * T, 16) <= seg_start;
  if (ok) {
    uint8_t* sg = a.out + seg_start;
    for (uint32_t j = tid; j < ntiles; j += kThreads)
      reinterpret_cast<uint32_t*>(sg + 32)[j] = (uint32_t)(ld64(&a.w.tile_rec[tb + j]) - 1 - seg_start);
    uint32_t dend = 32 + 4 * ntiles, dpad = (uint32_t)align_up(dend, 16) - dend;
    if (tid < dpad) sg[dend + tid] = 0;
    if (tid == 0) {
      const uint64_t bytes = seg_end - seg_start;
      uint32_t* h = reinterpret_cast<uint32_t*>(sg);
      h[0] = rows;
      h[1] = ntiles;
      h[2] = f2u(valid ? eb : 0.0f);
      h[3] = valid ? 1u : 0u;
      h[4] = U;
      h[5] = NO;
      reinterpret_cast<uint64_t*>(sg)[3] = bytes;
      reinterpret_cast<uint64_t*>(a.out + chunk_start)[t] = seg_start - chunk_start;
      if (a.report) a.report->seg_bytes[s] = bytes;
      if (a.seg_meta) {
        a.seg_meta[2 * s] = U;
        a.seg_meta[2 * s + 1] = valid ? 1u : 0u;
      }
    }
  } else if (tid == 0) {
    report_error(a.report, kDevErrTimeout);
  }
  if (tid == 0) {
    // seg_end (stored by tid 0 in place_record) is performed before seg_fin
    wait_vm();
    st32(&a.w.seg_fin[s], 1u);
  }
  if (ticket + 1 != a.sh.ntiles) return;  // not the stream's last tile

  // the stream's last tile: wait for every segment, then header + chunk table
  for (uint32_t q = tid; q < a.sh.nseg; q += kThreads) {
    uint32_t spins = 0;
    while (ld32(&a.w.seg_fin[q]) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        report_error(a.report, kDevErrTimeout);
        break;
      }
    }
  }
  __syncthreads();
  const uint32_t P = a.sh.P, D = a.sh.D;
  for (uint32_t q = tid; q < P; q += kThreads) {
    uint64_t cs = ld64(&a.w.chunk_start[q]) - 1;
    uint64_t ce = ld64(&a.w.seg_end[(uint64_t)q * T + T - 1]) - 1;
    if (cs + align_up(8ull * T, 16) > ce || ce > a.out_cap) {
      report_error(a.report, kDevErrTimeout);
      continue;
    }
    reinterpret_cast<uint64_t*>(a.out + 64)[q] = ce - cs;
    if (T & 1u) reinterpret_cast<uint64_t*>(a.out + cs)[T] = 0;  // pad of segment table
  }
  if ((P & 1u) && tid == 0) reinterpret_cast<uint64_t*>(a.out + 64)[P] = 0;
  if (tid == 0) {
    const uint64_t total = ld64(&a.w.seg_end[a.sh.nseg - 1]) - 1;
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

// Wait until every earlier tile of segment s has inserted its rows.
__device__ __forceinline__ void wait_inserted(const EncArgs& a, uint32_t s, uint32_t k) {
  const uint32_t tb = a.w.seg_tile_base[s];
  for (uint32_t j = threadIdx.x; j < k; j += kThreads) {
    uint32_t spins = 0;
    while (ld32(&a.w.tile_inserted[tb + j]) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kSpinLimit) {
        report_error(a.report, kDevErrTimeout);
        break;
      }
    }
  }
}

// RAW record body: the tile's rows verbatim (zero pad to 16).
__device__ __forceinline__ void write_raw_rows(uint8_t* rec, const float* xt, uint32_t ne,
                                               uint32_t D) {
  const uint32_t tid = threadIdx.x;
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
}

// Zero pad bytes between a BITPACK record's sections and after its planes.
__device__ __forceinline__ void write_record_pads(uint8_t* rec, const EncShared& sh, uint32_t n,
                                                  uint32_t rows) {
  const uint32_t tid = threadIdx.x;
  const uint32_t rb = rows <= 65536 ? 2 : 4;
  for (uint32_t b = sh.nblk + tid; b < sh.off_refs - 16; b += kThreads) rec[16 + b] = 0;
  uint32_t rend = sh.off_refs + rb * (n - sh.U);
  if (tid < sh.off_opos - rend) rec[rend + tid] = 0;
  uint32_t oend = sh.off_oval + 4 * sh.nout;
  if (tid < sh.off_pl - oend) rec[oend + tid] = 0;
  uint64_t pend = sh.off_pl + 8ull * sh.sumw;
  if (tid < sh.rec_size - pend) rec[pend + tid] = 0;
}

// ---------------------------------------------------------------------------
// generic encoder (any D): codes staged in LDS
// ---------------------------------------------------------------------------
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
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t D = a.sh.D, T = a.sh.T;

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

  if (tid == 0) take_tile(a, sh, blockIdx.x);
  __syncthreads();
  const uint32_t ticket = sh.ticket, s = sh.seg, k = sh.tile, n = sh.n, rows = sh.rows;
  const uint32_t pch = s / T, t = s % T;
  const uint32_t row0 = chunk_row0(a.sh, pch);
  const float* xs = a.x + ((uint64_t)t * a.sh.B + row0) * D;  // segment rows
  const float* xt = xs + (uint64_t)k * kTileRows * D;        // tile rows
  if (wv == 0) {
    bool v;
    float e = table_eb(a, t, v);
    if (lane == 0) {
      sh.eb = e;
      sh.valid = v;
      if (a.dbg_eb && k == 0) a.dbg_eb[s] = v ? e : 0.0f;
    }
  }
  __syncthreads();
  const float eb = sh.eb;
  const float s2 = eb + eb;
  const bool valid = sh.valid != 0;
  const uint32_t ne = n * D;

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
          uint64_t old = atomicCAS((unsigned long long*)&htab[slot], 0ull,
                                   (unsigned long long)mine);
          if (old == 0) {
            s_slot[i] = slot;
            active = false;
          } else if ((uint32_t)(old >> 32) == h32 && (uint32_t)old - 1u < rows) {
            need = true;
            cand = (uint32_t)old - 1u;
          } else {
            slot = (slot + 1) & cap_mask;
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
              atomic_min_performed(&htab[slot], mine);
              s_slot[i] = slot;
              active = false;
            } else {
              slot = (slot + 1) & cap_mask;
            }
          }
        }
        if (++guard > cap_mask + 2) {  // cannot happen: the table is at most a quarter full
          if (active) {
            report_error(a.report, kDevErrTimeout);
            s_slot[i] = slot;
            active = false;
          }
        }
      }
    }
    wait_vm();  // this wave's slot writes are performed before the flag
    __syncthreads();
    if (tid == 0) st32(&a.w.tile_inserted[ticket], 1u);
    wait_inserted(a, s, k);
    fence_wg();
    __syncthreads();
  }

  // ---- first occurrences, bitmap, uids (wave 0, lane = tile row) ----
  if (wv == 0) {
    bool inrow = lane < n;
    uint32_t first = k * kTileRows + lane;
    if (valid && inrow) first = (uint32_t)rmw_read64(&htab[s_slot[lane]]) - 1u;
    bool uniq = valid && inrow && first == k * kTileRows + lane;
    uint64_t bm = __ballot(uniq);
    if (inrow) s_first[lane] = first;
    if (uniq) s_urow[__popcll(bm & lanes_below())] = (uint8_t)lane;
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
  if (tid == 0) size_record(a, sh, valid, n, U, nblk, sumw, nout);
  __syncthreads();
  if (wv == 0) place_record(a, sh);
  __syncthreads();

  // ---- write the tile record ----
  if (n > 0 && sh.fits) {
    uint8_t* rec = a.out + sh.rec_abs;
    const uint32_t mode = sh.mode;
    if (tid == 0) {
      uint64_t w1 = (uint64_t)(mode ? nout : 0u) | ((uint64_t)U << 32) | ((uint64_t)mode << 48);
      reinterpret_cast<uint64_t*>(rec)[0] = bitmap;
      reinterpret_cast<uint64_t*>(rec)[1] = w1;
    }
    if (mode == 0) {
      write_raw_rows(rec, xt, ne, D);
    } else {
      const uint32_t rb = rows <= 65536 ? 2 : 4;
      const uint32_t off_refs = sh.off_refs, off_opos = sh.off_opos, off_oval = sh.off_oval;
      const uint32_t off_pl = sh.off_pl;
      for (uint32_t b = tid; b < nblk; b += kThreads) rec[16 + b] = s_width[b];
      if (tid < n && !((bitmap >> tid) & 1ull)) {
        uint32_t j = tid - (uint32_t)__popcll(bitmap & ((1ull << tid) - 1ull));
        if (rb == 2) reinterpret_cast<uint16_t*>(rec + off_refs)[j] = (uint16_t)s_first[tid];
        else reinterpret_cast<uint32_t*>(rec + off_refs)[j] = s_first[tid];
      }
      write_record_pads(rec, sh, n, rows);
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
          uint32_t o = s_obase[b] + (uint32_t)__popcll(om & lanes_below());
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
  complete_tile(a, sh, valid, eb);
}

// ---------------------------------------------------------------------------
// encoder for D = 64*C.  A 64-element block is one row chunk with element i in
// lane i.  The codes of two blocks are packed as the 16-bit halves of one
// register, and a 32x32 bit-matrix transpose in each half-wave turns them into
// bit planes: afterwards lane L holds the 32-bit half (L >> 5) of plane
// (L & 15) of block ((L >> 4) & 1) of the pair.  A block's width follows from
// which of its plane words are non-zero.  Plane words stay in registers until
// the record is written; LDS keeps only widths, outlier masks and row data.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// v + v + (bit `lane` of the wave-uniform mask m): appends one bit plane to
// codes being rebuilt most-significant plane first.
__device__ __forceinline__ uint32_t double_add_plane(uint32_t v, uint64_t m) {
  uint32_t r;
  uint64_t c;
  asm volatile("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(c) : "v"(v), "s"(m));
  return r;
}

// Exact quantization with a multiply by r = fl(1/s) (correctly rounded): the
// product is within 2^-11 of fl(x/s) for |x/s| < 2048, so whenever it lies at
// least 2^-10 away from every rounding boundary (k + 1/2) and well inside the
// code range, rint of it equals rint(fl(x/s)).  Otherwise the IEEE division
// decides, exactly as quantize() does.
__device__ __forceinline__ bool quantize_fast(float x, float eb, float s, float r, int& q) {
  float tp = x * r;
  float qp = rintf(tp);
  float f = tp - qp;
  float qf;
  if (fabsf(f) < 0.4990234375f && fabsf(tp) < 2046.5f) {
    qf = qp;
  } else {
    float t = x / s;
    if (!(fabsf(t) <= 2047.0f)) {
      q = 0;
      return true;
    }
    qf = rintf(t);
  }
  float xh = qf * s;
  float err = x - xh;
  if (!(fabsf(err) <= eb)) {
    q = 0;
    return true;
  }
  q = (int)qf;
  return false;
}

// Per-lane byte selectors, rotate amounts and masks of the transpose stages.
struct XposeSel {
  uint32_t p16, p8, r4, m4, r2, m2, r1, m1;
};
__device__ __forceinline__ XposeSel xpose_sel(uint32_t L) {
  XposeSel s;
  s.p16 = (L & 16) ? 0x03020706u : 0x05040100u;
  s.p8 = (L & 8) ? 0x03070105u : 0x06020400u;
  s.r4 = (L & 4) ? 4u : 28u;
  s.m4 = (L & 4) ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
  s.r2 = (L & 2) ? 2u : 30u;
  s.m2 = (L & 2) ? 0xCCCCCCCCu : 0x33333333u;
  s.r1 = (L & 1) ? 1u : 31u;
  s.m1 = (L & 1) ? 0xAAAAAAAAu : 0x55555555u;
  return s;
}

// 32x32 bit transpose inside each half-wave: bit i of lane 32h + j of the
// result is bit j of lane 32h + i of v.  Stage s exchanges, between lanes L and
// L ^ s, the bits whose position differs from the lane in bit s: the lower lane
// keeps the positions with bit s clear and takes the partner's ones moved up by
// s, the upper lane the converse.  Stages 16 and 8 move whole half-words and
// bytes (one byte permute); stages 4, 2, 1 rotate the partner word and merge.
__device__ __forceinline__ uint32_t xpose32(uint32_t v, const XposeSel& s) {
  uint32_t y = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);  // lane ^ 16
  v = __builtin_amdgcn_perm(y, v, s.p16);
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  v = __builtin_amdgcn_perm(y, v, s.p8);
  // lane ^ 4: banks 0 and 2 of each row read four lanes up, banks 1 and 3 down
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0x5, false);
  y = (uint32_t)__builtin_amdgcn_update_dpp((int)y, (int)v, 0x124, 0xF, 0xA, false);
  v = (v & s.m4) | (__builtin_amdgcn_alignbit(y, y, s.r4) & ~s.m4);
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // quad [2,3,0,1]
  v = (v & s.m2) | (__builtin_amdgcn_alignbit(y, y, s.r2) & ~s.m2);
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // quad [1,0,3,2]
  v = (v & s.m1) | (__builtin_amdgcn_alignbit(y, y, s.r1) & ~s.m1);
  return v;
}

// Buffer resources: loads past `bytes` return 0 and stores past it are
// dropped, which predicates them without branches.
constexpr uint32_t kOff = 0x80000000u;  // an offset past every range
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
// cache-policy operand of buffer stores: non-temporal (streaming) access
constexpr int kCacheStream = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float buf_ld_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));  // the bits, not a conversion
}
__device__ __forceinline__ uint32_t buf_ld_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint64_t buf_ld_u64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return ((uint64_t)v.y << 32) | v.x;
}
__device__ __forceinline__ void buf_st_u64(__amdgpu_buffer_rsrc_t r, uint32_t off, uint64_t v) {
  u32x2 w;
  w.x = (uint32_t)v;
  w.y = (uint32_t)(v >> 32);
  __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
}

// Zigzag codes of two blocks packed as 16-bit halves (|q| <= 2047).
typedef short short2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t zigzag_pair(int qa, int qb) {
  const uint32_t p = __builtin_amdgcn_perm((uint32_t)qb, (uint32_t)qa, 0x05040100u);
  const short2v v = __builtin_bit_cast(short2v, p);
  return __builtin_bit_cast(uint32_t, (short2v)((v << (short)1) ^ (v >> (short)15)));
}

// Sums over the wave of RB per-lane values at once (RB = 4, 8 or 16),
// halving the number of registers at each step while the lanes of one
// register come to hold partial sums of different rows.  Afterwards lane L
// holds the sum of row L / (64 / RB).
template <int RB>
__device__ __forceinline__ uint32_t rows_reduce(const uint32_t (&h)[RB], uint32_t lane) {
  uint32_t a[RB / 2], b[RB / 4];
#pragma unroll
  for (int r = 0; r < RB / 2; r++) {  // lanes 0-31: row r, 32-63: row r + RB/2
    const auto p = __builtin_amdgcn_permlane32_swap(h[r], h[r + RB / 2], false, false);
    a[r] = p[0] + p[1];
  }
#pragma unroll
  for (int r = 0; r < RB / 4; r++) {  // 16-lane groups: rows r, r+RB/4, r+RB/2, r+3RB/4
    const auto p = __builtin_amdgcn_permlane16_swap(a[r], a[r + RB / 4], false, false);
    b[r] = p[0] + p[1];
  }
  const bool l8 = lane & 8, l4 = lane & 4;
  auto ror8 = [](uint32_t u) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x128, 0xF, 0xF, false); };
  auto hmirror = [](uint32_t u) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, false); };
  uint32_t v;
  if constexpr (RB == 4) {
    v = b[0] + ror8(b[0]);
    v += hmirror(v);
  } else if constexpr (RB == 8) {  // 8-lane groups
    v = (l8 ? b[1] : b[0]) + ror8(l8 ? b[0] : b[1]);
    v += hmirror(v);
  } else {  // 8-lane groups, then 4-lane groups (partner from the mirrored half-row)
    const uint32_t c0 = (l8 ? b[2] : b[0]) + ror8(l8 ? b[0] : b[2]);
    const uint32_t c1 = (l8 ? b[3] : b[1]) + ror8(l8 ? b[1] : b[3]);
    v = (l4 ? c1 : c0) + hmirror(l4 ? c0 : c1);
  }
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  return v;
}

// v with lane P (an immediate) replaced by the wave-uniform s
template <int P>
__device__ __forceinline__ void put_lane(uint32_t& v, uint32_t s) {
  asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "n"(P));
}

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Stage layout (per tile): plane words [64 rows][C blocks][12 planes] u64
// (only planes below the block width are written), widths [64][C] u8 with
// bit 7 set on blocks holding outliers, outlier masks [64][C] u64 (flagged
// blocks only), hash slot of every row [64] u32.
constexpr uint32_t kStagePlanes = 12;
#ifndef EC_QUANT_PREFETCH
#define EC_QUANT_PREFETCH 0
#endif
constexpr uint8_t kOutlierFlag = 0x80;

// ---------------------------------------------------------------------------
// quantize pass for D = 64*C: codes, row hashes, bit planes and widths of one
// tile, staged in the workspace; the tile's rows go into the segment's hash
// table.  Nothing here waits on another workgroup.
// ---------------------------------------------------------------------------
template <int C>
__global__ void __launch_bounds__(kThreads) ec_quantize_fast(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  constexpr uint32_t kRowsPerWave = kTileRows / (kThreads / 64);  // 16
  constexpr uint32_t kRB = 16 / C;                                 // rows per batch (16 blocks)
  constexpr uint32_t kNB = kRowsPerWave / kRB;                     // batches per wave
  __shared__ EncShared sh;
  __shared__ __align__(4) uint8_t s_oflag[kTileRows][C];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t T = a.sh.T;

  uint32_t my_ticket = blockIdx.x;
  // (D = 256 has no range items: with them compiled in, that instance
  // spilled registers and ran at half speed)
  if constexpr (C < 4) {
    if (a.fuse_range) {  // the same arithmetic in every thread: the branch is uniform
      uint32_t rt = 0, ri = 0;
      my_ticket = fused_item(a, blockIdx.x, rt, ri);
      if (my_ticket == ~0u) {
        range_item(a, rt, ri);
        return;
      }
    }
  }
  if (tid == 0) take_tile(a, sh, my_ticket);
  for (uint32_t e = tid; e < kTileRows * C; e += kThreads) (&s_oflag[0][0])[e] = 0;
  __syncthreads();
  const uint32_t ticket = sh.ticket, s = sh.seg, k = sh.tile, n = sh.n, rows = sh.rows;
  const uint32_t pch = s / T, t = s % T;
  const uint32_t row0 = chunk_row0(a.sh, pch);
  const float* xs = a.x + ((uint64_t)t * a.sh.B + row0) * D;
  const float* xt = xs + (uint64_t)k * kTileRows * D;
  const uint32_t rbeg = wv * kRowsPerWave;
  // with kPrefetch the next batch loads while one is coded (two buffers);
  // without, other resident waves cover the load latency
  constexpr bool kPrefetch = EC_QUANT_PREFETCH;
  float xv[kPrefetch ? 2 : 1][kRB][C];
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xt, n * D * 4);  // rows past n read as 0
  auto load_batch = [&](uint32_t nb, float (&buf)[kRB][C]) {
#pragma unroll
    for (uint32_t rr = 0; rr < kRB; rr++)
#pragma unroll
      for (uint32_t j = 0; j < C; j++)
        buf[rr][j] = buf_ld_f32(rx, ((rbeg + nb * kRB + rr) * D + 64 * j + lane) * 4);
  };
  // the first batch is in flight while wave 0 reduces the range partials
  load_batch(0, xv[0]);
  if (wv == 0) {
    bool v;
    float e = table_eb(a, t, v);
    if (lane == 0) {
      sh.eb = e;
      sh.valid = v;
      if (a.dbg_eb && k == 0) a.dbg_eb[s] = v ? e : 0.0f;
      if (k == 0) a.w.seg_eb[s] = v ? f2u(e) : 0u;  // 0: raw segment
    }
  }
  __syncthreads();
  if (a.w.hhist && k == 0)  // the segment's Huffman histogram starts at zero
    for (uint32_t e = tid; e < kHuffTable; e += kThreads) a.w.hhist[(uint64_t)s * kHuffTable + e] = 0;
  const float eb = sh.eb;
  const float s2 = eb + eb;
  const float r2 = 1.0f / s2;
  const bool valid = sh.valid != 0;
  const uint64_t g0 = ((uint64_t)t * a.sh.B + row0 + (uint64_t)k * kTileRows) * D;
  const bool dbg = a.dbg_codes || a.dbg_outlier;
  if (!valid || n == 0) {
    if (dbg)
      for (uint32_t e = tid; e < n * D; e += kThreads) {
        if (a.dbg_codes) a.dbg_codes[g0 + e] = 0;
        if (a.dbg_outlier) a.dbg_outlier[g0 + e] = 0;
      }
    return;
  }

  const XposeSel xsel = xpose_sel(lane);
  uint32_t hk[C];  // odd 24-bit multipliers per element position
#pragma unroll
  for (uint32_t j = 0; j < C; j++) hk[j] = (fmix32(64 * j + lane + 0x9e3779b9u) & 0xffffffu) | 1u;
  // staging: after the half swap, lane L < 32 holds plane (L & 15) of block
  // A (L < 16) or B as one 64-bit word
  const __amdgpu_buffer_rsrc_t rst =
      buf_rsrc(a.w.stage_pl + (uint64_t)ticket * kTileRows * C * kStagePlanes, kTileRows * C * kStagePlanes * 8);
  // after the half swap of a group's transposes, lane L holds the plane word
  // of block (L >> 3) & 3 of the group, plane (L & 7) + 8 (L >> 5)
  const uint32_t lane_blk = (lane >> 3) & 3u, lane_plane = (lane & 7u) + 8u * (lane >> 5);
  const uint32_t lane_word = lane_blk * kStagePlanes + lane_plane;
  const uint32_t lane_m8 = lane < 32 ? 0xFFu >> (lane & 7u) : 0u;  // planes from the lane's own up
  uint32_t gm_lo = 0, gm_hi = 0;  // lane g: non-zero plane masks of block group g of the wave
  // insertion: lane L < 16 owns the wave's row rbeg + L; its first
  // compare-and-swap is issued as soon as its batch's row hash is known, so
  // that its round trip overlaps the batch's bit planes
  uint64_t* htab = a.w.hash + a.w.hash_off[s];
  const uint32_t cap_mask = (1u << a.w.hash_log2[s]) - 1u;
  uint32_t H = 0;      // the row's hash (tag and first slot)
  uint64_t old0 = 0;   // what the first compare-and-swap found in that slot
  // the wave's first row with the same hash (the row itself when it has
  // none): a later row compares with that row instead of going to the
  // table, so that a hot row costs one table operation per wave, not one
  // per occurrence (atomics on one slot serialize)
  uint32_t lead = lane;
  uint64_t leads = 0;  // wave-uniform: 4 bits per row of the wave, its first row's lane

  static_for<0, (int)kNB>([&](auto nbc) {
    constexpr uint32_t nb = decltype(nbc)::value;
    float (&xb)[kRB][C] = xv[kPrefetch ? (nb & 1) : 0];
    if (kPrefetch && nb + 1 < kNB) load_batch(nb + 1, xv[kPrefetch ? ((nb + 1) & 1) : 0]);
    if (!kPrefetch && nb > 0) load_batch(nb, xv[0]);
    const uint32_t ib = rbeg + nb * kRB;
    int q[kRB][C];
    uint64_t um = 0;
    // q = rint(x / 2eb) via the correctly rounded reciprocal r2: the product
    // tp and fl(x/s) differ by less than 2^-22 |tp|, so when tp is at least
    // 2^-21 |tp| inside a rounding interval (and well inside the code range)
    // rint(tp) = rint(fl(x/s)) and |x - fl(q s)| is strictly below eb: the
    // value is not an outlier.  f = tp - rint(tp) is exact (Sterbenz); NaN or
    // infinite products are unsure.
#pragma unroll
    for (uint32_t rr = 0; rr < kRB; rr++)
#pragma unroll
      for (uint32_t j = 0; j < C; j++) {
        const float tp = xb[rr][j] * r2;
        const float qf = rintf(tp);
        const float f = tp - qf;
        // two ballots of plain compares: the OR of the masks stays scalar
        um |= __ballot(!(fmaf(fabsf(tp), 0x1p-21f, fabsf(f)) < 0.5f));
        um |= __ballot(!(fabsf(tp) < 2046.5f));
        q[rr][j] = (int)qf;
      }
    uint32_t hs[kRB];
#pragma unroll
    for (uint32_t rr = 0; rr < kRB; rr++) hs[rr] = 0;
    if (um) {  // rare: the IEEE division and the reconstruction check decide
      // the batch reloaded (its registers died with the fast pass), every
      // load issued before the first is used
      float xr[kRB][C];
#pragma unroll
      for (uint32_t rr = 0; rr < kRB; rr++)
#pragma unroll
        for (uint32_t j = 0; j < C; j++) xr[rr][j] = buf_ld_f32(rx, ((ib + rr) * D + 64 * j + lane) * 4);
#pragma unroll
      for (uint32_t rr = 0; rr < kRB; rr++) {
        const uint32_t i = ib + rr;
#pragma unroll
        for (uint32_t j = 0; j < C; j++) {
          const float x = xr[rr][j];
          const float tp = x * r2;
          const float f = tp - rintf(tp);
          bool out = false;
          if (i < n && (!(fmaf(fabsf(tp), 0x1p-21f, fabsf(f)) < 0.5f) || !(fabsf(tp) < 2046.5f))) {
            const float tq = x / s2;
            const bool oor = !(fabsf(tq) <= 2047.0f);
            const float qf = rintf(tq);
            const float err = x - qf * s2;
            out = oor || !(fabsf(err) <= eb);
            q[rr][j] = out ? 0 : (int)qf;
            if (out) hs[rr] += (f2u(x) ^ 0x7f4a7c15u) * 0x85ebca6bu + hk[j];  // raw bits
          }
          const uint64_t om = __ballot(out);
          if (om) {
            if (lane == 0) {
              a.w.stage_om[((uint64_t)ticket * kTileRows + i) * C + j] = om;
              s_oflag[i][j] = kOutlierFlag;
            }
            if (a.dbg_outlier && i < n) a.dbg_outlier[g0 + (uint64_t)i * D + 64 * j + lane] = (om >> lane) & 1ull;
          }
        }
      }
    }
    // row hashes: position-weighted sums of the codes
#pragma unroll
    for (uint32_t rr = 0; rr < kRB; rr++)
#pragma unroll
      for (uint32_t j = 0; j < C; j++) hs[rr] += __umul24((uint32_t)q[rr][j], hk[j]);
    if (a.w.stage_sym) {  // Huffman segments: every row's symbols q + 2047 (outliers 2047)
      uint16_t* sy = a.w.stage_sym + (uint64_t)ticket * kTileRows * D;
#pragma unroll
      for (uint32_t rr = 0; rr < kRB; rr++)
#pragma unroll
        for (uint32_t j = 0; j < C; j++) sy[(ib + rr) * D + 64 * j + lane] = (uint16_t)(q[rr][j] + 2047);
    }
    if (dbg) {  // tests only
#pragma unroll
      for (uint32_t rr = 0; rr < kRB; rr++) {
        const uint32_t i = ib + rr;
        if (i >= n) continue;
#pragma unroll
        for (uint32_t j = 0; j < C; j++) {
          const uint64_t e = g0 + (uint64_t)i * D + 64 * j + lane;
          if (a.dbg_codes) a.dbg_codes[e] = q[rr][j];
          if (a.dbg_outlier && !s_oflag[i][j]) a.dbg_outlier[e] = 0;
        }
      }
    }
    {  // the batch's row hashes to their owner lanes nb kRB .. nb kRB + kRB - 1
      const uint32_t hv = rows_reduce<kRB>(hs, lane);
      const uint32_t h = fmix32(__shfl(hv, (int)(((lane - nb * kRB) % kRB) * (64 / kRB))));
      if (lane >= nb * kRB && lane < nb * kRB + kRB) H = h & (uint32_t)a.hash_keep;
      if (!a.window) {
        // first lane (row) of the wave so far with the hash of each row of the
        // batch, gathered in scalar registers
#pragma unroll
        for (uint32_t rr = 0; rr < kRB; rr++) {
          const uint32_t ol = nb * kRB + rr;
          const uint32_t hr = __builtin_amdgcn_readlane(H, ol);
          const uint64_t m = __ballot(H == hr) & ((2ull << ol) - 1ull);
          leads |= (uint64_t)__builtin_ctzll(m) << (4 * ol);
        }
        lead = lane < kRowsPerWave ? (uint32_t)(leads >> (4 * lane)) & 15u : lane;
        if (lane >= nb * kRB && lane < nb * kRB + kRB) {
          const uint32_t i = rbeg + lane;
          if (i < n)
            old0 = lead != lane
                       // a hit on the earlier row, taken without a table operation
                       ? ((uint64_t)H << 32) | (uint64_t)(k * kTileRows + rbeg + lead + 1)
                       : atomicCAS((unsigned long long*)&htab[H & cap_mask], 0ull,
                                   (unsigned long long)(((uint64_t)H << 32) | (uint64_t)(k * kTileRows + i + 1)));
        }
      }
    }
    // bit planes, four blocks at a time (blocks 4g .. 4g+3 of the batch, in
    // (row, block) order): the low bytes of a lane's four zigzag codes go
    // through one 32x32 bit transpose per half-wave, so that lane L holds
    // half L >> 5 of plane L & 7 of block (L >> 3) & 3; the high bits
    // (planes 8-11) take a second transpose only when a block needs them
    static_for<0, 4>([&](auto gc) {
      constexpr uint32_t g = decltype(gc)::value;
      constexpr uint32_t b0 = 4 * g;
      const uint32_t p01 = zigzag_pair(q[b0 / C][b0 % C], q[(b0 + 1) / C][(b0 + 1) % C]);
      const uint32_t p23 = zigzag_pair(q[(b0 + 2) / C][(b0 + 2) % C], q[(b0 + 3) / C][(b0 + 3) % C]);
      const uint32_t lo = __builtin_amdgcn_perm(p23, p01, 0x06040200u);  // low bytes of codes 0..3
      const uint32_t hi = __builtin_amdgcn_perm(p23, p01, 0x07050301u);  // high bytes (< 16)
      const uint32_t ylo = xpose32(lo, xsel);
      const uint64_t nlo = __ballot(ylo != 0);
      const uint32_t mlo = (uint32_t)nlo | (uint32_t)(nlo >> 32);  // bit 8k + p: plane p of block k
      uint32_t yhi = 0, mhi = 0;
      uint32_t above;  // non-zero planes of the lane's block from the lane's plane up
      if (__ballot(hi != 0)) {
        yhi = xpose32(hi, xsel);
        const uint64_t nhi = __ballot(yhi != 0);
        mhi = (uint32_t)nhi | (uint32_t)(nhi >> 32);  // bit 8k + p: plane 8 + p of block k
        above = (__builtin_amdgcn_ubfe(mlo, 8 * lane_blk, 8) | (__builtin_amdgcn_ubfe(mhi, 8 * lane_blk, 4) << 8)) >>
                lane_plane;
      } else {
        above = (mlo >> (lane & 31u)) & lane_m8;
      }
      put_lane<nb * 4 + g>(gm_lo, __builtin_amdgcn_readfirstlane(mlo));
      put_lane<nb * 4 + g>(gm_hi, __builtin_amdgcn_readfirstlane(mhi));
      // lanes 0-31: planes 0-7 of the four blocks, lanes 32-63: planes 8-15;
      // a plane is staged when it is below its block's width
      const auto hw = __builtin_amdgcn_permlane32_swap(ylo, yhi, false, false);
      const uint64_t word = ((uint64_t)hw[1] << 32) | hw[0];
      buf_st_u64(rst, above ? ((ib * C + b0) * kStagePlanes + lane_word) * 8 : kOff, word);
    });
  });
  // widths of the wave's blocks with their outlier flags, lane-parallel:
  // lane g < 4 kNB holds block group g (blocks 4g .. 4g+3 of the wave)
  if (lane < 4 * kNB) {
    uint32_t wp = 0;  // the group's widths, a byte each
#pragma unroll
    for (uint32_t k = 0; k < 4; k++) {
      const uint32_t bl = (gm_lo >> (8 * k)) & 0xFFu, bh = (gm_hi >> (8 * k)) & 0xFu;
      wp |= (bh ? 40u - __clz(bh) : (bl ? 32u - __clz(bl) : 0u)) << (8 * k);
    }
    const uint32_t bw = rbeg * C + 4 * lane;  // first block of the group in the tile
    const uint32_t of = *reinterpret_cast<const uint32_t*>(&s_oflag[0][0] + bw);
    *reinterpret_cast<uint32_t*>(a.w.stage_w + (uint64_t)ticket * kTileRows * C + bw) = wp | of;
  }

  // ---- insert: each wave owns 16 rows (lanes 0..15); compares use the wave ----
  // (windowed references: no table, the window pass reads the row hashes)
  const uint32_t i = rbeg + lane;
  bool active = lane < kRowsPerWave && i < n && !a.window;
  bool first = true;  // the first attempt's result is old0
  bool at_lead = lead != lane;  // old0 names the wave's earlier row with the hash
  bool via_lead = false;        // equal to that row: its slot is this row's
  uint32_t slot = H & cap_mask;
  const uint64_t mine = ((uint64_t)H << 32) | (uint64_t)(k * kTileRows + i + 1);
  uint32_t guard = 0;
  uint32_t seen = 0;  // the row (+ 1) of the slot value a tag hit was found in
  while (__ballot(active) != 0) {
    bool need = false;
    uint32_t cand = 0;
    if (active) {
      const uint64_t old =
          first ? old0 : atomicCAS((unsigned long long*)&htab[slot], 0ull, (unsigned long long)mine);
      first = false;
      if (old == 0) {
        active = false;
      } else if ((uint32_t)(old >> 32) == H && (uint32_t)old - 1u < rows) {
        need = true;
        cand = (uint32_t)old - 1u;
        seen = (uint32_t)old;
      } else {
        slot = (slot + 1) & cap_mask;
      }
    }
    // tag hits, kCmp at a time with all their row loads in flight together:
    // equal rows keep the smaller row in the slot (the slot is read by the
    // next launch only, so the minimum need not be awaited)
    constexpr int kCmp = C >= 4 ? 2 : 8 / C;
    uint64_t m = __ballot(need);
    while (m) {
      int Lk[kCmp];
      float va[kCmp][C], vb[kCmp][C];
#pragma unroll
      for (int kk = 0; kk < kCmp; kk++) {
        Lk[kk] = m ? __ffsll((long long)m) - 1 : -1;
        m &= m - 1;
        const int Ls = Lk[kk] < 0 ? Lk[0] : Lk[kk];  // no candidate: a copy of the first
        const uint32_t iL = __shfl(i, Ls), cL = __shfl(cand, Ls);
#pragma unroll
        for (int j = 0; j < C; j++) {
          va[kk][j] = xs[(uint64_t)cL * D + 64 * j + lane];
          vb[kk][j] = xt[(uint64_t)iL * D + 64 * j + lane];
        }
      }
#pragma unroll
      for (int kk = 0; kk < kCmp; kk++) {
        if (Lk[kk] < 0) continue;
        bool raw = true;
#pragma unroll
        for (int j = 0; j < C; j++) raw = raw && f2u(va[kk][j]) == f2u(vb[kk][j]);
        bool eq = __all(raw);
        if (!eq) {  // different bits: the same codes and outliers make the rows equal
          bool e = true;
#pragma unroll
          for (int j = 0; j < C; j++) {
            int qa, qb;
            const bool oa = quantize_fast(va[kk][j], eb, s2, r2, qa);
            const bool ob = quantize_fast(vb[kk][j], eb, s2, r2, qb);
            e = e && oa == ob && (oa ? f2u(va[kk][j]) == f2u(vb[kk][j]) : qa == qb);
          }
          eq = __all(e);
        }
        if ((int)lane == Lk[kk]) {
          if (eq) {
            // the smaller row is the first occurrence; the slot only ever
            // decreases from the value seen, so a larger row needs no update
            // (a row equal to the wave's earlier row is never the smaller)
            if ((uint32_t)mine < seen)
              __hip_atomic_fetch_min(&htab[slot], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            active = false;
            via_lead = at_lead;
          } else if (!at_lead) {
            slot = (slot + 1) & cap_mask;
          }
          // an earlier row of the wave with the same hash but another key:
          // the row goes to the table from its first slot
          at_lead = false;
        }
      }
    }
    if (++guard > cap_mask + 3) {  // cannot happen: the table is at most a quarter full
      if (active) {
        report_error(a.report, kDevErrTimeout);
        active = false;
      }
    }
  }
  // a row equal to the wave's earlier row lives in that row's slot (which is
  // final: every lane has left the loop)
  const uint32_t fslot = (uint32_t)__shfl((int)slot, (int)(via_lead ? lead : lane));
  if (lane < kRowsPerWave && i < n) a.w.stage_slot[(uint64_t)ticket * kTileRows + i] = a.window ? H : fslot;
}

// ---------------------------------------------------------------------------
// assembly for D = 64*C, after every row is in the hash table, in three
// launches that never wait on one another's workgroups:
//   size   two tiles per wave: first occurrences, record layout and size,
//          added into a sum per workgroup (8 tiles)
//   write  one workgroup per tile: its offset from those sums, the record, the
//          tile's directory entry and, from first tiles, the segment and
//          stream headers and tables
// ---------------------------------------------------------------------------
struct TileCoord {
  uint32_t s, k, rows, ntiles, n, pch, t;
};
__device__ __forceinline__ TileCoord tile_coord(const EncArgs& a, uint32_t ticket) {
  TileCoord c;
  if (a.sh.tiles_per_seg) {
    c.s = ticket / a.sh.tiles_per_seg;
    c.k = ticket - c.s * a.sh.tiles_per_seg;
  } else {
    c.s = find_segment(a.w.seg_tile_base, a.sh.nseg, ticket);
    c.k = ticket - a.w.seg_tile_base[c.s];
  }
  c.pch = c.s / a.sh.T;
  c.t = c.s % a.sh.T;
  const uint32_t r0 = chunk_row0(a.sh, c.pch);
  c.rows = chunk_row0(a.sh, c.pch + 1) - r0;
  c.ntiles = (c.rows + kTileRows - 1) / kTileRows;
  c.n = c.ntiles ? min(kTileRows, c.rows - c.k * kTileRows) : 0;
  return c;
}

// Record layout of a tile (same rules as size_record).
struct RecLayout {
  uint32_t mode, off_refs, off_opos, off_oval, off_pl;
  uint64_t rec;  // record bytes
};
// Bytes of one reference: a u8 distance with windowed references, else the
// referenced row as u16 (segments up to 65536 rows) or u32.
__device__ __forceinline__ uint32_t ref_bytes(uint32_t rows, uint32_t window) {
  return window ? 1u : (rows <= 65536 ? 2u : 4u);
}

__device__ __forceinline__ RecLayout rec_layout(uint32_t n, uint32_t U, uint32_t nblk, uint32_t sumw,
                                                uint32_t nout, uint32_t rows, uint32_t D, bool valid,
                                                uint32_t window) {
  RecLayout L;
  const uint32_t rb = ref_bytes(rows, window);
  L.off_refs = (uint32_t)align_up(16 + nblk, 4);
  L.off_opos = (uint32_t)align_up(L.off_refs + rb * (n - U), 4);
  L.off_oval = L.off_opos + 4 * nout;
  L.off_pl = (uint32_t)align_up(L.off_oval + 4 * nout, 8);
  const uint64_t bp = align_up(L.off_pl + 8ull * sumw, 16);
  const uint64_t raw = 16 + align_up(4ull * n * D, 16);
  L.mode = (valid && bp < raw) ? 1u : 0u;
  L.rec = n ? (L.mode ? bp : raw) : 0;
  return L;
}

__device__ __forceinline__ uint64_t seg_prefix_bytes(uint32_t ntiles) { return 32 + align_up(4ull * ntiles, 16); }

// Size pass: one workgroup per block of kBlockTiles tiles, EC_SIZE_Q tiles per
// wave (their loads are issued together); the block's item sum is stored once.
#ifndef EC_SIZE_Q
#define EC_SIZE_Q 2
#endif
constexpr uint32_t kSizeThreads = 256;
constexpr uint32_t kTilesPerWave = EC_SIZE_Q;
constexpr uint32_t kBlockTiles = kTilesPerWave * (kSizeThreads / 64);  // tiles per size workgroup
template <int C>
__global__ void __launch_bounds__(kSizeThreads) ec_size_fast(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  constexpr uint32_t Q = kTilesPerWave;
  __shared__ uint64_t s_sum[kSizeThreads / 64];
  const uint32_t lane = threadIdx.x & 63, wv = wave_id();
  const uint32_t t0 = blockIdx.x * kBlockTiles + wv * Q;
  TileCoord c[Q];
  uint32_t slot[Q];
  uint8_t wb[Q][C];
#pragma unroll
  for (uint32_t q = 0; q < Q; q++) {
    const uint32_t ticket = min(t0 + q, a.sh.ntiles - 1);  // past the end: a copy, unused
    c[q] = tile_coord(a, ticket);
    // staged slot and widths (garbage when the segment is stored raw, then unused)
    const uint64_t rowi = (uint64_t)ticket * kTileRows + lane;
    slot[q] = a.w.stage_slot[rowi];
#pragma unroll
    for (uint32_t j = 0; j < C; j++) wb[q][j] = a.w.stage_w[rowi * C + j];
  }
  // the segment's error bound, stored by its first quantize tile (0: raw)
  bool valid[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; q++) valid[q] = a.w.seg_eb[c[q].s] != 0u;
  uint32_t first[Q];
#pragma unroll
  for (uint32_t q = 0; q < Q; q++) {
    first[q] = c[q].k * kTileRows + lane;
    if (valid[q] && lane < c[q].n) {
      if (a.window) {  // the match found by the window pass
        first[q] = a.w.tile_first[(uint64_t)min(t0 + q, a.sh.ntiles - 1) * kTileRows + lane];
      } else {
        const uint32_t cap_mask = (1u << a.w.hash_log2[c[q].s]) - 1u;
        first[q] = (uint32_t)ld64(&a.w.hash[a.w.hash_off[c[q].s] + (slot[q] & cap_mask)]) - 1u;
      }
    }
  }
  uint64_t items = 0;
#pragma unroll
  for (uint32_t q = 0; q < Q; q++) {
    const uint32_t ticket = t0 + q;
    if (ticket >= a.sh.ntiles) continue;  // (no early exit: the loop must unroll)
    const TileCoord& cq = c[q];
    const uint64_t rowi = (uint64_t)ticket * kTileRows + lane;
    const bool inrow = lane < cq.n;
    const bool uniq = valid[q] && inrow && first[q] == cq.k * kTileRows + lane;
    const uint64_t bm = __ballot(uniq);
    uint32_t rw = 0, ro = 0;
    if (uniq) {
#pragma unroll
      for (uint32_t j = 0; j < C; j++) {
        rw += wb[q][j] & 0x7Fu;
        if (wb[q][j] & kOutlierFlag) ro += (uint32_t)__popcll(a.w.stage_om[rowi * C + j]);
      }
    }
    const uint32_t sumw = wave_sum_u32(rw), nout = wave_sum_u32(ro);
    const uint32_t U = (uint32_t)__popcll(bm);
    const RecLayout L = rec_layout(cq.n, U, U * C, sumw, nout, cq.rows, D, valid[q], a.window);
    if (inrow) a.w.tile_first[rowi] = first[q];
    if (a.dbg_first && inrow)
      a.dbg_first[(uint64_t)cq.t * a.sh.B + chunk_row0(a.sh, cq.pch) + cq.k * kTileRows + lane] = first[q];
    const uint64_t pre =
        cq.k == 0 ? seg_prefix_bytes(cq.ntiles) + (cq.t == 0 ? align_up(8ull * a.sh.T, 16) : 0) : 0;
    const uint64_t item = L.rec + pre;
    items += item;
    if (lane == 0) {
      a.w.tile_status[ticket] = item;
      uint4 info;
      info.x = U;
      info.y = L.mode ? nout : 0u;
      info.z = sumw;
      info.w = L.mode | (valid[q] ? 0x100u : 0u);
      reinterpret_cast<uint4*>(a.w.tile_info)[ticket] = info;
      a.w.tile_bitmap[ticket] = bm;
      a.w.tile_nout[ticket] = nout;  // the outliers of its first occurrences, however stored
    }
  }
  if (lane == 0) s_sum[wv] = items;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t sum = 0;
    for (uint32_t w = 0; w < kSizeThreads / 64; w++) sum += s_sum[w];
    a.w.block_status[blockIdx.x] = sum;
  }
}

// Stream bytes before tile j (its item included for no earlier tile), whole
// wave: the sums of the size workgroups' blocks before j's block plus the
// items of the tiles before j in its block, lane-parallel.
__device__ __forceinline__ uint64_t tiles_before(const EncArgs& a, uint32_t j) {
  static_assert(kBlockTiles <= 64, "one lane per tile of a block");
  const uint32_t lane = threadIdx.x & 63, blk = j / kBlockTiles, in = j - blk * kBlockTiles;
  uint64_t v = lane < in ? a.w.tile_status[blk * kBlockTiles + lane] : 0;
  // the block sums before j's block: eight loads per lane issued together
  // (one round trip up to 512 blocks, not one per 64)
  for (uint32_t b0 = 0; b0 < blk; b0 += 8 * 64) {
    uint64_t u[8];
#pragma unroll
    for (uint32_t q = 0; q < 8; q++) {
      const uint32_t b = b0 + 64 * q + lane;
      u[q] = b < blk ? a.w.block_status[b] : 0ull;
    }
#pragma unroll
    for (uint32_t q = 0; q < 8; q++) v += u[q];
  }
  return wave_sum_u64(v);
}

// The tile's entry in its segment's tile directory; a segment's first tile
// also writes the segment header, the directory pad and the segment's entry in
// its chunk table; the stream's first tile writes the chunk byte counts and the
// stream header.  Whole workgroup.  ss: segment start, se: segment end, cs:
// start of the segment's chunk, un: the segment's U and n_out.
// Bytes of the codebook at b (u16 lowest, u16 highest symbol, 4-bit lengths).
__device__ __forceinline__ uint32_t book_bytes(const uint8_t* b) {
  const uint32_t lo = b[0] | (uint32_t)b[1] << 8, hi = b[2] | (uint32_t)b[3] << 8;
  return hi < lo ? 4u : 4u + (hi - lo + 2) / 2;
}

__device__ void write_stream_tables(const EncArgs& a, const TileCoord& c, uint32_t ticket,
                                    uint64_t rec_abs, uint64_t ss, uint64_t se, uint64_t cs,
                                    const uint32_t* un, uint64_t total, bool huff) {
  const uint32_t tid = threadIdx.x, T = a.sh.T, P = a.sh.P;
  if (c.ntiles && tid == 0) reinterpret_cast<uint32_t*>(a.out + ss + 32)[c.k] = (uint32_t)(rec_abs - ss);
  if (c.k == 0) {
    uint8_t* sg = a.out + ss;
    const uint32_t dend = 32 + 4 * c.ntiles, dpad = (uint32_t)align_up(dend, 16) - dend;
    if (tid < dpad) sg[dend + tid] = 0;
    if (huff) {  // the codebook after the tile directory, zero-padded to 16
      const uint8_t* bk = a.w.hbooks + (uint64_t)c.s * kBookStride;
      const uint32_t nb = book_bytes(bk), at = dend + dpad, pad = (uint32_t)align_up(nb, 16);
      for (uint32_t i = tid; i < pad; i += kThreads) sg[at + i] = i < nb ? bk[i] : (uint8_t)0;
    }
    if (tid == 0) {
      const uint32_t ebw = a.w.seg_eb[c.s];
      uint32_t* h = reinterpret_cast<uint32_t*>(sg);
      h[0] = c.rows;
      h[1] = c.ntiles;
      h[2] = ebw;
      h[3] = ebw ? ((huff ? 3u : 1u) | (a.window ? 4u | (a.window << 8) : 0u)) : 0u;
      h[4] = un[0];
      h[5] = un[1];
      reinterpret_cast<uint64_t*>(sg)[3] = se - ss;
      reinterpret_cast<uint64_t*>(a.out + cs)[c.t] = ss - cs;
      if (c.t == T - 1 && (T & 1u)) reinterpret_cast<uint64_t*>(a.out + cs)[T] = 0;  // table pad
      if (a.report) a.report->seg_bytes[c.s] = se - ss;
      if (a.seg_meta) {
        a.seg_meta[2 * c.s] = un[0];
        a.seg_meta[2 * c.s + 1] = ebw ? 1u : 0u;
      }
      if (c.t == T - 1) reinterpret_cast<uint64_t*>(a.out + 64)[c.pch] = se - cs;  // chunk bytes
    }
  }
  if (ticket == 0 && tid == 0) {
    if (P & 1u) reinterpret_cast<uint64_t*>(a.out + 64)[P] = 0;
    uint32_t* h = reinterpret_cast<uint32_t*>(a.out);
    h[0] = kMagic;
    h[1] = kVersion | (a.coder << 16);
    h[2] = T;
    h[3] = a.sh.B;
    h[4] = a.sh.D;
    h[5] = P;
    h[6] = kTileRows;
    h[7] = a.eb_mode;
    uint64_t* h64 = reinterpret_cast<uint64_t*>(a.out);
    h64[4] = (uint64_t)a.iter;
    h64[5] = 4ull * T * a.sh.B * a.sh.D;
    h64[6] = total;
    h64[7] = 0;
    if (a.report) a.report->total_bytes = total;
  }
}

// D <= 128: eight waves per SIMD, at most 64 VGPRs (the kernel waits on memory,
// not ALUs; D = 256 would spill)
template <int C>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(C < 4 ? 8 : 1)))
ec_write_fast(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  __shared__ uint64_t s_omask[kTileRows][C];
  __shared__ uint32_t s_cbase[kTileRows][C];  // plane-word offset of each block in the record
  __shared__ uint32_t s_first[kTileRows], s_obase[kTileRows];
  __shared__ uint8_t s_w[kTileRows][C];
  __shared__ uint8_t s_urow[kTileRows];
  __shared__ uint64_t s_rec_abs, s_seg_start, s_seg_end, s_chunk_start, s_total, s_bitmap;
  __shared__ uint32_t s_un[2];
  __shared__ uint4 s_info;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x;
  if (a.fuse_range && tid == 0)  // the quantize pass is done with the range items' words
    for (uint32_t j = ticket; j < a.sh.T * a.range_items; j += a.sh.ntiles) a.w.range_slot[j] = 0;
  const TileCoord c = tile_coord(a, ticket);
  const uint32_t n = c.n;
  // a Huffman segment: its codebook follows the tile directory
  const bool huff = a.w.seg_coder && a.w.seg_coder[c.s] != 0;
  const uint32_t bookpad = huff ? (uint32_t)align_up(book_bytes(a.w.hbooks + (uint64_t)c.s * kBookStride), 16) : 0u;
  const float* xt = a.x + ((uint64_t)c.t * a.sh.B + chunk_row0(a.sh, c.pch) + (uint64_t)c.k * kTileRows) * D;
  // every staged plane word of the tile is requested before the metadata
  // (words above a block's width are loaded and then dropped)
  const __amdgpu_buffer_rsrc_t rsrc =
      buf_rsrc(a.w.stage_pl + (uint64_t)ticket * kTileRows * C * kStagePlanes, n * C * kStagePlanes * 8);
  constexpr uint32_t kPass = kTileRows * C / (kThreads / 16);
  const uint32_t b = tid & 15u;
  uint64_t wv_[kPass];
#pragma unroll
  for (uint32_t ps = 0; ps < kPass; ps++) {
    const uint32_t blk = ps * (kThreads / 16) + (tid >> 4);
    wv_[ps] = buf_ld_u64(rsrc, b < kStagePlanes ? (blk * kStagePlanes + b) * 8 : kOff);
  }
  if (wv == 0) {
    const uint64_t rowi = (uint64_t)ticket * kTileRows + lane;
    const uint64_t bitmap = a.w.tile_bitmap[ticket];
    const uint4 info = reinterpret_cast<const uint4*>(a.w.tile_info)[ticket];
    uint8_t wb[C];
#pragma unroll
    for (uint32_t j = 0; j < C; j++) wb[j] = a.w.stage_w[rowi * C + j];
    const uint32_t first = a.w.tile_first[rowi];
    const bool uniq = (bitmap >> lane) & 1ull;
    // the hash slot of a first occurrence goes back to zero (read by the size
    // pass, which is done): every slot in use belongs to exactly one first
    // occurrence, so the tables are clear for the next call
    if (uniq && !a.window) {
      const uint32_t cap_mask = (1u << a.w.hash_log2[c.s]) - 1u;
      a.w.hash[a.w.hash_off[c.s] + (a.w.stage_slot[rowi] & cap_mask)] = 0ull;
    }
    uint32_t rw = 0, ro = 0;
#pragma unroll
    for (uint32_t j = 0; j < C; j++) {
      const uint32_t w = uniq ? wb[j] & 0x7Fu : 0u;
      const uint64_t om = (uniq && (wb[j] & kOutlierFlag)) ? a.w.stage_om[rowi * C + j] : 0ull;
      s_omask[lane][j] = om;
      s_w[lane][j] = (uint8_t)w;
      rw += w;
      ro += (uint32_t)__popcll(om);
    }
    const uint32_t iw = wave_incl_u32(rw), io = wave_incl_u32(ro);  // inclusive scans over lanes
    uint32_t cb = iw - rw;
#pragma unroll
    for (uint32_t j = 0; j < C; j++) {
      s_cbase[lane][j] = cb;
      cb += s_w[lane][j];
    }
    s_obase[lane] = io - ro;
    s_first[lane] = first;
    if (uniq) s_urow[__popcll(bitmap & lanes_below())] = (uint8_t)lane;
    if (lane == 0) {
      s_bitmap = bitmap;
      s_info = info;
    }
  } else if (wv == 1) {  // the tile's and its segment's places in the stream
    const uint64_t before = tiles_before(a, ticket), seg_before = tiles_before(a, ticket - c.k);
    if (lane == 0) {
      const uint64_t chunk_prefix = c.t == 0 ? align_up(8ull * a.sh.T, 16) : 0;
      const uint64_t ss = a.sh.base_bytes + seg_before + chunk_prefix;
      s_seg_start = ss;
      s_rec_abs = c.k == 0 ? ss + seg_prefix_bytes(c.ntiles) + bookpad : a.sh.base_bytes + before;
    }
  } else if (wv == 2 && c.k == 0) {  // the segment's end and its chunk's start
    const uint32_t sched = c.ntiles ? c.ntiles : 1u;
    const uint64_t next = tiles_before(a, ticket + sched);
    const uint64_t cfirst = c.t == 0 ? 0 : tiles_before(a, a.w.seg_tile_base[c.pch * a.sh.T]);
    if (lane == 0) {
      s_seg_end = a.sh.base_bytes + next;
      s_chunk_start = a.sh.base_bytes + cfirst;
    }
  } else if (wv == 3 && c.k == 0) {  // the segment's U and n_out; the stream's size
    const uint32_t sched = c.ntiles ? c.ntiles : 1u;
    uint32_t u = 0, o = 0;
    for (uint32_t j = lane; j < sched; j += 64) {
      u += a.w.tile_info[4 * (ticket + j)];
      o += a.w.tile_info[4 * (ticket + j) + 1];
    }
    u = wave_sum_u32(u);
    o = wave_sum_u32(o);
    const uint64_t all = ticket == 0 ? tiles_before(a, a.sh.ntiles) : 0;
    if (lane == 0) {
      s_un[0] = u;
      s_un[1] = o;
      s_total = a.sh.base_bytes + all;
    }
  }
  __syncthreads();
  if (c.k == 0) {
    const uint64_t cs = c.t == 0 ? s_seg_start - align_up(8ull * a.sh.T, 16) : s_chunk_start;
    if (s_seg_end > a.out_cap) {  // cannot happen when out_cap >= the maximum stream size
      if (tid == 0) report_error(a.report, kDevErrTimeout);
      return;
    }
    write_stream_tables(a, c, ticket, s_rec_abs, s_seg_start, s_seg_end, cs, s_un, s_total, huff);
  } else {
    write_stream_tables(a, c, ticket, s_rec_abs, s_seg_start, 0, 0, s_un, 0, huff);
  }
  if (n == 0) return;
  const uint4 info = s_info;
  const uint32_t U = info.x, nout = info.y, sumw = info.z, mode = info.w & 0xFFu;
  const bool valid = (info.w >> 8) & 1u;
  const uint64_t bitmap = s_bitmap;
  const RecLayout L = rec_layout(n, U, U * C, sumw, mode ? nout : 0u, c.rows, D, valid, a.window);
  const uint64_t rec_bytes = mode == 2 ? a.w.tile_hsize[ticket] : L.rec;
  if (s_rec_abs + rec_bytes > a.out_cap) {  // cannot happen when out_cap >= the maximum stream size
    if (tid == 0) report_error(a.report, kDevErrTimeout);
    return;
  }
  uint8_t* rec = a.out + s_rec_abs;
  if (tid == 0) {
    const uint64_t w1 = (uint64_t)(mode ? nout : 0u) | ((uint64_t)U << 32) | ((uint64_t)mode << 48);
    reinterpret_cast<uint64_t*>(rec)[0] = bitmap;
    reinterpret_cast<uint64_t*>(rec)[1] = w1;
  }
  if (mode == 0) {
    write_raw_rows(rec, xt, n * D, D);
    return;
  }
  const uint32_t nblk = U * C;
  const uint32_t rb = ref_bytes(c.rows, a.window);
  // a Huffman record has no widths: its references start right after the header
  const uint32_t off_refs = mode == 2 ? 16u : L.off_refs;
  const uint32_t off_opos = mode == 2 ? (uint32_t)align_up(16 + rb * (n - U), 4) : L.off_opos;
  const uint32_t off_oval = off_opos + 4 * nout;
  if (mode == 1) {
    for (uint32_t b = tid; b < nblk; b += kThreads) rec[16 + b] = s_w[s_urow[b / C]][b % C];
    for (uint32_t b = nblk + tid; b < L.off_refs - 16; b += kThreads) rec[16 + b] = 0;
  }
  if (tid < n && !((bitmap >> tid) & 1ull)) {
    const uint32_t j = tid - (uint32_t)__popcll(bitmap & ((1ull << tid) - 1ull));
    if (rb == 1) rec[off_refs + j] = (uint8_t)(c.k * kTileRows + tid - s_first[tid]);  // distance
    else if (rb == 2) reinterpret_cast<uint16_t*>(rec + off_refs)[j] = (uint16_t)s_first[tid];
    else reinterpret_cast<uint32_t*>(rec + off_refs)[j] = s_first[tid];
  }
  {
    const uint32_t rend = off_refs + rb * (n - U);
    if (tid < off_opos - rend) rec[rend + tid] = 0;
  }
  if (mode == 1) {
    const uint32_t oend = L.off_oval + 4 * nout;
    if (tid < L.off_pl - oend) rec[oend + tid] = 0;
    const uint64_t pend = L.off_pl + 8ull * sumw;
    if (tid < L.rec - pend) rec[pend + tid] = 0;
  }
  if (mode == 1) {
    // staged plane words (loaded above): 16 lanes per block, lane = plane
    const __amdgpu_buffer_rsrc_t rdst = buf_rsrc(rec + L.off_pl, sumw * 8);
#pragma unroll
    for (uint32_t ps = 0; ps < kPass; ps++) {
      const uint32_t blk = ps * (kThreads / 16) + (tid >> 4), row = blk / C, j = blk % C;
      const bool use = blk < n * C && ((bitmap >> row) & 1ull) && b < s_w[row][j];
      buf_st_u64(rdst, use ? (s_cbase[row][j] + b) * 8 : kOff, wv_[ps]);
    }
  } else if (tid == 0) {
    a.w.tile_rec[ticket] = s_rec_abs + 1;  // the chunk table and words: ec_write_huff
  }
  if (nout) {
    uint32_t* opos = reinterpret_cast<uint32_t*>(rec + off_opos);
    uint32_t* oval = reinterpret_cast<uint32_t*>(rec + off_oval);
    for (uint32_t u = wv; u < U; u += kThreads / 64) {
      const uint32_t i = s_urow[u];
      uint32_t ob = s_obase[i];
#pragma unroll
      for (uint32_t j = 0; j < C; j++) {
        const uint64_t om = s_omask[i][j];
        if (om) {
          if ((om >> lane) & 1ull) {
            const uint32_t o = ob + (uint32_t)__popcll(om & lanes_below());
            opos[o] = u * D + 64 * j + lane;
            oval[o] = f2u(xt[(uint64_t)i * D + 64 * j + lane]);
          }
          ob += (uint32_t)__popcll(om);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Huffman segments: the entropy coder of section III-D ("Huffman Encoding")
// as a coder of whole segments of the stream, for D = 64*C.  After the size
// pass (first occurrences known), five launches:
//   hist    per tile: LDS histogram of the symbols q + 2047 of its
//           first-occurrence rows, merged into the segment's histogram
//   books   per segment: the Huffman coder's codebook builder (ec_huffman.hip)
//   hsize   per tile: the bytes of its Huffman record
//   choose  per segment: Huffman or bit planes (the plan's coder, sizes)
//   items   per size block: every tile's stream item and the block's sum again
// and after the write pass, for every Huffman record, its chunk table and
// words.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wave 0 of a workgroup: the tile's first-occurrence rows in order.
__device__ __forceinline__ void unique_rows(uint64_t bm, uint8_t* urow) {
  const uint32_t lane = threadIdx.x & 63;
  if ((bm >> lane) & 1ull) urow[__popcll(bm & lanes_below())] = (uint8_t)lane;
}

template <int C>
__global__ void __launch_bounds__(kThreads) ec_hist_tiles(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  __shared__ uint32_t h[kHuffTable];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x;
  if (ticket == 0 && tid == 0) a.w.hstat[0] = 0;  // the codebook builder's status
  const TileCoord c = tile_coord(a, ticket);
  if (c.n == 0 || a.w.seg_eb[c.s] == 0) return;
  for (uint32_t i = tid; i < kHuffTable; i += kThreads) h[i] = 0;
  const uint64_t bm = a.w.tile_bitmap[ticket];
  const uint16_t* sy = a.w.stage_sym + (uint64_t)ticket * kTileRows * D;
  // the symbols of the wave's rows (every staged row has them), loaded
  // eight rows at a time with all their loads in flight
  constexpr uint32_t kRowsPerWave = kTileRows / (kThreads / 64), kBatch = 8;
  uint32_t v[kRowsPerWave][C];
#pragma unroll
  for (uint32_t r = 0; r < kBatch; r++)
#pragma unroll
    for (uint32_t j = 0; j < C; j++) {
      const uint32_t i = wv + (kThreads / 64) * r;
      v[r][j] = i < c.n ? sy[i * D + 64 * j + lane] : 0u;
    }
  __syncthreads();
#pragma unroll
  for (uint32_t r0 = 0; r0 < kRowsPerWave; r0 += kBatch) {
    if (r0 + kBatch < kRowsPerWave) {
#pragma unroll
      for (uint32_t r = r0 + kBatch; r < r0 + 2 * kBatch; r++)
#pragma unroll
        for (uint32_t j = 0; j < C; j++) {
          const uint32_t i = wv + (kThreads / 64) * r;
          v[r][j] = i < c.n ? sy[i * D + 64 * j + lane] : 0u;
        }
    }
#pragma unroll
    for (uint32_t r = r0; r < r0 + kBatch; r++) {
      const uint32_t i = wv + (kThreads / 64) * r;
      if (i < c.n && ((bm >> i) & 1ull))
#pragma unroll
        for (uint32_t j = 0; j < C; j++) atomicAdd(&h[v[r][j]], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = a.w.hhist + (uint64_t)c.s * kHuffTable;
  for (uint32_t i = tid; i < kHuffTable; i += kThreads)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

// A segment's code table (kHuffTable words) into LDS, every load of a
// thread in flight before its stores.
__device__ __forceinline__ void copy_table(uint32_t* dst, const uint32_t* src, uint32_t tid) {
  constexpr uint32_t kQ = kHuffTable / 4 / kThreads;
  uint4 v[kQ];
#pragma unroll
  for (uint32_t q = 0; q < kQ; q++) v[q] = reinterpret_cast<const uint4*>(src)[kThreads * q + tid];
#pragma unroll
  for (uint32_t q = 0; q < kQ; q++) reinterpret_cast<uint4*>(dst)[kThreads * q + tid] = v[q];
}

// Lane L's four symbols E[256 ch + 4L .. + 3] of the tile (four symbols of
// one row: nE and every row start are multiples of 64), zero past nE.
template <uint32_t D>
__device__ __forceinline__ uint2 lane_syms(const uint16_t* sy, const uint8_t* urow, uint32_t ch, uint32_t nE) {
  const uint32_t e = ch * 256 + 4 * (threadIdx.x & 63);
  if (e >= nE) return make_uint2(0, 0);
  return *reinterpret_cast<const uint2*>(sy + (uint32_t)urow[e / D] * D + e % D);
}

// Bits of those four symbols (none past nE); with codes (enc: len << 16 |
// code) also their codes, first code in the high bits of *val.
__device__ __forceinline__ uint32_t lane_code_bits(uint2 w, bool has, const uint32_t* enc, uint64_t* val) {
  uint32_t bits = 0;
  uint64_t v = 0;
  if (has) {
    const uint32_t sym[4] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t ent = enc[sym[k]], l = ent >> 16;
      bits += l;
      v = (v << l) | (ent & 0xFFFFu);
    }
  }
  *val = v;
  return bits;
}

template <int C>
__global__ void __launch_bounds__(kThreads) ec_hsize_tiles(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  __shared__ __align__(16) uint32_t s_enc[kHuffTable];
  __shared__ uint8_t s_urow[kThreads / 64][kTileRows];
  __shared__ uint32_t s_words[kThreads / 64];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x;
  const TileCoord c = tile_coord(a, ticket);
  if (ticket == 0 && tid == 0 && a.w.hstat[0] != 0) report_error(a.report, kDevErrTimeout);
  if (c.n == 0 || a.w.seg_eb[c.s] == 0) {
    if (tid == 0) a.w.tile_hsize[ticket] = 0;
    return;
  }
  const uint32_t* enc = a.w.henc + (uint64_t)c.s * kHuffTable;
  const uint64_t bm = a.w.tile_bitmap[ticket];
  unique_rows(bm, s_urow[wv]);  // every wave its own copy: no barrier before the loads
  wave_lds_wait();
  const uint32_t U = (uint32_t)__popcll(bm), nE = U * D, nch = (nE + 255) / 256;
  const uint16_t* sy = a.w.stage_sym + (uint64_t)ticket * kTileRows * D;
  // the symbols of the wave's chunks, then the code table: all loads in flight
  constexpr uint32_t kChPerWave = kTileRows * D / 256 / (kThreads / 64);
  uint2 sw[kChPerWave];
#pragma unroll
  for (uint32_t k = 0; k < kChPerWave; k++) sw[k] = lane_syms<D>(sy, s_urow[wv], wv + (kThreads / 64) * k, nE);
  copy_table(s_enc, enc, tid);
  __syncthreads();
  uint32_t words = 0;
#pragma unroll
  for (uint32_t k = 0; k < kChPerWave; k++) {
    const uint32_t ch = wv + (kThreads / 64) * k;
    if (ch >= nch) break;
    uint64_t v;
    const uint32_t bits =
        wave_sum_u32(lane_code_bits(sw[k], ch * 256 + 4 * lane < nE, s_enc, &v));
    words += (bits + 31) / 32;
  }
  if (lane == 0) s_words[wv] = words;
  __syncthreads();
  if (tid == 0) {
    uint32_t w = 0;
    for (uint32_t q = 0; q < kThreads / 64; q++) w += s_words[q];
    const uint32_t rb = ref_bytes(c.rows, a.window), nout = a.w.tile_nout[ticket];
    const uint32_t off_ct = (uint32_t)align_up(16 + rb * (c.n - U), 4) + 8 * nout;
    a.w.tile_hsize[ticket] = (uint32_t)align_up(off_ct + 4ull * (nch + 1) + 4ull * w, 16);
  }
}

// Codebook reuse, one wave per segment, after the histograms: a segment that
// may be Huffman-coded keeps the code of the plan's previous call (henc,
// hbooks) while that code has a length for every symbol the segment holds
// (the builder then skips it); the segments that may be Huffman-coded hold a
// code after this call, the others none.
__global__ void __launch_bounds__(kThreads) ec_book_reuse(EncArgs a) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t s = blockIdx.x * (kThreads / 64) + wave_id();
  if (s >= a.sh.nseg) return;
  const uint32_t coder = a.w.table_coder ? a.w.table_coder[s % a.sh.T] : a.coder;
  const bool want = a.w.seg_eb[s] != 0 && coder != kCoderBitpack;
  bool covers = want && a.w.hhave[s] != 0;
  if (covers) {  // (uniform branch) sixteen pairs of loads per lane in flight at once
    const uint32_t* h = a.w.hhist + (uint64_t)s * kHuffTable;
    const uint32_t* e = a.w.henc + (uint64_t)s * kHuffTable;
    bool miss = false;
#pragma unroll
    for (uint32_t q = 0; q < 4; q++) {
      uint32_t hv[16], ev[16];
#pragma unroll
      for (uint32_t j = 0; j < 16; j++) {
        hv[j] = h[(q * 16 + j) * 64 + lane];
        ev[j] = e[(q * 16 + j) * 64 + lane];
      }
#pragma unroll
      for (uint32_t j = 0; j < 16; j++) miss = miss || (hv[j] != 0 && (ev[j] >> 16) == 0);
    }
    covers = !__any(miss);
  }
  if (lane == 0) {
    a.w.hskip[s] = covers ? 1u : 0u;
    a.w.hhave[s] = want ? 1u : 0u;
  }
}

// One wave per segment: Huffman (with coder 2, or with coder 3 when strictly
// smaller) or bit planes.  Both forms share the header and tile directory;
// the Huffman form adds the padded codebook.
__global__ void __launch_bounds__(kThreads) ec_seg_choose(EncArgs a) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t s = blockIdx.x * (kThreads / 64) + wave_id();
  if (s >= a.sh.nseg) return;
  const uint32_t coder = a.w.table_coder ? a.w.table_coder[s % a.sh.T] : a.coder;
  if (a.w.seg_eb[s] == 0 || coder == kCoderBitpack) {
    if (lane == 0) a.w.seg_coder[s] = 0;
    return;
  }
  const uint32_t D = a.sh.D, pch = s / a.sh.T;
  const uint32_t rows = chunk_row0(a.sh, pch + 1) - chunk_row0(a.sh, pch);
  const uint32_t nt = (rows + kTileRows - 1) / kTileRows, b = a.w.seg_tile_base[s];
  uint64_t bp = 0, hf = 0;
  for (uint32_t k = lane; k < nt; k += 64) {
    const uint32_t ticket = b + k, n = min(kTileRows, rows - k * kTileRows);
    const uint4 info = reinterpret_cast<const uint4*>(a.w.tile_info)[ticket];
    const RecLayout L =
        rec_layout(n, info.x, info.x * (D / 64), info.z, a.w.tile_nout[ticket], rows, D, true, a.window);
    const uint64_t raw = 16 + align_up(4ull * n * D, 16), h = a.w.tile_hsize[ticket];
    bp += L.rec;
    hf += h < raw ? h : raw;
  }
  bp = wave_sum_u64(bp);
  hf = wave_sum_u64(hf) + align_up(book_bytes(a.w.hbooks + (uint64_t)s * kBookStride), 16);
  if (lane == 0) a.w.seg_coder[s] = (coder == kCoderHuffman || hf < bp) ? 1u : 0u;
}

// One wave per size block: the items (record bytes plus the tables a tile
// writes first) of a Huffman segment's tiles, their record summaries, and
// the block's sum, again (bit-plane segments keep the size pass's values).
__global__ void __launch_bounds__(64) ec_items(EncArgs a) {
  const uint32_t lane = threadIdx.x;
  const uint32_t ticket = blockIdx.x * kBlockTiles + lane;
  uint64_t item = 0;
  if (lane < kBlockTiles && ticket < a.sh.ntiles) {
    const TileCoord c = tile_coord(a, ticket);
    item = a.w.tile_status[ticket];
    if (a.w.seg_coder[c.s]) {
      const uint64_t raw = c.n ? 16 + align_up(4ull * c.n * a.sh.D, 16) : 0;
      const uint32_t h = a.w.tile_hsize[ticket];
      const bool coded = c.n && h < raw;
      const uint64_t pre = c.k == 0 ? seg_prefix_bytes(c.ntiles) +
                                           align_up(book_bytes(a.w.hbooks + (uint64_t)c.s * kBookStride), 16) +
                                           (c.t == 0 ? align_up(8ull * a.sh.T, 16) : 0)
                                     : 0;
      item = (coded ? h : raw) + pre;
      a.w.tile_status[ticket] = item;
      uint4 info = reinterpret_cast<const uint4*>(a.w.tile_info)[ticket];
      info.y = coded ? a.w.tile_nout[ticket] : 0u;
      info.w = (coded ? 2u : 0u) | 0x100u;
      reinterpret_cast<uint4*>(a.w.tile_info)[ticket] = info;
    }
  }
  item = wave_sum_u64(item);
  if (lane == 0) a.w.block_status[blockIdx.x] = item;
}

// Chunk table and words of a Huffman record (the write pass wrote its header,
// references and outliers): per wave and chunk, the lanes' code bits are
// placed by a wave prefix sum and ORed into the wave's LDS buffer of 96
// words, which is then stored whole; the record's padding is zeroed.
template <int C>
__global__ void __launch_bounds__(kThreads) ec_write_huff(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  constexpr uint32_t kMaxCh = kTileRows * D / 256;
  __shared__ __align__(16) uint32_t s_enc[kHuffTable];
  __shared__ uint32_t s_buf[kThreads / 64][96];
  __shared__ uint32_t s_cw[kMaxCh + 1];
  __shared__ uint8_t s_urow[kThreads / 64][kTileRows];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x;
  const uint4 info = reinterpret_cast<const uint4*>(a.w.tile_info)[ticket];
  if ((info.w & 0xFFu) != 2u) return;
  const TileCoord c = tile_coord(a, ticket);
  const uint32_t n = c.n, U = info.x, nout = info.y;
  uint8_t* rec = a.out + (a.w.tile_rec[ticket] - 1);
  const uint32_t* enc = a.w.henc + (uint64_t)c.s * kHuffTable;
  const uint64_t bm = a.w.tile_bitmap[ticket];
  unique_rows(bm, s_urow[wv]);  // every wave its own copy: no barrier before the loads
  wave_lds_wait();
  const uint32_t rb = ref_bytes(c.rows, a.window);
  const uint32_t off_ct = (uint32_t)align_up(16 + rb * (n - U), 4) + 8 * nout;
  const uint32_t nE = U * D, nch = (nE + 255) / 256, off_w = off_ct + 4 * (nch + 1);
  const uint16_t* sy = a.w.stage_sym + (uint64_t)ticket * kTileRows * D;
  // the symbols of the wave's chunks (used twice), then the code table: all
  // loads in flight
  constexpr uint32_t kChPerWave = kMaxCh / (kThreads / 64);
  uint2 sw[kChPerWave];
#pragma unroll
  for (uint32_t k = 0; k < kChPerWave; k++) sw[k] = lane_syms<D>(sy, s_urow[wv], wv + (kThreads / 64) * k, nE);
  copy_table(s_enc, enc, tid);
  __syncthreads();
#pragma unroll
  for (uint32_t k = 0; k < kChPerWave; k++) {  // words of every chunk
    const uint32_t ch = wv + (kThreads / 64) * k;
    if (ch >= nch) break;
    uint64_t v;
    const uint32_t bits = wave_sum_u32(lane_code_bits(sw[k], ch * 256 + 4 * lane < nE, s_enc, &v));
    if (lane == 0) s_cw[ch] = (bits + 31) / 32;
  }
  __syncthreads();
  if (wv == 0) {  // word offsets of the chunks (at most 64) and the chunk table
    const uint32_t cw = lane < nch ? s_cw[lane] : 0u;
    const uint32_t inc = wave_incl_u32(cw);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    uint32_t* ct = reinterpret_cast<uint32_t*>(rec + off_ct);
    if (lane < nch) {
      ct[lane] = inc - cw;
      s_cw[lane] = inc - cw;
    }
    if (lane == 0) {
      ct[nch] = total;
      s_cw[kMaxCh] = total;
    }
  }
  __syncthreads();
  uint32_t* buf = s_buf[wv];
  uint32_t* words = reinterpret_cast<uint32_t*>(rec + off_w);
#pragma unroll
  for (uint32_t k = 0; k < kChPerWave; k++) {
    const uint32_t ch = wv + (kThreads / 64) * k;
    if (ch >= nch) break;
    buf[lane] = 0;
    if (lane < 32) buf[64 + lane] = 0;
    wave_lds_wait();
    uint64_t v;
    const uint32_t L = lane_code_bits(sw[k], ch * 256 + 4 * lane < nE, s_enc, &v);
    const uint32_t inc = wave_incl_u32(L), start = inc - L;
    if (L) {  // the bits [start, start + L) of the chunk, first bit in bit 31 of its word
      const uint32_t w0 = start >> 5, S = (start & 31u) + L;
      for (uint32_t k = 0; 32 * k < S; k++) {
        const int sh = (int)S - 32 * (int)(k + 1);
        const uint32_t part = sh >= 0 ? (uint32_t)(v >> sh) : (uint32_t)(v << -sh);
        atomicOr(&buf[w0 + k], part);
      }
    }
    wave_lds_wait();
    const uint32_t cw = ((uint32_t)__builtin_amdgcn_readlane((int)inc, 63) + 31) / 32;
    for (uint32_t i = lane; i < cw; i += 64) words[s_cw[ch] + i] = buf[i];
  }
  // zero padding after the words up to the record's 16-byte end
  const uint32_t end = off_w + 4 * s_cw[kMaxCh], pad = (uint32_t)align_up(end, 16) - end;
  if (tid < pad) rec[end + tid] = 0;
}

// ---------------------------------------------------------------------------
// offline analysis (section III-C, eq. (1)): the distinct original rows of
// every segment.  One workgroup per tile, 16 rows per wave: each row's hash of
// its raw bits goes into the segment's (empty) hash table by compare-and-swap
// with linear probing; a tag hit is confirmed by comparing the two rows' bits.
// Equal rows have equal hashes and so meet at the first empty slot of their
// common probe sequence, where exactly one of them wins: the winners, summed
// per segment, are the distinct rows.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) ec_distinct_raw(EncArgs a) {
  constexpr uint32_t kRowsPerWave = kTileRows / (kThreads / 64);
  __shared__ uint32_t s_won[kThreads / 64];
  const uint32_t lane = threadIdx.x & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x;
  const TileCoord c = tile_coord(a, ticket);
  const uint32_t D = a.sh.D, n = c.n;
  const float* xs = a.x + ((uint64_t)c.t * a.sh.B + chunk_row0(a.sh, c.pch)) * D;
  uint64_t* htab = a.w.hash + a.w.hash_off[c.s];
  const uint32_t cap_mask = (1u << a.w.hash_log2[c.s]) - 1u;
  const uint32_t rbeg = wv * kRowsPerWave;
  // lane L < 16 keeps the hash of the wave's row rbeg + L
  uint32_t H = 0;
  for (uint32_t rr = 0; rr < kRowsPerWave && rbeg + rr < n; rr++) {
    const float* xr = xs + (uint64_t)(c.k * kTileRows + rbeg + rr) * D;
    uint32_t h = 0;
    for (uint32_t d = lane; d < D; d += 64) h += fmix32(f2u(xr[d]) ^ (d * 0x9e3779b9u + 0x7f4a7c15u));
    h = fmix32(wave_sum_u32(h) + D) & (uint32_t)a.hash_keep;
    if (lane == rr) H = h;
  }
  const uint32_t row = c.k * kTileRows + rbeg + lane;  // segment row of the lane's row
  bool active = lane < kRowsPerWave && rbeg + lane < n;
  const uint64_t mine = ((uint64_t)H << 32) | (uint64_t)(row + 1);
  uint32_t slot = H & cap_mask, won = 0, cand = 0, guard = 0;
  while (__ballot(active) != 0) {
    bool need = false;
    if (active) {
      const uint64_t old = atomicCAS((unsigned long long*)&htab[slot], 0ull, (unsigned long long)mine);
      if (old == 0) {
        won = 1;
        active = false;
      } else if ((uint32_t)(old >> 32) == H && (uint32_t)old - 1u < c.rows) {
        need = true;
        cand = (uint32_t)old - 1u;
      } else {
        slot = (slot + 1) & cap_mask;
      }
    }
    uint64_t m = __ballot(need);
    while (m) {  // the whole wave compares one candidate pair at a time
      const int L = __ffsll((long long)m) - 1;
      m &= m - 1;
      const uint32_t ra = __shfl(row, L), rb = __shfl(cand, L);
      bool eq = true;
      for (uint32_t d = lane; d < D; d += 64)
        eq = eq && f2u(xs[(uint64_t)ra * D + d]) == f2u(xs[(uint64_t)rb * D + d]);
      eq = __all(eq);
      if ((int)lane == L) {
        if (eq) active = false;
        else slot = (slot + 1) & cap_mask;
      }
    }
    if (++guard > cap_mask + 2) {  // cannot happen: the table is at most a quarter full
      if (active) report_error(a.report, kDevErrTimeout);
      active = false;
    }
  }
  const uint32_t w = wave_sum_u32(won);
  if (lane == 0) s_won[wv] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (uint32_t q = 0; q < kThreads / 64; q++) t += s_won[q];
    a.w.tile_status[ticket] = t;
  }
}

// One wave per segment: the segment's distinct rows, summed over its tiles.
__global__ void __launch_bounds__(kThreads) ec_distinct_sum(EncArgs a) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t s = blockIdx.x * (kThreads / 64) + wave_id();
  if (s >= a.sh.nseg) return;
  const uint32_t b = a.w.seg_tile_base[s], e = a.w.seg_tile_base[s + 1];
  uint64_t v = 0;
  for (uint32_t j = b + lane; j < e; j += 64) v += a.w.tile_status[j];
  v = wave_sum_u64(v);
  if (lane == 0 && a.seg_norig) a.seg_norig[s] = (uint32_t)v;
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
constexpr uint32_t kOutCap = 256;  // outliers staged in LDS per tile

struct DecTile {
  const uint8_t* rec;   // record start
  uint64_t avail;       // bytes from the record start to the segment end
  uint64_t bitmap;
  uint32_t n, U, nout, mode, ok;
  uint32_t nblk, off_refs, off_opos, off_oval, off_pl;
  uint32_t nch, off_ct, off_w;  // Huffman records: chunks, chunk table, words
};

struct DecShared {
  uint32_t ok, seg, tile, n, rows, ntiles, valid, bad;
  uint32_t seg_ok, hseg;  // the segment's headers passed; it is a Huffman segment
  uint32_t win;           // W of a windowed segment, else 0
  float eb;
  uint64_t seg_off, seg_bytes, total, rec_lo;
  DecTile tl;
  uint32_t part[kThreads / 64];
};

// The stream is read-only while it is decoded: reading its bit planes
// through the constant address space lets wave-uniform loads be scalar loads.
typedef const __attribute__((address_space(4))) uint64_t const_u64;
__device__ __forceinline__ const_u64* as_const_u64(const uint8_t* p) {
  return (const_u64*)(uintptr_t)p;
}

__device__ __forceinline__ uint32_t uniform32(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  return ((uint64_t)uniform32((uint32_t)(v >> 32)) << 32) | uniform32((uint32_t)v);
}

// Stream words (read-only while decoding): through the constant address
// space, so a wave-uniform address becomes a scalar load.
typedef const __attribute__((address_space(4))) uint32_t const_u32;
__device__ __forceinline__ uint64_t rd64(const uint8_t* p) {
  return *(const_u64*)(uintptr_t)p;
}
__device__ __forceinline__ uint32_t rd32(const uint8_t* p) {
  return *(const_u32*)(uintptr_t)p;
}

// Locate and check tile record k of a segment; every read is bounds-checked
// against the segment.
// The stream header's version and coder: 1 bit planes only, 2 and 3 with
// Huffman segments (decodable only by a plan with the Huffman tables).
__device__ __forceinline__ bool header_coder_ok(uint32_t w, uint32_t huff, uint32_t& coder) {
  coder = w >> 16;
  return (w & 0xFFFFu) == kVersion && coder >= kCoderBitpack && coder <= kCoderAuto &&
         (huff || coder == kCoderBitpack);
}
// A segment's flags: bit 0 eb valid, bit 1 Huffman segment (only with bit 0,
// never in a coder-1 stream, always for a valid segment of a coder-2 stream),
// bit 2 windowed references with the window W in bits 8-15 (only with bit 0,
// and only for a plan that decodes them); win gets W.
__device__ __forceinline__ bool seg_flags_ok(uint32_t flags, uint32_t coder, bool allow_win,
                                             uint32_t& win) {
  win = (flags >> 8) & 0xFFu;
  const uint32_t f = flags & 0xFFu;
  if ((flags >> 16) != 0) return false;
  if (win == 0 ? (f > 3 || f == 2) : (!allow_win || (f != 5 && f != 7))) return false;
  const bool hs = (flags & 2u) != 0;
  return !(hs && coder == kCoderBitpack) && !(coder == kCoderHuffman && (flags & 1u) && !hs);
}

// Whole wave, wave-uniform arguments: loads that pull lines of a buffer of
// `bytes` bytes at p into the caches ahead of the dependent reads that need
// them, so that those reads wait for the L2 and not for HBM.  touch_lines:
// one word of each 128-byte line of the first min(bytes, 8 KiB); touch_word:
// the word at byte offset o (lane 0).  Nothing past the buffer (or past
// 2 GiB) is read.  The caller keeps the returned word alive until its
// dependent reads are done, so the wait for these loads lands there.
__device__ __forceinline__ uint32_t touch_lines(const uint8_t* p, uint64_t bytes) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t lim = (uint32_t)min(bytes, (uint64_t)8192);
  return buf_ld_u32(buf_rsrc(p, lim), lane * 128 + 4 <= lim ? lane * 128 : kOff);
}
__device__ __forceinline__ uint32_t touch_word(const uint8_t* p, uint64_t bytes, uint64_t o) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t lim = (uint32_t)min(bytes, (uint64_t)kOff);
  o &= ~3ull;
  return buf_ld_u32(buf_rsrc(p, lim), lane == 0 && o + 4 <= lim ? (uint32_t)o : kOff);
}

// Locate and check tile record k of a segment whose records start at rec_lo
// or later (after the tile directory, and the codebook of a Huffman segment);
// every read is bounds-checked against the segment.  With `touch` (a whole
// wave with uniform arguments), the record's first lines are pulled into the
// caches together with its header (touch_lines).
__device__ DecTile locate_tile(const uint8_t* seg, uint64_t seg_bytes, uint32_t ntiles,
                               uint32_t rows, uint32_t k, uint32_t D, bool valid, uint64_t rec_lo,
                               bool hseg, uint32_t win, uint32_t* touch = nullptr) {
  DecTile r{};
  r.ok = 0;
  if (k >= ntiles) return r;
  uint32_t off = rd32(seg + 32 + 4ull * k);
  if (off < rec_lo || (off & 15u) || (uint64_t)off + 16 > seg_bytes) return r;
  r.rec = seg + off;
  r.avail = seg_bytes - off;
  if (touch) {  // up to the next record (its directory entry is read with this one)
    const uint32_t nxt = k + 1 < ntiles ? rd32(seg + 32 + 4ull * (k + 1)) : 0u;
    *touch += touch_lines(r.rec, nxt > off ? min((uint64_t)(nxt - off), r.avail) : r.avail);
  }
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
  } else if (r.mode == 2) {
    if (!hseg) return r;
    uint64_t nE = (uint64_t)r.U * D;
    if (r.nout > nE) return r;
    uint32_t rb = ref_bytes(rows, win);
    uint64_t off_opos = align_up(16 + (uint64_t)rb * (r.n - r.U), 4);
    uint64_t off_ct = off_opos + 8ull * r.nout;
    uint64_t nch = (nE + 255) / 256;
    uint64_t off_w = off_ct + 4 * (nch + 1);
    if (off_w > r.avail) return r;
    r.off_refs = 16;
    r.off_opos = (uint32_t)off_opos;
    r.off_oval = (uint32_t)(off_opos + 4ull * r.nout);
    r.off_ct = (uint32_t)off_ct;
    r.nch = (uint32_t)nch;
    r.off_w = (uint32_t)off_w;
  } else if (r.mode == 1 && !hseg) {
    uint64_t nE = (uint64_t)r.U * D;
    if (r.nout > nE) return r;
    uint64_t nblk = (nE + 63) / 64;
    uint32_t rb = ref_bytes(rows, win);
    uint64_t off_refs = align_up(16 + nblk, 4);
    uint64_t off_opos = align_up(off_refs + (uint64_t)rb * (r.n - r.U), 4);
    uint64_t off_oval = off_opos + 4ull * r.nout;
    uint64_t off_pl = align_up(off_oval + 4ull * r.nout, 8);
    if (off_pl > r.avail) return r;
    r.nblk = (uint32_t)nblk;
    r.off_refs = (uint32_t)off_refs;
    r.off_opos = (uint32_t)off_opos;
    r.off_oval = (uint32_t)off_oval;
    r.off_pl = (uint32_t)off_pl;
  } else {
    return r;
  }
  r.ok = 1;
  return r;
}

// Whole wave, uniform control flow: the segment header's U and n_out (words 4
// and 5) must equal the sums over the segment's tile records.  Entries that
// fail their own checks are skipped here (their tiles' workgroups report
// them); every read stays inside the segment.
__device__ bool seg_totals_ok(const uint8_t* sg, uint64_t sbytes, uint32_t ntiles, uint64_t prefix) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t u = 0, o = 0;
  for (uint32_t j = lane; j < ntiles; j += 64) {
    const uint32_t off = reinterpret_cast<const uint32_t*>(sg + 32)[j];
    if (off >= prefix && !(off & 15u) && (uint64_t)off + 16 <= sbytes) {
      o += reinterpret_cast<const uint32_t*>(sg + off)[2];
      u += reinterpret_cast<const uint32_t*>(sg + off)[3] & 0xffffu;
    }
  }
  u = wave_sum_u32(u);
  o = wave_sum_u32(o);
  return u == reinterpret_cast<const uint32_t*>(sg)[4] && o == reinterpret_cast<const uint32_t*>(sg)[5];
}

// Whole wave, uniform control flow: the stream header's total equals the
// header and chunk table plus the sum of the P chunk byte counts (each
// already checked to lie inside the stream).
__device__ bool chunk_totals_ok(const uint8_t* in, uint32_t P, uint64_t total) {
  const uint32_t lane = threadIdx.x & 63;
  uint64_t sum = 0;
  for (uint32_t q = lane; q < P; q += 64) sum += reinterpret_cast<const uint64_t*>(in + 64)[q];
  sum = wave_sum_u64(sum);
  return sum + 64 + align_up(8ull * P, 16) == total;
}

// Decode the D values of E[e0 .. e0 + D) into y (whole wave, lane = element
// within a 64-wide chunk).  Block b's planes start at word boff(b):
//   boff given (LDS prefix):  boff[b];
//   boff == nullptr:          run0 + sum of widths[b0 .. b), with run0 the
//                             offset of block b0 = e0 / 64.
// Returns false if a width or a plane index is out of range.
template <typename WP, typename PP, typename OP>
__device__ __forceinline__ bool decode_span(float* y, uint32_t D, uint32_t e0, uint32_t nblk,
                                            WP widths, const uint32_t* boff, uint32_t run0,
                                            PP planes, uint64_t plane_words, OP opos, OP oval,
                                            uint32_t nout, float s2) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t olo = 0, ohi = nout;  // first outlier at or after e0
  while (olo < ohi) {
    uint32_t mid = (olo + ohi) >> 1;
    if (opos[mid] < e0) olo = mid + 1;
    else ohi = mid;
  }
  const uint32_t b0 = e0 >> 6;
  uint32_t run = run0;
  bool ok = true;
  for (uint32_t m = 0; m * 64 < D; m++) {
    const uint32_t A = b0 + m;
    const uint32_t wA = A < nblk ? widths[A] : 0;
    const uint32_t wB = A + 1 < nblk ? widths[A + 1] : 0;
    const uint32_t offA = boff ? (A < nblk ? boff[A] : 0) : run;
    const uint32_t offB = boff ? (A + 1 < nblk ? boff[A + 1] : 0) : run + wA;
    const uint32_t d = m * 64 + lane;
    const uint32_t e = e0 + d;
    const bool inB = (e >> 6) != A;
    const uint32_t w = inB ? wB : wA;
    const uint32_t off = inB ? offB : offA;
    const bool lane_ok = w <= 12 && (uint64_t)off + w <= plane_words;
    uint32_t zz = 0;
    if (d < D && lane_ok) {
      const uint32_t bit = e & 63;
      for (uint32_t j = 0; j < w; j++) zz |= (uint32_t)((planes[off + j] >> bit) & 1ull) << j;
    }
    ok = ok && (d >= D || lane_ok);
    float v = (float)unzigzag(zz) * s2;
    const uint32_t chunk_end = e0 + min(D, m * 64 + 64);
    while (olo < nout) {
      uint32_t pos = opos[olo];
      if (pos >= chunk_end) break;
      if (pos == e) v = __uint_as_float(oval[olo]);
      olo++;
    }
    if (d < D) y[d] = v;
    run += wA;
  }
  return __all(ok);
}

__global__ void __launch_bounds__(kThreads) ec_decode_kernel(DecArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ DecShared sh;
  __shared__ uint32_t s_src[kTileRows];      // local uid, or kExt | row for references
  __shared__ uint32_t s_xoff[kTileRows];     // external: record offset in the segment
  __shared__ uint32_t s_xu[kTileRows];       // external: uid (BITPACK) or row (RAW)
  __shared__ uint32_t s_xbase[kTileRows];    // external: plane word offset of the row's block
  constexpr uint32_t kExt = 0x80000000u, kBad = 0x40000000u;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t D = a.sh.D, T = a.sh.T, B = a.sh.B, P = a.sh.P;
  const uint32_t ticket = blockIdx.x;
  const uint32_t plane_cap = min(12u * D, 6144u);
  uint64_t* s_planes = reinterpret_cast<uint64_t*>(smem);
  uint32_t* s_boff = reinterpret_cast<uint32_t*>(smem + 8ull * plane_cap);
  uint8_t* s_width = reinterpret_cast<uint8_t*>(s_boff + D + 8);
  uint32_t* s_opos = reinterpret_cast<uint32_t*>(s_width + ((D + 8 + 15) / 16) * 16);
  uint32_t* s_oval = s_opos + kOutCap;

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
    sh.bad = 0;
    uint32_t ok = 1;
    const uint8_t* in = a.in;
    uint64_t total = 0;
    uint32_t coder = 0;
    if (a.cap < 64) ok = 0;
    if (ok) {
      const uint32_t* h = reinterpret_cast<const uint32_t*>(in);
      total = rd64(in + 48);
      ok = h[0] == kMagic && header_coder_ok(h[1], 0u, coder) && h[2] == T &&
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
      // (a coder-1 stream: no Huffman segment)
      uint32_t win = 0;
      if (rd32(sg) != rows || rd32(sg + 4) != nt || !seg_flags_ok(flags, coder, false, win) ||
          (int)(flags & 1u) != valid || sb > cb - so || sb < 32 + align_up(4ull * nt, 16))
        ok = 0;
      sh.eb = eb;
      sh.valid = flags & 1u;
    }
    sh.seg_off = chunk + so;
    sh.seg_bytes = sb;
    sh.total = total;
    sh.rec_lo = 32 + align_up(4ull * nt, 16);
    if (ok && nt) {
      DecTile tl = locate_tile(in + chunk + so, sb, nt, rows, k, D, sh.valid != 0, sh.rec_lo, false, 0);
      ok = tl.ok;
      sh.tl = tl;
    }
    sh.ok = ok;
  }
  __syncthreads();
  if (wv == 0 && sh.ok) {  // a segment's first tile checks its totals, tile 0 the chunk sizes
    bool good = sh.tile != 0 || seg_totals_ok(a.in + sh.seg_off, sh.seg_bytes, sh.ntiles, sh.rec_lo);
    if (ticket == 0) good = good && chunk_totals_ok(a.in, P, sh.total);
    if (!good && lane == 0) report_error(a.report, kDevErrCorrupt);
  }
  const uint32_t s = sh.seg, k = sh.tile, n = sh.n, rows = sh.rows;
  const uint32_t pch = s / T, t = s % T;
  float* yseg = a.y + ((uint64_t)t * B + chunk_row0(a.sh, pch)) * D;
  float* yt = yseg + (uint64_t)k * kTileRows * D;
  if (n == 0) {
    if (!sh.ok && tid == 0) report_error(a.report, kDevErrCorrupt);
    return;
  }
  if (!sh.ok) {
    for (uint32_t i = tid; i < n * D; i += kThreads) yt[i] = 0.0f;
    if (tid == 0) report_error(a.report, kDevErrCorrupt);
    return;
  }
  const DecTile tl = sh.tl;
  if (tl.mode == 0) {  // RAW: rows verbatim
    const float* src = reinterpret_cast<const float*>(tl.rec + 16);
    if ((D & 3) == 0) {
      const float4* s4 = reinterpret_cast<const float4*>(src);
      float4* y4 = reinterpret_cast<float4*>(yt);
      for (uint32_t i = tid; i < n * D / 4; i += kThreads) y4[i] = s4[i];
    } else {
      for (uint32_t i = tid; i < n * D; i += kThreads) yt[i] = src[i];
    }
    return;
  }

  // ---- BITPACK: stage widths (-> word offsets), bit planes, outliers ----
  const float eb = sh.eb, s2 = eb + eb;
  const uint8_t* sg = a.in + sh.seg_off;
  const uint64_t sbytes = sh.seg_bytes;
  const uint32_t rb = rows <= 65536 ? 2 : 4;
  const uint32_t nblk = tl.nblk;
  uint32_t badw = 0;
  for (uint32_t b = tid; b < nblk; b += kThreads) {
    uint32_t w = tl.rec[16 + b];
    badw |= w > 12;
    s_width[b] = (uint8_t)w;
    s_boff[b] = w;
  }
  if (badw) sh.bad = 1;
  // the scan reads each thread's share in its own order (past 256 blocks not
  // the one the widths were written in): every write must be visible first
  __syncthreads();
  const uint32_t sumw = nblk ? block_exclusive_scan(s_boff, nblk, sh.part) : 0;
  const uint64_t plane_words = (tl.avail - tl.off_pl) / 8;
  const uint64_t* g_planes = reinterpret_cast<const uint64_t*>(tl.rec + tl.off_pl);
  const uint32_t* g_opos = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_opos);
  const uint32_t* g_oval = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_oval);
  const bool planes_fit = sumw <= plane_words;
  const bool stage_planes = planes_fit && sumw <= plane_cap;
  const bool stage_out = tl.nout <= kOutCap;
  if (stage_planes)
    for (uint32_t i = tid; i < sumw; i += kThreads) s_planes[i] = g_planes[i];
  if (stage_out)
    for (uint32_t i = tid; i < tl.nout; i += kThreads) {
      s_opos[i] = g_opos[i];
      s_oval[i] = g_oval[i];
    }
  {
    // outlier positions index E (U*D values) and strictly increase; the
    // decoders' searches assume both, so a stream breaking either is corrupt
    const uint32_t nE = tl.U * D;
    uint32_t obad = 0;
    for (uint32_t i = tid; i < tl.nout; i += kThreads) {
      const uint32_t p = g_opos[i];
      obad |= p >= nE || (i > 0 && g_opos[i - 1] >= p);
    }
    if (obad) sh.bad = 1;
  }
  // source of every row: a uid of this record, or a reference into an
  // earlier record (resolved lane-parallel so the metadata loads overlap)
  if (tid < n) {
    const uint32_t i = tid, r = k * kTileRows + i;
    const uint64_t below = tl.bitmap & ((1ull << i) - 1ull);
    uint32_t src;
    if ((tl.bitmap >> i) & 1ull) {
      src = (uint32_t)__popcll(below);
    } else {
      const uint32_t j = i - (uint32_t)__popcll(below);
      const uint32_t ref = rb == 2 ? reinterpret_cast<const uint16_t*>(tl.rec + tl.off_refs)[j]
                                   : reinterpret_cast<const uint32_t*>(tl.rec + tl.off_refs)[j];
      if (ref >= r) {
        src = kBad;
      } else if (ref >= k * kTileRows) {
        const uint32_t i2 = ref - k * kTileRows;
        src = ((tl.bitmap >> i2) & 1ull) ? (uint32_t)__popcll(tl.bitmap & ((1ull << i2) - 1ull))
                                          : kBad;
      } else {
        const uint32_t k2 = ref / kTileRows, i2 = ref % kTileRows;
        DecTile t2 = locate_tile(sg, sbytes, sh.ntiles, rows, k2, D, true, sh.rec_lo, false, 0);
        src = kExt | i;
        if (!t2.ok || !((t2.bitmap >> i2) & 1ull)) {
          src = kBad;
        } else if (t2.mode == 0) {
          s_xoff[i] = (uint32_t)(t2.rec - sg);
          s_xu[i] = i2;
        } else {
          const uint32_t u2 = (uint32_t)__popcll(t2.bitmap & ((1ull << i2) - 1ull));
          const uint32_t b0 = (u2 * D) >> 6;
          // plane word offset of block b0: sum of the record's first b0 widths
          const uint32_t* w4 = reinterpret_cast<const uint32_t*>(t2.rec + 16);
          uint32_t base = 0;
          for (uint32_t q = 0; q < b0 / 4; q++) {
            uint32_t v = w4[q];
            v = (v & 0x00ff00ffu) + ((v >> 8) & 0x00ff00ffu);
            base += (v & 0xffffu) + (v >> 16);
          }
          for (uint32_t q = b0 & ~3u; q < b0; q++) base += t2.rec[16 + q];
          s_xoff[i] = (uint32_t)(t2.rec - sg);
          s_xu[i] = u2;
          s_xbase[i] = base;
        }
      }
    }
    s_src[i] = src;
  }
  __syncthreads();

  // ---- decode, one wave per output row ----
  for (uint32_t i = wv; i < n; i += kThreads / 64) {
    const uint32_t src = s_src[i];
    float* y = yt + (uint64_t)i * D;
    bool ok = (src & kBad) == 0;
    if (ok && !(src & kExt)) {
      const uint32_t e0 = src * D;
      if (stage_planes && stage_out)
        ok = decode_span(y, D, e0, nblk, s_width, s_boff, 0, s_planes, (uint64_t)sumw,
                         (const uint32_t*)s_opos, (const uint32_t*)s_oval, tl.nout, s2);
      else if (planes_fit)
        ok = decode_span(y, D, e0, nblk, s_width, s_boff, 0, g_planes, plane_words, g_opos,
                         g_oval, tl.nout, s2);
      else
        ok = false;
    } else if (ok) {
      const uint8_t* rec2 = sg + s_xoff[i];
      const uint32_t u2 = s_xu[i];
      const uint32_t w3 = rd32(rec2 + 12);
      if (((w3 >> 16) & 0xffu) == 0) {  // referenced row stored RAW: re-quantize it
        const float* src2 = reinterpret_cast<const float*>(rec2 + 16) + (uint64_t)u2 * D;
        for (uint32_t d = lane; d < D; d += 64) {
          float v = src2[d];
          int q;
          y[d] = quantize(v, eb, s2, q) ? v : (float)q * s2;
        }
      } else {
        DecTile t2;
        t2.rec = rec2;
        t2.avail = sbytes - (uint64_t)(rec2 - sg);
        t2.U = w3 & 0xffffu;
        t2.nout = rd32(rec2 + 8);
        // a referenced tile precedes the current one, so it is not the
        // segment's last tile and holds a full 64 rows
        const uint32_t n2 = kTileRows;
        const uint32_t nE = t2.U * D, nb2 = (nE + 63) / 64;
        const uint32_t off_refs = (uint32_t)align_up(16 + nb2, 4);
        const uint32_t off_opos = (uint32_t)align_up(off_refs + rb * (n2 - t2.U), 4);
        const uint32_t off_oval = off_opos + 4 * t2.nout;
        const uint32_t off_pl = (uint32_t)align_up(off_oval + 4 * t2.nout, 8);
        if (off_pl > t2.avail) {
          ok = false;
        } else {
          ok = decode_span(y, D, u2 * D, nb2, rec2 + 16, (const uint32_t*)nullptr, s_xbase[i],
                           reinterpret_cast<const uint64_t*>(rec2 + off_pl),
                           (t2.avail - off_pl) / 8,
                           reinterpret_cast<const uint32_t*>(rec2 + off_opos),
                           reinterpret_cast<const uint32_t*>(rec2 + off_oval), t2.nout, s2);
        }
      }
    }
    if (!ok || sh.bad) {
      for (uint32_t d = lane; d < D; d += 64) y[d] = 0.0f;
      if (lane == 0) report_error(a.report, kDevErrCorrupt);
    }
  }
}

// ---------------------------------------------------------------------------
// decoder for D = 64*C.  The stream and the output are restrict kernel
// arguments, so the wave-uniform bit-plane loads become scalar loads and each
// plane costs one conditional select per element (codes built MSB first).
// ---------------------------------------------------------------------------
// One whole wave (every lane computes the same): check the stream header,
// chunk table, segment header and tile record of tile `ticket`; lane 0 fills
// sh_out (offsets relative to `in`).  With `touch`, the lines its later
// steps read (the segment's chunk-table entry, the tile's directory entry,
// the record) are pulled into the caches as soon as their addresses are
// known; the word returned there must be kept alive by the caller.
__device__ void dec_locate(const DecArgs& a, const uint8_t* in, uint32_t ticket, DecShared& sh_out,
                           uint64_t& rec_off, uint32_t* touch = nullptr) {
  DecShared sh;  // computed by the whole wave (uniform), stored by lane 0
  const uint32_t T = a.sh.T, B = a.sh.B, D = a.sh.D, P = a.sh.P;
  uint32_t s, k;
  ticket_coords(a.sh, a.seg_tile_base, ticket, s, k);
  uint32_t pch = s / T, t = s % T;
  uint32_t r0 = chunk_row0(a.sh, pch), rows = chunk_row0(a.sh, pch + 1) - r0;
  uint32_t nt = (rows + kTileRows - 1) / kTileRows;
  sh.seg = s;
  sh.tile = k;
  sh.rows = rows;
  sh.ntiles = nt;
  sh.n = nt ? min(kTileRows, rows - k * kTileRows) : 0;
  sh.bad = 0;
  uint32_t ok = 1, coder = 0;
  uint64_t total = 0;
  if (a.cap < 64) ok = 0;
  if (ok) {
    const uint32_t* h = reinterpret_cast<const uint32_t*>(in);
    total = rd64(in + 48);
    ok = h[0] == kMagic && header_coder_ok(h[1], a.huff, coder) && h[2] == T &&
         h[3] == B && h[4] == D && h[5] == P && h[6] == kTileRows && h[7] <= 1 &&
         rd64(in + 40) == 4ull * T * B * D && rd64(in + 56) == 0 && total <= a.cap;
  }
  uint64_t base = 64 + align_up(8ull * P, 16);
  if (touch && pch == 0) *touch += touch_word(in, a.cap, base + 8ull * t);
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
    if (touch && ok) *touch += touch_word(in + chunk + so, cb - so, 32 + 4ull * k);
  }
  sh.hseg = 0;
  sh.win = 0;
  sh.rec_lo = 32 + align_up(4ull * nt, 16);
  if (ok) {
    const uint8_t* sg = in + chunk + so;
    uint32_t flags = rd32(sg + 12);
    float eb = __uint_as_float(rd32(sg + 8));
    sb = rd64(sg + 24);
    int valid = isfinite(eb) && eb > 0.0f && isfinite(eb + eb);
    uint32_t win = 0;
    if (rd32(sg) != rows || rd32(sg + 4) != nt || !seg_flags_ok(flags, coder, a.window != 0, win) ||
        (int)(flags & 1u) != valid || sb > cb - so || sb < sh.rec_lo)
      ok = 0;
    sh.win = win;
    sh.eb = eb;
    sh.valid = flags & 1u;
    sh.hseg = (flags >> 1) & 1u;
    if (ok && sh.hseg) {  // records start after the codebook
      if (sh.rec_lo + 4 > sb) {
        ok = 0;
      } else {
        const uint32_t bw = rd32(sg + sh.rec_lo), lo = bw & 0xFFFFu, hi = bw >> 16;
        sh.rec_lo += align_up(hi < lo ? 4u : 4u + (hi - lo + 2) / 2, 16);
        if (sh.rec_lo > sb) ok = 0;
      }
    }
  }
  sh.seg_ok = ok;
  sh.seg_off = chunk + so;
  sh.seg_bytes = sb;
  sh.total = total;
  rec_off = 0;
  if (ok && nt) {
    DecTile tl = locate_tile(in + chunk + so, sb, nt, rows, k, D, sh.valid != 0, sh.rec_lo,
                             sh.hseg != 0, sh.win, touch);
    ok = tl.ok;
    sh.tl = tl;
    rec_off = (uint64_t)(tl.rec - in);
  }
  sh.ok = ok;
  if ((threadIdx.x & 63) == 0) sh_out = sh;
}

// Decode one 64-element block (lane = element): w <= 12 planes from word
// `off` of `planes` (valid words: [0, nwords)).  The planes are fetched in
// one burst of 8 or 12 words when that stays inside the record's segment;
// bits past w are masked off.
template <typename PP>
__device__ __forceinline__ float decode_block(PP planes, uint32_t off, uint32_t w,
                                              uint64_t nwords, float s2) {
  uint32_t zz = 0;
  if (w <= 8 && (uint64_t)off + 8 <= nwords) {
    uint64_t p[8];
#pragma unroll
    for (int q = 0; q < 8; q++) p[q] = planes[off + q];
#pragma unroll
    for (int q = 7; q >= 0; q--) zz = double_add_plane(zz, p[q]);
  } else if ((uint64_t)off + 12 <= nwords) {
    uint64_t p[12];
#pragma unroll
    for (int q = 0; q < 12; q++) p[q] = planes[off + q];
#pragma unroll
    for (int q = 11; q >= 0; q--) zz = double_add_plane(zz, p[q]);
  } else {
    for (int q = (int)w - 1; q >= 0; q--) zz = double_add_plane(zz, planes[off + (uint32_t)q]);
  }
  zz &= (1u << w) - 1u;
  return (float)unzigzag(zz) * s2;
}

// Overwrite the outliers of E[e0, e0 + D) (sorted positions) in the row values.
template <int C, typename OP>
__device__ __forceinline__ void patch_outliers(float (&v)[C], uint32_t e0, OP opos, OP oval,
                                               uint32_t nout) {
  constexpr uint32_t D = 64u * C;
  const uint32_t lane = threadIdx.x & 63;
  uint32_t lo = 0, hi = nout;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (opos[mid] < e0) lo = mid + 1;
    else hi = mid;
  }
  for (; lo < nout; lo++) {
    const uint32_t pos = opos[lo];
    if (pos >= e0 + D) break;
    const uint32_t d = pos - e0;
#pragma unroll
    for (uint32_t j = 0; j < C; j++)
      if (d == 64 * j + lane) v[j] = __uint_as_float(oval[lo]);
  }
}

// Un-zigzag two codes packed as 16-bit halves; returns them sign-extended.
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unzigzag_pair(uint32_t zz2, int& qa, int& qb) {
  asm volatile("" : "+v"(zz2));  // keeps the transpose whole (no split by demanded bits)
  const ushort2v z = __builtin_bit_cast(ushort2v, zz2);
  const short2v q = (short2v)(z >> (unsigned short)1) ^ -(short2v)(z & (unsigned short)1);
  qa = q.x;
  qb = q.y;
}

// Sum of the m width bytes at byte `off` (16-aligned) of a segment read
// through its buffer resource (reads past the segment return 0): 16-byte
// loads issued four at a time, bytes past m masked off, v_sad_u8 sums.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t sum_widths(__amdgpu_buffer_rsrc_t rseg, uint32_t off, uint32_t m) {
  uint32_t s = 0;
  for (uint32_t c0 = 0; 16 * c0 < m; c0 += 4) {
    u32x4v v[4];
#pragma unroll
    for (uint32_t i = 0; i < 4; i++) {
      const uint32_t at = 16 * (c0 + i);
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rseg, at < m ? off + at : kOff, 0, 0);
    }
#pragma unroll
    for (uint32_t i = 0; i < 4; i++)
#pragma unroll
      for (uint32_t d = 0; d < 4; d++) {
        const int vb = (int)m - (int)(16 * (c0 + i) + 4 * d);  // bytes of this word below m
        const uint32_t mask = vb >= 4 ? 0xFFFFFFFFu : (vb <= 0 ? 0u : (1u << (8 * vb)) - 1u);
        s = __builtin_amdgcn_sad_u8(v[i][d] & mask, 0u, s);
      }
  }
  return s;
}

// Decoder for D = 64*C, in two launches:
//   index   one wave per tile: locate and check the tile record, scan its
//           widths, and resolve every row to where its bit planes are (this
//           tile's record, or the earlier tile a reference points into):
//           per block (segment word offset << 4 | width), per row its kind,
//           first-occurrence index and outlier list
//   decode  one workgroup per tile: two rounds of loads (descriptors, then
//           plane words), the 32x32 transpose per block pair, stores
// Lane L of a pair loads the 32-bit half (L >> 5) of plane (L & 15) of block
// ((L >> 4) & 1); the encoder's transpose, its own inverse, leaves both
// blocks' zigzag codes of element L in lane L.
constexpr uint32_t kRowPlanes = 0, kRowRawRef = 1, kRowBad = 2, kRowOutliers = 0x100;
constexpr uint32_t kTileOk = 1, kTileRaw = 2, kTileHuff = 4;

// LDS of the decoder's index step (one tile)
template <int C>
struct DecIndexLds {
  DecShared sh;
  uint64_t rec;
  uint4 td[2];                     // flags, eb, segment offset; record offset, segment bytes
  uint4 drow[kTileRows];           // kind | outliers flag, first-occurrence index, counts, offset
  uint32_t dblk[kTileRows * C];    // plane-word offset << 4 | width
  uint32_t boff[kTileRows * C];    // the record's block plane offsets
  uint8_t width[kTileRows * C];    // the record's block widths
  uint16_t ofirst[kTileRows];      // the record's outliers of first occurrence u:
  uint16_t oend[kTileRows];        //   positions [ofirst[u], oend[u]) of its sorted list
};
// LDS accesses of one wave complete in order; this waits for them and keeps
// the compiler from moving accesses across.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wave 0 of a decode workgroup: locate and check tile `ticket` and describe
// where every row's values are (the tile descriptor td[2], row descriptors
// drow[64] and block descriptors dblk[64*C], all in LDS).  LDS written by
// one lane and read by others of the same wave is ordered by lds_sync.
// First index in [0, n) whose position is at least v in a sorted list of
// positions (n if none), eight probes per round trip: the probes split the
// range into nine parts and the count of probes below v picks the part.
// On a list that is not sorted (a corrupt stream) the result stays in
// [0, n] and every read stays in [0, n).
__device__ __forceinline__ uint32_t lower_bound8(const uint32_t* op, uint32_t n, uint32_t v) {
  uint32_t lo = 0, hi = n;
  while (hi - lo > 8) {
    const uint32_t span = hi - lo;
    uint32_t pr[8], c = 0;
#pragma unroll
    for (uint32_t q = 0; q < 8; q++) pr[q] = op[lo + (uint32_t)(((uint64_t)(q + 1) * span) / 9)];
#pragma unroll
    for (uint32_t q = 0; q < 8; q++) c += pr[q] < v ? 1u : 0u;
    const uint32_t nlo = c ? lo + (uint32_t)(((uint64_t)c * span) / 9) + 1 : lo;
    const uint32_t nhi = c < 8 ? lo + (uint32_t)(((uint64_t)(c + 1) * span) / 9) : hi;
    lo = nlo;
    hi = nhi > nlo ? nhi : nlo;
  }
  uint32_t pr[8], c = 0;
#pragma unroll
  for (uint32_t q = 0; q < 8; q++) pr[q] = lo + q < hi ? op[lo + q] : v;
#pragma unroll
  for (uint32_t q = 0; q < 8; q++) c += pr[q] < v ? 1u : 0u;
  return lo + c;
}

template <int C>
__device__ __forceinline__ uint32_t index_tile(const uint8_t* __restrict__ in, const DecArgs& a, uint32_t ticket,
                                           DecIndexLds<C>& x) {
  constexpr uint32_t D = 64u * C;
  DecShared& sh = x.sh;
  const uint32_t lane = threadIdx.x & 63;
  uint32_t tv = 0;  // the lines pulled into the caches ahead (kept alive by the caller)
  {
    // every lane runs the same checks on the same (wave-uniform) words, so
    // the reads and the arithmetic can be scalar; lane 0 stores the result
    uint64_t ro;
    dec_locate(a, in, ticket, sh, ro, &tv);
    if (lane == 0) x.rec = ro;
  }
  lds_sync();
  const uint32_t k = sh.tile, n = sh.n, rows = sh.rows;
  uint4* dt = x.td;
  const uint64_t seg_off = sh.seg_off, rec_off = x.rec, sbytes = sh.seg_bytes;
  uint32_t flags = 0;
  auto put_tile = [&]() {
    if (lane == 0) {
      dt[0] = make_uint4(flags, f2u(sh.eb), (uint32_t)seg_off, (uint32_t)(seg_off >> 32));
      dt[1] = make_uint4((uint32_t)rec_off, (uint32_t)(rec_off >> 32), (uint32_t)sbytes, 0u);
    }
  };
  if (!sh.ok || sbytes >= (1ull << 31)) {
    if (lane == 0) report_error(a.report, kDevErrCorrupt);
    put_tile();
    return tv;
  }
  {  // a segment's first tile checks its totals, tile 0 the chunk sizes
    bool good = k != 0 || seg_totals_ok(in + seg_off, sbytes, sh.ntiles, sh.rec_lo);
    if (ticket == 0) good = good && chunk_totals_ok(in, a.sh.P, sh.total);
    if (!good && lane == 0) report_error(a.report, kDevErrCorrupt);
  }
  if (n == 0) {
    flags = kTileOk;
    put_tile();
    return tv;
  }
  const uint8_t* sg = in + seg_off;
  const uint8_t* rec = in + rec_off;
  const uint32_t rec_in_seg = (uint32_t)(rec_off - seg_off);
  const uint32_t mode = sh.tl.mode, U = sh.tl.U, nout = sh.tl.nout;
  if (mode == 0) {
    flags = kTileOk | kTileRaw;
    put_tile();
    return tv;
  }
  if (mode == 2) {  // a Huffman record: ec_decode_huff_pair / ec_decode_huff and ec_fill_refs
    flags = kTileOk | kTileHuff;
    put_tile();
    return tv;
  }
  const uint32_t rb = rows <= 65536 ? 2 : 4;
  const uint64_t bitmap = sh.tl.bitmap;
  const uint32_t nblk = U * C;
  const uint32_t off_refs = sh.tl.off_refs, off_opos = sh.tl.off_opos, off_pl = sh.tl.off_pl;
  // widths and their exclusive scan (each lane owns up to four consecutive blocks)
  uint32_t wl[4], lsum = 0, badw = 0;
#pragma unroll
  for (uint32_t q = 0; q < 4; q++) {
    const uint32_t b = 4 * lane + q;
    wl[q] = b < nblk ? rec[16 + b] : 0u;
    badw |= wl[q] > 12;
    lsum += wl[q];
  }
  const uint32_t incl = wave_incl_u32(lsum);
  uint32_t run = incl - lsum;
#pragma unroll
  for (uint32_t q = 0; q < 4; q++) {
    const uint32_t b = 4 * lane + q;
    if (b < nblk) {
      x.width[b] = (uint8_t)wl[q];
      x.boff[b] = run;
    }
    run += wl[q];
  }
  const uint32_t sumw = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  const uint64_t seg_words = sbytes / 8;
  const uint32_t pl_word0 = (rec_in_seg + off_pl) / 8;  // off_pl and records are 8-aligned
  const bool bad = __any(badw) || (uint64_t)pl_word0 + sumw > seg_words;
  lds_sync();
  if (bad) {
    if (lane == 0) report_error(a.report, kDevErrCorrupt);
    put_tile();
    return tv;
  }
  flags = kTileOk;
  put_tile();

  // ---- the record's outliers by first occurrence (u = position / D) ----
  // Lane-parallel over the sorted positions: a run of equal u starts where the
  // previous position has another u and ends where the next one does.
  // Positions must increase strictly and stay below U D, else the stream is
  // reported corrupt (runs then may come out wrong, never out of [0, nout),
  // and the patch step checks each position).
  if (nout) {
    x.ofirst[lane] = 0;
    x.oend[lane] = 0;
    lds_sync();
    const uint32_t* op = reinterpret_cast<const uint32_t*>(rec + off_opos);
    bool obad = false;
    for (uint32_t g0 = 0; g0 < nout; g0 += 64) {
      const uint32_t g = g0 + lane;
      const uint32_t p = g < nout ? op[g] : 0u;
      const uint32_t pp = g >= 1 && g - 1 < nout ? op[g - 1] : 0u;
      const uint32_t pn = g + 1 < nout ? op[g + 1] : 0u;
      if (g < nout) {
        const uint32_t uo = p / D;
        obad |= uo >= U || (g >= 1 && pp >= p);
        if (uo < U) {
          if (g == 0 || pp / D != uo) x.ofirst[uo] = (uint16_t)g;
          if (g + 1 == nout || pn / D != uo) x.oend[uo] = (uint16_t)(g + 1);
        }
      }
    }
    if (__any(obad) && lane == 0) report_error(a.report, kDevErrCorrupt);
    lds_sync();
  }

  // ---- where every row's planes are ----
  if (lane < n) {
    const uint32_t i = lane, r = k * kTileRows + i;
    const uint64_t below = bitmap & ((1ull << i) - 1ull);
    uint32_t kind = kRowPlanes, u = 0, orec = rec_in_seg, onum = nout, oofs = rec_in_seg + off_opos;
    uint32_t bo[C], bw[C];
#pragma unroll
    for (uint32_t j = 0; j < C; j++) {
      bo[j] = 0;
      bw[j] = 0;
    }
    bool local = true;
    if ((bitmap >> i) & 1ull) {
      u = (uint32_t)__popcll(below);
    } else {
      const uint32_t jr = i - (uint32_t)__popcll(below);
      // windowed references: the root found by the roots pass (a literal, or
      // any row of a RAW tile), else the first occurrence the record names
      const uint32_t ref = sh.win ? a.w.tile_first[(uint64_t)ticket * kTileRows + i]
                           : rb == 2 ? reinterpret_cast<const uint16_t*>(rec + off_refs)[jr]
                                     : reinterpret_cast<const uint32_t*>(rec + off_refs)[jr];
      if (ref >= r) {
        kind = kRowBad;
      } else if (ref >= k * kTileRows) {
        const uint32_t i2 = ref - k * kTileRows;
        if ((bitmap >> i2) & 1ull) u = (uint32_t)__popcll(bitmap & ((1ull << i2) - 1ull));
        else kind = kRowBad;
      } else {
        local = false;
        const uint32_t k2 = ref / kTileRows, i2 = ref % kTileRows;
        DecTile t2 = locate_tile(sg, sbytes, sh.ntiles, rows, k2, D, true, sh.rec_lo, false, sh.win);
        if (!t2.ok || !(((t2.bitmap >> i2) & 1ull) || (sh.win && t2.mode == 0))) {
          kind = kRowBad;
        } else {
          orec = (uint32_t)(t2.rec - sg);
          onum = t2.nout;
          oofs = orec + t2.off_opos;
          if (t2.mode == 0) {
            kind = kRowRawRef;
            u = i2;
          } else {
            u = (uint32_t)__popcll(t2.bitmap & ((1ull << i2) - 1ull));
            uint32_t at = (orec + t2.off_pl) / 8 +
                          sum_widths(buf_rsrc(sg, (uint32_t)sbytes), orec + 16, u * C);
#pragma unroll
            for (uint32_t j = 0; j < C; j++) {
              const uint32_t w = t2.rec[16 + u * C + j];
              bw[j] = w;
              bo[j] = at;
              at += w;
              if (w > 12 || (uint64_t)at > seg_words) kind = kRowBad;
            }
          }
        }
      }
    }
    if (kind == kRowPlanes && local) {
#pragma unroll
      for (uint32_t j = 0; j < C; j++) {
        bw[j] = x.width[u * C + j];
        bo[j] = pl_word0 + x.boff[u * C + j];
      }
    }
    // the outliers of this row's first occurrence: positions [u*D, u*D + D)
    // of the sorted list of its record (values follow all onum positions)
    uint32_t ocnt = 0, ofirst = oofs;
    if (kind == kRowPlanes && onum && local) {  // this record: from the runs above
      const uint32_t f = x.ofirst[u], e = x.oend[u];
      ocnt = e > f ? e - f : 0u;
      ofirst = oofs + 4 * f;
    } else if (kind == kRowPlanes && onum) {  // an earlier tile's record: 8-way searches
      const uint32_t* op = reinterpret_cast<const uint32_t*>(sg + oofs);
      const uint32_t lo = lower_bound8(op, onum, u * D);
      const uint32_t e = lower_bound8(op, onum, u * D + D);
      ocnt = e > lo ? e - lo : 0u;
      ofirst = oofs + 4 * lo;
    }
    // x: the kind (| kRowOutliers when the row has outliers); y: first-occurrence
    // index; z: the row's outliers | its record's outliers << 16; w: offset of
    // the row's first outlier position (RAW copy rows: of the record)
    x.drow[i] = make_uint4(
        kind | (ocnt ? kRowOutliers : 0u), u, ocnt | (onum << 16), kind == kRowRawRef ? orec : ofirst);
#pragma unroll
    for (uint32_t j = 0; j < C; j++) x.dblk[i * C + j] = (bo[j] << 4) | bw[j];
  }
  return tv;
}

// Rows of one decode step (row i0, and i0 + 1 when C = 1) that need more than
// the transposed planes: outliers to patch, a first occurrence stored RAW
// (re-quantized), or a corrupt reference (zeros, reported).  v holds the
// transposed values when all_planes.  Rare, so kept out of line.
template <int C, int ROWS>
__device__ __forceinline__ void decode_rows_special(const DecArgs& a, const uint8_t* sg, float* yt,
                                                    uint32_t i0, uint32_t n, float eb, float s2,
                                                    const uint4* drow, const uint32_t* dblk) {
  constexpr uint32_t D = 64u * C;
  const uint32_t lane = threadIdx.x & 63;
  bool ok = true;
  for (uint32_t rr = 0; rr < (uint32_t)ROWS; rr++) {
    const uint32_t ir = i0 + rr;
    if (ir >= n) continue;
    uint4 ri = drow[ir];  // kind, first-occurrence index, outliers, offset
    ri.x &= 0xFFu;
    float vr[C];
#pragma unroll
    for (uint32_t j = 0; j < C; j++) vr[j] = 0.0f;
    bool okr = ri.x != kRowBad;
    if (ri.x == kRowPlanes) {
      // a plane row in a group with a RAW-copy or corrupt row: decode it alone
#pragma unroll
      for (uint32_t j = 0; j < C; j++) {
        const uint32_t dsc = dblk[ir * C + j], w = dsc & 15u, o = dsc >> 4;
        uint32_t zz = 0;
        for (uint32_t b = 0; b < w; b++) {
          const uint64_t wd = reinterpret_cast<const uint64_t*>(sg)[o + b];
          zz |= (uint32_t)((wd >> lane) & 1ull) << b;
        }
        vr[j] = (float)unzigzag(zz) * s2;
      }
    }
    if (ri.x == kRowPlanes && (ri.z & 0xFFFFu)) {  // the row's outliers
      const uint32_t* op = reinterpret_cast<const uint32_t*>(sg + ri.w);
      patch_outliers<C>(vr, ri.y * D, op, op + (ri.z >> 16), ri.z & 0xFFFFu);
    } else if (ri.x == kRowRawRef) {  // first occurrence stored RAW: re-quantize it
      const float* src2 = reinterpret_cast<const float*>(sg + ri.w + 16) + (uint64_t)ri.y * D;
#pragma unroll
      for (uint32_t j = 0; j < C; j++) {
        const float xv = src2[64 * j + lane];
        int q;
        vr[j] = quantize(xv, eb, s2, q) ? xv : (float)q * s2;
      }
    }
    if (!okr) {
#pragma unroll
      for (uint32_t j = 0; j < C; j++) vr[j] = 0.0f;
      ok = false;
    }
    float* y = yt + (uint64_t)ir * D;
#pragma unroll
    for (uint32_t j = 0; j < C; j++) __builtin_nontemporal_store(vr[j], &y[64 * j + lane]);
  }
  if (!__all(ok) && lane == 0) report_error(a.report, kDevErrCorrupt);
}

// The decode step of one tile, after its index step (whole workgroup, no
// barrier), from its descriptors.
template <int C>
__device__ __forceinline__ void decode_tile(const uint8_t* __restrict__ in, float* __restrict__ yout,
                                            const DecArgs& a, uint32_t ticket, const uint4* td,
                                            const uint4* drow, const uint32_t* dblk) {
  constexpr uint32_t D = 64u * C;
  constexpr uint32_t kRowsPerWave = kTileRows / (kThreads / 64);  // 16
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t T = a.sh.T, B = a.sh.B;
  // tile coordinates (from the plan, not the stream)
  uint32_t s, k;
  ticket_coords(a.sh, a.seg_tile_base, ticket, s, k);
  const uint32_t pch = s / T, t = s % T;
  const uint32_t rows = chunk_row0(a.sh, pch + 1) - chunk_row0(a.sh, pch);
  const uint32_t n = rows ? min(kTileRows, rows - k * kTileRows) : 0u;
  if (n == 0) return;
  float* yt = yout + ((uint64_t)t * B + chunk_row0(a.sh, pch) + (uint64_t)k * kTileRows) * D;
  const uint4* dt = td;
  const uint32_t rbeg = wv * kRowsPerWave;
  // four blocks per transpose: group g of the wave holds its blocks
  // 4g .. 4g+3 in (row, block) order; lane L loads half L >> 5 of plane L & 7
  // (and of plane 8 + (L & 7)) of block (L >> 3) & 3 of the group
  constexpr uint32_t kGroupRows = 4 / C;
  constexpr uint32_t kGroups = kRowsPerWave * C / 4;
  const uint32_t gplane = lane & 7u, half = lane >> 5, gblk = (lane >> 3) & 3u;
  // the descriptors of the lane's row and block in every group (kind[]: the
  // row kind, with kRowOutliers when there are outliers to patch; garbage
  // for a raw or failed tile, and then unused)
  uint32_t kind[kGroups], desc[kGroups];
#pragma unroll
  for (uint32_t g = 0; g < kGroups; g++) {
    const uint32_t bi = 4 * g + gblk;
    const uint32_t i = min(rbeg + bi / C, n - 1);  // past n: a copy
    kind[g] = drow[i].x;
    desc[g] = dblk[i * C + bi % C];
  }
  const uint4 d0 = dt[0], d1 = dt[1];
  const uint32_t flags = d0.x;
  if (!(flags & kTileOk)) {  // the index step reported it
    for (uint32_t i = tid; i < n * D; i += kThreads) yt[i] = 0.0f;
    return;
  }
  if (flags & kTileHuff) return;  // decoded by ec_decode_huff_pair / ec_decode_huff and ec_fill_refs
  const uint8_t* sg = in + (((uint64_t)d0.w << 32) | d0.z);
  if (flags & kTileRaw) {  // RAW: rows verbatim
    const uint8_t* rec = in + (((uint64_t)d1.y << 32) | d1.x);
    const float4* s4 = reinterpret_cast<const float4*>(rec + 16);
    float4* y4 = reinterpret_cast<float4*>(yt);
    for (uint32_t i = tid; i < n * D / 4; i += kThreads) y4[i] = s4[i];
    return;
  }
  const float eb = __uint_as_float(d0.y), s2 = eb + eb;
  const __amdgpu_buffer_rsrc_t rseg = buf_rsrc(sg, d1.z);
  const __amdgpu_buffer_rsrc_t ry = buf_rsrc(yt, n * D * 4);
  const XposeSel xsel = xpose_sel(lane);
  // every plane word of the wave's rows (planes 8-11 exist only in blocks
  // wider than 8)
  uint32_t wlo[kGroups], whi[kGroups];
  bool wide = false;  // a block of the wave has planes 8-11
#pragma unroll
  for (uint32_t g = 0; g < kGroups; g++) wide = wide || (desc[g] & 15u) > 8;
  const bool any_wide = __any(wide);
#pragma unroll
  for (uint32_t g = 0; g < kGroups; g++) {
    const uint32_t w = desc[g] & 15u, o = desc[g] >> 4;
    const bool on = (kind[g] & 0xFFu) == kRowPlanes;
    wlo[g] = buf_ld_u32(rseg, on && gplane < w ? (2 * (o + gplane) + half) * 4 : kOff);
    whi[g] = any_wide ? buf_ld_u32(rseg, on && gplane + 8 < w ? (2 * (o + 8 + gplane) + half) * 4 : kOff) : 0u;
  }
  uint32_t special = 0;  // groups with RAW copies or corrupt rows: done last
  uint32_t patch = 0;    // groups with outliers: their raw values are stored last
#pragma unroll
  for (uint32_t g = 0; g < kGroups; g++) {
    const uint32_t i0 = rbeg + g * kGroupRows;
    if (i0 < n) {  // (no early exit: the loop must unroll to keep the words in registers)
      if (__all((kind[g] & 0xFFu) == kRowPlanes)) {
        if (__any(kind[g] & kRowOutliers)) patch |= 1u << g;
        // lane L: element L of the four blocks, low bytes of the codes, and
        // the high bits when a block is wider than 8
        const uint32_t ylo = xpose32(wlo[g], xsel);
        const uint32_t yhi = __ballot(whi[g] != 0) ? xpose32(whi[g], xsel) : 0u;
        int q[4];
        unzigzag_pair(__builtin_amdgcn_perm(yhi, ylo, 0x05010400u), q[0], q[1]);
        unzigzag_pair(__builtin_amdgcn_perm(yhi, ylo, 0x07030602u), q[2], q[3]);
        // rows past n fall outside ry's range; streaming stores (the output is
        // not read again here, and dirty lines left in the caches would be
        // written back while the next pass reads its input); the row offset
        // is wave-uniform and goes in the scalar offset
#pragma unroll
        for (uint32_t kk = 0; kk < 4; kk++)
          __builtin_amdgcn_raw_buffer_store_b32(
              f2u((float)q[kk] * s2), ry, 4 * lane,
              __builtin_amdgcn_readfirstlane(((i0 + kk / C) * D + 64 * (kk % C)) * 4), kCacheStream);
      } else {
        special |= 1u << g;
      }
    }
  }
  // outliers: the raw values over the stored codes (same wave, after its
  // stores are performed)
  if (patch) {
    wait_vm();
    for (uint32_t g = 0; g < kGroups; g++) {
      if (!((patch >> g) & 1u)) continue;
      for (uint32_t rr = 0; rr < kGroupRows; rr++) {
        const uint32_t ir = rbeg + g * kGroupRows + rr;
        if (ir >= n) continue;
        const uint4 ri = drow[ir];
        const uint32_t cnt = ri.z & 0xFFFFu;
        if (!(ri.x & kRowOutliers) || cnt == 0) continue;
        const uint32_t* op = reinterpret_cast<const uint32_t*>(sg + ri.w);
        const uint32_t* ov = op + (ri.z >> 16);
        for (uint32_t q = lane; q < cnt; q += 64) {
          const uint32_t d = op[q] - ri.y * D;  // element within the row
          if (d < D) yt[(uint64_t)ir * D + d] = __uint_as_float(ov[q]);
        }
      }
    }
  }
  // the rare groups, row by row
  for (uint32_t g = 0; g < kGroups; g++) {
    if (!((special >> g) & 1u)) continue;
    decode_rows_special<C, kGroupRows>(a, sg, yt, rbeg + g * kGroupRows, n, eb, s2, drow, dblk);
  }
}

// Two tiles per workgroup: waves 0 and 1 index both at once (their chains of
// dependent stream reads overlap), then the whole workgroup decodes one after
// the other.
constexpr uint32_t kDecTiles = 2;
template <int C>
__global__ void __launch_bounds__(kThreads) ec_decode_fast(const uint8_t* __restrict__ in,
                                                          float* __restrict__ yout, DecArgs a) {
  __shared__ DecIndexLds<C> xi[kDecTiles];
  const uint32_t wv = wave_id(), t0 = blockIdx.x * kDecTiles;
  uint32_t tv = 0;
  if (wv < kDecTiles && t0 + wv < a.sh.ntiles) tv = index_tile<C>(in, a, t0 + wv, xi[wv]);
  asm volatile("" ::"v"(tv));  // the lines the index step pulled ahead are in (see touch_lines)
  __syncthreads();
  for (uint32_t q = 0; q < kDecTiles && t0 + q < a.sh.ntiles; q++)
    decode_tile<C>(in, yout, a, t0 + q, xi[q].td, xi[q].drow, xi[q].dblk);
}

// ---------------------------------------------------------------------------
// decoding Huffman segments
//   books    per segment (one wave): the codebook of a Huffman segment copied
//            out of the stream (zero-padded; a placeholder for the others),
//            then the Huffman coder's table builder (ec_huffman.hip)
//   (the bit-plane decoder skips Huffman tiles)
//   decode   two Huffman tiles per wave (D = 64, 128; one per wave at
//            D = 256): chunks decoded one per lane by table lookups into
//            LDS, first-occurrence rows dequantized with their outliers
//   refs     per Huffman tile: repeated rows copied from their first
//            occurrences' decoded rows (re-quantized from a RAW record)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) ec_hbook_copy(DecArgs a) {
  __shared__ DecShared shs[kThreads / 64];
  const uint32_t lane = threadIdx.x & 63, wv = wave_id();
  const uint32_t s = blockIdx.x * (kThreads / 64) + wv;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.w.hstat[2] = 0;  // the table builder's zero word
  if (s >= a.sh.nseg) return;
  uint64_t ro;
  dec_locate(a, a.in, a.seg_tile_base[s], shs[wv], ro);
  wave_lds_wait();
  const DecShared& sh = shs[wv];
  uint8_t* bk = a.w.hdbooks + (uint64_t)s * kBookStride;
  uint64_t avail = 0;
  const uint8_t* src = a.in;
  if (sh.seg_ok && sh.hseg) {
    const uint64_t at = 32 + align_up(4ull * sh.ntiles, 16);  // after the tile directory
    src = a.in + sh.seg_off + at;
    avail = min(sh.seg_bytes - at, (uint64_t)kBookStride);
  }
  // every byte load of the lane in flight before the first store (a loop of
  // load-store pairs waited for each load in turn)
  constexpr uint32_t kPer = (kBookStride + 63) / 64;
  uint8_t v[kPer];
#pragma unroll
  for (uint32_t q = 0; q < kPer; q++) {
    const uint32_t i = 64 * q + lane;
    v[q] = i < avail ? src[i] : (uint8_t)(i == 0 && avail == 0 ? 1 : 0);
  }
#pragma unroll
  for (uint32_t q = 0; q < kPer; q++) {
    const uint32_t i = 64 * q + lane;
    if (i < kBookStride) bk[i] = v[q];
  }
}

// One wave per Huffman tile: lane c decodes chunk c of E (at most 64 chunks
// of 256 codes) by 12-bit table lookups in LDS, and stores every group of 8
// values straight into its first-occurrence row; the record's outliers are
// written over them afterwards.
template <int C>
__global__ void __launch_bounds__(64) ec_decode_huff(const uint8_t* __restrict__ in,
                                                    float* __restrict__ yout, DecArgs a) {
  constexpr uint32_t D = 64u * C, kMaxCh = kTileRows * D / 256;
  static_assert(kMaxCh <= 64, "one chunk per lane");
  // a record's words are staged in LDS when they average at most 56 per chunk
  // (a code of about 7 bits; larger records are read from global memory)
  constexpr uint32_t kStage = kMaxCh * 56;
  __shared__ DecShared sh;
  __shared__ __align__(16) uint16_t s_lut[kHuffTable];
  __shared__ uint32_t s_words[kStage];
  __shared__ uint8_t s_urow[kTileRows];
  const uint32_t lane = threadIdx.x;
  const uint32_t ticket = blockIdx.x;
  {
    uint64_t ro;
    dec_locate(a, in, ticket, sh, ro);
  }
  wave_lds_wait();
  // a Huffman segment's codebook is checked by the segment's first tile
  if (lane == 0 && sh.seg_ok && sh.hseg && sh.tile == 0) {
    const uint8_t* bk = a.w.hdbooks + (uint64_t)sh.seg * kBookStride;
    const bool empty = bk[0] == 1 && bk[1] == 0 && bk[2] == 0 && bk[3] == 0;
    if (!a.w.hvalid[sh.seg] && !empty) report_error(a.report, kDevErrCorrupt);
  }
  if (!sh.ok || sh.n == 0 || sh.tl.mode != 2) return;  // checked and reported elsewhere
  const DecTile tl = sh.tl;
  const uint32_t seg = sh.seg, n = sh.n, nout = tl.nout, nE = tl.U * D, nch = tl.nch;
  const bool book_ok = a.w.hvalid[seg] != 0;
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.w.hlut + (uint64_t)seg * kHuffTable);
#pragma unroll
    for (uint32_t i = 0; i < kHuffTable * 2 / 16 / 64; i++)
      reinterpret_cast<uint4*>(s_lut)[64 * i + lane] = src[64 * i + lane];
  }
  unique_rows(tl.bitmap, s_urow);
  wave_lds_wait();
  float* yt = yout + ((uint64_t)(seg % a.sh.T) * a.sh.B + chunk_row0(a.sh, seg / a.sh.T) +
                      (uint64_t)sh.tile * kTileRows) * D;
  const uint64_t wavail = (tl.avail - tl.off_w) / 4;  // words the segment still holds
  const uint32_t* ct = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_ct);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_w);
  const float s2 = sh.eb + sh.eb;
  bool bad = (nE > 0 && !book_ok) || ct[0] != 0;
  // the record's words into LDS when they fit and lie inside the segment
  const uint32_t total = ct[nch];
  const bool staged = total <= kStage && (uint64_t)total <= wavail;
  if (staged) {  // eight loads per lane in flight before their stores
    for (uint32_t i0 = 0; i0 < total; i0 += 8 * 64) {
      uint32_t v[8];
#pragma unroll
      for (uint32_t q = 0; q < 8; q++) {
        const uint32_t i = i0 + 64 * q + lane;
        v[q] = i < total ? words[i] : 0u;
      }
#pragma unroll
      for (uint32_t q = 0; q < 8; q++) {
        const uint32_t i = i0 + 64 * q + lane;
        if (i < total) s_words[i] = v[q];
      }
    }
  }
  wave_lds_wait();
  if (lane < nch && !bad) {
    // every chunk ends exactly in its last word (at most 96 words for 256 codes
    // of at most 12 bits), and the next one starts right after it
    const uint32_t c = lane, w0 = ct[c], w1 = ct[c + 1];
    const uint32_t rem = min(256u, nE - 256 * c);
    bad = !(w0 < w1 && w1 - w0 <= 96u && w1 <= total && (uint64_t)total <= wavail);
    // groups of codes of one row (D is a multiple of 32) into their row
    auto put = [&](uint32_t g, const uint32_t* pk, uint32_t cnt) {
      const uint32_t e = 256 * c + g;
      float* y = yt + (uint64_t)s_urow[e / D] * D + e % D;
      for (uint32_t k0 = 0; k0 < cnt; k0 += 4) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const uint32_t kk = k0 + k;
          v[k] = (float)((int)((pk[kk >> 1] >> (16 * (kk & 1))) & 0xFFFFu) - 2047) * s2;
        }
        if (k0 + 4 <= cnt) {
          *reinterpret_cast<float4*>(y + k0) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (uint32_t k = 0; k0 + k < cnt; k++) y[k0 + k] = v[k];
        }
      }
    };
    if (!bad && staged) {
      bad = !hd::decode_chunk_lds_sink(s_words + w0, w1 - w0, rem, s_lut,
                                       [&](uint32_t g, const uint32_t (&pk)[16], uint32_t cnt) { put(g, pk, cnt); },
                                       false);
    } else if (!bad) {
      bad = !hd::decode_chunk_sink(words + w0, w1 - w0, rem, s_lut,
                                   [&](uint32_t g, const uint32_t (&pk)[4], uint32_t cnt) { put(g, pk, cnt); },
                                   false);
    }
  }
  const uint32_t* opos = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_opos);
  const uint32_t* oval = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_oval);
  for (uint32_t g = lane; g < nout; g += 64) bad = bad || opos[g] >= nE || (g > 0 && opos[g - 1] >= opos[g]);
  wait_vm();  // this wave's stores are performed before any rewrite of the same words
  if (__ballot(bad) != 0) {
    for (uint32_t i = lane; i < n * D; i += 64) yt[i] = 0.0f;
    if (lane == 0) report_error(a.report, kDevErrCorrupt);
    return;
  }
  for (uint32_t g = lane; g < nout; g += 64) {
    const uint32_t p = opos[g];
    yt[(uint64_t)s_urow[p / D] * D + p % D] = __uint_as_float(oval[g]);
  }
}

// Huffman tiles of D = 64 and 128 (at most 32 chunks each), two per wave:
// half h decodes the chunks of tile 2 blockIdx.x + h, one per lane, so that
// every lane decodes and the workgroups (a table and two tiles' words in
// LDS, about 22 KB) all fit the chip at once.  Two tiles of one segment
// share the decode table; tiles of two segments, or a tile whose words do
// not fit half the stage, take one pass each with the whole stage.
// Checks, staging and the outlier pass are those of ec_decode_huff, per tile.
template <int C>
__global__ void __launch_bounds__(64) ec_decode_huff_pair(const uint8_t* __restrict__ in,
                                                         float* __restrict__ yout, DecArgs a) {
  constexpr uint32_t D = 64u * C, kMaxCh = kTileRows * D / 256;
  static_assert(kMaxCh <= 32, "one chunk per lane of a half-wave");
  // half the stage: a record's words averaging at most 52 per chunk
  constexpr uint32_t kStage = kMaxCh * 52;
  __shared__ DecShared sh[2];
  __shared__ __align__(16) uint16_t s_lut[kHuffTable];
  __shared__ uint32_t s_words[2][kStage];
  __shared__ uint8_t s_urow[2][kTileRows];
  const uint32_t lane = threadIdx.x, h = lane >> 5, hl = lane & 31;
  const uint32_t t0 = 2 * blockIdx.x;
  uint32_t act = 0;  // bit q: tile t0 + q is a Huffman tile, decoded here
#pragma unroll
  for (uint32_t q = 0; q < 2; q++) {
    if (t0 + q >= a.sh.ntiles) continue;
    uint64_t ro;
    dec_locate(a, in, t0 + q, sh[q], ro);
    wave_lds_wait();
    // a Huffman segment's codebook is checked by the segment's first tile
    if (lane == 0 && sh[q].seg_ok && sh[q].hseg && sh[q].tile == 0) {
      const uint8_t* bk = a.w.hdbooks + (uint64_t)sh[q].seg * kBookStride;
      const bool empty = bk[0] == 1 && bk[1] == 0 && bk[2] == 0 && bk[3] == 0;
      if (!a.w.hvalid[sh[q].seg] && !empty) report_error(a.report, kDevErrCorrupt);
    }
    if (sh[q].ok && sh[q].n != 0 && sh[q].tl.mode == 2) act |= 1u << q;  // others: checked elsewhere
  }
  act = uniform32(act);
  if (act == 0) return;
  // per tile: its record's chunk table and words, outliers, output rows
  struct TV {
    const uint32_t* ct;
    const uint32_t* words;
    const uint32_t* opos;
    const uint32_t* oval;
    float* yt;
    uint64_t wavail;
    uint32_t seg, n, nE, nch, nout, total;
    float s2;
    bool staged, tbad;
  };
  TV tv[2];
#pragma unroll
  for (uint32_t q = 0; q < 2; q++) {
    TV& v = tv[q];
    v = TV{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 0, 0, 0, 0, 0, 0.0f, false, false};
    if (!((act >> q) & 1u)) continue;
    const DecTile tl = sh[q].tl;
    v.seg = sh[q].seg;
    v.n = sh[q].n;
    v.nE = tl.U * D;
    v.nch = tl.nch;
    v.nout = tl.nout;
    v.ct = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_ct);
    v.words = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_w);
    v.opos = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_opos);
    v.oval = reinterpret_cast<const uint32_t*>(tl.rec + tl.off_oval);
    v.yt = yout + ((uint64_t)(v.seg % a.sh.T) * a.sh.B + chunk_row0(a.sh, v.seg / a.sh.T) +
                   (uint64_t)sh[q].tile * kTileRows) * D;
    v.wavail = (tl.avail - tl.off_w) / 4;  // words the segment still holds
    v.s2 = sh[q].eb + sh[q].eb;
    v.total = v.ct[v.nch];
    v.staged = v.total <= kStage && (uint64_t)v.total <= v.wavail;  // fits half the stage
    v.tbad = (v.nE > 0 && a.w.hvalid[v.seg] == 0) || v.ct[0] != 0;
  }
  // one pass for both tiles when they share a table and each fits half the
  // stage; else one pass per tile, which then has the whole stage (any valid
  // tile fits it: at most 96 words per chunk)
  static_assert(kMaxCh * 96 <= 2 * kStage, "a tile's words fit the whole stage");
  const bool split = act == 3u && (tv[0].seg != tv[1].seg || !tv[0].staged || !tv[1].staged);
  for (uint32_t pass = 0; pass < (split ? 2u : 1u); pass++) {
    const uint32_t pm = split ? (1u << pass) : act;  // the tiles of this pass
    const bool alone = pm != 3u;                       // one tile: the whole stage
    const uint32_t cap = alone ? 2 * kStage : kStage;
    bool st[2];  // the tile's words are staged (at s_words[q], or the whole stage when alone)
#pragma unroll
    for (uint32_t q = 0; q < 2; q++)
      st[q] = ((pm >> q) & 1u) && tv[q].total <= cap && (uint64_t)tv[q].total <= tv[q].wavail;
    uint32_t* const base0 = &s_words[0][0];
    uint32_t* const base1 = alone ? base0 : &s_words[1][0];
    {
      const uint32_t lseg = (pm & 1u) ? tv[0].seg : tv[1].seg;
      const uint4* src = reinterpret_cast<const uint4*>(a.w.hlut + (uint64_t)lseg * kHuffTable);
#pragma unroll
      for (uint32_t i = 0; i < kHuffTable * 2 / 16 / 64; i++)
        reinterpret_cast<uint4*>(s_lut)[64 * i + lane] = src[64 * i + lane];
    }
#pragma unroll
    for (uint32_t q = 0; q < 2; q++)
      if ((pm >> q) & 1u) unique_rows(sh[q].tl.bitmap, s_urow[q]);
    // both tiles' words into LDS, eight loads per lane and tile in flight
    const uint32_t tot0 = st[0] ? tv[0].total : 0u;
    const uint32_t tot1 = st[1] ? tv[1].total : 0u;
    for (uint32_t i0 = 0; i0 < max(tot0, tot1); i0 += 8 * 64) {
      uint32_t v0[8], v1[8];
#pragma unroll
      for (uint32_t k = 0; k < 8; k++) {
        const uint32_t i = i0 + 64 * k + lane;
        v0[k] = i < tot0 ? tv[0].words[i] : 0u;
        v1[k] = i < tot1 ? tv[1].words[i] : 0u;
      }
#pragma unroll
      for (uint32_t k = 0; k < 8; k++) {
        const uint32_t i = i0 + 64 * k + lane;
        if (i < tot0) base0[i] = v0[k];
        if (i < tot1) base1[i] = v1[k];
      }
    }
    wave_lds_wait();
    bool dbad = false;
    {
      const TV& v = h ? tv[1] : tv[0];
      if (((pm >> h) & 1u) && hl < v.nch && !v.tbad) {
        // every chunk ends exactly in its last word (at most 96 words for 256
        // codes of at most 12 bits), and the next one starts right after it
        const uint32_t c = hl, w0 = v.ct[c], w1 = v.ct[c + 1];
        const uint32_t rem = min(256u, v.nE - 256 * c);
        dbad = !(w0 < w1 && w1 - w0 <= 96u && w1 <= v.total && (uint64_t)v.total <= v.wavail);
        const uint8_t* urow = s_urow[h];
        float* const yt = v.yt;
        const float s2 = v.s2;
        // groups of codes of one row (D is a multiple of 32) into their row
        auto put = [&](uint32_t g, const uint32_t* pk, uint32_t cnt) {
          const uint32_t e = 256 * c + g;
          float* y = yt + (uint64_t)urow[e / D] * D + e % D;
          for (uint32_t k0 = 0; k0 < cnt; k0 += 4) {
            float f[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
              const uint32_t kk = k0 + k;
              f[k] = (float)((int)((pk[kk >> 1] >> (16 * (kk & 1))) & 0xFFFFu) - 2047) * s2;
            }
            if (k0 + 4 <= cnt) {
              *reinterpret_cast<float4*>(y + k0) = make_float4(f[0], f[1], f[2], f[3]);
            } else {
              for (uint32_t k = 0; k0 + k < cnt; k++) y[k0 + k] = f[k];
            }
          }
        };
        if (!dbad && (h ? st[1] : st[0])) {
          dbad = !hd::decode_chunk_lds_sink((h ? base1 : base0) + w0, w1 - w0, rem, s_lut,
                                            [&](uint32_t g, const uint32_t (&pk)[16], uint32_t cnt) { put(g, pk, cnt); },
                                            false);
        } else if (!dbad) {
          dbad = !hd::decode_chunk_sink(v.words + w0, w1 - w0, rem, s_lut,
                                        [&](uint32_t g, const uint32_t (&pk)[4], uint32_t cnt) { put(g, pk, cnt); },
                                        false);
        }
      }
    }
    wait_vm();  // this wave's stores are performed before any rewrite of the same words
    const uint64_t dbm = __ballot(dbad);
#pragma unroll
    for (uint32_t q = 0; q < 2; q++) {
      if (!((pm >> q) & 1u)) continue;
      const TV& v = tv[q];
      bool bad = v.tbad || (q ? (dbm >> 32) : (dbm & 0xFFFFFFFFull)) != 0;
      for (uint32_t g = lane; g < v.nout; g += 64)
        bad = bad || v.opos[g] >= v.nE || (g > 0 && v.opos[g - 1] >= v.opos[g]);
      if (__ballot(bad) != 0) {
        for (uint32_t i = lane; i < v.n * D; i += 64) v.yt[i] = 0.0f;
        if (lane == 0) report_error(a.report, kDevErrCorrupt);
        continue;
      }
      for (uint32_t g = lane; g < v.nout; g += 64) {
        const uint32_t p = v.opos[g];
        v.yt[(uint64_t)s_urow[q][p / D] * D + p % D] = __uint_as_float(v.oval[g]);
      }
    }
    wave_lds_wait();  // the next pass rewrites the table
  }
}

// Rows of a Huffman tile that repeat an earlier row: their first occurrences
// are decoded (this or an earlier Huffman tile) or stored RAW (re-quantized).
constexpr uint32_t kRefNone = 0, kRefCopy = 1, kRefRaw = 2, kRefBad = 3;
template <int C>
__global__ void __launch_bounds__(kThreads) ec_fill_refs(const uint8_t* __restrict__ in,
                                                        float* __restrict__ yout, DecArgs a) {
  constexpr uint32_t D = 64u * C;
  __shared__ DecShared sh;
  __shared__ uint32_t s_kind[kTileRows], s_src[kTileRows], s_roff[kTileRows];
  const uint32_t tid = threadIdx.x, lane = tid & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x;
  if (wv == 0) {
    uint64_t ro;
    dec_locate(a, in, ticket, sh, ro);
  }
  __syncthreads();
  if (!sh.ok || sh.n == 0 || sh.tl.mode != 2) return;
  const DecTile tl = sh.tl;
  const uint32_t seg = sh.seg, k = sh.tile, n = sh.n, rows = sh.rows;
  const uint8_t* sg = in + sh.seg_off;
  if (wv == 0) {
    uint32_t kind = kRefNone, src = 0, roff = 0;
    if (lane < n && !((tl.bitmap >> lane) & 1ull)) {
      const uint32_t rb = rows <= 65536 ? 2 : 4;
      const uint32_t j = lane - (uint32_t)__popcll(tl.bitmap & lanes_below());
      // windowed references: the root from the roots pass
      const uint32_t ref = sh.win ? a.w.tile_first[(uint64_t)ticket * kTileRows + lane]
                           : rb == 2 ? reinterpret_cast<const uint16_t*>(tl.rec + 16)[j]
                                     : reinterpret_cast<const uint32_t*>(tl.rec + 16)[j];
      const uint32_t k2 = ref / kTileRows, i2 = ref % kTileRows;
      kind = kRefBad;
      src = ref;
      if (ref >= k * kTileRows + lane) {
        // a reference must name an earlier row
      } else if (k2 == k) {
        if ((tl.bitmap >> i2) & 1ull) kind = kRefCopy;
      } else {
        const DecTile t2 =
            locate_tile(sg, sh.seg_bytes, sh.ntiles, rows, k2, D, true, sh.rec_lo, true, sh.win);
        if (t2.ok && (((t2.bitmap >> i2) & 1ull) || (sh.win && t2.mode == 0))) {
          kind = t2.mode == 0 ? kRefRaw : kRefCopy;
          roff = (uint32_t)(t2.rec - sg);
        }
      }
    }
    s_kind[lane] = kind;
    s_src[lane] = src;
    s_roff[lane] = roff;
  }
  __syncthreads();
  float* yseg = yout + ((uint64_t)(seg % a.sh.T) * a.sh.B + chunk_row0(a.sh, seg / a.sh.T)) * D;
  const float eb = sh.eb, s2 = eb + eb;
  bool bad = false;
  for (uint32_t i = wv; i < n; i += kThreads / 64) {
    const uint32_t kind = s_kind[i], src = s_src[i];
    if (kind == kRefNone) continue;
    float v[C];
#pragma unroll
    for (uint32_t j = 0; j < C; j++) {
      if (kind == kRefCopy) {
        v[j] = yseg[(uint64_t)src * D + 64 * j + lane];
      } else if (kind == kRefRaw) {
        const float xv = reinterpret_cast<const float*>(sg + s_roff[i] + 16)[(src % kTileRows) * D + 64 * j + lane];
        int q;
        v[j] = quantize(xv, eb, s2, q) ? xv : (float)q * s2;
      } else {
        v[j] = 0.0f;
      }
    }
    bad = bad || kind == kRefBad;
    float* y = yseg + ((uint64_t)k * kTileRows + i) * D;
#pragma unroll
    for (uint32_t j = 0; j < C; j++) y[64 * j + lane] = v[j];
  }
  if (bad && lane == 0) report_error(a.report, kDevErrCorrupt);
}

// ---------------------------------------------------------------------------
// windowed references for D = 64*C (the vector-based LZ of section III-D with
// the extended window of section III-E), after the quantize pass: one wave
// per tile, lane i for segment row r = 64k + i.  The row hashes of the tile
// and of the 256 rows before it (as far as a window of at most 255 reaches)
// go to LDS; each row scans back from distance 1 for an equal hash, and a hash
// hit is its match when the two rows' keys are equal (compared by the whole
// wave, as the hash-table insertion compares).  tile_first gets the match,
// or the row itself when none is within the window.
// ---------------------------------------------------------------------------
template <int C>
__global__ void __launch_bounds__(kThreads) ec_window_fast(EncArgs a) {
  constexpr uint32_t D = 64u * C;
  constexpr uint32_t kBack = 256;
  __shared__ uint32_t s_h[kThreads / 64][kBack + kTileRows];
  const uint32_t lane = threadIdx.x & 63, wv = wave_id();
  const uint32_t ticket = blockIdx.x * (kThreads / 64) + wv;
  if (ticket >= a.sh.ntiles) return;  // whole waves; no workgroup barrier follows
  const TileCoord c = tile_coord(a, ticket);
  const uint32_t n = c.n, r = c.k * kTileRows + lane;
  const uint64_t rowi = (uint64_t)ticket * kTileRows + lane;
  if (n == 0 || a.w.seg_eb[c.s] == 0u) {
    if (lane < n) a.w.tile_first[rowi] = r;
    return;
  }
  // hs[j]: hash of segment row 64k - 256 + j (tile k - b has ticket - b);
  // entries before the segment are never read
  uint32_t* hs = s_h[wv];
#pragma unroll
  for (uint32_t q = 0; q <= kBack / kTileRows; q++) {
    const uint32_t back = kBack / kTileRows - q;
    if (c.k >= back) hs[q * kTileRows + lane] = a.w.stage_slot[(uint64_t)(ticket - back) * kTileRows + lane];
  }
  wave_lds_wait();
  const float eb = __uint_as_float(a.w.seg_eb[c.s]), s2 = eb + eb, r2 = 1.0f / s2;
  const float* xs = a.x + ((uint64_t)c.t * a.sh.B + chunk_row0(a.sh, c.pch)) * D;
  const uint32_t h = hs[kBack + lane];
  const uint32_t dmax = lane < n ? min(a.window, r) : 0u;  // distances 1 .. dmax stay in the segment
  uint32_t d = 0;      // distances up to d are ruled out
  uint32_t match = r;  // no match: a literal
  bool active = lane < n;
  while (__ballot(active) != 0) {
    bool need = false;
    uint32_t cand = 0;
    if (active) {  // the nearest hash hit past d, eight distances at a time
      uint32_t dd = d + 1;
      bool hit = false;
      while (dd <= dmax) {
        uint32_t bits = 0;
#pragma unroll
        for (uint32_t u = 0; u < 8; u++) {
          const uint32_t e = min(dd + u, dmax);  // in 1 .. dmax
          bits |= (uint32_t)(hs[kBack + lane - e] == h && dd + u <= dmax) << u;
        }
        if (bits) {
          dd += (uint32_t)__builtin_ctz(bits);
          hit = true;
          break;
        }
        dd += 8;
      }
      if (hit) {
        need = true;
        cand = r - dd;
        d = dd;
      } else {
        active = false;
      }
    }
    // the hits, kCmp at a time with all their row loads in flight together
    constexpr int kCmp = C >= 4 ? 2 : 8 / C;
    uint64_t m = __ballot(need);
    while (m) {
      int Lk[kCmp];
      float va[kCmp][C], vb[kCmp][C];
#pragma unroll
      for (int kk = 0; kk < kCmp; kk++) {
        Lk[kk] = m ? __ffsll((long long)m) - 1 : -1;
        m &= m - 1;
        const int Ls = Lk[kk] < 0 ? Lk[0] : Lk[kk];  // no candidate: a copy of the first
        const uint32_t iL = __shfl(r, Ls), cL = __shfl(cand, Ls);
#pragma unroll
        for (int j = 0; j < C; j++) {
          va[kk][j] = xs[(uint64_t)cL * D + 64 * j + lane];
          vb[kk][j] = xs[(uint64_t)iL * D + 64 * j + lane];
        }
      }
#pragma unroll
      for (int kk = 0; kk < kCmp; kk++) {
        if (Lk[kk] < 0) continue;
        bool raw = true;
#pragma unroll
        for (int j = 0; j < C; j++) raw = raw && f2u(va[kk][j]) == f2u(vb[kk][j]);
        bool eq = __all(raw);
        if (!eq) {  // different bits: the same codes and outliers make the keys equal
          bool e = true;
#pragma unroll
          for (int j = 0; j < C; j++) {
            int qa, qb;
            const bool oa = quantize_fast(va[kk][j], eb, s2, r2, qa);
            const bool ob = quantize_fast(vb[kk][j], eb, s2, r2, qb);
            e = e && oa == ob && (oa ? f2u(va[kk][j]) == f2u(vb[kk][j]) : qa == qb);
          }
          eq = __all(e);
        }
        if ((int)lane == Lk[kk] && eq) {
          match = cand;
          active = false;
        }
      }
    }
  }
  if (lane < n) a.w.tile_first[rowi] = match;
}

// ---------------------------------------------------------------------------
// decoding windowed segments: every row's root, the row whose key it has that
// the decoders can read directly (a literal, or any row of a RAW tile).
//   links  one wave per tile: each repeated row of a coded tile links to its
//          match (the distance checked: 1 .. W and inside the segment, else
//          reported corrupt), every other row to itself
//   roots  one workgroup per segment: links always point back, so jumping
//          from link to link's link (in LDS) converges in log2(rows) rounds
// Links and then roots go to tile_first, where the decode kernels read them.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) ec_win_links(const uint8_t* __restrict__ in, DecArgs a) {
  __shared__ DecShared sh;
  const uint32_t lane = threadIdx.x, ticket = blockIdx.x;
  uint64_t ro;
  dec_locate(a, in, ticket, sh, ro);
  lds_sync();
  if (!sh.ok || sh.win == 0 || sh.n == 0) return;  // not windowed, or reported by the decoders
  const DecTile& t = sh.tl;
  const uint32_t r = sh.tile * kTileRows + lane, W = sh.win;
  uint32_t link = r;
  bool bad = false;
  if (t.mode != 0 && lane < sh.n && !((t.bitmap >> lane) & 1ull)) {
    const uint32_t j = lane - (uint32_t)__popcll(t.bitmap & lanes_below());
    const uint32_t dist = t.rec[t.off_refs + j];  // inside the record (checked by locate_tile)
    if (dist >= 1 && dist <= W && dist <= r) link = r - dist;
    else bad = true;
  }
  // links inside the tile jumped here already (six rounds reach across 64
  // rows): afterwards a row links to a root or to a row of an earlier tile
  const uint32_t r0 = sh.tile * kTileRows;
#pragma unroll
  for (int k = 0; k < 6; k++) {
    const uint32_t l2 = (uint32_t)__shfl((int)link, (int)(link >= r0 ? link - r0 : lane));
    if (link >= r0) link = l2;
  }
  if (lane < sh.n) a.w.tile_first[(uint64_t)ticket * kTileRows + lane] = link;
  if (bad) report_error(a.report, kDevErrCorrupt);
}

constexpr uint32_t kRootThreads = 1024;
__global__ void __launch_bounds__(kRootThreads) ec_win_roots(const uint8_t* __restrict__ in, DecArgs a) {
  constexpr uint32_t kPer = kWinMaxRows / kRootThreads;
  __shared__ uint16_t s_src[kWinMaxRows];
  __shared__ DecShared sh;
  const uint32_t tid = threadIdx.x, wv = wave_id();
  const uint32_t ticket0 = a.seg_tile_base[blockIdx.x];
  if (wv == 0) {
    uint64_t ro;
    dec_locate(a, in, ticket0, sh, ro);
  }
  __syncthreads();
  if (!sh.seg_ok || sh.win == 0 || sh.ntiles == 0 || sh.rows > kWinMaxRows) return;  // whole workgroup
  const uint32_t rows = sh.rows;
  uint32_t* lk = a.w.tile_first + (uint64_t)ticket0 * kTileRows;  // the segment's rows, in order
  // a tile whose record failed its checks wrote no links: its rows are roots
  // (their decode workgroups report the stream corrupt)
  for (uint32_t r = tid; r < rows; r += kRootThreads) {
    const uint32_t l = lk[r];
    s_src[r] = (uint16_t)(l < r ? l : r);
  }
  __syncthreads();
  for (;;) {
    uint16_t nv[kPer];
    bool changed = false;
#pragma unroll
    for (uint32_t q = 0; q < kPer; q++) {
      const uint32_t r = q * kRootThreads + tid;
      nv[q] = 0;
      if (r < rows) {
        const uint32_t l1 = s_src[r], l2 = s_src[l1];
        nv[q] = (uint16_t)l2;
        changed = changed || l2 != l1;
      }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t q = 0; q < kPer; q++) {
      const uint32_t r = q * kRootThreads + tid;
      if (r < rows) s_src[r] = nv[q];
    }
    if (!__syncthreads_or(changed)) break;
  }
  for (uint32_t r = tid; r < rows; r += kRootThreads) lk[r] = s_src[r];
}

// ---------------------------------------------------------------------------
// the library's own scratch for ec_compress_static (callers that cannot
// allocate): one copy per device, alive until the process ends
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[EC_STATIC_SCRATCH_BYTES];

__global__ void __launch_bounds__(kThreads) ec_copy_kernel(uint4* __restrict__ dst,
                                                          const uint4* __restrict__ src,
                                                          uint64_t n16) {
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
       i += (uint64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

// A call's last launch: its number into the pinned report, where the host
// waits for it (a release at system scope, so the report's other fields,
// written by the call's earlier kernels, are visible first)
__global__ void __launch_bounds__(64) ec_done_kernel(Report* r, uint32_t seq) {
  if (threadIdx.x == 0) __hip_atomic_store(&r->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

hipError_t launch_done(Report* r, uint32_t seq, hipStream_t s) {
  hipLaunchKernelGGL(ec_done_kernel, dim3(1), dim3(64), 0, s, r, seq);
  return hipGetLastError();
}

hipError_t static_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    // the array's name in host code is not a device address: every use goes
    // through the address the runtime reports for this device's copy
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_copy_words(void* dst, const void* src, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  uint64_t g = (n16 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(ec_copy_kernel, dim3((uint32_t)(g > 1024 ? 1024 : g)), dim3(kThreads), 0, s,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& a, uint32_t grid, hipStream_t s) {
  hipLaunchKernelGGL(ec_prep_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t set_encode_lds_limit(size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&ec_encode_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_encode(const EncArgs& a, hipStream_t s) {
  // with the range folded in, the quantize grid holds the range items too
  const dim3 grid(a.sh.ntiles + (a.fuse_range ? a.sh.T * a.range_items : 0u)), block(kThreads);
  switch (a.sh.D) {
    case 64:
      hipLaunchKernelGGL(ec_quantize_fast<1>, grid, block, 0, s, a);
      break;
    case 128:
      hipLaunchKernelGGL(ec_quantize_fast<2>, grid, block, 0, s, a);
      break;
    case 256:
      hipLaunchKernelGGL(ec_quantize_fast<4>, grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL(ec_encode_kernel, grid, block, encode_lds_bytes(a.sh.D), s, a);
  }
  return hipGetLastError();
}

bool encode_has_assembly(uint32_t D) { return D == 64 || D == 128 || D == 256; }

hipError_t launch_assemble_size(const EncArgs& a, hipStream_t s) {
  const dim3 blocks((a.sh.ntiles + kBlockTiles - 1) / kBlockTiles), sblock(kSizeThreads);
  switch (a.sh.D) {
    case 64: hipLaunchKernelGGL(ec_size_fast<1>, blocks, sblock, 0, s, a); break;
    case 128: hipLaunchKernelGGL(ec_size_fast<2>, blocks, sblock, 0, s, a); break;
    case 256: hipLaunchKernelGGL(ec_size_fast<4>, blocks, sblock, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_assemble_write(const EncArgs& a, hipStream_t s) {
  const dim3 tiles(a.sh.ntiles), block(kThreads);
  switch (a.sh.D) {
    case 64: hipLaunchKernelGGL(ec_write_fast<1>, tiles, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(ec_write_fast<2>, tiles, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(ec_write_fast<4>, tiles, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_assemble(const EncArgs& a, hipStream_t s) {
  const dim3 tiles(a.sh.ntiles), blocks((a.sh.ntiles + kBlockTiles - 1) / kBlockTiles);
  const dim3 block(kThreads), sblock(kSizeThreads);
  switch (a.sh.D) {
    case 64:
      hipLaunchKernelGGL(ec_size_fast<1>, blocks, sblock, 0, s, a);
      hipLaunchKernelGGL(ec_write_fast<1>, tiles, block, 0, s, a);
      break;
    case 128:
      hipLaunchKernelGGL(ec_size_fast<2>, blocks, sblock, 0, s, a);
      hipLaunchKernelGGL(ec_write_fast<2>, tiles, block, 0, s, a);
      break;
    case 256:
      hipLaunchKernelGGL(ec_size_fast<4>, blocks, sblock, 0, s, a);
      hipLaunchKernelGGL(ec_write_fast<4>, tiles, block, 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_window(const EncArgs& a, hipStream_t s) {
  const dim3 grid((a.sh.ntiles + kThreads / 64 - 1) / (kThreads / 64)), block(kThreads);
  switch (a.sh.D) {
    case 64: hipLaunchKernelGGL(ec_window_fast<1>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(ec_window_fast<2>, grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(ec_window_fast<4>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_window_roots(const DecArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ec_win_links, dim3(a.sh.ntiles), dim3(64), 0, s, a.in, a);
  hipLaunchKernelGGL(ec_win_roots, dim3(a.sh.nseg), dim3(kRootThreads), 0, s, a.in, a);
  return hipGetLastError();
}

hipError_t launch_distinct_raw(const EncArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ec_distinct_raw, dim3(a.sh.ntiles), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(ec_distinct_sum, dim3((a.sh.nseg + 3) / 4), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_huff_encode(const EncArgs& a, hipStream_t s) {
  const dim3 tiles(a.sh.ntiles), block(kThreads);
  const uint32_t segw = (a.sh.nseg + 3) / 4, blocks = (a.sh.ntiles + kBlockTiles - 1) / kBlockTiles;
  switch (a.sh.D) {
    case 64: hipLaunchKernelGGL(ec_hist_tiles<1>, tiles, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(ec_hist_tiles<2>, tiles, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(ec_hist_tiles<4>, tiles, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (a.reuse_books) hipLaunchKernelGGL(ec_book_reuse, dim3(segw), block, 0, s, a);
  hipError_t e = launch_seg_books(a.w.hhist, a.w.henc, a.w.hbooks, a.w.hstat,
                                  a.reuse_books ? a.w.hskip : nullptr, a.sh.nseg, s);
  if (e != hipSuccess) return e;
  switch (a.sh.D) {
    case 64: hipLaunchKernelGGL(ec_hsize_tiles<1>, tiles, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(ec_hsize_tiles<2>, tiles, block, 0, s, a); break;
    default: hipLaunchKernelGGL(ec_hsize_tiles<4>, tiles, block, 0, s, a); break;
  }
  hipLaunchKernelGGL(ec_seg_choose, dim3(segw), block, 0, s, a);
  hipLaunchKernelGGL(ec_items, dim3(blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_huff_write(const EncArgs& a, hipStream_t s) {
  const dim3 tiles(a.sh.ntiles), block(kThreads);
  switch (a.sh.D) {
    case 64: hipLaunchKernelGGL(ec_write_huff<1>, tiles, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(ec_write_huff<2>, tiles, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(ec_write_huff<4>, tiles, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_huff_tables(const DecArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(ec_hbook_copy, dim3((a.sh.nseg + 3) / 4), dim3(kThreads), 0, s, a);
  return launch_seg_luts(a.w.hdbooks, a.w.hstat + 2, a.w.hdenc, a.w.hlut, a.w.hvalid, a.w.hstat + 1,
                         a.sh.nseg, s);
}

hipError_t launch_huff_decode(const DecArgs& a, hipStream_t s) {
  const dim3 grid(a.sh.ntiles), block(kThreads);
  switch (a.sh.D) {
    case 64:
      hipLaunchKernelGGL(ec_decode_huff_pair<1>, dim3((a.sh.ntiles + 1) / 2), dim3(64), 0, s, a.in, a.y, a);
      hipLaunchKernelGGL(ec_fill_refs<1>, grid, block, 0, s, a.in, a.y, a);
      break;
    case 128:
      hipLaunchKernelGGL(ec_decode_huff_pair<2>, dim3((a.sh.ntiles + 1) / 2), dim3(64), 0, s, a.in, a.y, a);
      hipLaunchKernelGGL(ec_fill_refs<2>, grid, block, 0, s, a.in, a.y, a);
      break;
    case 256:
      hipLaunchKernelGGL(ec_decode_huff<4>, grid, dim3(64), 0, s, a.in, a.y, a);
      hipLaunchKernelGGL(ec_fill_refs<4>, grid, block, 0, s, a.in, a.y, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  const dim3 grid(a.sh.ntiles), block(kThreads);
  const dim3 grid2((a.sh.ntiles + kDecTiles - 1) / kDecTiles);
  switch (a.sh.D) {
    case 64:
      hipLaunchKernelGGL(ec_decode_fast<1>, grid2, block, 0, s, a.in, a.y, a);
      break;
    case 128:
      hipLaunchKernelGGL(ec_decode_fast<2>, grid2, block, 0, s, a.in, a.y, a);
      break;
    case 256:
      hipLaunchKernelGGL(ec_decode_fast<4>, grid2, block, 0, s, a.in, a.y, a);
      break;
    default:
      hipLaunchKernelGGL(ec_decode_kernel, grid, block, decode_lds_bytes(a.sh.D), s, a);
  }
  return hipGetLastError();
}

}  // namespace ec
