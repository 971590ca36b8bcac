// ec_huffman.hip -- canonical Huffman coder of quantization codes on gfx950
// (the lossless stage after the quantization encoder, arXiv 2407.04272
// section III-D "Huffman Encoding").  The stream layout and the rules that
// make the code unique are documented in include/ec_huffman.h.
//
// Encode: five launches on one stream.
//   clear   zero the histogram and the status word
//   hist    per-workgroup LDS histograms, merged by global atomics
//   book    one workgroup: sort the used symbols by frequency (bitonic, LDS),
//           build the tree with two queues (one lane, LDS), depths by pointer
//           jumping, length limit, lengths by rank, canonical codes by a
//           packed prefix count, codebook bytes
//   size    one wave per 256-symbol chunk: word count of the chunk
//   write   groups of chunks: offsets by a scan, then one wave per chunk packs
//           its codes (wave prefix of bit counts, LDS OR into a 96-word
//           buffer) and stores whole words
// Decode: two launches.
//   dec_book  one workgroup per segment: validate the codebook (workgroup 0
//             also zeroes the status word), canonical codes, a
//             4096-entry table from every 12-bit prefix to (symbol, length)
//   decode    128 chunks per workgroup: their words staged through LDS with
//             coalesced loads when they fit in 56 words per chunk on average
//             (else read from global memory), then one lane per chunk decodes
//             by table lookups, two words ahead of its bit buffer, and checks
//             that the chunk ends exactly in its last word.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ec.h"
#include "ec_huff_decode.h"
#include "ec_huffman.h"

namespace {

using ec::hd::decode_chunk;
using ec::hd::decode_chunk_lds;

constexpr int kNsym = (int)EC_HUFF_NSYM;      // 4095
constexpr int kMaxLen = (int)EC_HUFF_MAXLEN;  // 12
constexpr int kChunk = (int)EC_HUFF_CHUNK;    // 256
constexpr int kTable = 4096;                  // alphabet + one bin for invalid symbols
constexpr int kChunkWords = kChunk * kMaxLen / 32;  // 96: most words a chunk can take
constexpr int kMaxGroups = 2048;                    // chunk groups of size / write
constexpr int kMaxDepth = 64;  // a tree over fewer than 2^31 symbols is shallower
constexpr int kBookThreads = 1024;
constexpr int kThreads = 256;
constexpr int kDecChunks = 128;  // chunks (and lanes) per decode workgroup
constexpr int kStageWords = kDecChunks * 56;  // LDS words staged per decode workgroup

enum : uint32_t { kStBadSymbol = 1u, kStCorrupt = 2u, kStDepth = 4u };

// Workspace layout (bytes from the 256-byte aligned base) for nseg segments.
constexpr int kMaxSegments = (int)EC_HUFF_MAX_SEGMENTS;
constexpr size_t kBookStride = EC_HUFF_BOOK_MAX;

struct Ws {
  uint32_t* status;  // [0]: status bits of the last call
  uint32_t* valid;   // [nseg]: codebook of the segment passed validation (decode)
  uint32_t* hist;    // [nseg][4096]; bin 4095 counts symbols outside the alphabet
  uint32_t* enc;     // [nseg][4096]: len << 16 | code
  uint16_t* lut;     // [nseg][4096]: sym | len << 12, 0 = no code
  uint32_t* groups;  // [kMaxGroups]: words per encode group
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

size_t work_bytes(uint32_t nseg) {
  return 256 + round256(4ull * nseg) + (size_t)nseg * (4 + 4 + 2) * kTable + 4ull * kMaxGroups;
}

Ws ws_of(void* base, uint32_t nseg) {
  uint8_t* b = static_cast<uint8_t*>(base);
  Ws w;
  w.status = reinterpret_cast<uint32_t*>(b);
  b += 256;
  w.valid = reinterpret_cast<uint32_t*>(b);
  b += round256(4ull * nseg);
  w.hist = reinterpret_cast<uint32_t*>(b);
  b += (size_t)nseg * 4 * kTable;
  w.enc = reinterpret_cast<uint32_t*>(b);
  b += (size_t)nseg * 4 * kTable;
  w.lut = reinterpret_cast<uint16_t*>(b);
  b += (size_t)nseg * 2 * kTable;
  w.groups = reinterpret_cast<uint32_t*>(b);
  return w;
}

__device__ __forceinline__ void status_or(uint32_t* st, uint32_t bits) {
  __hip_atomic_fetch_or(st, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

// Inclusive prefix sum over the wave with DPP moves (no LDS round trips):
// shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes with no source
// add 0), then row 0's total into row 1 and row 2's into row 3 (broadcast of
// lane 15 of the row before), then lane 31's sum into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl(x), 63);
}

__device__ __forceinline__ uint64_t wave_incl64(uint64_t x) {
  const uint32_t ln = lane_id();
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t y = __shfl_up(x, d, 64);
    if (ln >= (uint32_t)d) x += y;
  }
  return x;
}

// Exclusive prefix sum over the workgroup (blockDim.x threads, a multiple of
// 64, at most 1024); *total gets the sum.  part holds 16 entries.
__device__ uint32_t block_excl(uint32_t x, uint32_t* part, uint32_t* total) {
  const uint32_t wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t inc = wave_incl(x);
  __syncthreads();
  if (lane_id() == 63) part[wv] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (uint32_t i = 0; i < nw; i++) {
    const uint32_t v = part[i];
    before += i < wv ? v : 0;
    all += v;
  }
  *total = all;
  return before + inc - x;
}

// ---------------------------------------------------------------------------
// Huffman tree of the sorted leaf weights wt[0, m) by two queues (leaves,
// then internal nodes in creation order; of two equal weights the leaf
// first): pr[v] gets the internal node that takes node v (internal node
// m + j is the j-th created).  Run by one wave, with uniform control flow.
// ---------------------------------------------------------------------------
constexpr uint32_t kNoNode = 0xFFFFFFFFu;  // weight of an empty queue (weights stay below 2^31)

// Element k (< 128, uniform) of a wave array held in two registers.
__device__ __forceinline__ uint32_t wave_at(uint32_t r0, uint32_t r1, uint32_t k) {
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)r0, (int)(k & 63u));
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)r1, (int)(k & 63u));
  return k < 64u ? a : b;
}

// m <= 127: the queues live in registers (leaf k and internal node m + k at
// lane k of two registers each), and places not filled (leaves past m,
// internal nodes not yet made) weigh kNoNode, so a step needs no tests of
// emptiness.  A step reads both fronts and both successors and takes its two
// picks by selects: a leaf first when it weighs at most the internal front,
// then the smaller of the next leaf and the internal front (leaf on a tie),
// or after an internal node the smaller of the leaf front and the next
// internal node.  It records only how many leaves it took (c_j): both queues
// are taken in order, so internal node m + j is the parent of leaves
// [L_j, L_j + c_j) and of internal nodes m + [2j - L_j, 2j - L_j + 2 - c_j),
// with L_j = c_0 + ... + c_{j-1}, which the whole wave writes afterwards.
// Every index read stays below 128 (leaves: at most m; internal nodes: at
// most m - 1).  (About 140 ns a step on one wave, C3's 95 symbols in 13 us;
// the former loop, branching per pick and storing each parent as it went,
// took about 190 ns a step.)
__device__ void tree_small(const uint32_t* wt, uint32_t* pr, uint32_t m) {
  const uint32_t lane = lane_id();
  const uint32_t l0 = lane < m ? wt[lane] : kNoNode, l1 = lane + 64u < m ? wt[lane + 64u] : kNoNode;
  uint32_t i0 = kNoNode, i1 = kNoNode;  // internal node weights
  uint32_t c0 = 0, c1 = 0;              // leaves taken by internal node m + j (lane j, j - 64)
  uint32_t lq = 0, iq = 0;              // fronts: leaf lq, internal node m + iq
  const uint32_t nint = m - 1;
  auto step = [&](uint32_t& ireg, uint32_t& creg, uint32_t at) {
    const uint32_t a0 = wave_at(l0, l1, lq), a1 = wave_at(l0, l1, lq + 1);
    const uint32_t b0 = wave_at(i0, i1, iq), b1 = wave_at(i0, i1, iq + 1);
    const uint32_t lf1 = a0 <= b0 ? 1u : 0u;  // first pick: the leaf front
    const uint32_t x = lf1 ? a1 : a0, y = lf1 ? b0 : b1;  // the second pick's candidates
    const uint32_t lf2 = x <= y ? 1u : 0u;    // second pick a leaf
    const uint32_t first = a0 <= b0 ? a0 : b0, second = x <= y ? x : y;
    const uint32_t c = lf1 + lf2;
    lq += c;
    iq += 2u - c;
    ireg = lane == at ? first + second : ireg;
    creg = lane == at ? c : creg;
  };
  uint32_t nj = 0;  // internal node m + nj is made by this step
  for (; nj < nint && nj < 64u; nj++) step(i0, c0, nj);
  for (; nj < nint; nj++) step(i1, c1, nj - 64u);
  // the parents: lane j (and j + 64) holds c_j; L_j is its exclusive prefix
  const uint32_t inc0 = wave_incl(c0), tot0 = (uint32_t)__builtin_amdgcn_readlane((int)inc0, 63);
  const uint32_t inc1 = wave_incl(c1) + tot0;
#pragma unroll
  for (uint32_t h = 0; h < 2; h++) {
    const uint32_t j = lane + 64u * h;
    if (j >= nint) continue;
    const uint32_t c = h ? c1 : c0, L = (h ? inc1 : inc0) - c, I = 2u * j - L;
    for (uint32_t q = 0; q < c; q++) pr[L + q] = m + j;
    for (uint32_t q = 0; q < 2u - c; q++) pr[m + I + q] = m + j;
  }
}

// First index in [lo, hi) whose weight is >= w (strict: > w).
template <bool kStrict>
__device__ __forceinline__ uint32_t wt_bound(const uint32_t* wt, uint32_t lo, uint32_t hi, uint32_t w) {
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    const uint32_t v = wt[mid];
    if (kStrict ? v <= w : v < w) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Any m, in rounds.  A round takes the first two picks, whose sum N is the
// round's first new node; every remaining older internal node (each at most
// N) and every leaf of weight at most N is picked before that node in the
// sequential order, so they are merged at once (a leaf before an internal
// node of equal weight) and paired in merged order; an odd one out waits for
// the next round, which then starts with it.  mrg holds at least 2m entries.
__device__ void tree_rounds(uint32_t* wt, uint32_t* pr, uint32_t* mrg, uint32_t m) {
  const uint32_t lane = lane_id();
  const uint32_t nn = 2 * m - 1;
  uint32_t p = 0, q = m, e = m;  // leaf front, internal front, next node
  while (e < nn) {
    uint32_t x[2], wx[2];
#pragma unroll
    for (int k = 0; k < 2; k++) {
      const uint32_t wl = p < m ? __builtin_amdgcn_readfirstlane(wt[p]) : kNoNode;
      const uint32_t wi = q < e ? __builtin_amdgcn_readfirstlane(wt[q]) : kNoNode;
      if (p < m && wl <= wi) {
        x[k] = p++;
        wx[k] = wl;
      } else {
        x[k] = q++;
        wx[k] = wi;
      }
    }
    const uint32_t n0 = wx[0] + wx[1];
    const uint32_t eo = e;  // the older internal nodes are [q, eo)
    if (lane == 0) {
      wt[eo] = n0;
      pr[x[0]] = eo;
      pr[x[1]] = eo;
    }
    e++;
    // leaves [p, p + na) weigh at most n0: blocks of s1 leaves, then one block
    const uint32_t span = m - p;
    uint32_t na = 0;
    if (span) {
      const uint32_t s1 = (span + 63u) >> 6;  // <= 64: m < 4096
      const uint32_t b0 = lane * s1;
      const bool full = b0 < span && wt[p + min(span, b0 + s1) - 1u] <= n0;
      const uint32_t c1 = (uint32_t)__builtin_popcountll(__ballot(full));
      const uint32_t base = c1 * s1;
      if (base >= span) {
        na = span;
      } else {
        const bool in = lane < s1 && base + lane < span && wt[p + base + lane] <= n0;
        na = base + (uint32_t)__builtin_popcountll(__ballot(in));
      }
    }
    const uint32_t nb = eo - q, tot = na + nb;
    for (uint32_t t = lane; t < tot; t += 64u) {
      if (t < na) {
        const uint32_t w = wt[p + t];
        mrg[t + wt_bound<false>(wt, q, eo, w) - q] = p + t;
      } else {
        const uint32_t j = t - na, w = wt[q + j];
        mrg[j + wt_bound<true>(wt, p, p + na, w) - p] = q + j;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint32_t np = tot >> 1;
    uint32_t nleaf = 0;
    for (uint32_t t = lane; t < np; t += 64u) {
      const uint32_t u = mrg[2 * t], v = mrg[2 * t + 1];
      wt[e + t] = wt[u] + wt[v];
      pr[u] = e + t;
      pr[v] = e + t;
      nleaf += (u < m) + (v < m);
    }
    nleaf = wave_sum(nleaf);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    p += nleaf;
    q += 2 * np - nleaf;
    e += np;
  }
}

// T.81 Annex K.3 on the counts per length (lane l of cl holds BITS[l], one
// wave, uniform control flow), a whole level at a time.  The single steps
// take two codes of the longest length i, one to length i-1 and the other,
// with a code of the longest length j < i-1 that exists, to j+1.  At level i
// the P = BITS[i]/2 steps use the codes below i-1 deepest first, and a code
// of length k < i-1 takes 2^(i-1-k) - 1 steps before its descendants are all
// at length i-1 (it becomes two codes of length k+1, each of which does the
// same): full codes are taken in bulk, a code taken in part leaves one or two
// codes on each level it passed.  Every code of length i-2 so taken adds two
// codes of length i-1, and every step one more.
__device__ uint32_t k3_levels(uint32_t cl) {
  const uint32_t lane = lane_id();
  auto at = [&](uint32_t l) { return (uint32_t)__builtin_amdgcn_readlane((int)cl, (int)l); };
  auto add = [&](uint32_t l, uint32_t d) { cl += lane == l ? d : 0u; };
  // codes of length k < i-1 that R steps use up in full (R < 2^11: P is at
  // most half the alphabet), and the steps each takes
  auto full = [&](uint32_t R, uint32_t sh, uint32_t have, uint32_t& f) {
    f = sh > 11 ? 0xFFFFFFFFu : (1u << sh) - 1u;
    return sh > 11 ? 0u : min(have, R / f);
  };
  for (;;) {
    const uint64_t nz = __ballot(cl != 0);
    if (nz == 0) break;
    const uint32_t i = 63u - (uint32_t)__builtin_clzll(nz);
    if (i <= (uint32_t)kMaxLen) break;
    const uint32_t P = at(i) >> 1;
    if (P == 0) break;  // an odd count at the deepest level: not a complete code
    uint32_t R = P, E = 0;
    for (uint32_t k = i - 2; R > 0 && k > 0; k--) {
      const uint32_t bk = at(k);
      if (bk == 0) continue;
      const uint32_t sh = i - 1 - k;  // a code of length k takes 2^sh - 1 steps
      uint32_t f;
      const uint32_t u = full(R, sh, bk, f);
      add(k, 0u - u);
      R -= u * f;
      if (u) E += u << (sh - 1);  // u > 0 only when sh <= 11
      if (R == 0) break;
      if (bk > u) {  // one more code of length k, taken in part
        add(k, 0u - 1u);
        R--;  // it becomes two codes of length k + 1
        uint32_t l = k + 1, cnt = 2;
        for (;;) {
          if (R == 0) {
            add(l, cnt);
            break;
          }
          const uint32_t shl = i - 1 - l;
          uint32_t fl;
          const uint32_t ul = full(R, shl, cnt, fl);
          R -= ul * fl;
          if (ul) E += ul << (shl - 1);
          cnt -= ul;
          if (R == 0) {
            add(l, cnt);
            break;
          }
          add(l, cnt - 1);  // the other stays; this one goes on a level
          R--;
          l++;
          cnt = 2;
          if (l + 1 >= i) break;  // cannot happen for a complete code
        }
        break;
      }
    }
    add(i, 0u - 2u * P);
    add(i - 1, P + 2u * E);
  }
  return cl;
}

// Canonical codes (RFC 1951 section 3.2.2): the code of symbol s with length
// l is first[l] plus the number of symbols below s that have length l.  Each
// thread owns kTable / blockDim.x consecutive symbols; the per-length counts
// travel as twelve 16-bit fields packed in three u64 (no field exceeds 4095,
// so no carry crosses a field).  enc[s] = len << 16 | code, 0 if unused.
__device__ void canonical_codes(const uint8_t* len, const uint32_t* first, uint32_t* enc,
                                uint64_t (*part)[3]) {
  const uint32_t per = kTable / blockDim.x;
  const uint32_t s0 = threadIdx.x * per;
  uint64_t c[3] = {0, 0, 0};
  for (uint32_t k = 0; k < per; k++) {
    const uint32_t l = len[s0 + k];
    if (l) c[(l - 1) >> 2] += 1ull << (16 * ((l - 1) & 3));
  }
  const uint32_t wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint64_t inc[3];
  for (int k = 0; k < 3; k++) inc[k] = wave_incl64(c[k]);
  if (lane_id() == 63)
    for (int k = 0; k < 3; k++) part[wv][k] = inc[k];
  __syncthreads();
  uint64_t e[3];
  for (int k = 0; k < 3; k++) {
    uint64_t before = 0;
    for (uint32_t i = 0; i < wv; i++) before += part[i][k];
    e[k] = before + inc[k] - c[k];
  }
  (void)nw;
  for (uint32_t k = 0; k < per; k++) {
    const uint32_t s = s0 + k, l = len[s];
    uint32_t v = 0;
    if (l) {
      const int f = (l - 1) >> 2, sh = 16 * ((l - 1) & 3);
      const uint32_t rank = (uint32_t)(e[f] >> sh) & 0xFFFFu;
      e[f] += 1ull << sh;
      v = (l << 16) | (first[l] + rank);
    }
    enc[s] = v;
  }
}

// Zero the status word, and the histograms of nhist segments.
__global__ void __launch_bounds__(kThreads) huff_clear(Ws w, uint32_t nhist) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < nhist * (uint32_t)kTable) w.hist[i] = 0;
  if (i == 0) w.status[0] = 0;
}

// Histogram of segment blockIdx.y (n symbols from sym + blockIdx.y * n).
__global__ void __launch_bounds__(kThreads) huff_hist(const uint16_t* __restrict__ sym0, uint64_t n,
                                                      Ws w) {
  const uint16_t* sym = sym0 + (uint64_t)blockIdx.y * n;
  uint32_t* hist = w.hist + (size_t)blockIdx.y * kTable;
  __shared__ uint32_t h[kTable];
  for (int i = threadIdx.x; i < kTable; i += kThreads) h[i] = 0;
  __syncthreads();
  auto add = [&](uint32_t s) { atomicAdd(&h[s < (uint32_t)kNsym ? s : (uint32_t)kNsym], 1u); };
  // 16-byte loads when every segment starts 16-byte aligned
  const uint64_t nv = (n & 7) == 0 ? n >> 3 : 0, stride = (uint64_t)gridDim.x * kThreads;
  const uint4* v = reinterpret_cast<const uint4*>(sym);
  // four 16-byte loads in flight per lane before their 32 LDS updates
  for (uint64_t i0 = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i0 < nv; i0 += 4 * stride) {
    uint4 q[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const uint64_t i = i0 + u * stride;
      q[u] = i < nv ? v[i] : make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
      if (i0 + u * stride >= nv) break;
      const uint32_t x[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
      for (int k = 0; k < 4; k++) {
        add(x[k] & 0xFFFFu);
        add(x[k] >> 16);
      }
    }
  }
  for (uint64_t i = (nv << 3) + (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    add(sym[i]);
  __syncthreads();
  for (int i = threadIdx.x; i < kTable; i += kThreads)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}

// Codebook of segment blockIdx.x (n symbols per segment).
__global__ void __launch_bounds__(kBookThreads) huff_book(Ws w, uint8_t* __restrict__ books,
                                                          uint32_t* __restrict__ chunk_off,
                                                          uint64_t n, const uint32_t* skip) {
  const uint32_t seg = blockIdx.x;
  if (skip && skip[seg]) return;  // the segment keeps its code (whole workgroup)
  const uint32_t* hist = w.hist + (size_t)seg * kTable;
  uint32_t* enc = w.enc + (size_t)seg * kTable;
  uint8_t* book = books + (size_t)seg * kBookStride;
  __shared__ uint64_t key[kTable];
  __shared__ uint32_t wt[2 * kTable];
  __shared__ uint32_t pr[2 * kTable];  // parent while building; then ancestor | distance << 16
  __shared__ uint16_t syms[kTable];
  __shared__ uint8_t len[kTable];
  __shared__ uint32_t bits[kMaxDepth];
  __shared__ uint32_t first[kMaxLen + 1], cum[kMaxLen + 1];
  __shared__ uint64_t part[16][3];
  __shared__ int s_m, s_lo, s_hi;
  const int t = threadIdx.x;

  if (t == 0) {
    s_m = 0;
    s_lo = kTable;
    s_hi = -1;
  }
  if (t < kMaxDepth) bits[t] = 0;
  __syncthreads();
  // keys: frequency, then the complement of the symbol (so that reading the
  // sorted keys backwards gives decreasing frequency, then increasing symbol)
  int cm = 0, lo = kTable, hi = -1;
  uint32_t hv[kTable / kBookThreads];  // every load in flight before the first is used
#pragma unroll
  for (int q = 0; q < kTable / kBookThreads; q++) hv[q] = hist[t + q * kBookThreads];
#pragma unroll
  for (int q = 0; q < kTable / kBookThreads; q++) {
    const int s = t + q * kBookThreads;
    const uint32_t f = hv[q];
    uint64_t k = ~0ull;
    if (s < kNsym && f) {
      k = ((uint64_t)f << 12) | (uint64_t)(4095 - s);
      cm++;
      lo = min(lo, s);
      hi = max(hi, s);
    }
    if (s == kNsym && f) status_or(w.status, kStBadSymbol);
    key[s] = k;
    len[s] = 0;
  }
  // per wave first (the compiler would serialize lane by lane), then one
  // update per wave
  for (int o = 32; o > 0; o >>= 1) {
    cm += __shfl_xor(cm, o, 64);
    lo = min(lo, __shfl_xor(lo, o, 64));
    hi = max(hi, __shfl_xor(hi, o, 64));
  }
  if ((t & 63) == 0 && cm) {
    atomicAdd(&s_m, cm);
    atomicMin(&s_lo, lo);
    atomicMax(&s_hi, hi);
  }
  __syncthreads();
  const int m = s_m;

  if (m >= 2 && m <= kBookThreads) {
    // small alphabet: gather the used keys, then each takes the rank that
    // the number of smaller keys gives it (keys are distinct)
    __shared__ uint64_t ck[kBookThreads];
    __shared__ int s_n;
    if (t == 0) s_n = 0;
    __syncthreads();
    for (int s = t; s < kTable; s += kBookThreads) {
      const uint64_t k = key[s];
      if (k != ~0ull) ck[atomicAdd(&s_n, 1)] = k;
    }
    __syncthreads();
    if (t < m) {
      const uint64_t k = ck[t];
      int r = 0;
      for (int i = 0; i < m; i++) r += ck[i] < k;
      key[r] = k;
    }
    __syncthreads();
  } else if (m > kBookThreads) {
    for (int size = 2; size <= kTable; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int p = t; p < kTable / 2; p += kBookThreads) {
          const int i = (p / stride) * 2 * stride + (p % stride), j = i + stride;
          const bool asc = (i & size) == 0;
          const uint64_t a = key[i], b = key[j];
          if ((a > b) == asc) {
            key[i] = b;
            key[j] = a;
          }
        }
        __syncthreads();
      }
    }
  }
  if (m >= 2) {
    for (int i = t; i < m; i += kBookThreads) {
      const uint64_t k = key[i];
      wt[i] = (uint32_t)(k >> 12);
      syms[i] = (uint16_t)(4095 - (uint32_t)(k & 0xFFFu));
    }
    __syncthreads();
    // two queues: sorted leaves [0, m) and internal nodes [m, 2m-1) in
    // creation order; of two equal weights the leaf is taken first (one wave;
    // the merge buffer of the rounds reuses the sort keys' space)
    if (t < 64) {
      if (m <= 127) tree_small(wt, pr, (uint32_t)m);
      else tree_rounds(wt, pr, reinterpret_cast<uint32_t*>(key), (uint32_t)m);
    }
    __syncthreads();
    const int nn = 2 * m - 1, root = nn - 1;
    for (int v = t; v < nn; v += kBookThreads) pr[v] = v == root ? (uint32_t)root : (pr[v] | 1u << 16);
    __syncthreads();
    // pointer jumping: every pair (ancestor, distance) stays true, and each
    // round at least doubles the distance until the root is reached
    for (int r = 0; r < 13; r++) {
      int open = 0;
      for (int v = t; v < nn; v += kBookThreads) {
        const uint32_t x = pr[v], y = pr[x & 0xFFFFu];
        const uint32_t z = (y & 0xFFFFu) | (((x >> 16) + (y >> 16)) << 16);
        pr[v] = z;
        open |= (z & 0xFFFFu) != (uint32_t)root;
      }
      if (!__syncthreads_or(open)) break;
    }
    for (int v = t; v < m; v += kBookThreads) {
      const uint32_t d = pr[v] >> 16;
      if (d < (uint32_t)kMaxDepth) atomicAdd(&bits[d], 1u);
      else status_or(w.status, kStDepth);
    }
  } else if (m == 1 && t == 0) {
    bits[1] = 1;
    syms[0] = (uint16_t)s_lo;
  }
  __syncthreads();
  if (t < 64) {
    // wave 0, one length count per lane (lane i holds BITS[i]).
    // ITU-T T.81 Annex K.3: while a code is longer than the limit, take two
    // codes of the longest length i: one moves to length i-1 (next to its
    // prefix), and the other becomes a sibling of a code of the longest
    // length j < i-1 that exists, which moves to j+1 with it
    const uint32_t cl = k3_levels(bits[t]);
    // cum[l]: codes of length <= l; first[l] = 2 (first[l-1] + BITS[l-1]),
    // i.e. the sum over k < l of BITS[k] << (l - k)
    const uint32_t inc = wave_incl(t >= 1 && t <= kMaxLen ? cl : 0u);
    uint32_t f = 0;
#pragma unroll
    for (int k = 1; k < kMaxLen; k++) {
      const uint32_t bk = (uint32_t)__builtin_amdgcn_readlane((int)cl, k);
      if (k < t) f += bk << (t - k);
    }
    if (t <= kMaxLen) {
      cum[t] = inc;
      first[t] = f;
    }
  }
  __syncthreads();
  // rank r (decreasing frequency, then increasing symbol) is the sorted key
  // m-1-r; ranks take the lengths shortest first
  for (int r = t; r < m; r += kBookThreads) {
    int l = 1;
    while (l < kMaxLen && cum[l] <= (uint32_t)r) l++;
    len[syms[m - 1 - r]] = (uint8_t)l;
  }
  __syncthreads();
  canonical_codes(len, first, enc, part);

  // codebook bytes
  if (m == 0) {
    if (t < 4) book[t] = (uint8_t)(t == 0 ? 1 : 0);
  } else {
    const int blo = s_lo, bhi = s_hi, nb = bhi - blo + 1;
    if (t == 0) {
      book[0] = (uint8_t)blo;
      book[1] = (uint8_t)(blo >> 8);
      book[2] = (uint8_t)bhi;
      book[3] = (uint8_t)(bhi >> 8);
    }
    for (int b = t; b < (nb + 1) / 2; b += kBookThreads) {
      const int s = blo + 2 * b;
      const uint32_t lo4 = len[s], hi4 = s + 1 <= bhi ? len[s + 1] : 0u;
      book[4 + b] = (uint8_t)(lo4 | hi4 << 4);
    }
  }
  if (n == 0 && seg == 0 && t == 0) chunk_off[0] = 0;
}

// Words of every chunk of group blockIdx.x of segment blockIdx.y (n symbols
// and nch chunks per segment; chunk c of segment s is chunk s*nch + c of the
// chunk table).
__global__ void __launch_bounds__(kThreads) huff_size(const uint16_t* __restrict__ sym0, uint64_t n,
                                                      Ws w, uint32_t* __restrict__ chunk_off,
                                                      uint32_t nch, uint32_t per_group) {
  __shared__ uint8_t lens[kTable];
  __shared__ uint32_t wsum[kThreads / 64];
  const uint32_t seg = blockIdx.y;
  const uint16_t* sym = sym0 + (uint64_t)seg * n;
  chunk_off += (size_t)seg * nch;
  const bool vec = (n & 3) == 0;  // 8-byte loads when segments start 8-byte aligned
  for (int i = threadIdx.x; i < kTable; i += kThreads)
    lens[i] = (uint8_t)(w.enc[(size_t)seg * kTable + i] >> 16);
  __syncthreads();
  const uint32_t wv = threadIdx.x >> 6, ln = lane_id();
  const uint32_t c0 = blockIdx.x * per_group, c1 = min(c0 + per_group, nch);
  uint32_t gsum = 0;
  for (uint32_t c = c0 + wv; c < c1; c += kThreads / 64) {
    const uint64_t base = (uint64_t)c * kChunk;
    const uint64_t cnt = min((uint64_t)kChunk, n - base);
    uint32_t b = 0;
    if (vec && cnt == (uint64_t)kChunk) {
      const uint2 q = reinterpret_cast<const uint2*>(sym + base)[ln];
      b = lens[min(q.x & 0xFFFFu, 4095u)] + lens[min(q.x >> 16, 4095u)] +
          lens[min(q.y & 0xFFFFu, 4095u)] + lens[min(q.y >> 16, 4095u)];
    } else {
      for (uint32_t k = 0; k < 4; k++) {
        const uint32_t i = ln * 4 + k;
        if (i < cnt) b += lens[min((uint32_t)sym[base + i], 4095u)];
      }
    }
    const uint32_t words = (wave_sum(b) + 31) >> 5;
    if (ln == 0) chunk_off[c + 1] = words;
    gsum += words;
  }
  if (ln == 0) wsum[wv] = gsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int i = 0; i < kThreads / 64; i++) s += wsum[i];
    w.groups[seg * gridDim.x + blockIdx.x] = s;
  }
}

// Chunk offsets and words of group blockIdx.x of segment blockIdx.y; groups
// are ordered segment by segment, so the words of all segments follow each
// other in one array.
__global__ void __launch_bounds__(kThreads) huff_write(const uint16_t* __restrict__ sym0, uint64_t n,
                                                       Ws w, uint32_t* __restrict__ chunk_off0,
                                                       uint32_t nch, uint32_t per_group,
                                                       uint32_t* __restrict__ words) {
  __shared__ __align__(16) uint32_t enc[kTable];
  __shared__ uint32_t offs[kThreads], cnts[kThreads];
  __shared__ uint32_t buf[kThreads / 64][kChunkWords];
  __shared__ uint32_t part[16];
  const uint32_t t = threadIdx.x, wv = t >> 6, ln = lane_id();
  const uint32_t seg = blockIdx.y, gi = seg * gridDim.x + blockIdx.x;
  const uint16_t* sym = sym0 + (uint64_t)seg * n;
  uint32_t* chunk_off = chunk_off0 + (size_t)seg * nch;
  const bool vec = (n & 3) == 0;
  {  // the segment's code table, every load of a thread in flight before its stores
    constexpr int kQ = kTable / 4 / kThreads;
    const uint4* src = reinterpret_cast<const uint4*>(w.enc + (size_t)seg * kTable);
    uint4 v[kQ];
#pragma unroll
    for (int q = 0; q < kQ; q++) v[q] = src[kThreads * q + t];
#pragma unroll
    for (int q = 0; q < kQ; q++) reinterpret_cast<uint4*>(enc)[kThreads * q + t] = v[q];
  }
  for (int i = t; i < kChunkWords * (kThreads / 64); i += kThreads) (&buf[0][0])[i] = 0;
  // words of all groups before this one
  uint32_t before = 0;
  for (uint32_t g = t; g < gi; g += kThreads) before += w.groups[g];
  uint32_t base;
  block_excl(before, part, &base);
  const uint32_t c0 = blockIdx.x * per_group, c1 = min(c0 + per_group, nch);
  if (gi == 0 && t == 0) chunk_off0[0] = 0;
  for (uint32_t r0 = c0; r0 < c1; r0 += kThreads) {
    const uint32_t c = r0 + t;
    const uint32_t cw = c < c1 ? chunk_off[c + 1] : 0u;
    uint32_t total;
    const uint32_t ex = block_excl(cw, part, &total);
    if (c < c1) chunk_off[c + 1] = base + ex + cw;
    offs[t] = base + ex;
    cnts[t] = cw;
    base += total;
    __syncthreads();
    // the wave's chunks of the round kBatch at a time, the loads of full
    // chunks all in flight
    constexpr uint32_t kBatch = 8, kW = kThreads / 64;
    for (uint32_t jb = 0; jb < (uint32_t)kThreads && r0 + jb < c1; jb += kBatch * kW) {
    uint2 qb[kBatch];
#pragma unroll
    for (uint32_t u = 0; u < kBatch; u++) {
      const uint32_t cc = r0 + jb + kW * u + wv;
      const bool full = vec && cc < c1 && (uint64_t)(cc + 1) * kChunk <= n;
      qb[u] = full ? reinterpret_cast<const uint2*>(sym + (uint64_t)cc * kChunk)[ln] : make_uint2(0, 0);
    }
#pragma unroll
    for (uint32_t u = 0; u < kBatch; u++) {
      const uint32_t j = jb + kW * u + wv, cc = r0 + j;
      const bool active = cc < c1;
      uint32_t nbits_wave = 0;
      if (active) {
        const uint64_t sbase = (uint64_t)cc * kChunk;
        const uint64_t cnt = min((uint64_t)kChunk, n - sbase);
        uint32_t s[4];
        if (vec && cnt == (uint64_t)kChunk) {
          const uint2 q = qb[u];
          s[0] = q.x & 0xFFFFu;
          s[1] = q.x >> 16;
          s[2] = q.y & 0xFFFFu;
          s[3] = q.y >> 16;
        } else {
          for (uint32_t k = 0; k < 4; k++) {
            const uint32_t i = ln * 4 + k;
            s[k] = i < cnt ? (uint32_t)sym[sbase + i] : 4095u;  // enc[4095] = 0: no bits
          }
        }
        uint64_t v = 0;
        uint32_t nb = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const uint32_t e = enc[min(s[k], 4095u)], l = e >> 16;
          v = (v << l) | (e & 0xFFFFu);
          nb += l;
        }
        const uint32_t inc = wave_incl(nb);
        nbits_wave = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        const uint32_t pos = inc - nb;
        if (nb) {
          const uint64_t top = v << (64 - nb);  // first code bit at bit 63
          const uint32_t w0 = pos >> 5, off = pos & 31u;
          const uint32_t a = (uint32_t)(top >> (32 + off));
          const uint32_t b = (uint32_t)(top >> off);
          const uint32_t c2 = off ? (uint32_t)(top << (32 - off)) : 0u;
          if (a && w0 < (uint32_t)kChunkWords) atomicOr(&buf[wv][w0], a);
          if (b && w0 + 1 < (uint32_t)kChunkWords) atomicOr(&buf[wv][w0 + 1], b);
          if (c2 && w0 + 2 < (uint32_t)kChunkWords) atomicOr(&buf[wv][w0 + 2], c2);
        }
      }
      // each wave owns its buffer, and a wave's LDS operations complete in
      // order: a wave-level fence orders the ORs before the reads and the
      // reads and clears before the next chunk's ORs
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (active) {
        // never more words than the size pass gave the chunk
        const uint32_t nw = min((nbits_wave + 31) >> 5, cnts[j]), o = offs[j];
        for (uint32_t i = ln; i < nw; i += 64) {
          words[o + i] = buf[wv][i];
          buf[wv][i] = 0;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    }
    __syncthreads();  // offs[] is rewritten by the next round
  }
}

// Validate the codebook of segment blockIdx.x (book_bytes readable bytes at
// books + blockIdx.x * EC_HUFF_BOOK_MAX) and build its prefix table.
// report: set the status word for a bad codebook (with no chunks to decode);
// else workgroup 0 zeroes the status word, and the decode kernel, which runs
// after this one, reports the segments whose codebook is not valid.
// Decode table of segment blockIdx.x, 1024 threads: thread t reads the
// lengths of symbols lo + 4t .. lo + 4t + 3 (two codebook bytes, loaded
// together with the range header), counts them per length in 16-bit fields
// (two lengths per word), and a prefix of those counts over the workgroup
// gives every symbol its rank among the codes of its length, i.e. its
// canonical code (RFC 1951 section 3.2.2).  Each wave forms the prefix over
// the waves' totals itself, so the totals and the per-length code ranges
// are wave-uniform.  Symbols go to LDS in code order; then thread t fills
// table entries 4t .. 4t + 3.  The codebook is validated as before: lengths
// up to 12, the first and last symbol of its range used, the padding nibble
// zero, a complete code.
constexpr int kDecBookThreads = 1024;
__global__ void __launch_bounds__(kDecBookThreads) huff_dec_book(const uint8_t* __restrict__ books,
                                                              uint64_t book_bytes,
                                                              const uint32_t* __restrict__ chunk_off,
                                                              uint64_t n, Ws w, int report) {
  constexpr int kPer = kTable / kDecBookThreads;  // 4 symbols and 4 table entries per thread
  constexpr int kWaves = kDecBookThreads / 64;
  static_assert(kPer == 4 && kWaves <= 64, "one 8-byte table store per thread");
  const uint32_t seg = blockIdx.x;
  const uint8_t* book = books + (size_t)seg * kBookStride;
  uint16_t* lut = w.lut + (size_t)seg * kTable;
  __shared__ uint16_t order[kTable];
  __shared__ uint32_t part[kWaves][8];  // per wave: six count words, Kraft sum, flags
  const uint32_t t = threadIdx.x, lane = t & 63u;
  const uint32_t wv = (uint32_t)__builtin_amdgcn_readfirstlane((int)(t >> 6));
  if (t == 0 && !report && seg == 0) w.status[0] = 0;
  // this thread's two length bytes, issued with the header loads; bytes past
  // the codebook's range are dropped once the header is known
  uint8_t raw[kPer / 2];
#pragma unroll
  for (int j = 0; j < kPer / 2; j++) {
    const uint64_t b = 4u + (uint64_t)kPer / 2 * t + j;
    raw[j] = b < book_bytes ? book[b] : (uint8_t)0;
  }
  bool bad = false;
  uint32_t lo = 1, hi = 0;
  if (book_bytes < 4) {
    bad = true;
  } else {
    lo = book[0] | (uint32_t)book[1] << 8;
    hi = book[2] | (uint32_t)book[3] << 8;
    if (hi < lo) bad = !(lo == 1 && hi == 0);
    else bad = hi >= (uint32_t)kNsym || 4 + (uint64_t)(hi - lo + 2) / 2 > book_bytes;
  }
  const bool empty = !bad && hi < lo;
  if (empty && n > 0) bad = true;
  if (seg == 0 && chunk_off[0] != 0) bad = true;
  const uint32_t nb = bad || empty ? 0u : hi - lo + 1, nbytes = (nb + 1) / 2;
  uint32_t lj[kPer];  // lengths of this thread's symbols, 0 past the range
  uint32_t cw[6] = {0, 0, 0, 0, 0, 0};  // count of length l in field (l-1) & 1 of word (l-1) >> 1
  uint32_t kr = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const uint32_t k = (uint32_t)kPer * t + j;
    const uint32_t by = (uint32_t)kPer / 2 * t + (j >> 1) < nbytes ? raw[j >> 1] : 0u;
    const uint32_t l = (by >> (4 * (j & 1))) & 15u;
    lj[j] = 0;
    if (k < nb && l) {
      if (l > (uint32_t)kMaxLen) {
        bad = true;
      } else {
        lj[j] = l;
        cw[(l - 1) >> 1] += 1u << (16 * ((l - 1) & 1));
        kr += 1u << (kMaxLen - l);
      }
    }
    if (k >= nb && l) bad = true;  // the padding nibble
    if (nb && (k == 0 || k == nb - 1) && !l) bad = true;  // lo and hi are used
  }
  // prefix of the counts within the wave, then over the waves' totals
  uint32_t inc[6];
#pragma unroll
  for (int q = 0; q < 6; q++) inc[q] = wave_incl(cw[q]);
  const uint32_t krw = wave_sum(kr);
  const uint64_t badw = __ballot(bad);
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 6; q++) part[wv][q] = inc[q];
    part[wv][6] = krw;
    part[wv][7] = badw != 0;
  }
  __syncthreads();
  uint32_t before[6], tot[6];  // wave-uniform: codes of each length in earlier waves, in all
  uint32_t kraft, anybad;
  {
    uint32_t x[8];
#pragma unroll
    for (int q = 0; q < 8; q++) x[q] = lane < (uint32_t)kWaves ? part[lane][q] : 0u;
#pragma unroll
    for (int q = 0; q < 6; q++) {
      const uint32_t c = wave_incl(x[q]);
      tot[q] = (uint32_t)__builtin_amdgcn_readlane((int)c, 63);
      before[q] = wv ? (uint32_t)__builtin_amdgcn_readlane((int)c, (int)wv - 1) : 0u;
    }
    kraft = wave_sum(x[6]);
    anybad = __ballot(x[7] != 0) != 0;
  }
  auto field = [](const uint32_t (&a)[6], uint32_t l) {  // the count of length l
    return (a[(l - 1) >> 1] >> (16 * ((l - 1) & 1))) & 0xFFFFu;
  };
  uint32_t m = 0;
  for (uint32_t l = 1; l <= (uint32_t)kMaxLen; l++) m += field(tot, l);
  if (!anybad && !empty) {
    const bool complete = m == 1 ? field(tot, 1) == 1 : kraft == (1u << kMaxLen);
    if (!complete) anybad = 1;
  }
  if (anybad) {
    if (t == 0) {
      if (report) status_or(w.status, kStCorrupt);
      w.valid[seg] = 0;
    }
    return;
  }
  if (t == 0) w.valid[seg] = 1;
  // per length l (every index below is a constant): the table range
  // [lo_l, hi_l) its codes cover, the code-order index of its first code
  // less the code itself, and where this thread's first code of length l goes
  uint32_t tlo[kMaxLen + 1], thi[kMaxLen + 1], tadj[kMaxLen + 1], tpos[kMaxLen + 1];
  {
    uint32_t code = 0, idx = 0;
#pragma unroll
    for (int l = 1; l <= kMaxLen; l++) {
      const uint32_t c = field(tot, (uint32_t)l);
      if (l > 1) code = (code + field(tot, (uint32_t)l - 1)) << 1;
      tadj[l] = idx - code;
      tlo[l] = code << (kMaxLen - l);
      thi[l] = (code + c) << (kMaxLen - l);
      const uint32_t q = (uint32_t)(l - 1) >> 1, sh = 16 * ((uint32_t)(l - 1) & 1);
      // codes of length l before this thread's: earlier waves and lanes
      tpos[l] = idx + ((before[q] >> sh) & 0xFFFFu) + (((inc[q] - cw[q]) >> sh) & 0xFFFFu);
      idx += c;
    }
  }
  // this thread's symbols in code order: a symbol's rank among the codes of
  // its length is the count before this thread plus the thread's own
  // earlier symbols of that length
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const uint32_t l = lj[j];
    uint32_t pos = 0;
#pragma unroll
    for (int q = 1; q <= kMaxLen; q++) pos = l == (uint32_t)q ? tpos[q] : pos;
#pragma unroll
    for (int jj = 0; jj < j; jj++) pos += lj[jj] == l ? 1u : 0u;
    if (l) order[pos] = (uint16_t)(lo + (uint32_t)kPer * t + j);
  }
  __syncthreads();
  // table entries 4t .. 4t + 3: entry i holds the code whose range of 12-bit
  // prefixes covers it (ranges of a complete code tile the table in order of
  // length).  A code of length 10 or less covers whole aligned blocks of
  // four, so the block's first entry fixes the rest unless it lies in the
  // ranges of lengths 11 and 12, which the other three entries look up.
  const uint32_t i0 = (uint32_t)kPer * t;
  uint32_t L0 = 0, at0 = 0;
#pragma unroll
  for (int l = 1; l <= kMaxLen; l++) {
    const bool in = i0 >= tlo[l] && i0 < thi[l];
    L0 = in ? (uint32_t)l : L0;
    at0 = in ? tadj[l] + (i0 >> (kMaxLen - l)) : at0;
  }
  uint32_t ev[kPer];
  ev[0] = L0 ? (uint32_t)order[at0] | L0 << 12 : 0u;
#pragma unroll
  for (int j = 1; j < kPer; j++) {
    const uint32_t i = i0 + j;
    uint32_t L = L0, at = at0;
#pragma unroll
    for (int l = kMaxLen - 1; l <= kMaxLen; l++) {
      const bool in = i >= tlo[l] && i < thi[l];
      L = in ? (uint32_t)l : L;
      at = in ? tadj[l] + (i >> (kMaxLen - l)) : at;
    }
    ev[j] = L ? (uint32_t)order[at] | L << 12 : 0u;
  }
  *reinterpret_cast<uint2*>(lut + i0) = make_uint2(ev[0] | ev[1] << 16, ev[2] | ev[3] << 16);
}

// Chunks [128 blockIdx.x, 128 blockIdx.x + 128) of segment blockIdx.y, one
// lane per chunk: the decode table and the group's words go to LDS (the
// words one wave at a time when they do not all fit), then every lane
// decodes its chunk from LDS.
__global__ void __launch_bounds__(kDecChunks) huff_decode(const uint32_t* __restrict__ words,
                                                          uint64_t words_cap,
                                                          const uint32_t* __restrict__ chunk_off0,
                                                          uint64_t n, uint32_t nch, Ws w,
                                                          uint16_t* __restrict__ sym0) {
  __shared__ __align__(16) uint16_t lut[kTable];
  __shared__ __align__(16) uint32_t stage[kStageWords];
  const uint32_t t = threadIdx.x, seg = blockIdx.y, wv = t >> 6, ln = t & 63u;
  const uint32_t c0 = blockIdx.x * kDecChunks, c = c0 + t;
  const uint32_t cend = min(c0 + kDecChunks, nch);
  const uint32_t* chunk_off = chunk_off0 + (size_t)seg * nch;
  uint16_t* sym = sym0 + (uint64_t)seg * n;
  const bool vec = (n & 7) == 0;  // 16-byte stores when segments start 16-byte aligned
  // the group's words [glo, ghi) from its bounding offsets; they go through
  // LDS from the 16-byte boundary at or below glo when they fit (the usual
  // case), loaded together with the table and the chunks' own offsets.  The
  // range is checked here only to keep the loads inside the buffer; every
  // chunk is validated below before anything is decoded.
  const uint32_t glo = chunk_off[c0], ghi = chunk_off[cend];
  const uint32_t q0 = glo >> 2, q1 = ghi >> 2;  // whole 16-byte quads [q0, q1), then a tail
  const bool staged = glo <= ghi && (uint64_t)ghi <= words_cap && ghi - 4 * q0 <= (uint32_t)kStageWords;
  {
    const uint4* src = reinterpret_cast<const uint4*>(w.lut + (size_t)seg * kTable);
    uint4* dst = reinterpret_cast<uint4*>(lut);
    uint4 v[kTable * 2 / 16 / kDecChunks];
#pragma unroll
    for (int j = 0; j < kTable * 2 / 16 / kDecChunks; j++) v[j] = src[j * kDecChunks + t];
#pragma unroll
    for (int j = 0; j < kTable * 2 / 16 / kDecChunks; j++) dst[j * kDecChunks + t] = v[j];
  }
  if (staged) {
    if (((uintptr_t)words & 15u) == 0) {
      constexpr int kQ = kStageWords / 4 / kDecChunks;  // quads per thread, all in flight
      const uint4* wq = reinterpret_cast<const uint4*>(words);
      uint4* sq = reinterpret_cast<uint4*>(stage);
      uint4 v[kQ];
#pragma unroll
      for (int j = 0; j < kQ; j++) {
        const uint32_t i = q0 + j * kDecChunks + t;
        v[j] = i < q1 ? wq[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kQ; j++) {
        const uint32_t i = q0 + j * kDecChunks + t;
        if (i < q1) sq[i - q0] = v[j];
      }
      const uint32_t i = 4 * q1 + t;
      if (t < 3 && i < ghi) stage[i - 4 * q0] = words[i];
    } else {
      for (uint32_t i = 4 * q0 + t; i < ghi; i += kDecChunks) stage[i - 4 * q0] = words[i];
    }
  }
  bool ok = w.valid[seg] != 0;
  uint32_t a = 0, b = 0;
  if (c < cend) {
    a = chunk_off[c];
    b = chunk_off[c + 1];
    ok = ok && a <= b && b - a <= (uint32_t)kChunkWords && (uint64_t)b <= words_cap;
    if (seg == 0 && c == 0) ok = ok && a == 0;
  }
  if (!__syncthreads_and(ok)) {
    if (t == 0) status_or(w.status, kStCorrupt);
    return;
  }
  const uint64_t sbase = (uint64_t)c * kChunk;
  const uint32_t rem = c < cend ? (uint32_t)min((uint64_t)kChunk, n - sbase) : 0u;
  // this lane's chunk from the staged words that start at word `base`
  auto decode_from = [&](const uint32_t* staged_words, uint32_t base) {
    if (c >= cend) return;
    const bool good = b != a && decode_chunk_lds(staged_words + (a - base), b - a, rem, lut, sym + sbase, vec);
    if (!good) status_or(w.status, kStCorrupt);
  };
  if (staged) {
    decode_from(stage, 4 * q0);
    return;
  }
  // The group's words do not fit (codes of about 7 bits and more): each
  // wave's 64 chunks (every chunk now checked, so the offsets increase) take
  // at most 64 * kChunkWords words, which fit the stage, so the waves take
  // turns: one stages its words and decodes while the other waits; every
  // wave passes every barrier.
  static_assert(64 * kChunkWords + 3 <= kStageWords, "a wave's words fit the stage");
  const uint32_t mid = chunk_off[min(c0 + 64u, cend)];  // wave 0: [glo, mid), wave 1: [mid, ghi)
  const uint32_t wlo = wv == 0 ? glo : mid, whi = wv == 0 ? mid : ghi, wq0 = wlo >> 2;
  auto stage_wave = [&](uint32_t* dst) {  // words [4 wq0, whi) of this wave into dst
    const uint4* wq = reinterpret_cast<const uint4*>(words);
    uint4* sq = reinterpret_cast<uint4*>(dst);
    const uint32_t wq1 = whi >> 2;
    for (uint32_t i0 = wq0 + ln; i0 < wq1; i0 += 8 * 64) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t i = i0 + 64 * j;
        v[j] = i < wq1 ? wq[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t i = i0 + 64 * j;
        if (i < wq1) sq[i - wq0] = v[j];
      }
    }
    const uint32_t i = 4 * wq1 + ln;
    if (ln < 3 && i < whi) dst[i - 4 * wq0] = words[i];
    // a wave's LDS operations complete in order: the fence keeps the
    // compiler from moving the chunk reads above these stores
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  if (((uintptr_t)words & 15u) != 0) {  // (aligned by the API's contract)
    if (c < cend) {
      const bool good = b != a && decode_chunk(words + a, b - a, rem, lut, sym + sbase, vec);
      if (!good) status_or(w.status, kStCorrupt);
    }
  } else {
    for (uint32_t pass = 0; pass < kDecChunks / 64; pass++) {
      if (wv == pass) {
        stage_wave(stage);
        decode_from(stage, 4 * wq0);
      }
      __syncthreads();  // the next wave rewrites the stage
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

uint32_t num_chunks(uint64_t n) { return (uint32_t)((n + kChunk - 1) / kChunk); }

uint64_t max_words(uint64_t n) {
  const uint64_t full = n / kChunk, rem = n % kChunk;
  return full * kChunkWords + (rem * kMaxLen + 31) / 32;
}

ec_status check_common(const void* d_books, const void* d_chunk_off, const void* d_sym,
                       const void* d_words, void* d_work, uint32_t nseg, uint64_t n) {
  if (!d_books || !d_chunk_off || !d_work || nseg == 0 || nseg > (uint32_t)kMaxSegments)
    return EC_ERR_INVALID;
  if ((uint64_t)nseg * n > EC_HUFF_MAX_SYMBOLS) return EC_ERR_INVALID;
  if (n && (!d_sym || !d_words)) return EC_ERR_INVALID;
  if (!aligned16(d_sym) || !aligned16(d_words) || ((uintptr_t)d_work & 255u)) return EC_ERR_INVALID;
  return EC_OK;
}

ec_status encode_impl(const uint16_t* d_sym, uint32_t nseg, uint64_t n, uint8_t* d_books,
                      uint32_t* d_chunk_off, uint32_t* d_words, uint64_t words_cap, void* d_work,
                      size_t wbytes, void* stream) {
  const ec_status st = check_common(d_books, d_chunk_off, d_sym, d_words, d_work, nseg, n);
  if (st != EC_OK) return st;
  if (wbytes < work_bytes(nseg) || words_cap < nseg * max_words(n)) return EC_ERR_CAPACITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws w = ws_of(d_work, nseg);
  hipLaunchKernelGGL(huff_clear, dim3(nseg * (kTable / kThreads)), dim3(kThreads), 0, s, w, nseg);
  if (n) {
    const uint64_t want = (n / 8 + kThreads * 4 - 1) / (kThreads * 4);
    const uint64_t cap = 1024 / nseg > 0 ? 1024 / nseg : 1;
    const uint32_t hb = (uint32_t)(want < 1 ? 1 : (want > cap ? cap : want));
    hipLaunchKernelGGL(huff_hist, dim3(hb, nseg), dim3(kThreads), 0, s, d_sym, n, w);
  }
  hipLaunchKernelGGL(huff_book, dim3(nseg), dim3(kBookThreads), 0, s, w, d_books, d_chunk_off, n,
                     (const uint32_t*)nullptr);
  if (n) {
    const uint32_t nch = num_chunks(n);
    uint32_t groups = (nch + 3) / 4;
    const uint32_t gmax = (uint32_t)kMaxGroups / nseg;
    if (groups > gmax) groups = gmax;
    const uint32_t per = (nch + groups - 1) / groups;
    groups = (nch + per - 1) / per;
    hipLaunchKernelGGL(huff_size, dim3(groups, nseg), dim3(kThreads), 0, s, d_sym, n, w,
                       d_chunk_off, nch, per);
    hipLaunchKernelGGL(huff_write, dim3(groups, nseg), dim3(kThreads), 0, s, d_sym, n, w,
                       d_chunk_off, nch, per, d_words);
  }
  return hipGetLastError() == hipSuccess ? EC_OK : EC_ERR_DEVICE;
}

ec_status decode_impl(const uint8_t* d_books, uint64_t book_bytes, const uint32_t* d_chunk_off,
                      const uint32_t* d_words, uint64_t words_cap, uint32_t nseg, uint64_t n,
                      uint16_t* d_sym, void* d_work, size_t wbytes, void* stream) {
  const ec_status st = check_common(d_books, d_chunk_off, d_sym, d_words, d_work, nseg, n);
  if (st != EC_OK) return st;
  if (wbytes < work_bytes(nseg)) return EC_ERR_CAPACITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Ws w = ws_of(d_work, nseg);
  if (n == 0) hipLaunchKernelGGL(huff_clear, dim3(1), dim3(kThreads), 0, s, w, 0u);
  hipLaunchKernelGGL(huff_dec_book, dim3(nseg), dim3(kDecBookThreads), 0, s, d_books, book_bytes,
                     d_chunk_off, n, w, n == 0 ? 1 : 0);
  if (n) {
    const uint32_t nch = num_chunks(n);
    hipLaunchKernelGGL(huff_decode, dim3((nch + kDecChunks - 1) / kDecChunks, nseg),
                       dim3(kDecChunks), 0, s, d_words, words_cap, d_chunk_off, n, nch, w, d_sym);
  }
  return hipGetLastError() == hipSuccess ? EC_OK : EC_ERR_DEVICE;
}

}  // namespace

namespace ec {

// Codebooks of the compressed stream's Huffman segments: huff_book over nseg
// histograms of 4096 bins (hist), giving len << 16 | code per symbol (enc)
// and the codebook bytes at books + seg * EC_HUFF_BOOK_MAX.  status gets the
// builder's error bits (zeroed first by the caller).
hipError_t launch_seg_books(uint32_t* hist, uint32_t* enc, uint8_t* books, uint32_t* status,
                            const uint32_t* skip, uint32_t nseg, hipStream_t s) {
  Ws w{};
  w.status = status;
  w.hist = hist;
  w.enc = enc;
  // n = 1: the chunk table (here the status word) is not written
  hipLaunchKernelGGL(huff_book, dim3(nseg), dim3(kBookThreads), 0, s, w, books, status, (uint64_t)1,
                     skip);
  return hipGetLastError();
}

// Decode tables from nseg codebooks at books + seg * EC_HUFF_BOOK_MAX (each
// padded with zeros past the bytes the stream held): lut[seg][4096] and
// valid[seg] (1 for a well-formed book with at least one symbol); enc is
// scratch, zero_word a device word holding 0, status a scratch word.
hipError_t launch_seg_luts(const uint8_t* books, const uint32_t* zero_word, uint32_t* enc,
                           uint16_t* lut, uint32_t* valid, uint32_t* status, uint32_t nseg,
                           hipStream_t s) {
  Ws w{};
  w.status = status;
  w.valid = valid;
  w.enc = enc;
  w.lut = lut;
  hipLaunchKernelGGL(huff_dec_book, dim3(nseg), dim3(kDecBookThreads), 0, s, books,
                     (uint64_t)kBookStride, zero_word, (uint64_t)1, w, 0);
  return hipGetLastError();
}

}  // namespace ec

extern "C" {

size_t ec_huff_workspace_bytes(void) { return work_bytes(1); }

size_t ec_huff_workspace_bytes_segments(uint32_t nseg) {
  return nseg == 0 || nseg > (uint32_t)kMaxSegments ? 0 : work_bytes(nseg);
}

uint64_t ec_huff_max_words(uint64_t n) { return max_words(n); }

ec_status ec_huff_encode(const uint16_t* d_sym, uint64_t n, uint8_t* d_book,
                         uint32_t* d_chunk_off, uint32_t* d_words, uint64_t words_cap,
                         void* d_work, size_t work_bytes, void* stream) {
  return encode_impl(d_sym, 1, n, d_book, d_chunk_off, d_words, words_cap, d_work, work_bytes,
                     stream);
}

ec_status ec_huff_encode_segments(const uint16_t* d_sym, uint32_t nseg, uint64_t seg_len,
                                  uint8_t* d_books, uint32_t* d_chunk_off, uint32_t* d_words,
                                  uint64_t words_cap, void* d_work, size_t work_bytes,
                                  void* stream) {
  return encode_impl(d_sym, nseg, seg_len, d_books, d_chunk_off, d_words, words_cap, d_work,
                     work_bytes, stream);
}

ec_status ec_huff_decode(const uint8_t* d_book, uint64_t book_bytes, const uint32_t* d_chunk_off,
                         const uint32_t* d_words, uint64_t words_cap, uint64_t n,
                         uint16_t* d_sym, void* d_work, size_t work_bytes, void* stream) {
  return decode_impl(d_book, book_bytes, d_chunk_off, d_words, words_cap, 1, n, d_sym, d_work,
                     work_bytes, stream);
}

ec_status ec_huff_decode_segments(const uint8_t* d_books, const uint32_t* d_chunk_off,
                                  const uint32_t* d_words, uint64_t words_cap, uint32_t nseg,
                                  uint64_t seg_len, uint16_t* d_sym, void* d_work,
                                  size_t work_bytes, void* stream) {
  return decode_impl(d_books, EC_HUFF_BOOK_MAX, d_chunk_off, d_words, words_cap, nseg, seg_len,
                     d_sym, d_work, work_bytes, stream);
}

ec_status ec_huff_status(void* d_work, void* stream) {
  if (!d_work) return EC_ERR_INVALID;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return EC_ERR_DEVICE;
  uint32_t st = 0;
  if (hipMemcpy(&st, d_work, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess) return EC_ERR_DEVICE;
  if (st & kStDepth) return EC_ERR_DEVICE;
  if (st & kStBadSymbol) return EC_ERR_INVALID;
  if (st & kStCorrupt) return EC_ERR_CORRUPT;
  return EC_OK;
}

}  // extern "C"
