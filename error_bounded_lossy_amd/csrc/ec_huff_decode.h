// ec_huff_decode.h -- decoding of one 256-symbol chunk of canonical Huffman
// codes by 12-bit table lookups (gfx950), shared by the standalone coder
// (ec_huffman.hip) and the Huffman segments of the compressed stream
// (ec_kernels.hip).  lut maps every 12-bit prefix to (symbol | length << 12),
// 0 where no code starts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ec {
namespace hd {

template <bool kFull, typename Sink>
__device__ __forceinline__ bool decode_chunk_body(const uint32_t* src, uint32_t nwords,
                                                  uint32_t rem, const uint16_t* lut, Sink&& sink) {
  // two words are loaded ahead of the bit buffer, so a refill never waits
  const uint32_t cnt = kFull ? 256u : rem;
  uint32_t q0 = nwords > 0 ? src[0] : 0u, q1 = nwords > 1 ? src[1] : 0u, p = 2;
  uint64_t bitbuf = 0;
  uint32_t have = 0, mn = 0xFFFFu;
  for (uint32_t g = 0; g < cnt; g += 8) {
    uint32_t pk[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 8; k++) {
      if (have <= 32) {
        bitbuf |= (uint64_t)q0 << (32 - have);
        have += 32;
        q0 = q1;
        q1 = p < nwords ? src[p] : 0u;
        p++;
      }
      const uint32_t ent = lut[bitbuf >> 52];
      const bool act = kFull || g + k < cnt;
      const uint32_t l = act ? ent >> 12 : 0u;
      mn = act ? min(mn, ent) : mn;
      bitbuf <<= l;
      have -= l;
      pk[k >> 1] |= (ent & 0xFFFu) << (16 * (k & 1));
    }
    sink(g, pk, min(cnt - g, 8u));
  }
  // no entry without a code, every consumed bit lies in the chunk (the bits
  // inserted, 32 per word, less what the buffer holds), the chunk's last word
  // holds some of them, and the bits after the last code are zero
  const uint32_t used = 32 * (p - 2) - have;
  return !(mn < (1u << 12) || used > 32 * nwords || used + 32 <= 32 * nwords || bitbuf != 0);
}

// Decode one chunk of `rem` symbols from its nwords words at src (LDS or
// global memory), handing every group of 8 symbols (packed as 16-bit halves
// of pk[4]; the group's first symbol index g, n of them valid) to
// sink(g, pk, n).  The bits are read as if zero words followed the chunk;
// whether it really ends in its last word is decided from the bits consumed.
// Returns false if the chunk is malformed.  A full chunk (256 symbols) runs
// without per-symbol bounds when split is set (as for decode_chunk_lds_sink).
template <typename Sink>
__device__ __forceinline__ bool decode_chunk_sink(const uint32_t* src, uint32_t nwords,
                                                  uint32_t rem, const uint16_t* lut, Sink&& sink,
                                                  bool split = true) {
  return split && rem == 256 ? decode_chunk_body<true>(src, nwords, rem, lut, sink)
                             : decode_chunk_body<false>(src, nwords, rem, lut, sink);
}

// The same, writing the symbols to out[0, rem).
__device__ __forceinline__ bool decode_chunk(const uint32_t* src, uint32_t nwords, uint32_t rem,
                                             const uint16_t* lut, uint16_t* out, bool vec) {
  return decode_chunk_sink(src, nwords, rem, lut, [&](uint32_t g, const uint32_t (&pk)[4], uint32_t n) {
    if (vec && n == 8) {
      *reinterpret_cast<uint4*>(out + g) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    } else {
      for (uint32_t k = 0; k < n; k++) out[g + k] = (uint16_t)(pk[k >> 1] >> (16 * (k & 1)));
    }
  });
}

// The same for a chunk staged in LDS, without branches in the symbol loop.
// The 64-bit buffer holds the chunk's bits [used, 32 p) at its top and zeros
// below; two codes (at most 24 bits) are decoded per refill, which inserts
// the next word wq when 32 or fewer bits remain, so every lookup sees at
// least 12 valid bits and a refill leaves at least 33.  The word after wq is
// loaded at the start of each pair and is needed only at its end.  Words
// past the chunk read as zero.  nwords >= 1.  A full chunk (256 symbols, all
// but a segment's last) runs without per-symbol bounds; an entry with no
// code is found as the smallest entry seen (every code's entry is at least
// 1 << 12).  Groups of 32 symbols go to sink(g, pk, n), packed as 16-bit
// halves of pk[16].
template <bool kFull, typename Sink>
__device__ __forceinline__ bool decode_chunk_lds_body(const uint32_t* src, uint32_t nwords,
                                                      uint32_t rem, const uint16_t* lut,
                                                      Sink&& sink) {
  const uint32_t last = nwords - 1;
  const uint32_t cnt = kFull ? 256u : rem;
  uint64_t bitbuf = (uint64_t)src[0] << 32 | (nwords > 1 ? src[1] : 0u);
  uint32_t used = 0;                         // bits consumed
  uint32_t p = 2;                            // words inserted
  uint32_t wq = nwords > 2 ? src[2] : 0u;    // the next word to insert
  uint32_t mn = 0xFFFFu;
  for (uint32_t g = 0; g < cnt; g += 32) {
    uint32_t pk[16];
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
      const uint32_t wn_raw = src[min(p + 1, last)];
      const uint32_t e1 = lut[bitbuf >> 52];
      const bool a1 = kFull || g + k < cnt;
      const uint32_t l1 = a1 ? e1 >> 12 : 0u;
      bitbuf <<= l1;
      const uint32_t e2 = lut[bitbuf >> 52];
      const bool a2 = kFull || g + k + 1 < cnt;
      const uint32_t l2 = a2 ? e2 >> 12 : 0u;
      bitbuf <<= l2;
      mn = min(mn, min(a1 ? e1 : 0xFFFFu, a2 ? e2 : 0xFFFFu));
      pk[k >> 1] = (e1 | e2 << 16) & 0x0FFF0FFFu;
      used += l1 + l2;
      // 32 p - used bits remain; wq goes right below them
      const uint32_t base = 32 * p - 32;
      const bool rf = used >= base;
      bitbuf |= (uint64_t)(rf ? wq : 0u) << ((used - base) & 63u);
      wq = rf ? (p + 1 <= last ? wn_raw : 0u) : wq;
      p += rf ? 1u : 0u;
    }
    sink(g, pk, min(cnt - g, 32u));
  }
  return !(mn < (1u << 12) || used > 32 * nwords || used + 32 <= 32 * nwords || bitbuf != 0);
}

// split: full chunks take the loop without bounds.  Where the lanes of a wave
// decode the chunks of one record (the last of which is usually partial),
// the two loops would run one after the other: there split is false.
template <typename Sink>
__device__ __forceinline__ bool decode_chunk_lds_sink(const uint32_t* src, uint32_t nwords,
                                                      uint32_t rem, const uint16_t* lut,
                                                      Sink&& sink, bool split = true) {
  return split && rem == 256 ? decode_chunk_lds_body<true>(src, nwords, rem, lut, sink)
                             : decode_chunk_lds_body<false>(src, nwords, rem, lut, sink);
}

__device__ __forceinline__ bool decode_chunk_lds(const uint32_t* src, uint32_t nwords,
                                                 uint32_t rem, const uint16_t* lut,
                                                 uint16_t* out, bool vec) {
  return decode_chunk_lds_sink(src, nwords, rem, lut,
                               [&](uint32_t g, const uint32_t (&pk)[16], uint32_t n) {
    if (vec && n == 32) {  // 64 bytes of one chunk at a time
#pragma unroll
      for (int q = 0; q < 4; q++)
        *reinterpret_cast<uint4*>(out + g + 8 * q) =
            make_uint4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
    } else {
      for (uint32_t k = 0; k < n; k++) out[g + k] = (uint16_t)(pk[k >> 1] >> (16 * (k & 1)));
    }
  });
}

}  // namespace hd
}  // namespace ec
