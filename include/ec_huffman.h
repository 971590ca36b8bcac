/*
 * ec_huffman.h -- C ABI of the canonical Huffman coder for quantization codes
 * (gfx950), the lossless stage that section III-D of arXiv 2407.04272 places
 * after the quantization encoder ("Huffman Encoding"; Table V and Fig. 11
 * give its compression ratios and throughputs).
 *
 * The pages fix no construction, code-length limit or bit order; this coder
 * fixes them so that exactly one stream is correct for a given input:
 *   - symbols are quantization codes q in [-2047, 2047] stored as q + 2047,
 *     an alphabet of EC_HUFF_NSYM = 4095 symbols (u16, values above 4094 are
 *     invalid input);
 *   - the code is an optimal Huffman code built with two queues, where of
 *     two equal weights the leaf is merged first; lengths above
 *     EC_HUFF_MAXLEN = 12 are removed by the count adjustment of ITU-T T.81
 *     Annex K.3 (without JPEG's reserved all-ones code word);
 *   - lengths are handed out shortest first in order of decreasing frequency,
 *     then increasing symbol; codes are canonical (RFC 1951 section 3.2.2);
 *   - codes are written most significant bit first into 32-bit words (bit 31
 *     of a word is its first bit); every EC_HUFF_CHUNK = 256 symbols start a
 *     new word, unused bits are zero;
 *   - the chunk table has ceil(n / 256) + 1 u32 entries: the word offset of
 *     every chunk, then the total word count;
 *   - the codebook is u16 lowest used symbol, u16 highest used symbol (both
 *     little-endian), then one 4-bit length per symbol of that range, low
 *     nibble first, the last byte's unused nibble zero.  With no symbol
 *     (n = 0) it is the 4 bytes lo = 1, hi = 0.  A single used symbol has
 *     length 1 (code 0).
 *
 * Conventions: as in ec.h.  Device pointers must be 16-byte aligned and stay
 * valid until the enqueued work has finished; `stream` is a hipStream_t (NULL
 * = default stream); the caller owns every buffer, including the workspace
 * (ec_huff_workspace_bytes() bytes, 256-byte aligned), which one call at a
 * time may use.  The entry points enqueue kernels and return; they never
 * allocate or synchronize, except ec_huff_status, which waits.  Argument
 * errors are returned before anything is enqueued; conditions found on the
 * device are reported by ec_huff_status.
 */
#ifndef EC_HUFFMAN_H
#define EC_HUFFMAN_H

#include <stddef.h>
#include <stdint.h>

#include "ec.h"

#ifdef __cplusplus
extern "C" {
#endif

#define EC_HUFF_NSYM 4095u
#define EC_HUFF_MAXLEN 12u
#define EC_HUFF_CHUNK 256u
#define EC_HUFF_BOOK_MAX (4u + (EC_HUFF_NSYM + 1u) / 2u) /* 2052 bytes        */
#define EC_HUFF_MAX_SYMBOLS 0x7FFFFFFFull                /* n < 2^31 in all   */
#define EC_HUFF_MAX_SEGMENTS 2048u

/* Workspace bytes one encode or decode call needs (independent of n). */
size_t ec_huff_workspace_bytes(void);

/* Workspace bytes of a call over nseg segments (0 if nseg is 0 or above
 * EC_HUFF_MAX_SEGMENTS). */
size_t ec_huff_workspace_bytes_segments(uint32_t nseg);

/* Words an encoded stream of n symbols can take at most (12 bits per symbol,
 * every chunk rounded up to whole words). */
uint64_t ec_huff_max_words(uint64_t n);

/* Encode n symbols (d_sym, u16 [n]).  Writes the codebook (d_book, capacity
 * EC_HUFF_BOOK_MAX bytes; its size follows from its first 4 bytes), the chunk
 * table (d_chunk_off, u32 [ceil(n/256) + 1]) and the words (d_words, u32
 * [words_cap], words_cap >= ec_huff_max_words(n)).  A symbol above 4094 makes
 * ec_huff_status return EC_ERR_INVALID and the output meaningless.
 * Returns EC_ERR_INVALID for NULL pointers or n > EC_HUFF_MAX_SYMBOLS,
 * EC_ERR_CAPACITY for a short words_cap or workspace. */
ec_status ec_huff_encode(const uint16_t* d_sym, uint64_t n, uint8_t* d_book,
                         uint32_t* d_chunk_off, uint32_t* d_words, uint64_t words_cap,
                         void* d_work, size_t work_bytes, void* stream);

/* Decode n symbols into d_sym (u16 [n]) from a codebook of book_bytes bytes,
 * a chunk table of ceil(n/256) + 1 entries and words_cap readable words.
 * Every field is validated on the device: a codebook that is short, not
 * tight (lowest and highest symbol unused) or not a complete code, a chunk
 * table that is not increasing from 0 or points past words_cap, a chunk that
 * needs bits past its end, does not end in its last word or has nonzero
 * padding make ec_huff_status return EC_ERR_CORRUPT; the symbols of such a
 * chunk are then unspecified. */
ec_status ec_huff_decode(const uint8_t* d_book, uint64_t book_bytes, const uint32_t* d_chunk_off,
                         const uint32_t* d_words, uint64_t words_cap, uint64_t n,
                         uint16_t* d_sym, void* d_work, size_t work_bytes, void* stream);

/* Segments: nseg consecutive runs of seg_len symbols each (one per embedding
 * table, say), every one coded with a codebook of its own, as ec_huff_encode
 * would code it alone.  Chunks never cross segments: segment s owns chunks
 * [s*C, (s+1)*C) of the chunk table, C = ceil(seg_len / 256), which has
 * nseg*C + 1 entries; the words of all segments follow each other in one
 * array (offsets in the table are from its start).  Codebook s sits at
 * d_books + s * EC_HUFF_BOOK_MAX.  words_cap >= nseg * ec_huff_max_words(
 * seg_len); the workspace holds ec_huff_workspace_bytes_segments(nseg) bytes.
 * Errors as for ec_huff_encode, plus EC_ERR_INVALID for nseg outside
 * [1, EC_HUFF_MAX_SEGMENTS] or nseg * seg_len > EC_HUFF_MAX_SYMBOLS. */
ec_status ec_huff_encode_segments(const uint16_t* d_sym, uint32_t nseg, uint64_t seg_len,
                                  uint8_t* d_books, uint32_t* d_chunk_off, uint32_t* d_words,
                                  uint64_t words_cap, void* d_work, size_t work_bytes,
                                  void* stream);

/* Decode what ec_huff_encode_segments wrote (each codebook has
 * EC_HUFF_BOOK_MAX readable bytes); validation as for ec_huff_decode, per
 * segment. */
ec_status ec_huff_decode_segments(const uint8_t* d_books, const uint32_t* d_chunk_off,
                                  const uint32_t* d_words, uint64_t words_cap, uint32_t nseg,
                                  uint64_t seg_len, uint16_t* d_sym, void* d_work,
                                  size_t work_bytes, void* stream);

/* Wait for `stream`, then return the device status of the last encode or
 * decode call that used this workspace: EC_OK, EC_ERR_INVALID (symbol out of
 * the alphabet), EC_ERR_CORRUPT (decode validation failed) or EC_ERR_DEVICE. */
ec_status ec_huff_status(void* d_work, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EC_HUFFMAN_H */
