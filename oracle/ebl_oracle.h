/*
 * ebl_oracle.h -- plain, slow, single-threaded CPU oracle for the
 * error-bounded lossy compressor of DLRM embedding traffic.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this code: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source with the HIP library.
 *
 * Method (arXiv 2407.04272, "Accelerating Communication in Deep Learning
 * Recommendation Model Training with Dual-Level Adaptive Lossy Compression"):
 *   - section III-D: a quantization encoder turns floats into integer bins,
 *     followed by a lossless encoder; no prediction step (III-B, observation 1,
 *     and Fig. 4 show the Lorenzo predictor breaking identical vectors);
 *   - section III-B observation 2 / III-D "Vector-based LZ Encoding": identical
 *     (quantized) embedding vectors are encoded once and referenced;
 *   - section III-C / Algorithm 1: per-table error bound times an
 *     iteration-wise decay factor;
 *   - section III-A stages 1-4 and III-E "Buffer Optimization" (Fig. 7): all
 *     tables of all destination chunks go into ONE contiguous stream whose
 *     per-chunk sizes are the metadata of the variable-size all-to-all.
 *
 * The byte layout below is this project's own (the pages fix no format).
 * All integers are little-endian; every padding byte and unused bit is zero.
 *
 * STREAM
 *   header, 64 bytes:
 *     0  u32 magic 0x434C4245 (bytes "EBLC")   4  u16 version = 1
 *     6  u16 coder: 1 bit-plane packing only, 2 Huffman for every segment
 *        with a valid eb, 3 per segment the smaller of the two
 *                                               8  u32 T (tables)
 *     12 u32 B (rows per table)                 16 u32 D (dim)
 *     20 u32 P (destination chunks)             24 u32 tile_rows = 64
 *     28 u32 eb_mode (0 absolute, 1 range-relative)
 *     32 i64 iter                               40 u64 uncompressed bytes 4*T*B*D
 *     48 u64 total stream bytes                 56 u64 reserved = 0
 *   chunk byte counts: P x u64, zero-padded to a multiple of 16 bytes
 *   chunk 0, chunk 1, ..., chunk P-1
 *
 * CHUNK p (rows [floor(p*B/P), floor((p+1)*B/P)) of every table)
 *   segment offset table: T x u64, offset of segment (p,t) from the chunk
 *   start, zero-padded to 16; then segments (p,0) .. (p,T-1).
 *
 * SEGMENT (p,t)  (16-byte aligned; its size is a multiple of 16)
 *   header, 32 bytes:
 *     0 u32 rows   4 u32 ntiles = ceil(rows/64)   8 f32 eb (0 when invalid)
 *     12 u32 flags (bit 0: eb valid; bit 1: Huffman segment, only with bit 0;
 *        bit 2: windowed references, only with bit 0, and then bits 8-15
 *        hold the window W in 1..255; every other bit 0)
 *     16 u32 U (first occurrences; in a windowed segment, literal rows)
 *     20 u32 n_out (outliers stored in coded tiles)   24 u64 segment bytes
 *   tile directory: ntiles x u32 offset of each tile record from the segment
 *   start, zero-padded to 16; in a Huffman segment then the codebook
 *   (ebl_huffman.c's layout, built from the histogram of the symbols q + 2047
 *   of EVERY first-occurrence row of the segment, outliers as q = 0),
 *   zero-padded to 16; then the tile records in order.
 *   With coder 3 a segment is Huffman iff its Huffman form is strictly
 *   smaller than its bit-plane form; with coder 2 every valid segment is.
 *   Coders chosen per table (Algorithm 2's table-wise configuration) apply
 *   these rules table by table; the stream's coder is then 1 when every
 *   table is 1, 2 when every table is 2, else 3.
 *
 * TILE RECORD (tile k = segment rows [64k, min(64k+64, rows)), n rows)
 *   header, 16 bytes:
 *     0 u64 first-occurrence bitmap (bit i: row 64k+i is the first row of the
 *           segment with its key; 0 for every tile of an invalid-eb segment)
 *     8 u32 n_out   12 u16 U_t = popcount(bitmap)   14 u8 mode   15 u8 0
 *   mode 0 RAW: n*D raw fp32 values, row-major; zero pad to 16.
 *   mode 1 BITPACK, with E = the codes of the tile's first-occurrence rows in
 *   row order, flattened (U_t*D elements), in blocks of 64 (tail padded with
 *   code 0), nblk = ceil(U_t*D/64):
 *     at 16:                  widths, nblk x u8
 *     at align4:              refs, (n-U_t) x (u16 if rows <= 65536 else u32),
 *                             the segment row of each repeated row's first
 *                             occurrence, in row order; in a windowed
 *                             segment (n-U_t) x u8, each the distance o in
 *                             1..W back to the nearest earlier row with the
 *                             same key (the vector-based LZ of section III-D
 *                             with the window of section III-E)
 *     at align4:              outlier positions, n_out x u32, ascending index
 *                             into E
 *     right after:            outlier values, n_out x u32 raw fp32 bits
 *     at align8:              bit planes: block b contributes w_b u64 words,
 *                             word j bit i = bit j of zigzag(E[64b+i])
 *     zero pad to 16.
 *   mode 2 HUFFMAN (Huffman segments only), same E as mode 1:
 *     at 16:                  refs as in mode 1
 *     at align4:              outlier positions and values as in mode 1
 *     right after:            chunk table, (ceil(U_t*D/256) + 1) x u32: word
 *                             offset of each 256-symbol chunk of E's symbols
 *                             q + 2047, then the word count
 *     right after:            the words (u32), each chunk's canonical codes
 *                             MSB first from a word boundary, unused bits 0
 *     zero pad to 16.
 *   A tile is BITPACK (HUFFMAN in a Huffman segment) iff its segment's eb is
 *   valid and that record is strictly smaller than the RAW record; otherwise
 *   RAW.
 *
 * WINDOWED SEGMENTS (window W >= 1): row r repeats when one of the W rows
 * before it in the segment has its key; its match is the nearest such row.
 * Rows without a match are the literals (bitmap bits).  The key of a row is
 * decoded as: a row of a RAW tile, its raw values re-quantized; a literal of
 * a coded tile, its codes and outliers; a repeated row of a coded tile, the
 * key of its match (matches may chain).  Without a window (W = 0) every
 * repeated row names the segment's first row with its key, a literal.
 */
#ifndef EBL_ORACLE_H
#define EBL_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EBO_MAGIC 0x434C4245u
#define EBO_VERSION 1u
#define EBO_CODER_BITPACK 1u
#define EBO_CODER_HUFFMAN 2u
#define EBO_CODER_AUTO 3u
#define EBO_BOOK_PAD 2064u /* largest codebook (4 + 2048 bytes) padded to 16 */
#define EBO_TILE_ROWS 64u
#define EBO_QMAX 2047

enum { EBO_OK = 0, EBO_ERR_INVALID = 1, EBO_ERR_CAPACITY = 2, EBO_ERR_CORRUPT = 3,
       EBO_ERR_OOM = 5 };
enum { EBO_EB_ABS = 0, EBO_EB_REL = 1 };
enum { EBO_SCHED_NONE = 0, EBO_SCHED_INV_SQRT = 1, EBO_SCHED_STEP = 2 };

typedef struct {
  uint32_t T, B, D, P;
  uint32_t eb_mode;          /* EBO_EB_ABS or EBO_EB_REL                  */
  const float* eb;           /* [T] absolute eb, or range factor (REL)     */
  const float* table_mult;   /* [T] table-class multiplier, NULL means 1   */
  int32_t sched_kind;        /* EBO_SCHED_*                                */
  int32_t sched_steps;       /* STEP: number of stairs                     */
  double sched_t0;           /* INV_SQRT: (1 + i/t0)^-1/2                  */
  double sched_k;            /* STEP: starting multiple of the base eb     */
  int64_t sched_phase;       /* STEP: length of the decay phase            */
  uint32_t coder;            /* EBO_CODER_*; 0 means EBO_CODER_BITPACK     */
  const int32_t* table_coder; /* [T] coder of each table, NULL: `coder`    */
  uint32_t window;           /* 0: references to first occurrences; 1..255:
                                windowed references (section III-E)        */
  uint8_t* book_len;         /* [P*T][EBO_HUFF_NSYM] code lengths kept from the
                                last call, or NULL: every Huffman segment
                                builds its code (see below); in/out        */
  uint8_t* book_have;        /* [P*T] 1: book_len[s] holds a code; in/out  */
} ebo_cfg;

/* Codebook reuse across calls (book_len != NULL): the value distribution of a
 * table changes little from one training iteration to the next (section IV,
 * Fig. 14), so a segment that may be Huffman-coded (valid eb, coder not bit
 * planes) keeps the code of its previous call while that code has a length
 * for every symbol the segment now holds; otherwise it builds a code from
 * its histogram and keeps that one.  Segments that cannot be Huffman-coded
 * keep no code.  The code used is the one stored in the segment. */

/* Iteration-wise factor (Algorithm 1 OnlineDecay, read non-cumulatively). */
double ebo_schedule(const ebo_cfg* c, int64_t iter);
/* f_t = (float)((double)eb[t] * (double)mult[t] * schedule(iter)). */
float ebo_table_factor(const ebo_cfg* c, uint32_t t, int64_t iter);
/* min/max over the non-NaN values (+INF/-INF when there are none). */
void ebo_range(const float* x, size_t n, float* lo, float* hi);
int ebo_eb_valid(float eb);
/* Linear quantization of one value; returns 1 for an outlier (q set to 0). */
int ebo_quantize(float x, float eb, int32_t* q);
float ebo_dequantize(int32_t q, float eb);
uint32_t ebo_zigzag(int32_t q);
int32_t ebo_unzigzag(uint32_t z);

/* Eq. (1) Homogenization Index: (N_original - N_compressed) / N_original. */
double ebo_homo_index(uint64_t n_original, uint64_t n_compressed);

/* The counts eq. (1) takes, per segment s = p*T + t (the "# Ori. Patterns"
 * and "# Quant. Patterns" columns of Tables III and IV): n_orig[s] = number of
 * distinct rows of the segment as fp32 bit patterns, n_quant[s] = number of
 * distinct quantized rows (the repeated-row key of the compressor, i.e. its
 * U).  A segment whose eb is invalid is not quantized: n_quant = n_orig. */
int ebo_homo_counts(const ebo_cfg* c, int64_t iter, const float* x, uint32_t* n_orig,
                    uint32_t* n_quant);

/* Algorithm 1, EMBClassification and OfflineAnalysis: table t is 'small'
 * (class 2, multiplier 1/beta) when hindex[t] > s_thresh, 'large' (class 0,
 * multiplier alpha) when hindex[t] < l_thresh, else 'medium' (class 1,
 * multiplier 1).  Multipliers are rounded once to fp32.  Returns -1 for
 * l_thresh > s_thresh or alpha, beta not finite and > 0. */
int ebo_classify(uint32_t T, const double* hindex, double l_thresh, double s_thresh,
                 double alpha, double beta, int32_t* cls, float* mult);

/* Eq. (2): the communication speed-up of a compressor with compression
 * ratio cr and compression / decompression throughputs tc, td over a link of
 * bandwidth bw (throughputs and bandwidth in the same unit):
 * 1 / (1/cr + bw * (1/tc + 1/td)). */
double ebo_speedup(double cr, double bw, double tc, double td);

/* Algorithm 2 (OfflineCompConfig): for each of T tables, the compressor of
 * the pool (ncomp of them; cr[c*T + t], tc[c], td[c]) with the largest
 * eq. (2) speed-up; on equal speed-ups the earlier compressor.  best[t] and,
 * if not NULL, its speed-up sp[t].  -1 for an empty pool or values that are
 * not finite and > 0. */
int ebo_select(uint32_t T, uint32_t ncomp, const double* cr, const double* tc, const double* td,
               double bw, int32_t* best, double* sp);

/* Per-table error bound used for every segment of table t (fp32). */
float ebo_table_eb(const ebo_cfg* c, uint32_t t, int64_t iter, const float* x);

/* Size of the stream when every tile is RAW: the compressed-size bound. */
size_t ebo_max_compressed_bytes(const ebo_cfg* c);

/*
 * Compress x[T][B][D] (row-major fp32) into out.  Optional outputs (NULL to
 * skip): codes[T*B*D] (0 for outliers), outlier[T*B*D] (0/1),
 * first[T*B] (segment row of each row's first occurrence, with a window its
 * match; the row itself for literals and invalid-eb segments), eb_seg[P*T]
 * (segment eb as stored).
 */
int ebo_compress(const ebo_cfg* c, int64_t iter, const float* x, uint8_t* out, size_t cap,
                 size_t* out_bytes, int32_t* codes, uint8_t* outlier, uint32_t* first,
                 float* eb_seg);

/* Decompress a stream whose header matches (T,B,D,P); y gets T*B*D floats. */
int ebo_decompress(const uint8_t* s, size_t nbytes, uint32_t T, uint32_t B, uint32_t D,
                   uint32_t P, float* y);

/*
 * Canonical Huffman coder of the quantization codes (ebl_huffman.c): the
 * entropy stage of section III-D, with the construction, length limit, bit
 * order and codebook layout fixed as described in that file's header.
 * Symbols are q + 2047 (EBO_HUFF_NSYM of them); codes are at most
 * EBO_HUFF_MAXLEN bits; every EBO_HUFF_CHUNK symbols start a new 32-bit word.
 */
#define EBO_HUFF_NSYM 4095
#define EBO_HUFF_MAXLEN 12
#define EBO_HUFF_CHUNK 256

/* Code lengths (0 = unused) from symbol frequencies; returns the number of
   used symbols.  One used symbol gets length 1. */
int ebo_huff_lengths(const uint64_t* freq, uint8_t* len);
/* Canonical code of every symbol (RFC 1951 section 3.2.2), right-aligned. */
void ebo_huff_codes(const uint8_t* len, uint32_t* code);
/* Encode n symbols; chunk_off gets ceil(n/256)+1 word offsets (the last is
   the word count, which is returned).  words must hold 12*n/32 + n/256 + 1. */
size_t ebo_huff_encode(const uint16_t* sym, size_t n, const uint8_t* len, const uint32_t* code,
                       uint32_t* words, uint32_t* chunk_off);
/* Decode n symbols; 0, or -1 if any chunk is malformed (a code that is not in
   the book, a chunk that does not end in its last word, nonzero padding). */
int ebo_huff_decode(const uint32_t* words, size_t nwords, const uint32_t* chunk_off, size_t n,
                    const uint8_t* len, uint16_t* sym);
/* Codebook: u16 lowest used symbol, u16 highest, 4-bit lengths low nibble
   first.  No used symbol is stored as lo = 1, hi = 0. */
size_t ebo_huff_book_bytes(const uint8_t* len);
size_t ebo_huff_book_write(const uint8_t* len, uint8_t* out);
/* 0, or -1 for a book that is short, not tight, or not a complete code. */
int ebo_huff_book_read(const uint8_t* in, size_t nbytes, uint8_t* len);

#ifdef __cplusplus
}
#endif
#endif
