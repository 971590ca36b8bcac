/*
 * ebl_huffman.c -- canonical Huffman coder of the oracle (plain C, slow,
 * single-threaded).  TEST INFRASTRUCTURE ONLY, like the rest of oracle/.
 *
 * The paper's entropy stage (section III-D "Huffman Encoding", Table V's
 * Huffman column) codes the quantization codes with a Huffman code; it fixes
 * neither the tree construction nor a code-length limit nor a bit order.
 * This file fixes them so that one stream is the only correct output:
 *
 *   symbols      sym = q + 2047 for codes q in [-2047, 2047] (an outlier's
 *                code counts as q = 0): an alphabet of 4095 symbols
 *   tree         two queues (leaves sorted by frequency, then symbol;
 *                internal nodes in creation order); of two equal weights the
 *                leaf is taken first
 *   length limit 12 bits: the counts of codes per length are adjusted as in
 *                ITU-T T.81 (JPEG) Annex K.3, without JPEG's removal of the
 *                all-ones code word, so the code stays complete
 *   lengths      given to the symbols in order of frequency (highest first),
 *                then symbol, shortest length first
 *   codes        canonical, as in RFC 1951 section 3.2.2 (by length, then
 *                symbol)
 *   bits         most significant bit first into 32-bit words; a word's bit
 *                31 is the first; each chunk of 256 symbols starts on a word
 *                boundary, unused bits are zero
 *   codebook     u16 lowest used symbol, u16 highest, then a 4-bit length per
 *                symbol of that range, low nibble first, the last byte
 *                zero-padded (lowest 1, highest 0 when no symbol is used)
 */
#include "ebl_oracle.h"

#include <stdlib.h>
#include <string.h>

/* order of leaves: frequency ascending, then symbol ascending */
static const uint64_t* g_sort_freq;
static int leaf_order(const void* a, const void* b) {
  uint16_t x = *(const uint16_t*)a, y = *(const uint16_t*)b;
  if (g_sort_freq[x] != g_sort_freq[y]) return g_sort_freq[x] < g_sort_freq[y] ? -1 : 1;
  return x < y ? -1 : (x > y ? 1 : 0);
}
/* order for handing out lengths: frequency descending, then symbol ascending */
static int rank_order(const void* a, const void* b) {
  uint16_t x = *(const uint16_t*)a, y = *(const uint16_t*)b;
  if (g_sort_freq[x] != g_sort_freq[y]) return g_sort_freq[x] > g_sort_freq[y] ? -1 : 1;
  return x < y ? -1 : (x > y ? 1 : 0);
}

int ebo_huff_lengths(const uint64_t* freq, uint8_t* len) {
  memset(len, 0, EBO_HUFF_NSYM);
  uint16_t leaves[EBO_HUFF_NSYM];
  int m = 0;
  for (int s = 0; s < EBO_HUFF_NSYM; s++)
    if (freq[s]) leaves[m++] = (uint16_t)s;
  if (m == 0) return 0;
  if (m == 1) {
    len[leaves[0]] = 1;
    return 1;
  }
  g_sort_freq = freq;
  qsort(leaves, (size_t)m, sizeof(uint16_t), leaf_order);

  /* nodes 0..m-1 are the sorted leaves, m..2m-2 internal nodes in creation
     order; parent[] links each node to the internal node that took it */
  int nn = 2 * m - 1;
  uint64_t* w = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)nn);
  int* parent = (int*)malloc(sizeof(int) * (size_t)nn);
  for (int i = 0; i < m; i++) w[i] = freq[leaves[i]];
  int lq = 0, iq = m, next = m; /* fronts of the two queues; next internal node */
  while (next < nn) {
    int pick[2];
    for (int k = 0; k < 2; k++) {
      int use_leaf;
      if (lq >= m) use_leaf = 0;
      else if (iq >= next) use_leaf = 1;
      else use_leaf = w[lq] <= w[iq]; /* equal weights: the leaf first */
      pick[k] = use_leaf ? lq++ : iq++;
    }
    w[next] = w[pick[0]] + w[pick[1]];
    parent[pick[0]] = parent[pick[1]] = next;
    next++;
  }
  /* depth of every leaf; BITS[l] = number of leaves at depth l */
  uint32_t* bits = (uint32_t*)calloc((size_t)m, sizeof(uint32_t)); /* depth < m */
  int maxd = 0;
  for (int i = 0; i < m; i++) {
    int d = 0;
    for (int v = i; v != nn - 1; v = parent[v]) d++;
    bits[d]++;
    if (d > maxd) maxd = d;
  }
  free(w);
  free(parent);

  /* T.81 Annex K.3: move pairs of the longest codes up until none is longer
     than the limit (each step keeps the Kraft sum at 1) */
  int i = maxd;
  while (i > EBO_HUFF_MAXLEN) {
    if (bits[i] > 0) {
      int j = i - 2;
      while (bits[j] == 0) j--;
      bits[i] -= 2;
      bits[i - 1] += 1;
      bits[j + 1] += 2;
      bits[j] -= 1;
    } else {
      i--;
    }
  }

  /* lengths, shortest first, to the symbols by descending frequency */
  qsort(leaves, (size_t)m, sizeof(uint16_t), rank_order);
  int at = 0;
  for (int l = 1; l <= EBO_HUFF_MAXLEN; l++)
    for (uint32_t c = 0; c < (l < m ? bits[l] : 0); c++) len[leaves[at++]] = (uint8_t)l;
  free(bits);
  return m;
}

void ebo_huff_codes(const uint8_t* len, uint32_t* code) {
  uint32_t count[EBO_HUFF_MAXLEN + 1], next[EBO_HUFF_MAXLEN + 2];
  memset(count, 0, sizeof(count));
  for (int s = 0; s < EBO_HUFF_NSYM; s++)
    if (len[s]) count[len[s]]++;
  uint32_t c = 0;
  next[1] = 0;
  for (int l = 1; l <= EBO_HUFF_MAXLEN; l++) {
    c = (c + (l > 1 ? count[l - 1] : 0)) << (l > 1 ? 1 : 0);
    next[l] = c;
  }
  for (int s = 0; s < EBO_HUFF_NSYM; s++) {
    code[s] = 0;
    if (len[s]) code[s] = next[len[s]]++;
  }
}

/* bit writer: MSB first into 32-bit words */
typedef struct {
  uint32_t* w;
  size_t word, nbits; /* current word, bits already in it */
} bitw;
static void put_bits(bitw* b, uint32_t v, int n) {
  for (int k = n - 1; k >= 0; k--) {
    uint32_t bit = (v >> k) & 1u;
    if (b->nbits == 0) b->w[b->word] = 0;
    b->w[b->word] |= bit << (31 - b->nbits);
    if (++b->nbits == 32) {
      b->word++;
      b->nbits = 0;
    }
  }
}

size_t ebo_huff_encode(const uint16_t* sym, size_t n, const uint8_t* len, const uint32_t* code,
                       uint32_t* words, uint32_t* chunk_off) {
  bitw b = {words, 0, 0};
  size_t nchunks = (n + EBO_HUFF_CHUNK - 1) / EBO_HUFF_CHUNK;
  for (size_t c = 0; c < nchunks; c++) {
    if (b.nbits) { /* the chunk starts on a word boundary */
      b.word++;
      b.nbits = 0;
    }
    chunk_off[c] = (uint32_t)b.word;
    size_t end = (c + 1) * EBO_HUFF_CHUNK < n ? (c + 1) * EBO_HUFF_CHUNK : n;
    for (size_t i = c * EBO_HUFF_CHUNK; i < end; i++) put_bits(&b, code[sym[i]], len[sym[i]]);
  }
  size_t total = b.word + (b.nbits ? 1 : 0);
  chunk_off[nchunks] = (uint32_t)total;
  return total;
}

int ebo_huff_decode(const uint32_t* words, size_t nwords, const uint32_t* chunk_off, size_t n,
                    const uint8_t* len, uint16_t* sym) {
  /* canonical decoding tables: per length the first code, the number of
     codes and the index of its first symbol in (length, symbol) order */
  uint32_t count[EBO_HUFF_MAXLEN + 1], first[EBO_HUFF_MAXLEN + 1], base[EBO_HUFF_MAXLEN + 1];
  uint16_t order[EBO_HUFF_NSYM];
  memset(count, 0, sizeof(count));
  int m = 0;
  for (int l = 1; l <= EBO_HUFF_MAXLEN; l++)
    for (int s = 0; s < EBO_HUFF_NSYM; s++)
      if (len[s] == l) {
        order[m++] = (uint16_t)s;
        count[l]++;
      }
  uint32_t c = 0, idx = 0;
  for (int l = 1; l <= EBO_HUFF_MAXLEN; l++) {
    c = (c + (l > 1 ? count[l - 1] : 0)) << (l > 1 ? 1 : 0);
    first[l] = c;
    base[l] = idx;
    idx += count[l];
  }
  size_t nchunks = (n + EBO_HUFF_CHUNK - 1) / EBO_HUFF_CHUNK;
  if (n && m == 0) return -1;
  if (chunk_off[0] != 0 || chunk_off[nchunks] > nwords) return -1;
  for (size_t ch = 0; ch < nchunks; ch++) {
    if (chunk_off[ch + 1] < chunk_off[ch]) return -1;
    size_t word = chunk_off[ch], lim = chunk_off[ch + 1], nbits = 0;
    size_t end = (ch + 1) * EBO_HUFF_CHUNK < n ? (ch + 1) * EBO_HUFF_CHUNK : n;
    for (size_t i = ch * EBO_HUFF_CHUNK; i < end; i++) {
      uint32_t v = 0;
      int l = 0, found = 0;
      while (l < EBO_HUFF_MAXLEN) {
        if (word >= lim) return -1;
        uint32_t bit = (words[word] >> (31 - nbits)) & 1u;
        if (++nbits == 32) {
          word++;
          nbits = 0;
        }
        v = (v << 1) | bit;
        l++;
        if (count[l] && v - first[l] < count[l]) {
          sym[i] = order[base[l] + (v - first[l])];
          found = 1;
          break;
        }
      }
      if (!found) return -1;
    }
    /* the chunk ends in its last word; its unused bits are zero */
    size_t used_end = word + (nbits ? 1 : 0);
    if (used_end != lim) return -1;
    if (nbits && (words[word] & (0xFFFFFFFFu >> nbits))) return -1;
  }
  return 0;
}

size_t ebo_huff_book_bytes(const uint8_t* len) {
  int lo = -1, hi = -1;
  for (int s = 0; s < EBO_HUFF_NSYM; s++)
    if (len[s]) {
      if (lo < 0) lo = s;
      hi = s;
    }
  if (lo < 0) return 4;
  return 4 + ((size_t)(hi - lo + 1) + 1) / 2;
}

size_t ebo_huff_book_write(const uint8_t* len, uint8_t* out) {
  int lo = -1, hi = -1;
  for (int s = 0; s < EBO_HUFF_NSYM; s++)
    if (len[s]) {
      if (lo < 0) lo = s;
      hi = s;
    }
  if (lo < 0) {
    lo = 1;
    hi = 0;
  }
  out[0] = (uint8_t)lo;
  out[1] = (uint8_t)(lo >> 8);
  out[2] = (uint8_t)hi;
  out[3] = (uint8_t)(hi >> 8);
  size_t nb = hi >= lo ? (size_t)(hi - lo + 1) : 0, bytes = (nb + 1) / 2;
  memset(out + 4, 0, bytes);
  for (size_t k = 0; k < nb; k++) out[4 + k / 2] |= (uint8_t)(len[lo + k] << (4 * (k & 1)));
  return 4 + bytes;
}

int ebo_huff_book_read(const uint8_t* in, size_t nbytes, uint8_t* len) {
  memset(len, 0, EBO_HUFF_NSYM);
  if (nbytes < 4) return -1;
  uint32_t lo = in[0] | (in[1] << 8), hi = in[2] | (in[3] << 8);
  if (hi < lo) return lo == 1 && hi == 0 ? 0 : -1;
  if (hi >= EBO_HUFF_NSYM) return -1;
  size_t nb = hi - lo + 1, bytes = (nb + 1) / 2;
  if (nbytes < 4 + bytes) return -1;
  for (size_t k = 0; k < nb; k++) {
    uint8_t l = (uint8_t)((in[4 + k / 2] >> (4 * (k & 1))) & 15u);
    if (l > EBO_HUFF_MAXLEN) return -1;
    len[lo + k] = l;
  }
  if ((nb & 1) && (in[4 + nb / 2] >> 4)) return -1; /* padding nibble */
  if (!len[lo] || !len[hi]) return -1;              /* the range is tight */
  /* a complete prefix code (or a single symbol of length 1) */
  uint64_t kraft = 0;
  int m = 0;
  for (int s = 0; s < EBO_HUFF_NSYM; s++)
    if (len[s]) {
      kraft += 1ull << (EBO_HUFF_MAXLEN - len[s]);
      m++;
    }
  if (m == 1) return len[lo] == 1 ? 0 : -1;
  return kraft == (1ull << EBO_HUFF_MAXLEN) ? 0 : -1;
}
