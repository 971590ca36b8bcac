/*
 * ebl_oracle.c -- the CPU oracle (test infrastructure only; see ebl_oracle.h
 * for the stream layout).  Single-threaded, plain loops, fp32 arithmetic in
 * IEEE single precision, built with -ffp-contract=off and no fast-math.
 *
 * Readings of the pages taken here (arXiv 2407.04272):
 *  - quantization q = round(x / (2 eb)), round half to even, |q| <= 2047;
 *    a value whose reconstruction misses the bound is kept verbatim
 *    (section III-D quantization encoder; the per-element bound is the
 *    "strict error control" of section I);
 *  - repeated vectors are detected AFTER quantization over the whole segment
 *    (section III-B observation 2, "Vector Homogenization"; Tables III/IV
 *    count quantized patterns);
 *  - the decay factor multiplies the configured table eb (Algorithm 1,
 *    OnlineDecay), applied non-cumulatively: f = eb_t * mult_t * sched(i).
 */
#include "ebl_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* little-endian byte access                                           */
/* ------------------------------------------------------------------ */
static void put_u8(uint8_t* p, uint8_t v) { p[0] = v; }
static void put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
}
static void put_u32(uint8_t* p, uint32_t v) {
  for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_f32(uint8_t* p, float f) {
  uint32_t v;
  memcpy(&v, &f, 4);
  put_u32(p, v);
}
static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t* p) {
  uint32_t v = 0;
  for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i);
  return v;
}
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}
static float get_f32(const uint8_t* p) {
  uint32_t v = get_u32(p);
  float f;
  memcpy(&f, &v, 4);
  return f;
}
static uint32_t f32_bits(float f) {
  uint32_t v;
  memcpy(&v, &f, 4);
  return v;
}
static float bits_f32(uint32_t v) {
  float f;
  memcpy(&f, &v, 4);
  return f;
}
static uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
static uint32_t popcount64(uint64_t v) {
  uint32_t c = 0;
  while (v) {
    c += (uint32_t)(v & 1u);
    v >>= 1;
  }
  return c;
}

/* ------------------------------------------------------------------ */
/* error-bound policy: Algorithm 1 and section III-C                   */
/* ------------------------------------------------------------------ */
double ebo_schedule(const ebo_cfg* c, int64_t iter) {
  int64_t i = iter < 0 ? 0 : iter;
  if (c->sched_kind == EBO_SCHED_INV_SQRT) {
    /* a smooth decay function: (1 + i/t0)^(-1/2) */
    return pow(1.0 + (double)i / c->sched_t0, -0.5);
  }
  if (c->sched_kind == EBO_SCHED_STEP) {
    /* step-wise (staircase) decay, the pages' default decay function:
       from k*eb down to eb in `steps` equal stairs over `phase` iterations,
       then constant (the "later phase") */
    int64_t ph = c->sched_phase;
    int64_t m = i < ph ? i : ph;
    int64_t stair = (int64_t)c->sched_steps * m / ph; /* integer floor */
    double drop = ((c->sched_k - 1.0) * (double)stair) / (double)c->sched_steps;
    return c->sched_k - drop;
  }
  return 1.0;
}

float ebo_table_factor(const ebo_cfg* c, uint32_t t, int64_t iter) {
  double mult = c->table_mult ? (double)c->table_mult[t] : 1.0;
  double f = (double)c->eb[t] * mult;
  f = f * ebo_schedule(c, iter);
  return (float)f;
}

void ebo_range(const float* x, size_t n, float* lo, float* hi) {
  float l = INFINITY, h = -INFINITY;
  for (size_t i = 0; i < n; i++) {
    float v = x[i];
    if (isnan(v)) continue;
    if (v < l) l = v;
    if (v > h) h = v;
  }
  *lo = l;
  *hi = h;
}

int ebo_eb_valid(float eb) {
  if (!isfinite(eb)) return 0;
  if (!(eb > 0.0f)) return 0;
  float s = eb + eb;
  return isfinite(s) ? 1 : 0;
}

float ebo_table_eb(const ebo_cfg* c, uint32_t t, int64_t iter, const float* x) {
  float f = ebo_table_factor(c, t, iter);
  if (c->eb_mode == EBO_EB_ABS) return f;
  /* range-relative: f times (max - min) of this call's lookups of table t */
  float lo = INFINITY, hi = -INFINITY;
  if (x && c->B > 0) ebo_range(x + (size_t)t * c->B * c->D, (size_t)c->B * c->D, &lo, &hi);
  float range = hi - lo;
  return f * range;
}

/* ------------------------------------------------------------------ */
/* quantization encoder (section III-D)                                */
/* ------------------------------------------------------------------ */
int ebo_quantize(float x, float eb, int32_t* q) {
  float s = eb + eb; /* bin width 2 eb: every bin centre is within eb of its bin */
  float t = x / s;
  if (!(fabsf(t) <= (float)EBO_QMAX)) { /* also NaN and +-Inf */
    *q = 0;
    return 1;
  }
  float qf = rintf(t); /* default rounding mode: to nearest, ties to even */
  float xh = qf * s;
  float err = x - xh;
  if (!(fabsf(err) <= eb)) {
    *q = 0;
    return 1;
  }
  *q = (int32_t)qf;
  return 0;
}

float ebo_dequantize(int32_t q, float eb) {
  float s = eb + eb;
  return (float)q * s;
}

uint32_t ebo_zigzag(int32_t q) {
  return q >= 0 ? (uint32_t)q * 2u : (uint32_t)(-(int64_t)q) * 2u - 1u;
}

int32_t ebo_unzigzag(uint32_t z) {
  return (z & 1u) ? -(int32_t)((z + 1u) / 2u) : (int32_t)(z / 2u);
}

double ebo_homo_index(uint64_t n_original, uint64_t n_compressed) {
  return ((double)n_original - (double)n_compressed) / (double)n_original;
}

/* ------------------------------------------------------------------ */
/* shape helpers                                                       */
/* ------------------------------------------------------------------ */
static uint32_t chunk_row0(const ebo_cfg* c, uint32_t p) {
  return (uint32_t)((uint64_t)p * c->B / c->P);
}
static uint32_t chunk_rows(const ebo_cfg* c, uint32_t p) {
  return chunk_row0(c, p + 1) - chunk_row0(c, p);
}
static uint64_t raw_record_bytes(uint32_t n, uint32_t D) {
  return 16 + align_up((uint64_t)4 * n * D, 16);
}
static uint64_t seg_prefix_bytes(uint32_t ntiles) {
  return 32 + align_up((uint64_t)4 * ntiles, 16);
}
static int cfg_ok(const ebo_cfg* c) {
  if (!c || !c->eb) return 0;
  if (c->T < 1 || c->D < 1 || c->P < 1) return 0;
  if (c->eb_mode != EBO_EB_ABS && c->eb_mode != EBO_EB_REL) return 0;
  if (c->coder > EBO_CODER_AUTO) return 0;
  if (c->window > 255) return 0;
  if ((c->book_len == NULL) != (c->book_have == NULL)) return 0;
  if (c->table_coder)
    for (uint32_t t = 0; t < c->T; t++)
      if (c->table_coder[t] < (int32_t)EBO_CODER_BITPACK || c->table_coder[t] > (int32_t)EBO_CODER_AUTO)
        return 0;
  if (c->sched_kind == EBO_SCHED_INV_SQRT && !(c->sched_t0 > 0.0)) return 0;
  if (c->sched_kind == EBO_SCHED_STEP && (c->sched_phase < 1 || c->sched_steps < 1))
    return 0;
  for (uint32_t p = 0; p < c->P; p++) {
    uint32_t rows = chunk_rows(c, p);
    uint32_t nt = (rows + 63) / 64;
    uint64_t worst = seg_prefix_bytes(nt) + (uint64_t)nt * 16 + (uint64_t)4 * rows * c->D +
                     (uint64_t)nt * 16 + EBO_BOOK_PAD;
    if (worst >= ((uint64_t)1 << 31)) return 0;
  }
  return 1;
}

size_t ebo_max_compressed_bytes(const ebo_cfg* c) {
  if (!cfg_ok(c)) return 0;
  uint64_t total = 64 + align_up((uint64_t)8 * c->P, 16);
  int huff = c->coder == EBO_CODER_HUFFMAN || c->coder == EBO_CODER_AUTO;
  if (c->table_coder) {
    huff = 0;
    for (uint32_t t = 0; t < c->T; t++) huff |= c->table_coder[t] != (int32_t)EBO_CODER_BITPACK;
  }
  for (uint32_t p = 0; p < c->P; p++) {
    uint32_t rows = chunk_rows(c, p);
    uint32_t nt = (rows + 63) / 64;
    /* a Huffman segment may carry a codebook on top of all-RAW records */
    uint64_t seg = seg_prefix_bytes(nt) + (huff ? EBO_BOOK_PAD : 0);
    for (uint32_t k = 0; k < nt; k++) {
      uint32_t n = rows - 64 * k < 64 ? rows - 64 * k : 64;
      seg += raw_record_bytes(n, c->D);
    }
    total += align_up((uint64_t)8 * c->T, 16) + (uint64_t)c->T * seg;
  }
  return (size_t)total;
}

/* ------------------------------------------------------------------ */
/* vector deduplication (section III-B obs. 2, III-D vector-based LZ)  */
/* ------------------------------------------------------------------ */
/* key of one element: (0, q) for a quantized value, (1, raw bits) for an
   outlier, so rows that share a key reconstruct to identical vectors */
static uint64_t elem_key(int32_t q, int outlier, float x) {
  if (outlier) return ((uint64_t)1 << 32) | f32_bits(x);
  return (uint64_t)(uint32_t)q;
}

static const uint64_t* g_sort_keys; /* qsort has no context argument */
static uint32_t g_sort_D;

static int cmp_rows(const void* a, const void* b) {
  uint32_t ra = *(const uint32_t*)a, rb = *(const uint32_t*)b;
  const uint64_t* ka = g_sort_keys + (size_t)ra * g_sort_D;
  const uint64_t* kb = g_sort_keys + (size_t)rb * g_sort_D;
  for (uint32_t d = 0; d < g_sort_D; d++) {
    if (ka[d] < kb[d]) return -1;
    if (ka[d] > kb[d]) return 1;
  }
  return ra < rb ? -1 : (ra > rb ? 1 : 0);
}

/* first[r] = smallest row r' with key(r') == key(r): sort rows by (key, row)
   and give every row of an equal-key run the run's first row. */
static int dedup_first(const uint64_t* keys, uint32_t rows, uint32_t D, uint32_t* first) {
  if (rows == 0) return 0;
  uint32_t* order = (uint32_t*)malloc(sizeof(uint32_t) * rows);
  if (!order) return -1;
  for (uint32_t r = 0; r < rows; r++) order[r] = r;
  g_sort_keys = keys;
  g_sort_D = D;
  qsort(order, rows, sizeof(uint32_t), cmp_rows);
  uint32_t head = order[0];
  first[head] = head;
  for (uint32_t i = 1; i < rows; i++) {
    uint32_t r = order[i];
    if (memcmp(keys + (size_t)r * D, keys + (size_t)head * D, sizeof(uint64_t) * D) != 0)
      head = r;
    first[r] = head;
  }
  free(order);
  return 0;
}

/* The window of section III-E ("Compressor Fine-tuning"): the vector-based
   LZ of section III-D looks back at most W rows for a row with the same key
   (the pattern length is one row, so rows are compared whole).  match[r] =
   the nearest earlier row within W rows with r's key, or r itself when
   there is none.  Sorting rows by (key, row) puts each row right after the
   nearest earlier row with its key. */
static int window_match(const uint64_t* keys, uint32_t rows, uint32_t D, uint32_t W,
                        uint32_t* match) {
  if (rows == 0) return 0;
  uint32_t* order = (uint32_t*)malloc(sizeof(uint32_t) * rows);
  if (!order) return -1;
  for (uint32_t r = 0; r < rows; r++) order[r] = r;
  g_sort_keys = keys;
  g_sort_D = D;
  qsort(order, rows, sizeof(uint32_t), cmp_rows);
  match[order[0]] = order[0];
  for (uint32_t i = 1; i < rows; i++) {
    uint32_t r = order[i], prev = order[i - 1];
    int same = memcmp(keys + (size_t)r * D, keys + (size_t)prev * D, sizeof(uint64_t) * D) == 0;
    match[r] = (same && r - prev <= W) ? prev : r;
  }
  free(order);
  return 0;
}

static uint32_t count_first(const uint32_t* first, uint32_t rows) {
  uint32_t n = 0;
  for (uint32_t r = 0; r < rows; r++) n += first[r] == r;
  return n;
}

/* eq. (1)'s counts: distinct original rows and distinct quantized rows of
   every segment, each found as the first occurrences of a sort by key */
int ebo_homo_counts(const ebo_cfg* c, int64_t iter, const float* x, uint32_t* n_orig,
                    uint32_t* n_quant) {
  if (!cfg_ok(c) || !n_orig || !n_quant || (!x && c->B > 0)) return EBO_ERR_INVALID;
  uint32_t T = c->T, B = c->B, D = c->D, P = c->P;
  int rc = EBO_OK;
  for (uint32_t t = 0; t < T && rc == EBO_OK; t++) {
    float eb = ebo_table_eb(c, t, iter, x);
    int valid = ebo_eb_valid(eb);
    for (uint32_t p = 0; p < P && rc == EBO_OK; p++) {
      uint32_t row0 = chunk_row0(c, p), rows = chunk_rows(c, p);
      size_t nel = (size_t)rows * D;
      const float* xs = x ? x + ((size_t)t * B + row0) * D : NULL;
      uint64_t* keys = (uint64_t*)calloc(nel + 1, sizeof(uint64_t));
      uint32_t* first = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)rows + 1));
      if (!keys || !first) {
        rc = EBO_ERR_OOM;
      } else {
        for (size_t i = 0; i < nel; i++) keys[i] = f32_bits(xs[i]);
        if (dedup_first(keys, rows, D, first) != 0) rc = EBO_ERR_OOM;
        uint32_t no = count_first(first, rows), nq = no;
        if (rc == EBO_OK && valid) {
          for (size_t i = 0; i < nel; i++) {
            int32_t q;
            int o = ebo_quantize(xs[i], eb, &q);
            keys[i] = elem_key(q, o, xs[i]);
          }
          if (dedup_first(keys, rows, D, first) != 0) rc = EBO_ERR_OOM;
          nq = count_first(first, rows);
        }
        n_orig[(size_t)p * T + t] = no;
        n_quant[(size_t)p * T + t] = nq;
      }
      free(keys);
      free(first);
    }
  }
  return rc;
}

double ebo_speedup(double cr, double bw, double tc, double td) {
  /* the time per uncompressed byte with compression (sending cr times fewer
     bytes, compressing and decompressing every byte) against without */
  return 1.0 / (1.0 / cr + bw * (1.0 / tc + 1.0 / td));
}

int ebo_select(uint32_t T, uint32_t ncomp, const double* cr, const double* tc, const double* td,
               double bw, int32_t* best, double* sp) {
  if (ncomp == 0 || !cr || !tc || !td || !best || !(bw > 0.0) || !isfinite(bw)) return -1;
  for (uint32_t c = 0; c < ncomp; c++) {
    if (!(tc[c] > 0.0) || !(td[c] > 0.0) || !isfinite(tc[c]) || !isfinite(td[c])) return -1;
    for (uint32_t t = 0; t < T; t++)
      if (!(cr[(size_t)c * T + t] > 0.0) || !isfinite(cr[(size_t)c * T + t])) return -1;
  }
  for (uint32_t t = 0; t < T; t++) {
    int32_t b = 0;
    double v = ebo_speedup(cr[t], bw, tc[0], td[0]);
    for (uint32_t c = 1; c < ncomp; c++) {
      double w = ebo_speedup(cr[(size_t)c * T + t], bw, tc[c], td[c]);
      if (w > v) {
        v = w;
        b = (int32_t)c;
      }
    }
    best[t] = b;
    if (sp) sp[t] = v;
  }
  return 0;
}

int ebo_classify(uint32_t T, const double* hindex, double l_thresh, double s_thresh,
                 double alpha, double beta, int32_t* cls, float* mult) {
  if (!hindex || !cls || !mult || !(l_thresh <= s_thresh)) return -1;
  if (!(alpha > 0.0) || !isfinite(alpha) || !(beta > 0.0) || !isfinite(beta)) return -1;
  for (uint32_t t = 0; t < T; t++) {
    if (hindex[t] > s_thresh) { /* strongly homogenized: small error bound */
      cls[t] = 2;
      mult[t] = (float)(1.0 / beta);
    } else if (hindex[t] < l_thresh) { /* weakly homogenized: large error bound */
      cls[t] = 0;
      mult[t] = (float)alpha;
    } else {
      cls[t] = 1;
      mult[t] = 1.0f;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* growable byte buffer                                                */
/* ------------------------------------------------------------------ */
typedef struct {
  uint8_t* p;
  size_t n, cap;
  int err;
} buf_t;

static uint8_t* buf_grow(buf_t* b, size_t extra) {
  if (b->err) return NULL;
  if (b->n + extra > b->cap) {
    size_t nc = b->cap ? b->cap : 256;
    while (nc < b->n + extra) nc *= 2;
    uint8_t* np = (uint8_t*)realloc(b->p, nc);
    if (!np) {
      b->err = 1;
      return NULL;
    }
    b->p = np;
    b->cap = nc;
  }
  uint8_t* at = b->p + b->n;
  memset(at, 0, extra);
  b->n += extra;
  return at;
}

/* ------------------------------------------------------------------ */
/* tile record encoder                                                 */
/* ------------------------------------------------------------------ */
typedef struct {
  uint32_t D, rows;         /* dim, rows in the segment */
  int valid;                /* eb valid */
  const float* x;           /* segment rows, row-major */
  const int32_t* q;         /* codes (0 for outliers) */
  const uint8_t* out;       /* outlier flags */
  const uint32_t* first;    /* first occurrence (windowed: match) per row */
  uint32_t window;          /* 0, or W of a windowed segment */
} seg_view;

/* bytes of one reference: a u8 distance in windowed segments, else the
   row as u16 or u32 */
static uint32_t ref_bytes(uint32_t rows, uint32_t window) {
  return window ? 1u : (rows <= 65536 ? 2u : 4u);
}
static void put_ref(uint8_t* at, uint32_t rb, uint32_t row, uint32_t target) {
  if (rb == 1) put_u8(at, (uint8_t)(row - target));
  else if (rb == 2) put_u16(at, (uint16_t)target);
  else put_u32(at, target);
}

/* Huffman-coded record of tile k (mode 2), when the segment's coder is the
   entropy coder of section III-D with code lengths hlen / codes hcode:
     header 16 | refs | outlier positions and raw bits (as in mode 1) |
     chunk table (nch + 1) x u32 word offsets | words, u32 | zero pad to 16
   with E's symbols q + 2047 (outliers as q = 0) in 256-symbol chunks.
   Returns the record bytes (0 on allocation failure); writes the record at
   out when out != NULL. */
static uint64_t huff_record(const seg_view* sv, uint32_t k, uint64_t bitmap, uint32_t U,
                            const uint8_t* hlen, const uint32_t* hcode, uint8_t* out,
                            uint32_t* nout_ret) {
  uint32_t D = sv->D, r0 = 64 * k;
  uint32_t n = sv->rows - r0 < 64 ? sv->rows - r0 : 64;
  uint32_t nE = U * D, nch = (nE + EBO_HUFF_CHUNK - 1) / EBO_HUFF_CHUNK;
  uint16_t* sym = (uint16_t*)malloc(sizeof(uint16_t) * ((size_t)nE + 1));
  uint32_t* opos = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)nE + 1));
  uint32_t* oval = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)nE + 1));
  uint32_t* words = (uint32_t*)calloc((size_t)EBO_HUFF_MAXLEN * nE / 32 + nch + 2, 4);
  uint32_t* coff = (uint32_t*)calloc((size_t)nch + 1, 4);
  uint64_t size = 0;
  if (sym && opos && oval && words && coff) {
    uint32_t nout = 0, e = 0;
    for (uint32_t i = 0; i < n; i++) {
      if (!((bitmap >> i) & 1u)) continue;
      size_t row = (size_t)(r0 + i) * D;
      for (uint32_t d = 0; d < D; d++, e++) {
        sym[e] = (uint16_t)(sv->q[row + d] + EBO_QMAX);
        if (sv->out[row + d]) {
          opos[nout] = e;
          oval[nout] = f32_bits(sv->x[row + d]);
          nout++;
        }
      }
    }
    size_t nw = ebo_huff_encode(sym, nE, hlen, hcode, words, coff);
    uint32_t rb = ref_bytes(sv->rows, sv->window);
    uint64_t off_opos = align_up(16 + (uint64_t)rb * (n - U), 4);
    uint64_t off_oval = off_opos + 4ull * nout;
    uint64_t off_ct = off_oval + 4ull * nout;
    uint64_t off_w = off_ct + 4ull * (nch + 1);
    size = align_up(off_w + 4ull * nw, 16);
    *nout_ret = nout;
    if (out) {
      put_u64(out + 0, bitmap);
      put_u32(out + 8, nout);
      put_u16(out + 12, (uint16_t)U);
      put_u8(out + 14, 2);
      uint32_t j = 0;
      for (uint32_t i = 0; i < n; i++) {
        if ((bitmap >> i) & 1u) continue;
        put_ref(out + 16 + rb * j, rb, r0 + i, sv->first[r0 + i]);
        j++;
      }
      for (uint32_t o = 0; o < nout; o++) {
        put_u32(out + off_opos + 4 * o, opos[o]);
        put_u32(out + off_oval + 4 * o, oval[o]);
      }
      for (uint32_t c = 0; c <= nch; c++) put_u32(out + off_ct + 4 * c, coff[c]);
      for (size_t w = 0; w < nw; w++) put_u32(out + off_w + 4 * w, words[w]);
    }
  }
  free(sym); free(opos); free(oval); free(words); free(coff);
  return size;
}

/* Append tile k's record to b; returns the n_out of the record (0 if RAW).
   hlen != NULL: the segment is Huffman-coded (records of mode 2 or 0). */
static uint32_t encode_tile(const seg_view* sv, uint32_t k, buf_t* b, uint32_t* u_tile,
                            const uint8_t* hlen, const uint32_t* hcode) {
  uint32_t D = sv->D;
  uint32_t r0 = 64 * k;
  uint32_t n = sv->rows - r0 < 64 ? sv->rows - r0 : 64;
  uint64_t bitmap = 0;
  uint32_t U = 0;
  if (sv->valid) {
    for (uint32_t i = 0; i < n; i++)
      if (sv->first[r0 + i] == r0 + i) {
        bitmap |= (uint64_t)1 << i;
        U++;
      }
  }
  *u_tile = U;
  uint64_t raw_bytes = raw_record_bytes(n, D);

  if (sv->valid && hlen) {
    /* a Huffman record when it is strictly smaller than the RAW record */
    uint32_t nout = 0;
    uint64_t size = huff_record(sv, k, bitmap, U, hlen, hcode, NULL, &nout);
    if (size == 0) {
      b->err = 1;
      return 0;
    }
    if (size < raw_bytes) {
      uint8_t* r = buf_grow(b, (size_t)size);
      if (r) huff_record(sv, k, bitmap, U, hlen, hcode, r, &nout);
      return nout;
    }
  } else if (sv->valid) {
    /* E: the first-occurrence rows' codes, row order, flattened */
    uint32_t nE = U * D;
    uint32_t nblk = (nE + 63) / 64;
    uint32_t* zz = (uint32_t*)calloc((size_t)nblk * 64 + 1, sizeof(uint32_t));
    uint32_t* opos = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)nE + 1));
    uint32_t* oval = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)nE + 1));
    uint8_t* w = (uint8_t*)calloc((size_t)nblk + 1, 1);
    if (!zz || !opos || !oval || !w) {
      free(zz); free(opos); free(oval); free(w);
      b->err = 1;
      return 0;
    }
    uint32_t nout = 0, e = 0;
    for (uint32_t i = 0; i < n; i++) {
      if (!((bitmap >> i) & 1u)) continue;
      size_t row = (size_t)(r0 + i) * D;
      for (uint32_t d = 0; d < D; d++, e++) {
        zz[e] = ebo_zigzag(sv->q[row + d]);
        if (sv->out[row + d]) {
          opos[nout] = e;
          oval[nout] = f32_bits(sv->x[row + d]);
          nout++;
        }
      }
    }
    uint64_t sumw = 0;
    for (uint32_t blk = 0; blk < nblk; blk++) {
      uint32_t m = 0;
      for (uint32_t i = 0; i < 64; i++)
        if (zz[64 * blk + i] > m) m = zz[64 * blk + i];
      uint32_t bits = 0;
      while (m) {
        bits++;
        m >>= 1;
      }
      w[blk] = (uint8_t)bits;
      sumw += bits;
    }
    uint32_t rb = ref_bytes(sv->rows, sv->window);
    uint64_t off_refs = align_up(16 + nblk, 4);
    uint64_t off_opos = align_up(off_refs + (uint64_t)rb * (n - U), 4);
    uint64_t off_oval = off_opos + 4ull * nout;
    uint64_t off_pl = align_up(off_oval + 4ull * nout, 8);
    uint64_t size = align_up(off_pl + 8 * sumw, 16);
    if (size < raw_bytes) {
      uint8_t* r = buf_grow(b, (size_t)size);
      if (r) {
        put_u64(r + 0, bitmap);
        put_u32(r + 8, nout);
        put_u16(r + 12, (uint16_t)U);
        put_u8(r + 14, 1);
        for (uint32_t blk = 0; blk < nblk; blk++) put_u8(r + 16 + blk, w[blk]);
        uint32_t j = 0;
        for (uint32_t i = 0; i < n; i++) {
          if ((bitmap >> i) & 1u) continue;
          put_ref(r + off_refs + rb * j, rb, r0 + i, sv->first[r0 + i]);
          j++;
        }
        for (uint32_t o = 0; o < nout; o++) {
          put_u32(r + off_opos + 4 * o, opos[o]);
          put_u32(r + off_oval + 4 * o, oval[o]);
        }
        uint64_t at = off_pl;
        for (uint32_t blk = 0; blk < nblk; blk++) {
          for (uint32_t bit = 0; bit < w[blk]; bit++) {
            uint64_t word = 0;
            for (uint32_t i = 0; i < 64; i++)
              word |= (uint64_t)((zz[64 * blk + i] >> bit) & 1u) << i;
            put_u64(r + at, word);
            at += 8;
          }
        }
      }
      free(zz); free(opos); free(oval); free(w);
      return nout;
    }
    free(zz); free(opos); free(oval); free(w);
  }
  /* RAW record */
  uint8_t* r = buf_grow(b, (size_t)raw_bytes);
  if (r) {
    put_u64(r + 0, bitmap);
    put_u32(r + 8, 0);
    put_u16(r + 12, (uint16_t)U);
    put_u8(r + 14, 0);
    const float* xs = sv->x + (size_t)r0 * D;
    for (uint64_t i = 0; i < (uint64_t)n * D; i++) put_f32(r + 16 + 4 * i, xs[i]);
  }
  return 0;
}

/* Code lengths of a segment's Huffman code: the histogram of E, the codes
   of every first-occurrence row (outliers as q = 0), as symbols q + 2047. */
static void segment_hist(const seg_view* sv, uint64_t* freq) {
  memset(freq, 0, sizeof(uint64_t) * EBO_HUFF_NSYM);
  for (uint32_t r = 0; r < sv->rows; r++) {
    if (sv->first[r] != r) continue;
    for (uint32_t d = 0; d < sv->D; d++) freq[sv->q[(size_t)r * sv->D + d] + EBO_QMAX]++;
  }
}

/* The code of a Huffman segment: built from its histogram, or with codebook
   reuse the kept code of segment s while it has a length for every symbol
   the segment holds (then kept as it is, else replaced by the new one). */
static void segment_lengths(const ebo_cfg* c, uint32_t s, const seg_view* sv, uint8_t* hlen) {
  uint64_t freq[EBO_HUFF_NSYM];
  segment_hist(sv, freq);
  if (c->book_len) {
    uint8_t* kept = c->book_len + (size_t)s * EBO_HUFF_NSYM;
    int covers = c->book_have[s] != 0;
    for (uint32_t x = 0; covers && x < EBO_HUFF_NSYM; x++) covers = !freq[x] || kept[x];
    if (covers) {
      memcpy(hlen, kept, EBO_HUFF_NSYM);
      return;
    }
    ebo_huff_lengths(freq, hlen);
    memcpy(kept, hlen, EBO_HUFF_NSYM);
    c->book_have[s] = 1;
    return;
  }
  ebo_huff_lengths(freq, hlen);
}

/* One whole segment into b (empty on entry): header, tile directory, the
   codebook when hlen != NULL (flags bit 1), tile records.  0, or -1. */
static int encode_segment(const seg_view* sv, uint32_t nt, float eb, const uint8_t* hlen,
                          buf_t* b) {
  uint32_t hcode[EBO_HUFF_NSYM];
  buf_grow(b, 32);
  buf_grow(b, (size_t)align_up(4ull * nt, 16));
  if (hlen) {
    ebo_huff_codes(hlen, hcode);
    uint8_t book[4 + (EBO_HUFF_NSYM + 1) / 2];
    size_t nb = ebo_huff_book_write(hlen, book);
    uint8_t* at = buf_grow(b, (size_t)align_up(nb, 16));
    if (at) memcpy(at, book, nb);
  }
  uint32_t Useg = 0, nout_seg = 0;
  for (uint32_t k = 0; k < nt; k++) {
    size_t rec = b->n;
    if (!b->err) put_u32(b->p + 32 + 4 * k, (uint32_t)rec);
    uint32_t ut = 0;
    nout_seg += encode_tile(sv, k, b, &ut, hlen, hlen ? hcode : NULL);
    Useg += ut;
  }
  if (b->err) return -1;
  uint8_t* sh = b->p;
  put_u32(sh + 0, sv->rows);
  put_u32(sh + 4, nt);
  put_f32(sh + 8, sv->valid ? eb : 0.0f);
  uint32_t flags = sv->valid ? 1u | (hlen ? 2u : 0u) : 0u;
  if (sv->valid && sv->window) flags |= 4u | (sv->window << 8);
  put_u32(sh + 12, flags);
  put_u32(sh + 16, Useg);
  put_u32(sh + 20, nout_seg);
  put_u64(sh + 24, (uint64_t)b->n);
  return 0;
}

/* ------------------------------------------------------------------ */
/* compressor                                                          */
/* ------------------------------------------------------------------ */
int ebo_compress(const ebo_cfg* c, int64_t iter, const float* x, uint8_t* out, size_t cap,
                 size_t* out_bytes, int32_t* codes, uint8_t* outlier, uint32_t* first_out,
                 float* eb_seg) {
  if (!cfg_ok(c) || !out_bytes || (!x && c->B > 0)) return EBO_ERR_INVALID;
  uint32_t T = c->T, B = c->B, D = c->D, P = c->P;
  for (uint32_t t = 0; t < T; t++) {
    if (c->eb_mode == EBO_EB_ABS && !ebo_eb_valid(c->eb[t])) return EBO_ERR_INVALID;
    if (c->eb_mode == EBO_EB_REL && !(c->eb[t] > 0.0f && isfinite(c->eb[t])))
      return EBO_ERR_INVALID;
    if (c->table_mult && !(c->table_mult[t] > 0.0f && isfinite(c->table_mult[t])))
      return EBO_ERR_INVALID;
  }
  size_t need = ebo_max_compressed_bytes(c);
  if (!out || cap < need) return EBO_ERR_CAPACITY;
  uint32_t coder = c->coder ? c->coder : EBO_CODER_BITPACK;
  if (c->table_coder) { /* the stream's coder from the tables' coders */
    int all1 = 1, all2 = 1;
    for (uint32_t t = 0; t < c->T; t++) {
      all1 &= c->table_coder[t] == (int32_t)EBO_CODER_BITPACK;
      all2 &= c->table_coder[t] == (int32_t)EBO_CODER_HUFFMAN;
    }
    coder = all1 ? EBO_CODER_BITPACK : (all2 ? EBO_CODER_HUFFMAN : EBO_CODER_AUTO);
  }

  float* eb_t = (float*)malloc(sizeof(float) * T);
  if (!eb_t) return EBO_ERR_OOM;
  for (uint32_t t = 0; t < T; t++) eb_t[t] = ebo_table_eb(c, t, iter, x);

  buf_t s = {0};
  uint8_t* h = buf_grow(&s, 64);
  if (h) {
    put_u32(h + 0, EBO_MAGIC);
    put_u16(h + 4, EBO_VERSION);
    put_u16(h + 6, (uint16_t)coder);
    put_u32(h + 8, T);
    put_u32(h + 12, B);
    put_u32(h + 16, D);
    put_u32(h + 20, P);
    put_u32(h + 24, EBO_TILE_ROWS);
    put_u32(h + 28, c->eb_mode);
    put_u64(h + 32, (uint64_t)iter);
    put_u64(h + 40, (uint64_t)4 * T * B * D);
  }
  buf_grow(&s, (size_t)align_up(8ull * P, 16)); /* chunk byte counts, filled below */

  int rc = EBO_OK;
  for (uint32_t p = 0; p < P && rc == EBO_OK; p++) {
    size_t chunk0 = s.n;
    uint32_t row0 = chunk_row0(c, p), rows = chunk_rows(c, p);
    uint32_t nt = (rows + 63) / 64;
    buf_grow(&s, (size_t)align_up(8ull * T, 16)); /* segment offset table */
    for (uint32_t t = 0; t < T && rc == EBO_OK; t++) {
      size_t seg0 = s.n;
      if (!s.err) put_u64(s.p + chunk0 + 8 * t, (uint64_t)(seg0 - chunk0));
      const float* xs = x ? x + ((size_t)t * B + row0) * D : NULL;
      float eb = eb_t[t];
      int valid = ebo_eb_valid(eb);
      size_t nel = (size_t)rows * D;
      int32_t* q = (int32_t*)calloc(nel + 1, sizeof(int32_t));
      uint8_t* o = (uint8_t*)calloc(nel + 1, 1);
      uint64_t* keys = (uint64_t*)calloc(nel + 1, sizeof(uint64_t));
      uint32_t* first = (uint32_t*)malloc(sizeof(uint32_t) * ((size_t)rows + 1));
      if (!q || !o || !keys || !first) {
        rc = EBO_ERR_OOM;
      } else {
        for (uint32_t r = 0; r < rows; r++) first[r] = r;
        if (valid) {
          for (size_t i = 0; i < nel; i++) {
            o[i] = (uint8_t)ebo_quantize(xs[i], eb, &q[i]);
            keys[i] = elem_key(q[i], o[i], xs[i]);
          }
          int e = c->window ? window_match(keys, rows, D, c->window, first)
                            : dedup_first(keys, rows, D, first);
          if (e != 0) rc = EBO_ERR_OOM;
        }
      }
      if (rc == EBO_OK) {
        if (codes) {
          for (size_t i = 0; i < nel; i++) codes[((size_t)t * B + row0) * D + i] = q[i];
        }
        if (outlier) {
          for (size_t i = 0; i < nel; i++) outlier[((size_t)t * B + row0) * D + i] = o[i];
        }
        if (first_out) {
          for (uint32_t r = 0; r < rows; r++) first_out[(size_t)t * B + row0 + r] = first[r];
        }
        if (eb_seg) eb_seg[(size_t)p * T + t] = valid ? eb : 0.0f;

        seg_view sv = {D, rows, valid, xs, q, o, first, c->window};
        /* the bit-plane segment, and with the Huffman coder also the Huffman
           segment; coder 3 keeps the Huffman one when it is strictly smaller */
        buf_t bp = {0}, hf = {0};
        if (encode_segment(&sv, nt, eb, NULL, &bp) != 0) rc = EBO_ERR_OOM;
        int use_huff = 0;
        uint32_t tcoder = c->table_coder ? (uint32_t)c->table_coder[t] : coder;
        if (c->book_len && !(valid && tcoder != EBO_CODER_BITPACK)) c->book_have[p * T + t] = 0;
        if (rc == EBO_OK && valid && tcoder != EBO_CODER_BITPACK) {
          uint8_t hlen[EBO_HUFF_NSYM];
          segment_lengths(c, p * T + t, &sv, hlen);
          if (encode_segment(&sv, nt, eb, hlen, &hf) != 0) rc = EBO_ERR_OOM;
          use_huff = tcoder == EBO_CODER_HUFFMAN || hf.n < bp.n;
        }
        if (rc == EBO_OK) {
          const buf_t* pick = use_huff ? &hf : &bp;
          uint8_t* at = buf_grow(&s, pick->n);
          if (at) memcpy(at, pick->p, pick->n);
        }
        free(bp.p);
        free(hf.p);
      }
      free(q); free(o); free(keys); free(first);
    }
    if (!s.err) put_u64(s.p + 64 + 8 * p, (uint64_t)(s.n - chunk0));
  }
  free(eb_t);
  if (s.err) rc = EBO_ERR_OOM;
  if (rc == EBO_OK) {
    put_u64(s.p + 48, (uint64_t)s.n);
    if (s.n > cap) rc = EBO_ERR_CAPACITY;
    else {
      memcpy(out, s.p, s.n);
      *out_bytes = s.n;
    }
  }
  free(s.p);
  return rc;
}

/* ------------------------------------------------------------------ */
/* decompressor (validates every field it reads)                       */
/* ------------------------------------------------------------------ */
typedef struct {
  const uint8_t* s;   /* segment start */
  uint64_t bytes;     /* segment bytes */
  uint32_t rows, ntiles, D;
  float eb;
  int valid;
  int huff;                       /* Huffman segment (flags bit 1) */
  uint32_t window;                /* W of a windowed segment (flags bit 2), else 0 */
  uint8_t hlen[EBO_HUFF_NSYM];    /* its code lengths */
  uint64_t rec_lo;                /* records start at or after this offset */
  uint16_t** sym;                 /* [ntiles]: decoded E symbols of mode-2 records */
} seg_in;

/* byte offsets inside a record of n rows with U first occurrences */
typedef struct {
  uint64_t refs, opos, oval, ct, words, pl;
  uint32_t nblk, nch;
} rec_lay;
static rec_lay record_layout(uint32_t mode, uint32_t n, uint32_t U, uint32_t nout, uint32_t D,
                             uint32_t rows, uint32_t window) {
  rec_lay L;
  uint64_t nE = (uint64_t)U * D;
  uint32_t rb = ref_bytes(rows, window);
  L.nblk = (uint32_t)((nE + 63) / 64);
  L.nch = (uint32_t)((nE + EBO_HUFF_CHUNK - 1) / EBO_HUFF_CHUNK);
  L.refs = mode == 2 ? 16 : align_up(16 + L.nblk, 4);
  L.opos = align_up(L.refs + (uint64_t)rb * (n - U), 4);
  L.oval = L.opos + 4ull * nout;
  L.ct = L.oval + 4ull * nout;          /* mode 2 */
  L.words = L.ct + 4ull * (L.nch + 1);  /* mode 2 */
  L.pl = align_up(L.oval + 4ull * nout, 8);  /* mode 1 */
  return L;
}

/* locate tile record k of segment g; 0 on success */
static int rec_locate(const seg_in* g, uint32_t k, const uint8_t** rec, uint64_t* avail) {
  uint32_t off = get_u32(g->s + 32 + 4 * (uint64_t)k);
  if (off < g->rec_lo || (off & 15u) || (uint64_t)off + 16 > g->bytes) return -1;
  *rec = g->s + off;
  *avail = g->bytes - off;
  return 0;
}

/* the reference of row i of a coded tile record (not a bitmap row): the row
   it names, or in a windowed segment the distance back */
static uint32_t get_ref(const seg_in* g, const uint8_t* rec, const rec_lay* L, uint64_t bitmap,
                        uint32_t i) {
  uint32_t j = i - popcount64(bitmap & (((uint64_t)1 << i) - 1));
  uint32_t rb = ref_bytes(g->rows, g->window);
  if (rb == 1) return rec[L->refs + j];
  return rb == 2 ? get_u16(rec + L->refs + 2 * j) : get_u32(rec + L->refs + 4 * j);
}

/* In a windowed segment, the row whose key row r has: follow the matches of
   repeated rows of coded tiles back (distances are at least 1, so the chain
   ends) to a literal or a row of a RAW tile.  Records are checked first. */
static uint32_t window_root(const seg_in* g, uint32_t r) {
  for (;;) {
    uint32_t k = r / 64, i = r % 64;
    const uint8_t* rec;
    uint64_t avail;
    if (rec_locate(g, k, &rec, &avail)) return r;
    uint64_t bitmap = get_u64(rec);
    uint32_t mode = rec[14];
    if (mode == 0 || ((bitmap >> i) & 1u)) return r;
    uint32_t n = g->rows - 64 * k < 64 ? g->rows - 64 * k : 64;
    rec_lay L = record_layout(mode, n, get_u16(rec + 12), get_u32(rec + 8), g->D, g->rows,
                              g->window);
    r -= get_ref(g, rec, &L, bitmap, i);
  }
}

/* reconstruct segment row r into y (D floats) as its KEY's values: a coded
   first-occurrence row is decoded, a row of a RAW tile is requantized, and in
   a windowed segment a repeated row takes its chain's root's key.  Used for
   every row that is the target of a reference.  Returns 0 on success. */
static int decode_key_row(const seg_in* g, uint32_t r, float* y) {
  if (g->window) r = window_root(g, r);
  uint32_t D = g->D, k = r / 64, i = r % 64;
  const uint8_t* rec;
  uint64_t avail;
  if (rec_locate(g, k, &rec, &avail)) return -1;
  uint64_t bitmap = get_u64(rec);
  uint32_t n = g->rows - 64 * k < 64 ? g->rows - 64 * k : 64;
  uint32_t nout = get_u32(rec + 8);
  uint32_t U = get_u16(rec + 12);
  uint32_t mode = rec[14];
  /* a reference must name a first occurrence (windowed: any row of a RAW
     tile, whose raw values give its key) */
  if (!((bitmap >> i) & 1u) && !(g->window && mode == 0)) return -1;
  if (mode == 0) {
    if (16 + 4ull * n * D > avail) return -1;
    for (uint32_t d = 0; d < D; d++) {
      float v = get_f32(rec + 16 + 4 * ((uint64_t)i * D + d));
      int32_t q;
      y[d] = ebo_quantize(v, g->eb, &q) ? v : ebo_dequantize(q, g->eb);
    }
    return 0;
  }
  if (mode != 1 && mode != 2) return -1;
  uint32_t u = popcount64(bitmap & (((uint64_t)1 << i) - 1));
  rec_lay L = record_layout(mode, n, U, nout, D, g->rows, g->window);
  if (mode == 2) {
    /* symbols decoded when the record was checked */
    if (!g->sym[k]) return -1;
    for (uint32_t d = 0; d < D; d++)
      y[d] = ebo_dequantize((int32_t)g->sym[k][(uint64_t)u * D + d] - EBO_QMAX, g->eb);
  } else {
    if (L.pl > avail) return -1;
    for (uint32_t d = 0; d < D; d++) {
      uint64_t e = (uint64_t)u * D + d;
      uint64_t blk = e / 64, bit = e % 64;
      uint64_t at = L.pl;
      for (uint64_t j = 0; j < blk; j++) at += 8ull * rec[16 + j];
      uint32_t w = rec[16 + blk];
      if (w > 12 || at + 8ull * w > avail) return -1;
      uint32_t zz = 0;
      for (uint32_t j = 0; j < w; j++)
        zz |= (uint32_t)((get_u64(rec + at + 8 * j) >> bit) & 1u) << j;
      y[d] = ebo_dequantize(ebo_unzigzag(zz), g->eb);
    }
  }
  for (uint32_t o = 0; o < nout; o++) {
    uint32_t pos = get_u32(rec + L.opos + 4 * o);
    if (pos >= (uint64_t)u * D && pos < (uint64_t)u * D + D)
      y[pos - (uint64_t)u * D] = bits_f32(get_u32(rec + L.oval + 4 * o));
  }
  return 0;
}

/* decode the chunks of a mode-2 record into g->sym[k]; 0 on success */
static int huff_record_decode(seg_in* g, uint32_t k, const uint8_t* rec, uint64_t avail,
                              const rec_lay* L, uint64_t nE) {
  if (L->words > avail) return -1;
  uint32_t* ct = (uint32_t*)malloc(4ull * (L->nch + 1));
  if (!ct) return -1;
  for (uint32_t c = 0; c <= L->nch; c++) ct[c] = get_u32(rec + L->ct + 4ull * c);
  uint64_t nw = ct[L->nch];
  int rc = -1;
  if (L->words + 4 * nw <= avail) {
    uint32_t* w = (uint32_t*)malloc(4 * (nw + 1));
    g->sym[k] = (uint16_t*)malloc(2 * (nE + 1));
    if (w && g->sym[k]) {
      for (uint64_t j = 0; j < nw; j++) w[j] = get_u32(rec + L->words + 4 * j);
      rc = ebo_huff_decode(w, (size_t)nw, ct, (size_t)nE, g->hlen, g->sym[k]) == 0 ? 0 : -1;
    }
    free(w);
  }
  free(ct);
  return rc;
}

static int check_record(seg_in* g, uint32_t k) {
  uint32_t D = g->D;
  const uint8_t* rec;
  uint64_t avail;
  if (rec_locate(g, k, &rec, &avail)) return -1;
  uint32_t n = g->rows - 64 * k < 64 ? g->rows - 64 * k : 64;
  uint64_t bitmap = get_u64(rec);
  uint32_t nout = get_u32(rec + 8);
  uint32_t U = get_u16(rec + 12);
  uint32_t mode = rec[14];
  if (rec[15] != 0) return -1;
  if (n < 64 && (bitmap >> n) != 0) return -1;
  if (popcount64(bitmap) != U) return -1;
  if (!g->valid && (bitmap != 0 || mode != 0)) return -1;
  if (mode == 0) {
    if (nout != 0 || 16 + 4ull * n * D > avail) return -1;
    return 0;
  }
  /* bit planes in bit-plane segments, Huffman chunks in Huffman segments */
  if (mode != (g->huff ? 2u : 1u)) return -1;
  uint64_t nE = (uint64_t)U * D;
  if (nout > nE) return -1;
  rec_lay L = record_layout(mode, n, U, nout, D, g->rows, g->window);
  if (mode == 1) {
    if (L.pl > avail) return -1;
    uint64_t sumw = 0;
    for (uint32_t j = 0; j < L.nblk; j++) {
      if (rec[16 + j] > 12) return -1;
      sumw += rec[16 + j];
    }
    if (L.pl + 8 * sumw > avail) return -1;
  } else if (huff_record_decode(g, k, rec, avail, &L, nE)) {
    return -1;
  }
  for (uint32_t i = 0; i < n; i++) {
    if ((bitmap >> i) & 1u) continue;
    uint32_t ref = get_ref(g, rec, &L, bitmap, i);
    if (g->window) { /* a distance 1..W back, inside the segment */
      if (ref < 1 || ref > g->window || ref > 64 * k + i) return -1;
    } else if (ref >= 64 * k + i) {
      return -1; /* must point to an earlier row */
    }
  }
  for (uint32_t o = 0; o < nout; o++) {
    uint32_t pos = get_u32(rec + L.opos + 4 * o);
    if (pos >= nE) return -1;
    if (o > 0 && pos <= get_u32(rec + L.opos + 4 * (o - 1))) return -1;
  }
  return 0;
}

static int decode_segment(seg_in* g, uint32_t U_seg, uint32_t nout_seg, float* y) {
  uint32_t D = g->D;
  uint64_t u_sum = 0, o_sum = 0;
  for (uint32_t k = 0; k < g->ntiles; k++) {
    if (check_record(g, k)) return -1;
    const uint8_t* rec;
    uint64_t avail;
    rec_locate(g, k, &rec, &avail);
    u_sum += get_u16(rec + 12);
    if (rec[14] != 0) o_sum += get_u32(rec + 8);
  }
  if (u_sum != U_seg || o_sum != nout_seg) return -1;
  for (uint32_t k = 0; k < g->ntiles; k++) {
    const uint8_t* rec;
    uint64_t avail;
    rec_locate(g, k, &rec, &avail);
    uint32_t n = g->rows - 64 * k < 64 ? g->rows - 64 * k : 64;
    uint64_t bitmap = get_u64(rec);
    uint32_t U = get_u16(rec + 12);
    uint32_t mode = rec[14];
    rec_lay L = record_layout(mode, n, U, get_u32(rec + 8), D, g->rows, g->window);
    for (uint32_t i = 0; i < n; i++) {
      float* yr = y + (size_t)(64 * k + i) * D;
      if (mode == 0) {
        for (uint32_t d = 0; d < D; d++) yr[d] = get_f32(rec + 16 + 4 * ((uint64_t)i * D + d));
      } else if ((bitmap >> i) & 1u) {
        if (decode_key_row(g, 64 * k + i, yr)) return -1;
      } else {
        uint32_t ref = get_ref(g, rec, &L, bitmap, i);
        if (g->window) ref = 64 * k + i - ref;
        if (decode_key_row(g, ref, yr)) return -1;
      }
    }
  }
  return 0;
}

int ebo_decompress(const uint8_t* s, size_t nbytes, uint32_t T, uint32_t B, uint32_t D,
                   uint32_t P, float* y) {
  if (!s || T < 1 || D < 1 || P < 1) return EBO_ERR_INVALID;
  if (nbytes < 64) return EBO_ERR_CORRUPT;
  uint32_t coder = get_u16(s + 6);
  if (get_u32(s) != EBO_MAGIC || get_u16(s + 4) != EBO_VERSION || coder < EBO_CODER_BITPACK ||
      coder > EBO_CODER_AUTO)
    return EBO_ERR_CORRUPT;
  if (get_u32(s + 8) != T || get_u32(s + 12) != B || get_u32(s + 16) != D ||
      get_u32(s + 20) != P || get_u32(s + 24) != EBO_TILE_ROWS || get_u32(s + 28) > 1)
    return EBO_ERR_CORRUPT;
  if (get_u64(s + 40) != (uint64_t)4 * T * B * D || get_u64(s + 56) != 0) return EBO_ERR_CORRUPT;
  uint64_t total = get_u64(s + 48);
  if (total > nbytes) return EBO_ERR_CORRUPT;
  ebo_cfg shape = {0};
  shape.T = T; shape.B = B; shape.D = D; shape.P = P;
  uint64_t base = 64 + align_up(8ull * P, 16);
  if (base > total) return EBO_ERR_CORRUPT;
  uint64_t at = base;
  int rc = EBO_OK;
  seg_in* g = (seg_in*)malloc(sizeof(seg_in));
  if (!g) return EBO_ERR_OOM;
  for (uint32_t p = 0; p < P && rc == EBO_OK; p++) {
    uint64_t cb = get_u64(s + 64 + 8 * p);
    uint64_t tab = align_up(8ull * T, 16);
    if (cb < tab || cb > total - at) {
      rc = EBO_ERR_CORRUPT;
      break;
    }
    const uint8_t* ch = s + at;
    uint32_t row0 = chunk_row0(&shape, p), rows = chunk_rows(&shape, p);
    uint32_t nt = (rows + 63) / 64;
    for (uint32_t t = 0; t < T && rc == EBO_OK; t++) {
      uint64_t so = get_u64(ch + 8 * t);
      if (so < tab || (so & 15u) || so + 32 > cb) {
        rc = EBO_ERR_CORRUPT;
        break;
      }
      g->s = ch + so;
      g->rows = get_u32(g->s + 0);
      g->ntiles = get_u32(g->s + 4);
      g->eb = get_f32(g->s + 8);
      uint32_t flags = get_u32(g->s + 12);
      g->bytes = get_u64(g->s + 24);
      g->D = D;
      g->sym = NULL;
      /* flags: 0, 1 or 3, or 5 / 7 with the window W (1..255) in bits 8-15 */
      uint32_t fl = flags & 0xFFu, win = (flags >> 8) & 0xFFu;
      int flags_ok = (flags >> 16) == 0 &&
                     ((win == 0 && (fl == 0 || fl == 1 || fl == 3)) ||
                      (win != 0 && (fl == 5 || fl == 7)));
      if (g->rows != rows || g->ntiles != nt || !flags_ok ||
          g->bytes > cb - so || g->bytes < seg_prefix_bytes(nt)) {
        rc = EBO_ERR_CORRUPT;
        break;
      }
      g->valid = (int)(flags & 1u);
      g->huff = (int)((flags >> 1) & 1u);
      g->window = win;
      if (g->valid != ebo_eb_valid(g->eb) || (g->huff && coder == EBO_CODER_BITPACK) ||
          (g->valid && !g->huff && coder == EBO_CODER_HUFFMAN)) {
        rc = EBO_ERR_CORRUPT;
        break;
      }
      g->rec_lo = seg_prefix_bytes(nt);
      if (g->huff) {
        /* the codebook follows the tile directory */
        uint64_t room = g->bytes - g->rec_lo;
        if (ebo_huff_book_read(g->s + g->rec_lo, (size_t)room, g->hlen) != 0) {
          rc = EBO_ERR_CORRUPT;
          break;
        }
        g->rec_lo += align_up(ebo_huff_book_bytes(g->hlen), 16);
        if (g->rec_lo > g->bytes) {
          rc = EBO_ERR_CORRUPT;
          break;
        }
      }
      g->sym = (uint16_t**)calloc((size_t)nt + 1, sizeof(uint16_t*));
      if (!g->sym) {
        rc = EBO_ERR_OOM;
        break;
      }
      if (decode_segment(g, get_u32(g->s + 16), get_u32(g->s + 20),
                         y + ((size_t)t * B + row0) * D))
        rc = EBO_ERR_CORRUPT;
      for (uint32_t k = 0; k < nt; k++) free(g->sym[k]);
      free(g->sym);
    }
    at += cb;
  }
  free(g);
  if (rc == EBO_OK && at != total) rc = EBO_ERR_CORRUPT;
  return rc;
}
