/*
 * ec.h -- C ABI of the MI355X (gfx950) error-bounded lossy compressor for
 * DLRM embedding traffic.
 *
 * The method is the one of arXiv 2407.04272, "Accelerating Communication in
 * Deep Learning Recommendation Model Training with Dual-Level Adaptive Lossy
 * Compression":
 *   - section I and III-D: an error-bounded lossy compressor applied to the
 *     embedding lookups (forward) and their gradients (backward) just before
 *     and after the all-to-all; every reconstructed element x^ satisfies
 *     |x - x^| <= eb for the error bound eb of its table;
 *   - section III-D: a quantization encoder (q = round(x / 2eb)) followed by
 *     a lossless encoder; repeated (homogenized) embedding vectors are
 *     stored once (the vector-based LZ idea) and the codes of the remaining
 *     vectors are bit-plane packed per 64-element block;
 *   - section III-C / Algorithm 1: the eb of table t at iteration i is the
 *     configured table eb (optionally scaled by the table's value range and by
 *     a per-table class multiplier) times an iteration-wise decay factor;
 *   - section III-A stages 1-4 and III-E "Buffer Optimization" (Fig. 7): all
 *     tables of all destination chunks are written by one pass into ONE
 *     contiguous stream; chunk p's bytes are one slice whose size is in the
 *     stream header (the metadata of the variable-size all-to-all).
 *
 * Conventions
 *   - Input x is fp32 [T][B][D], row-major, in device memory.  Chunk p holds
 *     rows [floor(p*B/P), floor((p+1)*B/P)) of every table; a (chunk, table)
 *     pair is a "segment", the unit that repeated rows are detected in.
 *   - Device pointers (d_*) must be 16-byte aligned and stay valid until the
 *     work enqueued on `stream` has finished.  `stream` is a hipStream_t
 *     passed as void*; NULL means the default stream.
 *   - The caller owns every device buffer (input, stream buffer, output,
 *     workspace).  The plan owns only host memory (a copy of the descriptor
 *     and a small pinned host block the device reports sizes into).
 *   - ec_compress / ec_decompress enqueue kernels and return; they never
 *     allocate, free or synchronize.  One plan serves one stream and one host
 *     thread at a time (its calls share the workspace, the report and the
 *     count of calls that ec_ratio waits for); separate plans are
 *     independent.
 *   - Every entry point returns ec_status; nothing is printed and no C++
 *     exception crosses the ABI.  Argument errors are detected on the host
 *     before anything is enqueued.  Conditions found on the device (corrupt
 *     stream, internal time-out) are sticky and returned by ec_ratio.
 */
#ifndef EC_H
#define EC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EC_ABI_VERSION 2u

typedef struct ec_plan_s* ec_plan_t;

typedef enum {
  EC_OK = 0,
  EC_ERR_INVALID = 1,     /* bad argument or descriptor                      */
  EC_ERR_CAPACITY = 2,    /* output or workspace smaller than required       */
  EC_ERR_CORRUPT = 3,     /* stream failed validation on the device          */
  EC_ERR_DEVICE = 4,      /* HIP error or device-side time-out               */
  EC_ERR_OOM = 5,         /* host allocation failed                          */
  EC_ERR_UNSUPPORTED = 6  /* shape beyond the library's limits (e.g. D > max) */
} ec_status;

typedef enum {
  EC_EB_ABS = 0,       /* eb[t] is the absolute error bound                  */
  EC_EB_REL_RANGE = 1  /* eb_t = eb[t] * (max - min) of this call's table t  */
} ec_eb_mode;

typedef enum {
  EC_SCHED_NONE = 0,     /* factor 1                                         */
  EC_SCHED_INV_SQRT = 1, /* (1 + i/t0)^(-1/2)                                */
  EC_SCHED_STEP = 2      /* k - (k-1) * floor(steps*min(i,phase)/phase)/steps:
                            staircase from k down to 1 (the pages' default
                            step-wise decay, section III-C; Fig. 10's
                            Decay_2x is k = 2, and its Drop_2x, k held for
                            the whole initial phase then 1, is steps = 1)  */
} ec_sched_kind;

/* The lossless stage after quantization and repeated-row detection (section
 * III-D: "a hybrid method" of the vector-based LZ and an entropy encoder such
 * as Huffman, chosen per table, section III-D "Selection Between Two
 * Encoders").  BITPACK: every segment's codes as bit planes per 64-element
 * block.  HUFFMAN: every segment with a valid eb Huffman-coded (a canonical
 * code per segment, built from the histogram of its first-occurrence rows;
 * ec_huffman.h states the code's rules).  AUTO: per segment, the Huffman form
 * when it is strictly smaller.  HUFFMAN and AUTO need D = 64, 128 or 256 and a
 * plan with a workspace; a BITPACK plan decodes bit-plane streams only. */
typedef enum { EC_CODER_BITPACK = 1, EC_CODER_HUFFMAN = 2, EC_CODER_AUTO = 3 } ec_coder;

/* Kernel ids for the profiling counters.  PREP is the value-range pass (and
 * the clearing of the per-call workspace).  For D = 64, 128 and 256,
 * compression runs ENCODE (quantize, bit planes, hash insertion) then ASSEMBLE
 * (first occurrences and record sizes, then placement and record writing: two
 * kernels timed together); DECODE checks and locates each record and decodes
 * it in one kernel.  For other D, ENCODE and DECODE are single kernels and
 * ASSEMBLE stays unused. */
typedef enum {
  EC_KERNEL_PREP = 0,
  EC_KERNEL_ENCODE = 1,
  EC_KERNEL_DECODE = 2,
  EC_KERNEL_ASSEMBLE = 3
} ec_kernel;

typedef struct {
  int32_t kind;   /* ec_sched_kind                  */
  int32_t steps;  /* STEP: number of stairs (>= 1)  */
  double t0;      /* INV_SQRT: > 0                  */
  double k;       /* STEP: starting multiple (>= 1) */
  int64_t phase;  /* STEP: decay-phase length (>= 1) */
} ec_schedule;

typedef struct {
  uint32_t abi_version;     /* EC_ABI_VERSION                                  */
  uint32_t num_tables;      /* T >= 1                                          */
  uint32_t rows;            /* B >= 0 rows per table                           */
  uint32_t dim;             /* 1 <= D <= ec_max_dim()                          */
  uint32_t num_chunks;      /* P >= 1 destination chunks                       */
  int32_t eb_mode;          /* ec_eb_mode                                      */
  const float* eb;          /* host [T]; ABS: finite > 0 with 2*eb finite;
                               REL: finite > 0.  Copied by ec_plan.            */
  const float* table_mult;  /* host [T] finite > 0 class multipliers (the
                               large/medium/small table classes of Algorithm 1)
                               or NULL for 1.  Copied by ec_plan.             */
  ec_schedule sched;        /* iteration-wise decay                            */
  int32_t coder;            /* ec_coder                                        */
  uint32_t debug_hash_bits; /* 0: normal.  1..32: keep only that many bits of
                               the internal row hash (forces hash collisions;
                               output bytes are unchanged).  Tests only.       */
  void* d_workspace;        /* device, >= ec_workspace_bytes(desc) bytes, 256-B
                               aligned; owned by the caller, used by the plan
                               until ec_plan_destroy                           */
  size_t workspace_bytes;
  uint32_t window;          /* 0: a repeated row references the first row of
                               its segment with its key; 1..255: the nearest
                               earlier row within `window` rows (the vector-
                               based LZ of section III-D with the extended
                               window of section III-E, Table VI), stored as a
                               u8 distance.  Needs D = 64, 128 or 256, a
                               workspace and at most 32768 rows per segment
                               (else EC_ERR_UNSUPPORTED); decoding windowed
                               segments needs a windowed plan.                */
  uint32_t reuse_books;     /* nonzero: a segment that may be Huffman-coded
                               keeps its code from the plan's previous call
                               while that code has a length for every symbol
                               it holds, else builds one and keeps it (value
                               distributions are stable over training,
                               section IV, Fig. 14).  Calls of one plan then
                               depend on its previous compress call; the
                               static-scratch entry point never reuses.       */
  const int32_t* table_coder; /* host [T] ec_coder of each table (Algorithm 2's
                               table-wise configuration, e.g. from
                               ec_select_coders) or NULL for `coder`; copied
                               by ec_plan.  The stream's coder field is then
                               BITPACK, HUFFMAN or AUTO as the tables' coders
                               are all bit planes, all Huffman, or mixed.     */
} ec_plan_desc;

/* Largest supported D on the current device (limited by LDS per workgroup). */
uint32_t ec_max_dim(void);

/* Workspace bytes the plan needs (0 if the descriptor is invalid).  The
 * workspace holds the per-table error bounds (section III-C), the hash tables
 * of the repeated-vector detection (section III-D "Vector-based LZ
 * Encoding") and the staging between the compression passes. */
size_t ec_workspace_bytes(const ec_plan_desc* desc);

/* Validate the descriptor and build a plan: the shape, the per-table error
 * bounds with their class multipliers and the iteration-wise schedule of
 * section III-C / Algorithm 1 (table-wise and iteration-wise levels).  Host
 * work plus one blocking copy of the per-table constants into the workspace.
 * d_workspace == NULL together with workspace_bytes == 0 builds a plan without
 * a workspace, usable with ec_compress_static, ec_decompress and ec_ratio
 * only (ec_compress then returns EC_ERR_INVALID).  *out is NULL on failure. */
ec_status ec_plan(const ec_plan_desc* desc, ec_plan_t* out);

/* Wait for the plan's last enqueued call, then release the plan's host
 * resources (the workspace stays the caller's). */
ec_status ec_plan_destroy(ec_plan_t plan);

/* Upper bound of a compressed stream (every tile stored raw); 0 for NULL.
 * Sizes the send buffer that section III-E "Buffer Optimization" writes the
 * whole multi-table stream into. */
size_t ec_max_compressed_bytes(ec_plan_t plan);

/* Compress d_in (fp32 [T][B][D]) at iteration `iter` into d_out (capacity
 * out_cap >= ec_max_compressed_bytes): the lossy compressor of sections I and
 * III-D (quantization encoder q = round(x / 2eb) with every reconstructed value
 * within eb, repeated vectors stored once, the codes bit-plane packed), all
 * tables of all destination chunks into ONE contiguous stream (section III-E,
 * Fig. 7).  The stream's size becomes known on the host through ec_ratio; on
 * the device it is the u64 at byte 48 of d_out, and chunk p's size is the u64
 * at byte 64 + 8p (the size metadata of section III-A, stage 2).  Errors:
 * EC_ERR_INVALID (NULL or misaligned pointers, a plan without a workspace),
 * EC_ERR_CAPACITY (out_cap too small), EC_ERR_DEVICE (a launch failed). */
ec_status ec_compress(ec_plan_t plan, int64_t iter, const float* d_in, void* d_out,
                      size_t out_cap, void* stream);

/* Decompress a stream of this plan's shape (d_stream holds stream_cap readable
 * bytes) into d_out (fp32 [T][B][D]): the inverse path of section III-A stage
 * 4 (the receiver decodes each source's slice; every row is written once).
 * Every field is validated on the device before use; a corrupt stream makes
 * ec_ratio return EC_ERR_CORRUPT and leaves the affected rows zero. */
ec_status ec_decompress(ec_plan_t plan, const void* d_stream, size_t stream_cap, float* d_out,
                        void* stream);

/* Wait for this plan's last enqueued call (its last launch stores the call's
 * number into the plan's pinned report; after 200 ms without it the whole
 * device is waited for), then report the last compression:
 * total_cr = 4*T*B*D / stream bytes (headers included), the stream bytes, and
 * per_segment_cr[p*T + t] = 4*rows(p)*D / segment bytes (may be NULL).  The
 * total is a ratio of total bytes, which is what Table V's "avg." row
 * averages (its values are harmonic means of the per-table ratios).  Returns
 * and clears the sticky device status. */
ec_status ec_ratio(ec_plan_t plan, double* total_cr, uint64_t* compressed_bytes,
                   double* per_segment_cr);

/* Offline analysis of section III-C (Algorithm 1, "OfflineAnalysis"), run on
 * a sampled batch: compresses d_in exactly as ec_compress does (the stream
 * lands in d_out), then counts for every segment s = p*T + t the numbers that
 * eq. (1) takes: n_orig[s] = distinct rows of the segment as fp32 bit patterns
 * (Tables III/IV "# Ori. Patterns") and n_quant[s] = distinct quantized rows
 * (the repeated-row key, "# Quant. Patterns"; n_orig[s] when the segment's eb
 * is invalid and nothing is quantized).  The Homogenization Index is then
 * (n_orig - n_quant) / n_orig.  Host arrays of P*T entries; the call waits for
 * the device.  Errors: those of ec_compress, EC_ERR_INVALID for NULL arrays,
 * EC_ERR_DEVICE for a device-side failure. */
ec_status ec_homo_counts(ec_plan_t plan, int64_t iter, const float* d_in, void* d_out,
                         size_t out_cap, uint32_t* n_orig, uint32_t* n_quant, void* stream);

typedef enum { EC_CLASS_LARGE = 0, EC_CLASS_MEDIUM = 1, EC_CLASS_SMALL = 2 } ec_table_class;

/* Algorithm 1, EMBClassification: table t is small-eb (EC_CLASS_SMALL,
 * multiplier 1/beta) when homo_index[t] > s_thresh, large-eb (EC_CLASS_LARGE,
 * multiplier alpha) when homo_index[t] < l_thresh, else medium (multiplier 1);
 * the multipliers (rounded once to fp32) go into ec_plan_desc.table_mult, so
 * LargeEB = eb * alpha and SmallEB = eb / beta.  Host only.  EC_ERR_INVALID
 * for NULL arrays, l_thresh > s_thresh, or alpha, beta not finite and > 0. */
ec_status ec_classify_tables(uint32_t num_tables, const double* homo_index, double l_thresh,
                             double s_thresh, double alpha, double beta, int32_t* table_class,
                             float* table_mult);

/* Eq. (2) of section III-D ("Selection Between Two Encoders"): the
 * communication speed-up of a compressor with compression ratio cr and
 * compression / decompression throughputs tc, td over a link of bandwidth bw
 * (all throughputs in one unit): 1 / (1/cr + bw * (1/tc + 1/td)).  Host only. */
double ec_speedup(double cr, double bw, double tc, double td);

/* Algorithm 2 (OfflineCompConfig): for each of num_tables tables, the
 * compressor of a pool of ncomp whose eq. (2) speed-up is largest, from the
 * ratios cr[c * num_tables + t] measured on a sample of the table and the
 * pool's throughputs tc[c], td[c] over bandwidth bw; on equal speed-ups the
 * earlier compressor.  best[t] gets the index, speedup[t] (may be NULL) its
 * speed-up.  Host only.  EC_ERR_INVALID for an empty pool, NULL arrays, or
 * values that are not finite and > 0. */
ec_status ec_select_coders(uint32_t num_tables, uint32_t ncomp, const double* cr, const double* tc,
                           const double* td, double bw, int32_t* best, double* speedup);

/* Bytes of the library's static device scratch (one copy per device). */
#define EC_STATIC_SCRATCH_BYTES (64ull << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): compress
 * exactly as ec_compress does (same stream bytes), but with the library's own
 * static device scratch of EC_STATIC_SCRATCH_BYTES instead of the plan's
 * workspace, so the plan may have none.  Allocates nothing and frees nothing.
 * The scratch is shared by every call on a device and keeps the last call's
 * contents: each call copies the plan's constants in and clears what must
 * start at zero, and calls that overlap on one device (any plan, any stream)
 * race and corrupt each other's streams.  Errors: those of ec_compress, and
 * EC_ERR_CAPACITY when the plan needs more than EC_STATIC_SCRATCH_BYTES
 * (ec_workspace_bytes of its descriptor; e.g. 26 x 8192 x 128 fits, 64 x
 * 16384 x 256 does not). */
ec_status ec_compress_static(ec_plan_t plan, int64_t iter, const float* d_in, void* d_out,
                             size_t out_cap, void* stream);

const char* ec_status_string(ec_status s);

/* Tests only: make subsequent ec_compress calls also write the quantization
 * codes (int32 [T*B*D], 0 for outliers), outlier flags (u8 [T*B*D]), the
 * first-occurrence segment row of every row (u32 [T*B]) and the eb of every
 * segment (f32 [P*T], 0 when invalid).  NULL disables an output. */
ec_status ec_debug_attach(ec_plan_t plan, int32_t* d_codes, uint8_t* d_outlier,
                          uint32_t* d_first, float* d_eb);

/* Profiling: when enabled, every kernel launch of the plan is bracketed by HIP
 * events on the launch stream (at most `max_launches` launches are kept).
 * ec_profile_read waits for them and returns the summed duration and count
 * for one ec_kernel id; ec_profile_enable(plan, 0, 0) clears and disables. */
ec_status ec_profile_enable(ec_plan_t plan, int enable, uint32_t max_launches);
ec_status ec_profile_read(ec_plan_t plan, int kernel, double* total_ms, uint64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* EC_H */
