// ec_internal.h -- argument blocks shared by the host runtime and the gfx950
// kernels.  Not part of the public ABI (include/ec.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ec {

constexpr uint32_t kTileRows = 64;    // rows per tile record (one bitmap word)
constexpr uint32_t kThreads = 256;    // threads per workgroup (4 wave64)
constexpr uint32_t kMagic = 0x434C4245u;
constexpr uint32_t kVersion = 1;
constexpr uint32_t kCoderBitpack = 1;
constexpr uint32_t kCoderHuffman = 2;   // every segment with a valid eb
constexpr uint32_t kCoderAuto = 3;      // per segment, the smaller form
constexpr uint32_t kHuffTable = 4096;   // Huffman alphabet (4095) + 1, per segment
constexpr uint32_t kBookStride = 2052;  // largest codebook (4 + 4095/2 rounded up)
constexpr uint32_t kBookPad = 2064;     // its size padded to 16
constexpr uint32_t kWinMaxRows = 32768; // rows of a segment with windowed references (decode LDS)

// Error codes the device stores into the host-visible status word.
constexpr uint32_t kDevErrCorrupt = 3;
constexpr uint32_t kDevErrTimeout = 4;

// Host-visible report block (pinned, device-mapped host memory).
struct Report {
  uint64_t total_bytes;
  uint32_t status;
  uint32_t seq;  // the number of the last call that has finished (stored by its last launch)
  uint64_t seg_bytes[1];  // [nseg], allocated past the struct
};

struct Shape {
  uint32_t T, B, D, P;
  uint32_t nseg;         // P * T
  uint32_t ntiles;       // scheduled tiles: sum over segments of max(ceil(rows/64), 1)
  uint64_t base_bytes;   // stream header + chunk byte counts
  uint32_t tiles_per_seg;  // scheduled tiles of every segment when all are equal, else 0
};

// Workspace pointers.  "Constant" arrays are written once at plan time; the
// dynamic region [dyn, dyn + dyn_words) is zeroed by the prep kernel of every
// compress call for D other than 64, 128, 256, and of a plan's first call for
// those (the write pass then leaves the hash tables zero: it clears the slot
// of every first occurrence, the only slots in use; the rest of the region
// is written before it is read).
struct Work {
  const float* eb_base;          // [T]
  const float* mult;             // [T]
  const uint32_t* seg_tile_base; // [nseg + 1] first scheduled tile of each segment
  const uint64_t* hash_off;      // [nseg] first slot of each segment's hash table
  const uint32_t* hash_log2;     // [nseg] log2 of each segment's slot count
  float* range_part;             // [T][nbr][2] per-workgroup (min, max)
  uint32_t nbr;                  // range workgroups per table
  // dynamic
  uint64_t* dyn;
  uint64_t dyn_words;
  uint64_t* seg_start;           // [nseg] absolute offset + 1 (0: not yet known)
  uint64_t* seg_end;             // [nseg] absolute end offset + 1
  uint64_t* chunk_start;         // [P] absolute offset + 1
  uint32_t* seg_fin;             // [nseg] segment header written
  uint64_t* tile_status;         // [ntiles] the tile's stream item (+ 1 once known, one-pass encoder)
  uint64_t* block_status;        // [ntiles] one-pass encoder, per 64 tiles: (flag << 62) | sum or
                                 // inclusive prefix; size pass, per size workgroup: its item sum
  uint32_t* tile_inserted;       // [ntiles] rows inserted into the hash table
  uint64_t* tile_rec;            // [ntiles] absolute record offset + 1 (record written)
  uint32_t* tile_U;              // [ntiles] first occurrences in the tile
  uint32_t* tile_nout;           // [ntiles] outliers stored by the tile
  uint64_t* hash;                // slots: (hash32 << 32) | (row + 1), 0 = empty
  uint64_t* range_slot;          // [T][range_items] (min, max) of each range item of the quantize
                                 // pass (as ordered keys), 0 until written
  // staging between the quantize and assemble passes (D = 64, 128, 256 only;
  // written by the quantize pass before it is read, never cleared)
  uint64_t* stage_pl;            // [ntiles][64][D/64][12] bit-plane words
  uint8_t* stage_w;              // [ntiles][64][D/64] width | 0x80 if outliers
  uint64_t* stage_om;            // [ntiles][64][D/64] outlier masks (flagged only)
  uint32_t* stage_slot;          // [ntiles][64] hash slot of each row (windowed: its hash)
  // per-tile results of the size pass (D = 64, 128, 256 only; written before
  // they are read)
  uint32_t* tile_info;           // [ntiles][4] U, n_out, plane words, mode | valid << 8
  uint64_t* tile_bitmap;         // [ntiles] first-occurrence rows
  uint32_t* tile_first;          // [ntiles][64] first occurrence of each row (windowed: its
                                 // match); decoding windowed segments: the root of each row
  uint32_t* seg_eb;              // [nseg] stored error bound bits (0: raw segment), from quantize
  // Huffman segments (D = 64, 128, 256 with the Huffman or automatic coder;
  // NULL otherwise)
  uint16_t* stage_sym;           // [ntiles][64][D] symbols q + 2047 of every row (outliers 2047)
  uint32_t* hhist;               // [nseg][4096] histogram of the segment's first-occurrence rows
  uint32_t* henc;                // [nseg][4096] len << 16 | code (also decode scratch)
  uint8_t* hbooks;               // [nseg][kBookStride] codebook bytes (encode: built; decode:
                                 // copied from the stream)
  uint32_t* hstat;               // [4] builder status words
  uint32_t* tile_hsize;          // [ntiles] Huffman record bytes
  uint32_t* seg_coder;           // [nseg] 1: the segment is Huffman-coded
  uint16_t* hlut;                // [nseg][4096] decode tables
  uint32_t* hvalid;              // [nseg] decode table valid
  uint32_t* hhave;               // [nseg] henc / hbooks hold the segment's code from the last
                                 // call (constant region: zero at plan time)
  uint32_t* hskip;               // [nseg] this call keeps that code (no build)
  uint8_t* hdbooks;              // [nseg][kBookStride] decoding: codebooks copied from the stream
  uint32_t* hdenc;               // [nseg][4096] decoding: the table builder's scratch
  const uint32_t* table_coder;   // [T] coder of each table (constant), or NULL: EncArgs::coder
};

struct PrepArgs {
  const float* x;
  Shape sh;
  Work w;
  int rel;    // per-table (min, max) partials
  int clear;  // zero the dynamic region
};

struct EncArgs {
  const float* x;
  uint8_t* out;
  uint64_t out_cap;
  Shape sh;
  Work w;
  uint32_t eb_mode;
  int64_t iter;
  double sched;                  // iteration-wise factor, computed on the host
  uint32_t coder;                // the stream's coder: kCoderBitpack, kCoderHuffman or kCoderAuto
  uint32_t window;               // W of windowed references (1..255), 0: first occurrences
  uint32_t fuse_range;           // the quantize pass finds the tables' ranges itself: range
                                 // items one table ahead of the tiles, in table-major order
  uint32_t tiles_per_table;      // scheduled tiles of each table (all chunks)
  uint32_t range_items;          // range items per table
  uint32_t range_ahead;          // tables whose range items go before the first tile
  uint32_t reuse_books;          // keep each segment's Huffman code while it covers the symbols
  uint64_t hash_keep;            // mask applied to row hashes (tests weaken it)
  Report* report;                // device pointer of the pinned report block
  uint32_t* seg_meta;            // in the report block: [nseg][2] U, eb valid (or NULL)
  uint32_t* seg_norig;           // in the report block: [nseg] distinct raw rows (or NULL)
  int32_t* dbg_codes;
  uint8_t* dbg_outlier;
  uint32_t* dbg_first;
  float* dbg_eb;
};

struct DecArgs {
  const uint8_t* in;
  uint64_t cap;
  float* y;
  Shape sh;
  const uint32_t* seg_tile_base;
  Report* report;
  uint32_t huff;  // the plan decodes Huffman segments (its workspace holds the tables)
  uint32_t window;  // the plan decodes windowed segments (its workspace holds the roots)
  Work w;         // the plan's workspace (Huffman and windowed segments)
};

// LDS bytes of the encode kernel for dimension D.
inline size_t encode_lds_bytes(uint32_t D) {
  size_t codes = ((size_t)2 * kTileRows * D + 15) / 16 * 16;
  size_t fixed = kTileRows * (8 + 4 + 4 + 1) + 16;
  size_t per_blk = (size_t)(D + 4) * (4 + 4 + 1) + 64;
  return codes + fixed + per_blk;
}

// LDS bytes of the decode kernel for dimension D: staged bit planes (at most
// 12 per 64-element block), block offsets, widths and up to 256 outliers.
inline size_t decode_lds_bytes(uint32_t D) {
  size_t planes = 8ull * (12ull * D < 6144 ? 12ull * D : 6144);
  return planes + 4ull * (D + 8) + ((D + 8 + 15) / 16) * 16 + 8ull * 256;
}

hipError_t launch_prep(const PrepArgs& a, uint32_t grid, hipStream_t s);
hipError_t launch_encode(const EncArgs& a, hipStream_t s);
// true when D runs as quantize + assembly (launch_assemble after launch_encode:
// size, place and write kernels)
bool encode_has_assembly(uint32_t D);
hipError_t launch_assemble(const EncArgs& a, hipStream_t s);
// its two kernels one at a time (the Huffman coder's passes run between them)
hipError_t launch_assemble_size(const EncArgs& a, hipStream_t s);
hipError_t launch_assemble_write(const EncArgs& a, hipStream_t s);
hipError_t launch_decode(const DecArgs& a, hipStream_t s);
// Windowed references (D = 64, 128, 256): the nearest earlier row within the
// window with the same key, after the quantize pass (encode), and every
// row's root before the decode kernels (decode).
hipError_t launch_window(const EncArgs& a, hipStream_t s);
hipError_t launch_window_roots(const DecArgs& a, hipStream_t s);
// Huffman segments of the stream (D = 64, 128, 256): after the size pass,
// histograms, codebooks, record sizes, the choice per segment and the tile
// items; after the write pass, the chunk words.
hipError_t launch_huff_encode(const EncArgs& a, hipStream_t s);
hipError_t launch_huff_write(const EncArgs& a, hipStream_t s);
// Decoding: codebooks gathered from the stream and their tables before the
// decode kernel, Huffman tiles and the references of their rows after it.
hipError_t launch_huff_tables(const DecArgs& a, hipStream_t s);
hipError_t launch_huff_decode(const DecArgs& a, hipStream_t s);
// in ec_huffman.hip: the codebook builder and the decode-table builder of the
// Huffman coder, over per-segment arrays
hipError_t launch_seg_books(uint32_t* hist, uint32_t* enc, uint8_t* books, uint32_t* status,
                            const uint32_t* skip, uint32_t nseg, hipStream_t s);
hipError_t launch_seg_luts(const uint8_t* books, const uint32_t* zero_word, uint32_t* enc,
                           uint16_t* lut, uint32_t* valid, uint32_t* status, uint32_t nseg,
                           hipStream_t s);
// Distinct rows of every segment as raw fp32 bit patterns (into empty hash
// tables), summed per segment into a.seg_norig: two kernels.
hipError_t launch_distinct_raw(const EncArgs& a, hipStream_t s);
hipError_t set_encode_lds_limit(size_t bytes);
// Address of the current device's copy of the library's static device scratch
// (EC_STATIC_SCRATCH_BYTES, include/ec.h), looked up once per device.
hipError_t static_scratch(void** out);
// Copy `bytes` (a multiple of 16) from src (device memory or device-mapped
// pinned host memory) to dst on stream s, with a kernel.
hipError_t launch_copy_words(void* dst, const void* src, uint64_t bytes, hipStream_t s);
// one wave that stores `seq` into the report once every earlier launch on s has finished
hipError_t launch_done(Report* r, uint32_t seq, hipStream_t s);

}  // namespace ec
