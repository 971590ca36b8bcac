// ec_runtime.cpp -- host side of the C ABI in include/ec.h: descriptor
// validation, workspace layout, the error-bound policy's iteration factor
// (arXiv 2407.04272, section III-C and Algorithm 1), kernel launches on the
// caller's stream, the pinned report block, and opt-in launch profiling.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "../../include/ec.h"
#include "ec_internal.h"

namespace {

uint64_t aup(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

struct Layout {
  // byte offsets inside the workspace
  uint64_t eb_base, mult, seg_tile_base, hash_off, hash_log2, range_part, table_coder = 0;
  uint32_t stream_coder = 1;  // the header's coder field
  uint64_t dyn, seg_start, seg_end, chunk_start, seg_fin;
  uint64_t tile_status, block_status, tile_inserted, tile_rec, tile_U, tile_nout, hash;
  uint64_t range_slot = 0;
  uint32_t range_items = 1;  // range items per table of the quantize pass (64 KiB of input each)
  uint64_t stage_pl = 0, stage_w = 0, stage_om = 0, stage_slot = 0;
  uint64_t tile_info = 0, tile_bitmap = 0, tile_first = 0, seg_eb = 0;
  uint64_t stage_sym = 0, hhist = 0, henc = 0, hbooks = 0, hstat = 0, tile_hsize = 0;
  uint64_t seg_coder = 0, hlut = 0, hvalid = 0, hhave = 0, hskip = 0, hdbooks = 0, hdenc = 0;
  bool huff = false;  // Huffman segments (coder 2 or 3)
  uint64_t dyn_bytes, total;
  uint32_t nbr;
  std::vector<uint32_t> seg_tile_base_v;
  std::vector<uint64_t> hash_off_v;
  std::vector<uint32_t> hash_log2_v;
  ec::Shape sh;
  uint64_t max_bytes;
};

uint32_t rows_of_chunk(uint32_t B, uint32_t P, uint32_t p) {
  uint64_t a = (uint64_t)p * B / P, b = (uint64_t)(p + 1) * B / P;
  return (uint32_t)(b - a);
}

int g_max_dim = -1;
size_t g_lds_limit = 0;

uint32_t device_max_dim() {
  if (g_max_dim >= 0) return (uint32_t)g_max_dim;
  int dev = 0;
  size_t limit = 65536;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
      limit = (size_t)v;
  }
  g_lds_limit = limit;
  uint32_t d = 1;
  while (d < 4096 && ec::encode_lds_bytes(d + 1) + 512 <= limit) d++;
  g_max_dim = (int)d;
  return d;
}

bool finite_pos(float v) { return std::isfinite(v) && v > 0.0f; }

// Validates the descriptor (host pointers only) and computes the layout.
ec_status make_layout(const ec_plan_desc* d, Layout* L) {
  if (!d || d->abi_version != EC_ABI_VERSION) return EC_ERR_INVALID;
  const uint32_t T = d->num_tables, B = d->rows, D = d->dim, P = d->num_chunks;
  if (T < 1 || D < 1 || P < 1 || !d->eb) return EC_ERR_INVALID;
  if (d->eb_mode != EC_EB_ABS && d->eb_mode != EC_EB_REL_RANGE) return EC_ERR_INVALID;
  auto coder_ok = [](int32_t c) {
    return c == EC_CODER_BITPACK || c == EC_CODER_HUFFMAN || c == EC_CODER_AUTO;
  };
  if (!coder_ok(d->coder)) return EC_ERR_INVALID;
  L->stream_coder = (uint32_t)d->coder;
  if (d->table_coder) {  // per table: the stream's coder follows from them
    bool all1 = true, all2 = true;
    for (uint32_t t = 0; t < T; t++) {
      if (!coder_ok(d->table_coder[t])) return EC_ERR_INVALID;
      all1 = all1 && d->table_coder[t] == EC_CODER_BITPACK;
      all2 = all2 && d->table_coder[t] == EC_CODER_HUFFMAN;
    }
    L->stream_coder = all1 ? EC_CODER_BITPACK : (all2 ? EC_CODER_HUFFMAN : EC_CODER_AUTO);
  }
  L->huff = L->stream_coder != EC_CODER_BITPACK;
  // Huffman segments: for the wave64 paths (D = 64, 128, 256) only
  if (L->huff && !ec::encode_has_assembly(D)) return EC_ERR_UNSUPPORTED;
  // windowed references: W <= 255 (u8 distances), on the wave64 paths, with
  // at most kWinMaxRows rows per segment (the decoder's roots pass)
  if (d->window > 255) return EC_ERR_INVALID;
  if (d->window && (!ec::encode_has_assembly(D) || (B + P - 1) / P > ec::kWinMaxRows))
    return EC_ERR_UNSUPPORTED;
  if (d->debug_hash_bits > 64) return EC_ERR_INVALID;
  const ec_schedule& s = d->sched;
  if (s.kind == EC_SCHED_INV_SQRT) {
    if (!(s.t0 > 0.0) || !std::isfinite(s.t0)) return EC_ERR_INVALID;
  } else if (s.kind == EC_SCHED_STEP) {
    if (s.phase < 1 || s.steps < 1 || !(s.k >= 1.0) || !std::isfinite(s.k)) return EC_ERR_INVALID;
  } else if (s.kind != EC_SCHED_NONE) {
    return EC_ERR_INVALID;
  }
  for (uint32_t t = 0; t < T; t++) {
    float e = d->eb[t];
    if (d->eb_mode == EC_EB_ABS) {
      if (!finite_pos(e) || !std::isfinite(e + e)) return EC_ERR_INVALID;
    } else if (!finite_pos(e)) {
      return EC_ERR_INVALID;
    }
    if (d->table_mult && !finite_pos(d->table_mult[t])) return EC_ERR_INVALID;
  }
  if (D > device_max_dim()) return EC_ERR_UNSUPPORTED;
  if ((uint64_t)T * B * D >= (1ull << 40)) return EC_ERR_UNSUPPORTED;

  const uint64_t nseg = (uint64_t)P * T;
  L->seg_tile_base_v.assign(nseg + 1, 0);
  L->hash_off_v.assign(nseg, 0);
  L->hash_log2_v.assign(nseg, 0);
  uint64_t tiles = 0, slots = 0, maxb = 64 + aup(8ull * P, 16);
  for (uint32_t p = 0; p < P; p++) {
    const uint32_t rows = rows_of_chunk(B, P, p);
    const uint32_t nt = (rows + 63) / 64;
    // per-segment stream size must fit the u32 tile directory
    uint64_t seg_max = 32 + aup(4ull * nt, 16) + 16ull * nt + 4ull * rows * D + 16ull * nt;
    if (seg_max >= (1ull << 31)) return EC_ERR_UNSUPPORTED;
    // hash slots: a power of two >= 4 rows, so the table is at most a quarter
    // full and a wave's 16 insertions rarely probe far (at half full the
    // longest of their linear-probing chains set the pace of the quantize pass)
    uint32_t lg = 6;
    while ((1ull << lg) < 4ull * rows) lg++;
    uint64_t seg_bytes = 32 + aup(4ull * nt, 16);
    for (uint32_t k = 0; k < nt; k++) {
      uint32_t n = rows - 64 * k < 64 ? rows - 64 * k : 64;
      seg_bytes += 16 + aup(4ull * n * D, 16);
    }
    // a Huffman segment may carry its codebook on top of all-RAW records
    if (L->huff) seg_bytes += ec::kBookPad;
    if (seg_bytes >= (1ull << 31)) return EC_ERR_UNSUPPORTED;
    maxb += aup(8ull * T, 16) + (uint64_t)T * seg_bytes;
    for (uint32_t t = 0; t < T; t++) {
      uint64_t sidx = (uint64_t)p * T + t;
      L->seg_tile_base_v[sidx] = (uint32_t)tiles;
      L->hash_off_v[sidx] = slots;
      L->hash_log2_v[sidx] = lg;
      tiles += nt ? nt : 1;
      slots += 1ull << lg;
    }
  }
  if (tiles >= (1ull << 31)) return EC_ERR_UNSUPPORTED;
  L->seg_tile_base_v[nseg] = (uint32_t)tiles;
  uint32_t tps = 0;
  for (uint32_t p = 0; p < P; p++) {
    uint32_t rows = rows_of_chunk(B, P, p), nt = (rows + 63) / 64;
    uint32_t v = nt ? nt : 1;
    if (p == 0) tps = v;
    else if (v != tps) tps = 0;
    if (tps == 0) break;
  }
  L->sh = {T, B, D, P, (uint32_t)nseg, (uint32_t)tiles, 64 + aup(8ull * P, 16), tps};
  L->max_bytes = maxb;

  const uint64_t nel = (uint64_t)B * D;
#ifndef EC_PREP_SPAN
#define EC_PREP_SPAN 8192
#endif
  uint64_t nbr = (nel + EC_PREP_SPAN - 1) / EC_PREP_SPAN;  // range workgroups per table
  L->nbr = (uint32_t)(nbr < 1 ? 1 : (nbr > 1024 ? 1024 : nbr));

  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    uint64_t at = aup(o, 256);
    o = at + bytes;
    return at;
  };
  L->eb_base = take(4ull * T);
  L->mult = take(4ull * T);
  L->seg_tile_base = take(4ull * (nseg + 1));
  L->hash_off = take(8ull * nseg);
  L->hash_log2 = take(4ull * nseg);
  if (d->table_coder) L->table_coder = take(4ull * T);
  if (L->huff) L->hhave = take(4ull * nseg);  // constant region: zero at plan time
  L->range_part = take(8ull * T * L->nbr);
  o = aup(o, 256);
  L->dyn = o;
  L->seg_start = take(8ull * nseg);
  L->seg_end = take(8ull * nseg);
  L->chunk_start = take(8ull * P);
  L->seg_fin = take(4ull * nseg);
  L->tile_status = take(8ull * tiles);
  L->block_status = take(8ull * tiles);  // one per block of at least one tile
  L->tile_inserted = take(4ull * tiles);
  L->tile_rec = take(8ull * tiles);
  L->tile_U = take(4ull * tiles);
  L->tile_nout = take(4ull * tiles);
  L->hash = take(8ull * slots);
  {
    const uint64_t items = (4ull * nel + 65535) / 65536;
    L->range_items = (uint32_t)(items < 1 ? 1 : (items > 256 ? 256 : items));
  }
  L->range_slot = take(8ull * T * L->range_items);
  o = aup(o, 256);
  L->dyn_bytes = o - L->dyn;
  if (ec::encode_has_assembly(D)) {
    const uint64_t blocks = tiles * 64ull * (D / 64);
    L->stage_pl = take(8ull * 12 * blocks);
    L->stage_w = take(blocks);
    L->stage_om = take(8ull * blocks);
    L->stage_slot = take(4ull * 64 * tiles);
    L->tile_info = take(16ull * tiles);
    L->tile_bitmap = take(8ull * tiles);
    L->tile_first = take(4ull * 64 * tiles);
    L->seg_eb = take(4ull * nseg);
    if (L->huff) {
      L->stage_sym = take(2ull * 64 * D * tiles);
      L->hhist = take(4ull * ec::kHuffTable * nseg);
      L->henc = take(4ull * ec::kHuffTable * nseg);
      L->hbooks = take((uint64_t)ec::kBookStride * nseg);
      L->hstat = take(16);
      L->tile_hsize = take(4ull * tiles);
      L->seg_coder = take(4ull * nseg);
      L->hlut = take(2ull * ec::kHuffTable * nseg);
      L->hvalid = take(4ull * nseg);
      L->hskip = take(4ull * nseg);
      L->hdbooks = take((uint64_t)ec::kBookStride * nseg);
      L->hdenc = take(4ull * ec::kHuffTable * nseg);
    }
    o = aup(o, 256);
  }
  L->total = o;
  return EC_OK;
}

// Tables whose range items the quantize pass takes before its first tile: far
// enough ahead that a tile rarely finds its table's range unfinished (on the
// 26-table dim-128 batch, 12 ahead beat 1, 2, 4, 6, 8, 10, 14, 16 and all by
// 0.5-2 us of the launch; the dim-64 batch does not tell them apart).
constexpr uint32_t kRangeAhead = 12;

double schedule_factor(const ec_schedule& s, int64_t iter) {
  int64_t i = iter < 0 ? 0 : iter;
  if (s.kind == EC_SCHED_INV_SQRT) return std::pow(1.0 + (double)i / s.t0, -0.5);
  if (s.kind == EC_SCHED_STEP) {
    int64_t m = i < s.phase ? i : s.phase;
    int64_t stair = (int64_t)s.steps * m / s.phase;
    double drop = ((s.k - 1.0) * (double)stair) / (double)s.steps;
    return s.k - drop;
  }
  return 1.0;
}

struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};

}  // namespace

struct ec_plan_s {
  Layout L;
  ec_plan_desc desc;
  std::vector<float> eb, mult;
  uint8_t* ws = nullptr;
  ec::Work work{};
  ec::Report* report_host = nullptr;
  ec::Report* report_dev = nullptr;
  size_t meta_off = 0, norig_off = 0;  // byte offsets in the report block
  // the workspace's constant region [0, L.dyn) as written at plan time, in
  // pinned device-mapped host memory: copied into the static scratch by every
  // ec_compress_static call, and read by decompression when the plan has no
  // workspace
  uint8_t* consts_host = nullptr;
  uint8_t* consts_dev = nullptr;
  uint32_t seq = 0;         // the number of the last call enqueued outside a graph capture
  bool have_done = false;   // such a call exists
  int32_t* dbg_codes = nullptr;
  uint8_t* dbg_outlier = nullptr;
  uint32_t* dbg_first = nullptr;
  float* dbg_eb = nullptr;
  bool hash_clear = false;  // the hash tables are zero (the last call's write pass cleared them)
  bool prof_on = false;
  std::vector<hipEvent_t> prof_pool;
  std::vector<ProfRec> prof_recs;
  size_t prof_next = 0;
  uint64_t prof_dropped = 0;
};

namespace {

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

template <typename F>
ec_status profiled(ec_plan_s* pl, int kernel, hipStream_t s, F&& launch) {
  hipEvent_t a = nullptr, b = nullptr;
  if (pl->prof_on && pl->prof_next + 2 <= pl->prof_pool.size()) {
    a = pl->prof_pool[pl->prof_next++];
    b = pl->prof_pool[pl->prof_next++];
    if (hipEventRecord(a, s) != hipSuccess) return EC_ERR_DEVICE;
  } else if (pl->prof_on) {
    pl->prof_dropped++;
  }
  if (launch() != hipSuccess) return EC_ERR_DEVICE;
  if (a) {
    if (hipEventRecord(b, s) != hipSuccess) return EC_ERR_DEVICE;
    pl->prof_recs.push_back({kernel, a, b});
  }
  return EC_OK;
}

// The call's completion, marked by its last launch: one wave that stores the
// call's number into the pinned report once the stream reaches it.  (An event
// recorded after every call holds the stream for several microseconds per
// call in its marker packet, several times what this wave costs.)  Not while
// the stream is captured: the number would be fixed in the graph.
ec_status mark_done(ec_plan_s* pl, hipStream_t s) {
  if (capturing(s)) return EC_OK;
  const uint32_t next = pl->seq + 1;
  if (ec::launch_done(pl->report_dev, next, s) != hipSuccess) return EC_ERR_DEVICE;
  pl->seq = next;
  pl->have_done = true;
  return EC_OK;
}

// Wait until the report holds the last marked call's number (or a later one,
// compared modulo 2^32).  Calls of one plan finish in order when they are
// ordered on the device, as they must be (they share the workspace); if the
// number has not arrived after 200 ms (a busy stream, or calls left unordered
// on two streams, whose numbers may arrive out of order), the whole device is
// waited for instead, after which every call has finished.
ec_status wait_done(ec_plan_s* pl) {
  if (!pl->have_done) return EC_OK;
  const volatile uint32_t* q = &pl->report_host->seq;
  const auto t0 = std::chrono::steady_clock::now();
  for (uint32_t k = 0; (int32_t)(*q - pl->seq) < 0; k++) {
    if (k < 256) {
      std::this_thread::yield();
      continue;
    }
    if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(200)) {
      if (hipDeviceSynchronize() != hipSuccess) return EC_ERR_DEVICE;
      break;
    }
    std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  return EC_OK;
}

// Workspace pointers of layout L inside the buffer at `ws` (a caller's
// workspace or the library's static scratch).
ec::Work make_work(const Layout& L, uint8_t* ws) {
  ec::Work w{};
  w.eb_base = reinterpret_cast<const float*>(ws + L.eb_base);
  w.mult = reinterpret_cast<const float*>(ws + L.mult);
  w.seg_tile_base = reinterpret_cast<const uint32_t*>(ws + L.seg_tile_base);
  w.hash_off = reinterpret_cast<const uint64_t*>(ws + L.hash_off);
  w.hash_log2 = reinterpret_cast<const uint32_t*>(ws + L.hash_log2);
  w.range_part = reinterpret_cast<float*>(ws + L.range_part);
  w.table_coder = L.table_coder ? reinterpret_cast<const uint32_t*>(ws + L.table_coder) : nullptr;
  w.nbr = L.nbr;
  w.dyn = reinterpret_cast<uint64_t*>(ws + L.dyn);
  w.dyn_words = L.dyn_bytes / 8;
  w.seg_start = reinterpret_cast<uint64_t*>(ws + L.seg_start);
  w.seg_end = reinterpret_cast<uint64_t*>(ws + L.seg_end);
  w.chunk_start = reinterpret_cast<uint64_t*>(ws + L.chunk_start);
  w.seg_fin = reinterpret_cast<uint32_t*>(ws + L.seg_fin);
  w.tile_status = reinterpret_cast<uint64_t*>(ws + L.tile_status);
  w.block_status = reinterpret_cast<uint64_t*>(ws + L.block_status);
  w.tile_inserted = reinterpret_cast<uint32_t*>(ws + L.tile_inserted);
  w.tile_rec = reinterpret_cast<uint64_t*>(ws + L.tile_rec);
  w.tile_U = reinterpret_cast<uint32_t*>(ws + L.tile_U);
  w.tile_nout = reinterpret_cast<uint32_t*>(ws + L.tile_nout);
  w.hash = reinterpret_cast<uint64_t*>(ws + L.hash);
  w.range_slot = reinterpret_cast<uint64_t*>(ws + L.range_slot);
  if (ec::encode_has_assembly(L.sh.D)) {
    w.stage_pl = reinterpret_cast<uint64_t*>(ws + L.stage_pl);
    w.stage_w = ws + L.stage_w;
    w.stage_om = reinterpret_cast<uint64_t*>(ws + L.stage_om);
    w.stage_slot = reinterpret_cast<uint32_t*>(ws + L.stage_slot);
    w.tile_info = reinterpret_cast<uint32_t*>(ws + L.tile_info);
    w.tile_bitmap = reinterpret_cast<uint64_t*>(ws + L.tile_bitmap);
    w.tile_first = reinterpret_cast<uint32_t*>(ws + L.tile_first);
    w.seg_eb = reinterpret_cast<uint32_t*>(ws + L.seg_eb);
  }
  if (L.huff) {
    w.stage_sym = reinterpret_cast<uint16_t*>(ws + L.stage_sym);
    w.hhist = reinterpret_cast<uint32_t*>(ws + L.hhist);
    w.henc = reinterpret_cast<uint32_t*>(ws + L.henc);
    w.hbooks = ws + L.hbooks;
    w.hstat = reinterpret_cast<uint32_t*>(ws + L.hstat);
    w.hhave = reinterpret_cast<uint32_t*>(ws + L.hhave);
    w.hskip = reinterpret_cast<uint32_t*>(ws + L.hskip);
    w.hdbooks = ws + L.hdbooks;
    w.hdenc = reinterpret_cast<uint32_t*>(ws + L.hdenc);
    w.tile_hsize = reinterpret_cast<uint32_t*>(ws + L.tile_hsize);
    w.seg_coder = reinterpret_cast<uint32_t*>(ws + L.seg_coder);
    w.hlut = reinterpret_cast<uint16_t*>(ws + L.hlut);
    w.hvalid = reinterpret_cast<uint32_t*>(ws + L.hvalid);
  }
  return w;
}

// Enqueue one compression into the workspace described by `work`: the range
// pass (and the clearing of the dynamic region when `clear`), quantization,
// and for D = 64, 128, 256 the assembly passes.
ec_status enqueue_compress(ec_plan_s* pl, const ec::Work& work, bool clear, int64_t iter,
                           const float* d_in, void* d_out, size_t out_cap, hipStream_t s);

}  // namespace

extern "C" {

uint32_t ec_max_dim(void) { return device_max_dim(); }

size_t ec_workspace_bytes(const ec_plan_desc* desc) {
  Layout L;
  if (make_layout(desc, &L) != EC_OK) return 0;
  return (size_t)L.total;
}

ec_status ec_plan(const ec_plan_desc* desc, ec_plan_t* out) {
  if (!out) return EC_ERR_INVALID;
  *out = nullptr;
  ec_plan_s* pl = new (std::nothrow) ec_plan_s();
  if (!pl) return EC_ERR_OOM;
  ec_status st = make_layout(desc, &pl->L);
  if (st != EC_OK) {
    delete pl;
    return st;
  }
  const Layout& L = pl->L;
  // no workspace at all: a plan for ec_compress_static (and ec_decompress) only
  const bool no_ws = !desc->d_workspace && desc->workspace_bytes == 0;
  if (no_ws && (L.huff || desc->window)) {  // their tables and roots live in the workspace
    delete pl;
    return EC_ERR_UNSUPPORTED;
  }
  if (!no_ws && (!desc->d_workspace || desc->workspace_bytes < L.total ||
                 ((uintptr_t)desc->d_workspace & 255u))) {
    delete pl;
    return desc->d_workspace && desc->workspace_bytes < L.total ? EC_ERR_CAPACITY
                                                                 : EC_ERR_INVALID;
  }
  pl->desc = *desc;
  const uint32_t T = L.sh.T;
  pl->eb.assign(desc->eb, desc->eb + T);
  pl->mult.assign(T, 1.0f);
  if (desc->table_mult) pl->mult.assign(desc->table_mult, desc->table_mult + T);
  pl->desc.eb = pl->eb.data();
  pl->desc.table_mult = nullptr;
  pl->desc.table_coder = nullptr;  // copied into the constants below
  pl->ws = static_cast<uint8_t*>(desc->d_workspace);

  size_t lds = ec::encode_lds_bytes(L.sh.D);
  if (lds > 65536 && ec::set_encode_lds_limit(lds) != hipSuccess) {
    delete pl;
    return EC_ERR_UNSUPPORTED;
  }
  // report block: the Report header with seg_bytes[nseg], then per segment
  // (U, eb valid) and the distinct raw rows of the last pattern count
  const size_t meta_off = aup(offsetof(ec::Report, seg_bytes) + 8ull * L.sh.nseg, 8);
  const size_t norig_off = meta_off + 8ull * L.sh.nseg;
  size_t rep_bytes = norig_off + 4ull * L.sh.nseg + 16;
  void* hp = nullptr;
  if (hipHostMalloc(&hp, rep_bytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    delete pl;
    return EC_ERR_DEVICE;
  }
  std::memset(hp, 0, rep_bytes);
  pl->report_host = static_cast<ec::Report*>(hp);
  void* dp = nullptr;
  if (hipHostGetDevicePointer(&dp, hp, 0) != hipSuccess) {
    (void)hipHostFree(hp);
    delete pl;
    return EC_ERR_DEVICE;
  }
  pl->report_dev = static_cast<ec::Report*>(dp);
  pl->meta_off = meta_off;
  pl->norig_off = norig_off;

  // the constant region, built on the host in pinned device-mapped memory
  void* cp = nullptr;
  void* cdp = nullptr;
  const uint64_t cbytes = L.dyn;
  if (hipHostMalloc(&cp, cbytes, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess ||
      hipHostGetDevicePointer(&cdp, cp, 0) != hipSuccess) {
    if (cp) (void)hipHostFree(cp);
    (void)hipHostFree(hp);
    delete pl;
    return EC_ERR_DEVICE;
  }
  pl->consts_host = static_cast<uint8_t*>(cp);
  pl->consts_dev = static_cast<uint8_t*>(cdp);
  uint8_t* img = pl->consts_host;
  std::memset(img, 0, cbytes);
  std::memcpy(img + L.eb_base, pl->eb.data(), 4ull * T);
  std::memcpy(img + L.mult, pl->mult.data(), 4ull * T);
  std::memcpy(img + L.seg_tile_base, L.seg_tile_base_v.data(), 4ull * L.seg_tile_base_v.size());
  std::memcpy(img + L.hash_off, L.hash_off_v.data(), 8ull * L.hash_off_v.size());
  std::memcpy(img + L.hash_log2, L.hash_log2_v.data(), 4ull * L.hash_log2_v.size());
  if (desc->table_coder) std::memcpy(img + L.table_coder, desc->table_coder, 4ull * T);
  // set-up of the static scratch on this device (its address, once per device)
  void* scr = nullptr;
  if (ec::static_scratch(&scr) != hipSuccess) {
    ec_plan_destroy(pl);
    return EC_ERR_DEVICE;
  }
  if (!no_ws) {
    // constants into the workspace (a blocking copy, plan time only)
    if (hipMemcpy(pl->ws, img, cbytes, hipMemcpyHostToDevice) != hipSuccess) {
      ec_plan_destroy(pl);
      return EC_ERR_DEVICE;
    }
    pl->work = make_work(L, pl->ws);
  }
  *out = pl;
  return EC_OK;
}

ec_status ec_plan_destroy(ec_plan_t pl) {
  if (!pl) return EC_ERR_INVALID;
  (void)wait_done(pl);
  for (hipEvent_t e : pl->prof_pool) (void)hipEventDestroy(e);
  if (pl->report_host) (void)hipHostFree(pl->report_host);
  if (pl->consts_host) (void)hipHostFree(pl->consts_host);
  delete pl;
  return EC_OK;
}

size_t ec_max_compressed_bytes(ec_plan_t pl) { return pl ? (size_t)pl->L.max_bytes : 0; }

ec_status ec_compress(ec_plan_t pl, int64_t iter, const float* d_in, void* d_out, size_t out_cap,
                      void* stream) {
  if (!pl || !d_out || !pl->ws) return EC_ERR_INVALID;
  const ec::Shape& sh = pl->L.sh;
  if (!d_in && (uint64_t)sh.B * sh.D > 0) return EC_ERR_INVALID;
  if (((uintptr_t)d_in & 15u) || ((uintptr_t)d_out & 15u)) return EC_ERR_INVALID;
  if (out_cap < pl->L.max_bytes) return EC_ERR_CAPACITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // D = 64, 128, 256: the dynamic region is zeroed on the plan's first call
  // only (the write pass leaves the hash tables clear); a call that fails to
  // launch all its kernels makes the next one clear again
  const bool assembled = ec::encode_has_assembly(sh.D);
  const bool clear = !assembled || !pl->hash_clear;
  pl->hash_clear = false;
  ec_status st = enqueue_compress(pl, pl->work, clear, iter, d_in, d_out, out_cap, s);
  if (st != EC_OK) return st;
  if (assembled) pl->hash_clear = true;
  return mark_done(pl, s);
}

ec_status ec_compress_static(ec_plan_t pl, int64_t iter, const float* d_in, void* d_out,
                             size_t out_cap, void* stream) {
  if (!pl || !d_out) return EC_ERR_INVALID;
  const ec::Shape& sh = pl->L.sh;
  if (!d_in && (uint64_t)sh.B * sh.D > 0) return EC_ERR_INVALID;
  if (((uintptr_t)d_in & 15u) || ((uintptr_t)d_out & 15u)) return EC_ERR_INVALID;
  if (out_cap < pl->L.max_bytes) return EC_ERR_CAPACITY;
  if (pl->L.total > EC_STATIC_SCRATCH_BYTES) return EC_ERR_CAPACITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scr = nullptr;  // this device's copy of the scratch (looked up once per device)
  if (ec::static_scratch(&scr) != hipSuccess) return EC_ERR_DEVICE;
  uint8_t* base = static_cast<uint8_t*>(scr);
  // the scratch holds whatever the last call on this device left there: the
  // plan's constants are copied in and the dynamic region is cleared, every call
  ec_status st = profiled(pl, EC_KERNEL_PREP, s, [&] {
    return ec::launch_copy_words(base, pl->consts_dev, pl->L.range_part, s);
  });
  if (st != EC_OK) return st;
  st = enqueue_compress(pl, make_work(pl->L, base), true, iter, d_in, d_out, out_cap, s);
  if (st != EC_OK) return st;
  return mark_done(pl, s);
}

ec_status ec_decompress(ec_plan_t pl, const void* d_stream, size_t stream_cap, float* d_out,
                        void* stream) {
  if (!pl || !d_stream) return EC_ERR_INVALID;
  const ec::Shape& sh = pl->L.sh;
  if (!d_out && (uint64_t)sh.B * sh.D > 0) return EC_ERR_INVALID;
  if (((uintptr_t)d_stream & 15u) || ((uintptr_t)d_out & 15u)) return EC_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  ec::DecArgs da{};
  da.in = static_cast<const uint8_t*>(d_stream);
  da.cap = stream_cap;
  da.y = d_out;
  da.sh = sh;
  // without a workspace the plan's pinned constants serve (read over the bus,
  // and only when the segments have different tile counts)
  da.seg_tile_base = pl->ws ? pl->work.seg_tile_base
                            : reinterpret_cast<const uint32_t*>(pl->consts_dev + pl->L.seg_tile_base);
  da.report = pl->report_dev;
  da.huff = pl->L.huff ? 1u : 0u;
  da.window = pl->desc.window ? 1u : 0u;
  da.w = pl->work;
  const ec_status st = profiled(pl, EC_KERNEL_DECODE, s, [&] {
    // windowed segments: every row's root before the decode kernels
    hipError_t e = da.window ? ec::launch_window_roots(da, s) : hipSuccess;
    if (e != hipSuccess || !pl->L.huff) return e == hipSuccess ? ec::launch_decode(da, s) : e;
    // the codebooks' tables first; Huffman tiles and their repeated rows after
    e = ec::launch_huff_tables(da, s);
    if (e == hipSuccess) e = ec::launch_decode(da, s);
    if (e == hipSuccess) e = ec::launch_huff_decode(da, s);
    return e;
  });
  if (st != EC_OK) return st;
  return mark_done(pl, s);
}

ec_status ec_ratio(ec_plan_t pl, double* total_cr, uint64_t* compressed_bytes,
                   double* per_segment_cr) {
  if (!pl) return EC_ERR_INVALID;
  if (wait_done(pl) != EC_OK) return EC_ERR_DEVICE;
  const ec::Shape& sh = pl->L.sh;
  volatile ec::Report* r = pl->report_host;
  uint64_t total = r->total_bytes;
  uint32_t status = r->status;
  r->status = 0;
  if (compressed_bytes) *compressed_bytes = total;
  if (total_cr) *total_cr = total ? (4.0 * sh.T * (double)sh.B * sh.D) / (double)total : 0.0;
  if (per_segment_cr) {
    for (uint32_t i = 0; i < sh.nseg; i++) {
      uint32_t p = i / sh.T;
      uint64_t b = r->seg_bytes[i];
      per_segment_cr[i] = b ? 4.0 * rows_of_chunk(sh.B, sh.P, p) * (double)sh.D / (double)b : 0.0;
    }
  }
  if (status == ec::kDevErrCorrupt) return EC_ERR_CORRUPT;
  if (status != 0) return EC_ERR_DEVICE;
  return EC_OK;
}

ec_status ec_homo_counts(ec_plan_t pl, int64_t iter, const float* d_in, void* d_out,
                         size_t out_cap, uint32_t* n_orig, uint32_t* n_quant, void* stream) {
  if (!pl || !n_orig || !n_quant) return EC_ERR_INVALID;
  if (pl->desc.window) return EC_ERR_UNSUPPORTED;  // its U counts literals, not distinct rows
  ec_status st = ec_compress(pl, iter, d_in, d_out, out_cap, stream);
  if (st != EC_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ec::Shape& sh = pl->L.sh;
  // the hash tables again, empty, for the raw rows (the next compression
  // clears them: they are left holding raw rows)
  pl->hash_clear = false;
  ec::PrepArgs pa{d_in, sh, pl->work, 0, 1};
  uint64_t g = (pl->work.dyn_words + 1023) / 1024;
  const uint32_t grid = (uint32_t)(g < 1 ? 1 : (g > 2048 ? 2048 : g));
  if (ec::launch_prep(pa, grid, s) != hipSuccess) return EC_ERR_DEVICE;
  ec::EncArgs ea{};
  ea.x = d_in;
  ea.sh = sh;
  ea.w = pl->work;
  uint32_t hb = pl->desc.debug_hash_bits;
  ea.hash_keep = (hb == 0 || hb >= 64) ? ~0ull : ((1ull << hb) - 1ull);
  ea.report = pl->report_dev;
  uint8_t* rep = reinterpret_cast<uint8_t*>(pl->report_dev);
  ea.seg_norig = reinterpret_cast<uint32_t*>(rep + pl->norig_off);
  if (ec::launch_distinct_raw(ea, s) != hipSuccess) return EC_ERR_DEVICE;
  if (mark_done(pl, s) != EC_OK || wait_done(pl) != EC_OK) return EC_ERR_DEVICE;
  const uint8_t* host = reinterpret_cast<const uint8_t*>(pl->report_host);
  const volatile uint32_t* meta = reinterpret_cast<const volatile uint32_t*>(host + pl->meta_off);
  const volatile uint32_t* norig = reinterpret_cast<const volatile uint32_t*>(host + pl->norig_off);
  for (uint32_t i = 0; i < sh.nseg; i++) {
    n_orig[i] = norig[i];
    n_quant[i] = meta[2 * i + 1] ? meta[2 * i] : norig[i];  // no valid eb: not quantized
  }
  if (pl->report_host->status != 0) return EC_ERR_DEVICE;
  return EC_OK;
}

double ec_speedup(double cr, double bw, double tc, double td) {
  return 1.0 / (1.0 / cr + bw * (1.0 / tc + 1.0 / td));
}

ec_status ec_select_coders(uint32_t num_tables, uint32_t ncomp, const double* cr, const double* tc,
                           const double* td, double bw, int32_t* best, double* speedup) {
  auto pos = [](double v) { return v > 0.0 && std::isfinite(v); };
  if (ncomp == 0 || !cr || !tc || !td || !best || !pos(bw)) return EC_ERR_INVALID;
  for (uint32_t c = 0; c < ncomp; c++) {
    if (!pos(tc[c]) || !pos(td[c])) return EC_ERR_INVALID;
    for (uint32_t t = 0; t < num_tables; t++)
      if (!pos(cr[(size_t)c * num_tables + t])) return EC_ERR_INVALID;
  }
  for (uint32_t t = 0; t < num_tables; t++) {
    int32_t b = 0;
    double v = ec_speedup(cr[t], bw, tc[0], td[0]);
    for (uint32_t c = 1; c < ncomp; c++) {
      const double w = ec_speedup(cr[(size_t)c * num_tables + t], bw, tc[c], td[c]);
      if (w > v) {
        v = w;
        b = (int32_t)c;
      }
    }
    best[t] = b;
    if (speedup) speedup[t] = v;
  }
  return EC_OK;
}

ec_status ec_classify_tables(uint32_t num_tables, const double* homo_index, double l_thresh,
                             double s_thresh, double alpha, double beta, int32_t* table_class,
                             float* table_mult) {
  if (!homo_index || !table_class || !table_mult || !(l_thresh <= s_thresh)) return EC_ERR_INVALID;
  if (!(alpha > 0.0) || !std::isfinite(alpha) || !(beta > 0.0) || !std::isfinite(beta))
    return EC_ERR_INVALID;
  for (uint32_t t = 0; t < num_tables; t++) {
    const double h = homo_index[t];
    if (h > s_thresh) {
      table_class[t] = EC_CLASS_SMALL;
      table_mult[t] = (float)(1.0 / beta);
    } else if (h < l_thresh) {
      table_class[t] = EC_CLASS_LARGE;
      table_mult[t] = (float)alpha;
    } else {
      table_class[t] = EC_CLASS_MEDIUM;
      table_mult[t] = 1.0f;
    }
  }
  return EC_OK;
}

const char* ec_status_string(ec_status s) {
  switch (s) {
    case EC_OK: return "ok";
    case EC_ERR_INVALID: return "invalid argument";
    case EC_ERR_CAPACITY: return "capacity too small";
    case EC_ERR_CORRUPT: return "corrupt stream";
    case EC_ERR_DEVICE: return "device error";
    case EC_ERR_OOM: return "out of host memory";
    case EC_ERR_UNSUPPORTED: return "unsupported shape";
  }
  return "unknown status";
}

ec_status ec_debug_attach(ec_plan_t pl, int32_t* d_codes, uint8_t* d_outlier, uint32_t* d_first,
                          float* d_eb) {
  if (!pl) return EC_ERR_INVALID;
  pl->dbg_codes = d_codes;
  pl->dbg_outlier = d_outlier;
  pl->dbg_first = d_first;
  pl->dbg_eb = d_eb;
  return EC_OK;
}

ec_status ec_profile_enable(ec_plan_t pl, int enable, uint32_t max_launches) {
  if (!pl) return EC_ERR_INVALID;
  (void)wait_done(pl);
  pl->prof_recs.clear();
  pl->prof_next = 0;
  pl->prof_dropped = 0;
  pl->prof_on = enable != 0;
  size_t want = enable ? 2ull * max_launches : 0;
  while (pl->prof_pool.size() < want) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return EC_ERR_DEVICE;
    pl->prof_pool.push_back(e);
  }
  return EC_OK;
}

ec_status ec_profile_read(ec_plan_t pl, int kernel, double* total_ms, uint64_t* launches) {
  if (!pl || !total_ms || !launches) return EC_ERR_INVALID;
  double sum = 0.0;
  uint64_t cnt = 0;
  for (const ProfRec& r : pl->prof_recs) {
    if (r.kernel != kernel) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return EC_ERR_DEVICE;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return EC_ERR_DEVICE;
    sum += ms;
    cnt++;
  }
  *total_ms = sum;
  *launches = cnt;
  return EC_OK;
}

}  // extern "C"

namespace {

ec_status enqueue_compress(ec_plan_s* pl, const ec::Work& work, bool clear, int64_t iter,
                           const float* d_in, void* d_out, size_t out_cap, hipStream_t s) {
  const ec::Shape& sh = pl->L.sh;
  ec::PrepArgs pa{d_in, sh, work, pl->desc.eb_mode == EC_EB_REL_RANGE ? 1 : 0, clear ? 1 : 0};
  // D = 64, 128: the quantize pass finds the tables' ranges itself, its range
  // items running ahead of its tiles (the input's first read overlaps the
  // quantization instead of preceding it; 26x4096x64: 51 -> 43 us,
  // 26x8192x128: 66 -> 55 us)
  const uint32_t tpt = sh.ntiles / sh.T;
  const bool fuse = pa.rel && sh.B > 0 && (sh.D == 64 || sh.D == 128);
  if (fuse) pa.rel = 0;
  uint32_t grid;
  if (pa.rel && sh.B > 0) {
    grid = sh.T * pl->L.nbr;
  } else {
    pa.rel = 0;
    uint64_t g = (work.dyn_words + 1023) / 1024;
    grid = (uint32_t)(g < 1 ? 1 : (g > 2048 ? 2048 : g));
  }
  ec_status st = EC_OK;
  if (pa.rel || pa.clear) st = profiled(pl, EC_KERNEL_PREP, s, [&] { return ec::launch_prep(pa, grid, s); });
  if (st != EC_OK) return st;

  ec::EncArgs ea{};
  ea.x = d_in;
  ea.out = static_cast<uint8_t*>(d_out);
  ea.out_cap = out_cap;
  ea.sh = sh;
  ea.w = work;
  ea.eb_mode = (uint32_t)pl->desc.eb_mode;
  ea.iter = iter;
  ea.sched = schedule_factor(pl->desc.sched, iter);
  ea.coder = pl->L.stream_coder;
  ea.window = pl->desc.window;
  ea.fuse_range = fuse ? 1u : 0u;
  ea.tiles_per_table = tpt;
  ea.range_items = pl->L.range_items;
  ea.range_ahead = kRangeAhead;
  ea.reuse_books = pl->desc.reuse_books && pl->L.huff ? 1u : 0u;
  uint32_t hb = pl->desc.debug_hash_bits;
  ea.hash_keep = (hb == 0 || hb >= 64) ? ~0ull : ((1ull << hb) - 1ull);
  ea.report = pl->report_dev;
  ea.seg_meta = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(pl->report_dev) + pl->meta_off);
  ea.seg_norig = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(pl->report_dev) + pl->norig_off);
  ea.dbg_codes = pl->dbg_codes;
  ea.dbg_outlier = pl->dbg_outlier;
  ea.dbg_first = pl->dbg_first;
  ea.dbg_eb = pl->dbg_eb;
  st = profiled(pl, EC_KERNEL_ENCODE, s, [&] {
    hipError_t e = ec::launch_encode(ea, s);
    if (e == hipSuccess && ea.window) e = ec::launch_window(ea, s);  // the matches
    return e;
  });
  if (st != EC_OK) return st;
  if (ec::encode_has_assembly(sh.D)) {
    st = profiled(pl, EC_KERNEL_ASSEMBLE, s, [&] {
      if (!pl->L.huff) return ec::launch_assemble(ea, s);
      // size pass, then the Huffman coder's passes, write pass, chunk words
      hipError_t e = ec::launch_assemble_size(ea, s);
      if (e == hipSuccess) e = ec::launch_huff_encode(ea, s);
      if (e == hipSuccess) e = ec::launch_assemble_write(ea, s);
      if (e == hipSuccess) e = ec::launch_huff_write(ea, s);
      return e;
    });
    if (st != EC_OK) return st;
  }
  return EC_OK;
}

}  // namespace
