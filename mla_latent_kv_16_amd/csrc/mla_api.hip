// extern "C" entry points of libmla (declared in include/mla.h): argument checks,
// partition choice, workspace layout and launches.  No device memory is allocated.
#include "../../include/mla.h"
#include "mla_device.h"
#include "mla_internal.h"

#include <math.h>
#include <stdlib.h>
#include <mutex>
#include <numeric>

namespace {

using namespace mla;

constexpr int kMaxDevices = 64;
// pool row formats
constexpr int kFormatBf16 = 0, kFormatE4m3 = 1, kFormatNope = 2;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

// Compute units of the current device (cached per device).
int cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::call_once(g_cu_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n = 0;
    g_cu_count[dev] = n;
  });
  if (g_cu_count[dev] <= 0) return MLA_ERR_HIP;
  *out = g_cu_count[dev];
  return MLA_OK;
}

// Geometry of one call: M-tile rows, M-tiles per request, rows per partial slot.
struct Geometry {
  int M, mt_rows, n_mt, slot_rows;
};

int geometry(int B, int Sq, int H, int max_pages, Geometry* g) {
  if (B < 1 || Sq < 1 || H < 1 || max_pages < 1) return MLA_ERR_INVALID_ARG;
  if (B > kMaxBatch) return MLA_ERR_UNSUPPORTED;
  const int64_t M = (int64_t)Sq * H;
  if (M > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)B * max_pages > 0x7fffffffLL / 2) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)max_pages * kPage > 0x7fffffffLL / 2) return MLA_ERR_UNSUPPORTED;
  g->M = (int)M;
  g->mt_rows = kMTile;
  g->n_mt = (int)((M + g->mt_rows - 1) / g->mt_rows);
  g->slot_rows = (int)(M < g->mt_rows ? M : g->mt_rows);
  return MLA_OK;
}

// Default partition count, from a cost model of one decode measured on MI355X: a
// workgroup walks its partition at about 2.8 us per page (two 32-row blocks), a
// split writes and re-reads its partial results (min(M, 64) rows x 513 floats per
// piece) at about 0.44 us per MB, and adds one merge launch (about 4 us).  Long
// contexts take the most partitions (the walk dominates); short ones trade
// parallelism against partial traffic.  Candidates are multiples of B, up to one
// (partition x M-tile) workgroup per compute unit, so that equal requests split
// evenly; below four pages per partition a candidate must also divide the page count,
// since a partition that straddles two requests walks and writes two pieces.  The
// page count is the block table's capacity, an upper bound of the real one.
//
// One refinement from the same measurements: with one M-tile per request and walks of
// 8 to 32 pages per workgroup, about 80% of the compute units already keep the HBM
// stream of the pages saturated, and the remaining partitions only add partials and
// merge work.  There the count is capped at about 80% of the compute units, rounded
// up to a multiple of B and of the eight XCDs (a spec-decode step of B = 4, Sq = 4,
// 65,540 rows: 75.7 us at 208 partitions against 79.5 us at 256, and 208 ahead of 204
// and 200, which leave the XCDs uneven; 32,772 rows: 47.0 against 49.7 us).  Longer walks (64 pages per workgroup:
// 232.6 us at 256 against 238.9 at 224) and shorter ones keep the plain model.  The
// cap does not depend on the pool format; E4M3 pools, whose walk is bound by the
// widening VALU rather than by HBM, would keep every compute unit (72.5 against
// 76.2 us at 208), but one count per shape keeps the split and combine calls of every
// format in step.
int pick_partitions(const Geometry& g, int B, int64_t pages, int64_t gmax) {
  constexpr double kUsPerPage = 2.8, kUsPerPartialMB = 0.44, kUsMerge = 4.0;
  const double piece_mb = (double)g.n_mt * g.slot_rows * (kNope + 1) * 4 * 1e-6;
  int64_t best = 1;
  double best_us = (double)pages * kUsPerPage;
  for (int64_t G = B; G <= gmax; G += B) {
    if (G == 1 || (pages < 4 * G && pages % G != 0)) continue;
    const double us = (double)pages / (double)G * kUsPerPage +
                      (double)G * piece_mb * kUsPerPartialMB + kUsMerge;
    if (us < best_us) {
      best_us = us;
      best = G;
    }
  }
  return (int)best;
}

int auto_partitions(const Geometry& g, int B, int max_pages, int cus) {
  const int64_t pages = (int64_t)B * max_pages;
  int64_t gmax = cus / g.n_mt;
  if (gmax > pages) gmax = pages;
  if (gmax < 1) gmax = 1;
  if (B > gmax) {  // fewer partitions than requests: at least about four pages each
    const int64_t by_pages = (pages + 3) / 4;
    return (int)(by_pages < gmax ? by_pages : gmax);
  }
  const int best = pick_partitions(g, B, pages, gmax);
  // 80% of the CUs, rounded up to a multiple of both B and the eight XCDs, so that the
  // requests split evenly and every XCD runs as many workgroups as the others
  const int64_t unit = std::lcm((int64_t)B, (int64_t)8);
  const int64_t cap = ((int64_t)cus * 4 / 5 + unit - 1) / unit * unit;
  if (g.n_mt == 1 && best > cap && pages >= 8 * (int64_t)best && pages <= 32 * (int64_t)best)
    return pick_partitions(g, B, pages, cap);
  return best;
}

int resolve_partitions(const Geometry& g, int B, int max_pages, int requested, int* G) {
  if (requested < 0) return MLA_ERR_INVALID_ARG;
  if (requested > 0) {
    if ((int64_t)requested * g.n_mt > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
    *G = requested;
    return MLA_OK;
  }
  int cus = 0;
  const int st = cu_count(&cus);
  if (st != MLA_OK) return st;
  *G = auto_partitions(g, B, max_pages, cus);
  return MLA_OK;
}

// Single-pass counters: arrive[B * n_mt] and done[B * n_mt], after the header.
size_t counter_bytes(const Geometry& g, int B) {
  return ((size_t)2 * B * g.n_mt * sizeof(uint32_t) + 255) & ~(size_t)255;
}

size_t workspace_bytes_for(const Geometry& g, int B, int G) {
  size_t bytes = kHeaderBytes;
  if (G > 1) {
    bytes += counter_bytes(g, B);
    const size_t slots = (size_t)(B + G) * g.n_mt;
    bytes += slots * g.slot_rows * kNope * sizeof(float);   // partial O
    bytes += ((slots * g.slot_rows * sizeof(float)) + 255) & ~(size_t)255;  // partial LSE
  }
  return bytes;
}

struct Layout {
  uint32_t* flags;
  uint32_t* arrive;
  uint32_t* done;
  float* part_o;
  float* part_lse;
};

// [256-byte header | counters | partial O | partial LSE]; only the header when G = 1
Layout carve(void* ws, const Geometry& g, int B, int G) {
  Layout l;
  uint8_t* base = static_cast<uint8_t*>(ws);
  l.flags = reinterpret_cast<uint32_t*>(base);
  const size_t slots = (size_t)(B + G) * g.n_mt;
  const size_t cnt = G > 1 ? counter_bytes(g, B) : 0;
  l.arrive = reinterpret_cast<uint32_t*>(base + kHeaderBytes);
  l.done = l.arrive + (size_t)B * g.n_mt;
  l.part_o = reinterpret_cast<float*>(base + kHeaderBytes + cnt);
  l.part_lse =
      reinterpret_cast<float*>(base + kHeaderBytes + cnt + slots * g.slot_rows * kNope * 4);
  return l;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Waits for the stream, then moves the workspace header's flag word to *flags and
// clears it.
int take_flags(void* workspace, hipStream_t s, uint32_t* flags) {
  if (hipStreamSynchronize(s) != hipSuccess) return MLA_ERR_HIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, workspace, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  const uint32_t zero = 0;
  if (hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
    return MLA_ERR_HIP;
  *flags = v;
  return MLA_OK;
}

// Checked mode (environment MLA_CHECK=1): a compute call that enqueued its work also
// waits for it and turns a raised data-fault flag into MLA_ERR_DEVICE_CHECK.  Off by
// default, since waiting forces a synchronisation on every call.
bool checked_mode() {
  const char* v = getenv("MLA_CHECK");
  return v && v[0] == '1' && v[1] == 0;
}

int finish(int st, void* workspace, hipStream_t s) {
  if (st != MLA_OK || !checked_mode()) return st;
  uint32_t flags = 0;
  const int rd = take_flags(workspace, s, &flags);
  if (rd != MLA_OK) return rd;
  return flags ? MLA_ERR_DEVICE_CHECK : MLA_OK;
}

struct Call {
  Geometry geo;
  int G;
  Layout lay;
};

// Shared checks of every compute entry point.
int prepare(const uint16_t* q_nope, const uint16_t* q_rope, const void* kv_pool,
            int64_t num_pages, int page_size, const int32_t* block_table, int max_pages,
            const int32_t* seq_lens, int B, int Sq, int H, float scale, int causal,
            int num_partitions, const float* O, const float* lse, void* ws, size_t ws_bytes,
            Call* call) {
  if (!q_nope || !q_rope || !kv_pool || !block_table || !seq_lens || !O || !lse)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(kv_pool) || !aligned16(O))
    return MLA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3) ||
      (reinterpret_cast<uintptr_t>(lse) & 3))
    return MLA_ERR_INVALID_ARG;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (num_pages < 1) return MLA_ERR_INVALID_ARG;
  if (num_pages > (int64_t)1 << 40) return MLA_ERR_UNSUPPORTED;
  if (!(scale == scale) || isinf(scale)) return MLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  int st = geometry(B, Sq, H, max_pages, &call->geo);
  if (st != MLA_OK) return st;
  st = resolve_partitions(call->geo, B, max_pages, num_partitions, &call->G);
  if (st != MLA_OK) return st;
  if (!ws || !aligned16(ws)) return MLA_ERR_WORKSPACE;
  if (ws_bytes < workspace_bytes_for(call->geo, B, call->G)) return MLA_ERR_WORKSPACE;
  call->lay = carve(ws, call->geo, B, call->G);
  return MLA_OK;
}

// Which split-KV kernel runs a call.  The quarter-split and eight-wave kernels apply to
// bf16 pools without draft trees in two-pass calls; elsewhere the four-wave kernel
// runs.  MLA_SPLITKV=4, =8 or =q in the environment forces the choice where it applies.
enum class SplitKernel { kFour, kEight, kQuarter };

SplitKernel split_kernel_for(const SplitArgs& a) {
  if (a.kv_e4m3 || a.kv_nope || a.tree_mask || a.arrive || a.wg_trace) return SplitKernel::kFour;
  const char* v = getenv("MLA_SPLITKV");
  if (v && v[0] == '8' && v[1] == 0) return SplitKernel::kEight;
  if (v && v[0] == 'q' && v[1] == 0) return SplitKernel::kQuarter;
  return SplitKernel::kFour;
}

int enqueue_split(const Call& c, const uint16_t* q_nope, const uint16_t* q_rope,
                  const void* kv_pool, int kv_format, float kv_scale, int64_t num_pages,
                  const int32_t* block_table, int max_pages, const int32_t* seq_lens,
                  const uint64_t* tree_mask, int B, int Sq, int H, float scale, int causal,
                  float* O, float* lse, bool single_pass, hipStream_t stream,
                  const int32_t* q_lens = nullptr, int32_t* wg_trace = nullptr,
                  int64_t* wg_time = nullptr) {
  SplitArgs a;
  a.wg_trace = wg_trace;
  a.wg_time = wg_time;
  a.tree_mask = tree_mask;
  a.q_lens = q_lens;
  a.len_min = q_lens ? 1 : Sq;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.kv_pool = kv_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.O = O;
  a.lse = lse;
  a.part_o = c.lay.part_o;
  a.part_lse = c.lay.part_lse;
  a.flags = c.lay.flags;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.B = B;
  a.Sq = Sq;
  a.H = H;
  a.M = c.geo.M;
  a.n_mt = c.geo.n_mt;
  a.G = c.G;
  a.slot_rows = c.geo.slot_rows;
  a.causal = causal;
  a.kv_e4m3 = kv_format == kFormatE4m3;
  a.kv_nope = kv_format == kFormatNope;
  a.kv_scale = kv_scale;
  a.scale_log2 = scale * kv_scale * 1.4426950408889634f;
  a.n_split = c.G * c.geo.n_mt;
  a.arrive = nullptr;
  a.done = nullptr;
  a.comb_rows = 0;
  if (single_pass && c.G > 1) {
    a.arrive = c.lay.arrive;
    a.done = c.lay.done;
    // as for the separate combine: a workgroup per row when there are many pieces
    // per request, else waves over runs of rows, about one workgroup per CU
    if ((int64_t)c.G < 16 * (int64_t)B) {
      int cus = 0;
      if (cu_count(&cus) != MLA_OK) return MLA_ERR_HIP;
      const int64_t rows = (int64_t)B * c.geo.M;
      const int64_t per_wave = (rows + (int64_t)kWaves * cus - 1) / ((int64_t)kWaves * cus);
      a.comb_rows = (int)(per_wave < 1 ? 1 : per_wave);
    }
    // The counters share the workspace with the partial results of calls of other
    // shapes (whose partial slots may lie where this call's counters are), so they
    // are zeroed before every single-pass launch rather than trusted to be zero.
    if (launch_clear_words(c.lay.arrive, 2 * (int64_t)B * c.geo.n_mt, stream) != hipSuccess)
      return MLA_ERR_HIP;
  }
  hipError_t e;
  switch (split_kernel_for(a)) {
    case SplitKernel::kEight: e = launch_splitkv8(a, stream); break;
    case SplitKernel::kQuarter: e = launch_splitkvq(a, stream); break;
    default: e = launch_splitkv(a, stream); break;
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int enqueue_combine(const Call& c, const int32_t* seq_lens, int max_pages, int B, int Sq, int H,
                    float* O, float* lse, hipStream_t stream) {
  if (c.G <= 1) return MLA_OK;
  CombineArgs a;
  a.seq_lens = seq_lens;
  a.O = O;
  a.lse = lse;
  a.part_o = c.lay.part_o;
  a.part_lse = c.lay.part_lse;
  a.flags = c.lay.flags;
  a.arrive = nullptr;
  a.done = nullptr;
  a.max_pages = max_pages;
  a.B = B;
  a.Sq = Sq;
  a.H = H;
  a.M = c.geo.M;
  a.n_mt = c.geo.n_mt;
  a.G = c.G;
  a.MT = c.geo.mt_rows;
  a.slot_rows = c.geo.slot_rows;
  return launch_combine(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// One decode: the split-KV pass, then the separate merge kernel, or both in one
// launch (single_pass).
int decode_call(const uint16_t* q_nope, const uint16_t* q_rope, const void* kv_pool, int kv_format,
                float kv_scale, int64_t num_pages, int page_size, const int32_t* block_table,
                int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq, int H,
                float softmax_scale, int causal, int num_partitions, float* O, float* lse,
                void* workspace, size_t workspace_bytes, void* stream, bool single_pass,
                const uint64_t* tree_mask = nullptr, const int32_t* q_lens = nullptr) {
  if (kv_format == kFormatE4m3 && (!(kv_scale > 0.0f) || isinf(kv_scale)))
    return MLA_ERR_INVALID_ARG;
  Call c;
  int st = prepare(q_nope, q_rope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                   seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                   workspace_bytes, &c);
  if (st != MLA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = enqueue_split(c, q_nope, q_rope, kv_pool, kv_format, kv_scale, num_pages, block_table,
                     max_pages_per_seq, seq_lens, tree_mask, B, Sq, H, softmax_scale, causal, O,
                     lse, single_pass, s, q_lens);
  if (st == MLA_OK && !single_pass)
    st = enqueue_combine(c, seq_lens, max_pages_per_seq, B, Sq, H, O, lse, s);
  return finish(st, workspace, s);
}

// ---- the no-allocation decode ------------------------------------------------------
// mla_decode_noalloc keeps its workspace (error-flag header, partial results) in this
// file-scope device array instead of a caller buffer.  Each device the library runs on
// holds its own copy until the process ends.  In host code the array's name is only a
// host-side stand-in: the device address is looked up once per device with
// hipGetSymbolAddress and kept in g_scratch, and only that address is ever passed on.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
void* g_scratch[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? p : nullptr;
  });
  if (!g_scratch[dev]) return MLA_ERR_HIP;
  *out = g_scratch[dev];
  return MLA_OK;
}

// Largest partition count <= G whose workspace fits the scratch array (1 always
// fits: a call without a split needs only the header).
int partitions_fitting(const Geometry& g, int B, int G) {
  while (G > 1 && workspace_bytes_for(g, B, G) > kScratchBytes) {
    const size_t piece = (size_t)g.n_mt * g.slot_rows * (kNope + 1) * sizeof(float);
    const size_t fixed = kHeaderBytes + counter_bytes(g, B) + 256;
    const int64_t fit = kScratchBytes > fixed ? (int64_t)((kScratchBytes - fixed) / piece) - B : 0;
    G = fit >= 2 && fit < G ? (int)fit : (fit < 2 ? 1 : G - 1);
  }
  return G;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: unsupported size or page size";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    case MLA_ERR_DEVICE_CHECK:
      return "MLA_ERR_DEVICE_CHECK: the kernels flagged a bad seq_lens or block_table entry "
             "(checked mode)";
    default: return "unknown mla status";
  }
}

int mla_decode_auto_partitions(int B, int Sq, int H, int max_pages_per_seq, int* num_partitions) {
  if (!num_partitions) return MLA_ERR_INVALID_ARG;
  Geometry g;
  int st = geometry(B, Sq, H, max_pages_per_seq, &g);
  if (st != MLA_OK) return st;
  return resolve_partitions(g, B, max_pages_per_seq, 0, num_partitions);
}

int mla_decode_workspace_size(int B, int Sq, int H, int max_pages_per_seq, int num_partitions,
                              size_t* bytes) {
  if (!bytes) return MLA_ERR_INVALID_ARG;
  Geometry g;
  int st = geometry(B, Sq, H, max_pages_per_seq, &g);
  if (st != MLA_OK) return st;
  int G = 0;
  st = resolve_partitions(g, B, max_pages_per_seq, num_partitions, &G);
  if (st != MLA_OK) return st;
  *bytes = workspace_bytes_for(g, B, G);
  return MLA_OK;
}

size_t mla_decode_workspace_bytes(int B, int Sq, int H, int max_pages_per_seq) {
  size_t bytes = 0;
  return mla_decode_workspace_size(B, Sq, H, max_pages_per_seq, 0, &bytes) == MLA_OK ? bytes : 0;
}

size_t mla_prefill_workspace_bytes(int B, int Sq, int H, int max_pages_per_seq) {
  // prefill runs the same passes with the same automatic partition count
  return mla_decode_workspace_bytes(B, Sq, H, max_pages_per_seq);
}

int mla_decode_splitkv(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                       int64_t num_pages, int page_size, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq, int H,
                       float softmax_scale, int causal, int num_partitions, float* O, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  Call c;
  int st = prepare(q_nope, q_rope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                   seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                   workspace_bytes, &c);
  if (st != MLA_OK) return st;
  return finish(enqueue_split(c, q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages,
                              block_table, max_pages_per_seq, seq_lens, nullptr, B, Sq, H,
                              softmax_scale, causal, O, lse, false,
                              static_cast<hipStream_t>(stream)),
                workspace, static_cast<hipStream_t>(stream));
}

int mla_decode_splitkv_placement(const uint16_t* q_nope, const uint16_t* q_rope,
                                 const uint16_t* kv_pool, int64_t num_pages, int page_size,
                                 const int32_t* block_table, int max_pages_per_seq,
                                 const int32_t* seq_lens, int B, int Sq, int H,
                                 float softmax_scale, int causal, int num_partitions, float* O,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 int32_t* wg_trace, int64_t wg_trace_len, void* stream) {
  Call c;
  int st = prepare(q_nope, q_rope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                   seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                   workspace_bytes, &c);
  if (st != MLA_OK) return st;
  if (!wg_trace || (reinterpret_cast<uintptr_t>(wg_trace) & 3)) return MLA_ERR_INVALID_ARG;
  if (wg_trace_len < 3 * (int64_t)c.G * c.geo.n_mt) return MLA_ERR_INVALID_ARG;
  return finish(enqueue_split(c, q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages,
                              block_table, max_pages_per_seq, seq_lens, nullptr, B, Sq, H,
                              softmax_scale, causal, O, lse, false,
                              static_cast<hipStream_t>(stream), nullptr, wg_trace),
                workspace, static_cast<hipStream_t>(stream));
}

int mla_decode_splitkv_timeline(const uint16_t* q_nope, const uint16_t* q_rope,
                                const uint16_t* kv_pool, int64_t num_pages, int page_size,
                                const int32_t* block_table, int max_pages_per_seq,
                                const int32_t* seq_lens, int B, int Sq, int H,
                                float softmax_scale, int causal, int num_partitions, float* O,
                                float* lse, void* workspace, size_t workspace_bytes,
                                int32_t* wg_trace, int64_t wg_trace_len, int64_t* wg_time,
                                int64_t wg_time_len, void* stream) {
  Call c;
  int st = prepare(q_nope, q_rope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                   seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                   workspace_bytes, &c);
  if (st != MLA_OK) return st;
  const int64_t nwg = (int64_t)c.G * c.geo.n_mt;
  if (!wg_trace || (reinterpret_cast<uintptr_t>(wg_trace) & 3)) return MLA_ERR_INVALID_ARG;
  if (wg_trace_len < 3 * nwg) return MLA_ERR_INVALID_ARG;
  if (!wg_time || (reinterpret_cast<uintptr_t>(wg_time) & 7)) return MLA_ERR_INVALID_ARG;
  if (wg_time_len < 5 * nwg) return MLA_ERR_INVALID_ARG;
  return finish(enqueue_split(c, q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages,
                              block_table, max_pages_per_seq, seq_lens, nullptr, B, Sq, H,
                              softmax_scale, causal, O, lse, false,
                              static_cast<hipStream_t>(stream), nullptr, wg_trace, wg_time),
                workspace, static_cast<hipStream_t>(stream));
}

int mla_decode_combine(const int32_t* seq_lens, int max_pages_per_seq, int B, int Sq, int H,
                       int num_partitions, float* O, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!seq_lens || !O || !lse) return MLA_ERR_INVALID_ARG;
  if (!aligned16(O) || (reinterpret_cast<uintptr_t>(lse) & 3)) return MLA_ERR_INVALID_ARG;
  Call c;
  int st = geometry(B, Sq, H, max_pages_per_seq, &c.geo);
  if (st != MLA_OK) return st;
  st = resolve_partitions(c.geo, B, max_pages_per_seq, num_partitions, &c.G);
  if (st != MLA_OK) return st;
  if (!workspace || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  if (workspace_bytes < workspace_bytes_for(c.geo, B, c.G)) return MLA_ERR_WORKSPACE;
  c.lay = carve(workspace, c.geo, B, c.G);
  return finish(enqueue_combine(c, seq_lens, max_pages_per_seq, B, Sq, H, O, lse,
                                static_cast<hipStream_t>(stream)),
                workspace, static_cast<hipStream_t>(stream));
}

int mla_decode(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
               int64_t num_pages, int page_size, const int32_t* block_table,
               int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq, int H,
               float softmax_scale, int causal, int num_partitions, float* O, float* lse,
               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, causal,
                     num_partitions, O, lse, workspace, workspace_bytes, stream, false);
}

int mla_decode_noalloc(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                       int64_t num_pages, int page_size, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq, int H,
                       float softmax_scale, int causal, int num_partitions, float* O,
                       float* lse, void* stream) {
  Geometry g;
  int st = geometry(B, Sq, H, max_pages_per_seq, &g);
  if (st != MLA_OK) return st;
  int G = 0;
  st = resolve_partitions(g, B, max_pages_per_seq, num_partitions, &G);
  if (st != MLA_OK) return st;
  if (num_partitions == 0)
    G = partitions_fitting(g, B, G);
  else if (workspace_bytes_for(g, B, G) > kScratchBytes)
    return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MLA_OK) return st;
  return decode_call(q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages, page_size,
                     block_table, max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, causal, G,
                     O, lse, ws, kScratchBytes, stream, false);
}

int mla_decode_single_pass(const uint16_t* q_nope, const uint16_t* q_rope,
                           const uint16_t* kv_pool, int64_t num_pages, int page_size,
                           const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                           int causal, int num_partitions, float* O, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_call(q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, causal,
                     num_partitions, O, lse, workspace, workspace_bytes, stream, true);
}

int mla_prefill_with_prefix(const uint16_t* q_nope, const uint16_t* q_rope,
                            const uint16_t* kv_pool, int64_t num_pages, int page_size,
                            const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                            int causal, int num_partitions, float* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode(q_nope, q_rope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                    seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                    workspace_bytes, stream);
}

int mla_decode_splitkv_e4m3(const uint16_t* q_nope, const uint16_t* q_rope,
                            const uint8_t* kv_pool, float kv_scale, int64_t num_pages,
                            int page_size, const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                            int causal, int num_partitions, float* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!(kv_scale > 0.0f) || isinf(kv_scale)) return MLA_ERR_INVALID_ARG;
  Call c;
  int st = prepare(q_nope, q_rope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                   seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                   workspace_bytes, &c);
  if (st != MLA_OK) return st;
  return finish(enqueue_split(c, q_nope, q_rope, kv_pool, kFormatE4m3, kv_scale, num_pages,
                              block_table, max_pages_per_seq, seq_lens, nullptr, B, Sq, H,
                              softmax_scale, causal, O, lse, false,
                              static_cast<hipStream_t>(stream)),
                workspace, static_cast<hipStream_t>(stream));
}

int mla_decode_e4m3(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* kv_pool,
                    float kv_scale, int64_t num_pages, int page_size, const int32_t* block_table,
                    int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq, int H,
                    float softmax_scale, int causal, int num_partitions, float* O, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(q_nope, q_rope, kv_pool, kFormatE4m3, kv_scale, num_pages, page_size,
                     block_table, max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, causal,
                     num_partitions, O, lse, workspace, workspace_bytes, stream, false);
}

int mla_decode_single_pass_e4m3(const uint16_t* q_nope, const uint16_t* q_rope,
                                const uint8_t* kv_pool, float kv_scale, int64_t num_pages,
                                int page_size, const int32_t* block_table, int max_pages_per_seq,
                                const int32_t* seq_lens, int B, int Sq, int H,
                                float softmax_scale, int causal, int num_partitions, float* O,
                                float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_call(q_nope, q_rope, kv_pool, kFormatE4m3, kv_scale, num_pages, page_size,
                     block_table, max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, causal,
                     num_partitions, O, lse, workspace, workspace_bytes, stream, true);
}

int mla_decode_tree(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                    int64_t num_pages, int page_size, const int32_t* block_table,
                    int max_pages_per_seq, const int32_t* seq_lens, const uint64_t* tree_mask,
                    int B, int Sq, int H, float softmax_scale, int num_partitions, float* O,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!tree_mask || (reinterpret_cast<uintptr_t>(tree_mask) & 7)) return MLA_ERR_INVALID_ARG;
  if (Sq > 64) return MLA_ERR_UNSUPPORTED;
  return decode_call(q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, 1, num_partitions, O,
                     lse, workspace, workspace_bytes, stream, false, tree_mask);
}

int mla_decode_tree_e4m3(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* kv_pool,
                         float kv_scale, int64_t num_pages, int page_size,
                         const int32_t* block_table, int max_pages_per_seq,
                         const int32_t* seq_lens, const uint64_t* tree_mask, int B, int Sq,
                         int H, float softmax_scale, int num_partitions, float* O, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!tree_mask || (reinterpret_cast<uintptr_t>(tree_mask) & 7)) return MLA_ERR_INVALID_ARG;
  if (Sq > 64) return MLA_ERR_UNSUPPORTED;
  return decode_call(q_nope, q_rope, kv_pool, kFormatE4m3, kv_scale, num_pages, page_size,
                     block_table, max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, 1,
                     num_partitions, O, lse, workspace, workspace_bytes, stream, false,
                     tree_mask);
}

int mla_decode_nope(const uint16_t* q_nope, const uint16_t* kv_pool, int64_t num_pages,
                    int page_size, const int32_t* block_table, int max_pages_per_seq,
                    const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                    int causal, int num_partitions, float* O, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  // the rope query is never read for NoPE rows: q_nope stands in for the pointer check
  return decode_call(q_nope, q_nope, kv_pool, kFormatNope, 1.0f, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, causal,
                     num_partitions, O, lse, workspace, workspace_bytes, stream, false);
}

int mla_decode_splitkv_nope(const uint16_t* q_nope, const uint16_t* kv_pool, int64_t num_pages,
                            int page_size, const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                            int causal, int num_partitions, float* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  Call c;
  int st = prepare(q_nope, q_nope, kv_pool, num_pages, page_size, block_table, max_pages_per_seq,
                   seq_lens, B, Sq, H, softmax_scale, causal, num_partitions, O, lse, workspace,
                   workspace_bytes, &c);
  if (st != MLA_OK) return st;
  return finish(enqueue_split(c, q_nope, q_nope, kv_pool, kFormatNope, 1.0f, num_pages,
                              block_table, max_pages_per_seq, seq_lens, nullptr, B, Sq, H,
                              softmax_scale, causal, O, lse, false,
                              static_cast<hipStream_t>(stream)),
                workspace, static_cast<hipStream_t>(stream));
}

int mla_decode_varlen(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                      int64_t num_pages, int page_size, const int32_t* block_table,
                      int max_pages_per_seq, const int32_t* seq_lens, const int32_t* q_lens,
                      int B, int Sq, int H, float softmax_scale, int num_partitions, float* O,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_lens || (reinterpret_cast<uintptr_t>(q_lens) & 3)) return MLA_ERR_INVALID_ARG;
  return decode_call(q_nope, q_rope, kv_pool, kFormatBf16, 1.0f, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, H, softmax_scale, 1, num_partitions, O,
                     lse, workspace, workspace_bytes, stream, false, nullptr, q_lens);
}

static int append_call(const uint16_t* kv_new, void* kv_pool, int e4m3, float kv_scale,
                       int64_t num_pages, int page_size, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!kv_new || !kv_pool || !block_table || !seq_lens) return MLA_ERR_INVALID_ARG;
  if (!aligned16(kv_new) || !aligned16(kv_pool)) return MLA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(block_table) & 3) || (reinterpret_cast<uintptr_t>(seq_lens) & 3))
    return MLA_ERR_INVALID_ARG;
  if (page_size != kPage) return MLA_ERR_UNSUPPORTED;
  if (num_pages < 1 || B < 1 || Sq < 1 || max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (e4m3 && (!(kv_scale > 0.0f) || isinf(kv_scale))) return MLA_ERR_INVALID_ARG;
  if ((int64_t)B * Sq > (1 << 24) || (int64_t)max_pages_per_seq * kPage > 0x3fffffff)
    return MLA_ERR_UNSUPPORTED;
  if (!workspace || !aligned16(workspace) || workspace_bytes < (size_t)kHeaderBytes)
    return MLA_ERR_WORKSPACE;
  AppendArgs a;
  a.kv_new = kv_new;
  a.kv_pool = kv_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.flags = static_cast<uint32_t*>(workspace);
  a.num_pages = num_pages;
  a.max_pages = max_pages_per_seq;
  a.B = B;
  a.Sq = Sq;
  a.e4m3 = e4m3;
  a.inv_scale = e4m3 ? 1.0f / kv_scale : 1.0f;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return finish(launch_append(a, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP, workspace, s);
}

int mla_kv_append(const uint16_t* kv_new, uint16_t* kv_pool, int64_t num_pages, int page_size,
                  const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                  int B, int Sq, void* workspace, size_t workspace_bytes, void* stream) {
  return append_call(kv_new, kv_pool, kFormatBf16, 1.0f, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, workspace, workspace_bytes, stream);
}

int mla_kv_append_e4m3(const uint16_t* kv_new, uint8_t* kv_pool, float kv_scale,
                       int64_t num_pages, int page_size, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return append_call(kv_new, kv_pool, kFormatE4m3, kv_scale, num_pages, page_size, block_table,
                     max_pages_per_seq, seq_lens, B, Sq, workspace, workspace_bytes, stream);
}

int mla_absorb_q(const uint16_t* q_heads, const uint16_t* w_uk_t, uint16_t* q_lat, int B, int Sq,
                 int H, void* stream) {
  if (!q_heads || !w_uk_t || !q_lat) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_heads) || !aligned16(w_uk_t) || !aligned16(q_lat)) return MLA_ERR_INVALID_ARG;
  if (B < 1 || Sq < 1 || H < 1) return MLA_ERR_INVALID_ARG;
  if ((int64_t)B * Sq > (1 << 24) || H > 65535) return MLA_ERR_UNSUPPORTED;
  return launch_absorb(q_heads, w_uk_t, q_lat, B * Sq, H, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_project_o(const float* O, const uint16_t* w_uv, float* out, int B, int Sq, int H,
                  void* stream) {
  if (!O || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned16(O) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
  if (B < 1 || Sq < 1 || H < 1) return MLA_ERR_INVALID_ARG;
  if ((int64_t)B * Sq > (1 << 24) || H > 65535) return MLA_ERR_UNSUPPORTED;
  return launch_project(O, w_uv, out, B * Sq, H, static_cast<hipStream_t>(stream)) == hipSuccess
             ? MLA_OK
             : MLA_ERR_HIP;
}

int mla_read_error_flags(void* workspace, void* stream, uint32_t* flags) {
  if (!workspace || !flags) return MLA_ERR_INVALID_ARG;
  return take_flags(workspace, static_cast<hipStream_t>(stream), flags);
}

}  // extern "C"
