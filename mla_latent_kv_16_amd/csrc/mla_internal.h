// Host <-> kernel interface of libmla: argument blocks and launch helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Arguments of the split-KV attention pass (passed by value as the kernel argument).
struct SplitArgs {
  const uint16_t* q_nope;      // [B, M, 512] bf16, M = Sq * H folded rows (m = t * H + h)
  const uint16_t* q_rope;      // [B, M, 64]
  const void* kv_pool;         // [num_pages, 64, 576] bf16, E4M3 codes when kv_e4m3,
                               // or [num_pages, 64, 512] bf16 when kv_nope
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* seq_lens;     // [B]
  const uint64_t* tree_mask;   // [B, Sq] draft-tree ancestor bits, or nullptr (a chain)
  const int32_t* q_lens;       // [B] drafts per request (<= Sq), or nullptr (Sq each)
  float* O;                    // [B, M, 512]
  float* lse;                  // [B, M]  natural log
  float* part_o;               // [slots, slot_rows, 512]  normalised partial outputs
  float* part_lse;             // [slots, slot_rows]       partial log2-sum-exp2
  uint32_t* flags;             // workspace header word
  int64_t num_pages;
  int max_pages;
  int B, Sq, H, M;
  int len_min;                 // smallest valid seq_lens entry: Sq, or 1 with q_lens
  int n_mt;                    // M-tiles per request
  int G;                       // KV partitions
  int slot_rows;               // min(M, M-tile rows)
  int causal;
  int kv_e4m3;                 // 1: the pool holds E4M3 codes scaled by kv_scale
  int kv_nope;                 // 1: NoPE rows (512 bf16, no rope part; q_rope unused)
  float kv_scale;              // dequantization scale of the pool (1 for bf16)
  float scale_log2;            // softmax_scale * kv_scale * log2(e)
  // Single pass (arrive != nullptr): workgroups past the first n_split merge the
  // partials.  A piece bumps arrive[b * n_mt + mt] once its partial is written; a
  // merged row bumps done[b * n_mt + mt], and the last row of the M-tile returns
  // both counters to zero.
  uint32_t* arrive;            // [B * n_mt]
  uint32_t* done;              // [B * n_mt]
  int n_split;                 // split-KV workgroups (G * n_mt)
  int comb_rows;               // single pass: 0 = a workgroup per row, else rows per wave
  // Placement record (or nullptr): split-KV workgroup w writes its XCD (the hardware
  // XCC id), partition and M-tile to wg_trace[3 w .. 3 w + 2].
  int32_t* wg_trace;           // [n_split, 3]
  // Timeline record (or nullptr; only with a placement record): split-KV workgroup w
  // writes ticks of the 100 MHz constant clock to wg_time[5 w .. 5 w + 4]: its start,
  // the page prefix built, the first block of its last piece landed, the end of that
  // piece's walk, and every store of the workgroup complete.
  int64_t* wg_time;            // [n_split, 5]
};

struct CombineArgs {
  const int32_t* seq_lens;
  float* O;
  float* lse;
  const float* part_o;
  const float* part_lse;
  uint32_t* flags;
  uint32_t* arrive;            // single pass: wait for the pieces (nullptr: two passes)
  uint32_t* done;
  int max_pages;
  int B, Sq, H, M;
  int n_mt, G, MT, slot_rows;
};

// Writing new latent rows into the pool (bf16 copy, or E4M3 codes of value * inv_scale).
constexpr int kAppendThreads = 256;
struct AppendArgs {
  const uint16_t* kv_new;      // [B, Sq, 576] bf16
  void* kv_pool;               // [num_pages, 64, 576] bf16, or E4M3 codes when e4m3
  const int32_t* block_table;  // [B, max_pages]
  const int32_t* seq_lens;     // [B]
  uint32_t* flags;             // workspace header word
  int64_t num_pages;
  int max_pages;
  int B, Sq;
  int e4m3;
  float inv_scale;             // fp32(1 / kv_scale) for E4M3 pools
};

// Absorb / project GEMMs around the attention: per-head width of the unabsorbed
// query and of the projected values (128, as in the 192^-0.5 = (128 + 64)^-0.5 scale).
constexpr int kHeadDim = 128;
constexpr int kProjThreads = 256;
hipError_t launch_absorb(const uint16_t* q_heads, const uint16_t* w_uk_t, uint16_t* q_lat,
                         int rows, int H, hipStream_t stream);
hipError_t launch_project(const float* O, const uint16_t* w_uv, float* out, int rows, int H,
                          hipStream_t stream);

// Launch helpers (defined next to the kernels).
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_splitkv(const SplitArgs& a, hipStream_t stream);
// The same pass with eight waves per workgroup (bf16 pools, causal or full masks,
// optional per-request draft counts; no trees, no single pass).
hipError_t launch_splitkv8(const SplitArgs& a, hipStream_t stream);
hipError_t launch_splitkvq(const SplitArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_clear_words(uint32_t* p, int64_t n, hipStream_t stream);

}  // namespace mla
