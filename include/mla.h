/*
 * mla.h - C ABI of the MI355X (gfx950) paged latent-KV MLA library (libmla.so).
 *
 * The library computes absorbed Multi-head Latent Attention over a paged cache
 * of latent rows.  Every head shares one cached row per token: 512 values of the
 * compressed latent c_kv followed by 64 values of the decoupled RoPE key
 * ("LLM inference systems atlas", §06 State architectures and §22 DeepSeek
 * V2 -> V3; the 512-wide latent: TokenSpeed review page, DeepSeek-V3 entry).  The
 * key up-projection is already folded into the query and the value up-projection
 * is applied by the caller afterwards ("absorb + project", TokenSpeed review
 * page, Attack 1), so for request b, draft token t and head h:
 *
 *   K_b[j]   = kv_pool[block_table[b, j / 64], j % 64, 0:576]        j < L_b
 *   n_vis    = L_b - Sq + t + 1  (causal)   or   L_b  (non-causal)
 *   s_j      = softmax_scale * (q_nope[b,t,h] . K_b[j][0:512] + q_rope[b,t,h] . K_b[j][512:576])
 *   lse      = ln(sum_{j < n_vis} exp(s_j))
 *   O[b,t,h] = sum_{j < n_vis} exp(s_j - lse) * K_b[j][0:512]
 *
 * L_b = seq_lens[b] counts every visible row including the Sq new rows, which
 * the caller has already written into the pool.  Draft t of a speculative verify
 * sees the prefix and drafts 0..t (atlas §16 Speculative decoding); a prefill
 * chunk of Sq tokens on a cached prefix sees it the same way (atlas §11 Chunked
 * prefill).  Sq = 1 is ordinary decode.  Pages are reached only through the
 * block table (atlas §07 PagedAttention).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensor pointers are DEVICE pointers to contiguous row-major arrays, aligned
 *   to 16 bytes.  bf16 values travel as their uint16_t bit patterns.
 * - The caller owns every buffer (inputs, outputs, workspace).  The library never
 *   allocates device memory and keeps no per-call state; the only state it holds
 *   is a per-device cache of the compute-unit count.  Calls on different streams
 *   are independent as long as they use different workspaces.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   compute entry point only enqueues work and returns; results are ready once the
 *   stream reaches that point.
 * - Errors are status codes, never exceptions.  Argument checks run on the host
 *   before anything is enqueued; on any error nothing is enqueued.
 * - Data the host cannot see (seq_lens and block_table contents) is checked by the
 *   kernels on every call: a length outside [Sq, 64 * max_pages_per_seq] or a page
 *   id outside [0, num_pages) is clamped so that no access leaves the buffers, and a
 *   flag is raised in the workspace header; mla_read_error_flags() reports it.
 *   Outputs of such a call are unspecified.  The clamp costs nothing on the fast
 *   path, so it is always on; only the REPORT is optional.  In checked mode
 *   (environment variable MLA_CHECK=1 when the call is made) every compute entry
 *   point that takes a workspace also waits for its own work, moves the flags out
 *   of the header and returns MLA_ERR_DEVICE_CHECK if any was raised.  Checked mode
 *   synchronises the stream on every call (no graph capture, no overlap), so it is
 *   for tests and debugging runs.
 * - Rows at or past L_b in a request's last page and block-table entries past
 *   ceil(L_b / 64) are never read; they may hold anything (NaN included).
 * - O and lse are written for every (b, t, h), and may not alias any input.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, non-positive size, NaN scale */
  MLA_ERR_UNSUPPORTED = -2,  /* page_size != 64, batch or grid beyond the library's limits */
  MLA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the size query returned */
  MLA_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
  MLA_ERR_DEVICE_CHECK = -5  /* checked mode only: the kernels raised a data-fault flag */
} mla_status_t;
/* Every entry point returns its status as a plain int holding one of these values
 * (an int has one size and calling convention in every C and C++ compiler, which an
 * enum return type does not guarantee across them). */

/* Device-side data faults reported through the workspace header. */
#define MLA_FLAG_BAD_SEQ_LEN 1u  /* some seq_lens[b] < Sq or > 64 * max_pages_per_seq */
#define MLA_FLAG_BAD_PAGE_ID 2u  /* some visible block_table entry outside [0, num_pages) */
#define MLA_FLAG_MERGE_WAIT 4u   /* a single-pass merge gave up waiting (one second) for the
                                    partials of its request: its outputs are unspecified */

#define MLA_PAGE_SIZE 64
#define MLA_NOPE_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_MAX_BATCH 1024

/* Text for a status code; never NULL. */
const char* mla_status_string(int status);

/*
 * Number of KV partitions ("splits") the decode entry points use when called with
 * num_partitions = 0, on the current HIP device.  Each partition is a contiguous
 * run of pages of the batch's concatenated page list.  The count comes from a cost
 * model measured on MI355X: at most one (partition x M-tile) workgroup per compute
 * unit, and fewer where the partial results a split writes and merges cost more than
 * its shorter page walks save (short contexts).  A result of 1 means no split and no
 * combine pass.  Returns a status; *num_partitions receives the count.  The model
 * counts B * max_pages_per_seq pages, the block table's capacity: a caller whose
 * table is much wider than its real contexts gets more partitions (and a larger
 * workspace) than the real page count would pick, and can pass an explicit count.
 */
int mla_decode_auto_partitions(int B, int Sq, int H, int max_pages_per_seq,
                               int* num_partitions);

/*
 * Workspace bytes a decode or prefill call with these sizes needs (a 256-byte
 * header holding the error flags, then, when the call splits the KV, the
 * single-pass arrival counters and the partial results of the split-KV pass).
 * num_partitions = 0 means the automatic count on the current device.
 */
int mla_decode_workspace_size(int B, int Sq, int H, int max_pages_per_seq,
                              int num_partitions, size_t* bytes);

/*
 * The same size for the automatic partition count of mla_decode (num_partitions =
 * 0) and of mla_prefill_with_prefix, on the current device, as a plain value: 0
 * where the sizes are invalid or unsupported (the compute call would reject them
 * too) or the device cannot be queried.  A caller that passes its own
 * num_partitions sizes the workspace with mla_decode_workspace_size instead.
 */
size_t mla_decode_workspace_bytes(int B, int Sq, int H, int max_pages_per_seq);
size_t mla_prefill_workspace_bytes(int B, int Sq, int H, int max_pages_per_seq);

/*
 * Speculative-verify / plain decode over the paged latent cache ("Faster kernels,
 * slower engine", §7.1 Gluon MLA decode: a split-KV pass that materialises
 * partial results and a second pass that reduces them by their log-sum-exp; the
 * query-length axis is folded into the head axis to fill the matrix tile:
 * TokenSpeed launch news, decode-kernel paragraph).  Enqueues the split-KV pass
 * and, when num_partitions > 1, the merge pass.
 *
 *   q_nope       bf16 [B, Sq, H, 512]   query with the key up-projection absorbed
 *   q_rope       bf16 [B, Sq, H, 64]    rotated RoPE part of the query
 *   kv_pool      bf16 [num_pages, 64, 576]  rows [c_kv 0..511 | k_rope 512..575]
 *   page_size    must be 64
 *   block_table  int32 [B, max_pages_per_seq]  physical page of each logical page
 *   seq_lens     int32 [B]   visible rows per request, Sq <= L_b <= 64 * max_pages_per_seq
 *   softmax_scale  multiplies the whole 576-wide dot product
 *   causal       1: draft t sees rows j <= L_b - Sq + t;  0: every row j < L_b
 *   num_partitions  0 = automatic, else the number of KV partitions to use
 *   O            fp32 [B, Sq, H, 512]   output (written)
 *   lse          fp32 [B, Sq, H]        natural-log log-sum-exp of the scaled scores
 *   workspace    device buffer of at least mla_decode_workspace_size() bytes,
 *                16-byte aligned, zero-filled before its first use (the error-flag
 *                word in its 256-byte header must start at zero; everything past the
 *                header is scratch that each call writes before it reads it).
 */
int mla_decode(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
               int64_t num_pages, int page_size,
               const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
               int B, int Sq, int H, float softmax_scale, int causal, int num_partitions,
               float* O, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Its workspace is a static 64 MiB device array inside the library, one
 * per GPU, held until the process ends; the library looks up its address once per
 * device and allocates nothing.  Same arguments, meaning and results as mla_decode
 * (bit for bit at the same partition count), minus workspace and workspace_bytes:
 *   num_partitions = 0  the automatic count, lowered where needed so that the
 *                       partial results fit the array (1 always fits)
 *   num_partitions > 0  that count; MLA_ERR_WORKSPACE if its partial results
 *                       (mla_decode_workspace_size) exceed 64 MiB, before anything
 *                       is enqueued
 * Every call on one GPU shares that GPU's array and leaves its contents behind
 * (each call writes every partial it reads), so calls that overlap on one GPU, on
 * any streams, race: a caller serialises them.  Data-fault flags land in the
 * array's header, where only checked mode (MLA_CHECK=1) reads them.
 */
int mla_decode_noalloc(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                       int64_t num_pages, int page_size, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq, int H,
                       float softmax_scale, int causal, int num_partitions, float* O,
                       float* lse, void* stream);

/*
 * The same decode in ONE launch ("Faster kernels, slower engine", §7.1: a
 * hand-written kernel can skip the second pass).  Workgroups appended to the
 * split-KV grid merge each request's partials as soon as its pieces have published
 * them through counters in the workspace.  Same arguments, meaning and results (bit
 * for bit) as mla_decode.  On MI355X it is slower than the two launches: publishing
 * the partials across the eight XCDs' L2 caches costs more than the second launch
 * saves.  Its arrival counters live in the workspace and are zeroed by a small
 * kernel launched ahead of the decode on the same stream, so a workspace can serve
 * single-pass and two-pass calls of any shapes in turn.  Calls that share a
 * workspace must not overlap.
 */
int mla_decode_single_pass(const uint16_t* q_nope, const uint16_t* q_rope,
                           const uint16_t* kv_pool, int64_t num_pages, int page_size,
                           const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                           int causal, int num_partitions, float* O, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * The two passes of mla_decode as separate calls, for callers that schedule or
 * time them apart.  Same arguments and meaning, and the same results as mla_decode
 * bit for bit; both calls of one decode must use the same sizes, num_partitions
 * and workspace.
 * mla_decode_splitkv writes the final O/lse of every request that one partition
 * covers whole and partial results for the others; mla_decode_combine merges those
 * partials (and is a no-op when the partition count is 1).
 */
int mla_decode_splitkv(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                       int64_t num_pages, int page_size,
                       const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                       int B, int Sq, int H, float softmax_scale, int causal, int num_partitions,
                       float* O, float* lse, void* workspace, size_t workspace_bytes,
                       void* stream);
int mla_decode_combine(const int32_t* seq_lens, int max_pages_per_seq, int B, int Sq, int H,
                       int num_partitions, float* O, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_splitkv plus a record of where its workgroups ran.  The GPU hands
 * workgroups to its eight XCDs round-robin, and an XCD's L2 serves only that XCD;
 * keeping the workgroups that share KV pages on one XCD is what keeps the L2 hit
 * rate up (TokenSpeed review page, "Optimizing Attention on MI300X" entry and the
 * Fleet entry on chiplet-aware L2 reuse).  The split pass numbers its workgroups so
 * that the M-tiles of one KV partition, and neighbouring partitions, share an XCD
 * (with one partition, where all M-tiles read the same pages, workgroup w instead
 * takes M-tile n - 1 - w of n, the causally longest first, spread over every XCD);
 * this entry point lets a caller check that on the device at hand.
 *   wg_trace      int32 device buffer; split-KV workgroup w (launch order,
 *                 0 <= w < num_partitions_used * ceil(Sq * H / 64)) writes
 *                 wg_trace[3 w] = the XCC id register of the XCD it ran on,
 *                 wg_trace[3 w + 1] = its KV partition, wg_trace[3 w + 2] = its M-tile
 *   wg_trace_len  entries available; fewer than 3 per workgroup -> MLA_ERR_INVALID_ARG
 *                 (as is a NULL or misaligned wg_trace), before anything is enqueued
 * Every other argument, and O, lse and the workspace contents, exactly as for
 * mla_decode_splitkv (the record changes no result).
 */
int mla_decode_splitkv_placement(const uint16_t* q_nope, const uint16_t* q_rope,
                                 const uint16_t* kv_pool, int64_t num_pages, int page_size,
                                 const int32_t* block_table, int max_pages_per_seq,
                                 const int32_t* seq_lens, int B, int Sq, int H,
                                 float softmax_scale, int causal, int num_partitions,
                                 float* O, float* lse, void* workspace, size_t workspace_bytes,
                                 int32_t* wg_trace, int64_t wg_trace_len, void* stream);

/*
 * The placement record plus a timeline of every split-KV workgroup, for measuring
 * where a split pass spends its time on the device at hand (start-up round trips, the
 * stream, the end skew between XCDs; "Faster kernels, slower engine", §7.1 on how
 * close a decode kernel's loads get to peak bandwidth).
 *   wg_trace, wg_trace_len  as for mla_decode_splitkv_placement
 *   wg_time       int64 device buffer, 8-byte aligned; workgroup w writes ticks of the
 *                 GPU's 100 MHz constant clock to wg_time[5 w .. 5 w + 4]: its start,
 *                 the batch's page prefix built, the first block of its last piece in
 *                 LDS, the end of that piece's walk, and all of its stores complete.
 *                 A workgroup whose partition holds no page writes only the first two.
 *   wg_time_len   entries available; fewer than 5 per workgroup -> MLA_ERR_INVALID_ARG
 *                 (as is a NULL or misaligned wg_time), before anything is enqueued
 * Every other argument, and O, lse and the workspace contents, exactly as for
 * mla_decode_splitkv (the records change no result).
 */
int mla_decode_splitkv_timeline(const uint16_t* q_nope, const uint16_t* q_rope,
                                const uint16_t* kv_pool, int64_t num_pages, int page_size,
                                const int32_t* block_table, int max_pages_per_seq,
                                const int32_t* seq_lens, int B, int Sq, int H,
                                float softmax_scale, int causal, int num_partitions, float* O,
                                float* lse, void* workspace, size_t workspace_bytes,
                                int32_t* wg_trace, int64_t wg_trace_len, int64_t* wg_time,
                                int64_t wg_time_len, void* stream);

/*
 * Chunked prefill on top of a long cached prefix (atlas §11 Chunked prefill;
 * TokenSpeed launch news, prefill-kernel paragraph).  Sq is the chunk length,
 * seq_lens[b] = cached prefix + chunk, and the chunk's own latent rows are already
 * in the pool.  Arguments as for mla_decode; with num_partitions = 0 the folded
 * chunk rows alone fill the device, so no split and no combine pass is used.
 */
int mla_prefill_with_prefix(const uint16_t* q_nope, const uint16_t* q_rope,
                            const uint16_t* kv_pool, int64_t num_pages, int page_size,
                            const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                            int causal, int num_partitions, float* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same decode over an FP8 latent pool ("Faster kernels, slower engine", section
 * "Three server boots, not one universal configuration": the MI355X serving runs
 * keep the KV cache in fp8, which halves the bytes moved per cached token).
 *
 *   kv_pool   OCP FP8 E4M3 codes (E4M3FN: bias 7, no infinity, 0x7F/0xFF NaN),
 *             uint8 [num_pages, 64, 576], rows [c_kv 0..511 | k_rope 512..575],
 *             16-byte aligned
 *   kv_scale  per-tensor dequantization scale: a row element is code_value * kv_scale;
 *             must be finite and > 0 (else MLA_ERR_INVALID_ARG)
 *
 * Every other argument, the workspace and the outputs are as for mla_decode /
 * mla_decode_splitkv / mla_decode_single_pass; the combine pass is
 * mla_decode_combine.  The scores and P V
 * run in bf16 on the exact widening of the codes (every E4M3 value is a bf16 value),
 * with kv_scale folded into the softmax scale and into O.
 */
int mla_decode_e4m3(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* kv_pool,
                    float kv_scale, int64_t num_pages, int page_size,
                    const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                    int B, int Sq, int H, float softmax_scale, int causal, int num_partitions,
                    float* O, float* lse, void* workspace, size_t workspace_bytes, void* stream);
int mla_decode_splitkv_e4m3(const uint16_t* q_nope, const uint16_t* q_rope,
                            const uint8_t* kv_pool, float kv_scale, int64_t num_pages,
                            int page_size, const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                            int causal, int num_partitions, float* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);
int mla_decode_single_pass_e4m3(const uint16_t* q_nope, const uint16_t* q_rope,
                                const uint8_t* kv_pool, float kv_scale, int64_t num_pages,
                                int page_size, const int32_t* block_table, int max_pages_per_seq,
                                const int32_t* seq_lens, int B, int Sq, int H,
                                float softmax_scale, int causal, int num_partitions, float* O,
                                float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Decode of a draft TREE (atlas §16 Speculative decoding: candidates are verified
 * in parallel, EAGLE-2 building them as a tree; the atlas node on tree-shaped
 * drafts).  The Sq drafts of a request are numbered parents first and occupy its
 * last Sq rows as in mla_decode; draft t sees the cached prefix (rows < L_b - Sq),
 * its own row L_b - Sq + t, and row L_b - Sq + u for every u < t whose bit u is set
 * in tree_mask[b * Sq + t] (its ancestors).  Bits above t are ignored.  A chain
 * (bits 0..t set) is exactly mla_decode with causal = 1.
 *
 *   tree_mask  uint64 [B, Sq], 8-byte aligned device memory; 1 <= Sq <= 64
 *              (Sq > 64: MLA_ERR_UNSUPPORTED)
 *
 * Every other argument is as for mla_decode (there is no causal flag); the E4M3
 * variant takes the pool and its scale as mla_decode_e4m3 does.
 */
int mla_decode_tree(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                    int64_t num_pages, int page_size, const int32_t* block_table,
                    int max_pages_per_seq, const int32_t* seq_lens, const uint64_t* tree_mask,
                    int B, int Sq, int H, float softmax_scale, int num_partitions, float* O,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream);
int mla_decode_tree_e4m3(const uint16_t* q_nope, const uint16_t* q_rope, const uint8_t* kv_pool,
                         float kv_scale, int64_t num_pages, int page_size,
                         const int32_t* block_table, int max_pages_per_seq,
                         const int32_t* seq_lens, const uint64_t* tree_mask, int B, int Sq,
                         int H, float softmax_scale, int num_partitions, float* O, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * NoPE-MLA decode: the cached row is the 512-wide latent alone, with no decoupled
 * RoPE key ("Faster kernels, slower engine", "Two stacks, one inverted flag": the
 * MI355X runs there serve Kimi-K3, whose MLA layers are NoPE-MLA).  Scores are
 * softmax_scale * q_nope . c_kv; values are c_kv.  There is no q_rope argument.
 *
 *   kv_pool  bf16 [num_pages, 64, 512], 16-byte aligned
 *
 * Every other argument, the workspace, the outputs and the combine pass are as for
 * mla_decode; mla_decode_splitkv_nope is its split-KV pass alone (then
 * mla_decode_combine), as mla_decode_splitkv is for mla_decode.
 */
int mla_decode_nope(const uint16_t* q_nope, const uint16_t* kv_pool, int64_t num_pages,
                    int page_size, const int32_t* block_table, int max_pages_per_seq,
                    const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                    int causal, int num_partitions, float* O, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);
int mla_decode_splitkv_nope(const uint16_t* q_nope, const uint16_t* kv_pool, int64_t num_pages,
                            int page_size, const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* seq_lens, int B, int Sq, int H, float softmax_scale,
                            int causal, int num_partitions, float* O, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode with a per-request number of drafts (atlas §16 Speculative decoding: the
 * number of candidates verified per request varies).  Request b verifies
 * q_lens[b] drafts, 1 <= q_lens[b] <= min(Sq, L_b), held in its first q_lens[b]
 * query slots and its last q_lens[b] cached rows, each draft t seeing rows
 * j <= L_b - q_lens[b] + t.  Query slots t >= q_lens[b] are padding: their O rows
 * are 0 and their LSE is -inf.  A q_lens entry out of range is clamped and raises
 * MLA_FLAG_BAD_SEQ_LEN.  seq_lens[b] must be at least q_lens[b] (not Sq).
 *
 *   q_lens  int32 [B], 4-byte aligned device memory
 *
 * Every other argument is as for mla_decode with causal = 1.
 */
int mla_decode_varlen(const uint16_t* q_nope, const uint16_t* q_rope, const uint16_t* kv_pool,
                      int64_t num_pages, int page_size, const int32_t* block_table,
                      int max_pages_per_seq, const int32_t* seq_lens, const int32_t* q_lens,
                      int B, int Sq, int H, float softmax_scale, int num_partitions, float* O,
                      float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Writes the new tokens' latent rows into the pool: kv_new[b, t] becomes logical
 * row L_b - Sq + t of request b (the rows mla_decode then verifies as its drafts),
 * found through the block table.  The rows around the attention are the pages'
 * "absorb + project" brackets (TokenSpeed review page, Attack 1); this is the cache
 * write that comes first.  The E4M3 variant stores the code of
 * value * fp32(1 / kv_scale): the nearest E4M3 value, ties to the even code,
 * saturated at +-448 (non-finite values saturate too).
 *
 *   kv_new      bf16 [B, Sq, 576], 16-byte aligned device memory
 *   kv_pool     the pool (bf16 or E4M3 codes, [num_pages, 64, 576], 16-byte aligned)
 *   seq_lens    visible rows per request INCLUDING the Sq new ones (as for the decode)
 *   workspace   at least its 256-byte error-flag header (zeroed before first use)
 *
 * A request whose length is outside [Sq, 64 * max_pages_per_seq], or a row whose
 * page id is outside [0, num_pages), is not written and raises the matching
 * MLA_FLAG_*.  Rows written by one call must not share a pool row.
 */
int mla_kv_append(const uint16_t* kv_new, uint16_t* kv_pool, int64_t num_pages, int page_size,
                  const int32_t* block_table, int max_pages_per_seq, const int32_t* seq_lens,
                  int B, int Sq, void* workspace, size_t workspace_bytes, void* stream);
int mla_kv_append_e4m3(const uint16_t* kv_new, uint8_t* kv_pool, float kv_scale,
                       int64_t num_pages, int page_size, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* seq_lens, int B, int Sq,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The per-head GEMMs that bracket the latent attention (TokenSpeed review page,
 * Attack 1: "absorb + project").  Per-head widths are 128 (the unabsorbed query
 * part and the projected values; the softmax scale (128 + 64)^-0.5 of the
 * configurations).  Both run on bf16 MFMA with fp32 accumulation; rows are the
 * B * Sq (request, draft) pairs.
 *
 * mla_absorb_q: q_lat[b,t,h,c] = sum_k q_heads[b,t,h,k] * W_UK[h][k][c], rounded to
 * bf16 (nearest, ties to even) -- the q_nope that mla_decode takes.
 *   q_heads  bf16 [B, Sq, H, 128]
 *   w_uk_t   bf16 [H, 512, 128]: element [h][c][k] = W_UK[h][k][c] (W_UK of each head
 *            transposed once, so that every 128-long k run is contiguous)
 *   q_lat    bf16 [B, Sq, H, 512] (written)
 *
 * mla_project_o: out[b,t,h,v] = sum_c O[b,t,h,c] * W_UV[h][v][c], with O rounded to
 * bf16 for the MFMA and the sum kept in fp32.
 *   O        fp32 [B, Sq, H, 512] (mla_decode's output)
 *   w_uv     bf16 [H, 128, 512]: element [h][v][c] = W_UV[h][v][c]
 *   out      fp32 [B, Sq, H, 128] (written)
 *
 * Pointers are 16-byte aligned device memory; B, Sq, H >= 1 (B * Sq <= 2^24,
 * H <= 65535).  Each only enqueues one kernel on `stream`.
 */
int mla_absorb_q(const uint16_t* q_heads, const uint16_t* w_uk_t, uint16_t* q_lat, int B, int Sq,
                 int H, void* stream);
int mla_project_o(const float* O, const uint16_t* w_uv, float* out, int B, int Sq, int H,
                  void* stream);

/*
 * Waits for `stream`, then copies the workspace header's error flags
 * (MLA_FLAG_*) to *flags and clears them.  Reading forces a synchronisation, so
 * callers use it in checked runs and tests, not on the hot path.
 */
int mla_read_error_flags(void* workspace, void* stream, uint32_t* flags);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
