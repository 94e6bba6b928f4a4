// Internal interface between the host runtime (qd_runtime.cpp) and the HIP
// kernels (qd_kernels.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

struct qd_config;
struct qd_handle;

namespace qd {

// Host runtime services for the serving loop (qd_engine.cpp): the handle's
// configuration, and recording an error message on the handle (returned by
// qd_last_error) together with its code.
const qd_config* handle_config(const qd_handle* h);
int handle_fail(qd_handle* h, int code, const std::string& msg);

// Packed weight layout ("tile-major").  A [N][K] bf16 matrix is stored as
// tiles of 16 rows x 32 columns, tile (rt, kt) at element offset
// (rt * (K/32) + kt) * 512; inside a tile, lane l of a wave owns the 16 bytes
// at element offset l * 8: row rt*16 + l%16, columns kt*32 + (l/16)*8 .. +8.
// One 64-lane 16-byte load therefore reads one whole 1 KB tile, and the lane
// ownership is exactly the A operand of a 16x16x32 bf16 MFMA.
// q|k|v are stacked into one matrix; gate and up are interleaved by halves
// of a row tile: packed row tile t holds gate rows 8t..8t+7 in its rows 0-7
// and up rows 8t..8t+7 in its rows 8-15, so any row tile yields 8 SwiGLU
// channels by itself.
constexpr int kTileRows = 16;
constexpr int kTileCols = 32;
constexpr int kTileElems = kTileRows * kTileCols;  // 512 bf16 = 1 KB
constexpr int kRowsPerGroup = 64;                  // rows one GEMV workgroup finishes
constexpr int kPage = 16;                          // tokens per KV page
constexpr int kMaxBatch = 64;
constexpr int kMaxTilesInFlight = 20;              // weight tiles a wave keeps in flight
constexpr int kSsqRows = 16;    // rows per partial sum of squares of the residual stream
constexpr int kTraceItems = 4096;  // (trace builds) items with event slots per launch
constexpr int kCntStride = 32;  // words between arrival counters: one 128-byte line each
                                // (atomics on one line serialise at the memory side)

// Epilogues of the GEMV kernel.
enum GemvMode : int {
  kStore = 0,   // out[b][n] = y
  kResid = 1,   // x[b][n] += y, and partial sums of squares of the new x
  kSwiGLU = 2,  // act[b][i] = silu(gate_i) * up_i  (gate|up interleaved by half tiles)
  kArgmax = 3,  // optional logits, then argmax over all rows per batch column
  kPartial = 4, // no reduction: every item leaves its K-split partial for the consumer
};

// What an attention launch does with the step's K/V rows.
enum KvMode : int {
  kAppendAttend = 0,  // decode: append each row's k, v and attend
  kAppendOnly = 1,    // prefill, first launch of a layer: append only
  kAttendOnly = 2,    // prefill, second launch: attend over the filled pages
};

// The weight tiles of the next projection launch, read into the L2 of the
// XCD that each of its items will run on (workgroup i of a launch runs on
// XCD i % 8, and the L2 keeps its lines across launches), by n_wg extra
// workgroups of a launch that leaves HBM mostly idle.  w = null: none.
struct L2Prefetch {
  const uint16_t* w;   // the next GEMV launch's packed weights
  int KT;              // its k-tiles per row tile
  int rt, S, kps;      // its plan: row tiles per item, K splits, k-tiles per split
  int items;           // how many of its items, from its first (at most its grid)
  int n_wg;            // prefetching workgroups here (a multiple of 8)
};

// One GEMV work item covers rt row tiles (16*rt rows) and one of S slices
// of K (kps k-tiles); its 4 waves take the row tiles and, when rt < 4,
// split the item's K slice between them (reduced in LDS).
struct GemvArgs {
  const uint16_t* w;   // packed tiles, N x K
  int N, K, B, Bmax;
  int S, kps;          // K split count and k-tiles per split
  int rt;              // row tiles per item: 1, 2, 4 or 8
  int wide;            // 1: chunk-streamed items of 128 rows (gemv_wide_item)
  const float* x;      // VALU input activations [B][K] fp32
  const uint16_t* xh;  // MFMA input: bf16 pairs [64][K] of the input (times the RMSNorm gain)
  const uint16_t* xl;
  const float* ssq;    // if non-null: RMSNorm the input; [K/16][Bmax] partial sums of squares
  const float* gain;   // [K] RMSNorm gain
  float eps;
  float* part;         // split-K partials [items][16*rt][B] (kPartial: the consumer's input)
  unsigned* counters;  // [N/(16*rt)] split-K arrival counters, kCntStride apart (zero between uses)
  float* out;          // kStore: [B][N]; kResid: x [B][N]; kSwiGLU: [B][N/2]
  const float* res_in; // kResid: the old residual [B][N] if not out (fused launches
                       // write the new residual to another buffer)
  float* ssq_out;      // kResid: [N/16][Bmax]
  uint16_t* xo_hi;     // kResid, kSwiGLU: if non-null, also the bf16 pairs [64][cols] of the
  uint16_t* xo_lo;     // output (kResid: times xo_gain) for an MFMA consumer
  const float* xo_gain;
  float* logits;       // kArgmax: [B][N] or null
  float* amax_val;     // kArgmax (rt = 4): [N/64][Bmax] row-group maxima
  int* amax_idx;
  float* amax_val2;    // kArgmax: [ceil(N/64/64)][Bmax] maxima of groups of 64 row groups
  int* amax_idx2;
  unsigned* amax_counter;  // kArgmax: ceil(N/64/64) + 1 counters, kCntStride apart
  int* next_ids;       // kArgmax: [B]
  unsigned long long* trace;  // builds with QD_STEP_TRACE only: 8 event timestamps per item, or null
  L2Prefetch pf;       // (standalone kernel) workgroups after the items prefetch these
  int* dev_flags;      // 32- and 64-column items: a bounded wait that times out is flagged here
};

struct AttnArgs {
  const float* qkv;        // [B][(Hq+2Hkv)D], or null when read from qkv_part
  const float* qkv_part;   // if non-null: the QKV projection's qkv_S split partials
  int qkv_S, qkv_rows;     // (qkv_rows rows per QKV item)
  const float* q_gain;     // [D]
  const float* k_gain;     // [D]
  const float* rope_cos;   // [max_pos][D/2]
  const float* rope_sin;
  int max_pos;
  unsigned char* pool_layer;  // this layer's slice of the pool: [P][2][Hkv][16][D] elements
  int num_pages;
  int kv_fp8;              // pool elements: 0 bf16, 1 E4M3 codes (value = code * scale)
  float k_scale, v_scale;  // kv_fp8: the scales, and their inverses for encoding
  float k_inv, v_inv;
  const int* positions;    // [B]
  const int* block_tables; // [B][max_pages]
  int max_pages;
  int B, Hq, Hkv;
  float eps, scale;
  int S_max;               // most splits a sequence can have (sizes o_part, ml_part)
  int grid;                // workgroups of the standalone kernel (they share the items)
  float* o_part;           // [B*Hq][S_max][D]
  float* ml_part;          // [B*Hq][S_max][2]  (running max, running sum)
  unsigned* counters;      // [B*Hkv] split arrival counters, kCntStride apart (zero between uses)
  float* out;              // [B][Hq][D]
  uint16_t* out_hi;        // if non-null: bf16 pairs of out for an MFMA consumer
  uint16_t* out_lo;
  float* tap_q;            // optional [B][Hq][D] (after norm and RoPE, unscaled)
  float* tap_k;            // optional [B][Hkv][D] (before bf16 rounding)
  int* dev_flags;
  unsigned long long* trace;  // builds with QD_STEP_TRACE only: item event timestamps, or null
  int kv_mode;             // kAppendAttend (decode), or a prefill layer's kAppendOnly then
                           // kAttendOnly launch (standalone kernel only)
  L2Prefetch pf;           // (standalone kernel) workgroups after the grid's prefetch these
};

struct EmbedArgs {
  const uint16_t* table;   // packed [V][H]
  int V, H, B, Bmax;
  const int* tokens;
  float* x;                // [B][H]
  float* ssq_out;          // [H/16][Bmax]
  uint16_t* xo_hi;         // if non-null: bf16 pairs [64][H] of x times xo_gain
  uint16_t* xo_lo;
  const float* xo_gain;
  int* dev_flags;
  unsigned* zero;          // if non-null: counters (kCntStride apart) the first row clears
  int nzero;
};

// The MLP half of a layer as one launch at batches 2-16 (MFMA items):
// [gate/up items | down items].  A finished gate/up row group counts in
// cnt_g[the K slice of down its SwiGLU channels feed] (kCntStride apart);
// a down item issues its weight tiles, then waits until its slice's count
// is complete, so that down's weights stream while gate/up finishes.  The
// launch clears the counters it does not use (cnt_other) for the next one.
struct FusedMlpArgs {
  GemvArgs gu, d;      // gate/up (kSwiGLU) and down (kResid)
  int ng, nd;          // items of each
  unsigned* cnt_g;     // [down K slices]
  unsigned* cnt_other; // the next launch's counters, cleared here: [n_other]
  int n_other;
  int* dev_flags;
  unsigned spin_limit;
  L2Prefetch pf;       // workgroups after the items prefetch these
};

// Per-layer pointers for the streaming step kernel (device-resident array).
struct LayerDev {
  const uint16_t *qkv, *o, *gu, *down;
  const float *in_norm, *post_norm, *q_norm, *k_norm;
};

// Dependency counters of one streaming step, all zero at launch.
constexpr int kCntEmbed = 0;
constexpr int kCntPerLayer = 5;  // qkv, attention, o, gate_up, down finalised
constexpr int cnt_index(int layer, int phase) { return 1 + layer * kCntPerLayer + phase; }

struct StreamRun;

// Arguments of the batch-1 streaming step kernel (qd_stream.hip): the whole
// step in one cooperative launch whose waves stream their share of every
// projection's weights through rings in LDS.
constexpr int kStreamRing = 24;  // 1 KB weight tiles a wave keeps loaded or in flight
constexpr int kStreamMaxLayers = 64;
// Longest block-table row (pages) of a handle that runs batch 1 as the
// streaming kernel: its attention runs on few workgroups while the others
// hold their weight rings, which pays for short contexts only.
constexpr int kStreamMaxPages = 128;
constexpr int kStreamStageVec = 16;  // 4-float groups of a staged input per thread
struct StreamArgs {
  EmbedArgs embed;
  AttnArgs attn;             // attention at batch 1; pool_layer is layer 0's slice
  const LayerDev* layers;
  // packed weights of layer l, projection p (QKV, O, gate/up, down) at
  // [4*l + p]: read with scalar loads from the kernel arguments
  const uint16_t* w[4 * kStreamMaxLayers];
  int L, H, QD, I, V, NQKV, Bmax;
  const uint16_t* lm;        // packed [V][H]
  const float* final_norm;
  float eps;
  float* x;                  // [H] residual stream
  float* ssq;                // [H/16][Bmax] partial sums of squares of x (column 0)
  float* qkv;                // [NQKV] q|k|v
  float* attn_out;           // [Hq*D]
  float* act;                // [I]
  float* logits;             // [V] or null
  float* amax_val;           // [grid] per-workgroup maxima of the LM head
  int* amax_idx;
  int* next_ids;             // [1]
  size_t pool_layer_elems;   // elements of one layer's slice of the pool
  const struct StreamRun* runs;  // every wave's weight-tile runs (see qd_stream_plan.h)
  const int* run_off;        // [grid][4] first run of each wave
  int qkv_S;                 // K splits of each QKV row tile (attention sums the partials)
  float* qkv_part;           // [NQKV/16][qkv_S][16] QKV split partials
  int in_floats;             // LDS floats for a stage input plus the old residual rows
  int res_off;               // float offset of the old residual rows in that region
  int rt_max;                // most row tiles of one projection a workgroup owns
  unsigned* cnt;             // [2 + L*kCntPerLayer] dependency counters (zero at launch)
  unsigned* flags;           // [grid][32] per-workgroup completed-stage flags
  unsigned* exit_cnt;
  unsigned* abort_flag;
  int* dev_flags;
  unsigned spin_limit;
  unsigned long long* trace;  // builds with QD_STEP_TRACE only: per-stage timestamps
  // Stage taps (checking only): at layer tap_layer (-1: none) workgroup 0
  // copies each stage's result out once every workgroup has finished it
  // (fp32, the qd_taps layouts; any pointer may be null), and the attention
  // items run with attn_tap (attn plus tap_q / tap_k).
  int tap_layer;
  float *tap_x_in, *tap_qkv, *tap_attn, *tap_x_mid, *tap_act, *tap_x_out, *tap_final_h;
  AttnArgs attn_tap;
};

// Batch columns a GEMV item is compiled for: VALU at batch 1; MFMA above, 8
// columns (the input's hi and lo halves side by side in one 16-column
// operand) up to batch 8, blocks of 16 beyond.  (Batches 2-4 as VALU items
// were measured slower on the 4B shape: 3.08, 3.51, 3.60 ms per step against
// 2.75, 2.80, 2.88 with the 8-column MFMA items.)
constexpr int gemv_nb(int B) {
  return B <= 1 ? 1 : B <= 8 ? 8 : B <= 16 ? 16 : B <= 32 ? 32 : 64;
}
constexpr bool gemv_mfma(int B) { return gemv_nb(B) >= 8; }

// Attention workgroups: the standalone kernel has 8 waves with 1 KV page
// each in flight up to batch 8 on handles sized for short contexts, and 3
// at larger batches or for long contexts (there fewer, busier workgroups are
// worth the extra pages per wave: batch 16, context 256, 4.00 against
// 4.44 ms per step with 1 page; batch 1, context 8192, 2.95 against 3.45;
// but batch 8, context 256, 3.39 with 1 page against 3.44 with 3); the
// streaming kernel's attention items have 4 waves with 1 page.  A split of a
// sequence covers waves * pages.
constexpr int kAttnWaves = 8;
constexpr int kAttnWavesPersistent = 4;
constexpr int kAttnPagesPersistent = 1;
// Handles of at least this many pages per sequence give batches up to 8
// three pages per wave too: contexts that long have splits to spare, and a
// third as many to combine (Qwen3-8B, batch 8, contexts 580-1841: 4.92 ms
// per step with one page, 4.74 with two, 4.43 with three, a wave's pages
// scored before one softmax update); shorter handles keep one page per
// wave, so that short contexts spread over more workgroups (batch 8,
// context 256: 2.83 ms against 2.87 with three and 2.92 with two).  Four
// pages spill registers at head dim 128 (batch 1 at 8K: 2.90 against 2.81).
constexpr int kMidCtxPages = 64;
constexpr int attn_pages_per_wave(int B, bool persistent, bool long_ctx = false,
                                  bool mid_ctx = false) {
  return persistent ? kAttnPagesPersistent : B <= 8 && !long_ctx && !mid_ctx ? 1 : 3;
}
constexpr int attn_pages_per_split(int B, bool persistent, bool long_ctx = false,
                                   bool mid_ctx = false) {
  return (persistent ? kAttnWavesPersistent : kAttnWaves) *
         attn_pages_per_wave(B, persistent, long_ctx, mid_ctx);
}
// An 8-bit pool loads half the bytes per page: its items hold more pages
// per wave (2 instead of 1, 5 instead of 3: 6 would spill registers at head
// dim 128 with 4 query heads per KV head), so that about the same registers
// keep as many bytes in flight and a sequence has fewer splits to combine.
constexpr int attn_pages_per_wave_kv(int B, bool long_ctx, bool kv_fp8, bool mid_ctx = false) {
  return !kv_fp8 ? attn_pages_per_wave(B, false, long_ctx, mid_ctx)
                 : attn_pages_per_wave(B, false, long_ctx) == 3 ? 5 : 2;
}
// Splits of one sequence the final combine can hold (its (max, sum) pairs sit in LDS).
constexpr int kMaxSplitsStaged = 512;

// On-device sampling (qd_sample.hip): G workgroups per row of logits, each
// owning C of them; top_k up to kFastTopK is merged from per-chunk lists of
// 64 candidates, larger top_k and top-p nuclei beyond those 64 tokens are
// selected by all G workgroups of the row together (radix passes).
constexpr int kFastTopK = 64;
constexpr int kSampleChunk = 8192;  // most logits per workgroup
constexpr int kMaxSampleChunks = 64;  // most workgroups per row (vocab <= 524288)
constexpr int kPassHists = 8;  // radix passes of the third launch: 4 by count, 4 by weight
struct SampleArgs {
  const float* logits;       // [B][V]
  int V;
  const float* temperature;  // [B]
  const int* top_k;          // [B]
  const float* top_p;        // [B]
  const float* uniform;      // [B] draws in [0, 1)
  int* out;                  // [B] sampled token ids
  int G, C;                  // workgroups per row, logits per workgroup (sample_split)
  float* part_max;           // [B][G] chunk maxima and their ids
  int* part_idx;
  unsigned long long* cand;  // [B][G][64] each chunk's first 64 tokens in rank order
  unsigned* counters;        // [B] at stride kCntStride, zero between calls
  double* part_sum;          // [B][G] chunk weight sums (rows without limits)
  unsigned* counters2;       // [B] at stride kCntStride, for the second launch
  double* row_hist;          // [B][256] weight per top key byte (top-p rows), zero between calls
  // the third launch (top-p nuclei beyond the first 64 tokens, top_k above
  // kFastTopK)
  double* pass_hist;         // [B][kPassHists][256] count or weight per key byte, zero between calls
  double* part_sum2;         // [B][G] chunk count or weight at a cut key
  double* part_sum3;         // [B][G] chunk weight kept
  unsigned* counters3;       // [B] at stride kCntStride, the row's barriers, zero between calls
  int* row_flag;             // [B] 1: the third launch finishes a top-p row (set by the second)
  int* row_cut;              // [B][2] the last id kept at the top-k and top-p cut keys
  int* dev_flags;            // a wait that timed out is flagged here (or null)
};
void sample_split(int V, int* G, int* C);
hipError_t launch_sample(const SampleArgs& a, int B, hipStream_t s);

// Launchers (qd_kernels.hip).  All return the launch status.
// Source row r lands in packed row (r / blk) * stride + off + r % blk.
hipError_t launch_repack(const uint16_t* src, int rows, int K, uint16_t* dst, int blk,
                         int stride, int off, hipStream_t s);
hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t s);
hipError_t launch_embed(const EmbedArgs& a, hipStream_t s);
hipError_t launch_gemv(const GemvArgs& a, int mode, hipStream_t s);
// waves, pages: kAttnWaves with 1 or 3 pages per wave (bf16 pool), 2 or 5
// (8-bit pool).
hipError_t launch_attention(const AttnArgs& a, int head_dim, int group, int waves, int pages,
                            hipStream_t s);
hipError_t launch_rmsnorm_rows(const float* x, const float* ssq, const float* gain, int H,
                               int B, int Bmax, float eps, float* out, hipStream_t s);

// Batch-1 streaming step: LDS bytes, largest co-resident grid (0 when it
// does not fit), cooperative launch; built for (head_dim, group) = (128, 4)
// and (64, 2) only (stream_lds_bytes returns 0 for other shapes).
size_t stream_lds_bytes(int head_dim, int group, int in_floats, int rt_max);
hipError_t stream_max_grid(int head_dim, int group, size_t lds, int num_cus, int* grid);
hipError_t launch_stream(const StreamArgs& a, int head_dim, int group, int grid, size_t lds,
                         hipStream_t s);

// Records msg as the error qd_last_error(NULL) reports (entry points without
// a handle); returns code.
int set_global_error(int code, const std::string& msg);

// Plain streaming read of the first bytes/1024 KB of src (measurement).
hipError_t launch_read_ceiling(const void* src, size_t bytes, int grid, hipStream_t s);

// The fused MLP launch (batches 2-16).
bool fused_supported(int B);
hipError_t launch_fused_mlp(const FusedMlpArgs& a, size_t lds, hipStream_t s);

// LDS bytes a GEMV workgroup needs for its input slice.
// LDS of a GEMV item of rt row tiles (the head grows with the item's rows)
size_t gemv_lds_bytes(int B, int kps, int rt);

// ------------------------------------------------------------------ prefill
// A prompt chunk of M rows on the GEMM path (qd_prefill_prompts).  The chunk
// holds nseg segments back to back: segment s is rows [row0[s], row0[s+1])
// and holds the tokens at positions pos0[s], pos0[s]+1, ... of the sequence
// whose block-table row is s.  Activations that feed a matrix-core
// projection are stored as "operand tiles": a [M][K] matrix as bf16 hi/lo
// pairs in tiles of 16 rows x 32 columns, tile (mt, kt) holding hi at
// element offset ((mt * (K/32) + kt) * 2) * 512 and lo 512 elements further,
// with element (m, k) at ((k%32)/8 * 16 + m%16) * 8 + k%8 inside a tile: the
// lane layout of the weight tiles, so that lane l's 16 bytes are the B
// operand of a 16x16x32 MFMA (rows m%16 = l%16, columns k = 8*(l/16)..+7).
constexpr int kPfMaxSegs = 64;
constexpr int kPfMaxRows = 16384;
constexpr int kPfRowAlign = 128;  // operand-tile buffers hold whole 128-row blocks

struct PfSegs {
  int n;
  int row0[kPfMaxSegs + 1];
  int pos0[kPfMaxSegs];
  int qb0[kPfMaxSegs + 1];  // first 16-row query block of each segment; qb0[n] = all blocks
};

// Element offset of (m, k) in operand tiles with KT = K/32 k-tiles (hi; lo is +512).
__host__ __device__ constexpr size_t pf_tile_off(int m, int k, int KT) {
  return (((size_t)(m >> 4) * KT + (k >> 5)) * 2) * kTileElems +
         (size_t)((((k & 31) >> 3) << 4) + (m & 15)) * 8 + (k & 7);
}

// Epilogues of the prefill GEMM.
enum PfMode : int {
  kPfStore = 0,   // out[m][n] = y
  kPfResid = 1,   // out[m][n] += y (the residual stream)
  kPfSwiGLU = 2,  // act operand tiles of silu(gate) * up (gate|up interleaved by half tiles)
};

struct PfGemmArgs {
  const uint16_t* w;   // packed weight tiles, N x K
  const uint16_t* x;   // operand tiles of the input, [Mp/16][K/32]
  int N, K, M;
  int nb_n, nb_m;      // workgroup tiles along N and along M
  float* out;          // kPfStore / kPfResid: [M][ldo]
  int ldo;
  uint16_t* act;       // kPfSwiGLU: operand tiles [Mp/16][N/2/32]
};

struct PfAttnArgs {
  const float* qkv;         // [M][(Hq+2Hkv)D] projection output
  const float* q_gain;      // [D]
  const float* k_gain;
  const float* rope_cos;    // [max_pos][D/2]
  const float* rope_sin;
  unsigned char* pool_layer;  // this layer's slice of the pool: [P][2][Hkv][16][D] elements
  int num_pages;
  int kv_fp8;               // pool elements: 0 bf16, 1 E4M3 codes (value = code * scale)
  float k_scale, v_scale, k_inv, v_inv;
  const int* block_tables;  // [nseg][max_pages]
  int max_pages;
  int M, Hq, Hkv;
  float eps, scale;
  uint16_t* q_hi;           // [M][Hq][D] q after norm, RoPE and scale, bf16 pair
  uint16_t* q_lo;
  uint16_t* out;            // attention output as operand tiles, K = Hq*D
  int* dev_flags;
  PfSegs seg;
};

// Prefill launchers (qd_prefill.hip).  wn, wm: the GEMM workgroup tile is
// 32*wn weight rows x 32*wm input rows (4 waves of 16*wn x 16*wm).
hipError_t launch_pf_embed(const uint16_t* table, int V, int H, const int* tokens, int M,
                           float* x, int* dev_flags, hipStream_t s);
hipError_t launch_pf_norm(const float* x, const float* gain, int K, int M, int Mpad, float eps,
                          uint16_t* out, hipStream_t s);
hipError_t launch_pf_gemm(const PfGemmArgs& a, int mode, int wn, int wm, hipStream_t s);
hipError_t launch_pf_qk(const PfAttnArgs& a, int head_dim, hipStream_t s);
hipError_t launch_pf_attn(const PfAttnArgs& a, int head_dim, int group, hipStream_t s);
hipError_t launch_pf_head_rows(const float* x, int H, const PfSegs& seg, int n, const float* gain,
                               float* x_out, float* ssq_out, int Bmax, uint16_t* xo_hi,
                               uint16_t* xo_lo, hipStream_t s);

}  // namespace qd
