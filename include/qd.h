/*
 * qd - one batched autoregressive decode step of a Qwen3-style GQA decoder
 * on AMD MI355X (gfx950).  C ABI: plain pointers and sizes, no C++ types.
 *
 * Sources (the pages this library follows, by title):
 *   [blog]    "GPU 算子与执行优化：从 26 到 100 token/s" (qwen3-runtime)
 *   [engine]  "从零构建 Qwen3-8B 推理引擎，C++/CUDA 实现性能追平 98%"
 *   [infer]   "推理引擎里面发生了什么"
 *   [graphs]  "突破vLLM推理性能瓶颈：CUDA Graph深度优化实战指南"
 *
 * The step, for each sequence b of the batch, with token t = token_ids[b]
 * at position p = positions[b] (context = p + 1 tokens, the new one
 * included):
 *   x = E[t]                                          (embedding lookup)
 *   per layer ([engine] 4.2.2 pre-norm layer; [blog] Part 6 op list):
 *     h = RMSNorm(x) ; q,k,v = h Wq^T, h Wk^T, h Wv^T (one fused QKV
 *         projection, [engine] 4.4.3)
 *     q,k per head: RMSNorm over head_dim, then NeoX RoPE at p ([blog] Part 6)
 *     k,v (bf16) appended to the paged pool at position p ([blog] Part 4;
 *         [infer] PagedAttention: 16-token blocks and a per-request table)
 *     o = softmax(q K^T / sqrt(D)) V over positions 0..p, query head h using
 *         KV head h / (Hq/Hkv) ([engine] 4.4.2), computed split-KV with a
 *         log-sum-exp combine ([blog] Part 8)
 *     x += o Wo^T
 *     x += (silu(RMSNorm(x) Wg^T) * (RMSNorm(x) Wu^T)) Wd^T   ([blog] Part 6)
 *   logits = RMSNorm(x) Wlm^T (tied: Wlm = E) ; next = argmax ([blog] Part 3,
 *   greedy sampling on the device, only the token id leaves the step)
 * Weights and the KV pool are bf16; all accumulation is fp32.
 *
 * Around the step: qd_prefill runs a chunk of prompt tokens through the same
 * layers (causal across the chunk, logits only where asked), qd_sample draws
 * the next token on the device (temperature, top-k, top-p), and qd_blocks_*
 * manage the pool's pages on the host (free pool, forks, prefix cache).
 *
 * Threading: a handle is used by one host thread at a time.  Calls are
 * asynchronous on the handle's stream unless stated otherwise.
 */
#ifndef QD_H
#define QD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  0 is success; every failure is negative. */
#define QD_OK 0
#define QD_EINVAL -1        /* a NULL pointer, a bad size or an unknown name */
#define QD_EUNSUPPORTED -2  /* a shape or option this build does not handle */
#define QD_ESTATE -3        /* e.g. decode before every weight was loaded */
#define QD_EHIP -4          /* a HIP runtime call failed; see qd_last_error */
#define QD_ENOMEM -5        /* device allocation failed */

/* Bits reported by qd_device_status (input errors the kernels detected). */
#define QD_DEV_BAD_TOKEN 1     /* a token id outside [0, vocab) (clamped) */
#define QD_DEV_BAD_POSITION 2  /* a position outside [0, max_pages_per_seq*16) */
#define QD_DEV_BAD_PAGE 4      /* a block-table entry outside [0, num_pages) */
#define QD_DEV_TIMEOUT 8       /* the streaming step gave up waiting (results invalid) */

typedef struct qd_handle qd_handle;

/* Model and capacity.  Shapes follow the HF Qwen3 config names. */
typedef struct qd_config {
  int32_t num_layers;          /* L */
  int32_t hidden;              /* H; multiple of 64, at most 8192 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq / Hkv is 1, 2 or 4 */
  int32_t head_dim;            /* D; 64 or 128 */
  int32_t intermediate;        /* I; multiple of 32 */
  int32_t vocab;               /* V; multiple of 64 */
  int32_t tie_embeddings;      /* 1: the LM head is the embedding matrix */
  float rms_eps;               /* RMSNorm epsilon (Qwen3: 1e-6) */
  double rope_theta;           /* RoPE base (Qwen3: 1e6) */
  int32_t page_size;           /* tokens per KV page; must be 16 */
  int32_t max_batch;           /* largest batch passed to qd_decode_step (1..64) */
  int32_t max_pages_per_seq;   /* block-table row length; at most 2048 (32768 tokens) */
  int32_t num_pages;           /* pages in the caller's pool */
  int32_t use_graphs;          /* 1: replay one captured hipGraph per batch size */
  int32_t persistent;          /* 1: run batch 1 as one cooperative kernel that
                                  streams each wave's share of the weights through LDS
                                  across stage boundaries and computes the projections
                                  with MFMA on a bf16 hi/lo split of their input (about
                                  16 significant bits; the per-stage batch-1 kernels
                                  keep the input in fp32).  Needs head_dim 128 with 4
                                  query heads per KV head or head_dim 64 with 2,
                                  max_pages_per_seq <= 128, at most 64 layers, hidden
                                  <= 8192 and every projection input <= 16384; other
                                  handles, and every batch above 1, take the per-stage
                                  kernels (qd_step_path tells which) */
  int32_t max_prefill_rows;    /* largest chunk passed to qd_prefill_prompts (rows of
                                  all its prompts together, at most 16384); the handle
                                  keeps a workspace of at most rows * (8*hidden +
                                  12*q_dim + 8*kv_dim + 4*intermediate) bytes for it
                                  (q_dim = Hq*D, kv_dim = Hkv*D; 60 MB for 512 rows of
                                  Qwen3-4B).  0: no workspace, and qd_prefill_prompts
                                  is refused */
  int32_t kv_dtype;            /* element type of the caller's KV pool: 0 = bf16;
                                  1 = 8-bit OCP E4M3 codes (the pages' FP8 KV cache:
                                  "推理引擎里面发生了什么", Quantization 对 Kernel 的影响),
                                  stored code = E4M3(value / scale), round to nearest
                                  even, saturating at +-448, read back as code * scale.
                                  Halves the pool's bytes; batch 1 then takes the
                                  per-stage kernels (qd_step_path tells) */
  float k_scale;               /* kv_dtype 1: the scale of every K element (> 0) */
  float v_scale;               /* kv_dtype 1: the scale of every V element (> 0) */
} qd_config;

/* A caller tensor for qd_load_weights.  data is a DEVICE pointer to a
 * row-major bf16 array (dtype 0), shape [rows, cols] or [n] for norm gains. */
typedef struct qd_tensor_desc {
  const char* name;   /* HF name, e.g. "model.layers.3.self_attn.q_proj.weight" */
  const void* data;   /* device pointer, bf16 */
  int32_t ndim;       /* 1 or 2 */
  int64_t shape[2];
  int32_t dtype;      /* 0 = bf16 (the only one accepted) */
} qd_tensor_desc;

/* Create a decoder for `cfg`, bound to HIP stream `hip_stream` (a
 * hipStream_t; NULL means the null stream) on the current device.  Allocates
 * the packed-weight arena, activations, split-KV and split-K scratch and the
 * RoPE table (cos/sin of p * theta^(-2i/D) computed in double, stored fp32).
 * Everything a step touches besides the caller's buffers is allocated here,
 * once, so that its addresses stay fixed for every later step and captured
 * graph (the blog "GPU 算子与执行优化：从 26 到 100 token/s", Part 5: the
 * decode-graph runner allocates its static buffers before capture and the
 * graph freezes every address it uses).
 * Returns QD_OK and *out, or an error (then *out is NULL).  Synchronous. */
int qd_create(const qd_config* cfg, void* hip_stream, qd_handle** out);

/* Copy weights in.  Accepts the HF tensor names of a Qwen3 checkpoint
 * (model.embed_tokens, model.layers.N.{input_layernorm, self_attn.{q,k,v,o}_proj,
 * self_attn.{q,k}_norm, post_attention_layernorm, mlp.{gate,up,down}_proj},
 * model.norm, lm_head when untied) with their HF shapes ([out, in] for
 * projections), as a checkpoint's tensors come, with no offline conversion,
 * and lays them out in the order the step reads them (the rkmt page "从零构建
 * Qwen3-8B 推理引擎", 4.2.1 tensors and weight loading; 4.4.3 fused QKV).
 * Tensors may come in several calls.  The library repacks them into its own
 * tile layout (q|k|v fused, gate and up paired) and keeps no reference to
 * the caller's memory once the call returns.  QD_EINVAL on an unknown name
 * or a wrong shape; QD_EHIP if a repack launch fails.  Synchronous. */
int qd_load_weights(qd_handle* h, const qd_tensor_desc* tensors, int32_t n);

/* One chunk of prompt tokens (chunked prefill; the blog "GPU 算子与执行优化：
 * 从 26 到 100 token/s", Part 7: only the positions whose next token is
 * wanted reach the LM head, and chunks that end no prompt compute no logits).
 * `rows` (1 <= rows <= max_batch) prompt tokens, from one or several
 * sequences, each row laid out as a decode step's row (DEVICE pointers):
 *   token_ids    int32 [rows]        the prompt token at that position
 *   positions    int32 [rows]        its position; a sequence's rows may come
 *                                    in any order but must not repeat a position
 *   block_tables int32 [rows][max_pages_per_seq]  the row's sequence's pages
 *                                    (the same row content for every row of
 *                                    one sequence)
 *   kv_pool      as for qd_decode_step; every row's K/V is written
 *   n_logits     0 .. rows: rows 0 .. n_logits-1 get the final RMSNorm, the
 *                                    LM head and the greedy next id (put each
 *                                    prompt's last token there); 0 = none
 *   out_next_ids int32 [n_logits]    or NULL when n_logits is 0
 *   out_logits   fp32 [n_logits][vocab] or NULL
 * Attention is causal across the chunk: a row attends to every position of
 * its sequence up to its own, including rows of this same chunk (each layer
 * appends all rows' K/V in one launch, then attends in a second).  Positions
 * before the chunk must already be in the pool.  The result equals running
 * the rows one position at a time through qd_decode_step, up to rounding.
 * Kernels are launched directly on the handle's stream (no graph), always
 * the per-stage kernels (also on a persistent handle).  Asynchronous.
 * QD_EINVAL on a NULL pointer, rows out of range or n_logits outside
 * 0..rows; QD_ESTATE before all weights are loaded. */
int qd_prefill(qd_handle* h, int32_t rows, const int32_t* token_ids, const int32_t* positions,
               const int32_t* block_tables, void* kv_pool, int32_t n_logits,
               int32_t* out_next_ids, float* out_logits);

/* Prompts on the matrix cores: n_seqs prompt segments, packed back to back
 * into one chunk of rows = sum(seq_rows) <= max_prefill_rows, run through
 * the layers as one batch, causally masked, with only each prompt's last
 * position reaching the LM head (the blog "GPU 算子与执行优化：从 26 到 100
 * token/s", Part 7; the rkmt page "从零构建 Qwen3-8B 推理引擎", 4.1.2: a
 * prefill writes the prompt's K/V into the cache, then decoding starts from
 * its last logits).  The projections run as GEMMs (bf16 weights times a
 * bf16 hi/lo pair of the input, fp32 accumulation), attention as a tiled
 * causal kernel over the pool's pages.  Segment s holds the tokens of
 * positions start_pos[s] .. start_pos[s] + seq_rows[s] - 1 of one sequence;
 * positions below start_pos[s] (an earlier chunk of the same prompt, or a
 * shared prefix) must already be in the pool.
 *   n_seqs       1 .. 64
 *   seq_rows     int32 [n_seqs]  HOST: rows of each segment, >= 1
 *   start_pos    int32 [n_seqs]  HOST: position of each segment's first row;
 *                                start_pos[s] + seq_rows[s] <= max_pages_per_seq*16
 *   token_ids    int32 [rows]    DEVICE: segment 0's tokens, then segment 1's, ...
 *   block_tables int32 [n_seqs][max_pages_per_seq]  DEVICE: each segment's pages
 *   kv_pool      as for qd_decode_step; every row's K/V is written at its slot
 *   n_logits     0 .. min(n_seqs, max_batch): segments 0 .. n_logits-1 get
 *                the final RMSNorm, the LM head and the greedy next id of
 *                their last row (put the segments that end a prompt first)
 *   out_next_ids int32 [n_logits] DEVICE, or NULL when n_logits is 0
 *   out_logits   fp32 [n_logits][vocab] DEVICE, or NULL
 * The result equals running each segment's rows one position at a time
 * through qd_decode_step, up to rounding.  Kernels are launched directly on
 * the handle's stream (no graph); the host arrays are read before the call
 * returns.  Asynchronous.  QD_EINVAL on a NULL pointer or a size out of
 * range; QD_EUNSUPPORTED on a handle created with max_prefill_rows = 0;
 * QD_ESTATE before all weights are loaded.  Block-table entries outside the
 * pool and token ids outside the vocabulary are clamped and reported by
 * qd_device_status. */
int qd_prefill_prompts(qd_handle* h, int32_t n_seqs, const int32_t* seq_rows,
                       const int32_t* start_pos, const int32_t* token_ids,
                       const int32_t* block_tables, void* kv_pool, int32_t n_logits,
                       int32_t* out_next_ids, float* out_logits);

/* One decode step for `batch` sequences (1 <= batch <= max_batch): token
 * ids and positions in, one next token id per sequence out, and nothing but
 * ids and control crosses the call (the rkmt page "从零构建 Qwen3-8B 推理引擎",
 * 4.1.2: DecodeStep returns the sampled next token; the blog "GPU 算子与执行优化：
 * 从 26 到 100 token/s", Part 5: replay copies the dynamic ids and positions
 * into frozen buffers and launches the captured step once; Part 3: the argmax
 * runs on the device and logits leave only when asked for).  All
 * pointers are DEVICE pointers:
 *   token_ids    int32 [batch]       token decoded by each sequence
 *   positions    int32 [batch]       its position p (= tokens already cached)
 *   block_tables int32 [batch][max_pages_per_seq]  physical page ids; entries
 *                                    0 .. p/16 must name pages of kv_pool
 *   kv_pool      bf16 (or kv_dtype 1: E4M3 bytes) [L][num_pages][2][Hkv][16][D]  caller-owned paged pool
 *                                    (index 0 = K, 1 = V); this step writes
 *                                    K/V of position p of every sequence and
 *                                    reads positions 0..p
 *   out_next_ids int32 [batch]       greedy next token (lowest index on ties)
 *   out_logits   fp32 [batch][vocab] or NULL
 * Sequences in one call must not write the same pool slot.  Asynchronous.
 * On the streaming path (see persistent) the step is one cooperative kernel
 * whose workgroups walk the stages in order and wait on device counters
 * (every wait is bounded; a timeout sets QD_DEV_TIMEOUT).  Otherwise, with
 * use_graphs, the first call
 * for a (batch, pointer set) captures a hipGraph of the per-stage kernels and
 * later calls replay it (new pointers cause a new capture).  A handle keeps
 * at most 64 graphs: beyond that the least recently replayed one is
 * destroyed (after its stream drains) to make room.
 * Kernels clamp out-of-range ids, positions and page ids instead of reading
 * out of bounds, and record them for qd_device_status. */
int qd_decode_step(qd_handle* h, int32_t batch, const int32_t* token_ids,
                   const int32_t* positions, const int32_t* block_tables, void* kv_pool,
                   int32_t* out_next_ids, float* out_logits);

/* Sample the next token of each sequence from a step's logits on the
 * device, so that only the token id leaves the GPU (the yuzheng310 page,
 * "GPU 算子与执行优化", part 3: argmax and the top-p/top-k filters run on
 * the device; the rkmt page, "从零构建 Qwen3-8B 推理引擎", section 4.1.2:
 * temperature and top_p travel with a request).  All pointers are DEVICE
 * buffers of `batch` entries (logits: [batch][vocab] fp32, as qd_decode_step
 * writes them to out_logits), owned by the caller:
 *   temperature  fp32   <= 0 or NaN: greedy (lowest index among the largest)
 *   top_k        int32  keep the top_k highest logits (ties: lower id first);
 *                       <= 0 or >= vocab: no limit; 1: greedy
 *   top_p        fp32   then keep the shortest run of those, highest first,
 *                       whose weight reaches top_p of their total; >= 1 or
 *                       NaN: no limit; <= 0: greedy
 *   uniform      fp32   the caller's draw in [0, 1) (below 0 or NaN: 0)
 *   out_ids      int32  the sampled token ids
 * Weights are exp((logit - max) / temperature) in fp32, each counted as the
 * integer floor(w * 2^32) so that every sum is exact; the sampled token is
 * the kept one, in increasing id order, at which the running weight first
 * exceeds floor(uniform * total).  Logits must be finite and 16-byte
 * aligned.  Asynchronous on the handle's stream; no allocation (scratch
 * owned by the handle: calls on one handle must not overlap).  QD_EINVAL for
 * a NULL or misaligned pointer or a batch outside 1..max_batch. */
int qd_sample(qd_handle* h, int32_t batch, const float* logits, const float* temperature,
              const int32_t* top_k, const float* top_p, const float* uniform,
              int32_t* out_ids);

/* qd_sample without a handle and without allocating anything: for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments and
 * results as qd_sample (DEVICE pointers, `batch` rows of `vocab` fp32
 * logits, 16-byte aligned), plus the vocabulary size and the HIP stream
 * (a hipStream_t; NULL = null stream) the three sampling launches and one
 * small fill launch go to.  Scratch is one static device array of ~2.2 MB
 * per GPU (held until the process ends), sized for batch <= 64 and vocab <=
 * 262144: larger sizes return QD_EINVAL with a message in qd_last_error(NULL).
 * Every call on a GPU shares that GPU's array (its counters are cleared at
 * the start of each call): calls that overlap on one GPU (different streams
 * or threads) race and must be serialised by the caller.  No hipMalloc,
 * hipFree or hipMemset is called.  Asynchronous.  QD_EINVAL also for a NULL
 * or misaligned pointer; QD_EUNSUPPORTED for a vocab too small to chunk;
 * QD_EHIP on a launch error. */
int qd_sample_noalloc(int32_t batch, int32_t vocab, const float* logits, const float* temperature,
                      const int32_t* top_k, const float* top_p, const float* uniform,
                      int32_t* out_ids, void* hip_stream);

/* Intermediate values of one layer, for checking each stage of the step
 * (fp32 DEVICE buffers; any may be NULL):
 *   x_in [B][H]  qkv [B][(Hq+2Hkv)D]  q_rot [B][Hq][D]  k_rot [B][Hkv][D]
 *   attn [B][Hq][D]  x_mid [B][H]  act [B][I]  x_out [B][H]  final_h [B][H] */
typedef struct qd_taps {
  int32_t layer;
  float *x_in, *qkv, *q_rot, *k_rot, *attn, *x_mid, *act, *x_out, *final_h;
} qd_taps;

/* The step as per-stage kernels launched one by one (no graph, and no
 * streaming kernel even on a persistent handle), also filling `taps` (may be
 * NULL). */
int qd_decode_step_taps(qd_handle* h, int32_t batch, const int32_t* token_ids,
                        const int32_t* positions, const int32_t* block_tables,
                        void* kv_pool, int32_t* out_next_ids, float* out_logits,
                        const qd_taps* taps);

/* Checking only: one batch-1 step as the weight-streaming kernel (the one
 * qd_decode_step runs at batch 1 on a handle whose qd_step_path is
 * QD_PATH_STREAM), also filling `taps` (may be NULL): workgroup 0 copies
 * each stage's result of layer taps->layer out of the running kernel once
 * every workgroup has finished that stage.  Same arguments and effects as
 * qd_decode_step at batch 1.  QD_EUNSUPPORTED on a handle that does not
 * stream batch 1. */
int qd_stream_step_taps(qd_handle* h, const int32_t* token_ids, const int32_t* positions,
                        const int32_t* block_tables, void* kv_pool, int32_t* out_next_ids,
                        float* out_logits, const qd_taps* taps);

/* Kernel classes timed by qd_profile_step. */
#define QD_PROF_EMBED 0    /* embedding gather */
#define QD_PROF_QKV 1      /* RMSNorm + fused QKV projection */
#define QD_PROF_ATTN 2     /* q/k norm + RoPE + KV append + split-KV attention */
#define QD_PROF_O 3        /* O projection + residual */
#define QD_PROF_GATE_UP 4  /* RMSNorm + gate/up projection + SwiGLU */
#define QD_PROF_DOWN 5     /* down projection + residual */
#define QD_PROF_LM_HEAD 6  /* final RMSNorm + LM head + argmax */
#define QD_PROF_CLASSES 7

/* Run the step as the per-stage kernels twice on the handle's stream, the
 * second time with a HIP event between consecutive kernels (enqueued while
 * the GPU runs the first, so its kernels run back to back), and return per
 * class the summed time between the events around its kernels in
 * milliseconds (class_ms[QD_PROF_CLASSES]) and the number of launches
 * (class_launches[QD_PROF_CLASSES]).  Same arguments and effects as
 * qd_decode_step (the repeat rewrites the same KV slots with the same
 * values).  Synchronous. */
int qd_profile_step(qd_handle* h, int32_t batch, const int32_t* token_ids,
                    const int32_t* positions, const int32_t* block_tables, void* kv_pool,
                    int32_t* out_next_ids, float* out_logits, float* class_ms,
                    int32_t* class_launches);

/* Time one projection class alone (QD_PROF_QKV, _O, _GATE_UP, _DOWN or
 * _LM_HEAD): its kernels for every layer (the LM head: once), launched as in
 * qd_decode_step at this batch size with the real per-layer weights, are
 * captured into a graph that is replayed `reps` times between two HIP events
 * on the handle's stream; *avg_us is the mean time per launch.  Inputs are
 * whatever the handle's scratch activations hold; the kernels overwrite that
 * scratch (the next qd_decode_step recomputes it) and touch no caller
 * buffer and no KV pool.  QD_EUNSUPPORTED for the other classes.
 * Synchronous. */
int qd_profile_class(qd_handle* h, int32_t batch, int32_t cls, int32_t reps, float* avg_us);

/* Measurement: the device's plain streaming-read rate in GB/s (*gbps), the
 * practical ceiling of the weight-streaming pattern that the step's kernels
 * follow, for comparison with the nominal HBM peak (the locsic page
 * "推理引擎里面发生了什么", HBM bandwidth wall: decode is bound by the rate
 * at which weights stream from HBM).  Reads the first floor(bytes/1024) KB
 * of the DEVICE buffer `buf` (caller-owned, contents irrelevant, >= 1 GiB
 * recommended so that the caches do not hold it) `reps` times with 16-byte
 * nontemporal loads, 1, 2 and 4 workgroups per CU, and reports the best
 * rate; timed with HIP events on `hip_stream` (a hipStream_t, NULL = null
 * stream).  Needs no handle and allocates nothing.  Synchronous.  QD_EINVAL
 * for a NULL pointer, bytes < 1024 or reps < 1; QD_EHIP on a launch error
 * (message in qd_last_error(NULL)). */
int qd_read_ceiling(const void* buf, int64_t bytes, int32_t reps, void* hip_stream, float* gbps);

/* Wait for the handle's stream, then return (and clear) the QD_DEV_* bits
 * the kernels recorded since the last call in *flags.  Synchronous. */
int qd_device_status(qd_handle* h, int32_t* flags);

/* The handle's stream (a hipStream_t), for callers that time or order work. */
void* qd_stream(const qd_handle* h);

/* How qd_decode_step runs a step of `batch` sequences on this handle. */
#define QD_PATH_STAGED 0      /* per-stage kernels launched one by one */
#define QD_PATH_GRAPH 1       /* per-stage kernels replayed from a captured hipGraph */
#define QD_PATH_STREAM 3      /* batch 1: the weight-streaming cooperative kernel */

/* One of QD_PATH_*, or QD_EINVAL for a NULL handle or a batch outside
 * 1..max_batch.  No GPU work. */
int qd_step_path(const qd_handle* h, int32_t batch);

/* ---- Page manager for the paged KV pool (host only, no GPU work) ----
 * Fixed 16-token pages taken from and returned to a free pool in O(1), one
 * page list per sequence (its block-table row for qd_decode_step), forks
 * that share full pages, and a prefix cache: full pages registered under
 * their token prefix are kept after their sequences end and handed to a
 * new sequence whose tokens start the same way (the rkmt page, "从零构建
 * Qwen3-8B 推理引擎", sections 4.3.1 paged KV cache and 4.4.4 automatic
 * prefix cache).  A page is shared only while full; cached pages nobody
 * references are evicted, least recently released first (a sequence's
 * pages from its last to its first), when the free pool is empty.  Pages
 * are ids 0..num_pages-1 of the caller's pool; the first page taken is 0.
 * Not thread-safe.  Errors: QD_EINVAL (NULL pointer, unknown or duplicate
 * sequence id, bad size), QD_ENOMEM (not enough pages: nothing changed),
 * QD_EUNSUPPORTED (more than max_pages_per_seq pages). */
typedef struct qd_blocks qd_blocks;

int qd_blocks_create(int32_t num_pages, int32_t max_pages_per_seq, qd_blocks** out);
void qd_blocks_destroy(qd_blocks* m);
/* A new sequence with no pages. */
int qd_blocks_add(qd_blocks* m, int64_t seq);
/* Make the sequence's pages cover token positions [0, n_tokens) (a step
 * at position p needs n_tokens = p + 1); never shrinks. */
int qd_blocks_reserve(qd_blocks* m, int64_t seq, int32_t n_tokens);
/* End the sequence: its pages return to the pool, or to the cache. */
int qd_blocks_release(qd_blocks* m, int64_t seq);
/* New sequence dst with src's positions: it shares src's full pages; if src
 * has a partly filled page, dst gets a fresh page that the caller must fill
 * by copying page *copy_src to page *copy_dst on the device (both -1 when
 * there is none).  Returns the number of copies (0 or 1). */
int qd_blocks_fork(qd_blocks* m, int64_t src, int64_t dst, int32_t* copy_src,
                   int32_t* copy_dst);
/* Block-table rows [n][max_pages_per_seq] (host int32) of the listed
 * sequences, unused entries set to pad_page. */
int qd_blocks_tables(const qd_blocks* m, const int64_t* seqs, int32_t n, int32_t pad_page,
                     int32_t* out);
/* Token positions the sequence's pages cover. */
int qd_blocks_length(const qd_blocks* m, int64_t seq);
/* Pages obtainable now (free plus cached and unreferenced). */
int qd_blocks_available(const qd_blocks* m);
/* Register the sequence's full pages for tokens[0, n) (n <= its length;
 * the KV of those positions must be in the pages) in the prefix cache;
 * returns the number of pages newly registered. */
int qd_blocks_publish(qd_blocks* m, int64_t seq, const int32_t* tokens, int32_t n);
/* For a sequence with no pages: take the cached full pages whose prefix
 * matches tokens[0, n), longest first; returns the positions they cover
 * (a multiple of 16), which need no prefill. */
int qd_blocks_match(qd_blocks* m, int64_t seq, const int32_t* tokens, int32_t n);

/* ---- Serving loop: continuous (iteration-level) batching ----
 * Requests wait in arrival order; every qd_engine_step admits as many as
 * the batch has room for, prefills their prompts (qd_prefill_prompts;
 * prompt pages found in the prefix cache are taken over instead), runs one
 * decode step (qd_decode_step) for every request that already has a token,
 * and returns the new tokens.  A request joins the decode batch in the
 * iteration after its prompt is done and leaves it on its end-of-sequence
 * token or at its token limit, so the batch size changes between
 * iterations; each batch size replays its own captured graph (the locsic
 * page "推理引擎里面发生了什么", section Continuous Batching; the rkmt page
 * "从零构建 Qwen3-8B 推理引擎", sections 4.3.2 on the batching scheduler and
 * 4.4.4 on the automatic prefix cache).
 *
 * The engine owns a page manager (qd_blocks) over all num_pages pages of
 * the pool and small device buffers; a request takes every page it can need
 * (prompt plus max_new_tokens) when it is admitted, so nothing is ever
 * preempted; a request whose pages are not available stays first in line
 * until others leave.  Prompt rows per iteration are limited by the
 * handle's max_prefill_rows (a longer prompt continues over several
 * iterations).  When a request leaves, the full pages of its tokens are
 * registered in the prefix cache.  Not thread-safe; the handle must outlive
 * the engine and no other work may use the handle or the pool while the
 * engine lives.  Errors set qd_last_error(h); an error from the GPU or the
 * page manager leaves the engine unusable (later calls: QD_ESTATE). */
typedef struct qd_engine qd_engine;

/* kv_pool: the DEVICE pool laid out as for qd_decode_step.  QD_EUNSUPPORTED
 * when the handle was created with max_prefill_rows = 0. */
int qd_engine_create(qd_handle* h, void* kv_pool, qd_engine** out);
/* Waits for the handle's stream, then frees the engine (not the handle or
 * the pool).  NULL is a no-op. */
void qd_engine_destroy(qd_engine* e);
/* A request for qd_engine_submit.  Tokens are greedy (the step's argmax)
 * when temperature <= 0, else drawn on the device by qd_sample's rule with
 * temperature, top_k and top_p (the rkmt page, "从零构建 Qwen3-8B 推理引擎",
 * 4.1.2: temperature and top_p travel with a request); the uniform draw for
 * the request's k-th generated token (k = 0, 1, ...) is SplitMix64's output
 * for the state seed + (k + 1) * 0x9E3779B97F4A7C15, its top 24 bits times
 * 2^-24, so a request's draws do not depend on the requests it is batched
 * with. */
typedef struct qd_engine_request {
  int64_t id;              /* the caller's id, unique among unfinished requests */
  const int32_t* prompt;   /* HOST int32 [n_prompt], copied */
  int32_t n_prompt;        /* >= 1 */
  int32_t max_new_tokens;  /* >= 1 */
  int32_t eos_id;          /* the token that ends the request early; -1: none */
  float temperature;
  int32_t top_k;
  float top_p;
  uint64_t seed;
} qd_engine_request;

/* Queue a request.  QD_EINVAL on a bad argument or token id; QD_EUNSUPPORTED
 * when n_prompt + max_new_tokens - 1 positions exceed max_pages_per_seq*16
 * or the whole pool. */
int qd_engine_submit(qd_engine* e, const qd_engine_request* r);
/* One iteration (synchronous).  Writes *n_out entries (at most max_batch)
 * to the HOST arrays out_req / out_token / out_done of max_out >= max_batch
 * entries: a request id, its next token, and 1 when that token is its last
 * (the request has left).  *n_out = 0 with nothing queued. */
int qd_engine_step(qd_engine* e, int32_t max_out, int64_t* out_req, int32_t* out_token,
                   int32_t* out_done, int32_t* n_out);

typedef struct qd_engine_stats {
  int64_t steps;          /* iterations that ran GPU work */
  int64_t prefill_rows;   /* prompt positions prefilled */
  int64_t cached_rows;    /* prompt positions taken from the prefix cache */
  int64_t decode_rows;    /* sequence positions decoded */
  int64_t tokens_out;     /* tokens returned */
  int64_t sampled_iterations; /* iterations whose tokens came from qd_sample */
  int64_t gpu_us;         /* summed GPU time of the iterations, from each one's
                             first launch to its last kernel (HIP events);
                             the rest of an iteration's wall time is host work */
  int32_t waiting;        /* requests not admitted yet */
  int32_t running;        /* admitted requests (prefilling or decoding) */
  int32_t pages_available;
  int32_t reserved;
} qd_engine_stats;

int qd_engine_get_stats(const qd_engine* e, qd_engine_stats* out);

/* Free everything the handle owns: captured graphs, packed weights,
 * scratch (it waits for its stream first; the caller's pool and buffers are
 * untouched).  Call it before the HIP runtime is torn down (before process
 * exit), like any other release of device memory.  NULL is a no-op.  The
 * pages name no teardown; this is the counterpart of qd_create. */
void qd_destroy(qd_handle* h);

/* Text of the last error on this handle (or of the last failed qd_create when
 * h is NULL).  Valid until the next call on the handle.  Errors never cross
 * the ABI as exceptions (the rkmt page "从零构建 Qwen3-8B 推理引擎", 4.1.1: a
 * fault of the compute layer must not take down the layer above it). */
const char* qd_last_error(const qd_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* QD_H */
